// Attention router of Polar Sparsity on gfx950: one fully connected layer on
// the token's hidden state, then the per-request top-k heads (or GQA groups).
//
// papernotes.org notes on Polar Sparsity, 损失函数 / 训练策略: the attention
// router is a single FC layer trained on the top-k of the per-head attention
// output norm; atlas.scime.ai summary, "Approach": routers pick the top-k
// attention heads or GQA groups per request.  The selection is produced on
// the device in the layout the selective head attention consumes
// (batch_head_index [B, top_k], ascending), so router -> attention needs no
// host synchronisation.
//
//   scores kernel: one wave per (batch row, 8 consecutive heads); lanes split
//                  the hidden dimension in 16-byte pieces (v_dot2 for 16-bit
//                  inputs, fp32 accumulation), DPP + shuffle wave sums.
//   top-k kernel : one wave per batch row; k rounds of a wave-wide argmax
//                  (ties to the lower head index, NaN ranked as -inf), then
//                  the picked heads are written in ascending order with a
//                  ballot prefix count.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sha_device.h"
#include "sha_launch.h"

namespace sha {
namespace {

using namespace detail;

__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);          // inside each 16-lane row
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

template <int DT>
__global__ __launch_bounds__(256) void sha_router_scores_kernel(RouterArgs a) {
  using E = Elem<DT>;
  constexpr int VEC = E::VEC;
  constexpr int ES = 16 / VEC;
  const int nhg = (a.H + 7) / 8;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int b = wid / nhg, hg = wid % nhg;
  if (b >= a.B) return;
  const int lane = threadIdx.x & 63;
  const char* xr = static_cast<const char*>(a.x) + static_cast<size_t>(b) * a.d * ES;
  const char* wb = static_cast<const char*>(a.w);
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int k = lane * VEC; k < a.d; k += 64 * VEC) {
    const uint4 xv = ld16(xr + k * ES);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int h = hg * 8 + j;
      if (h < a.H) acc[j] += E::dot(xv, ld16(wb + (static_cast<size_t>(h) * a.d + k) * ES));
    }
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float s = wave_sum(acc[j]);
    const int h = hg * 8 + j;
    if (lane == j && h < a.H)
      a.scores[static_cast<size_t>(b) * a.H + h] = s + (a.bias ? a.bias[h] : 0.f);
  }
}

constexpr int kRouterSlots = kRouterMaxH / 64;   // scores per lane

// (value, index) ordering of the top-k: larger value first, then lower index.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void sha_router_topk_kernel(RouterArgs a) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (b >= a.B) return;
  const int lane = threadIdx.x & 63;
  const float* srow = a.scores + static_cast<size_t>(b) * a.H;
  float v[kRouterSlots];
#pragma unroll
  for (int i = 0; i < kRouterSlots; ++i) {
    const int h = lane + 64 * i;
    float x = h < a.H ? srow[h] : kNegInf;
    v[i] = (x != x) ? kNegInf : x;  // NaN ranks like -inf
  }
  uint32_t taken = 0;
  for (int r = 0; r < a.top_k; ++r) {
    float bv = kNegInf;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int i = 0; i < kRouterSlots; ++i) {
      const int h = lane + 64 * i;
      if (!((taken >> i) & 1u) && better(v[i], h, bv, bi)) {
        bv = v[i];
        bi = h;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
  }
  // Picked heads in ascending order: slot i holds heads 64 i .. 64 i + 63.
  int base = 0;
  int32_t* irow = a.index + static_cast<size_t>(b) * a.top_k;
#pragma unroll
  for (int i = 0; i < kRouterSlots; ++i) {
    const bool mine = (taken >> i) & 1u;
    const unsigned long long mask = __ballot(mine);
    if (mine) irow[base + __popcll(mask & ((1ull << lane) - 1ull))] = lane + 64 * i;
    base += __popcll(mask);
  }
}

template <int DT>
hipError_t launch_router_t(const RouterArgs& a, hipStream_t st) {
  const long long waves = static_cast<long long>(a.B) * ((a.H + 7) / 8);
  hipLaunchKernelGGL((sha_router_scores_kernel<DT>), dim3(static_cast<unsigned>((waves + 3) / 4)),
                     dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.top_k == 0) return e;
  hipLaunchKernelGGL(sha_router_topk_kernel, dim3(static_cast<unsigned>((a.B + 3) / 4)), dim3(256),
                     0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, int dtype, hipStream_t st) {
  switch (dtype) {
    case kF32: return launch_router_t<kF32>(a, st);
    case kF16: return launch_router_t<kF16>(a, st);
    default: return launch_router_t<kBF16>(a, st);
  }
}

}  // namespace sha
