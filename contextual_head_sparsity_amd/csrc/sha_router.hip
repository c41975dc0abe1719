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
//   scores kernel: one workgroup per (batch row, 4 consecutive heads; 2 when
//                  the grid would not fill the CUs); its eight waves take
//                  64-piece blocks of the hidden dimension in turn, 16-byte
//                  pieces (v_dot2 for 16-bit inputs, fp32 accumulation), DPP
//                  + shuffle wave sums, the waves' partials added in a fixed
//                  order.
//   top-k kernel : one workgroup of four waves per batch row; each head's
//                  rank in the (score descending, index ascending) order
//                  (NaN ranked as -inf) is a count of larger 64-bit keys
//                  (order-preserving score bits, then the inverted head id)
//                  staged in LDS, each wave counting a quarter of the row;
//                  the heads of rank < k are written in ascending order with
//                  a ballot prefix count.
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

constexpr int kScoreWaves = 8;  // waves per scores workgroup
constexpr int kTopkWaves = 4;   // waves per top-k workgroup (one batch row)

// One workgroup per (batch row, HEADS consecutive heads).  The hidden
// dimension is cut into blocks of 64 16-byte pieces and wave w takes blocks
// w, w + 8, ...: a lane dots its piece of the row against the same piece of
// each head.  Whole blocks keep the waves' shares within one block of each
// other and spend no load on clamped duplicates except in a ragged last
// block.  Sums: per lane in block order, a wave sum, then the 8 waves'
// partials added in a fixed order, so the result does not depend on timing.
template <int DT, int HEADS>
__global__ __launch_bounds__(kScoreWaves * 64) void sha_router_scores_kernel(RouterArgs a) {
  using E = Elem<DT>;
  constexpr int VEC = E::VEC;
  constexpr int ES = 16 / VEC;
  __shared__ float part[kScoreWaves][HEADS];
  const int nhg = (a.H + HEADS - 1) / HEADS;
  const int b = blockIdx.x / nhg, hg = blockIdx.x % nhg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int pieces = a.d / VEC;
  const int nblk = (pieces + 63) / 64;
  const char* xr = static_cast<const char*>(a.x) + static_cast<size_t>(b) * a.d * ES;
  const char* wr[HEADS];
  // Heads past H read head H - 1 and are never stored.
#pragma unroll
  for (int j = 0; j < HEADS; ++j)
    wr[j] = static_cast<const char*>(a.w) +
            static_cast<size_t>(min(hg * HEADS + j, a.H - 1)) * a.d * ES;
  float acc[HEADS];
#pragma unroll
  for (int j = 0; j < HEADS; ++j) acc[j] = 0.f;
  for (int blk = wave; blk < nblk; blk += kScoreWaves) {
    const int piece = blk * 64 + lane;
    // Unconditional loads (a ragged last block clamps to the last piece),
    // all in flight together.
    const size_t p = static_cast<size_t>(min(piece, pieces - 1)) * 16;
    const uint4 xv = ld16(xr + p);
    uint4 wv[HEADS];
#pragma unroll
    for (int j = 0; j < HEADS; ++j) wv[j] = ld16(wr[j] + p);
    // Keep every load above the first use: the scheduler would otherwise
    // interleave them with the dot products and wait on each in turn.
    __builtin_amdgcn_sched_barrier(0);
    const bool ok = piece < pieces;
#pragma unroll
    for (int j = 0; j < HEADS; ++j) {
      const float t = E::dot(xv, wv[j]);
      acc[j] += ok ? t : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < HEADS; ++j) {
    const float s = wave_sum(acc[j]);
    if (lane == 0) part[wave][j] = s;
  }
  __syncthreads();
  if (threadIdx.x < HEADS) {
    const int j = threadIdx.x, h = hg * HEADS + j;
    if (h < a.H) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kScoreWaves; ++w) s += part[w][j];
      a.scores[static_cast<size_t>(b) * a.H + h] = s + (a.bias ? a.bias[h] : 0.f);
    }
  }
}

// Sort key of head h with score x in the (score descending, index
// ascending) order: a larger key ranks first.  NaN becomes -inf and -0
// becomes +0 (equal floats, equal keys); the float's bits are mapped to an
// unsigned integer of the same order (sign bit set: all bits flipped, else
// the sign bit flipped), and the low word holds ~h so that of two equal
// scores the lower head id has the larger key.
__device__ __forceinline__ unsigned long long topk_key(float x, int h) {
  x = (x != x) ? kNegInf : (x == 0.f ? 0.f : x);
  unsigned u = __float_as_uint(x);
  u ^= (u >> 31) ? 0xffffffffu : 0x80000000u;
  return (static_cast<unsigned long long>(u) << 32) | static_cast<unsigned>(~h);
}

// One workgroup of 4 waves per batch row.  Head h is picked when fewer than
// top_k heads rank before it, i.e. have a larger key.  The row's keys are
// staged in LDS (64 SLOTS entries; those past H hold -inf with an index of
// H or more, so they never rank before a real head); wave w counts, for
// every head, the larger keys among entries [w Q, (w + 1) Q), read as
// broadcasts, and wave 0 adds the four counts and writes the picked heads
// in ascending order with a ballot prefix count.  SLOTS = heads per lane
// (H <= 64 SLOTS), a compile-time count so that the loops have no
// branches.
template <int SLOTS>
__global__ __launch_bounds__(kTopkWaves * 64) void sha_router_topk_kernel(RouterArgs a) {
  constexpr int N = 64 * SLOTS;
  constexpr int Q = N / kTopkWaves;
  __shared__ unsigned long long keys[N];
  __shared__ int part[kTopkWaves][N];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x;
  const float* srow = a.scores + static_cast<size_t>(b) * a.H;
#pragma unroll
  for (int i = 0; i < (N + kTopkWaves * 64 - 1) / (kTopkWaves * 64); ++i) {
    const int h = threadIdx.x + kTopkWaves * 64 * i;
    if (h < N) keys[h] = topk_key(h < a.H ? srow[h] : kNegInf, h);
  }
  __syncthreads();
  unsigned long long mine[SLOTS];
  int rank[SLOTS];
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    mine[i] = keys[lane + 64 * i];
    rank[i] = 0;
  }
#pragma unroll
  for (int o = 0; o < Q; ++o) {
    const unsigned long long k = keys[wave * Q + o];
#pragma unroll
    for (int i = 0; i < SLOTS; ++i) rank[i] += k > mine[i] ? 1 : 0;
  }
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) part[wave][lane + 64 * i] = rank[i];
  __syncthreads();
  if (wave != 0) return;
  int base = 0;
  int32_t* irow = a.index + static_cast<size_t>(b) * a.top_k;
#pragma unroll
  for (int i = 0; i < SLOTS; ++i) {
    const int h = lane + 64 * i;
    int r = 0;
#pragma unroll
    for (int w = 0; w < kTopkWaves; ++w) r += part[w][h];
    const bool mine_pick = h < a.H && r < a.top_k;
    const unsigned long long mask = __ballot(mine_pick);
    if (mine_pick) irow[base + __popcll(mask & ((1ull << lane) - 1ull))] = h;
    base += __popcll(mask);
  }
}

template <int SLOTS>
hipError_t launch_topk(const RouterArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((sha_router_topk_kernel<SLOTS>), dim3(static_cast<unsigned>(a.B)),
                     dim3(kTopkWaves * 64), 0, st, a);
  return hipGetLastError();
}

template <int DT, int HEADS>
void launch_scores(const RouterArgs& a, hipStream_t st) {
  const long long wgs = static_cast<long long>(a.B) * ((a.H + HEADS - 1) / HEADS);
  hipLaunchKernelGGL((sha_router_scores_kernel<DT, HEADS>), dim3(static_cast<unsigned>(wgs)),
                     dim3(kScoreWaves * 64), 0, st, a);
}

template <int DT>
hipError_t launch_router_t(const RouterArgs& a, int num_cus, hipStream_t st) {
  // 4 heads per workgroup; 2 when that leaves CUs idle (small batches or
  // few heads), trading more reads of the row for more workgroups.
  if (static_cast<long long>(a.B) * ((a.H + 3) / 4) < num_cus)
    launch_scores<DT, 2>(a, st);
  else
    launch_scores<DT, 4>(a, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.top_k == 0) return e;
  const int slots = (a.H + 63) / 64;
  if (slots <= 1) return launch_topk<1>(a, st);
  if (slots <= 2) return launch_topk<2>(a, st);
  if (slots <= 4) return launch_topk<4>(a, st);
  if (slots <= 8) return launch_topk<8>(a, st);
  return launch_topk<kRouterMaxH / 64>(a, st);
}

}  // namespace

hipError_t launch_router(const RouterArgs& a, int dtype, int num_cus, hipStream_t st) {
  switch (dtype) {
    case kF32: return launch_router_t<kF32>(a, num_cus, st);
    case kF16: return launch_router_t<kF16>(a, num_cus, st);
    default: return launch_router_t<kBF16>(a, num_cus, st);
  }
}

}  // namespace sha
