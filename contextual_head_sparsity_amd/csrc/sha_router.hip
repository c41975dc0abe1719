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
//   K-split form (16-bit inputs, H <= 128, B <= 4096, a caller workspace):
//                  a workgroup of four waves owns 16 batch rows and 256
//                  hidden elements (64 per wave in two 32-element
//                  v_mfma_f32_16x16x32 steps: A = 16 rows of x, B = 16 heads
//                  of w, every head block of the layer), the waves' products
//                  added in LDS in wave order and stored as one fp32 partial
//                  per (row, 256-element chunk, head); the top-k workgroup of
//                  a row adds its partials in chunk order, adds the bias and
//                  writes the scores before ranking them.  Each workgroup
//                  reads 16 rows x 256 elements of x once and the same 256
//                  columns of w, so the whole call reads x once and w once per
//                  16 rows (from L2 after the first).  Many short workgroups
//                  instead of a long dot product per (row, heads) pay where
//                  the call has many multiply-adds (B H d >= 2^24); below
//                  that the one-pass kernels are faster.
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

typedef __bf16 rbf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 rf16x8_t __attribute__((ext_vector_type(8)));
typedef float rf32x4 __attribute__((ext_vector_type(4)));

// 16 x 16 x 32 matrix-core product with fp32 accumulation.  Operand layout
// (lane l, q = l / 16, c = l % 16): A[i][k] holds i = c, k = 8q .. 8q+7;
// B[k][j] holds j = c, k = 8q .. 8q+7; the result D[i][j] holds
// i = 4q .. 4q+3, j = c.
template <int DT>
__device__ __forceinline__ rf32x4 mma16(uint4 a, uint4 b, rf32x4 c);
template <>
__device__ __forceinline__ rf32x4 mma16<kF16>(uint4 a, uint4 b, rf32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(rf16x8_t, a),
                                                __builtin_bit_cast(rf16x8_t, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ rf32x4 mma16<kBF16>(uint4 a, uint4 b, rf32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(rbf16x8_t, a),
                                                 __builtin_bit_cast(rbf16x8_t, b), c, 0, 0, 0);
}

constexpr int kPartWaves = 4;                          // waves per partial workgroup
constexpr int kPartRows = 16;                          // batch rows per workgroup

// Workgroup (row block rb, chunk ch) of the K-split form, NHB = ceil(H / 16)
// head blocks.  Wave w covers hidden elements [ch*256 + w*64, +64); every
// load of the wave is issued before the first product.  Rows past B read
// row B - 1 and heads past H read head H - 1 (never stored); hidden
// elements past d (a ragged last chunk; d is a multiple of 8, so a lane's
// 8 elements are all in or all out) are zeroed in both operands.
template <int DT, int NHB>
__global__ __launch_bounds__(kPartWaves * 64) void sha_router_part_kernel(RouterArgs a) {
  constexpr int kPartWaveK = kRouterChunk / kPartWaves;  // hidden elements per wave
  constexpr int kPartSteps = kPartWaveK / 32;            // matrix-core steps per wave
  __shared__ float red[kPartWaves][kPartRows][NHB * 16 + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = lane >> 4, c = lane & 15;
  const int ch = blockIdx.x % a.nchunk, rb = blockIdx.x / a.nchunk;
  const size_t pitch = static_cast<size_t>(a.d) * 2;  // bytes per row of x and of w
  const char* xr = static_cast<const char*>(a.x) +
                   static_cast<size_t>(min(rb * kPartRows + c, a.B - 1)) * pitch;
  const char* wr[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
    wr[hb] = static_cast<const char*>(a.w) + static_cast<size_t>(min(hb * 16 + c, a.H - 1)) * pitch;
  const int k0 = ch * kRouterChunk + wave * kPartWaveK + q * 8;
  uint4 av[kPartSteps], bv[kPartSteps][NHB];
#pragma unroll
  for (int j = 0; j < kPartSteps; ++j) {
    const int k = k0 + 32 * j;
    const size_t off = static_cast<size_t>(k < a.d ? k : 0) * 2;
    av[j] = ld16(xr + off);
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) bv[j][hb] = ld16(wr[hb] + off);
  }
  __builtin_amdgcn_sched_barrier(0);
  rf32x4 acc[NHB];
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) acc[hb] = rf32x4{0.f, 0.f, 0.f, 0.f};
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int j = 0; j < kPartSteps; ++j) {
    const bool in = k0 + 32 * j < a.d;
    const uint4 x = in ? av[j] : zero;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) acc[hb] = mma16<DT>(x, in ? bv[j][hb] : zero, acc[hb]);
  }
  // Lane (q, c) holds rows 4q .. 4q+3 of head hb*16 + c.
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][4 * q + r][hb * 16 + c] = acc[hb][r];
  __syncthreads();
  for (int p = threadIdx.x; p < kPartRows * NHB * 16; p += kPartWaves * 64) {
    const int r = p / (NHB * 16), h = p % (NHB * 16);
    const int row = rb * kPartRows + r;
    if (row < a.B && h < a.H) {
      float s = red[0][r][h];
#pragma unroll
      for (int w = 1; w < kPartWaves; ++w) s += red[w][r][h];
      a.part[(static_cast<size_t>(row) * a.nchunk + ch) * a.H + h] = s;
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
//
// SUM (the K-split form, H <= 128): the row's scores are first formed from
// its partials.  The 256 threads are G = 256 / H groups of H (one head per
// thread); group g adds chunks g, g + G, ... in order, the G group sums are
// added in group order, then the bias; the result is written to scores and
// ranked from LDS.  With top_k = 0 only the scores are written.
template <int SLOTS, bool SUM>
__global__ __launch_bounds__(kTopkWaves * 64) void sha_router_topk_kernel(RouterArgs a) {
  constexpr int N = 64 * SLOTS;
  constexpr int Q = N / kTopkWaves;
  constexpr int T = kTopkWaves * 64;
  __shared__ unsigned long long keys[N];
  __shared__ int part[kTopkWaves][N];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x;
  if constexpr (SUM) {
    static_assert(N <= kRouterSplitMaxH, "one head per thread of a group");
    __shared__ float gsum[T];
    __shared__ float srow[N];
    const int G = T / a.H;
    const int g = threadIdx.x / a.H, h = threadIdx.x - g * a.H;
    // The bias is loaded with the partials, not after them.
    const float bias = (a.bias && threadIdx.x < a.H) ? a.bias[threadIdx.x] : 0.f;
    float s = 0.f;
    if (g < G) {
      const float* p = a.part + static_cast<size_t>(b) * a.nchunk * a.H + h;
      const size_t st = static_cast<size_t>(G) * a.H;
      int ch = g;
      // Eight loads in flight, added in chunk order.
      for (; ch + 7 * G < a.nchunk; ch += 8 * G) {
        const float* pc = p + static_cast<size_t>(ch) * a.H;
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = pc[u * st];
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
      {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int c = ch + u * G;
          v[u] = c < a.nchunk ? p[static_cast<size_t>(c) * a.H] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) s += v[u];
      }
    }
    gsum[threadIdx.x] = s;
    __syncthreads();
    if (threadIdx.x < N) {
      float t = kNegInf;
      if (threadIdx.x < a.H) {
        t = 0.f;
        for (int q = 0; q < G; ++q) t += gsum[q * a.H + threadIdx.x];
        t += bias;
        a.scores[static_cast<size_t>(b) * a.H + threadIdx.x] = t;
      }
      srow[threadIdx.x] = t;
    }
    if (a.top_k == 0) return;
    __syncthreads();
    if (threadIdx.x < N) keys[threadIdx.x] = topk_key(srow[threadIdx.x], threadIdx.x);
  } else {
    const float* srow = a.scores + static_cast<size_t>(b) * a.H;
#pragma unroll
    for (int i = 0; i < (N + T - 1) / T; ++i) {
      const int h = threadIdx.x + T * i;
      if (h < N) keys[h] = topk_key(h < a.H ? srow[h] : kNegInf, h);
    }
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

template <int SLOTS, bool SUM = false>
hipError_t launch_topk(const RouterArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((sha_router_topk_kernel<SLOTS, SUM>), dim3(static_cast<unsigned>(a.B)),
                     dim3(kTopkWaves * 64), 0, st, a);
  return hipGetLastError();
}

template <int DT, int NHB>
void launch_part(const RouterArgs& a, hipStream_t st) {
  const long long wgs = static_cast<long long>(a.nchunk) * ((a.B + kPartRows - 1) / kPartRows);
  hipLaunchKernelGGL((sha_router_part_kernel<DT, NHB>), dim3(static_cast<unsigned>(wgs)),
                     dim3(kPartWaves * 64), 0, st, a);
}

// K-split form: partials, then the summing top-k kernel (always launched:
// it writes the scores).
template <int DT>
hipError_t launch_router_split(const RouterArgs& a, hipStream_t st) {
  switch ((a.H + 15) / 16) {
    case 1: launch_part<DT, 1>(a, st); break;
    case 2: launch_part<DT, 2>(a, st); break;
    case 3: launch_part<DT, 3>(a, st); break;
    case 4: launch_part<DT, 4>(a, st); break;
    case 5: launch_part<DT, 5>(a, st); break;
    case 6: launch_part<DT, 6>(a, st); break;
    case 7: launch_part<DT, 7>(a, st); break;
    default: launch_part<DT, 8>(a, st); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return a.H <= 64 ? launch_topk<1, true>(a, st) : launch_topk<2, true>(a, st);
}

template <int DT, int HEADS>
void launch_scores(const RouterArgs& a, hipStream_t st) {
  const long long wgs = static_cast<long long>(a.B) * ((a.H + HEADS - 1) / HEADS);
  hipLaunchKernelGGL((sha_router_scores_kernel<DT, HEADS>), dim3(static_cast<unsigned>(wgs)),
                     dim3(kScoreWaves * 64), 0, st, a);
}

template <int DT>
hipError_t launch_router_t(const RouterArgs& a, int num_cus, hipStream_t st) {
  if constexpr (DT != kF32) {
    if (a.part) return launch_router_split<DT>(a, st);
  }
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
