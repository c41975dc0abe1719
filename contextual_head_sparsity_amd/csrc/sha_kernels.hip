// HIP kernels for Selective Head Attention (SHA) decode on gfx950 (CDNA4).
//
// The method: Polar Sparsity reproducibility page (ri.k117.org), "Pseudocode",
// Algorithm 1 "Selective Head Flash Attention (Decode)": each unit (b, k)
// resolves head_idx = batch_head_index[b, k], streams K/V of that head in
// tiles while keeping a running max m, running sum l and output accumulator,
// then writes O[b, head_idx, 0, :].  Only active heads are read and written
// (Polar Sparsity notes, papernotes.org, "Selective Head Attention (SHA)
// Kernel").
//
// MI355X mapping (our design, not the pages' A100 kernel):
//   * A workgroup is one (unit, KV split).  Inside it, every aligned group of
//     LPR = d*elem/16 lanes owns one key row per load: one 128-bit load per
//     lane per row, so a wave64 reads 64*16 = 1 KiB of contiguous K (or V)
//     per load instruction.  Each lane group is an independent online-softmax
//     stream over its rows; streams are merged at the end (shuffles inside a
//     wave, LDS across waves).  Each K/V byte is consumed by exactly the lane
//     that loaded it, so K/V go HBM -> VGPR with no LDS round trip.
//   * q.k partial dot products use v_dot2_f32_{f16,bf16} (exact fp16/bf16
//     products, fp32 accumulate) and a DPP butterfly inside the lane group.
//   * Scores carry scale*log2(e), so every exponential is one v_exp_f32 (2^x).
//   * The running max is only moved when a chunk's max exceeds it by more
//     than kRescaleSlack (base-2 units): probabilities stay <= 2^8, the final
//     O = o / l is unchanged, and the per-chunk rescale of o is skipped in the
//     common case.  This is the same running-max algebra as Algorithm 1's
//     merge, with a lazier update rule.
//   * O is accumulated unnormalised and divided by l once at the end (the
//     value of Algorithm 1's per-tile normalisation, fewer divides).
//   * KV split (flash-decoding): a unit's keys are cut into nsplit contiguous
//     chunks so that small B*top_k still fills 256 CUs; each split writes
//     fp32 (o, m, l) partials and a second kernel merges them in a fixed
//     order (the same running-max merge across splits).  The kernel boundary
//     makes the
//     partials visible across XCDs without atomics.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sha_device.h"
#include "sha_launch.h"

namespace sha {
namespace {

using namespace detail;

// One iteration of a lane group's online softmax over U key rows
// (rows r0, r0 + RSTEP, ...).  MASK handles the ragged last iteration: rows at
// or beyond ke get score -inf and their (clamped, in-bounds) loads are unused.
template <int DT, int LPR, int RSTEP, int U, bool MASK, int NH, class Rows>
__device__ __forceinline__ void online_step(const Rows& rows, int col, const uint4 (&qv)[NH],
                                            int r0, int ke, float sl2, float (&m)[NH],
                                            float (&l)[NH],
                                            float (&o)[NH][Elem<DT>::VEC]) {
  using E = Elem<DT>;
  constexpr int VEC = E::VEC;
  uint4 kr[U], vr[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = MASK ? min(r0 + u * RSTEP, ke - 1) : r0 + u * RSTEP;
    kr[u] = ld16_stream(rows.k(r) + col);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int r = MASK ? min(r0 + u * RSTEP, ke - 1) : r0 + u * RSTEP;
    vr[u] = ld16_stream(rows.v(r) + col);
  }
  float s[NH][U];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    float mc = kNegInf;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float x = group_sum<LPR>(E::dot(qv[j], kr[u])) * sl2;
      if (MASK && r0 + u * RSTEP >= ke) x = kNegInf;
      s[j][u] = x;
      mc = fmaxf(mc, x);
    }
    if (mc > m[j] + kRescaleSlack) {
      const float alpha = exp2_hw(m[j] - mc);  // 0 on the first update (m = -inf)
      l[j] *= alpha;
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[j][i] *= alpha;
      m[j] = mc;
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float vf[VEC];
    E::widen(vr[u], vf);
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      // A lane group that has seen only masked rows still has m = -inf.
      const float mu = MASK ? (m[j] == kNegInf ? 0.f : m[j]) : m[j];
      const float p = exp2_hw(s[j][u] - mu);
      l[j] += p;
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[j][i] = fmaf(p, vf[i], o[j][i]);
    }
  }
}

// Merge the (m, l, o) streams of the lane groups of one wave (xor butterfly
// over the group index).
template <int LPR, int VEC, int NH>
__device__ __forceinline__ void merge_wave(float (&m)[NH], float (&l)[NH], float (&o)[NH][VEC]) {
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const float m2 = __shfl_xor(m[j], off);
      const float l2 = __shfl_xor(l[j], off);
      const float M = fmaxf(m[j], m2);
      const float Mu = (M == kNegInf) ? 0.f : M;
      const float a1 = exp2_hw(m[j] - Mu), a2 = exp2_hw(m2 - Mu);
      l[j] = a1 * l[j] + a2 * l2;
#pragma unroll
      for (int i = 0; i < VEC; ++i) o[j][i] = a1 * o[j][i] + a2 * __shfl_xor(o[j][i], off);
      m[j] = M;
    }
  }
}

// Shared body of the head kernel (NH = 1) and the group kernel (NH heads of
// one KV group).  heads[j] < 0 marks an unused head slot of the last chunk.
// A split that holds none of row b's keys (a short row) leaves m = -inf,
// l = 0, o = 0: the merges give it zero weight and a row with no keys at all
// gets zeros.
template <int DT, int D, int WAVES, int U, int NH, int LAYOUT>
__device__ __forceinline__ void decode_unit(const Args& a, int unit, int split, int b, int g,
                                            const int (&heads)[NH], int part_head0,
                                            int part_heads) {
  using E = Elem<DT>;
  constexpr int VEC = E::VEC;
  constexpr int ES = 16 / VEC;            // bytes per element
  constexpr int ROWB = D * ES;            // bytes per key row
  constexpr int LPR = D / VEC;            // lanes per key row
  constexpr int RPW = 64 / LPR;           // rows per wave per load
  constexpr int RSTEP = WAVES * RPW;      // rows per unroll step (whole workgroup)
  constexpr int RITER = RSTEP * U;        // rows per iteration

  __shared__ float sm_o[WAVES][NH][D];
  __shared__ float sm_ml[WAVES][NH][2];
  __shared__ int sm_pages[LAYOUT == kKvPaged ? kMaxSplitPages : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int grp = lane / LPR, sub = lane % LPR;

  const int ks = split * a.chunk;
  const int ke = min(ks + a.chunk, row_keys(a, b));

  KvRows<LAYOUT, ROWB, ES> rows;
  rows.init(a, b, g, ks, ke, sm_pages);
  const int col = sub * VEC * ES;

  uint4 qv[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    qv[j] = make_uint4(0, 0, 0, 0);
    if (heads[j] >= 0)
      qv[j] = ld16(static_cast<const char*>(a.q) +
                   ((static_cast<size_t>(b) * a.H + heads[j]) * D + sub * VEC) * ES);
  }

  float m[NH], l[NH], o[NH][VEC];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    m[j] = kNegInf;
    l[j] = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[j][i] = 0.f;
  }

  const int lrow = wave * RPW + grp;
  int base = ks;
  const int nfull = (ke - ks) / RITER;
  for (int it = 0; it < nfull; ++it, base += RITER)
    online_step<DT, LPR, RSTEP, U, false, NH>(rows, col, qv, base + lrow, ke, a.scale_log2, m, l, o);
  if (base < ke)
    online_step<DT, LPR, RSTEP, U, true, NH>(rows, col, qv, base + lrow, ke, a.scale_log2, m, l, o);

  merge_wave<LPR, VEC, NH>(m, l, o);

  if (grp == 0) {
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int i = 0; i < VEC; ++i) sm_o[wave][j][sub * VEC + i] = o[j][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      sm_ml[wave][j][0] = m[j];
      sm_ml[wave][j][1] = l[j];
    }
  }
  __syncthreads();

  // Merge across waves: one output element per thread.
  for (int e = tid; e < NH * D; e += WAVES * 64) {
    const int j = e / D, c = e % D;
    if (heads[j] < 0) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sm_ml[w][j][0]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const float wt = exp2_hw(sm_ml[w][j][0] - Mu);
      L += wt * sm_ml[w][j][1];
      acc += wt * sm_o[w][j][c];
    }
    if (a.nsplit == 1) {
      E::store(a.o, (static_cast<size_t>(b) * a.H + heads[j]) * D + c, L > 0.f ? acc / L : 0.f);
    } else {
      const size_t p = (static_cast<size_t>(unit) * part_heads + part_head0 + j) * a.nsplit + split;
      a.part_o[p * D + c] = acc;
      if (c == 0) {
        a.part_ml[2 * p] = M;
        a.part_ml[2 * p + 1] = L;
      }
    }
  }
}

// Head-indexed unit: blockIdx.x = unit * nsplit + split.
template <int DT, int D, int WAVES, int U, int LAYOUT>
__global__ __launch_bounds__(WAVES * 64) void sha_decode_mha_kernel(Args a) {
  const int split = blockIdx.x % a.nsplit;
  const int unit = blockIdx.x / a.nsplit;
  const int h = a.idx[unit];
  if (h < 0 || h >= a.H) return;  // padding / out-of-range entry: no read, no write
  const int heads[1] = {h};
  decode_unit<DT, D, WAVES, U, 1, LAYOUT>(a, unit, split, unit / a.top_k, h / a.G, heads, 0, 1);
}

// Group-indexed unit: blockIdx.x = (unit * nchunk + chunk) * nsplit + split;
// the workgroup computes query heads g*G + chunk*NH + j of group g.
template <int DT, int D, int WAVES, int U, int NH, int LAYOUT>
__global__ __launch_bounds__(WAVES * 64) void sha_decode_gqa_kernel(Args a) {
  const int nchunk = (a.G + NH - 1) / NH;
  const int split = blockIdx.x % a.nsplit;
  const int rest = blockIdx.x / a.nsplit;
  const int chunk = rest % nchunk;
  const int unit = rest / nchunk;
  const int g = a.idx[unit];
  if (g < 0 || g >= a.H_kv) return;
  int heads[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    const int hj = chunk * NH + j;
    heads[j] = (hj < a.G) ? g * a.G + hj : -1;
  }
  decode_unit<DT, D, WAVES, U, NH, LAYOUT>(a, unit, split, unit / a.top_k, g, heads, chunk * NH, a.G);
}

// Merge the nsplit partials of one (unit, head): blockIdx.x = unit *
// heads_per_unit + j, one thread per output element, fixed split order.
template <int DT, int D>
__global__ __launch_bounds__(D) void sha_combine_kernel(Args a, int gqa) {
  const int hpu = gqa ? a.G : 1;
  const int unit = blockIdx.x / hpu, j = blockIdx.x % hpu;
  const int id = a.idx[unit];
  int h;
  if (gqa) {
    if (id < 0 || id >= a.H_kv) return;
    h = id * a.G + j;
  } else {
    if (id < 0 || id >= a.H) return;
    h = id;
  }
  const int c = threadIdx.x;
  const size_t p0 = static_cast<size_t>(blockIdx.x) * a.nsplit;
  float M = kNegInf;
  for (int s = 0; s < a.nsplit; ++s) M = fmaxf(M, a.part_ml[2 * (p0 + s)]);
  const float Mu = (M == kNegInf) ? 0.f : M;
  float L = 0.f, acc = 0.f;
  for (int s = 0; s < a.nsplit; ++s) {
    const float wt = exp2_hw(a.part_ml[2 * (p0 + s)] - Mu);
    L += wt * a.part_ml[2 * (p0 + s) + 1];
    acc += wt * a.part_o[(p0 + s) * D + c];
  }
  // L == 0: the row has no keys (every split empty); its output is zero.
  Elem<DT>::store(a.o, (static_cast<size_t>(unit / a.top_k) * a.H + h) * D + c,
                  L > 0.f ? acc / L : 0.f);
}

// ---------------------------------------------------------------------------
// Launch variants: (waves per workgroup, rows per lane group per iteration).
// Variant 0 is the default; the others exist for tuning sweeps.
// ---------------------------------------------------------------------------
constexpr KernelShape kMhaShapes[] = {{4, 8}, {4, 4}, {4, 2}, {8, 2}, {8, 4}, {2, 8}, {1, 8}, {2, 4}};
constexpr int kNumMha = sizeof(kMhaShapes) / sizeof(kMhaShapes[0]);
constexpr KernelShape kGqaShapes[] = {{4, 2}, {4, 1}, {2, 2}, {8, 1}, {4, 4}};
constexpr int kNumGqa = sizeof(kGqaShapes) / sizeof(kGqaShapes[0]);

template <int DT, int D>
hipError_t launch_combine_t(const Args& a, int gqa, hipStream_t st) {
  const unsigned blocks = static_cast<unsigned>(a.B) * a.top_k * (gqa ? a.G : 1);
  hipLaunchKernelGGL((sha_combine_kernel<DT, D>), dim3(blocks), dim3(D), 0, st, a, gqa);
  return hipGetLastError();
}

template <int DT, int D, int V, int LAYOUT = kKvContig>
hipError_t launch_mha_v(const Args& a, hipStream_t st) {
  constexpr KernelShape s = kMhaShapes[V];
  const unsigned blocks = static_cast<unsigned>(a.B) * a.top_k * a.nsplit;
  hipLaunchKernelGGL((sha_decode_mha_kernel<DT, D, s.waves, s.unroll, LAYOUT>), dim3(blocks),
                     dim3(s.waves * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.nsplit > 1) e = launch_combine_t<DT, D>(a, 0, st);
  return e;
}

template <int DT, int D, int V, int NH, int LAYOUT = kKvContig>
hipError_t launch_gqa_v(const Args& a, hipStream_t st) {
  constexpr KernelShape s = kGqaShapes[V];
  const unsigned nchunk = (a.G + NH - 1) / NH;
  const unsigned blocks = static_cast<unsigned>(a.B) * a.top_k * nchunk * a.nsplit;
  hipLaunchKernelGGL((sha_decode_gqa_kernel<DT, D, s.waves, s.unroll, NH, LAYOUT>), dim3(blocks),
                     dim3(s.waves * 64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.nsplit > 1) e = launch_combine_t<DT, D>(a, 1, st);
  return e;
}

// Strided and paged layouts run the default shape only; the tuning variants
// exist for the contiguous layout.
template <int DT, int D>
hipError_t launch_mha_d(const Args& a, int variant, hipStream_t st) {
  if (a.layout == kKvStrided) return launch_mha_v<DT, D, 0, kKvStrided>(a, st);
  if (a.layout == kKvPaged) return launch_mha_v<DT, D, 0, kKvPaged>(a, st);
  switch (variant) {
    case 1: return launch_mha_v<DT, D, 1>(a, st);
    case 2: return launch_mha_v<DT, D, 2>(a, st);
    case 3: return launch_mha_v<DT, D, 3>(a, st);
    case 4: return launch_mha_v<DT, D, 4>(a, st);
    case 5: return launch_mha_v<DT, D, 5>(a, st);
    case 6: return launch_mha_v<DT, D, 6>(a, st);
    case 7: return launch_mha_v<DT, D, 7>(a, st);
    default: return launch_mha_v<DT, D, 0>(a, st);
  }
}

template <int DT, int D, int NH>
hipError_t launch_gqa_nh(const Args& a, int variant, hipStream_t st) {
  if (a.layout == kKvStrided) return launch_gqa_v<DT, D, 0, NH, kKvStrided>(a, st);
  if (a.layout == kKvPaged) return launch_gqa_v<DT, D, 0, NH, kKvPaged>(a, st);
  switch (variant) {
    case 1: return launch_gqa_v<DT, D, 1, NH>(a, st);
    case 2: return launch_gqa_v<DT, D, 2, NH>(a, st);
    case 3: return launch_gqa_v<DT, D, 3, NH>(a, st);
    case 4: return launch_gqa_v<DT, D, 4, NH>(a, st);
    default: return launch_gqa_v<DT, D, 0, NH>(a, st);
  }
}

template <int DT, int D>
hipError_t launch_gqa_d(const Args& a, int variant, hipStream_t st) {
  switch (gqa_heads_per_wg(a.G, false)) {
    case 2: return launch_gqa_nh<DT, D, 2>(a, variant, st);
    case 4: return launch_gqa_nh<DT, D, 4>(a, variant, st);
    default: return launch_gqa_nh<DT, D, 8>(a, variant, st);
  }
}

template <int DT>
hipError_t launch_mha_dt(const Args& a, int d, int variant, hipStream_t st) {
  return d == 64 ? launch_mha_d<DT, 64>(a, variant, st) : launch_mha_d<DT, 128>(a, variant, st);
}

template <int DT>
hipError_t launch_gqa_dt(const Args& a, int d, int variant, hipStream_t st) {
  return d == 64 ? launch_gqa_d<DT, 64>(a, variant, st) : launch_gqa_d<DT, 128>(a, variant, st);
}

int clamp_variant(int v, int n) { return (v < 0 || v >= n) ? 0 : v; }

}  // namespace


int gqa_heads_per_wg(int G, bool mfma) {
  if (mfma) return 16;
  return G <= 2 ? 2 : (G <= 4 ? 4 : 8);
}


hipError_t launch_combine(const Args& a, int dtype, int d, int gqa, hipStream_t st) {
  switch (dtype) {
    case kF32: return d == 64 ? launch_combine_t<kF32, 64>(a, gqa, st) : launch_combine_t<kF32, 128>(a, gqa, st);
    case kF16: return d == 64 ? launch_combine_t<kF16, 64>(a, gqa, st) : launch_combine_t<kF16, 128>(a, gqa, st);
    default: return d == 64 ? launch_combine_t<kBF16, 64>(a, gqa, st) : launch_combine_t<kBF16, 128>(a, gqa, st);
  }
}

hipError_t launch_mha(const Args& a, int dtype, int d, int variant, hipStream_t st) {
  variant = clamp_variant(variant, kNumMha);
  switch (dtype) {
    case kF32: return launch_mha_dt<kF32>(a, d, variant, st);
    case kF16: return launch_mha_dt<kF16>(a, d, variant, st);
    default: return launch_mha_dt<kBF16>(a, d, variant, st);
  }
}

hipError_t launch_gqa(const Args& a, int dtype, int d, int variant, bool mfma, hipStream_t st) {
  if (mfma && dtype != kF32) return launch_gqa_mfma(a, dtype, d, st);
  variant = clamp_variant(variant, kNumGqa);
  switch (dtype) {
    case kF32: return launch_gqa_dt<kF32>(a, d, variant, st);
    case kF16: return launch_gqa_dt<kF16>(a, d, variant, st);
    default: return launch_gqa_dt<kBF16>(a, d, variant, st);
  }
}

}  // namespace sha
