// GQA group-sparsity SHA decode on the matrix cores of gfx950.
//
// In the group variant (Polar Sparsity notes, papernotes.org, SHA Kernel
// bullet on GQA; atlas.scime.ai summary, "Approach") the G query heads of an
// active KV group share one K/V stream, so each key tile meets a real dense
// contraction: S^T = K_tile Q_g^T (keys x heads) and O^T += V_tile^T P^T
// (d x heads).  With G = 8 and d = 128 that is 8 flop per K/V byte, which on
// the vector ALUs costs as much issue time as the HBM stream itself; on MFMA
// it is a few percent of the matrix-core budget.  The online softmax between
// the two products is Algorithm 1's tile update (reproducibility page,
// ri.k117.org, "Pseudocode"), kept per head in base 2 with lazy rescaling.
//
// Wave tile: 32 keys.  Operand layouts of v_mfma_f32_16x16x32_{bf16,f16}
// (lane l, q = l / 16, c = l % 16):
//   A[i][k] : lane holds i = c, k = 8q .. 8q+7
//   B[k][j] : lane holds j = c, k = 8q .. 8q+7
//   D[i][j] : lane holds i = 4q .. 4q+3, j = c
// QK: A = K rows (keys 16*mb + c, d = 32*kc + 8q ..), B = Q^T (head c, same
// d range) held in registers.  Loading A straight from HBM would make every
// wave load touch 16 rows x 64 bytes, a pattern that streams markedly slower
// on this GPU than whole 1 KiB runs; so the K tile is loaded like V (1 KiB
// contiguous per wave load) into LDS rows padded by 16 bytes, where the 16
// lanes of each 128-bit read phase (rows c = 0..15, one pitch apart) fall on
// distinct banks, and read back in the A layout.
// The D layout leaves each lane with 4 keys (4q + r) of head c per 16-key
// block; the PV product's K index is ordered so that lane (q, c) owns keys
// {4q .. 4q+3, 16+4q .. 16+4q+3} of head c, which is exactly what the
// scores left in that lane, so P^T needs no data movement.
// PV: A = V^T needs, per lane, 8 keys of one d column.  V rows go to LDS
// (row pitch padded by 32 bytes) and come back with ds_read_b64_tr_b16: a
// transposed read in which lane i of each 16-lane group receives element i%4
// of the 8 bytes addressed by lane 4*j + i/4 of its group, for j = 0..3.
// Pointing lane s of group q at row 4q + s/4, columns 4*(s%4) .. +3 of the
// d block therefore yields V[4q + j][d_block + i], j = 0..3, for lane i.
// P is split into a high and a low 16-bit part (p = hi + lo) and both go
// through the PV product, so the probabilities keep ~16 significant bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sha_device.h"
#include "sha_launch.h"

namespace sha {
namespace {

using namespace detail;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __fp16 fp16x4_vs_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef __attribute__((address_space(3))) fp16x4_vs_t lds_f16x4_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) float lds_float_t;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;

template <int DT>
struct Mma;

template <>
struct Mma<kBF16> {
  __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static uint2 tr_read(const lds_char_t* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                                         (lds_bf16x4_t*)(p)));
  }
  // Two fp32 values to two 16-bit values (round to nearest even), packed.
  __device__ static uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2_t));
  }
  __device__ static float lo_val(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static float hi_val(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
};

template <>
struct Mma<kF16> {
  __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static uint2 tr_read(const lds_char_t* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16(
                                         (lds_f16x4_t*)(p)));
  }
  __device__ static uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, f16x2_t));
  }
  __device__ static float lo_val(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w & 0xFFFFu)));
  }
  __device__ static float hi_val(uint32_t w) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
  }
};

// Pack 8 probabilities into a B operand (high parts) and the rounding
// remainders into a second one (low parts).
template <int DT>
__device__ __forceinline__ void split_pack(const float (&p)[8], uint4& hi, uint4& lo) {
  using M = Mma<DT>;
  uint32_t h[4], r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = M::pack(p[2 * i], p[2 * i + 1]);
    r[i] = M::pack(p[2 * i] - M::lo_val(h[i]), p[2 * i + 1] - M::hi_val(h[i]));
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(r[0], r[1], r[2], r[3]);
}

// Lanes of a wave exchange K and V rows through the wave's own LDS buffers:
// a lane reads rows other lanes stored, and the next tile overwrites them.
// LDS operations of one wave complete in order; this keeps the compiler from
// moving a store past a read of the same buffer (or the reverse) as well.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

constexpr int kTileKeys = 32;   // keys per wave tile (K of the PV product)
constexpr int kCols = 16;       // query heads per workgroup (N of both products)

// blockIdx.x = (unit * nchunk + chunk) * nsplit + split; the workgroup
// computes query heads g*G + chunk*16 + c (c < 16) of group g.  A split
// holding none of row b's keys leaves (m, l, o) = (-inf, 0, 0).
template <int DT, int D, int WAVES, int LAYOUT>
__global__ __launch_bounds__(WAVES * 64) void sha_decode_gqa_mfma_kernel(Args a) {
  using M = Mma<DT>;
  constexpr int KC = D / 32;                 // d chunks of the QK product
  constexpr int DB = D / 16;                 // d blocks of the PV product
  constexpr int ROWB = D * 2;                // bytes per key row
  constexpr int PITCH = ROWB + 32;           // LDS row pitch: conflict-free transposed reads
  constexpr int VBUF = kTileKeys * PITCH;    // LDS bytes per wave (V tile, later the partial O)
  constexpr int VLD = kTileKeys * ROWB / 1024;  // 128-bit K (and V) loads per lane per tile
  constexpr int LPRW = ROWB / 16;            // lanes per K/V row in a load
  constexpr int PO = D + 4;                  // partial-O row pitch (floats): conflict-free writes
  static_assert(kCols * PO * 4 + kCols * 2 * 4 <= VBUF, "partial O must fit the V buffer");
  constexpr int KPITCH = ROWB + 16;          // K rows: conflict-free 128-bit operand reads
  constexpr int KBUF = kTileKeys * KPITCH;

  __shared__ __attribute__((aligned(16))) char smem[WAVES * VBUF];
  __shared__ __attribute__((aligned(16))) char smem_k[WAVES * KBUF];
  __shared__ int sm_pages[LAYOUT == kKvPaged ? kMaxSplitPages : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, col = lane & 15;

  const int nchunk = (a.G + kCols - 1) / kCols;
  const int split = blockIdx.x % a.nsplit;
  const int rest = blockIdx.x / a.nsplit;
  const int chunk = rest % nchunk;
  const int unit = rest / nchunk;
  const int g = a.idx[unit];
  if (g < 0 || g >= a.H_kv) return;  // padding / out-of-range entry: no read, no write
  const int b = unit / a.top_k;
  const int head0 = chunk * kCols;
  const int nh = min(kCols, a.G - head0);

  const int ks = split * a.chunk;
  const int ke = min(ks + a.chunk, row_keys(a, b));

  KvRows<LAYOUT, ROWB, 2> rows;
  rows.init(a, b, g, ks, ke, sm_pages);

  // Q^T operands: head col, d = 32*kc + 8*q4 .. +8 (zero for heads past the group).
  uint4 qb[KC];
  {
    const char* qrow = static_cast<const char*>(a.q) +
                       (static_cast<size_t>(b) * a.H + g * a.G + head0 + col) * ROWB;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc)
      qb[kc] = col < nh ? ld16(qrow + kc * 64 + q4 * 16) : make_uint4(0, 0, 0, 0);
  }

  f32x4 acc[DB];
#pragma unroll
  for (int i = 0; i < DB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.f;

  // All shared-memory accesses go through address-space-3 pointers.
  lds_char_t* const sbase = (lds_char_t*)(smem);
  lds_char_t* const vt = sbase + wave * VBUF;
  lds_char_t* const kt = (lds_char_t*)(smem_k) + wave * KBUF;

  for (int base = ks + wave * kTileKeys; base < ke; base += WAVES * kTileKeys) {
    const bool full = base + kTileKeys <= ke;
    // K tile: 1 KiB contiguous per wave load, like V.
    uint4 kl[VLD];
#pragma unroll
    for (int u = 0; u < VLD; ++u) {
      int row = base + u * (1024 / ROWB) + lane / LPRW;
      if (!full) row = min(row, ke - 1);
      kl[u] = ld16_stream(rows.k(row) + (lane % LPRW) * 16);
    }
    wave_lds_sync();  // the previous tile's K and V reads are done
#pragma unroll
    for (int u = 0; u < VLD; ++u) {
      const int rr = u * (1024 / ROWB) + lane / LPRW;
      *(lds_u32x4_t*)(kt + rr * KPITCH + (lane % LPRW) * 16) = __builtin_bit_cast(u32x4_t, kl[u]);
    }
    wave_lds_sync();
    uint4 kr[2][KC];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int kc = 0; kc < KC; ++kc)
        kr[mb][kc] = __builtin_bit_cast(
            uint4, *(lds_u32x4_t*)(kt + (16 * mb + col) * KPITCH + kc * 64 + q4 * 16));
    // Scores S^T = K Q^T: lane holds keys 16*mb + 4*q4 + r of head col.
    f32x4 s[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      s[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < KC; ++kc) s[mb] = M::mma(kr[mb][kc], qb[kc], s[mb]);
    }
    // V tile: 1 KiB contiguous per wave load, issued once the K tile is in
    // LDS, so it streams while the softmax of this tile runs.  (Issuing it
    // with the K loads was 5% slower on the LLaMA-3.1-70B layer at its
    // planned two splits, four workgroups per CU.)
    uint4 vr[VLD];
#pragma unroll
    for (int u = 0; u < VLD; ++u) {
      int row = base + u * (1024 / ROWB) + lane / LPRW;
      if (!full) row = min(row, ke - 1);
      vr[u] = ld16_stream(rows.v(row) + (lane % LPRW) * 16);
    }
    float sc[8];
    float tmax = kNegInf;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = s[mb][r] * a.scale_log2;
        if (!full && base + 16 * mb + 4 * q4 + r >= ke) x = kNegInf;
        sc[mb * 4 + r] = x;
        tmax = fmaxf(tmax, x);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (tmax > m + kRescaleSlack) {
      const float alpha = exp2_hw(m - tmax);  // 0 on the first tile
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < DB; ++i) acc[i] *= alpha;
      m = tmax;
    }
    const float mu = (m == kNegInf) ? 0.f : m;
    float p[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2_hw(sc[e] - mu);
      lsum += p[e];
    }
    uint4 phi, plo;
    split_pack<DT>(p, phi, plo);

    // V tile to LDS (padded rows), then transposed reads feed the PV product.
#pragma unroll
    for (int u = 0; u < VLD; ++u) {
      const int rr = u * (1024 / ROWB) + lane / LPRW;
      *(lds_u32x4_t*)(vt + rr * PITCH + (lane % LPRW) * 16) = __builtin_bit_cast(u32x4_t, vr[u]);
    }
    wave_lds_sync();
    const int trow = 4 * q4 + (col >> 2);
    const int tcol = (col & 3) * 8;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const uint2 x0 = M::tr_read(vt + trow * PITCH + db * 32 + tcol);
      const uint2 x1 = M::tr_read(vt + (16 + trow) * PITCH + db * 32 + tcol);
      const uint4 va = make_uint4(x0.x, x0.y, x1.x, x1.y);
      acc[db] = M::mma(va, phi, acc[db]);
      acc[db] = M::mma(va, plo, acc[db]);
    }
  }

  // Per-head sums over the four lanes that share a head column.
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);

  // Partial O^T of this wave into its own LDS buffer: [head][d] with rows
  // PO floats apart (PO = 4 mod 64 words: the 16 heads of a 128-bit write
  // pass fall on distinct banks), then (m, l).
  lds_float_t* po = (lds_float_t*)(vt);
  lds_float_t* pml = po + kCols * PO;
#pragma unroll
  for (int db = 0; db < DB; ++db)
    *(lds_f32x4_t*)(po + col * PO + db * 16 + 4 * q4) = acc[db];
  if (q4 == 0) {
    pml[2 * col] = m;
    pml[2 * col + 1] = lsum;
  }
  __syncthreads();

  // Merge the waves: one output element per thread.
  for (int e = tid; e < nh * D; e += WAVES * 64) {
    const int j = e / D, c = e % D;
    float Mx = kNegInf;
#pragma unroll
    for (int w = 0; w < WAVES; ++w)
      Mx = fmaxf(Mx, ((const lds_float_t*)(sbase + w * VBUF))[kCols * PO + 2 * j]);
    const float Mu = (Mx == kNegInf) ? 0.f : Mx;
    float L = 0.f, accv = 0.f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      const lds_float_t* pw = (const lds_float_t*)(sbase + w * VBUF);
      const float wt = exp2_hw(pw[kCols * PO + 2 * j] - Mu);
      L += wt * pw[kCols * PO + 2 * j + 1];
      accv += wt * pw[j * PO + c];
    }
    const int h = g * a.G + head0 + j;
    if (a.nsplit == 1) {
      Elem<DT>::store(a.o, (static_cast<size_t>(b) * a.H + h) * D + c, L > 0.f ? accv / L : 0.f);
    } else {
      const size_t pi = (static_cast<size_t>(unit) * a.G + head0 + j) * a.nsplit + split;
      a.part_o[pi * D + c] = accv;
      if (c == 0) {
        a.part_ml[2 * pi] = Mx;
        a.part_ml[2 * pi + 1] = L;
      }
    }
  }
}

template <int DT, int D, int WAVES>
hipError_t launch_t(const Args& a, hipStream_t st) {
  const unsigned nchunk = (a.G + kCols - 1) / kCols;
  const dim3 grid(static_cast<unsigned>(a.B) * a.top_k * nchunk * a.nsplit), block(WAVES * 64);
  if (a.layout == kKvStrided)
    hipLaunchKernelGGL((sha_decode_gqa_mfma_kernel<DT, D, WAVES, kKvStrided>), grid, block, 0, st, a);
  else if (a.layout == kKvPaged)
    hipLaunchKernelGGL((sha_decode_gqa_mfma_kernel<DT, D, WAVES, kKvPaged>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((sha_decode_gqa_mfma_kernel<DT, D, WAVES, kKvContig>), grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && a.nsplit > 1) e = launch_combine(a, DT, D, 1, st);
  return e;
}

template <int DT, int D>
hipError_t launch_w(const Args& a, hipStream_t st) {
  return a.waves == 2 ? launch_t<DT, D, 2>(a, st) : launch_t<DT, D, 4>(a, st);
}

}  // namespace

hipError_t launch_gqa_mfma(const Args& a, int dtype, int d, hipStream_t st) {
  if (dtype == kF16) return d == 64 ? launch_w<kF16, 64>(a, st) : launch_w<kF16, 128>(a, st);
  return d == 64 ? launch_w<kBF16, 64>(a, st) : launch_w<kBF16, 128>(a, st);
}

}  // namespace sha
