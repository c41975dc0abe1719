// Selective MLP ("Selective GEMM") of Polar Sparsity on gfx950.
//
// papernotes.org notes on Polar Sparsity, 方法详解 > 关键设计 > "MLP 层动态稀疏":
// for a decode batch x [B, d], MLP_{S_B}(x) = sigma(x W1[:, S_B]) W2[:, S_B]^T
// where S_B is the union over the batch of every row's active neurons, and
// the indexing is fused into the matrix products (no gather/scatter pass).
// sigma is ReLU (the selective MLP is applied to OPT models).  Weights are
// stored neuron-major: w1t = W1^T and w2t = W2^T, both [D, d], so a selected
// neuron is one contiguous row of each.
//
// Kernels:
//   union  - a flag byte per neuron in a workspace: cleared, marked by every
//            row's entries (plain byte stores, any order gives the same flags),
//            then every 4096-flag block counts the flags before it (its
//            output offset), writes its marked neurons in ascending order,
//            and the last block writes the total (deterministic, on device).
//   up     - H^T = W1t[S] x^T on MFMA (v_mfma_f32_16x16x32, 16-bit inputs):
//            a workgroup owns 128 selected neurons x 64 batch rows over a K
//            range; weight rows stream in 256-byte runs (non-temporal
//            128-bit loads, two stages ahead) through swizzled LDS into A
//            operands, x pieces come from L2 as B operands.  With one K
//            split it applies ReLU and writes H (16-bit); with several it
//            writes fp32 partials and `up_finalize` sums them.
//   down   - y = H W2t[S] on MFMA: a workgroup owns 64 batch rows x 256
//            output columns over a range of the selected neurons; the
//            gathered W2t rows are staged in LDS and read back transposed
//            (ds_read_b64_tr_b16) as B operands, H comes from LDS as A.
//            Split ranges of neurons write fp32 partials that
//            `down_finalize` sums in a fixed order.
// The selection count is read on the device, so union -> up -> down needs no
// host synchronisation; grids are sized for the caller's upper bound n_max
// and workgroups past the actual count exit or mask.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "sha_device.h"
#include "sha_launch.h"

namespace sha {
namespace {

using namespace detail;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __fp16 fp16x4_vs_t __attribute__((__vector_size__(4 * sizeof(__fp16))));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) u32x4_t lds_u32x4_t;
typedef __attribute__((address_space(3))) u32x2_t lds_u32x2_t;
typedef __attribute__((address_space(3))) uint32_t lds_u32_t;
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) fp16x4_vs_t lds_f16x4_t;

template <int DT>
struct Mx;

template <>
struct Mx<kBF16> {
  __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static uint2 tr_read(const lds_char_t* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)(p)));
  }
  __device__ static uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, bf16x2_t));
  }
};

template <>
struct Mx<kF16> {
  __device__ static f32x4 mma(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static uint2 tr_read(const lds_char_t* p) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_f16x4_t*)(p)));
  }
  __device__ static uint32_t pack(float x, float y) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x, y}, f16x2_t));
  }
};

// ---------------------------------------------------------------------------
// union of the rows' neuron lists: one flag byte per neuron in a workspace
// ---------------------------------------------------------------------------
// flags[0 .. D) = 0 (16-byte stores; the flag buffer is padded to 256 bytes).
__global__ __launch_bounds__(256) void sha_mlp_union_clear_kernel(uint8_t* flags, int D) {
  const int n16 = (D + 15) / 16;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n16; i += gridDim.x * 256)
    reinterpret_cast<uint4*>(flags)[i] = make_uint4(0, 0, 0, 0);
}

// flags[j] = 1 for every entry j in [0, D).  Concurrent stores of the same
// value to one byte need no atomics and leave the same result in any order.
__global__ __launch_bounds__(256) void sha_mlp_union_mark_kernel(const int32_t* rows, int total,
                                                                 int D, uint8_t* flags) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256) {
    const int j = rows[i];
    if (j >= 0 && j < D) flags[j] = 1;
  }
}

// Compaction in one launch over blocks of kUnionBlockFlags flags (one
// 16-flag word per thread): a block counts the set flags of all the blocks
// before its own (its output offset; at most D bytes, read from L2), scans
// its words, gathers its neurons in LDS in ascending order and copies them
// out with contiguous stores; the last block also stores the total.
constexpr int kUnionBlockFlags = 4096;
constexpr int kUnionBlockThreads = kUnionBlockFlags / 16;

__device__ __forceinline__ uint32_t flag_count(uint4 f) {
  return __popc(f.x & 0x01010101u) + __popc(f.y & 0x01010101u) + __popc(f.z & 0x01010101u) +
         __popc(f.w & 0x01010101u);
}

// Inclusive sum over the workgroup's threads (kUnionBlockThreads = 4 waves).
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wave_sums, uint32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(v, off);
    if (lane >= off) v += u;
  }
  if (lane == 63) wave_sums[wave] = v;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int q = 0; q < kUnionBlockThreads / 64; ++q) {
    const uint32_t ws = wave_sums[q];
    if (q < wave) before += ws;
    all += ws;
  }
  *total = all;
  return v + before;
}

__global__ __launch_bounds__(kUnionBlockThreads) void sha_mlp_union_write_kernel(
    const uint8_t* flags, int D, int32_t* sel, int32_t* n_sel) {
  __shared__ uint32_t wave_sums[kUnionBlockThreads / 64];
  __shared__ int32_t staged[kUnionBlockFlags];
  __shared__ uint32_t base_sh;
  const int tid = threadIdx.x;
  const uint4* fw = reinterpret_cast<const uint4*>(flags);
  // Output offset of this block: the set flags of the blocks before it.
  uint32_t part = 0;
  const int words_before = static_cast<int>(blockIdx.x) * kUnionBlockThreads;
  for (int q = tid; q < words_before; q += kUnionBlockThreads) part += flag_count(fw[q]);
  uint32_t base;
  block_scan(part, wave_sums, &base);
  if (tid == 0) base_sh = base;
  __syncthreads();  // wave_sums is reused below
  base = base_sh;

  const int word = words_before + tid;
  const int n16 = (D + 15) / 16;   // flags past D in the last word are cleared zeros
  const uint4 f = word < n16 ? fw[word] : make_uint4(0, 0, 0, 0);
  const uint32_t cnt = flag_count(f);
  uint32_t n_block;
  uint32_t pos = block_scan(cnt, wave_sums, &n_block) - cnt;
  const uint32_t w[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((w[q] >> (8 * e)) & 1u) staged[pos++] = word * 16 + 4 * q + e;
  __syncthreads();
  for (uint32_t i = tid; i < n_block; i += kUnionBlockThreads) sel[base + i] = staged[i];
  if (blockIdx.x == gridDim.x - 1 && tid == 0) *n_sel = static_cast<int32_t>(base + n_block);
}

// ---------------------------------------------------------------------------
// up projection: H = relu(x W1t[S]^T)
// ---------------------------------------------------------------------------
__device__ __forceinline__ int sel_count(const MlpArgs& a) {
  const int n = *a.n_sel;
  return n < 0 ? 0 : (n > a.n_max ? a.n_max : n);
}

// Weight row of selection entry n (< count); entries outside [0, D) read row 0
// and are zeroed where their activation is produced.
__device__ __forceinline__ int sel_row(const MlpArgs& a, int n) {
  const int r = a.sel[n];
  return (r >= 0 && r < a.D) ? r : 0;
}
__device__ __forceinline__ bool sel_valid(const MlpArgs& a, int n, int count) {
  if (n >= count) return false;
  const int r = a.sel[n];
  return r >= 0 && r < a.D;
}

// A workgroup owns kUpN = 128 selected neurons x 64 batch rows over a K
// range, in stages of kUpKc = 128 k.  Each stage's weights (128 rows x
// 256 B) are read with 128-bit non-temporal loads, four rows of 256
// contiguous bytes per wave instruction, three stages ahead of their use
// (two register sets: a set is reloaded as soon as it is written to LDS),
// and written one stage ahead into a double-buffered LDS tile with an XOR
// swizzle of the 16-byte pieces (slot = piece ^ (row & 15)), so that the
// A-operand reads (16 rows x one piece per quarter wave) hit distinct banks;
// one barrier per stage both publishes the next tile and retires the one
// just read.  Wave w multiplies all 128 neurons by batch block w: its x
// pieces (B operands) come from L2 into registers one stage ahead, and no two
// waves read the same x.  Every x byte read serves 128 neurons: x comes from
// L2 at half the weight bytes (at 64 neurons per workgroup it matched them
// and cost about a fifth of the kernel's time).  Each step issues its x
// loads before its weight loads: waiting for a stage's x then leaves the
// younger weight stages in flight (loads complete in order).
// Workgroup id = ((btile * up_splits) + split) * nblocks + nblock.
constexpr int kUpN = kMlpUpNeurons;         // neurons per workgroup
constexpr int kUpNB = kUpN / 16;            // MFMA neuron blocks
constexpr int kUpKc = kMlpUpKc;             // k per stage
constexpr int kUpRowB = kUpKc * 2;          // bytes of one weight row per stage
constexpr int kUpPieces = kUpRowB / 16;     // 16-byte pieces per row per stage
constexpr int kUpLoads = kUpN * kUpPieces / 256;  // weight pieces per thread per stage
constexpr int kUpX = kUpKc / 32;            // x pieces (MFMA K steps) per lane per stage
static_assert(kUpPieces == 16, "the swizzle and the row mapping assume 16 pieces per row");

struct UpW {
  uint4 v[kUpLoads];
};
struct UpX {
  uint4 v[kUpX];
};

template <int DT>
__global__ __launch_bounds__(256, 2) void sha_mlp_up_kernel(MlpArgs a) {
  using M = Mx<DT>;
  __shared__ __attribute__((aligned(16))) char wsm_[2 * kUpN * kUpRowB];
  const int nblocks = a.n_pad / kUpN;
  int t = blockIdx.x;
  const int nblk = t % nblocks;
  t /= nblocks;
  const int split = t % a.up_splits;
  const int btile = t / a.up_splits;
  const int n_sel = sel_count(a);
  const int n0 = nblk * kUpN;
  if (n0 >= n_sel) return;                    // whole workgroup: past the selection
  const int b0 = btile * 64;
  const int kbeg = split * a.up_kper;
  const int kend = min(kbeg + a.up_kper, a.d);
  const int nst = kend > kbeg ? (kend - kbeg) / kUpKc : 0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, c = lane & 15;
  lds_char_t* const wl = (lds_char_t*)(wsm_);

  // Weight pieces of this thread: piece index p = tid + 256 i -> row p >> 4
  // (= (tid >> 4) + 16 i), 16-byte column p & 15; 32-bit byte offsets of the
  // rows (one weight matrix is below 4 GiB, checked on the host) and the LDS
  // slot of each piece.
  const char* w1 = static_cast<const char*>(a.w1t) + static_cast<size_t>(kbeg) * 2;
  uint32_t woff[kUpLoads];
  int wdst[kUpLoads];
#pragma unroll
  for (int i = 0; i < kUpLoads; ++i) {
    const int r = (tid >> 4) + 16 * i, col = tid & 15;
    const int row = sel_row(a, min(n0 + r, n_sel - 1));
    woff[i] = static_cast<uint32_t>(row) * static_cast<uint32_t>(a.d) * 2u + col * 16;
    wdst[i] = r * kUpRowB + ((col ^ (r & 15)) * 16);
  }
  // x row of this lane.  Padding rows past B read row B - 1: their H rows
  // are finite and no output row reads them (the down projection stores only
  // rows < B), so x is not masked (a mask applied to freshly loaded x made
  // the wave wait for the weight loads in flight before it).
  const int b = b0 + 16 * wave + c;
  const bool xok = b < a.B;
  const char* xsrc = static_cast<const char*>(a.x) +
                     (static_cast<size_t>(xok ? b : a.B - 1) * a.d + kbeg + 8 * q4) * 2;

  f32x4 acc[kUpNB];  // [neuron block]; batch block = wave
#pragma unroll
  for (int i = 0; i < kUpNB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_w = [&](int st, UpW& d) {
#pragma unroll
    for (int i = 0; i < kUpLoads; ++i) d.v[i] = ld16_stream(w1 + woff[i] + st * kUpRowB);
  };
  auto load_x = [&](int st, UpX& d) {
#pragma unroll
    for (int s = 0; s < kUpX; ++s) d.v[s] = ld16(xsrc + st * kUpRowB + s * 64);
  };
  auto write_w = [&](int st, const UpW& w) {
    lds_char_t* const buf = wl + (st & 1) * (kUpN * kUpRowB);
#pragma unroll
    for (int i = 0; i < kUpLoads; ++i)
      *(lds_u32x4_t*)(buf + wdst[i]) = __builtin_bit_cast(u32x4_t, w.v[i]);
  };
  // Step st: the weights of st + 1 go from registers to LDS, which frees
  // their register set for the weights of st + 3; x of st + 1 goes out
  // first; stage st is multiplied; one barrier closes the step (CHECK: only
  // work inside the K range).  Weights of stage j live in set j % 2, x of
  // stage j in x set j % 2.
  auto step = [&](int st, UpW& wnext, UpX& xcur, UpX& xnext, auto check) {
    constexpr bool C = decltype(check)::value;
    if (!C || st + 1 < nst) write_w(st + 1, wnext);
    if (!C || st + 1 < nst) load_x(st + 1, xnext);
    // x before the weights, as written: the scheduler may otherwise sink the
    // x loads below them, and the next step's wait for x would then wait for
    // the weights as well.
    __builtin_amdgcn_sched_barrier(0);
    if (!C || st + 3 < nst) load_w(st + 3, wnext);
    const lds_char_t* const buf = wl + (st & 1) * (kUpN * kUpRowB);
#pragma unroll
    for (int s = 0; s < kUpX; ++s) {
      const uint4 xv = xcur.v[s];
      const uint4 xb = xv;
      const int piece = 4 * s + q4;         // 16-byte piece of the row this lane reads
#pragma unroll
      for (int mb = 0; mb < kUpNB; ++mb) {
        const u32x4_t av = *(const lds_u32x4_t*)(buf + (16 * mb + c) * kUpRowB + ((piece ^ c) * 16));
        acc[mb] = M::mma(__builtin_bit_cast(uint4, av), xb, acc[mb]);
      }
    }
    __syncthreads();
  };

  if (nst > 0) {
    // The prologue loads the same sets on every path into the loop (short
    // ranges load their last stage again): with conditional loads here the
    // compiler cannot tell which loads are still in flight at the loop head
    // and waits for all of them there, once per pass.
    UpW wa, wb;
    UpX x0, x1;
    load_x(0, x0);
    load_w(0, wa);
    load_w(min(1, nst - 1), wb);
    write_w(0, wa);
    load_w(min(2, nst - 1), wa);
    __syncthreads();
    // Two steps per pass; passes whose look-ahead work all lies inside the K
    // range run without checks.
    using Chk = std::true_type;
    using NoChk = std::false_type;
    int st = 0;
    for (; st + 5 <= nst; st += 2) {
      step(st, wb, x0, x1, NoChk{});
      step(st + 1, wa, x1, x0, NoChk{});
    }
    for (; st + 2 <= nst; st += 2) {
      step(st, wb, x0, x1, Chk{});
      step(st + 1, wa, x1, x0, Chk{});
    }
    if (st < nst) step(st, wb, x0, x1, Chk{});
  }

  // lane holds H^T[n = n0 + 16 mb + 4 q4 + r][b] (b < b_pad)
#pragma unroll
  for (int mb = 0; mb < kUpNB; ++mb) {
    const int nbase = n0 + 16 * mb + 4 * q4;
    // Entries outside [0, D) (and past the count) produce no activation.
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (!sel_valid(a, nbase + r, n_sel)) acc[mb][r] = 0.f;
    if (a.up_splits == 1) {
      const uint32_t lo = M::pack(fmaxf(acc[mb][0], 0.f), fmaxf(acc[mb][1], 0.f));
      const uint32_t hi = M::pack(fmaxf(acc[mb][2], 0.f), fmaxf(acc[mb][3], 0.f));
      *reinterpret_cast<uint2*>(static_cast<char*>(a.h) +
                                (static_cast<size_t>(b) * a.n_pad + nbase) * 2) = make_uint2(lo, hi);
    } else {
      float* p = a.up_part + (static_cast<size_t>(split) * a.b_pad + b) * a.n_pad + nbase;
      *reinterpret_cast<float4*>(p) = make_float4(acc[mb][0], acc[mb][1], acc[mb][2], acc[mb][3]);
    }
  }
}

// H = relu(sum of the K-split partials), fixed order; one thread per 4 neurons.
template <int DT>
__global__ __launch_bounds__(256) void sha_mlp_up_finalize_kernel(MlpArgs a) {
  using M = Mx<DT>;
  const int n_sel = sel_count(a);
  const size_t quads = static_cast<size_t>(a.b_pad) * (a.n_pad / 4);
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < quads; i += static_cast<size_t>(gridDim.x) * 256) {
    const size_t b = i / (a.n_pad / 4);
    const int n4 = static_cast<int>(i % (a.n_pad / 4)) * 4;
    if (n4 >= n_sel) continue;
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < a.up_splits; ++sp) {
      const float4 v = *reinterpret_cast<const float4*>(
          a.up_part + (static_cast<size_t>(sp) * a.b_pad + b) * a.n_pad + n4);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const uint32_t lo = M::pack(fmaxf(s.x, 0.f), fmaxf(s.y, 0.f));
    const uint32_t hi = M::pack(fmaxf(s.z, 0.f), fmaxf(s.w, 0.f));
    *reinterpret_cast<uint2*>(static_cast<char*>(a.h) + (b * a.n_pad + n4) * 2) = make_uint2(lo, hi);
  }
}

// ---------------------------------------------------------------------------
// down projection: y = H W2t[S]
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;                    // accelerator dies (XCDs) of MI355X
constexpr int kDnKc = 64;                   // neurons per LDS chunk (2 MFMA K steps)
constexpr int kDnCols = 256;                // output columns per workgroup
constexpr int kDnWPitch = kDnCols * 2 + 32; // 544 B: conflict-free transposed reads
constexpr int kDnHPitch = kDnKc * 2 + 16;   // 144 B: conflict-free H reads

// Two workgroups per CU (the planner's assumption): the register budget is
// held at 256 per lane, accumulators included.
template <int DT>
__global__ __launch_bounds__(256, 2) void sha_mlp_down_kernel(MlpArgs a) {
  using M = Mx<DT>;
  __shared__ __attribute__((aligned(16))) char ws_[kDnKc * kDnWPitch];
  __shared__ __attribute__((aligned(16))) char hs_[64 * kDnHPitch];
  const int n_sel = sel_count(a);
  // Workgroup -> (column block, neuron split, batch tile), XCD-aware.  The
  // dispatcher deals workgroups to the 8 XCDs in turn (id mod 8); each XCD
  // is given a contiguous run of the split-major item list instead, so the
  // workgroups on one XCD share a few neuron splits and the H slices those
  // read stay in that XCD's L2 (with the plain order every XCD would read
  // all of H, more than its L2 holds).
  const int ncol = a.d / kDnCols;
  const int nitems = static_cast<int>(gridDim.x);  // ncol * dn_splits * batch tiles
  const int L = blockIdx.x, xcd = L % kXcds, slot = L / kXcds;
  const int q8 = nitems / kXcds, r8 = nitems % kXcds;
  const int item = xcd * q8 + min(xcd, r8) + slot;  // a bijection of [0, nitems)
  const int col0 = (item % ncol) * kDnCols;
  const int split = (item / ncol) % a.dn_splits;
  const int b0 = (item / (ncol * a.dn_splits)) * 64;
  // This split's neuron range (whole MFMA K steps).
  const int per = ((n_sel + a.dn_splits - 1) / a.dn_splits + 31) / 32 * 32;
  const int nbeg = min(split * per, n_sel);
  const int nend = min(nbeg + per, n_sel);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, c = lane & 15;
  lds_char_t* const wl = (lds_char_t*)(ws_);
  lds_char_t* const hl = (lds_char_t*)(hs_);

  f32x4 acc[4][4];  // [m block (batch)][n block (columns)]
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Gathered W2t rows of a chunk: 64 rows x 512 B = 2048 pieces (8 per
  // thread); H chunk: 64 rows x 128 B = 512 pieces (2 per thread), neurons at
  // or past nend read as zero.  Piece tid + 256 i of the weights is row
  // 2 wave + (lane >> 5) + 8 i, so each load instruction needs two selection
  // entries that are the same for the whole wave: they are read with scalar
  // loads (own counter), and the vector loads of earlier chunks need not
  // complete before the next chunk's addresses are known.  H pieces are read
  // unconditionally (offsets clamped inside the row) and masked only when
  // they are written to LDS: masking at load time would make the wave wait
  // for them, and (loads complete in order) for every older load, at once.
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const bool upper = lane >= 32;
  auto load_chunk = [&](int k0, uint4 (&wv)[8], uint4 (&hv)[2]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r0 = k0 + 2 * wu + 8 * i;
      const int s0 = a.sel[min(r0, nend - 1)], s1 = a.sel[min(r0 + 1, nend - 1)];
      const int row0 = (s0 >= 0 && s0 < a.D) ? s0 : 0, row1 = (s1 >= 0 && s1 < a.D) ? s1 : 0;
      const int row = upper ? row1 : row0;
      wv[i] = ld16_stream(static_cast<const char*>(a.w2t) +
                          (static_cast<size_t>(row) * a.d + col0 + (lane & 31) * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 3, piece = idx & 7;
      const int nc = min(k0 + piece * 8, a.n_pad - 8);  // past n_pad: past nend, masked
      hv[i] = ld16(static_cast<const char*>(a.h) +
                   (static_cast<size_t>(b0 + r) * a.n_pad + nc) * 2);
    }
  };

  // Chunk j (neurons nbeg + 64 j ..) lives in register set j % 2.  Step j:
  // wait for the previous chunk's LDS reads, write chunk j to LDS, reload its
  // set with chunk j + 2 (two chunks in flight during the products), publish
  // and multiply.  CHECK: only load inside the range.
  const int nch = nend > nbeg ? (nend - nbeg + kDnKc - 1) / kDnKc : 0;
  auto step = [&](int j, uint4 (&w)[8], uint4 (&h)[2], auto check) {
    constexpr bool C = decltype(check)::value;
    __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 5, piece = idx & 31;
      *(lds_u32x4_t*)(wl + r * kDnWPitch + piece * 16) = __builtin_bit_cast(u32x4_t, w[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 256 * i;
      const int r = idx >> 3, piece = idx & 7;
      const int cnt = min(max(nend - (nbeg + j * kDnKc + piece * 8), 0), 8);  // valid neurons
      uint32_t m[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        m[e] = (2 * e < cnt ? 0x0000FFFFu : 0u) | (2 * e + 1 < cnt ? 0xFFFF0000u : 0u);
      const u32x4_t hm = {h[i].x & m[0], h[i].y & m[1], h[i].z & m[2], h[i].w & m[3]};
      *(lds_u32x4_t*)(hl + r * kDnHPitch + piece * 16) = hm;
    }
    if (!C || j + 2 < nch) load_chunk(nbeg + (j + 2) * kDnKc, w, h);
    // Keep the loads ahead of the products: the scheduler would otherwise
    // spread them among the MFMAs and wait for them there.
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kDnKc / 32; ++ks) {
      // K-slot order of a 32-neuron step: lane group q4 owns neurons
      // 4q4 .. 4q4+3 and 16+4q4 .. 16+4q4+3 of the step.
      uint4 ha[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const lds_char_t* hr = hl + (16 * mb + c) * kDnHPitch + ks * 64;
        const u32x2_t p0 = *(const lds_u32x2_t*)(hr + 8 * q4);
        const u32x2_t p1 = *(const lds_u32x2_t*)(hr + 32 + 8 * q4);
        ha[mb] = make_uint4(p0.x, p0.y, p1.x, p1.y);
      }
      const int trow = ks * 32 + 4 * q4 + (c >> 2);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int cb = (64 * wave + 16 * nb) * 2 + (c & 3) * 8;
        const uint2 x0 = M::tr_read(wl + trow * kDnWPitch + cb);
        const uint2 x1 = M::tr_read(wl + (trow + 16) * kDnWPitch + cb);
        const uint4 wb = make_uint4(x0.x, x0.y, x1.x, x1.y);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb][nb] = M::mma(ha[mb], wb, acc[mb][nb]);
      }
    }
  };

  if (nch > 0) {
    // Both sets are loaded on every path into the loop (a one-chunk range
    // loads its chunk twice), so the compiler sees the same loads in flight
    // at the loop head from the entry and from the back edge and can leave
    // the younger set in flight; a conditional second load makes it wait
    // for everything there.
    uint4 wa[8], ha0[2], wb8[8], hb0[2];
    load_chunk(nbeg, wa, ha0);
    load_chunk(nbeg + min(1, nch - 1) * kDnKc, wb8, hb0);
    using Chk = std::true_type;
    using NoChk = std::false_type;
    int j = 0;
    for (; j + 4 <= nch; j += 2) {
      step(j, wa, ha0, NoChk{});
      step(j + 1, wb8, hb0, NoChk{});
    }
    for (; j + 2 <= nch; j += 2) {
      step(j, wa, ha0, Chk{});
      step(j + 1, wb8, hb0, Chk{});
    }
    if (j < nch) step(j, wa, ha0, Chk{});
  }

  // lane holds y[b = b0 + 16 mb + 4 q4 + r][col = col0 + 64 wave + 16 nb + c]
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int b = b0 + 16 * mb + 4 * q4 + r;
      if (b >= a.B) continue;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int col = col0 + 64 * wave + 16 * nb + c;
        if (a.dn_splits == 1)
          Elem<DT>::store(a.y, static_cast<size_t>(b) * a.d + col, acc[mb][nb][r]);
        else
          a.dn_part[(static_cast<size_t>(split) * a.b_pad + b) * a.d + col] = acc[mb][nb][r];
      }
    }
}

// y = sum of the neuron-split partials, fixed order; one thread per 4
// consecutive columns (d is a multiple of 256).
template <int DT>
__global__ __launch_bounds__(256) void sha_mlp_down_finalize_kernel(MlpArgs a) {
  const size_t quads = static_cast<size_t>(a.B) * (a.d / 4);
  const size_t plane = static_cast<size_t>(a.b_pad) * a.d;
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < quads; i += static_cast<size_t>(gridDim.x) * 256) {
    const float4* p = reinterpret_cast<const float4*>(a.dn_part) + i;  // row-major [b][d] of plane 0
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp = 0; sp < a.dn_splits; ++sp) {
      const float4 v = p[sp * (plane / 4)];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    const size_t e = i * 4;
    Elem<DT>::store(a.y, e, s.x);
    Elem<DT>::store(a.y, e + 1, s.y);
    Elem<DT>::store(a.y, e + 2, s.z);
    Elem<DT>::store(a.y, e + 3, s.w);
  }
}

template <int DT>
hipError_t launch_mlp_t(const MlpArgs& a, hipStream_t st) {
  const unsigned btiles = static_cast<unsigned>(a.b_pad / 64);
  const long long up_wgs = static_cast<long long>(a.n_pad / kUpN) * a.up_splits * btiles;
  hipLaunchKernelGGL((sha_mlp_up_kernel<DT>), dim3(static_cast<unsigned>(up_wgs)), dim3(256), 0,
                     st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.up_splits > 1) {
    const size_t quads = static_cast<size_t>(a.b_pad) * (a.n_pad / 4);
    const unsigned blocks = static_cast<unsigned>(quads < 256 * 1024 ? (quads + 255) / 256 : 1024);
    hipLaunchKernelGGL((sha_mlp_up_finalize_kernel<DT>), dim3(blocks), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 1-D over (column block, split, batch tile): the kernel maps the ids
  // onto XCDs itself.
  hipLaunchKernelGGL((sha_mlp_down_kernel<DT>),
                     dim3(static_cast<unsigned>((a.d / kDnCols) * a.dn_splits) * btiles),
                     dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.dn_splits > 1) {
    const size_t total = static_cast<size_t>(a.B) * (a.d / 4);
    const unsigned blocks = static_cast<unsigned>(total < 256 * 2048 ? (total + 255) / 256 : 2048);
    hipLaunchKernelGGL((sha_mlp_down_finalize_kernel<DT>), dim3(blocks), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

int mlp_union_blocks(int D) { return (D + kUnionBlockFlags - 1) / kUnionBlockFlags; }

hipError_t launch_mlp_union(const int32_t* rows, int total, int D, int32_t* sel, int32_t* n_sel,
                            uint8_t* flags, hipStream_t st) {
  const int n16 = (D + 15) / 16;
  hipLaunchKernelGGL(sha_mlp_union_clear_kernel, dim3(min((n16 + 255) / 256, 1024)), dim3(256), 0,
                     st, flags, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (total > 0) {
    hipLaunchKernelGGL(sha_mlp_union_mark_kernel, dim3(min((total + 255) / 256, 2048)), dim3(256),
                       0, st, rows, total, D, flags);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(sha_mlp_union_write_kernel, dim3(mlp_union_blocks(D)),
                     dim3(kUnionBlockThreads), 0, st, flags, D, sel, n_sel);
  return hipGetLastError();
}

hipError_t launch_selective_mlp(const MlpArgs& a, int dtype, hipStream_t st) {
  return dtype == kF16 ? launch_mlp_t<kF16>(a, st) : launch_mlp_t<kBF16>(a, st);
}


}  // namespace sha
