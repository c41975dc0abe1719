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
//            Up to 8192 row entries, one workgroup does all of it with the
//            flags as LDS bits (one launch).
//   up     - H^T = W1t[S] x^T on MFMA (v_mfma_f32_16x16x32, 16-bit inputs):
//            a workgroup owns 128 selected neurons (144 for full batch
//            tiles when that makes whole rounds of resident workgroups) x
//            64 batch rows over a K range; weight rows stream in 256-byte
//            runs (non-temporal 128-bit loads, three stages ahead) through
//            swizzled LDS into A operands, x pieces come from L2 as B
//            operands.  With one K split it applies ReLU and writes H
//            (16-bit); with several it writes fp32 partials and
//            `up_finalize` sums them.  Full batch tiles whose grid is about
//            one round at one workgroup per CU take 512 threads in two K
//            groups instead of K splits: the halves of K are summed on chip.
//   down   - y = H W2t[S] on MFMA: a workgroup of 8 waves owns 64 batch
//            rows x 512 output columns (4 waves x 256 columns when d is not
//            a multiple of 512) over a range of the selected neurons; the
//            gathered W2t rows are staged in LDS and read back transposed
//            (ds_read_b64_tr_b16) as B operands, H comes from LDS as A.
//            Split ranges of neurons write fp32 partials that
//            `down_finalize` sums in a fixed order.  For one or two batch
//            blocks with 2-4 up K splits it sums the up partials itself as
//            it loads H (the up finalize's arithmetic; no finalize launch).
//   Batches of at most 16 (32) rows compute only the 1 (2) batch blocks of
//   16 rows that hold rows: in the up projection the waves then split the
//   tile's neurons instead of its batch blocks, and the waves sharing a
//   batch block share its x through LDS (`sha_mlp_upx_kernel`).
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
typedef __attribute__((address_space(3))) float lds_float_t;
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
  // Output offset of this block: the set flags of the blocks before it,
  // read eight words per thread at a time (unconditional loads, clamped to
  // the last word before the block, all eight in flight, then counted where
  // in range), so a late block waits for memory once per eight blocks
  // before it rather than once per block.
  uint32_t part = 0;
  const int words_before = static_cast<int>(blockIdx.x) * kUnionBlockThreads;
  for (int q0 = tid; q0 < words_before; q0 += 8 * kUnionBlockThreads) {
    uint4 f[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) f[u] = fw[min(q0 + u * kUnionBlockThreads, words_before - 1)];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      part += q0 + u * kUnionBlockThreads < words_before ? flag_count(f[u]) : 0u;
  }
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

// Small unions in one launch: one 1024-thread workgroup keeps a bit per
// neuron in LDS (cleared, then set by every row entry with LDS atomic ors,
// eight entries per thread in flight), then each thread counts the bits of
// its run of words, a workgroup scan gives its output offset, and it writes
// its neurons in ascending order; the last thread writes the total.  Used
// for at most kSmallUnionMaxTotal entries and kSmallUnionMaxD neurons (one
// workgroup reads every entry); it needs no workspace and gives the same
// sel and count as the three kernels above.
constexpr int kSmallUnionThreads = 1024;
constexpr int kSmallUnionMaxD = 1 << 18;       // 32 KiB of LDS bits
constexpr int kSmallUnionMaxTotal = 1 << 13;   // past ~8K entries the three kernels win

__global__ __launch_bounds__(kSmallUnionThreads) void sha_mlp_union_small_kernel(
    const int32_t* rows, int total, int D, int32_t* sel, int32_t* n_sel) {
  __shared__ uint32_t bits[kSmallUnionMaxD / 32];
  __shared__ uint32_t wave_sums[kSmallUnionThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = (D + 31) / 32;
  for (int w = tid; w < nw; w += kSmallUnionThreads) bits[w] = 0u;
  __syncthreads();
  for (int i0 = 0; i0 < total; i0 += 8 * kSmallUnionThreads) {
    int j[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kSmallUnionThreads + tid;
      j[u] = i < total ? rows[i] : -1;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (j[u] >= 0 && j[u] < D) atomicOr(&bits[j[u] >> 5], 1u << (j[u] & 31));
  }
  __syncthreads();
  // Thread t owns words [t per, (t + 1) per) (ascending neurons in thread order).
  const int per = (nw + kSmallUnionThreads - 1) / kSmallUnionThreads;
  const int w0 = min(tid * per, nw), w1 = min(w0 + per, nw);
  uint32_t cnt = 0;
  for (int w = w0; w < w1; ++w) cnt += __popc(bits[w]);
  uint32_t incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == 63) wave_sums[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
  for (int q = 0; q < wave; ++q) before += wave_sums[q];
  incl += before;
  uint32_t pos = incl - cnt;
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bits[w];
    while (m) {
      sel[pos++] = w * 32 + (__ffs(m) - 1);
      m &= m - 1u;
    }
  }
  if (tid == kSmallUnionThreads - 1) *n_sel = static_cast<int32_t>(incl);
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
constexpr int kUpKc = kMlpUpKc;             // k per stage
constexpr int kUpRowB = kUpKc * 2;          // bytes of one weight row per stage
constexpr int kUpPieces = kUpRowB / 16;     // 16-byte pieces per row per stage
constexpr int kUpLoads = kUpN * kUpPieces / 256;  // weight pieces per thread per stage
constexpr int kUpX = kUpKc / 32;            // x pieces (MFMA K steps) per lane per stage
static_assert(kUpPieces == 16, "the swizzle and the row mapping assume 16 pieces per row");

template <int L>
struct UpWn {
  uint4 v[L];
};
using UpW = UpWn<kUpLoads>;
struct UpX {
  uint4 v[kUpX];
};

// BB = 16-row batch blocks computed per 64-row tile (1 for B <= 16, 2 for
// B <= 32, else 4).  The four waves split the tile's NU / 16 neuron blocks
// into 4 / BB groups: wave w multiplies neuron blocks of group w / BB by
// batch block w % BB, so no wave multiplies padding rows of a small batch.
// NU = neurons per workgroup: 128, or 144 for full batch tiles where that
// fills whole rounds of workgroups (OPT-66B: 36864 / 144 = 256 tiles, two
// K splits, exactly one round at two per CU; 128 leaves a 1.125-round
// grid); a last tile past n_pad stores nothing there.
//
// KG = K groups per workgroup: 1, or 2 (512 threads, one workgroup per CU):
// two sets of four waves, each the four-wave form above with its own LDS
// tiles, multiply the first and the second half of the stages, and the
// halves are summed on chip ((0 + first) + second, the order in which the
// two-split finalize sums them, so H is bit-identical to that form) and H
// leaves as 16-byte pieces of whole rows.  For full batch tiles whose
// grid is one round at one workgroup per CU (OPT-66B: 256 tiles of 144
// neurons), this replaces two K splits: no fp32 partials go through HBM and
// no finalize launch follows.  The host takes it only with one K split and
// an even stage count (d / 128 is even for every d it accepts).
template <int DT, int BB, int NU, int KG>
__global__ __launch_bounds__(256 * KG, 2 / KG) void sha_mlp_up_kernel(MlpArgs a) {
  using M = Mx<DT>;
  static_assert(BB == 1 || BB == 2 || BB == 4, "batch blocks per tile");
  static_assert(NU % 16 == 0 && (NU / 16) * BB % 4 == 0, "whole neuron blocks per wave");
  static_assert(KG == 1 || KG == 2, "K groups per workgroup");
  constexpr int kUpN = NU;                    // neurons per workgroup
  constexpr int kUpNB = kUpN / 16;            // MFMA neuron blocks
  constexpr int kUpLoads = kUpN * kUpPieces / 256;  // weight pieces per thread per stage
  using UpW = UpWn<kUpLoads>;
  constexpr int NBW = kUpNB * BB / 4;         // neuron blocks per wave
  constexpr int kTileB = 2 * kUpN * kUpRowB;  // LDS bytes of one K group's weight tiles
  __shared__ __attribute__((aligned(16))) char wsm_[KG * kTileB];
  const int nblocks = (a.n_pad + kUpN - 1) / kUpN;
  int t = blockIdx.x;
  const int nblk = t % nblocks;
  t /= nblocks;
  const int split = t % a.up_splits;
  const int btile = t / a.up_splits;
  const int n_sel = sel_count(a);
  const int n0 = nblk * kUpN;
  if (n0 >= n_sel) return;                    // whole workgroup: past the selection
  const int b0 = btile * 64;
  const int kg = KG == 1 ? 0 : static_cast<int>(threadIdx.x >> 8);  // K group of this wave
  int kbeg = split * a.up_kper;
  const int kend = min(kbeg + a.up_kper, a.d);
  int nst = kend > kbeg ? (kend - kbeg) / kUpKc : 0;
  if (KG == 2) {
    nst /= 2;                                 // even on the host's plans
    kbeg += kg * nst * kUpKc;
  }

  const int tid = threadIdx.x & 255, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, c = lane & 15;
  lds_char_t* const wl = (lds_char_t*)(wsm_) + kg * kTileB;

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
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const int grp = wu / BB;                    // neuron blocks grp * NBW .. + NBW - 1
  const int b = b0 + 16 * (wu % BB) + c;
  const bool xok = b < a.B;
  const char* xsrc = static_cast<const char*>(a.x) +
                     (static_cast<size_t>(xok ? b : a.B - 1) * a.d + kbeg + 8 * q4) * 2;

  f32x4 acc[NBW];  // [neuron block of the group]; batch block = wave % BB
#pragma unroll
  for (int i = 0; i < NBW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

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
      for (int i = 0; i < NBW; ++i) {
        const int mb = grp * NBW + i;
        const u32x4_t av = *(const lds_u32x4_t*)(buf + (16 * mb + c) * kUpRowB + ((piece ^ c) * 16));
        acc[i] = M::mma(__builtin_bit_cast(uint4, av), xb, acc[i]);
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

  // lane holds H^T[n = n0 + 16 mb + 4 q4 + r][b]: the computed rows of the
  // tile (16 BB of its 64).
  if constexpr (KG == 2) {
    // The second K group's sums go to its own LDS tiles (lane-linear 16-byte
    // slots), the first group adds them, masks, applies ReLU and writes the
    // 16-bit H tile to its LDS tiles, and all 512 threads copy whole rows out.
    constexpr int kHPitch = kUpN * 2 + 16;    // bytes per staged H row
    static_assert(4 * NBW * 64 * 16 <= kTileB && 16 * BB * kHPitch <= kTileB, "staging fits");
    lds_char_t* const red = (lds_char_t*)(wsm_) + kTileB;
    lds_char_t* const hl = (lds_char_t*)(wsm_);
    __syncthreads();                          // the last stage's LDS reads are done
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < NBW; ++i)
        *(lds_u32x4_t*)(red + ((wave * NBW + i) * 64 + lane) * 16) =
            __builtin_bit_cast(u32x4_t, acc[i]);
    }
    __syncthreads();
    if (kg == 0) {
      const int row = 16 * (wu % BB) + c;
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const f32x4 v = __builtin_bit_cast(
            f32x4, *(const lds_u32x4_t*)(red + ((wave * NBW + i) * 64 + lane) * 16));
        const int nl = 16 * (grp * NBW + i) + 4 * q4;
        float s[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          s[r] = (0.f + acc[i][r]) + v[r];
          if (!sel_valid(a, n0 + nl + r, n_sel)) s[r] = 0.f;
        }
        const uint32_t lo = M::pack(fmaxf(s[0], 0.f), fmaxf(s[1], 0.f));
        const uint32_t hi = M::pack(fmaxf(s[2], 0.f), fmaxf(s[3], 0.f));
        *(lds_u32x2_t*)(hl + row * kHPitch + nl * 2) = u32x2_t{lo, hi};
      }
    }
    __syncthreads();
    constexpr int kHPieces = kUpN / 8;        // 16-byte pieces per H row
    char* const hbase = static_cast<char*>(a.h) + (static_cast<size_t>(b0) * a.n_pad + n0) * 2;
#pragma unroll
    for (int i = 0; i < (16 * BB * kHPieces + 511) / 512; ++i) {
      const int idx = static_cast<int>(threadIdx.x) + 512 * i;
      if (idx < 16 * BB * kHPieces) {
        const int rr = idx / kHPieces, q = idx % kHPieces;
        if (n0 + 8 * q < a.n_pad) {
          const u32x4_t v = *(const lds_u32x4_t*)(hl + rr * kHPitch + q * 16);
          *reinterpret_cast<uint4*>(hbase + (static_cast<size_t>(rr) * a.n_pad + 8 * q) * 2) =
              __builtin_bit_cast(uint4, v);
        }
      }
    }
    return;
  }
  if (a.up_splits > 1 && a.up_stage) {
    // fp32 K-split partials of a one-round grid leave in one burst: through
    // the weight tile in LDS as 16-byte pieces of whole rows (NU neurons of
    // one batch row contiguous) instead of float4 stores in 64-byte segments.
    constexpr int kPitch = kUpN * 4 + 16;     // bytes per staged row
    static_assert(16 * BB * kPitch <= 2 * kUpN * kUpRowB, "staged rows fit the weight tile");
    __syncthreads();                          // the last stage's LDS reads are done
    const int row = 16 * (wu % BB) + c;
#pragma unroll
    for (int i = 0; i < NBW; ++i) {
      const int nl = 16 * (grp * NBW + i) + 4 * q4;
      float4 v = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
      if (!sel_valid(a, n0 + nl, n_sel)) v.x = 0.f;
      if (!sel_valid(a, n0 + nl + 1, n_sel)) v.y = 0.f;
      if (!sel_valid(a, n0 + nl + 2, n_sel)) v.z = 0.f;
      if (!sel_valid(a, n0 + nl + 3, n_sel)) v.w = 0.f;
      *(lds_u32x4_t*)(wl + row * kPitch + nl * 4) = __builtin_bit_cast(u32x4_t, v);
    }
    __syncthreads();
    constexpr int kQuads = kUpN / 4;          // 16-byte pieces per row
    float* const base = a.up_part + (static_cast<size_t>(split) * a.b_pad + b0) * a.n_pad + n0;
#pragma unroll
    for (int i = 0; i < (16 * BB * kQuads + 255) / 256; ++i) {
      const int idx = tid + 256 * i;
      if (idx < 16 * BB * kQuads) {
        const int rr = idx / kQuads, q = idx % kQuads;
        if (n0 + 4 * q < a.n_pad) {
          const u32x4_t v = *(const lds_u32x4_t*)(wl + rr * kPitch + q * 16);
          *reinterpret_cast<uint4*>(base + static_cast<size_t>(rr) * a.n_pad + 4 * q) =
              __builtin_bit_cast(uint4, v);
        }
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int nbase = n0 + 16 * (grp * NBW + i) + 4 * q4;
    if (nbase >= a.n_pad) continue;             // a last tile past the padding
    // Entries outside [0, D) (and past the count) produce no activation.
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (!sel_valid(a, nbase + r, n_sel)) acc[i][r] = 0.f;
    if (a.up_splits == 1) {
      const uint32_t lo = M::pack(fmaxf(acc[i][0], 0.f), fmaxf(acc[i][1], 0.f));
      const uint32_t hi = M::pack(fmaxf(acc[i][2], 0.f), fmaxf(acc[i][3], 0.f));
      *reinterpret_cast<uint2*>(static_cast<char*>(a.h) +
                                (static_cast<size_t>(b) * a.n_pad + nbase) * 2) = make_uint2(lo, hi);
    } else {
      float* p = a.up_part + (static_cast<size_t>(split) * a.b_pad + b) * a.n_pad + nbase;
      *reinterpret_cast<float4*>(p) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    }
  }
}

// One or two computed batch blocks (B <= 16, B <= 32): 4 / BB waves of the
// 128-neuron workgroup multiply the same 16 x rows, so instead of each
// loading all of them, the waves sharing a batch block split its piece
// columns (BB 16-byte pieces per lane per stage each), load them two stages
// ahead, write the pieces of stage st + 1 into a double-buffered 16 BB-row
// x tile in LDS (XOR-swizzled like the weights, 2 x 4 BB KB), and every
// wave reads its B operands there: each x byte is read from L2 once per
// workgroup instead of 4 / BB times.  Weights move exactly as in the
// general form; per neuron the products accumulate over the same K stages
// in the same order, so its outputs are bit-identical.
constexpr int kUp1N = kMlpUpNeurons;        // neurons per workgroup (128)
constexpr int kUp1Loads = kUp1N * kUpPieces / 256;  // weight pieces per thread per stage

struct UpW1 {
  uint4 v[kUp1Loads];
};
template <int BB>
struct UpXs {
  uint4 v[BB];
};

template <int DT, int BB>
__global__ __launch_bounds__(256, 2) void sha_mlp_upx_kernel(MlpArgs a) {
  using M = Mx<DT>;
  static_assert(BB == 1 || BB == 2, "one or two batch blocks");
  constexpr int NBW = 2 * BB;                 // neuron blocks per wave
  using UpX1 = UpXs<BB>;
  __shared__ __attribute__((aligned(16))) char wsm_[2 * kUp1N * kUpRowB];
  __shared__ __attribute__((aligned(16))) char xsm_[2 * 16 * BB * kUpRowB];
  const int nblocks = a.n_pad / kUp1N;
  int t = blockIdx.x;
  const int nblk = t % nblocks;
  t /= nblocks;
  const int split = t % a.up_splits;
  const int btile = t / a.up_splits;
  const int n_sel = sel_count(a);
  const int n0 = nblk * kUp1N;
  if (n0 >= n_sel) return;                    // whole workgroup: past the selection
  const int b0 = btile * 64;
  const int kbeg = split * a.up_kper;
  const int kend = min(kbeg + a.up_kper, a.d);
  const int nst = kend > kbeg ? (kend - kbeg) / kUpKc : 0;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q4 = lane >> 4, c = lane & 15;
  lds_char_t* const wl = (lds_char_t*)(wsm_);
  lds_char_t* const xl = (lds_char_t*)(xsm_);

  // Weight pieces of this thread: piece p = tid + 256 i -> row (tid >> 4) +
  // 16 i, 16-byte column tid & 15 (rows past the selection read its last
  // entry; their outputs are masked).
  const char* w1 = static_cast<const char*>(a.w1t) + static_cast<size_t>(kbeg) * 2;
  uint32_t woff[kUp1Loads];
  int wdst[kUp1Loads];
#pragma unroll
  for (int i = 0; i < kUp1Loads; ++i) {
    const int r = (tid >> 4) + 16 * i, col = tid & 15;
    const int row = sel_row(a, min(n0 + r, n_sel - 1));
    woff[i] = static_cast<uint32_t>(row) * static_cast<uint32_t>(a.d) * 2u + col * 16;
    wdst[i] = r * kUpRowB + ((col ^ (r & 15)) * 16);
  }
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const int grp = wu / BB, bblk = wu % BB;    // neuron blocks grp * NBW .., batch block
  // x row of this lane (padding rows past B read row B - 1, as in the
  // general form); this wave loads pieces 4 s + q4 of it for
  // s = grp * BB .. grp * BB + BB - 1.
  const int b = b0 + 16 * bblk + c;
  const bool xok = b < a.B;
  const char* xsrc = static_cast<const char*>(a.x) +
                     (static_cast<size_t>(xok ? b : a.B - 1) * a.d + kbeg + 8 * q4) * 2;
  const int xrow = (16 * bblk + c) * kUpRowB;

  f32x4 acc[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_w = [&](int st, UpW1& d) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kUp1Loads; ++i) d.v[i] = ld16_stream(w1 + woff[i] + st * kUpRowB);
  };
  auto write_w = [&](int st, const UpW1& w) __attribute__((always_inline)) {
    lds_char_t* const buf = wl + (st & 1) * (kUp1N * kUpRowB);
#pragma unroll
    for (int i = 0; i < kUp1Loads; ++i)
      *(lds_u32x4_t*)(buf + wdst[i]) = __builtin_bit_cast(u32x4_t, w.v[i]);
  };
  auto load_x = [&](int st, UpX1& d) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < BB; ++j) d.v[j] = ld16(xsrc + st * kUpRowB + (grp * BB + j) * 64);
  };
  auto write_x = [&](int st, const UpX1& d) __attribute__((always_inline)) {
    lds_char_t* const buf = xl + (st & 1) * (16 * BB * kUpRowB);
#pragma unroll
    for (int j = 0; j < BB; ++j) {
      const int piece = 4 * (grp * BB + j) + q4;
      *(lds_u32x4_t*)(buf + xrow + ((piece ^ c) * 16)) = __builtin_bit_cast(u32x4_t, d.v[j]);
    }
  };
  // Step st: weights and x of st + 1 go from registers to LDS; x of st + 2
  // is loaded into the x set just written, then the weights of st + 3 into
  // the weight set just written; stage st is multiplied; one barrier closes
  // the step (CHECK: only work inside the K range).
  auto step = [&](int st, UpW1& wnext, UpX1& xr, auto check) __attribute__((always_inline)) {
    constexpr bool C = decltype(check)::value;
    if (!C || st + 1 < nst) {
      write_w(st + 1, wnext);
      write_x(st + 1, xr);
    }
    if (!C || st + 2 < nst) load_x(st + 2, xr);
    __builtin_amdgcn_sched_barrier(0);
    if (!C || st + 3 < nst) load_w(st + 3, wnext);
    const lds_char_t* const wbuf = wl + (st & 1) * (kUp1N * kUpRowB);
    const lds_char_t* const xbuf = xl + (st & 1) * (16 * BB * kUpRowB);
#pragma unroll
    for (int s = 0; s < kUpX; ++s) {
      const int piece = 4 * s + q4;
      const u32x4_t xv = *(const lds_u32x4_t*)(xbuf + xrow + ((piece ^ c) * 16));
      const uint4 xb = __builtin_bit_cast(uint4, xv);
#pragma unroll
      for (int i = 0; i < NBW; ++i) {
        const int mb = NBW * grp + i;
        const u32x4_t av = *(const lds_u32x4_t*)(wbuf + (16 * mb + c) * kUpRowB + ((piece ^ c) * 16));
        acc[i] = M::mma(__builtin_bit_cast(uint4, av), xb, acc[i]);
      }
    }
    __syncthreads();
  };

  if (nst > 0) {
    // Unconditional prologue loads (short ranges load their last stage
    // again), as in the general form.
    UpW1 wa, wb;
    UpX1 xr;
    load_x(0, xr);
    load_w(0, wa);
    load_w(min(1, nst - 1), wb);
    write_x(0, xr);
    load_x(min(1, nst - 1), xr);
    write_w(0, wa);
    load_w(min(2, nst - 1), wa);
    __syncthreads();
    using Chk = std::true_type;
    using NoChk = std::false_type;
    int st = 0;
    for (; st + 5 <= nst; st += 2) {
      step(st, wb, xr, NoChk{});
      step(st + 1, wa, xr, NoChk{});
    }
    for (; st + 2 <= nst; st += 2) {
      step(st, wb, xr, Chk{});
      step(st + 1, wa, xr, Chk{});
    }
    if (st < nst) step(st, wb, xr, Chk{});
  }

  // lane holds H^T[n = n0 + 16 mb + 4 q4 + r][b]: the computed rows of the
  // tile (16 BB of its 64).
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int nbase = n0 + 16 * (NBW * grp + i) + 4 * q4;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (!sel_valid(a, nbase + r, n_sel)) acc[i][r] = 0.f;
    if (a.up_splits == 1) {
      const uint32_t lo = M::pack(fmaxf(acc[i][0], 0.f), fmaxf(acc[i][1], 0.f));
      const uint32_t hi = M::pack(fmaxf(acc[i][2], 0.f), fmaxf(acc[i][3], 0.f));
      *reinterpret_cast<uint2*>(static_cast<char*>(a.h) +
                                (static_cast<size_t>(b) * a.n_pad + nbase) * 2) = make_uint2(lo, hi);
    } else {
      float* p = a.up_part + (static_cast<size_t>(split) * a.b_pad + b) * a.n_pad + nbase;
      *reinterpret_cast<float4*>(p) = make_float4(acc[i][0], acc[i][1], acc[i][2], acc[i][3]);
    }
  }
}


// H = relu(sum of the K-split partials), fixed order; one thread per 4
// neurons of a computed row (rows 16 bb of each 64-row tile).  The splits'
// loads are issued together (at most kMlpMaxUpSplits), then summed in order.
template <int DT>
__global__ __launch_bounds__(256) void sha_mlp_up_finalize_kernel(MlpArgs a) {
  using M = Mx<DT>;
  const int n_sel = sel_count(a);
  const int rows = 16 * a.bb;                  // computed rows per tile
  const size_t quads = static_cast<size_t>(a.b_pad / 64) * rows * (a.n_pad / 4);
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < quads; i += static_cast<size_t>(gridDim.x) * 256) {
    const size_t rq = i / (a.n_pad / 4);
    const size_t b = (rq / rows) * 64 + rq % rows;
    const int n4 = static_cast<int>(i % (a.n_pad / 4)) * 4;
    if (n4 >= n_sel) continue;
    float4 v[kMlpMaxUpSplits];
#pragma unroll
    for (int sp = 0; sp < kMlpMaxUpSplits; ++sp)
      if (sp < a.up_splits)
        v[sp] = *reinterpret_cast<const float4*>(
            a.up_part + (static_cast<size_t>(sp) * a.b_pad + b) * a.n_pad + n4);
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int sp = 0; sp < kMlpMaxUpSplits; ++sp)
      if (sp < a.up_splits) {
        s.x += v[sp].x; s.y += v[sp].y; s.z += v[sp].z; s.w += v[sp].w;
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
constexpr int kDnHPitch = kDnKc * 2 + 16;   // 144 B: conflict-free H reads

// NW = waves per workgroup: each wave owns 64 output columns, so a
// workgroup owns 64 NW columns (256 with 4 waves, two workgroups per CU; 512
// with 8 waves, one per CU, which halves the H rows every column block
// reads).  The register budget is 256 per lane either way, accumulators
// included.  BB = 16-row batch blocks computed per 64-row tile (as in the up
// projection): only those rows of H are multiplied.
//
// FU (one or two batch blocks, 2-4 up K splits): the up finalize is folded
// in.  Instead of H, a workgroup loads each chunk's fp32 up partials (every
// split, unconditionally, the split index clamped), sums them in split
// order from zero, applies ReLU and rounds to 16 bits as it writes the
// chunk's H rows to LDS: exactly the finalize's arithmetic, so H and y are
// bit-identical, and the finalize launch is gone.
constexpr int kFuSplits = 4;                // up K splits the folded form reads (at most)
template <int DT, int BB, int NW, bool FU>
__global__ __launch_bounds__(64 * NW, 8 / NW) void sha_mlp_down_kernel(MlpArgs a) {
  using M = Mx<DT>;
  static_assert(BB == 1 || BB == 2 || BB == 4, "batch blocks per tile");
  static_assert(NW == 4 || NW == 8, "waves per workgroup");
  static_assert(!FU || BB <= 2, "the folded up finalize: one or two batch blocks");
  constexpr int T = 64 * NW;                  // threads
  constexpr int kDnCols = 64 * NW;            // output columns per workgroup
  constexpr int kDnWPitch = kDnCols * 2 + 32; // 544 / 1056 B: conflict-free transposed reads
  constexpr int RP = kDnCols / 8;             // 16-byte pieces per weight row
  constexpr int HL = (BB == 4 ? 512 : 256) / T > 0 ? (BB == 4 ? 512 : 256) / T : 1;  // H pieces per thread
  // Folded finalize: each thread sums kFuE consecutive neurons of one H row.
  constexpr int kFuE = 16 * BB * kDnKc / T;
  static_assert(!FU || kFuE == 2 || kFuE == 4 || kFuE == 8, "neurons per thread");
  struct HSet {
    uint4 v[HL];
  };
  struct PSet {
    float v[kFuSplits * (kFuE > 0 ? kFuE : 1)];
  };
  using HR = std::conditional_t<FU, PSet, HSet>;
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

  f32x4 acc[BB][4];  // [m block (batch)][n block (columns)]
#pragma unroll
  for (int i = 0; i < BB; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Gathered W2t rows of a chunk: 64 rows x 128 NW bytes = 512 NW pieces (8
  // per thread); H chunk: HL T / 8 rows x 128 B (HL pieces per thread; at
  // least the 16 BB computed rows), neurons at or past nend read as zero.
  // Piece tid + T i of the weights is row tid / RP + 8 i: with 4 waves each
  // load instruction covers two rows (2 wave + (lane >> 5)), with 8 waves
  // one (wave), so it needs one or two selection entries that are the same
  // for the whole wave: they are read with scalar loads (own counter), and
  // the vector loads of earlier chunks need not complete before the next
  // chunk's addresses are known.  H pieces are read
  // unconditionally (offsets clamped inside the row) and masked only when
  // they are written to LDS: masking at load time would make the wave wait
  // for them, and (loads complete in order) for every older load, at once.
  const int wu = __builtin_amdgcn_readfirstlane(wave);
  const bool upper = lane >= 32;
  auto load_chunk = [&](int k0, uint4 (&wv)[8], HR& hv) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int row;
      if constexpr (NW == 4) {
        const int r0 = k0 + 2 * wu + 8 * i;
        const int s0 = a.sel[min(r0, nend - 1)], s1 = a.sel[min(r0 + 1, nend - 1)];
        const int row0 = (s0 >= 0 && s0 < a.D) ? s0 : 0, row1 = (s1 >= 0 && s1 < a.D) ? s1 : 0;
        row = upper ? row1 : row0;
      } else {
        const int s0 = a.sel[min(k0 + wu + 8 * i, nend - 1)];
        row = (s0 >= 0 && s0 < a.D) ? s0 : 0;
      }
      wv[i] = ld16_stream(static_cast<const char*>(a.w2t) +
                          (static_cast<size_t>(row) * a.d + col0 + (lane % RP) * 8) * 2);
    }
    if constexpr (FU) {
      // Partials of neurons nc .. nc + kFuE - 1 of row r, every split (a
      // split past up_splits reads the last one again and is not summed).
      const int r = tid / (kDnKc / kFuE), ng = tid % (kDnKc / kFuE);
      const int nc = min(k0 + ng * kFuE, a.n_pad - kFuE);  // past n_pad: past nend, masked
#pragma unroll
      for (int sp = 0; sp < kFuSplits; ++sp) {
        const int sv = min(sp, a.up_splits - 1);
        const float* src =
            a.up_part + (static_cast<size_t>(sv) * a.b_pad + b0 + r) * a.n_pad + nc;
        if constexpr (kFuE == 2) {
          const float2 t = *reinterpret_cast<const float2*>(src);
          hv.v[sp * kFuE] = t.x;
          hv.v[sp * kFuE + 1] = t.y;
        } else {
#pragma unroll
          for (int q = 0; q < kFuE / 4; ++q) {
            const float4 t = *reinterpret_cast<const float4*>(src + 4 * q);
            hv.v[sp * kFuE + 4 * q] = t.x;
            hv.v[sp * kFuE + 4 * q + 1] = t.y;
            hv.v[sp * kFuE + 4 * q + 2] = t.z;
            hv.v[sp * kFuE + 4 * q + 3] = t.w;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < HL; ++i) {
        const int idx = tid + T * i;
        const int r = idx >> 3, piece = idx & 7;
        const int nc = min(k0 + piece * 8, a.n_pad - 8);  // past n_pad: past nend, masked
        hv.v[i] = ld16(static_cast<const char*>(a.h) +
                       (static_cast<size_t>(b0 + r) * a.n_pad + nc) * 2);
      }
    }
  };

  // Chunk j (neurons nbeg + 64 j ..) lives in register set j % 2.  Step j:
  // wait for the previous chunk's LDS reads, write chunk j to LDS, reload its
  // set with chunk j + 2 (two chunks in flight during the products), publish
  // and multiply.  CHECK: only load inside the range.
  const int nch = nend > nbeg ? (nend - nbeg + kDnKc - 1) / kDnKc : 0;
  auto step = [&](int j, uint4 (&w)[8], HR& h, auto check) {
    constexpr bool C = decltype(check)::value;
    __syncthreads();  // the previous chunk's LDS reads are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int idx = tid + T * i;
      const int r = idx / RP, piece = idx % RP;
      *(lds_u32x4_t*)(wl + r * kDnWPitch + piece * 16) = __builtin_bit_cast(u32x4_t, w[i]);
    }
    if constexpr (FU) {
      // The finalize's sum (from zero, in split order), ReLU and rounding;
      // neurons at or past nend are zero.
      const int r = tid / (kDnKc / kFuE), ng = tid % (kDnKc / kFuE);
      const int kk0 = nbeg + j * kDnKc + ng * kFuE;
      float sum[kFuE];
#pragma unroll
      for (int e = 0; e < kFuE; ++e) sum[e] = 0.f;
#pragma unroll
      for (int sp = 0; sp < kFuSplits; ++sp)
        if (sp < a.up_splits) {
#pragma unroll
          for (int e = 0; e < kFuE; ++e) sum[e] += h.v[sp * kFuE + e];
        }
      uint32_t pk[kFuE / 2];
#pragma unroll
      for (int e = 0; e < kFuE / 2; ++e) {
        const float lo = kk0 + 2 * e < nend ? fmaxf(sum[2 * e], 0.f) : 0.f;
        const float hi = kk0 + 2 * e + 1 < nend ? fmaxf(sum[2 * e + 1], 0.f) : 0.f;
        pk[e] = M::pack(lo, hi);
      }
      lds_char_t* const dst = hl + r * kDnHPitch + ng * kFuE * 2;
      if constexpr (kFuE == 2) {
        *(lds_u32_t*)(dst) = pk[0];
      } else if constexpr (kFuE == 4) {
        *(lds_u32x2_t*)(dst) = u32x2_t{pk[0], pk[1]};
      } else {
        *(lds_u32x4_t*)(dst) = u32x4_t{pk[0], pk[1], pk[2], pk[3]};
      }
    } else {
#pragma unroll
      for (int i = 0; i < HL; ++i) {
        const int idx = tid + T * i;
        const int r = idx >> 3, piece = idx & 7;
        const int cnt = min(max(nend - (nbeg + j * kDnKc + piece * 8), 0), 8);  // valid neurons
        uint32_t m[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          m[e] = (2 * e < cnt ? 0x0000FFFFu : 0u) | (2 * e + 1 < cnt ? 0xFFFF0000u : 0u);
        const u32x4_t hm = {h.v[i].x & m[0], h.v[i].y & m[1], h.v[i].z & m[2], h.v[i].w & m[3]};
        *(lds_u32x4_t*)(hl + r * kDnHPitch + piece * 16) = hm;
      }
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
      uint4 ha[BB];
#pragma unroll
      for (int mb = 0; mb < BB; ++mb) {
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
        for (int mb = 0; mb < BB; ++mb) acc[mb][nb] = M::mma(ha[mb], wb, acc[mb][nb]);
      }
    }
  };

  if (nch > 0) {
    // Both sets are loaded on every path into the loop (a one-chunk range
    // loads its chunk twice), so the compiler sees the same loads in flight
    // at the loop head from the entry and from the back edge and can leave
    // the younger set in flight; a conditional second load makes it wait
    // for everything there.
    uint4 wa[8], wb8[8];
    HR ha0, hb0;
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
  if (a.dn_splits == 1 || !a.dn_stage) {
#pragma unroll
    for (int mb = 0; mb < BB; ++mb)
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
    return;
  }
  // fp32 split partials: every workgroup of the (one-round) grid reaches
  // this point at about the same time, so the stores are one burst.  They
  // go through the weight tile in LDS, up to 32 rows at a time, and leave
  // as 16-byte pieces of whole rows (a wave writes 1 KB contiguous) instead
  // of 4-byte stores in 64-byte row segments.
  constexpr int kRows = 16 * BB < 32 ? 16 * BB : 32;      // rows per pass
  constexpr int kPitch = kDnCols * 4 + 16;                // bytes per staged row
  static_assert(kRows * kPitch <= kDnKc * kDnWPitch, "staged rows fit the weight tile");
  float* const pout = a.dn_part + static_cast<size_t>(split) * a.b_pad * a.d;
#pragma unroll
  for (int pass = 0; pass < (16 * BB) / kRows; ++pass) {
    __syncthreads();  // the last products' (or the previous pass's) LDS reads are done
#pragma unroll
    for (int mb = 0; mb < BB; ++mb) {
      if (mb * 16 / kRows != pass) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mb + 4 * q4 + r - pass * kRows;
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          *(lds_float_t*)(wl + row * kPitch + (64 * wave + 16 * nb + c) * 4) = acc[mb][nb][r];
      }
    }
    __syncthreads();
    constexpr int kPieces = kRows * kDnCols / 4;         // 16-byte pieces of the pass
#pragma unroll
    for (int i = 0; i < (kPieces + T - 1) / T; ++i) {
      const int idx = tid + T * i;
      if (idx < kPieces) {
        const int row = idx / (kDnCols / 4), piece = idx % (kDnCols / 4);
        const int b = b0 + pass * kRows + row;
        if (b < a.B) {
          const u32x4_t v = *(const lds_u32x4_t*)(wl + row * kPitch + piece * 16);
          *reinterpret_cast<uint4*>(pout + static_cast<size_t>(b) * a.d + col0 + piece * 4) =
              __builtin_bit_cast(uint4, v);
        }
      }
    }
  }
}

// y = sum of the neuron-split partials, fixed order; one thread per 4
// consecutive columns (d is a multiple of 256).  Loads of sixteen splits are
// issued together (the usual counts, up to 16, wait for memory once), then
// summed in order.
template <int DT>
__global__ __launch_bounds__(256) void sha_mlp_down_finalize_kernel(MlpArgs a) {
  const size_t quads = static_cast<size_t>(a.B) * (a.d / 4);
  const size_t plane = static_cast<size_t>(a.b_pad) * a.d;
  for (size_t i = blockIdx.x * 256 + threadIdx.x; i < quads; i += static_cast<size_t>(gridDim.x) * 256) {
    const float4* p = reinterpret_cast<const float4*>(a.dn_part) + i;  // row-major [b][d] of plane 0
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sp0 = 0; sp0 < a.dn_splits; sp0 += 16) {
      float4 v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (sp0 + u < a.dn_splits) v[u] = p[(sp0 + u) * (plane / 4)];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (sp0 + u < a.dn_splits) {
          s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
        }
    }
    const size_t e = i * 4;
    Elem<DT>::store(a.y, e, s.x);
    Elem<DT>::store(a.y, e + 1, s.y);
    Elem<DT>::store(a.y, e + 2, s.z);
    Elem<DT>::store(a.y, e + 3, s.w);
  }
}

template <int DT, int BB>
hipError_t launch_mlp_bb(const MlpArgs& a, hipStream_t st) {
  const int dn_cols = 64 * a.dn_waves;
  const unsigned btiles = static_cast<unsigned>(a.b_pad / 64);
  const long long up_wgs =
      static_cast<long long>((a.n_pad + a.up_nu - 1) / a.up_nu) * a.up_splits * btiles;
  // The two-K-group form writes H itself: one K split, two equal halves.
  if (a.up_kg == 2 && (BB != 4 || a.up_splits != 1 || (a.d / kMlpUpKc) % 2 != 0))
    return hipErrorInvalidValue;
  if (BB <= 2 && a.up_xlds)
    hipLaunchKernelGGL((sha_mlp_upx_kernel<DT, BB <= 2 ? BB : 1>), dim3(static_cast<unsigned>(up_wgs)),
                       dim3(256), 0, st, a);
  else if (BB == 4 && a.up_kg == 2 && a.up_nu == 144)
    hipLaunchKernelGGL((sha_mlp_up_kernel<DT, 4, 144, 2>), dim3(static_cast<unsigned>(up_wgs)),
                       dim3(512), 0, st, a);
  else if (BB == 4 && a.up_kg == 2)
    hipLaunchKernelGGL((sha_mlp_up_kernel<DT, 4, 128, 2>), dim3(static_cast<unsigned>(up_wgs)),
                       dim3(512), 0, st, a);
  else if (BB == 4 && a.up_nu == 144)
    hipLaunchKernelGGL((sha_mlp_up_kernel<DT, 4, 144, 1>), dim3(static_cast<unsigned>(up_wgs)),
                       dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((sha_mlp_up_kernel<DT, BB, 128, 1>), dim3(static_cast<unsigned>(up_wgs)),
                       dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // With the finalize folded into the down projection, H is never written.
  const bool fold = BB <= 2 && a.dn_fuse_up;
  if (fold && (a.up_splits < 2 || a.up_splits > kFuSplits)) return hipErrorInvalidValue;
  if (a.up_splits > 1 && !fold) {
    const size_t quads = static_cast<size_t>(btiles) * 16 * BB * (a.n_pad / 4);
    const unsigned blocks = static_cast<unsigned>(quads < 256 * 1024 ? (quads + 255) / 256 : 1024);
    hipLaunchKernelGGL((sha_mlp_up_finalize_kernel<DT>), dim3(blocks), dim3(256), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // 1-D over (column block, split, batch tile): the kernel maps the ids
  // onto XCDs itself.
  const dim3 dn_grid(static_cast<unsigned>((a.d / dn_cols) * a.dn_splits) * btiles);
  constexpr int BF = BB <= 2 ? BB : 1;       // batch blocks of the folded form
  if (fold && a.dn_waves == 8)
    hipLaunchKernelGGL((sha_mlp_down_kernel<DT, BF, 8, true>), dn_grid, dim3(512), 0, st, a);
  else if (fold)
    hipLaunchKernelGGL((sha_mlp_down_kernel<DT, BF, 4, true>), dn_grid, dim3(256), 0, st, a);
  else if (a.dn_waves == 8)
    hipLaunchKernelGGL((sha_mlp_down_kernel<DT, BB, 8, false>), dn_grid, dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((sha_mlp_down_kernel<DT, BB, 4, false>), dn_grid, dim3(256), 0, st, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (a.dn_splits > 1) {
    const size_t total = static_cast<size_t>(a.B) * (a.d / 4);
    const unsigned blocks = static_cast<unsigned>(total < 256 * 2048 ? (total + 255) / 256 : 2048);
    hipLaunchKernelGGL((sha_mlp_down_finalize_kernel<DT>), dim3(blocks), dim3(256), 0, st, a);
    e = hipGetLastError();
  }
  return e;
}

template <int DT>
hipError_t launch_mlp_t(const MlpArgs& a, hipStream_t st) {
  switch (a.bb) {
    case 1: return launch_mlp_bb<DT, 1>(a, st);
    case 2: return launch_mlp_bb<DT, 2>(a, st);
    case 4: return launch_mlp_bb<DT, 4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int mlp_union_blocks(int D) { return (D + kUnionBlockFlags - 1) / kUnionBlockFlags; }

hipError_t launch_mlp_union(const int32_t* rows, int total, int D, int32_t* sel, int32_t* n_sel,
                            uint8_t* flags, int small_max, hipStream_t st) {
  const int lim = small_max < 0 ? kSmallUnionMaxTotal : small_max;
  if (small_max != 0 && total <= lim && D <= kSmallUnionMaxD) {
    hipLaunchKernelGGL(sha_mlp_union_small_kernel, dim3(1), dim3(kSmallUnionThreads), 0, st, rows,
                       total, D, sel, n_sel);
    return hipGetLastError();
  }
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
