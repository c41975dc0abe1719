// Internal interface between the C ABI (sha_api.cpp) and the SHA decode
// kernels (sha_kernels.hip, sha_gqa_mfma.hip).  Not installed; callers use
// include/sha.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace sha {

// How key/value rows are found in memory.
//   kKvContig : [B, H_kv, Nkv, d] contiguous (compile-time row pitch).
//   kKvStrided: row r of (b, g) at base + b*bs + g*hs + r*rs (element strides).
//   kKvPaged  : row r of (b, g) on page block_table[b, r / P], at
//               base + page*bs + g*hs + (r % P)*rs (bs is the page stride).
enum KvLayout { kKvContig = 0, kKvStrided = 1, kKvPaged = 2 };

// Page ids one workgroup stages in LDS for its key range (paged layout); the
// host keeps every split within this many pages.
constexpr int kMaxSplitPages = 1024;

// Everything a launch needs, validated by the host before it gets here.
struct Args {
  const void* q;        // [B, H, 1, d]
  const void* k;        // keys, addressed as `layout` says
  const void* v;        // values, addressed as `layout` says
  const int32_t* idx;   // [B, top_k]: head ids (MHA) or group ids (GQA)
  void* o;              // [B, H, 1, d]
  float* part_o;        // split partials: [units * heads_per_unit * nsplit, d] (unnormalised)
  float* part_ml;       // split partials: [units * heads_per_unit * nsplit, 2] = (m, l), log2 domain
  int B, H, H_kv, Nkv, top_k;
  int G;                // H / H_kv
  int nsplit;           // effective split count (every split holds >= 1 key)
  int chunk;            // keys per split (last split may hold fewer)
  int waves;            // waves per workgroup of the matrix-core group kernel (2 or 4)
  float scale_log2;     // scale * log2(e): scores are kept in the base-2 domain
  // KV addressing (strided / paged layouts); strides in elements.
  int layout;           // KvLayout
  long long k_bs, k_hs, k_rs;
  long long v_bs, v_hs, v_rs;
  const int32_t* seqlens;      // [B] keys per row (clamped to [0, Nkv]) or null (all Nkv)
  const int32_t* block_table;  // [B, bt_stride] page ids (paged)
  int bt_stride;
  int page_shift;              // log2(rows per page) (paged)
  int num_pages;               // page ids are clamped into [0, num_pages) (paged)
};

enum Dtype { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Shape of a vector-ALU split kernel: waves per workgroup and key rows per
// lane group per iteration.
struct KernelShape {
  int waves;
  int unroll;
};

// Query heads one GQA workgroup computes: 16 on the matrix-core path (one
// MFMA column per head), <= 8 on the vector path; a group of G heads takes
// ceil(G / gqa_heads_per_wg(...)) workgroups per split.
int gqa_heads_per_wg(int G, bool mfma);

hipError_t launch_mha(const Args& a, int dtype, int d, int variant, hipStream_t stream);
// Vector-ALU GQA kernel (any dtype) or, with mfma, the matrix-core kernel
// (f16 / bf16 only).
hipError_t launch_gqa(const Args& a, int dtype, int d, int variant, bool mfma, hipStream_t stream);
hipError_t launch_gqa_mfma(const Args& a, int dtype, int d, hipStream_t stream);
// Split merge for nsplit > 1 (gqa != 0: every head of each selected group).
hipError_t launch_combine(const Args& a, int dtype, int d, int gqa, hipStream_t stream);

}  // namespace sha
