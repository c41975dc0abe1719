// Internal interface between the C ABI (sha_api.cpp, sha_step.cpp) and the
// HIP kernels.  Not installed; callers use include/sha.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "sha_decode.h"

namespace sha {

// Selective MLP (batch union of active neurons).  Sizes validated on the host;
// the selection count is device data, clamped to n_max by the kernels.
// Up-projection tile: kMlpUpNeurons selected neurons x 64 batch rows per
// workgroup, in K stages of kMlpUpKc.
constexpr int kMlpUpNeurons = 128;
constexpr int kMlpUpKc = 128;
constexpr int kMlpMaxUpSplits = 8;     // K splits of the up projection (at most)
struct MlpArgs {
  const void* x;        // [B, d]
  const void* w1t;      // [D, d]  (W1^T, neuron-major)
  const void* w2t;      // [D, d]  (W2^T, neuron-major)
  const int32_t* sel;   // [>= n_max] selected neurons; entries outside [0, D) contribute nothing
  const int32_t* n_sel; // device count of valid leading entries of sel
  void* y;              // [B, d]
  void* h;              // workspace: relu(x W1[:, S]), [b_pad, n_pad] 16-bit
  float* up_part;       // workspace: up-projection K-split partials [up_splits, b_pad, n_pad]
  float* dn_part;       // workspace: down-projection split partials [dn_splits, b_pad, d]
  int B, d, D, n_max;
  int n_pad, b_pad;     // n_max rounded up to kMlpUpNeurons, B rounded up to 64
  int bb;               // 16-row batch blocks computed per 64-row tile: 1 (B <= 16),
                        // 2 (B <= 32) or 4; rows 16 bb .. 63 of a tile are never
                        // computed, read for an output row, or stored
  int up_xlds;          // bb <= 2: x shared through LDS by the up workgroup's waves
  int up_nu;            // neurons per up workgroup: 128, or 144 (bb = 4)
  int up_stage;         // up split partials stored through LDS as whole-row pieces
  int up_kg;            // K groups per up workgroup: 1, or 2 (bb = 4, one K split,
                        // an even stage count; 512 threads)
  int up_splits, up_kper;  // K splits of the up projection and K elements per split
  int dn_splits;        // neuron-range splits of the down projection
  int dn_stage;         // down split partials stored through LDS as whole-row pieces
  int dn_waves;         // waves per down workgroup (64 output columns each): 4, or 8
                        // when d is a multiple of 512
  int dn_fuse_up;       // bb <= 2 with 2-4 up K splits: the down projection sums the
                        // up partials itself (no up finalize; H unused)
};

// flags: round_up(D, 256) bytes of workspace.
int mlp_union_blocks(int D);
// small_max: unions of at most that many entries (and 2^18 neurons) run as
// one workgroup (flags unused); -1 takes the library's bound, 0 never.
hipError_t launch_mlp_union(const int32_t* rows, int total, int D, int32_t* sel, int32_t* n_sel,
                            uint8_t* flags, int small_max, hipStream_t stream);
hipError_t launch_selective_mlp(const MlpArgs& a, int dtype, hipStream_t stream);

// Attention router: scores = x w^T (+ bias), per-row top-k heads.
constexpr int kRouterMaxH = 1024;
struct RouterArgs {
  const void* x;        // [B, d]
  const void* w;        // [H, d]
  const float* bias;    // [H] or null
  float* scores;        // [B, H] fp32 (output)
  int32_t* index;       // [B, top_k] (output, ascending head ids)
  int B, d, H, top_k;
  float* part;          // [B, nchunk, H] fp32 K-split partials, or null (one-pass form)
  int nchunk;           // hidden-dimension chunks of kRouterChunk elements
};

// K-split router form: 16-bit inputs, at most kRouterSplitMaxH heads and
// kRouterSplitMaxB rows; one partial per (row, chunk of kRouterChunk hidden
// elements, head).
constexpr int kRouterChunk = 256;
constexpr int kRouterSplitMaxH = 128;
constexpr int kRouterSplitMaxB = 4096;

// num_cus: the device's compute units (picks the heads per scores workgroup).
hipError_t launch_router(const RouterArgs& a, int dtype, int num_cus, hipStream_t stream);

// Records the hipError_t that sha_last_hip_error() reports on this thread.
void set_last_hip_error(int e);

}  // namespace sha
