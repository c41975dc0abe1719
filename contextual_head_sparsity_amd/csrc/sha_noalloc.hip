// sha_decode_noalloc: the explicit-workspace decode with its split partials
// in a fixed device array instead of a caller or library allocation, for
// callers that cannot allocate (code under graph capture, serving loops that
// forbid allocation).  The contract is in include/sha.h.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy until the process ends.  In host code its name is only a
// stand-in for the symbol, not a device address, so the host never passes it
// to a kernel or a copy; it resolves the array's address on each device once,
// with hipGetSymbolAddress, and uses that pointer.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sha.h"
#include "sha_launch.h"

namespace {

constexpr size_t kScratchBytes = SHA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch` (looked up on its first use there).
sha_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    sha::set_last_hip_error(e);
    return SHA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return SHA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      sha::set_last_hip_error(e);
      return SHA_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SHA_OK;
}

}  // namespace

extern "C" {

sha_status sha_decode_noalloc(const void* q, const void* k, const void* v, const int32_t* index,
                              int B, int H, int H_kv, int Nkv, int d, int top_k, float scale,
                              void* o, hipStream_t stream, sha_dtype dtype, int gqa,
                              int nsplit) {
  if (nsplit < 0 || (gqa != 0 && gqa != 1)) return SHA_ERR_INVALID_ARG;
  // Partials this call needs (0 for an unsplit or an invalid call: the
  // decode entry point then runs or reports the error itself).
  const size_t need = sha_workspace_bytes(B, H, H_kv, Nkv, d, top_k, gqa, dtype, nsplit, 0);
  if (need > kScratchBytes) return SHA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    const sha_status st = scratch_ptr(&ws);
    if (st != SHA_OK) return st;
  }
  return gqa ? sha_decode_gqa_ex(q, k, v, index, B, H, H_kv, Nkv, d, top_k, scale, o, stream,
                                 dtype, nsplit, ws, need)
             : sha_decode_ex(q, k, v, index, B, H, H_kv, Nkv, d, top_k, scale, o, stream, dtype,
                             nsplit, ws, need);
}

}  // extern "C"
