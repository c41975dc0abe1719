// Device-side helpers shared by the SHA decode kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sha_decode.h"

namespace sha {
namespace detail {

constexpr float kNegInf = -__builtin_inff();
// Lazy-rescale slack in base-2 units: probabilities are bounded by 2^8.
constexpr float kRescaleSlack = 8.0f;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of LPR lanes; every lane of the group receives
// the same total.
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPR == 8 || LPR == 16 || LPR == 32, "lanes per key row");
  x += dpp<0xB1>(x);                               // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);                               // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);                              // row_half_mirror (8 lanes)
  if constexpr (LPR >= 16) x += dpp<0x140>(x);     // row_mirror (16 lanes)
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Element types: 16 bytes per lane per load.
template <int DT>
struct Elem;

template <>
struct Elem<kF32> {
  static constexpr int VEC = 4;
  __device__ static float dot(uint4 q, uint4 k) {
    float s = __uint_as_float(q.x) * __uint_as_float(k.x);
    s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
    s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
    return fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
  }
  __device__ static void widen(uint4 v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static void store(void* base, size_t i, float x) { static_cast<float*>(base)[i] = x; }
};

template <>
struct Elem<kF16> {
  static constexpr int VEC = 8;
  __device__ static float dot(uint4 q, uint4 k) {
    float s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, q.x), __builtin_bit_cast(h2_t, k.x), 0.f, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, q.y), __builtin_bit_cast(h2_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, q.z), __builtin_bit_cast(h2_t, k.z), s, false);
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, q.w), __builtin_bit_cast(h2_t, k.w), s, false);
  }
  __device__ static void widen2(uint32_t w, float* f) {
    const h2_t h = __builtin_bit_cast(h2_t, w);
    f[0] = static_cast<float>(h.x);
    f[1] = static_cast<float>(h.y);
  }
  __device__ static void widen(uint4 v, float* f) {
    widen2(v.x, f);
    widen2(v.y, f + 2);
    widen2(v.z, f + 4);
    widen2(v.w, f + 6);
  }
  __device__ static void store(void* base, size_t i, float x) {
    static_cast<_Float16*>(base)[i] = static_cast<_Float16>(x);
  }
};

template <>
struct Elem<kBF16> {
  static constexpr int VEC = 8;
  __device__ static float dot(uint4 q, uint4 k) {
    float s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, q.x), __builtin_bit_cast(b2_t, k.x), 0.f, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, q.y), __builtin_bit_cast(b2_t, k.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, q.z), __builtin_bit_cast(b2_t, k.z), s, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2_t, q.w), __builtin_bit_cast(b2_t, k.w), s, false);
  }
  // bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32 bits.
  __device__ static void widen2(uint32_t w, float* f) {
    f[0] = __uint_as_float(w << 16);
    f[1] = __uint_as_float(w & 0xFFFF0000u);
  }
  __device__ static void widen(uint4 v, float* f) {
    widen2(v.x, f);
    widen2(v.y, f + 2);
    widen2(v.z, f + 4);
    widen2(v.w, f + 6);
  }
  __device__ static void store(void* base, size_t i, float x) {
    static_cast<__bf16*>(base)[i] = static_cast<__bf16>(x);  // round to nearest even
  }
};

__device__ __forceinline__ uint4 ld16(const char* p) { return *reinterpret_cast<const uint4*>(p); }

// Streaming 128-bit load for K/V: each byte is read exactly once per call,
// so the load is marked non-temporal (global_load_dwordx4 ... nt).  On MI355X
// this lifts a streaming read from ~6.0 to ~6.8-7.0 TB/s.
typedef uint32_t u32x4_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const char* p) {
  return __builtin_bit_cast(uint4,
                            __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt_t*>(p)));
}

// Keys row b holds: seqlens[b] clamped to [0, Nkv], or Nkv without seqlens.
__device__ __forceinline__ int row_keys(const Args& a, int b) {
  if (!a.seqlens) return a.Nkv;
  return min(max(a.seqlens[b], 0), a.Nkv);
}

// Row addressing of one (batch row b, KV head g) stream for a workgroup whose
// keys are [ks, ke).  k(r) / v(r) return the first byte of key row r; callers
// add their column offset.  The paged form stages the page ids of [ks, ke)
// in LDS (`pages`, kMaxSplitPages entries) and synchronises the workgroup,
// so init() must be reached by every thread of the workgroup.
template <int LAYOUT, int ROWB, int ES>
struct KvRows {
  const char* kb;
  const char* vb;
  long long krs, vrs;   // row strides in bytes (strided / paged)
  long long kps, vps;   // page strides in bytes (paged)
  const int* pages;
  int ps, pm, p0;

  __device__ __forceinline__ void init(const Args& a, int b, int g, int ks, int ke, int* lds_pages) {
    const char* k = static_cast<const char*>(a.k);
    const char* v = static_cast<const char*>(a.v);
    if constexpr (LAYOUT == kKvContig) {
      const size_t slab = (static_cast<size_t>(b) * a.H_kv + g) * static_cast<size_t>(a.Nkv) * ROWB;
      kb = k + slab;
      vb = v + slab;
    } else if constexpr (LAYOUT == kKvStrided) {
      kb = k + (b * a.k_bs + g * a.k_hs) * ES;
      vb = v + (b * a.v_bs + g * a.v_hs) * ES;
      krs = a.k_rs * ES;
      vrs = a.v_rs * ES;
    } else {
      kb = k + g * a.k_hs * ES;
      vb = v + g * a.v_hs * ES;
      krs = a.k_rs * ES;
      vrs = a.v_rs * ES;
      kps = a.k_bs * ES;
      vps = a.v_bs * ES;
      ps = a.page_shift;
      pm = (1 << a.page_shift) - 1;
      p0 = ks >> a.page_shift;
      const int n = ke > ks ? ((ke - 1) >> a.page_shift) - p0 + 1 : 0;
      const int32_t* bt = a.block_table + static_cast<size_t>(b) * a.bt_stride + p0;
      for (int i = threadIdx.x; i < n; i += blockDim.x)
        lds_pages[i] = min(max(bt[i], 0), a.num_pages - 1);
      pages = lds_pages;
      __syncthreads();
    }
  }
  __device__ __forceinline__ const char* k(int r) const {
    if constexpr (LAYOUT == kKvContig) return kb + static_cast<size_t>(r) * ROWB;
    else if constexpr (LAYOUT == kKvStrided) return kb + r * krs;
    else return kb + pages[(r >> ps) - p0] * kps + (r & pm) * krs;
  }
  __device__ __forceinline__ const char* v(int r) const {
    if constexpr (LAYOUT == kKvContig) return vb + static_cast<size_t>(r) * ROWB;
    else if constexpr (LAYOUT == kKvStrided) return vb + r * vrs;
    else return vb + pages[(r >> ps) - p0] * vps + (r & pm) * vrs;
  }
};

}  // namespace detail
}  // namespace sha
