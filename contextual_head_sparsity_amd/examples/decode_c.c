/*
 * Selective head attention decode called from plain C through the library's
 * C ABI (include/sha.h): device buffers from hipMalloc, a head-indexed call
 * and a group-indexed call on the default stream, no Python anywhere.
 *
 * Check: with q = 0 every score is 0, the softmax weights are uniform and
 * the selected heads' outputs equal the mean of their V rows (the closed
 * form of attention with equal scores).  Slots the index does not select
 * must keep the NaN payload they were filled with, bit for bit.  Exit
 * status 0 when both calls pass.
 *
 * Build: cc -std=c11 -I<repo>/include -I/opt/rocm/include -D__HIP_PLATFORM_AMD__
 *        decode_c.c -L<package dir> -lsha -L/opt/rocm/lib -lamdhip64
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sha.h"

#define SENTINEL 0x7FC5A5A5u

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

/* Small deterministic values in [-1, 1). */
static float next_value(uint32_t* s) {
  *s = *s * 1664525u + 1013904223u;
  return (float)((*s >> 8) & 0xFFFF) / 32768.0f - 1.0f;
}

/* One call: B rows, H query heads, H_kv K/V heads, Nkv keys of d floats;
 * index [B, top_k] names heads (gqa = 0) or groups (gqa = 1). */
static int run_case(int gqa, int B, int H, int H_kv, int Nkv, int d, int top_k,
                    const int32_t* index) {
  const size_t nq = (size_t)B * H * d, nkv = (size_t)B * H_kv * Nkv * d;
  float* hq = calloc(nq, sizeof(float));          /* q = 0 */
  float* hk = malloc(nkv * sizeof(float));
  float* hv = malloc(nkv * sizeof(float));
  uint32_t* ho = malloc(nq * sizeof(uint32_t));
  uint32_t seed = 12345u + (uint32_t)gqa;
  int ok = 1;
  for (size_t i = 0; i < nkv; ++i) hk[i] = next_value(&seed);
  for (size_t i = 0; i < nkv; ++i) hv[i] = next_value(&seed);
  for (size_t i = 0; i < nq; ++i) ho[i] = SENTINEL;

  void *dq = NULL, *dk = NULL, *dv = NULL, *dout = NULL, *didx = NULL;
  ok = hip_ok(hipMalloc(&dq, nq * sizeof(float)), "hipMalloc q") &&
       hip_ok(hipMalloc(&dk, nkv * sizeof(float)), "hipMalloc k") &&
       hip_ok(hipMalloc(&dv, nkv * sizeof(float)), "hipMalloc v") &&
       hip_ok(hipMalloc(&dout, nq * sizeof(float)), "hipMalloc o") &&
       hip_ok(hipMalloc(&didx, (size_t)B * top_k * sizeof(int32_t)), "hipMalloc index") &&
       hip_ok(hipMemcpy(dq, hq, nq * sizeof(float), hipMemcpyHostToDevice), "copy q") &&
       hip_ok(hipMemcpy(dk, hk, nkv * sizeof(float), hipMemcpyHostToDevice), "copy k") &&
       hip_ok(hipMemcpy(dv, hv, nkv * sizeof(float), hipMemcpyHostToDevice), "copy v") &&
       hip_ok(hipMemcpy(dout, ho, nq * sizeof(float), hipMemcpyHostToDevice), "copy o") &&
       hip_ok(hipMemcpy(didx, index, (size_t)B * top_k * sizeof(int32_t),
                        hipMemcpyHostToDevice), "copy index");
  if (ok) {
    const float scale = 1.0f / sqrtf((float)d);
    const sha_status st =
        gqa ? sha_decode_gqa_f32(dq, dk, dv, (const int32_t*)didx, B, H, H_kv, Nkv, d, top_k,
                                 scale, dout, NULL)
            : sha_decode_f32(dq, dk, dv, (const int32_t*)didx, B, H, H_kv, Nkv, d, top_k, scale,
                             dout, NULL);
    if (st != SHA_OK) {
      fprintf(stderr, "sha_decode%s_f32: %s\n", gqa ? "_gqa" : "", sha_status_string(st));
      ok = 0;
    }
  }
  ok = ok && hip_ok(hipDeviceSynchronize(), "synchronize") &&
       hip_ok(hipMemcpy(ho, dout, nq * sizeof(float), hipMemcpyDeviceToHost), "copy o back");

  if (ok) {
    const int G = H / H_kv;
    double max_err = 0.0;
    int selected_slots = 0;
    for (int b = 0; b < B && ok; ++b)
      for (int h = 0; h < H && ok; ++h) {
        int selected = 0;
        for (int k = 0; k < top_k; ++k)
          selected |= gqa ? (index[b * top_k + k] == h / G) : (index[b * top_k + k] == h);
        const uint32_t* out = ho + ((size_t)b * H + h) * d;
        if (!selected) {
          for (int c = 0; c < d; ++c)
            if (out[c] != SENTINEL) {
              fprintf(stderr, "unselected slot (%d, %d) was written\n", b, h);
              ok = 0;
              break;
            }
          continue;
        }
        ++selected_slots;
        const float* vr = hv + ((size_t)b * H_kv + h / G) * Nkv * d;
        for (int c = 0; c < d; ++c) {
          double mean = 0.0;
          for (int n = 0; n < Nkv; ++n) mean += vr[(size_t)n * d + c];
          mean /= Nkv;
          float got;
          memcpy(&got, &out[c], sizeof(float));
          const double err = fabs((double)got - mean);
          if (!(err <= 1e-5)) ok = 0;
          if (err > max_err || err != err) max_err = err;
        }
      }
    printf("%s: %d selected slots, max |O - mean V| = %.3e, unselected slots untouched: %s\n",
           gqa ? "group-indexed" : "head-indexed", selected_slots, max_err, ok ? "yes" : "no");
  }
  hipFree(dq);
  hipFree(dk);
  hipFree(dv);
  hipFree(dout);
  hipFree(didx);
  free(hq);
  free(hk);
  free(hv);
  free(ho);
  return ok;
}

int main(void) {
  /* Head-indexed: 2 rows, 6 heads, 2 selected per row; 3000 keys make the
   * library split the keys (and use its own workspace and combine). */
  const int32_t heads[4] = {1, 4, 0, 5};
  /* Group-indexed: 8 query heads in 2 groups of 4, one group per row. */
  const int32_t groups[2] = {1, 0};
  const int ok = run_case(0, 2, 6, 6, 3000, 64, 2, heads) &&
                 run_case(1, 2, 8, 2, 777, 128, 1, groups);
  printf("%s\n", ok ? "PASS" : "FAIL");
  return ok ? 0 : 1;
}
