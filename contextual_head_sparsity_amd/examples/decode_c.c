/*
 * The library's C ABI (include/sha.h) from plain C: device buffers from
 * hipMalloc, calls on the default stream, no Python anywhere.
 *
 * 1. Selective head attention, head-indexed and group-indexed.  With q = 0
 *    every score is 0, the softmax weights are uniform and the selected
 *    heads' outputs equal the mean of their V rows (the closed form of
 *    attention with equal scores).  Slots the index does not select must
 *    keep the NaN payload they were filled with, bit for bit.
 * 2. The sparse layer's other calls, on exact inputs: the attention router
 *    with unit-vector weight rows (scores = the hidden state's first H
 *    entries, so the top-k is known), its index then used for a decode
 *    call; the router's K-split form with a caller workspace (f16 small
 *    integers over two hidden chunks, exact scores and top-k); the batch
 *    union of the rows' neuron lists (with -1 padding); and
 *    the selective MLP on small integers (x in {0, 1}, weights in
 *    {-1, 0, 1}), whose every intermediate and output is an integer that
 *    f16 and fp32 hold exactly, so the check is equality.
 * Exit status 0 when every call passes.
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

/* IEEE half bits of an integer n with |n| <= 2048 (exact). */
static uint16_t half_of_int(int n) {
  if (n == 0) return 0;
  const uint16_t sign = n < 0 ? 0x8000u : 0u;
  unsigned m = (unsigned)(n < 0 ? -n : n);
  int e = 0;
  while ((m >> (e + 1)) != 0) ++e;                 /* m in [2^e, 2^(e+1)) */
  const unsigned frac = (e <= 10 ? m << (10 - e) : m >> (e - 10)) & 0x3FFu;  /* exact for m <= 2048 */
  return (uint16_t)(sign | (unsigned)((e + 15) << 10) | frac);
}

/* Value of half bits (normal numbers and zero, all these checks produce). */
static double int_of_half(uint16_t h) {
  const int e = (h >> 10) & 0x1F;
  const double frac = (double)(h & 0x3FF) / 1024.0;
  const double v = e == 0 ? frac * ldexp(1.0, -14) : (1.0 + frac) * ldexp(1.0, e - 15);
  return (h & 0x8000u) ? -v : v;
}

/* Router -> decode: scores[b, h] = x[b, h] (w rows are unit vectors), the
 * top 2 of 6 heads per row, ascending, then a head-indexed decode call on
 * that index (q = 0: outputs are the mean of V). */
static int run_router(void) {
  enum { B = 2, D = 8, H = 6, K = 2 };
  const float hx[B * D] = {0.5f, 3.f, -1.f, 2.f, 7.f, 1.f, 9.f, 9.f,
                           4.f, 4.f, -2.f, 0.f, 6.f, 5.f, 9.f, 9.f};
  /* row 0: heads 4 (7) and 1 (3); row 1: heads 4 (6) and 5 (5) */
  const int32_t want[B * K] = {1, 4, 4, 5};
  float hw[H * D];
  memset(hw, 0, sizeof(hw));
  for (int h = 0; h < H; ++h) hw[h * D + h] = 1.0f;
  float* dx = NULL;
  float* dw = NULL;
  float* dsc = NULL;
  int32_t* didx = NULL;
  int ok = hip_ok(hipMalloc((void**)&dx, sizeof(hx)), "hipMalloc x") &&
           hip_ok(hipMalloc((void**)&dw, sizeof(hw)), "hipMalloc w") &&
           hip_ok(hipMalloc((void**)&dsc, B * H * sizeof(float)), "hipMalloc scores") &&
           hip_ok(hipMalloc((void**)&didx, B * K * sizeof(int32_t)), "hipMalloc index") &&
           hip_ok(hipMemcpy(dx, hx, sizeof(hx), hipMemcpyHostToDevice), "copy x") &&
           hip_ok(hipMemcpy(dw, hw, sizeof(hw), hipMemcpyHostToDevice), "copy w");
  if (ok) {
    const sha_status st = sha_router_topk(dx, dw, NULL, B, D, H, K, didx, dsc, NULL, SHA_F32);
    if (st != SHA_OK) {
      fprintf(stderr, "sha_router_topk: %s\n", sha_status_string(st));
      ok = 0;
    }
  }
  int32_t got[B * K];
  float sc[B * H];
  ok = ok && hip_ok(hipDeviceSynchronize(), "synchronize") &&
       hip_ok(hipMemcpy(got, didx, sizeof(got), hipMemcpyDeviceToHost), "copy index back") &&
       hip_ok(hipMemcpy(sc, dsc, sizeof(sc), hipMemcpyDeviceToHost), "copy scores back");
  if (ok) {
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        if (sc[b * H + h] != hx[b * D + h]) ok = 0;
    for (int i = 0; i < B * K; ++i)
      if (got[i] != want[i]) ok = 0;
    printf("router: index [%d %d | %d %d], scores exact: %s\n", got[0], got[1], got[2], got[3],
           ok ? "yes" : "no");
  }
  /* The router's index (the host copy made above) drives a head-indexed
   * decode call, checked like the first case. */
  if (ok) ok = run_case(0, B, H, H, 300, 64, K, got);
  hipFree(dx);
  hipFree(dw);
  hipFree(dsc);
  hipFree(didx);
  return ok;
}

/* Union -> selective MLP (f16): y = relu(x W1[:, S]) W2[:, S]^T on
 * integers, checked exactly against the same sums on the host. */
static int run_mlp(void) {
  enum { B = 2, d = 256, Dn = 40, k = 4 };
  const int32_t rows[B * k] = {7, 3, 30, -1, 3, 12, 39, 7};   /* S = {3, 7, 12, 30, 39} */
  const int32_t want_sel[5] = {3, 7, 12, 30, 39};
  uint16_t hx[B * d], hw1[Dn * d], hw2[Dn * d], hy[B * d];
  int x[B * d], w1[Dn * d], w2[Dn * d];
  /* x: 85 or 86 ones per row; w1 in {-1, 0, 1, 2} (mean 1/2, so most
   * activations are positive); w2 in {-1, 0, 1}.  |h| <= 172 and
   * |y| <= 5 * 172 = 860: integers that f16 and fp32 hold exactly. */
  for (int i = 0; i < B * d; ++i) x[i] = i % 3 == 0;
  for (int i = 0; i < Dn * d; ++i) {
    w1[i] = (i * 5 + i / 7) % 4 - 1;
    w2[i] = (i * 11 + i / 3) % 3 - 1;
  }
  for (int i = 0; i < B * d; ++i) hx[i] = half_of_int(x[i]);
  for (int i = 0; i < Dn * d; ++i) {
    hw1[i] = half_of_int(w1[i]);
    hw2[i] = half_of_int(w2[i]);
  }
  const size_t uws = sha_mlp_union_workspace_bytes(Dn);
  const int n_max = B * k < Dn ? B * k : Dn;
  const size_t mws = sha_selective_mlp_workspace_bytes(B, d, Dn, n_max, 0);
  void *dx = NULL, *dw1 = NULL, *dw2 = NULL, *dy = NULL, *du = NULL, *dm = NULL;
  int32_t *drows = NULL, *dsel = NULL, *dn = NULL;
  int ok = hip_ok(hipMalloc(&dx, sizeof(hx)), "hipMalloc x") &&
           hip_ok(hipMalloc(&dw1, sizeof(hw1)), "hipMalloc w1t") &&
           hip_ok(hipMalloc(&dw2, sizeof(hw2)), "hipMalloc w2t") &&
           hip_ok(hipMalloc(&dy, sizeof(hy)), "hipMalloc y") &&
           hip_ok(hipMalloc(&du, uws), "hipMalloc union workspace") &&
           hip_ok(hipMalloc(&dm, mws), "hipMalloc mlp workspace") &&
           hip_ok(hipMalloc((void**)&drows, sizeof(rows)), "hipMalloc rows") &&
           hip_ok(hipMalloc((void**)&dsel, n_max * sizeof(int32_t)), "hipMalloc sel") &&
           hip_ok(hipMalloc((void**)&dn, sizeof(int32_t)), "hipMalloc n_sel") &&
           hip_ok(hipMemcpy(dx, hx, sizeof(hx), hipMemcpyHostToDevice), "copy x") &&
           hip_ok(hipMemcpy(dw1, hw1, sizeof(hw1), hipMemcpyHostToDevice), "copy w1t") &&
           hip_ok(hipMemcpy(dw2, hw2, sizeof(hw2), hipMemcpyHostToDevice), "copy w2t") &&
           hip_ok(hipMemcpy(drows, rows, sizeof(rows), hipMemcpyHostToDevice), "copy rows");
  if (ok) {
    sha_status st = sha_mlp_union(drows, B, k, Dn, dsel, dn, NULL, du, uws);
    if (st == SHA_OK)
      st = sha_selective_mlp(dx, dw1, dw2, dsel, dn, n_max, B, d, Dn, dy, NULL, SHA_F16, dm, mws);
    if (st != SHA_OK) {
      fprintf(stderr, "union / selective MLP: %s\n", sha_status_string(st));
      ok = 0;
    }
  }
  int32_t sel[8], n_sel = 0;
  ok = ok && hip_ok(hipDeviceSynchronize(), "synchronize") &&
       hip_ok(hipMemcpy(&n_sel, dn, sizeof(int32_t), hipMemcpyDeviceToHost), "copy n_sel back") &&
       hip_ok(hipMemcpy(sel, dsel, n_max * sizeof(int32_t), hipMemcpyDeviceToHost), "copy sel") &&
       hip_ok(hipMemcpy(hy, dy, sizeof(hy), hipMemcpyDeviceToHost), "copy y back");
  if (ok) {
    ok = n_sel == 5;
    for (int i = 0; ok && i < 5; ++i) ok = sel[i] == want_sel[i];
    long worst = 0;
    for (int b = 0; ok && b < B; ++b)
      for (int c = 0; c < d; ++c) {
        long y = 0;
        for (int s = 0; s < 5; ++s) {
          const int j = want_sel[s];
          long h = 0;
          for (int t = 0; t < d; ++t) h += (long)x[b * d + t] * w1[j * d + t];
          if (h < 0) h = 0;
          y += h * w2[j * d + c];
        }
        const double got = int_of_half(hy[b * d + c]);
        if (labs(y) > worst) worst = labs(y);
        if (got != (double)y) {
          fprintf(stderr, "y[%d, %d] = %g, want %ld\n", b, c, got, y);
          ok = 0;
          break;
        }
      }
    if (worst < 50) {
      fprintf(stderr, "selective MLP check is degenerate (max |y| = %ld)\n", worst);
      ok = 0;
    }
    printf("union: %d neurons [%d %d %d %d %d]; selective MLP: y exact (max |y| = %ld): %s\n",
           n_sel, sel[0], sel[1], sel[2], sel[3], sel[4], worst, ok ? "yes" : "no");
  }
  hipFree(dx);
  hipFree(dw1);
  hipFree(dw2);
  hipFree(dy);
  hipFree(du);
  hipFree(dm);
  hipFree(drows);
  hipFree(dsel);
  hipFree(dn);
  return ok;
}

/* f16 bit pattern of a small integer (|n| < 2048: exact). */
static uint16_t f16_bits(int n) {
  if (n == 0) return 0;
  const uint16_t sign = n < 0 ? 0x8000u : 0u;
  unsigned m = (unsigned)(n < 0 ? -n : n);
  int e = 0;
  while ((m >> (e + 1)) != 0) ++e;
  return (uint16_t)(sign | (unsigned)(15 + e) << 10 | ((m - (1u << e)) << (10 - e)));
}

/* The router's K-split form through sha_router_topk_ex with a hipMalloc'd
 * workspace of sha_router_split_bytes: f16 hidden states of small integers
 * over 264 hidden elements (two 256-element chunks, the second holding one
 * 8-element piece); head h's weight row holds 1 at elements h and 256 + h,
 * so scores[b, h] = x[b, h] + x[b, 256 + h] exactly, a sum of the two
 * chunks' partials. */
static int run_router_split(void) {
  enum { B = 2, D = 264, H = 6, K = 3 };
  const int xa[B][H] = {{1, 5, -2, 7, 0, 3}, {4, -1, 6, 2, 9, 2}};   /* elements 0..5 */
  const int xb[B][H] = {{2, -1, 8, 0, 1, 3}, {0, 3, -3, 1, -2, 5}};  /* elements 256..261 */
  /* scores row 0: 3 4 6 7 1 6 -> heads 2, 3, 5 (ties: lower id first);
   *        row 1: 4 2 3 3 7 7 -> heads 0, 4, 5 */
  const int32_t want[B * K] = {2, 3, 5, 0, 4, 5};
  uint16_t hx[B * D], hw[H * D];
  memset(hx, 0, sizeof(hx));
  memset(hw, 0, sizeof(hw));
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      hx[b * D + h] = f16_bits(xa[b][h]);
      hx[b * D + 256 + h] = f16_bits(xb[b][h]);
    }
  for (int h = 0; h < H; ++h) hw[h * D + h] = hw[h * D + 256 + h] = f16_bits(1);
  const size_t ws_bytes = sha_router_split_bytes(B, D, H, SHA_F16);
  void *dx = NULL, *dw = NULL, *dws = NULL;
  float* dsc = NULL;
  int32_t* didx = NULL;
  int ok = ws_bytes == (size_t)256 &&   /* 2 rows x 2 chunks x 6 heads x 4 B, rounded */
           hip_ok(hipMalloc(&dx, sizeof(hx)), "hipMalloc x") &&
           hip_ok(hipMalloc(&dw, sizeof(hw)), "hipMalloc w") &&
           hip_ok(hipMalloc(&dws, ws_bytes), "hipMalloc workspace") &&
           hip_ok(hipMalloc((void**)&dsc, B * H * sizeof(float)), "hipMalloc scores") &&
           hip_ok(hipMalloc((void**)&didx, B * K * sizeof(int32_t)), "hipMalloc index") &&
           hip_ok(hipMemcpy(dx, hx, sizeof(hx), hipMemcpyHostToDevice), "copy x") &&
           hip_ok(hipMemcpy(dw, hw, sizeof(hw), hipMemcpyHostToDevice), "copy w");
  if (ok) {
    /* a workspace one byte short is refused before any launch */
    ok = sha_router_topk_ex(dx, dw, NULL, B, D, H, K, didx, dsc, NULL, SHA_F16, dws,
                            ws_bytes - 1) == SHA_ERR_WORKSPACE;
    const sha_status st =
        sha_router_topk_ex(dx, dw, NULL, B, D, H, K, didx, dsc, NULL, SHA_F16, dws, ws_bytes);
    if (st != SHA_OK) {
      fprintf(stderr, "sha_router_topk_ex: %s\n", sha_status_string(st));
      ok = 0;
    }
  }
  int32_t got[B * K];
  float sc[B * H];
  ok = ok && hip_ok(hipDeviceSynchronize(), "synchronize") &&
       hip_ok(hipMemcpy(got, didx, sizeof(got), hipMemcpyDeviceToHost), "copy index back") &&
       hip_ok(hipMemcpy(sc, dsc, sizeof(sc), hipMemcpyDeviceToHost), "copy scores back");
  if (ok) {
    for (int b = 0; b < B; ++b)
      for (int h = 0; h < H; ++h)
        if (sc[b * H + h] != (float)(xa[b][h] + xb[b][h])) ok = 0;
    for (int i = 0; i < B * K; ++i)
      if (got[i] != want[i]) ok = 0;
    printf("router (K-split, caller workspace): index [%d %d %d | %d %d %d], split scores "
           "exact: %s\n",
           got[0], got[1], got[2], got[3], got[4], got[5], ok ? "yes" : "no");
  }
  hipFree(dx);
  hipFree(dw);
  hipFree(dws);
  hipFree(dsc);
  hipFree(didx);
  return ok;
}

int main(void) {
  /* Head-indexed: 2 rows, 6 heads, 2 selected per row; 3000 keys make the
   * library split the keys (and use its own workspace and combine). */
  const int32_t heads[4] = {1, 4, 0, 5};
  /* Group-indexed: 8 query heads in 2 groups of 4, one group per row. */
  const int32_t groups[2] = {1, 0};
  const int ok = run_case(0, 2, 6, 6, 3000, 64, 2, heads) &&
                 run_case(1, 2, 8, 2, 777, 128, 1, groups) && run_router() &&
                 run_router_split() && run_mlp();
  printf("%s\n", ok ? "PASS" : "FAIL");
  return ok ? 0 : 1;
}
