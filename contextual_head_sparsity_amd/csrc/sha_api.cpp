// C ABI of the SHA decode library: host-side validation, split planning,
// workspace handling and launch.  Declarations and the contract of every
// entry point are in include/sha.h.
#include "sha.h"

#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "sha_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

constexpr int kMaxGroup = 64;

struct Problem {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* idx;
  void* o;
  int B, H, H_kv, Nkv, d, top_k;
  float scale;
  int dtype;
  bool gqa;
  const sha_kv_layout* kv;  // null: contiguous [B, H_kv, Nkv, d], every row Nkv keys
};

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Scalar checks, in a fixed order; `empty` is set for B == 0 or top_k == 0.
sha_status check_scalars(int B, int H, int H_kv, int Nkv, int d, int top_k, int gqa, int dtype,
                         bool* empty) {
  *empty = false;
  if (B < 0 || top_k < 0 || H < 1 || H_kv < 1 || Nkv < 1 || d < 1) return SHA_ERR_INVALID_ARG;
  if (H % H_kv != 0) return SHA_ERR_INVALID_ARG;
  if (dtype != SHA_F32 && dtype != SHA_F16 && dtype != SHA_BF16) return SHA_ERR_UNSUPPORTED;
  if (d != 64 && d != 128) return SHA_ERR_UNSUPPORTED;
  if (gqa && H / H_kv > kMaxGroup) return SHA_ERR_UNSUPPORTED;
  if (top_k > (gqa ? H_kv : H)) return SHA_ERR_INVALID_ARG;
  if (B == 0 || top_k == 0) *empty = true;
  return SHA_OK;
}

int device_cus(int num_cus) {
  if (num_cus > 0) return num_cus;
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

// Tuning hooks for sweeps: SHA_MHA_VARIANT / SHA_GQA_VARIANT pick a kernel
// shape from the table in sha_kernels.hip (0 = default).
int env_int(const char* name, int dflt) {
  const char* s = getenv(name);
  return s ? atoi(s) : dflt;
}
int mha_variant() {
  static const int v = env_int("SHA_MHA_VARIANT", 0);
  return v;
}
int gqa_variant() {
  static const int v = env_int("SHA_GQA_VARIANT", 0);
  return v;
}
// Group calls in f16 / bf16 run on the matrix cores; SHA_GQA_VALU=1 selects
// the vector-ALU kernel instead (for comparisons).
bool gqa_mfma(int dtype) {
  static const bool force_valu = env_int("SHA_GQA_VALU", 0) != 0;
  return dtype != SHA_F32 && !force_valu;
}

// Workgroups one split of the whole call launches.
long long wgs_per_split(int B, int H, int H_kv, int top_k, int gqa, int dtype) {
  long long per_unit = 1;
  if (gqa) {
    const int G = H / H_kv;
    const int nh = sha::gqa_heads_per_wg(G, gqa_mfma(dtype));
    per_unit = G == 1 ? 1 : (G + nh - 1) / nh;
  }
  return static_cast<long long>(B) * top_k * per_unit;
}

// Split count (flash-decoding split-K over the keys), from measurements on
// MI355X.  No split is shorter than kMinSplitKeys keys.
//
// Head-indexed workgroups (4 waves, 16 KiB of loads in flight per wave)
// stream ~22 GB/s each, so about one workgroup per CU saturates HBM and
// splitting further only adds partials and tail.
//
// The matrix-core group kernel runs with 4-wave workgroups (2 resident per
// CU) or, when one split already has at least one workgroup per CU, 2-wave
// workgroups (4 per CU, the same waves): with many units the smaller
// workgroups fill the last round better (LLaMA-3.1-70B layer: 202 against
// 208 us; 128 rows of 1 K keys: 58 against 65 us), with few units they
// stream slower.  Its best split count swings with how the last round of
// workgroups fills the chip, so it is chosen with a round model of the
// grid: rounds of slots-per-CU x CUs resident workgroups, each streaming at
// most a per-workgroup rate while all of them share kGqaHbmGBs, plus
// kGqaRoundUs of start-up and drain per round and nothing extra for the
// combine.  The 4-wave constants are a fit to 99 timed (shape, split) pairs
// (8-1024 units, 1 K-32 K keys), whose picks are within ~2% of the best
// measured split on average; the 2-wave rate was fitted the same way.
constexpr int kMinSplitKeys = 512;
constexpr int kMaxSplits = 64;
constexpr double kGqaHbmGBs = 6800.0;
constexpr double kGqaRoundUs = 4.0;

struct GqaShape {
  int waves;         // waves per workgroup
  int slots_per_cu;  // resident workgroups per CU
  double wg_gbs;     // streaming rate of one workgroup
};
constexpr GqaShape kGqaWide{4, 2, 20.0};
constexpr GqaShape kGqaNarrow{2, 4, 13.0};

void split_geometry(int Nkv, int nsplit_req, int page, int* nsplit, int* chunk);

// Modelled time (us) of the group kernel with `ns` splits.
double gqa_round_model_us(long long wgs, int Nkv, int d, int ns, int cus, const GqaShape& sh,
                          int* ns_eff) {
  int chunk = Nkv;
  split_geometry(Nkv, ns, 0, ns_eff, &chunk);
  const long long T = wgs * *ns_eff;
  const long long slots = static_cast<long long>(sh.slots_per_cu) * cus;
  const double bytes = 4.0 * chunk * d;  // K + V rows of one workgroup, 16-bit
  const double full_rate = std::min(kGqaHbmGBs, sh.wg_gbs * static_cast<double>(slots));
  const long long full = T / slots, rem = T % slots;
  double t = static_cast<double>(full) *
             (bytes * static_cast<double>(slots) / full_rate / 1e3 + kGqaRoundUs);
  if (rem > 0) {
    const double rate = std::min(sh.wg_gbs, kGqaHbmGBs / static_cast<double>(rem));
    t += bytes / rate / 1e3 + kGqaRoundUs;
  }
  return t;
}

// Best modelled split count of one workgroup shape (*t_best: its time).
int gqa_best_split(long long wgs, int Nkv, int d, int cus, const GqaShape& sh, long long max_ns,
                   double* t_best) {
  int ns = 1;
  double best = 0.0;
  for (int c = 1; c <= max_ns; ++c) {
    int eff = 1;
    const double t = gqa_round_model_us(wgs, Nkv, d, c, cus, sh, &eff);
    if (eff != c) continue;  // same geometry as a smaller request
    if (c == 1 || t < best) {
      best = t;
      ns = c;
    }
  }
  *t_best = best;
  return ns;
}

long long max_splits(int Nkv) {
  long long max_ns = Nkv / kMinSplitKeys > 1 ? Nkv / kMinSplitKeys : 1;
  return max_ns > kMaxSplits ? kMaxSplits : max_ns;
}

// Workgroup shape of the matrix-core group kernel for one problem (it does
// not depend on a requested split count).  2-wave workgroups only where a
// split already has a workgroup per CU and the model puts them at least 1%
// ahead (with few units they stream slower than the model says).
GqaShape gqa_shape(long long wgs, int Nkv, int d, int cus) {
  const int env = env_int("SHA_GQA_WAVES", 0);  // tuning hook: 2 or 4
  if (env == 2) return kGqaNarrow;
  if (env == 4) return kGqaWide;
  if (wgs < cus) return kGqaWide;
  double t_wide = 0.0, t_narrow = 0.0;
  gqa_best_split(wgs, Nkv, d, cus, kGqaWide, max_splits(Nkv), &t_wide);
  gqa_best_split(wgs, Nkv, d, cus, kGqaNarrow, max_splits(Nkv), &t_narrow);
  return t_narrow < 0.99 * t_wide ? kGqaNarrow : kGqaWide;
}

int plan_nsplit(int B, int H, int H_kv, int Nkv, int d, int top_k, int gqa, int dtype,
                int num_cus) {
  const long long wgs = wgs_per_split(B, H, H_kv, top_k, gqa, dtype);
  if (wgs <= 0) return 1;
  const int cus = device_cus(num_cus);
  const bool mfma = gqa && H / H_kv > 1 && gqa_mfma(dtype);
  const long long max_ns = max_splits(Nkv);
  long long ns = 1;
  if (mfma) {
    double t = 0.0;
    ns = gqa_best_split(wgs, Nkv, d, cus, gqa_shape(wgs, Nkv, d, cus), max_ns, &t);
  } else {
    ns = (cus + wgs - 1) / wgs;
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
  }
  const int env = env_int("SHA_NSPLIT", 0);
  if (env > 0) ns = env;
  return static_cast<int>(ns);
}

// Effective split geometry: `chunk` keys per split (when there is more than
// one split: a multiple of 16 keys, of 128 keys for splits of 512 keys or
// more, and of the page size for a paged cache), every split non-empty.  A paged cache (page > 0) also keeps every
// split within sha::kMaxSplitPages pages, the page ids a workgroup stages.
void split_geometry(int Nkv, int nsplit_req, int page, int* nsplit, int* chunk) {
  int ns = nsplit_req < 1 ? 1 : (nsplit_req > Nkv ? Nkv : nsplit_req);
  if (page > 0) {
    const long long span = static_cast<long long>(sha::kMaxSplitPages) * page;
    const int min_ns = static_cast<int>((Nkv + span - 1) / span);
    if (ns < min_ns) ns = min_ns;
  }
  if (ns == 1) {
    *nsplit = 1;
    *chunk = Nkv;
    return;
  }
  int c = (Nkv + ns - 1) / ns;
  // Splits of 512 keys or more end on a whole kernel iteration (128 keys:
  // 4 waves x 4 rows x 8 for the head kernel, 4 waves x 32-key tiles for the
  // group kernel), so that only the last split has a ragged tail.
  int align = c >= 512 ? 128 : 16;
  if (page > align) align = page;
  c = (c + align - 1) / align * align;
  *chunk = c;
  *nsplit = (Nkv + c - 1) / c;
}

// KV layout checks.  Sets *kind (sha::KvLayout) and *page (rows per page, 0
// unless paged).  A strided layout whose strides are the contiguous ones
// runs as contiguous.
sha_status check_kv(const sha_kv_layout* L, int H_kv, int Nkv, int d, int dtype, int* kind,
                    int* page) {
  *kind = sha::kKvContig;
  *page = 0;
  if (!L) return SHA_OK;
  const int64_t unit = dtype == SHA_F32 ? 4 : 8;  // elements per 16 bytes
  const int64_t st[6] = {L->k_batch_stride, L->k_head_stride, L->k_row_stride,
                         L->v_batch_stride, L->v_head_stride, L->v_row_stride};
  for (int64_t x : st) {
    if (x < 0 || x > (int64_t(1) << 40)) return SHA_ERR_INVALID_ARG;
    if (x % unit != 0) return SHA_ERR_MISALIGNED;
  }
  if (L->seqlens && !aligned(L->seqlens, 4)) return SHA_ERR_MISALIGNED;
  if (L->block_table) {
    const int P = L->page_size;
    if (P < 16 || P > 65536 || (P & (P - 1)) != 0) return SHA_ERR_INVALID_ARG;
    if (L->num_pages < 1) return SHA_ERR_INVALID_ARG;
    if (L->block_table_stride < (Nkv + P - 1) / P) return SHA_ERR_INVALID_ARG;
    if (!aligned(L->block_table, 4)) return SHA_ERR_MISALIGNED;
    const long long span = static_cast<long long>(sha::kMaxSplitPages) * P;
    if ((Nkv + span - 1) / span > kMaxSplits) return SHA_ERR_UNSUPPORTED;
    *kind = sha::kKvPaged;
    *page = P;
    return SHA_OK;
  }
  const int64_t rs = d, hs = static_cast<int64_t>(Nkv) * d, bs = hs * H_kv;
  const bool contig = L->k_batch_stride == bs && L->k_head_stride == hs && L->k_row_stride == rs &&
                      L->v_batch_stride == bs && L->v_head_stride == hs && L->v_row_stride == rs;
  *kind = contig ? sha::kKvContig : sha::kKvStrided;
  return SHA_OK;
}

size_t partial_bytes(int B, int H, int H_kv, int d, int top_k, int gqa, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t heads = gqa ? static_cast<size_t>(H / H_kv) : 1;
  const size_t n = static_cast<size_t>(B) * top_k * heads * nsplit;
  const size_t o_bytes = (n * d * sizeof(float) + 255) / 256 * 256;
  return o_bytes + n * 2 * sizeof(float);
}

sha_status run(const Problem& p, int nsplit_req, void* ws, size_t ws_bytes, hipStream_t stream);

// Internal workspace for the calls without an explicit workspace: one
// grow-only buffer per (device, stream).  A buffer that is
// outgrown is kept, not freed, until the process ends: work already queued
// on the stream, or a graph that captured a call, may still use it.  Growing
// needs an allocation, which a stream under capture cannot take: such a call
// returns SHA_ERR_WORKSPACE instead.
std::mutex g_ws_mutex;
std::map<std::pair<int, hipStream_t>, std::pair<void*, size_t>> g_ws;
std::vector<void*> g_ws_retired;

bool stream_capturing(hipStream_t stream) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return true;  // unknown: do not allocate
  }
  return cs != hipStreamCaptureStatusNone;
}

sha_status run_auto(const Problem& p, hipStream_t stream) {
  bool empty = false;
  sha_status st = check_scalars(p.B, p.H, p.H_kv, p.Nkv, p.d, p.top_k, p.gqa, p.dtype, &empty);
  if (st != SHA_OK || empty) return st;
  const int ns_plan = plan_nsplit(p.B, p.H, p.H_kv, p.Nkv, p.d, p.top_k, p.gqa, p.dtype, 0);
  int ns = 1, chunk = p.Nkv;
  split_geometry(p.Nkv, ns_plan, 0, &ns, &chunk);
  const bool gqa_eff = p.gqa && p.H / p.H_kv > 1;
  const size_t need = partial_bytes(p.B, p.H, p.H_kv, p.d, p.top_k, gqa_eff, ns);
  if (need == 0) return run(p, ns, nullptr, 0, stream);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = e;
    return SHA_ERR_HIP;
  }
  auto& slot = g_ws[{dev, stream}];
  if (slot.second < need) {
    if (stream_capturing(stream)) return SHA_ERR_WORKSPACE;
    void* ptr = nullptr;
    e = hipMalloc(&ptr, need);
    if (e != hipSuccess) {
      g_last_hip_error = e;
      return SHA_ERR_HIP;
    }
    if (slot.first) g_ws_retired.push_back(slot.first);
    slot = {ptr, need};
  }
  return run(p, ns, slot.first, slot.second, stream);
}

sha_status run(const Problem& p, int nsplit_req, void* ws, size_t ws_bytes, hipStream_t stream) {
  bool empty = false;
  sha_status st = check_scalars(p.B, p.H, p.H_kv, p.Nkv, p.d, p.top_k, p.gqa, p.dtype, &empty);
  if (st != SHA_OK || empty) return st;
  if (!p.q || !p.k || !p.v || !p.idx || !p.o) return SHA_ERR_INVALID_ARG;
  if (!(isfinite(p.scale))) return SHA_ERR_INVALID_ARG;
  if (!aligned(p.q, 16) || !aligned(p.k, 16) || !aligned(p.v, 16) || !aligned(p.o, 16) ||
      !aligned(p.idx, 4))
    return SHA_ERR_MISALIGNED;
  int kind = sha::kKvContig, page = 0;
  st = check_kv(p.kv, p.H_kv, p.Nkv, p.d, p.dtype, &kind, &page);
  if (st != SHA_OK) return st;

  const bool gqa_eff = p.gqa && p.H / p.H_kv > 1;
  int ns = 1, chunk = p.Nkv;
  const int req = nsplit_req > 0
                      ? nsplit_req
                      : plan_nsplit(p.B, p.H, p.H_kv, p.Nkv, p.d, p.top_k, p.gqa, p.dtype, 0);
  split_geometry(p.Nkv, req, page, &ns, &chunk);

  // Grid limit: blocks * threads per block (at most 512) must fit 32 bits.
  const long long blocks = wgs_per_split(p.B, p.H, p.H_kv, p.top_k, p.gqa, p.dtype) * ns;
  if (blocks > (1LL << 23)) return SHA_ERR_INVALID_ARG;

  sha::Args a{};
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.idx = p.idx;
  a.o = p.o;
  a.B = p.B;
  a.H = p.H;
  a.H_kv = p.H_kv;
  a.Nkv = p.Nkv;
  a.top_k = p.top_k;
  a.G = p.H / p.H_kv;
  a.nsplit = ns;
  a.chunk = chunk;
  a.waves = gqa_eff && gqa_mfma(p.dtype)
                ? gqa_shape(wgs_per_split(p.B, p.H, p.H_kv, p.top_k, p.gqa, p.dtype), p.Nkv, p.d,
                            device_cus(0)).waves
                : 4;
  a.scale_log2 = static_cast<float>(static_cast<double>(p.scale) * 1.4426950408889634);
  a.layout = kind;
  if (p.kv) {
    a.k_bs = p.kv->k_batch_stride;
    a.k_hs = p.kv->k_head_stride;
    a.k_rs = p.kv->k_row_stride;
    a.v_bs = p.kv->v_batch_stride;
    a.v_hs = p.kv->v_head_stride;
    a.v_rs = p.kv->v_row_stride;
    a.seqlens = p.kv->seqlens;
    if (kind == sha::kKvPaged) {
      a.block_table = p.kv->block_table;
      a.bt_stride = p.kv->block_table_stride;
      a.page_shift = __builtin_ctz(static_cast<unsigned>(page));
      a.num_pages = p.kv->num_pages;
    }
  }

  const size_t need = partial_bytes(p.B, p.H, p.H_kv, p.d, p.top_k, gqa_eff, ns);
  if (need > 0) {
    if (!ws || ws_bytes < need) return SHA_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return SHA_ERR_MISALIGNED;
    const size_t heads = gqa_eff ? static_cast<size_t>(a.G) : 1;
    const size_t n = static_cast<size_t>(p.B) * p.top_k * heads * ns;
    a.part_o = static_cast<float*>(ws);
    a.part_ml = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                         (n * p.d * sizeof(float) + 255) / 256 * 256);
  }

  (void)hipGetLastError();  // do not report an earlier, unrelated error as ours
  const hipError_t e = gqa_eff ? sha::launch_gqa(a, p.dtype, p.d, gqa_variant(), gqa_mfma(p.dtype), stream)
                               : sha::launch_mha(a, p.dtype, p.d, mha_variant(), stream);
  if (e != hipSuccess) {
    g_last_hip_error = e;
    return SHA_ERR_HIP;
  }
  return SHA_OK;
}

// ---------------------------------------------------------------------------
// selective MLP planning
// ---------------------------------------------------------------------------
struct MlpPlan {
  int n_pad, b_pad, bb, up_nu, up_kg, up_splits, up_kper, dn_splits, dn_waves;
  size_t h_bytes, up_bytes, dn_bytes;
};

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

// Grid sizes from the selection bound.  Both products stream weights, so the
// planner fills the chip without leaving a small second round of work.
//   up  : one workgroup per kMlpUpNeurons selected neurons x 64 batch rows
//         (2 resident per CU); its K (d) is split in whole kMlpUpKc stages,
//         ceil(0.95 x resident slots / workgroups) ways (at most 8).
//   down: one workgroup per 512 output columns (8 waves, one per CU; 256
//         columns and 4 waves, two per CU, when d is not a multiple of 512)
//         x 64 rows; the neuron range is split for about one round of
//         workgroups (each range keeps >= 64 neurons, at most 64 splits).
// The constants come from split sweeps of the OPT MLPs on MI355X.
constexpr int kUpWgsPerCu = 2;
constexpr int kDownWgsPerCu = 2;

int up_split_count(long long items, int kstages, int cus) {
  // The K splits bring the grid to about one round of resident workgroups
  // (fewer leave HBM idle: 288 unsplit OPT-66B workgroups stream 3.8 TB/s);
  // a grid already past that takes no splits beyond it.
  const long long slots = static_cast<long long>(kUpWgsPerCu) * cus;
  long long us = (slots * 95 / 100 + items - 1) / items;
  if (us > sha::kMlpMaxUpSplits) us = sha::kMlpMaxUpSplits;
  if (us > kstages) us = kstages;
  return us < 1 ? 1 : static_cast<int>(us);
}

MlpPlan mlp_plan(int B, int d, int n_max, int num_cus) {
  MlpPlan p{};
  const int cus = device_cus(num_cus);
  constexpr int NU = sha::kMlpUpNeurons;
  p.n_pad = ((n_max > 0 ? n_max : 1) + NU - 1) / NU * NU;
  p.b_pad = (B + 63) / 64 * 64;
  const int kstages = d / sha::kMlpUpKc;
  // Up tile: 128 neurons, or for full batch tiles 144 when that leaves
  // fewer idle slots in the grid's last round of resident workgroups
  // (OPT-66B: 256 tiles x 2 splits = 512 workgroups, one round, against
  // 288 x 2 = 576 with 128); SHA_MLP_UP_TILE = 128 or 144 forces one (a
  // tuning hook).
  //
  // Two K groups per up workgroup (8 waves, one workgroup per CU, the halves
  // of K summed on chip) replace K splits for full batch tiles whose tiles
  // alone make about a round at one per CU while the four-wave form would
  // split K (OPT-66B: 256 tiles of 144 neurons, no fp32 partials and no
  // finalize); the tile is then the one with fewer idle CUs in the last
  // round.  SHA_MLP_UP_KG = 1 or 2 forces one form (2 where d / 128 is even;
  // a tuning hook); SHA_MLP_UP_SPLITS keeps the four-wave form.
  auto items_of = [&](int nu) {
    return static_cast<long long>((p.n_pad + nu - 1) / nu) * (p.b_pad / 64);
  };
  auto kg2_fits = [&](int nu) {
    const long long items = items_of(nu);
    return items * 100 >= 95LL * cus && up_split_count(items, kstages, cus) >= 2;
  };
  const int kg_env = env_int("SHA_MLP_UP_KG", 0);
  const bool kg2_allowed = kstages % 2 == 0 && env_int("SHA_MLP_UP_SPLITS", 0) <= 0 && kg_env != 1;
  const bool kg2_fill = kg2_fits(NU) || kg2_fits(144);
  // Batch blocks: 1 for B <= 16, 2 for B <= 32, else 4; batches of 17-32
  // rows also compute the whole 64-row tile (padding rows repeat row B - 1,
  // and no output row reads them) when the two-K-group form then fills the
  // chip: the two-block grid of 128-neuron tiles runs past one round once
  // the union passes ~33K neurons (OPT-66B B = 32, union + MLP in a graph:
  // 244.4 -> 224.9 us; B = 24: 236.9 -> 216.3 us; B = 20 even).
  // SHA_MLP_BB = 2 or 4 (a tuning hook) forces the blocks where B fits them.
  p.bb = B <= 16 ? 1 : (B <= 32 && !(kg2_allowed && kg2_fill) ? 2 : 4);
  {
    const int bb = env_int("SHA_MLP_BB", 0);
    if ((bb == 2 && B <= 32) || bb == 4) p.bb = bb;
  }
  p.up_nu = NU;
  p.up_kg = 1;
  if (p.bb == 4) {
    if (kg2_allowed && (kg_env == 2 || kg2_fill)) {
      p.up_kg = 2;
      auto idle = [&](int nu) {
        const long long items = items_of(nu);
        return (items + cus - 1) / cus * cus - items;
      };
      if (idle(144) < idle(NU)) p.up_nu = 144;
    } else {
      const long long slots = static_cast<long long>(kUpWgsPerCu) * cus;
      auto idle = [&](int nu) {
        const long long items = items_of(nu);
        const long long wgs = items * up_split_count(items, kstages, cus);
        const long long rounds = (wgs + slots - 1) / slots;
        return rounds * slots - wgs;
      };
      if (idle(144) < idle(NU)) p.up_nu = 144;
    }
    const int tile = env_int("SHA_MLP_UP_TILE", 0);
    if (tile == 128 || tile == 144) p.up_nu = tile;
  }
  const long long up_items =
      static_cast<long long>((p.n_pad + p.up_nu - 1) / p.up_nu) * (p.b_pad / 64);
  int us = p.up_kg == 2 ? 1 : up_split_count(up_items, kstages, cus);
  if (env_int("SHA_MLP_UP_SPLITS", 0) > 0) us = env_int("SHA_MLP_UP_SPLITS", 0);  // tuning hook
  if (us > sha::kMlpMaxUpSplits) us = sha::kMlpMaxUpSplits;
  if (us > kstages) us = kstages;
  p.up_kper = (kstages + us - 1) / us * sha::kMlpUpKc;
  p.up_splits = (d + p.up_kper - 1) / p.up_kper;
  // Down workgroups: 8 waves x 64 columns, one per CU, when d is a multiple
  // of 512 (each column block, and its read of H from L2, covers 512
  // columns: OPT-66B down projection 137.5 -> 123.0 us against the 4-wave
  // form), else 4 waves x 64 columns, two per CU; SHA_MLP_DN_WAVES = 4 or 8
  // forces one where d allows (a tuning hook).
  const int dn_env = env_int("SHA_MLP_DN_WAVES", 0);
  p.dn_waves = (d % 512 == 0 && dn_env != 4) ? 8 : 4;
  const int dn_cols = 64 * p.dn_waves;
  const int dn_per_cu = p.dn_waves == 8 ? kDownWgsPerCu / 2 : kDownWgsPerCu;
  const long long dn_items = static_cast<long long>(d / dn_cols) * (p.b_pad / 64);
  long long ds = static_cast<long long>(dn_per_cu) * cus / dn_items;
  const long long ds_max = n_max / 64 > 1 ? n_max / 64 : 1;
  if (ds > ds_max) ds = ds_max;
  if (ds > 64) ds = 64;
  if (ds < 1) ds = 1;
  if (env_int("SHA_MLP_DN_SPLITS", 0) > 0) ds = env_int("SHA_MLP_DN_SPLITS", 0);  // tuning hook
  p.dn_splits = static_cast<int>(ds);
  p.h_bytes = round256(static_cast<size_t>(p.b_pad) * p.n_pad * 2);
  p.up_bytes = p.up_splits > 1 ? round256(static_cast<size_t>(p.up_splits) * p.b_pad * p.n_pad * 4) : 0;
  p.dn_bytes = p.dn_splits > 1 ? round256(static_cast<size_t>(p.dn_splits) * p.b_pad * d * 4) : 0;
  return p;
}

sha_status check_mlp(int B, int d, int D, int n_max, int dtype) {
  if (B < 0 || d < 1 || D < 1 || n_max < 0 || n_max > D) return SHA_ERR_INVALID_ARG;
  if (dtype != SHA_F16 && dtype != SHA_BF16) return SHA_ERR_UNSUPPORTED;
  if (d % 256 != 0) return SHA_ERR_UNSUPPORTED;
  if (B > 65535 * 64) return SHA_ERR_INVALID_ARG;
  // The up projection addresses weight rows with 32-bit byte offsets.
  if (static_cast<uint64_t>(D) * static_cast<uint64_t>(d) * 2u > 0xFFFFFFFFull)
    return SHA_ERR_UNSUPPORTED;
  return SHA_OK;
}

Problem make(const void* q, const void* k, const void* v, const int32_t* idx, int B, int H,
             int H_kv, int Nkv, int d, int top_k, float scale, void* o, int dtype, bool gqa,
             const sha_kv_layout* kv = nullptr) {
  return Problem{q, k, v, idx, o, B, H, H_kv, Nkv, d, top_k, scale, dtype, gqa, kv};
}

}  // namespace

namespace sha {
void set_last_hip_error(int e) { g_last_hip_error = e; }
}  // namespace sha

extern "C" {

sha_status sha_decode(const void* q, const void* k, const void* v,
                      const int32_t* batch_head_index, int B, int H, int H_kv, int Nkv, int d,
                      int top_k, float scale, void* o, hipStream_t stream, sha_dtype dtype) {
  return run_auto(make(q, k, v, batch_head_index, B, H, H_kv, Nkv, d, top_k, scale, o, dtype,
                       false),
                  stream);
}

sha_status sha_decode_f32(const void* q, const void* k, const void* v,
                          const int32_t* batch_head_index, int B, int H, int H_kv, int Nkv,
                          int d, int top_k, float scale, void* o, hipStream_t stream) {
  return sha_decode(q, k, v, batch_head_index, B, H, H_kv, Nkv, d, top_k, scale, o, stream,
                    SHA_F32);
}

sha_status sha_decode_f16(const void* q, const void* k, const void* v,
                          const int32_t* batch_head_index, int B, int H, int H_kv, int Nkv,
                          int d, int top_k, float scale, void* o, hipStream_t stream) {
  return sha_decode(q, k, v, batch_head_index, B, H, H_kv, Nkv, d, top_k, scale, o, stream,
                    SHA_F16);
}

sha_status sha_decode_bf16(const void* q, const void* k, const void* v,
                           const int32_t* batch_head_index, int B, int H, int H_kv, int Nkv,
                           int d, int top_k, float scale, void* o, hipStream_t stream) {
  return sha_decode(q, k, v, batch_head_index, B, H, H_kv, Nkv, d, top_k, scale, o, stream,
                    SHA_BF16);
}

sha_status sha_decode_gqa(const void* q, const void* k, const void* v,
                          const int32_t* batch_group_index, int B, int H, int H_kv, int Nkv,
                          int d, int top_k, float scale, void* o, hipStream_t stream,
                          sha_dtype dtype) {
  return run_auto(make(q, k, v, batch_group_index, B, H, H_kv, Nkv, d, top_k, scale, o, dtype,
                       true),
                  stream);
}

sha_status sha_decode_gqa_f32(const void* q, const void* k, const void* v,
                              const int32_t* batch_group_index, int B, int H, int H_kv, int Nkv,
                              int d, int top_k, float scale, void* o, hipStream_t stream) {
  return sha_decode_gqa(q, k, v, batch_group_index, B, H, H_kv, Nkv, d, top_k, scale, o, stream,
                        SHA_F32);
}

sha_status sha_decode_gqa_f16(const void* q, const void* k, const void* v,
                              const int32_t* batch_group_index, int B, int H, int H_kv, int Nkv,
                              int d, int top_k, float scale, void* o, hipStream_t stream) {
  return sha_decode_gqa(q, k, v, batch_group_index, B, H, H_kv, Nkv, d, top_k, scale, o, stream,
                        SHA_F16);
}

sha_status sha_decode_gqa_bf16(const void* q, const void* k, const void* v,
                               const int32_t* batch_group_index, int B, int H, int H_kv, int Nkv,
                               int d, int top_k, float scale, void* o, hipStream_t stream) {
  return sha_decode_gqa(q, k, v, batch_group_index, B, H, H_kv, Nkv, d, top_k, scale, o, stream,
                        SHA_BF16);
}

sha_status sha_decode_ex(const void* q, const void* k, const void* v,
                         const int32_t* batch_head_index, int B, int H, int H_kv, int Nkv, int d,
                         int top_k, float scale, void* o, hipStream_t stream, sha_dtype dtype,
                         int nsplit, void* workspace, size_t workspace_bytes) {
  if (nsplit < 0) return SHA_ERR_INVALID_ARG;
  return run(make(q, k, v, batch_head_index, B, H, H_kv, Nkv, d, top_k, scale, o, dtype, false),
             nsplit, workspace, workspace_bytes, stream);
}

sha_status sha_decode_gqa_ex(const void* q, const void* k, const void* v,
                             const int32_t* batch_group_index, int B, int H, int H_kv, int Nkv,
                             int d, int top_k, float scale, void* o, hipStream_t stream,
                             sha_dtype dtype, int nsplit, void* workspace,
                             size_t workspace_bytes) {
  if (nsplit < 0) return SHA_ERR_INVALID_ARG;
  return run(make(q, k, v, batch_group_index, B, H, H_kv, Nkv, d, top_k, scale, o, dtype, true),
             nsplit, workspace, workspace_bytes, stream);
}

sha_status sha_decode_kv(const void* q, const void* k, const void* v,
                         const int32_t* batch_head_index, int B, int H, int H_kv, int Nkv, int d,
                         int top_k, float scale, void* o, hipStream_t stream, sha_dtype dtype,
                         const sha_kv_layout* layout, int nsplit, void* workspace,
                         size_t workspace_bytes) {
  if (nsplit < 0) return SHA_ERR_INVALID_ARG;
  return run(make(q, k, v, batch_head_index, B, H, H_kv, Nkv, d, top_k, scale, o, dtype, false,
                  layout),
             nsplit, workspace, workspace_bytes, stream);
}

sha_status sha_decode_gqa_kv(const void* q, const void* k, const void* v,
                             const int32_t* batch_group_index, int B, int H, int H_kv, int Nkv,
                             int d, int top_k, float scale, void* o, hipStream_t stream,
                             sha_dtype dtype, const sha_kv_layout* layout, int nsplit,
                             void* workspace, size_t workspace_bytes) {
  if (nsplit < 0) return SHA_ERR_INVALID_ARG;
  return run(make(q, k, v, batch_group_index, B, H, H_kv, Nkv, d, top_k, scale, o, dtype, true,
                  layout),
             nsplit, workspace, workspace_bytes, stream);
}

int sha_plan_nsplit(int B, int H, int H_kv, int Nkv, int d, int top_k, int gqa, sha_dtype dtype,
                    int num_cus) {
  bool empty = false;
  if (check_scalars(B, H, H_kv, Nkv, d, top_k, gqa, dtype, &empty) != SHA_OK) return 0;
  if (empty) return 1;
  int ns = 1, chunk = Nkv;
  split_geometry(Nkv, plan_nsplit(B, H, H_kv, Nkv, d, top_k, gqa, dtype, num_cus), 0, &ns,
                 &chunk);
  return ns;
}

size_t sha_workspace_bytes_kv(int B, int H, int H_kv, int Nkv, int d, int top_k, int gqa,
                              sha_dtype dtype, int nsplit, int num_cus,
                              const sha_kv_layout* layout) {
  bool empty = false;
  if (check_scalars(B, H, H_kv, Nkv, d, top_k, gqa, dtype, &empty) != SHA_OK || empty) return 0;
  int kind = sha::kKvContig, page = 0;
  if (check_kv(layout, H_kv, Nkv, d, dtype, &kind, &page) != SHA_OK) return 0;
  const int req = nsplit > 0 ? nsplit : plan_nsplit(B, H, H_kv, Nkv, d, top_k, gqa, dtype, num_cus);
  int ns = 1, chunk = Nkv;
  split_geometry(Nkv, req, page, &ns, &chunk);
  return partial_bytes(B, H, H_kv, d, top_k, gqa && H / H_kv > 1, ns);
}

size_t sha_workspace_bytes(int B, int H, int H_kv, int Nkv, int d, int top_k, int gqa,
                           sha_dtype dtype, int nsplit, int num_cus) {
  return sha_workspace_bytes_kv(B, H, H_kv, Nkv, d, top_k, gqa, dtype, nsplit, num_cus, nullptr);
}

size_t sha_mlp_union_workspace_bytes(int D) {
  return D < 1 ? 0 : round256(static_cast<size_t>(D));
}

sha_status sha_mlp_union(const int32_t* row_neurons, int B, int k, int D, int32_t* sel,
                         int32_t* n_sel, hipStream_t stream, void* workspace,
                         size_t workspace_bytes) {
  if (B < 0 || k < 0 || D < 1) return SHA_ERR_INVALID_ARG;
  const long long total = static_cast<long long>(B) * k;
  if (total > 0x7FFFFFFFLL) return SHA_ERR_INVALID_ARG;
  if (!sel || !n_sel || (total > 0 && !row_neurons)) return SHA_ERR_INVALID_ARG;
  if (!aligned(sel, 4) || !aligned(n_sel, 4) || (row_neurons && !aligned(row_neurons, 4)))
    return SHA_ERR_MISALIGNED;
  if (!workspace || workspace_bytes < sha_mlp_union_workspace_bytes(D)) return SHA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return SHA_ERR_MISALIGNED;
  (void)hipGetLastError();
  // SHA_MLP_UNION_SMALL (a tuning hook): 0 keeps small unions on the
  // three-kernel path, a value above 1 sets the one-workgroup bound (entries).
  const int small = env_int("SHA_MLP_UNION_SMALL", 1);
  const hipError_t e = sha::launch_mlp_union(row_neurons, static_cast<int>(total), D, sel, n_sel,
                                             static_cast<uint8_t*>(workspace),
                                             small == 1 ? -1 : (small < 0 ? 0 : small), stream);
  if (e != hipSuccess) {
    g_last_hip_error = e;
    return SHA_ERR_HIP;
  }
  return SHA_OK;
}

size_t sha_selective_mlp_workspace_bytes(int B, int d, int D, int n_max, int num_cus) {
  if (check_mlp(B, d, D, n_max, SHA_BF16) != SHA_OK || B == 0) return 0;
  const MlpPlan p = mlp_plan(B, d, n_max, num_cus);
  return p.h_bytes + p.up_bytes + p.dn_bytes;
}

sha_status sha_selective_mlp(const void* x, const void* w1t, const void* w2t, const int32_t* sel,
                             const int32_t* n_sel, int n_max, int B, int d, int D, void* y,
                             hipStream_t stream, sha_dtype dtype, void* workspace,
                             size_t workspace_bytes) {
  const sha_status st = check_mlp(B, d, D, n_max, dtype);
  if (st != SHA_OK || B == 0) return st;
  if (!x || !w1t || !w2t || !sel || !n_sel || !y) return SHA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w1t, 16) || !aligned(w2t, 16) || !aligned(y, 16) ||
      !aligned(sel, 4) || !aligned(n_sel, 4))
    return SHA_ERR_MISALIGNED;
  const MlpPlan p = mlp_plan(B, d, n_max, 0);
  // Both products launch 1-D grids: their workgroup counts must fit one
  // grid dimension (and an int in the kernels).
  const long long btiles = p.b_pad / 64;
  if (static_cast<long long>((p.n_pad + p.up_nu - 1) / p.up_nu) * p.up_splits * btiles > 0x7FFFFFFFLL ||
      static_cast<long long>(d / 256) * p.dn_splits * btiles > 0x7FFFFFFFLL)
    return SHA_ERR_INVALID_ARG;
  const size_t need = p.h_bytes + p.up_bytes + p.dn_bytes;
  if (!workspace || workspace_bytes < need) return SHA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return SHA_ERR_MISALIGNED;
  sha::MlpArgs a{};
  a.x = x;
  a.w1t = w1t;
  a.w2t = w2t;
  a.sel = sel;
  a.n_sel = n_sel;
  a.y = y;
  char* ws = static_cast<char*>(workspace);
  a.h = ws;
  a.up_part = p.up_bytes ? reinterpret_cast<float*>(ws + p.h_bytes) : nullptr;
  a.dn_part = p.dn_bytes ? reinterpret_cast<float*>(ws + p.h_bytes + p.up_bytes) : nullptr;
  a.B = B;
  a.d = d;
  a.D = D;
  a.n_max = n_max;
  a.n_pad = p.n_pad;
  a.b_pad = p.b_pad;
  a.bb = p.bb;
  a.up_nu = p.up_nu;
  a.up_kg = p.up_kg;
  // K-split partials through LDS as whole-row pieces (OPT-66B B = 64, union
  // + MLP in a graph: 252.8-255.6 -> 247.6-250.4 us); SHA_MLP_UP_STAGE=0
  // (a tuning hook) keeps the direct float4 stores.
  a.up_stage = env_int("SHA_MLP_UP_STAGE", 1) != 0;
  // One or two computed batch blocks: x shared through LDS by the up
  // workgroup's waves (OPT-6.7B B = 16: 61.0-61.3 -> 59.3-59.6 us);
  // SHA_MLP_UP_XLDS=0 (a tuning hook) keeps each wave loading all of its x,
  // SHA_MLP_UP_XLDS=1 shares it for one batch block only.
  const int xlds = env_int("SHA_MLP_UP_XLDS", 2);
  a.up_xlds = (p.bb == 1 && xlds >= 1) || (p.bb == 2 && xlds >= 2);
  a.up_splits = p.up_splits;
  a.up_kper = p.up_kper;
  a.dn_splits = p.dn_splits;
  a.dn_waves = p.dn_waves;
  // Split partials through LDS as whole-row pieces (down kernel 130.5 ->
  // 126.8 us at OPT-66B B = 64); SHA_MLP_DN_STAGE=0 (a tuning hook) keeps
  // the direct 4-byte stores.
  a.dn_stage = env_int("SHA_MLP_DN_STAGE", 1) != 0;
  // One or two batch blocks with 2-4 up K splits: the down projection sums
  // the up partials as it loads H (no up finalize launch; OPT-6.7B B = 16 and
  // OPT-66B B = 8); SHA_MLP_FUSE_UP=0 (a tuning hook) keeps the finalize.
  a.dn_fuse_up = p.bb <= 2 && p.up_splits >= 2 && p.up_splits <= 4 &&
                 env_int("SHA_MLP_FUSE_UP", 1) != 0;
  (void)hipGetLastError();
  const hipError_t e = sha::launch_selective_mlp(a, dtype, stream);
  if (e != hipSuccess) {
    g_last_hip_error = e;
    return SHA_ERR_HIP;
  }
  return SHA_OK;
}

size_t sha_router_split_bytes(int B, int d, int H, sha_dtype dtype) {
  if (dtype != SHA_F16 && dtype != SHA_BF16) return 0;
  // d <= 2^30 keeps the kernel's 32-bit hidden offsets and its grid
  // (ceil(B / 16) * ceil(d / 256) workgroups) in range.
  if (B < 1 || d < 8 || d % 8 != 0 || d > (1 << 30) || H < 1 || H > sha::kRouterSplitMaxH ||
      B > sha::kRouterSplitMaxB)
    return 0;
  const size_t nchunk = (static_cast<size_t>(d) + sha::kRouterChunk - 1) / sha::kRouterChunk;
  return (static_cast<size_t>(B) * nchunk * H * sizeof(float) + 255) / 256 * 256;
}

size_t sha_router_workspace_bytes(int B, int d, int H, sha_dtype dtype) {
  // Measured in HIP graphs: the split form pays from about 2^24 multiply-adds
  // per call (OPT-66B's 64 x 72 x 9216: 8.8 against 9.6 us); the smaller
  // layers' calls are faster one-pass.
  const long long macs = static_cast<long long>(B) * H * d;
  static const bool on = env_int("SHA_ROUTER_SPLIT", 1) != 0;  // tuning hook: 0 = one-pass
  if (macs < (1LL << 24) || !on) return 0;
  return sha_router_split_bytes(B, d, H, dtype);
}

sha_status sha_router_topk(const void* x, const void* w, const float* bias, int B, int d, int H,
                           int top_k, int32_t* batch_head_index, float* scores,
                           hipStream_t stream, sha_dtype dtype) {
  return sha_router_topk_ex(x, w, bias, B, d, H, top_k, batch_head_index, scores, stream, dtype,
                            nullptr, 0);
}

sha_status sha_router_topk_ex(const void* x, const void* w, const float* bias, int B, int d,
                              int H, int top_k, int32_t* batch_head_index, float* scores,
                              hipStream_t stream, sha_dtype dtype, void* workspace,
                              size_t workspace_bytes) {
  if (B < 0 || d < 1 || H < 1 || top_k < 0 || top_k > H) return SHA_ERR_INVALID_ARG;
  if (dtype != SHA_F32 && dtype != SHA_F16 && dtype != SHA_BF16) return SHA_ERR_UNSUPPORTED;
  if (H > sha::kRouterMaxH) return SHA_ERR_UNSUPPORTED;
  if (d % (dtype == SHA_F32 ? 4 : 8) != 0) return SHA_ERR_UNSUPPORTED;
  // The scores grid has up to B * ceil(H / 2) workgroups of 512 threads.
  if (static_cast<long long>(B) * ((H + 1) / 2) > (1LL << 22)) return SHA_ERR_INVALID_ARG;
  if (B == 0) return SHA_OK;
  if (!x || !w || !scores || (top_k > 0 && !batch_head_index)) return SHA_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(scores, 4) ||
      (bias && !aligned(bias, 4)) || (batch_head_index && !aligned(batch_head_index, 4)))
    return SHA_ERR_MISALIGNED;
  sha::RouterArgs a{x, w, bias, scores, batch_head_index, B, d, H, top_k, nullptr, 0};
  // The K-split form runs when the call passes a workspace and its shape has
  // one; otherwise the one-pass kernels run.
  const size_t need = workspace ? sha_router_split_bytes(B, d, H, dtype) : 0;
  if (need > 0) {
    if (workspace_bytes < need) return SHA_ERR_WORKSPACE;
    if (!aligned(workspace, 16)) return SHA_ERR_MISALIGNED;
    a.part = static_cast<float*>(workspace);
    a.nchunk = (d + sha::kRouterChunk - 1) / sha::kRouterChunk;
  }
  (void)hipGetLastError();
  const hipError_t e = sha::launch_router(a, dtype, device_cus(0), stream);
  if (e != hipSuccess) {
    g_last_hip_error = e;
    return SHA_ERR_HIP;
  }
  return SHA_OK;
}

const char* sha_status_string(sha_status s) {
  switch (s) {
    case SHA_OK: return "SHA_OK";
    case SHA_ERR_INVALID_ARG: return "SHA_ERR_INVALID_ARG";
    case SHA_ERR_UNSUPPORTED: return "SHA_ERR_UNSUPPORTED";
    case SHA_ERR_MISALIGNED: return "SHA_ERR_MISALIGNED";
    case SHA_ERR_WORKSPACE: return "SHA_ERR_WORKSPACE";
    case SHA_ERR_HIP: return "SHA_ERR_HIP";
  }
  return "SHA_ERR_UNKNOWN";
}

int sha_last_hip_error(void) { return g_last_hip_error; }

const char* sha_version(void) { return "0.1.0"; }

}  // extern "C"
