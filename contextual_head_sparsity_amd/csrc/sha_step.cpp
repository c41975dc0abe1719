// Multi-layer decode step: the library's router, selective head attention and
// selective MLP calls for n layers on one stream, optionally captured once
// into a HIP graph.  Built only on the public C ABI (include/sha.h); the
// contract is documented there.
#include <stdlib.h>

#include <new>
#include <vector>

#include "sha.h"
#include "sha_launch.h"

struct sha_step {
  sha_step_config cfg;
  std::vector<sha_step_layer> layers;
  std::vector<sha_kv_layout> kv;       // per layer copy of the caller's layout
  std::vector<int> nsplit;             // per layer split count (fixed at create)
  void* attn_ws = nullptr;              // SHA split partials; also the router's K-split
  size_t attn_ws_bytes = 0;              // partials (the router runs first on the stream)
  size_t router_ws_bytes = 0;
  int32_t* dense_index = nullptr;      // [B, H or H_kv] = 0 .. n-1 per row
  int32_t* sel = nullptr;              // MLP union output [max(1, n_max)]
  int32_t* n_sel = nullptr;
  void* union_ws = nullptr;
  size_t union_ws_bytes = 0;
  void* mlp_ws = nullptr;
  size_t mlp_ws_bytes = 0;
  int n_max = 0;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
};

namespace {

sha_status hip_fail(hipError_t e) {
  sha::set_last_hip_error(e);
  return SHA_ERR_HIP;
}

void release(sha_step* s) {
  if (!s) return;
  if (s->exec) (void)hipGraphExecDestroy(s->exec);
  if (s->graph) (void)hipGraphDestroy(s->graph);
  for (void* p : {s->attn_ws, static_cast<void*>(s->dense_index), static_cast<void*>(s->sel),
                  static_cast<void*>(s->n_sel), s->union_ws, s->mlp_ws})
    if (p) (void)hipFree(p);
  delete s;
}

bool has_mlp(const sha_step_layer& L) { return L.mlp_w1t != nullptr; }

// Every call of one step, in order, on `stream`.
sha_status enqueue(sha_step* s, hipStream_t stream) {
  const sha_step_config& c = s->cfg;
  const int n_sel_heads = c.gqa ? c.H_kv : c.H;
  for (size_t l = 0; l < s->layers.size(); ++l) {
    const sha_step_layer& L = s->layers[l];
    const sha_kv_layout* kv = L.kv ? &s->kv[l] : nullptr;
    const int32_t* index = L.index;
    int top_k = c.top_k;
    sha_status st;
    if (L.dense) {
      index = s->dense_index;
      top_k = n_sel_heads;
    } else {
      st = sha_router_topk_ex(L.router_x, L.router_w, L.router_bias, c.B, c.router_d,
                              n_sel_heads, top_k, L.index, L.router_scores, stream, c.dtype,
                              s->router_ws_bytes ? s->attn_ws : nullptr, s->attn_ws_bytes);
      if (st != SHA_OK) return st;
    }
    st = c.gqa ? sha_decode_gqa_kv(L.q, L.k, L.v, index, c.B, c.H, c.H_kv, c.Nkv, c.d, top_k,
                                   c.scale, L.o, stream, c.dtype, kv, s->nsplit[l], s->attn_ws,
                                   s->attn_ws_bytes)
               : sha_decode_kv(L.q, L.k, L.v, index, c.B, c.H, c.H_kv, c.Nkv, c.d, top_k, c.scale,
                               L.o, stream, c.dtype, kv, s->nsplit[l], s->attn_ws,
                               s->attn_ws_bytes);
    if (st != SHA_OK) return st;
    if (has_mlp(L)) {
      st = sha_mlp_union(L.mlp_rows, c.B, c.mlp_k, c.mlp_D, s->sel, s->n_sel, stream, s->union_ws,
                         s->union_ws_bytes);
      if (st != SHA_OK) return st;
      st = sha_selective_mlp(L.mlp_x, L.mlp_w1t, L.mlp_w2t, s->sel, s->n_sel, s->n_max, c.B,
                             c.mlp_d, c.mlp_D, L.mlp_y, stream, c.dtype, s->mlp_ws,
                             s->mlp_ws_bytes);
      if (st != SHA_OK) return st;
    }
  }
  return SHA_OK;
}

sha_status dev_alloc(void** p, size_t bytes) {
  if (bytes == 0) return SHA_OK;
  const hipError_t e = hipMalloc(p, bytes);
  return e == hipSuccess ? SHA_OK : hip_fail(e);
}

sha_status create(const sha_step_config* cfg, const sha_step_layer* layers, int n_layers,
                  int use_graph, sha_step* s) {
  const sha_step_config& c = *cfg;
  s->cfg = c;
  s->layers.assign(layers, layers + n_layers);
  s->kv.resize(n_layers);
  s->nsplit.resize(n_layers);
  const int n_sel_heads = c.gqa ? c.H_kv : c.H;
  bool any_mlp = false;
  for (int l = 0; l < n_layers; ++l)
    if (!layers[l].dense && (!layers[l].index || !layers[l].router_scores))
      return SHA_ERR_INVALID_ARG;
  for (int l = 0; l < n_layers; ++l) {
    const sha_step_layer& L = layers[l];
    if (L.kv) s->kv[l] = *L.kv;
    const int top_k = L.dense ? n_sel_heads : c.top_k;
    const int plan = sha_plan_nsplit(c.B, c.H, c.H_kv, c.Nkv, c.d, top_k, c.gqa, c.dtype, 0);
    if (plan == 0) return SHA_ERR_INVALID_ARG;
    s->nsplit[l] = plan;
    const size_t ws = sha_workspace_bytes_kv(c.B, c.H, c.H_kv, c.Nkv, c.d, top_k, c.gqa, c.dtype,
                                             plan, 0, L.kv ? &s->kv[l] : nullptr);
    if (ws > s->attn_ws_bytes) s->attn_ws_bytes = ws;
    any_mlp = any_mlp || has_mlp(L);
  }
  s->router_ws_bytes = sha_router_workspace_bytes(c.B, c.router_d, n_sel_heads, c.dtype);
  if (s->router_ws_bytes > s->attn_ws_bytes) s->attn_ws_bytes = s->router_ws_bytes;
  sha_status st = dev_alloc(&s->attn_ws, s->attn_ws_bytes);
  if (st != SHA_OK) return st;

  // Dense index: every head (group) of every row, built on the host once.
  if (c.B > 0 && n_sel_heads > 0) {
    std::vector<int32_t> host(static_cast<size_t>(c.B) * n_sel_heads);
    for (size_t i = 0; i < host.size(); ++i) host[i] = static_cast<int32_t>(i % n_sel_heads);
    st = dev_alloc(reinterpret_cast<void**>(&s->dense_index), host.size() * sizeof(int32_t));
    if (st != SHA_OK) return st;
    const hipError_t e = hipMemcpy(s->dense_index, host.data(), host.size() * sizeof(int32_t),
                                   hipMemcpyHostToDevice);
    if (e != hipSuccess) return hip_fail(e);
  }

  if (any_mlp) {
    if (c.mlp_D < 1 || c.mlp_k < 0 || c.mlp_d < 1) return SHA_ERR_INVALID_ARG;
    const long long total = static_cast<long long>(c.B) * c.mlp_k;
    s->n_max = static_cast<int>(total < c.mlp_D ? total : c.mlp_D);
    s->union_ws_bytes = sha_mlp_union_workspace_bytes(c.mlp_D);
    s->mlp_ws_bytes = sha_selective_mlp_workspace_bytes(c.B, c.mlp_d, c.mlp_D, s->n_max, 0);
    const size_t sel_bytes = static_cast<size_t>(s->n_max > 0 ? s->n_max : 1) * sizeof(int32_t);
    if ((st = dev_alloc(reinterpret_cast<void**>(&s->sel), sel_bytes)) != SHA_OK ||
        (st = dev_alloc(reinterpret_cast<void**>(&s->n_sel), sizeof(int32_t))) != SHA_OK ||
        (st = dev_alloc(&s->union_ws, s->union_ws_bytes)) != SHA_OK ||
        (st = dev_alloc(&s->mlp_ws, s->mlp_ws_bytes)) != SHA_OK)
      return st;
  }

  // Capture on a private stream (default priority).  Capturing runs every
  // call's host-side validation without executing anything, so an argument
  // error surfaces here, from the underlying call, in both modes; the graph
  // is instantiated and kept only for graph runs.
  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e);
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    (void)hipStreamDestroy(cs);
    return hip_fail(e);
  }
  st = enqueue(s, cs);
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);
  (void)hipStreamDestroy(cs);
  if (st != SHA_OK) {
    if (g) (void)hipGraphDestroy(g);
    return st;
  }
  if (e != hipSuccess) return hip_fail(e);
  s->graph = g;
  if (!use_graph) return SHA_OK;
  e = hipGraphInstantiate(&s->exec, g, nullptr, nullptr, 0);
  if (e != hipSuccess) return hip_fail(e);
  return SHA_OK;
}

}  // namespace

extern "C" {

sha_status sha_step_create(const sha_step_config* cfg, const sha_step_layer* layers, int n_layers,
                           int use_graph, sha_step** step) {
  if (!step) return SHA_ERR_INVALID_ARG;
  *step = nullptr;
  if (!cfg || n_layers < 1 || !layers) return SHA_ERR_INVALID_ARG;
  if (cfg->B < 1 || cfg->top_k < 1) return SHA_ERR_INVALID_ARG;
  sha_step* s = new (std::nothrow) sha_step();
  if (!s) return SHA_ERR_INVALID_ARG;
  const sha_status st = create(cfg, layers, n_layers, use_graph, s);
  if (st != SHA_OK) {
    release(s);
    return st;
  }
  *step = s;
  return SHA_OK;
}

sha_status sha_step_run(sha_step* step, hipStream_t stream) {
  if (!step) return SHA_ERR_INVALID_ARG;
  if (!step->exec) return enqueue(step, stream);
  const hipError_t e = hipGraphLaunch(step->exec, stream);
  return e == hipSuccess ? SHA_OK : hip_fail(e);
}

sha_status sha_step_destroy(sha_step* step) {
  if (!step) return SHA_ERR_INVALID_ARG;
  release(step);
  return SHA_OK;
}

}  // extern "C"
