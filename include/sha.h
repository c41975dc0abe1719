/*
 * sha.h - C ABI of the Selective Head Attention (SHA) decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every batch row b and every slot k of an index
 * tensor, one decode-attention pass of a single query vector over all Nkv
 * keys of its head:
 *
 *     O[b, h, 0, :] = softmax(scale * q K^T) V,   q = Q[b, h, 0, :],
 *                     K = K[b, g, :, :], V = V[b, g, :, :]
 *
 * Definition: Polar Sparsity notes (papernotes.org), section 方法详解 >
 * 关键设计 > "Attention Head 稀疏性" (per-head softmax(Q K^T / sqrt(d_h)) V).
 * Selection: the same notes, "Selective Head Attention (SHA) Kernel" (the
 * kernel takes a batch head index tensor, one thread-block per batch row and
 * head, only active heads are read and written, GQA models use group
 * sparsity), and the Polar Sparsity reproducibility page (ri.k117.org),
 * "Pseudocode", Algorithm 1 "Selective Head Flash Attention (Decode)": a unit
 * (b, k) resolves head_idx = batch_head_index[b, k], streams K/V of that
 * head in tiles with a running max / running sum softmax and writes
 * O[b, head_idx, 0, :].
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; they must
 *     stay valid until the work queued on `stream` has finished.  The library
 *     keeps no caller pointer after a call returns.
 *   - Layouts are contiguous row-major:
 *         q, o : [B, H, 1, d]          (H = number of query heads)
 *         k, v : [B, H_kv, Nkv, d]
 *         index: [B, top_k] int32
 *     q, k, v and o share one element type (dtype); accumulation is fp32,
 *     the result is rounded to the element type (round to nearest even).
 *   - d must be 64 or 128 (else SHA_ERR_UNSUPPORTED).  q, k, v, o and a
 *     workspace must be 16-byte aligned, the index 4-byte aligned (else
 *     SHA_ERR_MISALIGNED).
 *   - B == 0 or top_k == 0 is an empty call: nothing is read or written and
 *     SHA_OK is returned (null pointers are then allowed).  Nkv must be >= 1
 *     (a softmax over no keys is undefined).
 *   - Output slots [b, h] that no index entry selects are never written: a
 *     caller that needs zeros there zeroes o first.
 *   - An index entry outside [0, H) (head entry points) or [0, H_kv) (group
 *     entry points), for example -1 used as padding, is skipped: that unit
 *     reads and writes nothing.  Duplicate entries compute the same slot
 *     twice with identical bits.  Index contents are device data and are not
 *     checked on the host (that would need a device synchronisation).
 *   - Calls are asynchronous: they validate on the host, enqueue on `stream`
 *     and return.  Scalar/pointer errors are returned before anything is
 *     enqueued; a failing launch returns SHA_ERR_HIP (the raw hipError_t is
 *     available from sha_last_hip_error()); device faults surface at the
 *     caller's next synchronisation.
 *   - Results are deterministic: no atomics, fixed reduction order.  The
 *     split count (see sha_decode_ex) changes the rounding order, so results
 *     are bitwise reproducible for a fixed split count.
 */
#ifndef SHA_H_
#define SHA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SHA_F32 = 0, SHA_F16 = 1, SHA_BF16 = 2 } sha_dtype;

typedef enum {
  SHA_OK = 0,
  SHA_ERR_INVALID_ARG = 1,  /* bad scalar (negative size, H % H_kv != 0, top_k out of range, Nkv < 1, non-finite scale) or null pointer */
  SHA_ERR_UNSUPPORTED = 2,  /* head dimension other than 64 / 128, unknown dtype, group size > 64 */
  SHA_ERR_MISALIGNED = 3,   /* pointer alignment below what the 128-bit loads need */
  SHA_ERR_WORKSPACE = 4,    /* workspace null or smaller than sha_workspace_bytes(), or an internal workspace that would have to grow on a stream under capture */
  SHA_ERR_HIP = 5           /* a HIP runtime call or launch failed */
} sha_status;

/*
 * Head-indexed SHA decode (the Algorithm 1 unit: one query head per index
 * entry).  batch_head_index[b, k] names a query head in [0, H).  With
 * H_kv < H (H % H_kv == 0, G = H / H_kv) head h reads KV head h / G.
 *   scale : score scale, normally 1/sqrt(d) (Algorithm 1's s); must be finite.
 *   stream: HIP stream to enqueue on (0 = the null stream).
 * The library picks the split count and uses an internal workspace when it
 * needs one: one buffer per (device, stream), allocated on first
 * need and replaced by a larger one when a call needs more; outgrown buffers
 * are kept, not freed, until the process ends (queued work or a captured
 * graph may still use them).  Calls from several host threads are
 * serialised around it.  On a stream that is being captured into a graph the
 * library does not allocate: a call that would need to grow the workspace
 * then returns SHA_ERR_WORKSPACE and enqueues nothing (a call the existing
 * workspace covers is captured normally).  Callers that must not allocate
 * use sha_decode_ex.
 * The three typed forms take exactly these arguments; sha_decode adds dtype.
 */
sha_status sha_decode_f32(const void* q, const void* k, const void* v,
                          const int32_t* batch_head_index, int B, int H, int H_kv,
                          int Nkv, int d, int top_k, float scale, void* o,
                          hipStream_t stream);
sha_status sha_decode_f16(const void* q, const void* k, const void* v,
                          const int32_t* batch_head_index, int B, int H, int H_kv,
                          int Nkv, int d, int top_k, float scale, void* o,
                          hipStream_t stream);
sha_status sha_decode_bf16(const void* q, const void* k, const void* v,
                           const int32_t* batch_head_index, int B, int H, int H_kv,
                           int Nkv, int d, int top_k, float scale, void* o,
                           hipStream_t stream);
sha_status sha_decode(const void* q, const void* k, const void* v,
                      const int32_t* batch_head_index, int B, int H, int H_kv, int Nkv,
                      int d, int top_k, float scale, void* o, hipStream_t stream,
                      sha_dtype dtype);

/*
 * Group-indexed SHA decode (GQA group sparsity).  batch_group_index[b, k]
 * names a KV group g in [0, H_kv); all G = H / H_kv query heads
 * g*G .. g*G+G-1 of the group are computed against K/V[b, g], which is
 * streamed once per unit and shared by the G heads.  top_k counts groups
 * (1 <= top_k <= H_kv).  G may be 1..64.  Other arguments as sha_decode.
 * Group sparsity: Polar Sparsity notes (papernotes.org), SHA Kernel bullet on
 * GQA; atlas.scime.ai summary, "Approach" (routers pick top-k heads or GQA
 * groups).  The contiguous head-to-group numbering is the usual grouped-query
 * layout (the pages do not spell it out).
 */
sha_status sha_decode_gqa_f32(const void* q, const void* k, const void* v,
                              const int32_t* batch_group_index, int B, int H, int H_kv,
                              int Nkv, int d, int top_k, float scale, void* o,
                              hipStream_t stream);
sha_status sha_decode_gqa_f16(const void* q, const void* k, const void* v,
                              const int32_t* batch_group_index, int B, int H, int H_kv,
                              int Nkv, int d, int top_k, float scale, void* o,
                              hipStream_t stream);
sha_status sha_decode_gqa_bf16(const void* q, const void* k, const void* v,
                               const int32_t* batch_group_index, int B, int H, int H_kv,
                               int Nkv, int d, int top_k, float scale, void* o,
                               hipStream_t stream);
sha_status sha_decode_gqa(const void* q, const void* k, const void* v,
                          const int32_t* batch_group_index, int B, int H, int H_kv,
                          int Nkv, int d, int top_k, float scale, void* o,
                          hipStream_t stream, sha_dtype dtype);

/*
 * Explicit-workspace forms: no allocation inside the call.
 *   nsplit   : number of KV splits per unit (flash-decoding split-K); 0 lets
 *              the library choose (sha_plan_nsplit).  Values above Nkv are
 *              clamped.  With an effective split count above 1 the call runs
 *              the split kernel and then a combine kernel that merges the
 *              per-split (o, m, l) partials with the same running-max rule
 *              as Algorithm 1's tile merge.
 *   workspace: device buffer of at least sha_workspace_bytes(...) bytes for
 *              the same arguments (may be null when that is 0), owned by the
 *              caller; its contents on entry do not matter.  Calls that
 *              share one workspace must be ordered (same stream).
 */
sha_status sha_decode_ex(const void* q, const void* k, const void* v,
                         const int32_t* batch_head_index, int B, int H, int H_kv, int Nkv,
                         int d, int top_k, float scale, void* o, hipStream_t stream,
                         sha_dtype dtype, int nsplit, void* workspace, size_t workspace_bytes);
sha_status sha_decode_gqa_ex(const void* q, const void* k, const void* v,
                             const int32_t* batch_group_index, int B, int H, int H_kv,
                             int Nkv, int d, int top_k, float scale, void* o,
                             hipStream_t stream, sha_dtype dtype, int nsplit,
                             void* workspace, size_t workspace_bytes);

/*
 * For callers that cannot allocate device memory (code under graph capture,
 * serving loops and harnesses that forbid hipMalloc): sha_decode_ex
 * (gqa == 0) or sha_decode_gqa_ex (gqa == 1) with the split partials in a
 * fixed device array of SHA_NOALLOC_SCRATCH_BYTES bytes that the library
 * holds on every GPU it runs on, until the process ends, instead of a
 * caller workspace.  Other arguments and results as those entry points.
 * The call allocates nothing.  A call whose partials (sha_workspace_bytes
 * for the same arguments) exceed the array returns SHA_ERR_WORKSPACE and
 * enqueues nothing.  Every call on one GPU shares that GPU's array and its
 * kernels overwrite what an earlier call left there (the partials need no
 * clearing), so calls that may overlap on one GPU (several streams or host
 * threads) race: order them, or give each its own workspace through
 * sha_decode_ex.
 */
#define SHA_NOALLOC_SCRATCH_BYTES (8u << 20)
sha_status sha_decode_noalloc(const void* q, const void* k, const void* v,
                              const int32_t* index, int B, int H, int H_kv, int Nkv, int d,
                              int top_k, float scale, void* o, hipStream_t stream,
                              sha_dtype dtype, int gqa, int nsplit);

/*
 * KV cache layouts and per-row cache lengths.  A decode batch mixes requests
 * whose caches hold different numbers of keys, and serving stacks keep the
 * cache as [B, Nkv, H_kv, d], as per-head slabs, or in fixed-size pages.
 * The pages run SHA inside such a decode loop (Polar Sparsity notes,
 * papernotes.org, 实验关键数据: batched decoding throughput of full models);
 * Algorithm 1 itself (reproducibility page, ri.k117.org, "Pseudocode") has
 * one Nkv for every unit.  Row b attends to its first len_b =
 * clamp(seqlens[b], 0, Nkv) keys; a row with len_b = 0 gets zeros in the
 * selected slots.
 *
 *   Strided (block_table == NULL): key row r of batch row b, KV head g is at
 *       k + (b * k_batch_stride + g * k_head_stride + r * k_row_stride) elements
 *   (likewise v), so [B, Nkv, H_kv, d] has strides (Nkv*H_kv*d, d, H_kv*d).
 *   Paged (block_table != NULL): rows are grouped in pages of page_size rows;
 *       page p = block_table[b * block_table_stride + r / page_size],
 *       k + (p * k_batch_stride + g * k_head_stride + (r % page_size) * k_row_stride)
 *   i.e. k_batch_stride is the page stride of a pool of num_pages pages
 *   (for a pool [num_pages, page_size, H_kv, d]: (page_size*H_kv*d, d, H_kv*d)).
 *   Only the entries of pages that hold rows < len_b are read.  Page ids are
 *   device data and are not checked on the host; an id outside
 *   [0, num_pages) is clamped into that range (no out-of-pool read, but the
 *   row's result is then meaningless).
 * Every stride is >= 0 and a multiple of 16 bytes (16 / element-size
 * elements), else SHA_ERR_MISALIGNED; page_size is a power of two in
 * [16, 65536], block_table_stride >= ceil(Nkv / page_size) and
 * num_pages >= 1, else SHA_ERR_INVALID_ARG.  seqlens (device int32 [B]) may
 * be NULL: every row then holds Nkv keys.  A paged call keeps each KV split
 * within 1024 pages (the split count is raised if needed; Nkv above
 * 64 * 1024 * page_size is SHA_ERR_UNSUPPORTED).
 */
typedef struct sha_kv_layout {
  int64_t k_batch_stride, k_head_stride, k_row_stride;
  int64_t v_batch_stride, v_head_stride, v_row_stride;
  const int32_t* seqlens;      /* [B] or NULL */
  const int32_t* block_table;  /* [B, block_table_stride] or NULL (not paged) */
  int32_t block_table_stride;
  int32_t page_size;
  int32_t num_pages;
} sha_kv_layout;

/*
 * sha_decode_ex / sha_decode_gqa_ex over a caller-described KV layout
 * (layout == NULL: the contiguous [B, H_kv, Nkv, d] layout, all rows Nkv
 * keys).  q and o stay contiguous [B, H, 1, d].  Nkv is the longest row
 * (the bound the split plan and seqlens clamp use).  The workspace is sized
 * by sha_workspace_bytes_kv for the same arguments.
 */
sha_status sha_decode_kv(const void* q, const void* k, const void* v,
                         const int32_t* batch_head_index, int B, int H, int H_kv, int Nkv,
                         int d, int top_k, float scale, void* o, hipStream_t stream,
                         sha_dtype dtype, const sha_kv_layout* layout, int nsplit,
                         void* workspace, size_t workspace_bytes);
sha_status sha_decode_gqa_kv(const void* q, const void* k, const void* v,
                             const int32_t* batch_group_index, int B, int H, int H_kv,
                             int Nkv, int d, int top_k, float scale, void* o,
                             hipStream_t stream, sha_dtype dtype, const sha_kv_layout* layout,
                             int nsplit, void* workspace, size_t workspace_bytes);

/*
 * Launch planning (host only, no device work).
 *   sha_plan_nsplit    : the split count the library would use; num_cus <= 0
 *                        queries the current device's compute-unit count.
 *                        Returns a value >= 1, or 0 for invalid arguments.
 *   sha_workspace_bytes: workspace bytes needed for nsplit (0 = planned
 *                        split count, same num_cus rule); 0 when no
 *                        workspace is needed.  gqa != 0 selects the group
 *                        entry points' accounting.
 */
int sha_plan_nsplit(int B, int H, int H_kv, int Nkv, int d, int top_k, int gqa,
                    sha_dtype dtype, int num_cus);
size_t sha_workspace_bytes(int B, int H, int H_kv, int Nkv, int d, int top_k, int gqa,
                           sha_dtype dtype, int nsplit, int num_cus);
/* Workspace of sha_decode_kv / sha_decode_gqa_kv (layout may be NULL). */
size_t sha_workspace_bytes_kv(int B, int H, int H_kv, int Nkv, int d, int top_k, int gqa,
                              sha_dtype dtype, int nsplit, int num_cus,
                              const sha_kv_layout* layout);

/*
 * Attention router: the per-request active heads (or GQA groups) that feed
 * sha_decode / sha_decode_gqa.  Polar Sparsity notes (papernotes.org),
 * 损失函数 / 训练策略 (the attention router is a single fully connected layer
 * trained on the top-k of the per-head attention output norm); atlas.scime.ai
 * summary, "Approach" (routers pick the top-k heads or GQA groups per
 * request).
 *     scores[b, h] = x[b, :] . w[h, :] (+ bias[h])        (fp32 accumulation)
 *     batch_head_index[b, :] = the top_k heads of scores[b, :], ascending
 * Ties go to the lower head id; a NaN score ranks like -inf.
 *   x     : [B, d] device, element type dtype;  w: [H, d] device (one row per
 *           head or group), same type;  bias: [H] fp32 device or null.
 *   scores: [B, H] fp32 device output (always written);
 *   batch_head_index: [B, top_k] int32 device output (may be null if top_k = 0).
 * Limits: 1 <= H <= 1024, 0 <= top_k <= H, d a multiple of 8 (4 for f32),
 * else SHA_ERR_INVALID_ARG / SHA_ERR_UNSUPPORTED; B * ceil(H / 2) at most
 * 2^22 (the scores grid), else SHA_ERR_INVALID_ARG.  B == 0 is an empty call.
 * x and w 16-byte aligned, the others 4-byte aligned (SHA_ERR_MISALIGNED).
 */
sha_status sha_router_topk(const void* x, const void* w, const float* bias, int B, int d, int H,
                           int top_k, int32_t* batch_head_index, float* scores,
                           hipStream_t stream, sha_dtype dtype);

/*
 * The same router with a caller workspace, which lets 16-bit calls of up to
 * 128 heads and 4096 rows split the hidden dimension: matrix-core partial
 * products per 256 hidden elements (fp32), added per row in a fixed order by
 * the top-k kernel; two launches as before, the first of many short
 * workgroups.  Results are those of sha_router_topk up to fp32 rounding
 * order; a call repeated on the same inputs returns the same bits.
 *   sha_router_split_bytes: bytes the split form needs for this shape,
 *     B * ceil(d / 256) * H * 4 rounded up to 256; 0 when the shape has no
 *     split form (f32, H > 128, B > 4096, d not a multiple of 8 or above
 *     2^30, B < 1).
 *   sha_router_workspace_bytes: the same where the split form is the faster
 *     one (B * H * d >= 2^24 multiply-adds), else 0.  Callers pass a
 *     workspace of that size, or null when it is 0.
 *   workspace: device memory, 16-byte aligned (SHA_ERR_MISALIGNED), owned by
 *     the caller; its contents on entry do not matter.  On a shape with a
 *     split form a non-null workspace selects that form and must hold
 *     sha_router_split_bytes (SHA_ERR_WORKSPACE); otherwise, or when null,
 *     the one-pass kernels of sha_router_topk run and it is not touched.
 *     Calls that may overlap (several streams) need separate workspaces.
 * Other arguments, limits and errors as sha_router_topk.
 */
size_t sha_router_split_bytes(int B, int d, int H, sha_dtype dtype);
size_t sha_router_workspace_bytes(int B, int d, int H, sha_dtype dtype);
sha_status sha_router_topk_ex(const void* x, const void* w, const float* bias, int B, int d,
                              int H, int top_k, int32_t* batch_head_index, float* scores,
                              hipStream_t stream, sha_dtype dtype, void* workspace,
                              size_t workspace_bytes);

/*
 * Selective MLP ("Selective GEMM") over the batch union of active neurons.
 * Polar Sparsity notes (papernotes.org), 方法详解 > 关键设计 > "MLP 层动态稀疏":
 * MLP_{S_B}(x) = sigma(x W1[:, S_B]) W2[:, S_B]^T, where S_B is the union of
 * the active neurons of every row of the batch and the index selection is
 * fused into the matrix products.  sigma is ReLU (the pages apply the
 * selective MLP to OPT models); the equation has no bias and none is added.
 *
 * Weights are stored neuron-major: w1t = W1^T and w2t = W2^T, both [D, d]
 * row-major, so neuron j's input and output weights are rows j.  x and y are
 * [B, d].  f16 and bf16 only (matrix cores; SHA_ERR_UNSUPPORTED otherwise);
 * d must be a multiple of 256 and one weight matrix below 4 GiB
 * (D * d * 2 < 2^32), else SHA_ERR_UNSUPPORTED.  Accumulation is fp32;
 * relu(x W1[:, S]) is rounded once to the element type before the second
 * product.
 */

/*
 * S_B on the device: the sorted union of the entries of row_neurons [B, k]
 * (int32, device) that lie in [0, D) (others, e.g. -1 padding, are skipped).
 * Writes the union to sel[0 .. n-1] (sel must hold min(D, B*k) entries) and
 * n to *n_sel (device int32).  Deterministic; no host synchronisation.
 *   workspace: caller-owned device buffer of at least
 *              sha_mlp_union_workspace_bytes(D) bytes (one flag byte per
 *              neuron, 256-byte padded), 16-byte aligned; contents on entry
 *              do not matter.
 * Errors: D < 1, B < 0 or k < 0 -> SHA_ERR_INVALID_ARG; null sel / n_sel
 * (or row_neurons when B*k > 0) -> SHA_ERR_INVALID_ARG; short workspace ->
 * SHA_ERR_WORKSPACE.
 */
size_t sha_mlp_union_workspace_bytes(int D);
sha_status sha_mlp_union(const int32_t* row_neurons, int B, int k, int D, int32_t* sel,
                         int32_t* n_sel, hipStream_t stream, void* workspace,
                         size_t workspace_bytes);

/*
 * y = relu(x w1t[S]^T) w2t[S] for S = sel[0 .. *n_sel - 1].
 *   sel, n_sel: device int32; *n_sel is read on the device and clamped to
 *               [0, n_max]; selection entries outside [0, D) contribute
 *               nothing.  n_max (host, 0 <= n_max <= D) bounds the count and
 *               sizes the grids and the workspace.
 *   workspace : caller-owned device buffer of at least
 *               sha_selective_mlp_workspace_bytes(B, d, D, n_max, num_cus = 0)
 *               bytes, 16-byte aligned; contents on entry do not matter.
 * B == 0 is an empty call.  y is fully written (zeros when S is empty).
 */
size_t sha_selective_mlp_workspace_bytes(int B, int d, int D, int n_max, int num_cus);
sha_status sha_selective_mlp(const void* x, const void* w1t, const void* w2t, const int32_t* sel,
                             const int32_t* n_sel, int n_max, int B, int d, int D, void* y,
                             hipStream_t stream, sha_dtype dtype, void* workspace,
                             size_t workspace_bytes);

/*
 * Multi-layer decode step.  The pages measure batched decoding throughput of
 * whole models with the routers included, captured in CUDA graphs, and keep
 * layer 0's attention dense because that layer's heads always matter most
 * (Polar Sparsity notes, papernotes.org: 方法详解 > 关键设计 > "Attention Head
 * 稀疏性", findings; 亮点与洞察, integration with CUDA Graphs; reproducibility
 * page, ri.k117.org, "Software Dependencies").  A sha_step strings the sparse parts of one
 * decode step together for n_layers layers, in order, on one stream:
 *
 *   sparse layer: sha_router_topk_ex(router_x, router_w, router_bias) -> index
 *                 (the K-split form where sha_router_workspace_bytes picks it,
 *                 in the step's own workspace)
 *                 sha_decode_kv / sha_decode_gqa_kv(q, k, v, index) -> o
 *   dense layer : sha_decode_kv / sha_decode_gqa_kv over every head (group)
 *   both, when mlp_w1t != NULL:
 *                 sha_mlp_union(mlp_rows) -> S_B, sha_selective_mlp -> mlp_y
 *
 * and, with use_graph != 0, captures that sequence once into a HIP graph so
 * that sha_step_run is a single graph launch.  The projections around these
 * calls (QKV, output, the MLP router) are the caller's: the step reads its
 * inputs from the pointers given here on every run, so a caller refreshes
 * them in place between runs.  All pointers are device pointers owned by the
 * caller and must stay valid until sha_step_destroy.  The step owns its
 * workspaces (allocated in sha_step_create) and the dense index.
 * Each layer's attention uses the library's split plan for the shared
 * shape; cfg->top_k applies to sparse layers; a dense layer selects all H
 * heads (H_kv groups when gqa != 0).
 * Errors: any argument error of the underlying calls is returned by
 * sha_step_create (nothing is captured or kept); SHA_ERR_HIP for a failing
 * allocation, capture or launch.  Runs of one step must be ordered (they
 * share its workspaces), and sha_step_destroy is called once the last run
 * has finished (it frees the workspaces).  sha_step_create checks every
 * call by capturing the sequence once (nothing executes); with
 * use_graph == 0 the capture is kept only as that check and sha_step_run
 * enqueues the calls one by one.
 */
typedef struct sha_step_config {
  int B, H, H_kv, Nkv, d, top_k, gqa;
  float scale;
  sha_dtype dtype;
  int router_d;          /* router input width */
  int mlp_d, mlp_D, mlp_k;  /* selective MLP shape; mlp_k = neurons per row */
} sha_step_config;

typedef struct sha_step_layer {
  const void* router_x;      /* [B, router_d] (sparse layers) */
  const void* router_w;      /* [H or H_kv, router_d] */
  const float* router_bias;  /* [H or H_kv] or NULL */
  float* router_scores;      /* [B, H or H_kv] fp32 output (sparse layers) */
  int32_t* index;            /* [B, top_k] router output (sparse layers; unused when dense) */
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const sha_kv_layout* kv;   /* NULL: contiguous; copied at create */
  int dense;                 /* 1: all heads, no router */
  const void* mlp_x;         /* [B, mlp_d] */
  const void* mlp_w1t;       /* [mlp_D, mlp_d] or NULL (no MLP in this layer) */
  const void* mlp_w2t;       /* [mlp_D, mlp_d] */
  void* mlp_y;               /* [B, mlp_d] */
  const int32_t* mlp_rows;   /* [B, mlp_k] */
} sha_step_layer;

typedef struct sha_step sha_step;

sha_status sha_step_create(const sha_step_config* cfg, const sha_step_layer* layers, int n_layers,
                           int use_graph, sha_step** step);
sha_status sha_step_run(sha_step* step, hipStream_t stream);
sha_status sha_step_destroy(sha_step* step);

/* Human-readable name of a status code (static storage). */
const char* sha_status_string(sha_status s);
/* Raw hipError_t of the last SHA_ERR_HIP returned on the calling thread. */
int sha_last_hip_error(void);
/* Library version, "major.minor.patch" (static storage). */
const char* sha_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SHA_H_ */
