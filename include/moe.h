/*
 * moe.h -- C ABI of libmoe.so: the forward hot path of a Mixture-of-Experts
 * (MoE) layer on one AMD MI355X (gfx950) GPU, and its backward pass.
 *
 * The layer (per token x_t, N routed experts, top-K):
 *   logits = W_r . x_t (+ b_r) (+ offset)            router scoring
 *   sel    = TopK(logits + sel_bias), w = softmax over the K chosen logits
 *   dispatch: (token, slot) pairs -> contiguous per-expert row blocks,
 *             at most C rows per expert when a capacity is set
 *   E_e(x) = W2_e . GELU(W1_e . x + b1_e) + b2_e     per-expert FFN
 *   out_t  = sum_k w[t,k] * E_{sel_k}(x_t) (+ E_shared(x_t))
 *   aux    = alpha * N * sum_e f_e * P_e             Switch load-balance loss
 *
 * Sources (by page title and section):
 *   lmnt.cn MoE walkthrough (news/351908): §1.2 per-token flow; §2.1 gate
 *     scoring equation (score = Softmax(TopK(W_g x))); §3.1 dispatch; §3.2
 *     combine equation; §3.3 capacity equation; §5.1-5.2 balance loss.
 *   yunthe.com "MoE混合专家模型实战": "MoE架构的稀疏激活原理与Transformer实现"
 *     (output equation, reference forward, grouped GEMM over same-expert
 *     tokens); "专家负载均衡与辅助损失函数设计" (aux loss, per-expert bias b_i,
 *     capacity drop).
 *   wiblog.cn "MoE 专家路由如何实现稀疏激活": fine-grained and shared experts.
 *   lmnt.cn §4.3 and yunthe.com's deployment section: expert weights stored
 *     as INT8 or INT4 for inference (weight-only quantisation).
 *
 * Conventions for every entry point:
 *   - Ownership: the caller owns every buffer.  The library never allocates
 *     device memory (beyond the fixed scratch array of
 *     moe_layer_forward_noalloc, which exists once per GPU), never frees,
 *     and never synchronises the stream; every call only enqueues kernels on
 *     `stream` and returns.
 *   - Pointers marked [dev] are device pointers, 16-byte aligned; [host]
 *     pointers are read during the call only.
 *   - Layout: row-major; weight matrices use the nn.Linear [out, in] layout,
 *     so the reduction dimension is contiguous.  dtype MOE_BF16 means
 *     bfloat16 storage with fp32 accumulation; MOE_F32 means fp32 throughout.
 *   - Sizes: buffers are sized for the worst case M_max = T*K permuted rows.
 *     Data-dependent counts stay on the device.
 *   - Errors: arguments are checked on the host before any launch; a non-OK
 *     return enqueues nothing.  moe_last_error() gives a thread-local message.
 *     A failed launch returns MOE_ERR_HIP.  No C++ exception crosses the ABI.
 *   - Limits: 1 <= K <= N <= 256, K <= 64, T >= 1, d_model, d_ff and
 *     d_ff_shared multiples of 64, T*K*max(d_model, d_ff) < 2^31,
 *     d_model*d_ff and d_model*d_ff_shared < 2^31.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs on every call.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or config */
  MOE_ERR_UNSUPPORTED = -2, /* valid MoE shape outside this build's limits */
  MOE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required  */
  MOE_ERR_HIP = -4          /* a kernel launch failed                      */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Storage of the routed experts' weights w1 / w2.  MOE_WQ_INT8: int8 codes q
 * with one fp32 scale per output row (w1_scale [N, f], w2_scale [N, d]); the
 * expert uses the weights scale * q (moe_quantize_int8 makes them).
 * MOE_WQ_INT4: 4-bit codes q in [-7, 7], two per byte along the row (element
 * 2i in the low nibble of byte i, 4-bit two's complement), so w1 is
 * [N, f, d/2] bytes and w2 [N, d, f/2] bytes, with the same fp32 row scales
 * (moe_quantize_int4 makes them); needs d_model and d_ff multiples of 128.
 * Quantised weights need dtype MOE_BF16; the shared expert and the router
 * stay in dtype. */
typedef enum { MOE_WQ_NONE = 0, MOE_WQ_INT8 = 1, MOE_WQ_INT4 = 2 } moe_weight_quant_t;

/* How moe_route forms the logits (lmnt.cn §2.1 gate scoring; the Top-K
 * decisions are the same on both paths).
 * MOE_ROUTER_EXACT: every dot product accumulated in fp64 on the fp64
 *   matrix cores, rounded once to fp32.
 * MOE_ROUTER_CERTIFIED (dtype MOE_BF16 only): the bf16 matrix cores with
 *   fp32 sums of 32 products folded into fp64, plus a proven bound B on the
 *   error of each dot product.  A token whose Top-K set and order follow
 *   from the bounds alone keeps these approximate logits; for every other
 *   token each expert whose score interval reaches the K-th largest lower
 *   bound is recomputed in fp64 before the selection.  topk_idx is the same
 *   as on the exact path; a logit may differ from the exact one by the
 *   bound (B <= ~4e-6 * |x_t| * |W_r[e]|), the K chosen logits of a
 *   recomputed token not at all.
 * MOE_ROUTER_AUTO: CERTIFIED for bf16 layers with 2 T N d >= 2^31 (where
 *   the fp64 router GEMM is a visible share of the layer), else EXACT. */
typedef enum {
  MOE_ROUTER_AUTO = 0,
  MOE_ROUTER_EXACT = 1,
  MOE_ROUTER_CERTIFIED = 2
} moe_router_t;

typedef struct {
  int32_t T;           /* tokens in the batch                                  */
  int32_t d_model;     /* d                                                    */
  int32_t d_ff;        /* f, hidden width of every routed expert               */
  int32_t n_experts;   /* N routed experts                                     */
  int32_t top_k;       /* K experts per token                                  */
  int32_t capacity;    /* C: <= 0 dropless; else at most C rows per expert     */
  int32_t d_ff_shared; /* 0: no shared expert; else its hidden width f_s       */
  int32_t dtype;       /* moe_dtype_t of x, expert weights, intermediates, out */
  float aux_alpha;     /* alpha of the aux loss (used by moe_layer_forward)    */
  int32_t weight_quant;/* moe_weight_quant_t of the routed experts' w1 / w2    */
  int32_t router;      /* moe_router_t: how the router logits are formed        */
} moe_config_t;

typedef struct {
  const void *w_router;     /* [dev] [N, d] dtype                                  */
  const float *b_router;    /* [dev] [N] fp32 or NULL: added to the logits         */
  const float *logit_offset;/* [dev] [N] fp32 or NULL: added to the logits         */
  const float *sel_bias;    /* [dev] [N] fp32 or NULL: added for selection only    */
  const void *w1;           /* [dev] [N, f, d] dtype (codes: see moe_weight_quant_t) */
  const void *b1;           /* [dev] [N, f] dtype or NULL                          */
  const void *w2;           /* [dev] [N, d, f] dtype (codes: see moe_weight_quant_t) */
  const void *b2;           /* [dev] [N, d] dtype or NULL                          */
  const void *ws1;          /* [dev] [f_s, d] dtype (shared expert) or NULL        */
  const void *ws2;          /* [dev] [d, f_s] dtype (shared expert) or NULL        */
  const float *w1_scale;    /* [dev] [N, f] fp32 with quantised weights, else ignored */
  const float *w2_scale;    /* [dev] [N, d] fp32 with quantised weights, else ignored */
} moe_weights_t;

typedef enum {
  MOE_STAGE_ROUTE = 0,
  MOE_STAGE_DISPATCH = 1,
  MOE_STAGE_EXPERT_FFN = 2,
  MOE_STAGE_COMBINE = 3,
  MOE_STAGE_AUX = 4,
  MOE_STAGE_LAYER = 5,
  MOE_STAGE_EXPERT_FFN_TRAIN = 6,    /* moe_expert_ffn_train     */
  MOE_STAGE_LAYER_TRAIN = 7,         /* moe_layer_forward_train  */
  MOE_STAGE_EXPERT_FFN_BACKWARD = 8, /* moe_expert_ffn_backward  */
  MOE_STAGE_ROUTE_BACKWARD = 9,      /* moe_route_backward       */
  MOE_STAGE_LAYER_BACKWARD = 10      /* moe_layer_backward       */
} moe_stage_t;

/* Bytes of device workspace the entry point of `stage` needs for `cfg`
 * (0 if none; (size_t)-1 if cfg is invalid).  Any buffer of at least this
 * size, 256-byte aligned, may be passed as `ws`; its contents on entry do
 * not matter and are clobbered. */
size_t moe_workspace_size(const moe_config_t *cfg, moe_stage_t stage);

/* capacity = ceil(T / N * capacity_factor), computed exactly for the binary
 * value of capacity_factor (lmnt.cn walkthrough §3.3, capacity equation).
 * Returns -1 for T < 1, N < 1 or capacity_factor not finite and > 0. */
int32_t moe_capacity_from_factor(int32_t T, int32_t n_experts, double capacity_factor);

/* Bytes of the routing-partials buffer of moe_route ((size_t)-1 if cfg is
 * invalid).  With nb = ceil(T / 4) blocks of four consecutive tokens it holds,
 * in this order, each array starting on a 256-byte boundary:
 *   ppart [nb, N] fp64  sum over the block's tokens of softmax_N(logits_t)
 *   zpart [nb]    fp64  sum over the block's tokens of (logsumexp logits_t)^2
 *   spw   [nb, N] fp64  sum of the routing weights topk_w[t, k] routed to e
 *   spcnt [nb, N] int32 number of (t, k) routed to e (before capacity drops)
 * (sums in token order, pairs in (token, slot) order).  moe_aux_loss,
 * moe_router_z_loss and moe_routing_stats reduce it without reading the
 * logits or the routing again. */
size_t moe_route_partials_size(const moe_config_t *cfg);

/* The router path (MOE_ROUTER_EXACT or MOE_ROUTER_CERTIFIED) that cfg->router
 * resolves to; -1 if cfg is invalid or asks for CERTIFIED with fp32. */
int moe_router_path(const moe_config_t *cfg);

/* Router scoring and Top-K routing (lmnt.cn §2.1 gate scoring equation and
 * the TopK-then-Softmax order; yunthe.com reference forward; yunthe.com
 * per-expert bias b_i for selection).
 *   x        [dev] [T, d] dtype
 *   logits   [dev] [T, N] fp32 out, or NULL.  logits = fp32 rounding of the
 *            dot product accumulated in fp64, plus b_router and
 *            logit_offset added in fp64 before that single rounding (on the
 *            certified path the dot product may be the bounded
 *            approximation, see moe_router_t).
 *   topk_idx [dev] [T, K] int32 out: the K experts with the largest
 *            fp32(logit + sel_bias), ordered by (score desc, index asc);
 *            NaN scores order as -inf.
 *   topk_w   [dev] [T, K] fp32 out: softmax over the K chosen unbiased logits
 *            (computed in fp64, rounded once).
 *   partials [dev] out or NULL, 256-byte aligned, moe_route_partials_size(cfg)
 *            bytes: the routing partials of the aux loss (P, lmnt.cn §5.1-5.2),
 *            the z-loss (lmnt.cn §5.3) and the routing statistics (lmnt.cn
 *            §8.2), formed while each token's logits are in registers.
 *   ws       [dev] >= moe_workspace_size(cfg, MOE_STAGE_ROUTE) bytes (partial
 *            dot products). */
int moe_route(const moe_config_t *cfg, const void *x, const moe_weights_t *w, float *logits,
              int32_t *topk_idx, float *topk_w, void *partials, void *ws, size_t ws_bytes,
              hipStream_t stream);

/* Dispatch: permute tokens from token order to contiguous per-expert blocks
 * (lmnt.cn §3.1), with the capacity limit of lmnt.cn §3.3.  (token, slot)
 * pairs are taken token-major; within an expert they keep token order; a pair
 * is kept iff fewer than C earlier pairs chose its expert.
 *   topk_idx       [dev] [T, K] int32 in.  Indices outside [0, N) are ignored
 *                  (slot_row -1, counted as dropped).
 *   x              [dev] [T, d] dtype in.
 *   counts         [dev] [N] int32 out: pre-drop pairs per expert.
 *   expert_offsets [dev] [N+1] int32 out: exclusive scan of min(counts, C).
 *   slot_row       [dev] [T, K] int32 out: row of the pair in x_perm, -1 if dropped.
 *   row_token      [dev] [T*K] int32 out: token of each row (first M rows valid,
 *                  M = expert_offsets[N]).
 *   x_perm         [dev] [T*K, d] dtype out: x_perm[r] = x[row_token[r]] (first M rows).
 *   n_dropped      [dev] [1] int32 out: T*K - M.
 *   ws             [dev] >= moe_workspace_size(cfg, MOE_STAGE_DISPATCH) bytes. */
int moe_dispatch(const moe_config_t *cfg, const int32_t *topk_idx, const void *x,
                 int32_t *counts, int32_t *expert_offsets, int32_t *slot_row,
                 int32_t *row_token, void *x_perm, int32_t *n_dropped, void *ws,
                 size_t ws_bytes, hipStream_t stream);

/* Per-expert FFN as grouped GEMMs over the ragged expert blocks (yunthe.com
 * reference forward: Linear, GELU, Linear; batched per expert as a grouped
 * GEMM).  GELU(z) = z/2 (1 + erf(z / sqrt 2)), fused into the first GEMM's
 * epilogue: fp32 layers use the library erff; bf16 layers (every GEMM path)
 * use erf from Abramowitz-Stegun formula 7.1.26, whose GELU is within 2.2e-7
 * absolute of the exact one (<= 0.013 bf16 ulp of the result for |z| < 3).
 *   x_perm         [dev] [T*K, d] dtype in (first expert_offsets[N] rows used).
 *   expert_offsets [dev] [N+1] int32 in (as written by moe_dispatch).
 *   x              [dev] [T, d] dtype in: input of the shared expert; may be
 *                  NULL when cfg->d_ff_shared == 0.
 *   y_perm         [dev] [T*K, d] dtype out: E_e(x_perm[r]) for the rows of e.
 *   y_shared       [dev] [T, d] dtype out: E_shared(x_t); NULL iff no shared expert.
 *   ws             [dev] >= moe_workspace_size(cfg, MOE_STAGE_EXPERT_FFN) bytes
 *                  (holds the hidden activations). */
int moe_expert_ffn(const moe_config_t *cfg, const void *x_perm, const int32_t *expert_offsets,
                   const moe_weights_t *w, const void *x, void *y_perm, void *y_shared,
                   void *ws, size_t ws_bytes, hipStream_t stream);

/* Combine: restore token order and sum the K expert outputs weighted by the
 * routing weights (lmnt.cn §3.2 combine equation; yunthe.com output
 * equation), in slot order k = 0..K-1, fp32 accumulation; dropped slots
 * (slot_row -1) contribute 0 and the other weights are not renormalised;
 * then the shared expert's output is added with weight 1 (wiblog.cn shared
 * expert).  The residual add is the caller's.
 *   y_perm   [dev] [T*K, d] dtype in;  slot_row [dev] [T, K] int32 in;
 *   topk_w   [dev] [T, K] fp32 in;     y_shared [dev] [T, d] dtype in or NULL;
 *   out      [dev] [T, d] dtype out. */
int moe_combine(const moe_config_t *cfg, const void *y_perm, const int32_t *slot_row,
                const float *topk_w, const void *y_shared, void *out, hipStream_t stream);

/* Switch auxiliary load-balance loss (yunthe.com "专家负载均衡与辅助损失函数设计";
 * lmnt.cn §5.1): alpha * N * sum_e f_e * P_e, with f_e = counts[e] / T (mean
 * of the pre-drop 0/1 selection mask, so sum f = K) and P_e the mean over
 * tokens of softmax_N(logits[t])_e.  Exponentials in fp32, all sums and
 * products in fp64, with a fixed reduction order (deterministic); written as
 * fp32.  Relative error ~1e-7.  The same bits from the logits or from
 * moe_route's partials.
 *   logits   [dev] [T, N] fp32 in, or NULL;
 *   partials [dev] in (moe_route's), or NULL: exactly one of the two;
 *   counts [dev] [N] int32 in: moe_dispatch's pre-drop counts (f needs only
 *            the per-expert selection counts, which dispatch has already
 *            histogrammed; no pass over topk_idx);
 *   loss_out [dev] [1] fp32 out;  alpha = cfg->aux_alpha;
 *   ws [dev] >= moe_workspace_size(cfg, MOE_STAGE_AUX) bytes. */
int moe_aux_loss(const moe_config_t *cfg, const float *logits, const void *partials,
                 const int32_t *counts, float *loss_out, void *ws, size_t ws_bytes,
                 hipStream_t stream);

/* Routing statistics (lmnt.cn MoE walkthrough §8.2, measuring the routing
 * distribution: tokens received per expert and the mean routing weight; the
 * drop count is moe_dispatch's n_dropped): counts_out[e] = number of (t, k) with topk_idx[t, k] == e (before
 * capacity drops, equal to moe_dispatch's counts); weight_mean_out[e] = the
 * mean of topk_w[t, k] over those pairs, 0 for an expert nobody chose.  Sums
 * in fp64 with a fixed order (deterministic); the means are written as fp32.
 *   topk_idx [dev] [T, K] int32 in;  topk_w [dev] [T, K] fp32 in (moe_route);
 *            both NULL when partials are given;
 *   partials [dev] in (moe_route's) or NULL;
 *   counts_out [dev] [N] int32 out or NULL;  weight_mean_out [dev] [N] fp32 out;
 *   ws [dev] >= moe_workspace_size(cfg, MOE_STAGE_AUX) bytes.
 * Errors: MOE_ERR_INVALID_ARG for NULL or misaligned required pointers or
 * both inputs given, MOE_ERR_WORKSPACE for a short or misaligned workspace. */
int moe_routing_stats(const moe_config_t *cfg, const int32_t *topk_idx, const float *topk_w,
                      const void *partials, int32_t *counts_out, float *weight_mean_out, void *ws,
                      size_t ws_bytes, hipStream_t stream);

/* Router z-loss (lmnt.cn MoE walkthrough §5.3, router z-loss equation):
 * beta * (1/T) sum_t (logsumexp_e logits[t, e])^2, which penalises large
 * router logits.  Exponentials in fp32, sums and logarithm in fp64, with a
 * fixed reduction order (deterministic); written as fp32.
 *   logits [dev] [T, N] fp32 in (from moe_route), or NULL;
 *   partials [dev] in (moe_route's), or NULL: exactly one of the two;
 *   beta: finite weight;  loss_out [dev] [1] fp32 out;
 *   ws [dev] >= moe_workspace_size(cfg, MOE_STAGE_AUX) bytes.
 * Errors: MOE_ERR_INVALID_ARG for neither or both of logits / partials, NULL
 * loss_out or a non-finite beta, MOE_ERR_WORKSPACE for a short or misaligned
 * workspace. */
int moe_router_z_loss(const moe_config_t *cfg, const float *logits, const void *partials,
                      float beta, float *loss_out, void *ws, size_t ws_bytes, hipStream_t stream);

/* The whole layer (lmnt.cn §1.2 per-token flow: gate scores, Top-K experts,
 * dispatch, expert computation, weighted combine): route -> dispatch ->
 * expert FFN (+ shared expert) -> combine (-> aux loss when aux_out != NULL,
 * from the routing partials the route stage writes).  Same kernels and
 * results as calling the stages in order.
 *   x [dev] [T, d] dtype in;  out [dev] [T, d] dtype out;
 *   aux_out [dev] [1] fp32 out or NULL;  counts_out [dev] [N] int32 out or NULL;
 *   n_dropped_out [dev] [1] int32 out or NULL;
 *   ws [dev] >= moe_workspace_size(cfg, MOE_STAGE_LAYER) bytes. */
int moe_layer_forward(const moe_config_t *cfg, const void *x, const moe_weights_t *w,
                      void *out, float *aux_out, int32_t *counts_out, int32_t *n_dropped_out,
                      void *ws, size_t ws_bytes, hipStream_t stream);

/* The layer with its training signals and routing statistics (lmnt.cn §5.1-5.3
 * balance loss and router z-loss; §8.2 per-step monitoring of tokens per
 * expert, mean routing weight and drops).  Every field is optional. */
typedef struct {
  float *aux_out;          /* [dev] [1] fp32 or NULL: aux loss with cfg->aux_alpha  */
  float zloss_beta;        /* z-loss weight beta (finite; used with zloss_out)      */
  float *zloss_out;        /* [dev] [1] fp32 or NULL: beta * mean_t lse_t^2         */
  int32_t *counts_out;     /* [dev] [N] int32 or NULL: pre-drop pairs per expert    */
  int32_t *n_dropped_out;  /* [dev] [1] int32 or NULL: pairs dropped by capacity    */
  float *weight_mean_out;  /* [dev] [N] fp32 or NULL: mean routing weight per expert */
} moe_layer_stats_t;

/* moe_layer_forward with the outputs of `stats`: the aux loss, z-loss and
 * mean routing weights come from the routing partials the select kernel
 * writes while it holds each token's logits (no further pass over the
 * logits), with the same bits as moe_aux_loss / moe_router_z_loss /
 * moe_routing_stats.
 *   stats [host] read during the call;  other arguments as moe_layer_forward;
 *   ws [dev] >= moe_workspace_size(cfg, MOE_STAGE_LAYER) bytes. */
int moe_layer_forward_stats(const moe_config_t *cfg, const void *x, const moe_weights_t *w,
                            void *out, const moe_layer_stats_t *stats, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* The same layer as moe_layer_forward, for callers that cannot allocate
 * device memory: code being captured into a HIP graph, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace is a device array the
 * library holds itself (MOE_NOALLOC_SCRATCH_BYTES per GPU, from the first
 * call on that GPU until the process ends), so the call allocates nothing and
 * takes no workspace argument; results are those of moe_layer_forward,
 * bit for bit.
 *   Arguments as moe_layer_forward without ws / ws_bytes.
 *   Limit: moe_workspace_size(cfg, MOE_STAGE_LAYER) must not exceed
 *   MOE_NOALLOC_SCRATCH_BYTES (decode-shaped and small-batch layers fit);
 *   otherwise MOE_ERR_WORKSPACE and nothing is enqueued.
 *   Concurrency: every call on one GPU uses that GPU's one scratch array;
 *   calls that overlap on one GPU (other streams or threads, without an
 *   ordering between them) race and give undefined results.
 *   Errors: as moe_layer_forward; MOE_ERR_HIP if the scratch address cannot
 *   be obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int moe_layer_forward_noalloc(const moe_config_t *cfg, const void *x, const moe_weights_t *w,
                              void *out, float *aux_out, int32_t *counts_out,
                              int32_t *n_dropped_out, hipStream_t stream);

/* Weight-only INT8 quantisation of a weight matrix, one fp32 scale per row
 * (lmnt.cn §4.3: expert weights compressed to INT8 for inference; the pages
 * fix no scheme, this is the symmetric per-output-channel one):
 *   scale[r] = fp32(max_c |w[r, c]| / 127)
 *   q[r, c]  = clamp(round_half_even(fp32(w[r, c] / scale[r])), -127, 127)
 * with IEEE fp32 divisions, so the codes are reproducible bit for bit; a row
 * of zeros gets scale 0 and codes 0.  For the experts' w1 [N, f, d] call it
 * with rows = N*f, cols = d (w2: rows = N*d, cols = f).
 *   w     [dev] [rows, cols] dtype (MOE_BF16 or MOE_F32) in;
 *   q     [dev] [rows, cols] int8 out;  scale [dev] [rows] fp32 out.
 * Errors: MOE_ERR_INVALID_ARG for NULL or misaligned pointers, rows < 1, cols
 * not a positive multiple of 64, or an unknown dtype. */
int moe_quantize_int8(const void *w, int32_t dtype, int64_t rows, int32_t cols, int8_t *q,
                      float *scale, hipStream_t stream);

/* Weight-only INT4 quantisation, one fp32 scale per row (lmnt.cn §4.3 names
 * INT4 beside INT8 for the expert weights, a quarter of their 16-bit memory
 * and bandwidth; the scheme is moe_quantize_int8's with 4-bit codes):
 *   scale[r] = fp32(max_c |w[r, c]| / 7)
 *   q[r, c]  = clamp(round_half_even(fp32(w[r, c] / scale[r])), -7, 7)
 * IEEE fp32 divisions (codes reproducible bit for bit); a row of zeros gets
 * scale 0 and codes 0.  Codes are packed two per byte: element 2i of a row in
 * the low nibble of byte i, element 2i+1 in the high nibble (4-bit two's
 * complement).  For w1 [N, f, d]: rows = N*f, cols = d (w2: rows = N*d,
 * cols = f).
 *   w     [dev] [rows, cols] dtype (MOE_BF16 or MOE_F32) in;
 *   q     [dev] [rows, cols/2] bytes out;  scale [dev] [rows] fp32 out.
 * Errors: MOE_ERR_INVALID_ARG for NULL or misaligned pointers, rows < 1, cols
 * not a positive multiple of 64, or an unknown dtype. */
int moe_quantize_int4(const void *w, int32_t dtype, int64_t rows, int32_t cols, uint8_t *q,
                      float *scale, hipStream_t stream);

/* ------------------------------------------------------------------ training
 * The backward pass (lmnt.cn MoE walkthrough §2.2: in training the K routing
 * weights take part in back-propagation, which is how the gate learns its
 * scores; §5.1-5.3: the balance loss and the z-loss act on the gate through
 * its probabilities and logits; §4.1: under mixed precision the gradients are
 * kept in 16 bits like the weights; §6.2: an expert that receives no tokens
 * gets no gradient).
 *
 * What is differentiated: the forward above with the Top-K choice and the
 * capacity drops held at their forward values (both are piecewise constant
 * in the inputs), the fp32 rounding of the logits taken as the identity,
 * sel_bias and logit_offset constants, and the aux loss's f_e (a count)
 * constant.  The scalar is
 *   L = <d_out, out> + aux_grad * aux + zloss_grad * zloss_beta * mean_t lse_t^2
 * with aux = cfg->aux_alpha * N * sum_e f_e P_e as in moe_aux_loss.
 *
 * Precision: the expert GEMMs run on the forward's kernels (bf16 operands,
 * fp32 accumulation, results rounded to dtype); d_h, d_z and the expert
 * weight and bias gradients are stored in dtype; every sum over rows or
 * tokens is fp32 with a fixed order (deterministic); the router gradients
 * d_w_router, d_b_router and the router's share of d_x are fp32.
 * Quantised experts are inference-only: every training entry point returns
 * MOE_ERR_UNSUPPORTED for MOE_WQ_INT8 and MOE_WQ_INT4, and for
 * max(d_model, d_ff, d_ff_shared) * (T*K + 32*N) >= 2^31.
 */

/* Tensors the training forward keeps for the backward.  All [dev],
 * caller-owned, 16-byte aligned; rows past expert_offsets[N] are unused. */
typedef struct {
  float *logits;            /* [T, N] fp32                                    */
  int32_t *topk_idx;        /* [T, K]                                         */
  float *topk_w;            /* [T, K] fp32                                    */
  int32_t *counts;          /* [N] pre-drop selections                        */
  int32_t *expert_offsets;  /* [N+1]                                          */
  int32_t *slot_row;        /* [T, K]                                         */
  int32_t *row_token;       /* [T*K]                                          */
  int32_t *n_dropped;       /* [1]                                            */
  void *x_perm;             /* [T*K, d] dtype                                 */
  void *z;                  /* [T*K, f] dtype: W1 x + b1, before the GELU     */
  void *h;                  /* [T*K, f] dtype: GELU(z)                        */
  void *y_perm;             /* [T*K, d] dtype                                 */
  void *zs;                 /* [T, f_s] dtype (shared expert), or NULL        */
  void *hs;                 /* [T, f_s] dtype (shared expert), or NULL        */
} moe_saved_t;

/* Gradients.  All [dev], caller-owned, overwritten (not accumulated). */
typedef struct {
  float *d_w_router;        /* [N, d] fp32                                    */
  float *d_b_router;        /* [N] fp32, or NULL: not written                 */
  void *d_w1;               /* [N, f, d] dtype                                */
  void *d_b1;               /* [N, f] dtype, or NULL: not written             */
  void *d_w2;               /* [N, d, f] dtype                                */
  void *d_b2;               /* [N, d] dtype, or NULL: not written             */
  void *d_ws1;              /* [f_s, d] dtype (shared expert), or NULL        */
  void *d_ws2;              /* [d, f_s] dtype (shared expert), or NULL        */
} moe_grads_t;

/* moe_expert_ffn that keeps its intermediates: GEMM1 writes z = W1 x + b1
 * (no GELU), a GELU pass writes h = GELU(z), GEMM2 reads h.  Same arguments
 * as moe_expert_ffn plus z, h [T*K, f] and, with a shared expert, zs, hs
 * [T, f_s] (all [dev] dtype out).  The rounding of z to dtype before the GELU
 * is the only difference from moe_expert_ffn.
 *   ws [dev] >= moe_workspace_size(cfg, MOE_STAGE_EXPERT_FFN_TRAIN) bytes. */
int moe_expert_ffn_train(const moe_config_t *cfg, const void *x_perm,
                         const int32_t *expert_offsets, const moe_weights_t *w, const void *x,
                         void *z, void *h, void *y_perm, void *zs, void *hs, void *y_shared,
                         void *ws, size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward that fills `saved` (route, dispatch and
 * moe_expert_ffn_train into the caller's buffers, then combine; the aux loss
 * when aux_out != NULL).
 *   x [dev] [T, d] dtype in;  out [dev] [T, d] dtype out;
 *   aux_out [dev] [1] fp32 out or NULL;  saved: every pointer [dev] out;
 *   ws [dev] >= moe_workspace_size(cfg, MOE_STAGE_LAYER_TRAIN) bytes. */
int moe_layer_forward_train(const moe_config_t *cfg, const void *x, const moe_weights_t *w,
                            void *out, float *aux_out, const moe_saved_t *saved, void *ws,
                            size_t ws_bytes, hipStream_t stream);

/* Combine backward (the transpose of lmnt.cn §3.2's weighted sum):
 *   d_y_perm[slot_row[t,k]] = topk_w[t,k] * d_out[t]       (kept slots only)
 *   d_topk_w[t,k] = <d_out[t], y_perm[slot_row[t,k]]>      (0 if dropped)
 * dot products in fp32 with a fixed order.
 *   d_out [dev] [T, d] dtype in;  y_perm [dev] [T*K, d] dtype in;
 *   slot_row [dev] [T, K] int32 in;  topk_w [dev] [T, K] fp32 in;
 *   d_y_perm [dev] [T*K, d] dtype out;  d_topk_w [dev] [T, K] fp32 out. */
int moe_combine_backward(const moe_config_t *cfg, const void *d_out, const void *y_perm,
                         const int32_t *slot_row, const float *topk_w, void *d_y_perm,
                         float *d_topk_w, hipStream_t stream);

/* Expert FFN backward, routed experts then the shared one (whose upstream
 * gradient is d_out itself, weight 1):
 *   d_h = d_y W2_e,  d_z = d_h * GELU'(z),  d_x_perm = d_z W1_e,
 *   d_w2[e] = d_y_e^T h_e,  d_b2[e] = sum of d_y_e's rows,
 *   d_w1[e] = d_z_e^T x_perm_e,  d_b1[e] = sum of d_z_e's rows;
 * an expert with no rows gets zeros.
 *   x_perm, expert_offsets, z, h: as saved by the training forward;
 *   x [dev] [T, d], zs, hs [dev] [T, f_s]: shared expert (NULL without one);
 *   d_y_perm [dev] [T*K, d] dtype in (moe_combine_backward);
 *   d_out [dev] [T, d] dtype in (shared expert only; may be NULL without one);
 *   d_x_perm [dev] [T*K, d] dtype out;  d_x_shared [dev] [T, d] dtype out, NULL
 *   iff no shared expert;  grads: d_w1, d_w2 (+ d_b1, d_b2 if not NULL; d_ws1,
 *   d_ws2 with a shared expert) written;
 *   ws [dev] >= moe_workspace_size(cfg, MOE_STAGE_EXPERT_FFN_BACKWARD) bytes
 *   (transposed weights and activations). */
int moe_expert_ffn_backward(const moe_config_t *cfg, const void *x_perm,
                            const int32_t *expert_offsets, const moe_weights_t *w, const void *x,
                            const void *z, const void *h, const void *zs, const void *hs,
                            const void *d_y_perm, const void *d_out, void *d_x_perm,
                            void *d_x_shared, const moe_grads_t *grads, void *ws, size_t ws_bytes,
                            hipStream_t stream);

/* Router backward:
 *   d_logits[t, sel_k] = w_k (d_w_k - sum_j w_j d_w_j)          (softmax over K)
 *     + aux_grad * cfg->aux_alpha * N / T * p_te (f_e - sum_e' f_e' p_te')
 *     + zloss_grad * 2 * zloss_beta / T * lse_t * p_te,
 *   p_t = softmax_N(logits_t) (fp32), f_e = counts[e] / T;
 *   d_w_router = d_logits^T x,  d_b_router = sum_t d_logits,
 *   d_x_router = d_logits W_r   (all fp32, fixed-order sums).
 *   x [dev] [T, d] dtype in;  logits, topk_idx, topk_w: from the forward;
 *   d_topk_w [dev] [T, K] fp32 in (moe_combine_backward);
 *   counts [dev] [N] int32 in (needed when aux_alpha * aux_grad != 0);
 *   d_logits [dev] [T, N] fp32 out or NULL;  d_x_router [dev] [T, d] fp32 out
 *   or NULL;  grads: d_w_router (+ d_b_router if not NULL) written;
 *   ws [dev] >= moe_workspace_size(cfg, MOE_STAGE_ROUTE_BACKWARD) bytes. */
int moe_route_backward(const moe_config_t *cfg, const void *x, const moe_weights_t *w,
                       const float *logits, const int32_t *topk_idx, const float *topk_w,
                       const float *d_topk_w, const int32_t *counts, float aux_grad,
                       float zloss_beta, float zloss_grad, float *d_logits, float *d_x_router,
                       const moe_grads_t *grads, void *ws, size_t ws_bytes, hipStream_t stream);

/* Dispatch backward (the transpose of lmnt.cn §3.1's permutation):
 *   d_x[t] = sum over kept slots k of d_x_perm[slot_row[t,k]] (slot order)
 *            + d_x_shared[t] + d_x_router[t],
 * fp32 sums rounded once to dtype.
 *   d_x_perm [dev] [T*K, d] dtype in;  slot_row [dev] [T, K] int32 in;
 *   d_x_shared [dev] [T, d] dtype in or NULL;  d_x_router [dev] [T, d] fp32 in
 *   or NULL;  d_x [dev] [T, d] dtype out. */
int moe_dispatch_backward(const moe_config_t *cfg, const void *d_x_perm, const int32_t *slot_row,
                          const void *d_x_shared, const float *d_x_router, void *d_x,
                          hipStream_t stream);

/* The whole backward: combine, expert FFN (+ shared), router and dispatch
 * backward in that order, from the tensors moe_layer_forward_train saved.
 *   x [dev] [T, d] dtype in (the forward's input);  d_out [dev] [T, d] dtype in;
 *   aux_grad, zloss_beta, zloss_grad: finite (0 leaves that loss out);
 *   d_x [dev] [T, d] dtype out;  grads: every non-NULL field written;
 *   ws [dev] >= moe_workspace_size(cfg, MOE_STAGE_LAYER_BACKWARD) bytes. */
int moe_layer_backward(const moe_config_t *cfg, const void *x, const moe_weights_t *w,
                       const moe_saved_t *saved, const void *d_out, float aux_grad,
                       float zloss_beta, float zloss_grad, void *d_x, const moe_grads_t *grads,
                       void *ws, size_t ws_bytes, hipStream_t stream);

/* Thread-local text of the last non-OK return on this thread ("" if none). */
const char *moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
