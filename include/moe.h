/*
 * moe.h -- C ABI of the sparse MoE FFN layer forward for MI355X (gfx950).
 *
 * The layer (one forward, one GPU):
 *   router affinity  l = x W_r^T (+ logit_add)
 *   scores           s = softmax(l) per token, or sigmoid(l) per expert
 *   selection        top-k of key = fl32(s + b) (b: selection-only bias),
 *                    optionally restricted to the best topk_groups of
 *                    n_groups contiguous expert groups
 *   gates            g = s_chosen / sum(s_chosen)  (or raw s)
 *   capacity         C = floor(cf*T/N) (or max(int(cf*k*T/N), k)); the
 *                    earliest assignments to an expert keep their slot
 *   dispatch         flat token-major assignments a = t*k + j, stably grouped
 *                    by expert into contiguous segments
 *   experts          E_e(x) = W2_e (silu(W_gate,e x) * (W_up,e x))  (SwiGLU)
 *   shared expert    always on, weight 1, added
 *   combine          y_t = sum_{kept j} g_tj E_{e_tj}(x_t) + S(x_t)
 *   balancing step   b_i -= step * sign(load_i - mean load);  N sum f_i P_i
 *
 * Sources (page titles; sections):
 *   "MoE architecture in practice" (deepseekmodel.com blog): routing math
 *     (bias-free gate, jitter, softmax, top-k, renormalisation, capacity,
 *     earliest-arrival drop); load-balancing loss (f_i P_i statistic,
 *     selection-only bias with a sign update); shared expert; expert
 *     parallelism and all-to-all (token-major flatten, stable grouping,
 *     grouped GEMM over contiguous expert segments).
 *   llm-compass "MoE" page: gate equation g = softmax(TopK(x W_g, k)),
 *     y = sum g_i E_i(x); aux-loss-free selection TopK(s_i + b_i) with
 *     weights from s_i; aux loss alpha N sum f_i P_i; capacity =
 *     capacity_factor * tokens / N.
 *   "MoE common taste of open models", section 7: sigmoid scores + top-k +
 *     normalisation; router kept in fp32.
 *   "MoE industrial evolution" (alishangtian.com), section 4: node/group
 *     limited routing.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never allocates or frees memory.  Scratch space is the
 *     caller's workspace `ws` of `ws_bytes` >= moe_workspace_bytes(shape),
 *     256-byte aligned (moe_forward_noalloc alone uses a static device
 *     array of the library instead).  Entry points that take a workspace use disjoint
 *     regions of the same layout, so one workspace serves every call of one
 *     shape; two calls sharing a workspace must not overlap in time.
 *   - Activation and weight pointers (x, w_router, w1, w2, w1_shared,
 *     w2_shared, h, h_shared, y_perm, y_shared, y) must be 16-byte aligned,
 *     the fp32/int32 arrays 4-byte aligned (any fresh hipMalloc or PyTorch
 *     allocation is); a misaligned pointer is rejected with MOE_ERR_INVALID
 *     before anything is enqueued.
 *   - `stream` is a hipStream_t (NULL = default stream).  Every call only
 *     enqueues work; it returns before the GPU finishes.  Outputs are valid
 *     once the stream is synchronised.  No call synchronises the host.
 *   - Layouts are row-major and dense:
 *       x, y        [T, d_model]                 dtype
 *       w_router    [N, d_model]                 fp32
 *       logit_add   [T, N]                       fp32
 *       bias        [N]                          fp32
 *       w1          [N, 2*d_ff, d_model]         dtype (gate rows, then up rows)
 *       w2          [N, d_model, d_ff]           dtype
 *       w1_shared   [2*d_ff_shared, d_model]     dtype
 *       w2_shared   [d_model, d_ff_shared]       dtype
 *       scores      [T, N]   fp32;   topk_idx, topk_w  [T, k] int32 / fp32
 *       counts [N], offsets [N+1], slot [T*k], perm [T*k]  int32
 *     topk columns are in descending key order, ties to the lower expert.
 *     slot[a] = -1 marks a dropped assignment; perm[0..R) lists the kept
 *     assignment ids a = t*k + j expert by expert, ascending inside each
 *     segment; perm[R..T*k) is left unspecified.
 *   - dtype MOE_DTYPE_F32: activations and expert weights fp32 (all math
 *     fp32).  MOE_DTYPE_BF16: bf16 activations/weights, bf16 MFMA with fp32
 *     accumulation, SwiGLU intermediate rounded to bf16, fp32 combine.
 *     MOE_DTYPE_MXFP8 (MXFP8 experts: "MoE common taste of open models",
 *     section 2 and its closing recipe table; "MoE architecture in
 *     practice", precision section): x, y, y_perm, y_shared bf16; the expert
 *     weights and the SwiGLU intermediate (w1, w2, w1_shared, w2_shared, h,
 *     h_shared) are packed MX matrices (below); x is quantised to MXFP8
 *     along d and h along d_ff inside the expert call; E4M3 x E4M3 MFMA with
 *     the block scales applied, fp32 accumulation.  The router (GEMM,
 *     scores, selection, gates) is fp32 in all three.
 *   - Packed MX matrix of R rows and K values per row (OCP Microscaling
 *     Formats v1.0, MXFP8 with E4M3 elements): R*K code bytes, row-major,
 *     then R*K/32 scale bytes, row-major, scale byte = X + 127 for the block
 *     value 2^X.  A stack of N such matrices (w1, w2) holds the N code
 *     arrays first, then the N scale arrays; h [T*k, d_ff] and h_shared
 *     [T, d_ff_shared] are packed over all T*k (T) rows.  moe_quantize_mx
 *     writes this layout.
 *   - Errors: every argument is validated before anything is enqueued; on
 *     an error nothing is launched and the status says why.  No C++
 *     exception crosses this interface.  MOE_ERR_HIP reports a failed
 *     launch (the HIP error is then retrievable with hipGetLastError()).
 *   - Threads: every entry point may be called from several host threads at
 *     once (host state is read-only after its first initialisation, which
 *     is race-free); calls that share a workspace or an output must still
 *     not overlap on the GPU.
 *   - Determinism: every output is bitwise reproducible run to run, and the
 *     routing of a token does not depend on the other tokens of the batch
 *     (dropless) -- no atomics decide any value or order.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID = 1,     /* null required pointer or inconsistent shape */
  MOE_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels handle   */
  MOE_ERR_WORKSPACE = 3,   /* ws NULL or ws_bytes too small              */
  MOE_ERR_HIP = 4,         /* a kernel launch failed                      */
  MOE_ERR_SCRATCH = 5      /* moe_forward_noalloc: the shape needs more
                              scratch than MOE_NOALLOC_SCRATCH_BYTES       */
} moe_status;

enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1, MOE_DTYPE_MXFP8 = 2 };
/* capacity rule: TOKENS  C = floor(cf*T/N)               (llm-compass page)
 *                ASSIGNMENTS C = max(int(cf*k*T/N), k)    (deepseekmodel.com
 *                                                          TopKRouter)      */
enum { MOE_CAP_TOKENS = 0, MOE_CAP_ASSIGNMENTS = 1 };

typedef struct moe_shape {
  int64_t T;              /* tokens (batch x sequence flattened), >= 1      */
  int32_t d_model;        /* hidden size d                                  */
  int32_t n_experts;      /* routed experts N, 1..512                       */
  int32_t top_k;          /* experts per token k, 1..min(N,16)              */
  int32_t d_ff;           /* routed expert intermediate size                */
  int32_t d_ff_shared;    /* shared expert intermediate size; 0 = none      */
  int32_t score_fn;       /* MOE_SCORE_*                                    */
  int32_t renormalize;    /* 1: g = s / sum_chosen s; 0: g = s              */
  int32_t n_groups;       /* expert groups (1 = no group limit); divides N  */
  int32_t topk_groups;    /* groups kept per token; divides k               */
  float capacity_factor;  /* <= 0: dropless                                 */
  int32_t capacity_rule;  /* MOE_CAP_*                                      */
  int32_t dtype;          /* MOE_DTYPE_*: activations and expert weights    */
} moe_shape;

/* Version of this interface (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Human-readable name of a status. Never NULL. */
const char* moe_status_string(moe_status status);

/* Validate a shape without touching the GPU: MOE_OK, MOE_ERR_INVALID or
 * MOE_ERR_UNSUPPORTED.  Invalid: T < 1, N < 1, k < 1 or k > N, d_model or
 * d_ff < 1, d_ff_shared < 0, unknown enum values, n_groups < 1 or not
 * dividing N, topk_groups < 1 or > n_groups, k % topk_groups != 0,
 * k/topk_groups > N/n_groups, NaN capacity_factor.  Unsupported: N > 512,
 * k > 16, n_groups > 64, d_model, d_ff, d_ff_shared not multiples of 128
 * (MXFP8), 64 (bf16) or 32 (fp32), T*k*max(d_model, d_ff, d_ff_shared) >= 2^31,
 * 2*d_ff*d_model >= 2^31. */
moe_status moe_check_shape(const moe_shape* shape);

/* Expert capacity C the dispatch applies, or -1 when dropless.  Host-only. */
int64_t moe_capacity(const moe_shape* shape);

/* Workspace bytes that every entry point below needs for this shape
 * (0 on an invalid shape). */
size_t moe_workspace_bytes(const moe_shape* shape);

/* MXFP8 quantisation (OCP MX v1.0) of a row-major [rows, cols] matrix `in`
 * (in_dtype MOE_DTYPE_BF16 or MOE_DTYPE_F32; cols a multiple of 32) into the
 * packed MX layout at `out` (rows*cols*33/32 bytes): each block of 32
 * consecutive values of a row gets X = floor(log2 max|v|) - 8 (8 = the top
 * E4M3 binade), clamped to [-127, 127] (an all-zero block: -127; a block
 * holding an infinity: 127; NaN does not enter the maximum), and each value
 * the E4M3 code of v / 2^X: nearest, ties to the even mantissa, magnitudes
 * beyond 448 saturate, NaN gives the NaN code, the sign bit is kept.  For
 * a stack of expert matrices call it once per stack with rows = N * rows
 * per expert.  in, out 16-byte aligned device pointers.  Errors:
 * MOE_ERR_INVALID (NULL or misaligned pointer, bad dtype, rows < 1, cols
 * not a positive multiple of 32), MOE_ERR_UNSUPPORTED (rows*cols >= 2^40). */
moe_status moe_quantize_mx(const void* in, int32_t in_dtype, int64_t rows,
                           int64_t cols, void* out, void* stream);

/* Router: logits, scores, selection and gates for all T tokens.
 * x [T,d] dtype; w_router [N,d] fp32; logit_add [T,N] or NULL (added to the
 * logits: train-time jitter, logit offsets); bias [N] or NULL (selection
 * only).  scores_in [T,N] fp32 or NULL: when given, the GEMM and score
 * function are skipped and these scores are selected on (x and w_router
 * may then be NULL).  Outputs: logits_out [T,N] = x W_r^T, the affinity
 * GEMM before logit_add (NULL: not written; ignored with scores_in),
 * scores_out [T,N] (NULL: not written), topk_idx [T,k], topk_w [T,k]
 * (required).  Per-expert counts come from moe_dispatch, which needs the
 * selection anyway.
 * Source: "MoE architecture in practice", routing-math section (linear
 * affinity without a bias, softmax, top-k, renormalised gates) and
 * load-balancing section (selection on s + b, gates from s alone);
 * llm-compass "MoE" page, gate equation and aux-loss-free selection;
 * "MoE common taste of open models", section 7 (sigmoid scores, fp32
 * router); "MoE industrial evolution", section 4 (group-limited routing). */
moe_status moe_route(const moe_shape* shape, const void* x,
                     const float* w_router, const float* logit_add,
                     const float* scores_in, const float* bias,
                     float* logits_out, float* scores_out, int32_t* topk_idx,
                     float* topk_w, void* ws, size_t ws_bytes, void* stream);

/* Dispatch: per-expert counts, capacity drop and the stable permutation.
 * topk_idx [T,k] with values in [0,N).  Outputs (all required): counts [N]
 * (pre-drop), offsets [N+1] (exclusive scan of kept counts), slot [T*k],
 * perm [T*k], n_kept_dropped [2] = {R, T*k - R}.  No permuted copy of x is
 * written: the gate/up projection gathers its rows through perm.
 * Source: "MoE architecture in practice", capacity-factor section (the
 * earliest assignments keep their slots, overflow is dropped) and
 * expert-parallelism section (token-major flatten, stable grouping by
 * expert into contiguous segments); llm-compass "MoE" page, capacity
 * formula. */
moe_status moe_dispatch(const moe_shape* shape, const int32_t* topk_idx,
                        int32_t* counts, int32_t* offsets, int32_t* slot,
                        int32_t* perm, int32_t* n_kept_dropped, void* ws,
                        size_t ws_bytes, void* stream);

/* Work lists of the two expert projections for the segments in `offsets`
 * (from moe_dispatch), written to the workspace: each expert segment is cut
 * into near-equal row blocks, each row block into weight-column tiles, and
 * the list into eight ranges of equal estimated cost, one per XCD.  The
 * moe_expert_* calls build these lists themselves when given offsets; given
 * offsets = NULL they reuse the lists already in `ws`, which must then come
 * from an earlier moe_expert_plan or moe_expert_* call with the same shape,
 * workspace and segments, ordered before it on the stream. */
moe_status moe_expert_plan(const moe_shape* shape, const int32_t* offsets,
                           void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs over the dispatched rows (one grouped launch per projection).
 * x [T,d]; perm, offsets from moe_dispatch (offsets NULL: reuse the work
 * lists in ws, see moe_expert_plan); w1, w2 routed weights;
 * w1_shared/w2_shared required iff d_ff_shared > 0.  Outputs: y_perm
 * [T*k, d] dtype, row s = E_e(x_t) for the kept assignment perm[s]
 * (rows >= R untouched); y_shared [T,d] dtype = S(x_t) (required iff
 * d_ff_shared > 0). */
moe_status moe_expert_ffn(const moe_shape* shape, const void* x,
                          const int32_t* perm, const int32_t* offsets,
                          const void* w1, const void* w2,
                          const void* w1_shared, const void* w2_shared,
                          void* y_perm, void* y_shared, void* ws,
                          size_t ws_bytes, void* stream);

/* The two projections of moe_expert_ffn as separate calls (same kernels).
 * gate_up: h[s] = silu(x_t W_gate,e^T) * (x_t W_up,e^T) for every kept row s
 * (t = perm[s] / k, e its expert), h [T*k, d_ff] dtype (rows >= R untouched),
 * and h_shared [T, d_ff_shared] for the shared expert (required iff
 * d_ff_shared > 0).  down: y_perm[s] = h[s] W2_e^T, y_shared = h_shared
 * W2s^T.  offsets as produced by moe_dispatch, or NULL to reuse the work
 * lists in ws (see moe_expert_plan); all pointers device memory.
 * Source: "MoE architecture in practice", expert-parallelism section (one
 * grouped GEMM over the contiguous expert segments); the SwiGLU expert. */
moe_status moe_expert_gate_up(const moe_shape* shape, const void* x,
                              const int32_t* perm, const int32_t* offsets,
                              const void* w1, const void* w1_shared, void* h,
                              void* h_shared, void* ws, size_t ws_bytes,
                              void* stream);
moe_status moe_expert_down(const moe_shape* shape, const void* h,
                           const void* h_shared, const int32_t* offsets,
                           const void* w2, const void* w2_shared, void* y_perm,
                           void* y_shared, void* ws, size_t ws_bytes,
                           void* stream);

/* Combine: y_t = sum_j [slot_tj >= 0] g_tj y_perm[slot_tj] (+ y_shared_t),
 * fp32 accumulation in ascending j, then the shared term; dropped
 * assignments add nothing.  y_shared NULL when there is no shared expert.
 * Source: llm-compass "MoE" page, output equation y = sum_i g_i E_i(x) and
 * shared-expert equation; "MoE architecture in practice", expert-
 * parallelism section (combine back to token order) and capacity-factor
 * section (a dropped assignment contributes nothing). */
moe_status moe_combine(const moe_shape* shape, const void* y_perm,
                       const void* y_shared, const int32_t* slot,
                       const float* topk_w, void* y, void* stream);

/* Balancing step after a forward: with load_i = counts[i] (pre-drop) and
 * mean load T*k/N,  bias_i <- fl32(bias_i - fl32(step * sign(N*load_i -
 * T*k))), then clamped to [-clamp, clamp] when clamp > 0.  If scores and
 * aux_out are given, aux_out[0] = N * sum_i (counts_i / T) * mean_t s_ti
 * (computed before the bias changes; it does not depend on the bias).
 * counts, scores [T,N], bias [N], aux_out [1]: device pointers; counts and
 * bias required, step finite.  ws holds the per-expert score means.
 * Source: "MoE architecture in practice", load-balancing-loss section (the
 * selection-only bias moved by a sign step against the mean load, and the
 * N sum f_i P_i statistic); llm-compass "MoE" page, aux-loss and
 * aux-loss-free equations. */
moe_status moe_bias_update(const moe_shape* shape, const int32_t* counts,
                           const float* scores, float step, float clamp,
                           float* bias, float* aux_out, void* ws,
                           size_t ws_bytes, void* stream);

/* Router telemetry: the indicators that "MoE architecture in practice"
 * (section on scale drift between experts, and its implementation
 * checklist) and the "MoE landscape" page (first-class training indicators)
 * name, from what one forward produced.  All reductions in fp64, fixed
 * order (bitwise reproducible).
 *   counts [N] (pre-drop), offsets [N+1] from moe_dispatch; topk_w [T,k];
 *   scores [T,N] (NULL: score entropy 0); bias [N] (NULL: norms 0);
 *   y_perm [T*k, d] dtype from the expert FFNs (NULL: output moments 0);
 *   y_shared [T, d] (NULL, or given iff d_ff_shared > 0).
 * Output `stats`: moe_router_stats_count(shape) = 16 + 8*(N+1) doubles,
 * device memory, 8-byte aligned:
 *   [0] T  [1] T*k  [2] dropped assignments  [3] dropped / (T*k)
 *   [4] usage CV = population std / mean of counts  [5] experts with count 0
 *   [6] ||bias||_2  [7] max |bias|  [8] mean over tokens of the entropy of
 *   its k gates (normalised to sum 1)  [9] mean entropy of its N scores
 *   (normalised to sum 1)  [10..15] 0
 *   then per expert e = 0..N-1 and e = N (the shared expert; zeros without
 *   one), 8 doubles: load, kept, dropped, dropped/load (0 if load is 0),
 *   mean, population std, max and max |.| of the expert's output rows
 *   (y_perm rows [offsets[e], offsets[e+1]); all d columns; zeros if empty). */
size_t moe_router_stats_count(const moe_shape* shape);
moe_status moe_router_stats(const moe_shape* shape, const int32_t* counts,
                            const int32_t* offsets, const float* topk_w,
                            const float* scores, const float* bias,
                            const void* y_perm, const void* y_shared,
                            double* stats, void* ws, size_t ws_bytes,
                            void* stream);

/* Per-sequence balancing step ("MoE architecture in practice", section
 * "load-balancing loss": update_bias averages loads over sequences so that
 * long sequences do not dominate).  The batch holds n_seq sequences of
 * tokens [seq_offsets[s], seq_offsets[s+1]) (device int32 [n_seq+1],
 * seq_offsets[0] = 0, strictly increasing, seq_offsets[n_seq] = T).  With
 * c_si the pre-drop count of expert i among sequence s's k*L_s assignments:
 *   score_i = (sum_s c_si / (k L_s)) / n_seq,  mean = sum_i score_i / N,
 *   bias_i <- fl32(bias_i + step * sign(mean - score_i)), then clamped to
 *   [-clamp, clamp] when clamp > 0.
 * The sums are fp64, one IEEE operation at a time in s then i order.
 * topk_idx [T,k] from moe_route.  If the device offsets are malformed the
 * bias is left unchanged and *err_out (optional, device int32) is set to 1,
 * else 0.  1 <= n_seq <= T, step finite. */
moe_status moe_bias_update_seq(const moe_shape* shape, const int32_t* topk_idx,
                               const int32_t* seq_offsets, int32_t n_seq,
                               float step, float clamp, float* bias,
                               int32_t* err_out, void* ws, size_t ws_bytes,
                               void* stream);

/* Expert-choice routing ("MoE architecture in practice", routing-math
 * section: each expert takes the top-C tokens its capacity allows, perfectly
 * balanced, no overflow, not causal; "MoE landscape" page).  Scores as in
 * token choice (score_fn; logit_add), then every expert e takes the
 * Cp = min(C, T) tokens with the largest s[t, e] -- ties to the lower token,
 * NaN lowest, -0 == +0 -- where C = moe_capacity(shape) (capacity_factor > 0
 * required).  The raw score is the gate; a token no expert took gets only the
 * shared expert.  top_k only sizes the buffers (N*Cp <= T*top_k required,
 * else MOE_ERR_UNSUPPORTED); the selection bias and the group limit do not
 * apply.
 * moe_ec_capacity: Cp, or -1 for an invalid shape or no capacity.
 * moe_route_ec outputs (all required): counts [N] (= Cp each), offsets [N+1]
 *   (e*Cp), perm [T*top_k] (rows [0, N*Cp): t*top_k for the token of the
 *   row, segment by segment, tokens ascending -- the layout moe_expert_ffn
 *   reads), row_of [T, N] int32 (row of the pair, -1 if e did not take t);
 *   scores_out [T, N] optional; scores_in replaces the router (as in
 *   moe_route).
 * moe_combine_ec: y_t = sum over e ascending with row_of[t,e] >= 0 of
 *   scores[t,e] * y_perm[row_of[t,e]] (+ y_shared_t), fp32 accumulation.
 * moe_forward_ec: route_ec -> expert FFNs -> combine_ec on `stream`;
 *   scores_out, offsets, row_of optional outputs. */
int64_t moe_ec_capacity(const moe_shape* shape);
moe_status moe_route_ec(const moe_shape* shape, const void* x,
                        const float* w_router, const float* logit_add,
                        const float* scores_in, float* scores_out,
                        int32_t* counts, int32_t* offsets, int32_t* perm,
                        int32_t* row_of, void* ws, size_t ws_bytes,
                        void* stream);
moe_status moe_combine_ec(const moe_shape* shape, const void* y_perm,
                          const void* y_shared, const int32_t* row_of,
                          const float* scores, void* y, void* stream);
moe_status moe_forward_ec(const moe_shape* shape, const void* x,
                          const float* w_router, const float* logit_add,
                          const void* w1, const void* w2,
                          const void* w1_shared, const void* w2_shared,
                          void* y, float* scores_out, int32_t* offsets,
                          int32_t* row_of, void* ws, size_t ws_bytes,
                          void* stream);

/* The whole layer: route -> dispatch -> expert FFNs -> combine on `stream`.
 * Required: x, w_router, w1, w2, y (and the shared weights iff
 * d_ff_shared > 0).  Optional inputs logit_add, bias; optional outputs
 * (NULL: kept in the workspace only) scores_out [T,N], topk_idx, topk_w
 * [T,k], counts [N], offsets [N+1], slot [T*k], n_kept_dropped [2].  The
 * SwiGLU intermediate h and the expert outputs y_perm, y_shared stay in the
 * workspace.  Source: the layer of the header comment above -- llm-compass
 * "MoE" page (gate and output equations, capacity formula, shared expert);
 * "MoE architecture in practice", routing-math, capacity-factor,
 * shared-expert and expert-parallelism sections. */
moe_status moe_forward(const moe_shape* shape, const void* x,
                       const float* w_router, const float* logit_add,
                       const float* bias, const void* w1, const void* w2,
                       const void* w1_shared, const void* w2_shared, void* y,
                       float* scores_out, int32_t* topk_idx, float* topk_w,
                       int32_t* counts, int32_t* offsets, int32_t* slot,
                       int32_t* n_kept_dropped, void* ws, size_t ws_bytes,
                       void* stream);

/* moe_forward without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, kernels and outputs as
 * moe_forward (bitwise equal results), minus ws / ws_bytes: the scratch the
 * layer needs (moe_workspace_bytes(shape) bytes) comes from a static device
 * array of MOE_NOALLOC_SCRATCH_BYTES (64 MiB) that the library holds on every
 * GPU it runs on until the process ends -- enough for decode-sized layers
 * (e.g. 64 tokens, d_model 2048, 128 experts top-8, d_ff 768 takes about
 * 5 MiB).  The call allocates nothing and never synchronises; its first
 * call on a device looks up that device's array once (with the device
 * current).  Every call on one GPU shares the array and leaves the last
 * call's contents in it: calls that overlap in time on one GPU (two
 * streams, or two host threads) race and give undefined results; calls
 * ordered on one stream are safe.  Errors: those of moe_forward, and
 * MOE_ERR_SCRATCH when moe_workspace_bytes(shape) exceeds the array
 * (checked before anything is enqueued); MOE_ERR_HIP if the array's address
 * cannot be obtained. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_forward_noalloc(const moe_shape* shape, const void* x,
                               const float* w_router, const float* logit_add,
                               const float* bias, const void* w1,
                               const void* w2, const void* w1_shared,
                               const void* w2_shared, void* y, float* scores_out,
                               int32_t* topk_idx, float* topk_w,
                               int32_t* counts, int32_t* offsets, int32_t* slot,
                               int32_t* n_kept_dropped, void* stream);

/* LatentMoE layer forward ("MoE common taste of open models", section 10:
 * the routed-expert path runs in a low-dimensional latent space -- the
 * hidden state is projected down first, and the experts' compute,
 * parameters and payload are paid in the latent width, at the price of an
 * extra down- and up-projection).  Router, selection, gates, capacity and
 * dispatch exactly as moe_forward, on the hidden state x [T, d_model];
 * then z = x W_down^T, the routed experts E_e act on z (w1 [N, 2*d_ff,
 * d_latent], w2 [N, d_latent, d_ff]), y_lat_t = sum_kept g_tj E_j(z_t)
 * (rounded to the activation dtype), and y = y_lat W_up^T + S(x), the
 * shared expert at full width (w1_shared [2*d_ff_shared, d_model],
 * w2_shared [d_model, d_ff_shared]) added before the final rounding.
 * w_down [d_latent, d_model], w_up [d_model, d_latent], activation dtype
 * (MOE_DTYPE_F32 or MOE_DTYPE_BF16; MXFP8 is MOE_ERR_UNSUPPORTED).  d_latent
 * obeys the d_model rules of moe_check_shape.  Optional outputs as in
 * moe_forward.  The workspace is moe_latent_workspace_bytes(shape,
 * d_latent) bytes (0 on an invalid shape or width); it is not
 * interchangeable with a moe_workspace_bytes one. */
size_t moe_latent_workspace_bytes(const moe_shape* shape, int32_t d_latent);
moe_status moe_forward_latent(const moe_shape* shape, int32_t d_latent,
                              const void* x, const float* w_router,
                              const float* logit_add, const float* bias,
                              const void* w_down, const void* w_up,
                              const void* w1, const void* w2,
                              const void* w1_shared, const void* w2_shared,
                              void* y, float* scores_out, int32_t* topk_idx,
                              float* topk_w, int32_t* counts, int32_t* offsets,
                              int32_t* slot, int32_t* n_kept_dropped, void* ws,
                              size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
