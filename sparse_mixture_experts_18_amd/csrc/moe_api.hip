// C ABI entry points: argument validation, workspace layout, launch order.
#include <math.h>

#include <initializer_list>
#include <mutex>

#include "moe_internal.h"

namespace moe {

namespace {

constexpr size_t kAlign = 256;

inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_ERR_INVALID;
  if (s->T < 1 || s->n_experts < 1 || s->top_k < 1 || s->top_k > s->n_experts ||
      s->d_model < 1 || s->d_ff < 1 || s->d_ff_shared < 0)
    return MOE_ERR_INVALID;
  if (s->score_fn != MOE_SCORE_SOFTMAX && s->score_fn != MOE_SCORE_SIGMOID)
    return MOE_ERR_INVALID;
  if (s->dtype != MOE_DTYPE_F32 && s->dtype != MOE_DTYPE_BF16 && s->dtype != MOE_DTYPE_MXFP8)
    return MOE_ERR_INVALID;
  if (s->capacity_rule != MOE_CAP_TOKENS && s->capacity_rule != MOE_CAP_ASSIGNMENTS)
    return MOE_ERR_INVALID;
  if (s->renormalize != 0 && s->renormalize != 1) return MOE_ERR_INVALID;
  if (isnan(s->capacity_factor)) return MOE_ERR_INVALID;
  if (s->n_groups < 1 || s->n_experts % s->n_groups != 0) return MOE_ERR_INVALID;
  if (s->topk_groups < 1 || s->topk_groups > s->n_groups) return MOE_ERR_INVALID;
  if (s->top_k % s->topk_groups != 0) return MOE_ERR_INVALID;
  if (s->top_k / s->topk_groups > s->n_experts / s->n_groups) return MOE_ERR_INVALID;
  if (s->n_experts > 512 || s->top_k > 16 || s->n_groups > 64) return MOE_ERR_UNSUPPORTED;
  // reduction lengths come in whole k-slices of 128 bytes per row
  const int q = s->dtype == MOE_DTYPE_MXFP8 ? 128 : s->dtype == MOE_DTYPE_BF16 ? 64 : 32;
  if (s->d_model % q || s->d_ff % q || s->d_ff_shared % q) return MOE_ERR_UNSUPPORTED;
  const long long A = s->T * (long long)s->top_k;
  long long wmax = s->d_model;
  if (s->d_ff > wmax) wmax = s->d_ff;
  if (s->d_ff_shared > wmax) wmax = s->d_ff_shared;
  if (A * wmax >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (2LL * s->d_ff * s->d_model >= (1LL << 31) ||
      2LL * s->d_ff_shared * s->d_model >= (1LL << 31))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

inline moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// every pointer given (non-NULL) is aligned to `a` bytes: activation and
// weight rows move in 16-byte vectors, the fp32/int32 arrays element-wise
inline bool aligned(uintptr_t a, std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p && (reinterpret_cast<uintptr_t>(p) & (a - 1))) return false;
  return true;
}
inline bool aligned16(std::initializer_list<const void*> ps) { return aligned(16, ps); }
inline bool aligned4(std::initializer_list<const void*> ps) { return aligned(4, ps); }

}  // namespace

int64_t capacity_of(const moe_shape& s) {
  const double cf = (double)s.capacity_factor;
  if (!(cf > 0.0)) return -1;
  const double T = (double)s.T, N = (double)s.n_experts, k = (double)s.top_k;
  if (s.capacity_rule == MOE_CAP_TOKENS) return (int64_t)floor(cf * T / N);
  int64_t c = (int64_t)(k * T / N * cf);
  return c > s.top_k ? c : s.top_k;
}

// Regions of a workspace: routing and dispatch sized by `sr`, the expert
// projections by `se` (the same shape, except in a LatentMoE layer, whose
// experts run at the latent width without the shared expert).
static Workspace layout_regions(const moe_shape& sr, const moe_shape& se, char* base,
                                size_t& off) {
  Workspace w{};
  const size_t T = (size_t)sr.T, N = (size_t)sr.n_experts, k = (size_t)sr.top_k;
  const size_t A = T * k, d = (size_t)sr.d_model, de = (size_t)se.d_model;
  // bytes per activation element (an MXFP8 h takes 1 + 1/32 bytes: fits in 2)
  const size_t es = act_bf16(se) ? 2 : 4;
  const size_t nchunks = (A + kDispatchChunk - 1) / kDispatchChunk;
  plan_caps(se, w.plan1_cap, w.plan2_cap);
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? base + off : nullptr;
    off += align_up(bytes ? bytes : 1);
    return p;
  };
  w.logits = static_cast<float*>(take(T * N * 4));
  w.scores = static_cast<float*>(take(T * N * 4));
  w.topk_idx = static_cast<int32_t*>(take(A * 4));
  w.topk_w = static_cast<float*>(take(A * 4));
  w.counts = static_cast<int32_t*>(take(N * 4));
  w.offsets = static_cast<int32_t*>(take((N + 1) * 4));
  w.slot = static_cast<int32_t*>(take(A * 4));
  w.perm = static_cast<int32_t*>(take(A * 4));
  w.nkd = static_cast<int32_t*>(take(2 * 4));
  w.rank = static_cast<int32_t*>(take(A * 4));
  w.hist = static_cast<int32_t*>(take(nchunks * N * 4));
  w.base = static_cast<int32_t*>(take(nchunks * N * 4));
  w.plan1_hdr = static_cast<int32_t*>(take(32 * 4));
  w.plan1 = static_cast<WorkItem*>(take((size_t)w.plan1_cap * sizeof(WorkItem)));
  w.plan2_hdr = static_cast<int32_t*>(take(32 * 4));
  w.plan2 = static_cast<WorkItem*>(take((size_t)w.plan2_cap * sizeof(WorkItem)));
  w.h = take(A * (size_t)se.d_ff * es);
  w.h_shared = take(T * (size_t)se.d_ff_shared * es);
  w.y_perm = take(A * de * es);
  w.y_shared = take(T * de * es);
  w.pmean = static_cast<double*>(take(N * 8));
  w.wsplit = static_cast<bf16_t*>(take(act_bf16(sr) ? 3 * N * d * 2 : 0));
  w.router_part = static_cast<float*>(take((size_t)router_split_chunks(sr) * T * N * 4));
  w.stats_rows = static_cast<double*>(take((A + T) * 4 * 8));
  w.stats_ent = static_cast<double*>(take(T * 2 * 8));
  w.ec_row = static_cast<int32_t*>(take(T * N * 4));
  w.xq = static_cast<unsigned char*>(
      take(se.dtype == MOE_DTYPE_MXFP8 ? T * de + T * de / kMxBlock : 0));
  return w;
}

Workspace layout_workspace(const moe_shape& s, void* ws) {
  size_t off = 0;
  Workspace w = layout_regions(s, s, static_cast<char*>(ws), off);
  w.total = off;
  return w;
}

moe_shape latent_expert_shape(const moe_shape& s, int d_latent) {
  moe_shape e = s;
  e.d_model = d_latent;
  e.d_ff_shared = 0;
  return e;
}

LatentWorkspace layout_latent(const moe_shape& s, int d_latent, void* ws) {
  LatentWorkspace L{};
  size_t off = 0;
  char* base = static_cast<char*>(ws);
  const moe_shape se = latent_expert_shape(s, d_latent);
  L.w = layout_regions(s, se, base, off);
  auto take = [&](size_t bytes) -> void* {
    void* p = base ? base + off : nullptr;
    off += align_up(bytes ? bytes : 1);
    return p;
  };
  const size_t T = (size_t)s.T, es = act_bf16(s) ? 2 : 4;
  const int fs = s.d_ff_shared;
  L.z = take(T * d_latent * es);
  L.y_lat = take(T * d_latent * es);
  L.h_sh = take(T * (size_t)fs * es);
  L.y_sh = take(T * (size_t)s.d_model * es);
  L.cap_sh1 = fs > 0 ? dense_plan_cap(s, fs, true) : 1;
  L.cap_down = dense_plan_cap(s, d_latent, false);
  L.cap_up = dense_plan_cap(s, s.d_model, false);
  L.hdr_sh1 = static_cast<int32_t*>(take(32 * 4));
  L.plan_sh1 = static_cast<WorkItem*>(take((size_t)L.cap_sh1 * sizeof(WorkItem)));
  L.hdr_down = static_cast<int32_t*>(take(32 * 4));
  L.plan_down = static_cast<WorkItem*>(take((size_t)L.cap_down * sizeof(WorkItem)));
  L.hdr_up = static_cast<int32_t*>(take(32 * 4));
  L.plan_up = static_cast<WorkItem*>(take((size_t)L.cap_up * sizeof(WorkItem)));
  L.total = off;
  return L;
}

}  // namespace moe

using namespace moe;

namespace {
moe_status check_ws(const moe_shape* s, const void* ws, size_t ws_bytes, Workspace& w) {
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % 256) != 0) return MOE_ERR_WORKSPACE;
  w = layout_workspace(*s, const_cast<void*>(ws));
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}
}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID: return "MOE_ERR_INVALID: null required pointer or inconsistent shape";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape outside the kernels' limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: kernel launch failed";
    case MOE_ERR_SCRATCH:
      return "MOE_ERR_SCRATCH: the shape needs more scratch than the static 64 MiB array of "
             "moe_forward_noalloc";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status moe_check_shape(const moe_shape* shape) { return check_shape(shape); }

int64_t moe_capacity(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return -1;
  return capacity_of(*shape);
}

size_t moe_workspace_bytes(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return layout_workspace(*shape, nullptr).total;
}

moe_status moe_quantize_mx(const void* in, int32_t in_dtype, int64_t rows, int64_t cols,
                           void* out, void* stream) {
  if (!in || !out || rows < 1 || cols < kMxBlock || cols % kMxBlock) return MOE_ERR_INVALID;
  if (in_dtype != MOE_DTYPE_F32 && in_dtype != MOE_DTYPE_BF16) return MOE_ERR_INVALID;
  if (!aligned16({in, out})) return MOE_ERR_INVALID;
  if (rows > (int64_t(1) << 40) / cols) return MOE_ERR_UNSUPPORTED;
  unsigned char* codes = static_cast<unsigned char*>(out);
  return hip_status(launch_mx_quantize(in, in_dtype, rows, cols, codes, codes + rows * cols,
                                       static_cast<hipStream_t>(stream)));
}

moe_status moe_route(const moe_shape* shape, const void* x, const float* w_router,
                     const float* logit_add, const float* scores_in, const float* bias,
                     float* logits_out, float* scores_out, int32_t* topk_idx, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!topk_idx || !topk_w) return MOE_ERR_INVALID;
  if (!scores_in && (!x || !w_router)) return MOE_ERR_INVALID;
  if (!aligned16({x, w_router}) ||
      !aligned4({logit_add, scores_in, bias, logits_out, scores_out, topk_idx, topk_w}))
    return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (scores_in)
    return hip_status(launch_topk(*shape, scores_in, 1, nullptr, nullptr, true, bias, scores_out,
                                  topk_idx, topk_w, s));
  float* logits = logits_out ? logits_out : w.logits;
  int np = 1;
  hipError_t e = launch_router_gemm(*shape, x, w_router, logits, w, s, &np);
  if (e != hipSuccess) return MOE_ERR_HIP;
  // a k-split router leaves partial sums; top-k adds them and fills logits_out
  return hip_status(launch_topk(*shape, np > 1 ? w.router_part : logits, np,
                                np > 1 ? logits_out : nullptr, logit_add, false, bias,
                                scores_out, topk_idx, topk_w, s));
}

moe_status moe_dispatch(const moe_shape* shape, const int32_t* topk_idx, int32_t* counts,
                        int32_t* offsets, int32_t* slot, int32_t* perm, int32_t* n_kept_dropped,
                        void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!topk_idx || !counts || !offsets || !slot || !perm || !n_kept_dropped)
    return MOE_ERR_INVALID;
  if (!aligned4({topk_idx, counts, offsets, slot, perm, n_kept_dropped})) return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  return hip_status(launch_dispatch(*shape, topk_idx, counts, offsets, slot, perm,
                                    n_kept_dropped, w, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_plan(const moe_shape* shape, const int32_t* offsets, void* ws,
                           size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!offsets) return MOE_ERR_INVALID;
  if (!aligned4({offsets})) return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  return hip_status(launch_plan(*shape, offsets, w, static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_ffn(const moe_shape* shape, const void* x, const int32_t* perm,
                          const int32_t* offsets, const void* w1, const void* w2,
                          const void* w1_shared, const void* w2_shared, void* y_perm,
                          void* y_shared, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !perm || !w1 || !w2 || !y_perm) return MOE_ERR_INVALID;
  if (shape->d_ff_shared > 0 && (!w1_shared || !w2_shared || !y_shared)) return MOE_ERR_INVALID;
  if (!aligned16({x, w1, w2, w1_shared, w2_shared, y_perm, y_shared}) ||
      !aligned4({perm, offsets}))
    return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool sh = shape->d_ff_shared > 0;
  if (offsets && launch_plan(*shape, offsets, w, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_gemm1(*shape, x, perm, w1, w1_shared, w.h, w.h_shared, w, s) != hipSuccess)
    return MOE_ERR_HIP;
  return hip_status(launch_gemm2(*shape, w.h, w.h_shared, w2, w2_shared, y_perm,
                                 sh ? y_shared : nullptr, w, s));
}

moe_status moe_expert_gate_up(const moe_shape* shape, const void* x, const int32_t* perm,
                              const int32_t* offsets, const void* w1, const void* w1_shared,
                              void* h, void* h_shared, void* ws, size_t ws_bytes,
                              void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !perm || !w1 || !h) return MOE_ERR_INVALID;
  if (shape->d_ff_shared > 0 && (!w1_shared || !h_shared)) return MOE_ERR_INVALID;
  if (!aligned16({x, w1, w1_shared, h, h_shared}) || !aligned4({perm, offsets}))
    return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (offsets && launch_plan(*shape, offsets, w, s) != hipSuccess) return MOE_ERR_HIP;
  return hip_status(launch_gemm1(*shape, x, perm, w1, w1_shared, h,
                                 shape->d_ff_shared > 0 ? h_shared : nullptr, w, s));
}

moe_status moe_expert_down(const moe_shape* shape, const void* h, const void* h_shared,
                           const int32_t* offsets, const void* w2, const void* w2_shared,
                           void* y_perm, void* y_shared, void* ws, size_t ws_bytes,
                           void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!h || !w2 || !y_perm) return MOE_ERR_INVALID;
  if (shape->d_ff_shared > 0 && (!h_shared || !w2_shared || !y_shared)) return MOE_ERR_INVALID;
  if (!aligned16({h, h_shared, w2, w2_shared, y_perm, y_shared}) || !aligned4({offsets}))
    return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (offsets && launch_plan(*shape, offsets, w, s) != hipSuccess) return MOE_ERR_HIP;
  const bool sh = shape->d_ff_shared > 0;
  return hip_status(launch_gemm2(*shape, h, sh ? h_shared : nullptr, w2, w2_shared, y_perm,
                                 sh ? y_shared : nullptr, w, s));
}

moe_status moe_combine(const moe_shape* shape, const void* y_perm, const void* y_shared,
                       const int32_t* slot, const float* topk_w, void* y, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!y_perm || !slot || !topk_w || !y) return MOE_ERR_INVALID;
  if (shape->d_ff_shared > 0 && !y_shared) return MOE_ERR_INVALID;
  if (!aligned16({y_perm, y_shared, y}) || !aligned4({slot, topk_w})) return MOE_ERR_INVALID;
  return hip_status(launch_combine(*shape, y_perm, shape->d_ff_shared > 0 ? y_shared : nullptr,
                                   slot, topk_w, y, static_cast<hipStream_t>(stream)));
}

moe_status moe_bias_update(const moe_shape* shape, const int32_t* counts, const float* scores,
                           float step, float clamp, float* bias, float* aux_out, void* ws,
                           size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!counts || !bias || !isfinite(step) || isnan(clamp)) return MOE_ERR_INVALID;
  if (!aligned4({counts, scores, bias, aux_out})) return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  return hip_status(launch_bias_update(*shape, counts, scores, step, clamp, bias, aux_out,
                                       w.pmean, static_cast<hipStream_t>(stream)));
}

size_t moe_router_stats_count(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return 0;
  return (size_t)kStatsGlobal + (size_t)kStatsPerExpert * (shape->n_experts + 1);
}

moe_status moe_router_stats(const moe_shape* shape, const int32_t* counts,
                            const int32_t* offsets, const float* topk_w, const float* scores,
                            const float* bias, const void* y_perm, const void* y_shared,
                            double* stats, void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!counts || !offsets || !topk_w || !stats) return MOE_ERR_INVALID;
  if (y_shared && shape->d_ff_shared == 0) return MOE_ERR_INVALID;
  if (!aligned16({y_perm, y_shared}) || !aligned4({counts, offsets, topk_w, scores, bias}) ||
      !aligned(8, {stats}))
    return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  return hip_status(launch_router_stats(*shape, counts, offsets, topk_w, scores, bias, y_perm,
                                        y_shared, stats, w, static_cast<hipStream_t>(stream)));
}

moe_status moe_bias_update_seq(const moe_shape* shape, const int32_t* topk_idx,
                               const int32_t* seq_offsets, int32_t n_seq, float step,
                               float clamp, float* bias, int32_t* err_out, void* ws,
                               size_t ws_bytes, void* stream) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!topk_idx || !seq_offsets || !bias || !isfinite(step) || isnan(clamp))
    return MOE_ERR_INVALID;
  if (n_seq < 1 || n_seq > shape->T) return MOE_ERR_INVALID;
  if (!aligned4({topk_idx, seq_offsets, bias, err_out})) return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  return hip_status(launch_bias_update_seq(*shape, topk_idx, seq_offsets, n_seq, step, clamp,
                                           bias, err_out, w, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {
// expert choice needs a capacity, and its N*min(C,T) rows must fit the T*k
// rows the buffers hold
moe_status check_ec(const moe_shape* shape) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  const int64_t Cp = ec_capacity(*shape);
  if (Cp <= 0) return MOE_ERR_INVALID;
  if (Cp * shape->n_experts > shape->T * (int64_t)shape->top_k) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// scores of every (token, expert) pair: the token-choice scores, without a
// selection (a top-1 pass whose picks are discarded)
hipError_t ec_scores(const moe_shape& sh, const void* x, const float* w_router,
                     const float* logit_add, float* scores, const Workspace& w, hipStream_t s) {
  moe_shape s1 = sh;
  s1.top_k = 1;
  s1.n_groups = 1;
  s1.topk_groups = 1;
  s1.renormalize = 1;
  int np = 1;
  hipError_t e = launch_router_gemm(s1, x, w_router, w.logits, w, s, &np);
  if (e != hipSuccess) return e;
  return launch_topk(s1, np > 1 ? w.router_part : w.logits, np, nullptr, logit_add, false,
                     nullptr, scores, w.topk_idx, w.topk_w, s);
}
}  // namespace

extern "C" {

int64_t moe_ec_capacity(const moe_shape* shape) {
  if (check_shape(shape) != MOE_OK) return -1;
  return ec_capacity(*shape);
}

moe_status moe_route_ec(const moe_shape* shape, const void* x, const float* w_router,
                        const float* logit_add, const float* scores_in, float* scores_out,
                        int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* row_of,
                        void* ws, size_t ws_bytes, void* stream) {
  moe_status st = check_ec(shape);
  if (st != MOE_OK) return st;
  if (!counts || !offsets || !perm || !row_of) return MOE_ERR_INVALID;
  if (!scores_in && (!x || !w_router)) return MOE_ERR_INVALID;
  if (!aligned16({x, w_router}) ||
      !aligned4({logit_add, scores_in, scores_out, counts, offsets, perm, row_of}))
    return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float* sc = scores_in;
  if (!sc) {
    float* so = scores_out ? scores_out : w.scores;
    if (ec_scores(*shape, x, w_router, logit_add, so, w, s) != hipSuccess) return MOE_ERR_HIP;
    sc = so;
  }
  return hip_status(launch_ec_select(*shape, sc, counts, offsets, perm, row_of, w, s));
}

moe_status moe_combine_ec(const moe_shape* shape, const void* y_perm, const void* y_shared,
                          const int32_t* row_of, const float* scores, void* y, void* stream) {
  moe_status st = check_ec(shape);
  if (st != MOE_OK) return st;
  if (!y_perm || !row_of || !scores || !y) return MOE_ERR_INVALID;
  if (shape->d_ff_shared > 0 && !y_shared) return MOE_ERR_INVALID;
  if (!aligned16({y_perm, y_shared, y}) || !aligned4({row_of, scores})) return MOE_ERR_INVALID;
  return hip_status(launch_ec_combine(*shape, y_perm, shape->d_ff_shared > 0 ? y_shared : nullptr,
                                      row_of, scores, y, static_cast<hipStream_t>(stream)));
}

moe_status moe_forward_ec(const moe_shape* shape, const void* x, const float* w_router,
                          const float* logit_add, const void* w1, const void* w2,
                          const void* w1_shared, const void* w2_shared, void* y,
                          float* scores_out, int32_t* offsets, int32_t* row_of, void* ws,
                          size_t ws_bytes, void* stream) {
  moe_status st = check_ec(shape);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !w1 || !w2 || !y) return MOE_ERR_INVALID;
  if (shape->d_ff_shared > 0 && (!w1_shared || !w2_shared)) return MOE_ERR_INVALID;
  if (!aligned16({x, w_router, w1, w2, w1_shared, w2_shared, y}) ||
      !aligned4({logit_add, scores_out, offsets, row_of}))
    return MOE_ERR_INVALID;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe_shape& sh = *shape;
  float* sc = scores_out ? scores_out : w.scores;
  int32_t* of = offsets ? offsets : w.offsets;
  int32_t* ro = row_of ? row_of : w.ec_row;
  const bool shared = sh.d_ff_shared > 0;
  if (ec_scores(sh, x, w_router, logit_add, sc, w, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_ec_select(sh, sc, w.counts, of, w.perm, ro, w, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_plan(sh, of, w, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_gemm1(sh, x, w.perm, w1, w1_shared, w.h, w.h_shared, w, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (launch_gemm2(sh, w.h, w.h_shared, w2, w2_shared, w.y_perm, shared ? w.y_shared : nullptr,
                   w, s) != hipSuccess)
    return MOE_ERR_HIP;
  return hip_status(launch_ec_combine(sh, w.y_perm, shared ? w.y_shared : nullptr, ro, sc, y, s));
}

}  // extern "C"

// ---- the layer forward (moe_forward and moe_forward_noalloc) ----
namespace {
moe_status check_forward_args(const moe_shape* shape, const void* x, const float* w_router,
                              const float* logit_add, const float* bias, const void* w1,
                              const void* w2, const void* w1_shared, const void* w2_shared,
                              void* y, float* scores_out, int32_t* topk_idx, float* topk_w,
                              int32_t* counts, int32_t* offsets, int32_t* slot,
                              int32_t* n_kept_dropped) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !w1 || !w2 || !y) return MOE_ERR_INVALID;
  if (shape->d_ff_shared > 0 && (!w1_shared || !w2_shared)) return MOE_ERR_INVALID;
  if (!aligned16({x, w_router, w1, w2, w1_shared, w2_shared, y}) ||
      !aligned4({logit_add, bias, scores_out, topk_idx, topk_w, counts, offsets, slot,
                 n_kept_dropped}))
    return MOE_ERR_INVALID;
  return MOE_OK;
}

moe_status run_forward(const moe_shape& sh, const void* x, const float* w_router,
                       const float* logit_add, const float* bias, const void* w1,
                       const void* w2, const void* w1_shared, const void* w2_shared, void* y,
                       float* scores_out, int32_t* topk_idx, float* topk_w, int32_t* counts,
                       int32_t* offsets, int32_t* slot, int32_t* n_kept_dropped,
                       const Workspace& w, hipStream_t s) {
  float* sc = scores_out ? scores_out : w.scores;
  int32_t* ti = topk_idx ? topk_idx : w.topk_idx;
  float* tw = topk_w ? topk_w : w.topk_w;
  int32_t* cn = counts ? counts : w.counts;
  int32_t* of = offsets ? offsets : w.offsets;
  int32_t* sl = slot ? slot : w.slot;
  int32_t* nk = n_kept_dropped ? n_kept_dropped : w.nkd;
  const bool shared = sh.d_ff_shared > 0;
  int np = 1;
  if (launch_router_gemm(sh, x, w_router, w.logits, w, s, &np) != hipSuccess) return MOE_ERR_HIP;
  if (launch_topk(sh, np > 1 ? w.router_part : w.logits, np, nullptr, logit_add, false, bias, sc,
                  ti, tw, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (launch_dispatch(sh, ti, cn, of, sl, w.perm, nk, w, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_plan(sh, of, w, s) != hipSuccess) return MOE_ERR_HIP;
  if (launch_gemm1(sh, x, w.perm, w1, w1_shared, w.h, w.h_shared, w, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (launch_gemm2(sh, w.h, w.h_shared, w2, w2_shared, w.y_perm,
                   shared ? w.y_shared : nullptr, w, s) != hipSuccess)
    return MOE_ERR_HIP;
  return hip_status(
      launch_combine(sh, w.y_perm, shared ? w.y_shared : nullptr, sl, tw, y, s));
}


// The allocation-free forward's scratch: one static device array.  In host
// code `noalloc_scratch_array` names a host-side stand-in, never a device
// address: its device address is looked up once per device, with that device
// current, and only that address is handed to kernels.
constexpr size_t kNoallocScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char noalloc_scratch_array[kNoallocScratchBytes];

hipError_t noalloc_scratch(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch_array));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255)) return hipErrorInvalidValue;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

moe_status moe_forward(const moe_shape* shape, const void* x, const float* w_router,
                       const float* logit_add, const float* bias, const void* w1,
                       const void* w2, const void* w1_shared, const void* w2_shared, void* y,
                       float* scores_out, int32_t* topk_idx, float* topk_w, int32_t* counts,
                       int32_t* offsets, int32_t* slot, int32_t* n_kept_dropped, void* ws,
                       size_t ws_bytes, void* stream) {
  moe_status st = check_forward_args(shape, x, w_router, logit_add, bias, w1, w2, w1_shared,
                                     w2_shared, y, scores_out, topk_idx, topk_w, counts,
                                     offsets, slot, n_kept_dropped);
  if (st != MOE_OK) return st;
  Workspace w;
  if ((st = check_ws(shape, ws, ws_bytes, w)) != MOE_OK) return st;
  return run_forward(*shape, x, w_router, logit_add, bias, w1, w2, w1_shared, w2_shared, y,
                     scores_out, topk_idx, topk_w, counts, offsets, slot, n_kept_dropped, w,
                     static_cast<hipStream_t>(stream));
}

moe_status moe_forward_noalloc(const moe_shape* shape, const void* x, const float* w_router,
                               const float* logit_add, const float* bias, const void* w1,
                               const void* w2, const void* w1_shared, const void* w2_shared,
                               void* y, float* scores_out, int32_t* topk_idx, float* topk_w,
                               int32_t* counts, int32_t* offsets, int32_t* slot,
                               int32_t* n_kept_dropped, void* stream) {
  moe_status st = check_forward_args(shape, x, w_router, logit_add, bias, w1, w2, w1_shared,
                                     w2_shared, y, scores_out, topk_idx, topk_w, counts,
                                     offsets, slot, n_kept_dropped);
  if (st != MOE_OK) return st;
  if (layout_workspace(*shape, nullptr).total > kNoallocScratchBytes) return MOE_ERR_SCRATCH;
  void* base = nullptr;
  if (noalloc_scratch(&base) != hipSuccess) return MOE_ERR_HIP;
  const Workspace w = layout_workspace(*shape, base);
  return run_forward(*shape, x, w_router, logit_add, bias, w1, w2, w1_shared, w2_shared, y,
                     scores_out, topk_idx, topk_w, counts, offsets, slot, n_kept_dropped, w,
                     static_cast<hipStream_t>(stream));
}

}  // extern "C"

// ---- LatentMoE ----

namespace {
moe_status check_latent(const moe_shape* shape, int32_t d_latent) {
  moe_status st = check_shape(shape);
  if (st != MOE_OK) return st;
  if (d_latent < 1) return MOE_ERR_INVALID;
  if (shape->dtype == MOE_DTYPE_MXFP8) return MOE_ERR_UNSUPPORTED;
  const moe_shape se = latent_expert_shape(*shape, d_latent);
  return check_shape(&se);
}
}  // namespace

extern "C" {

size_t moe_latent_workspace_bytes(const moe_shape* shape, int32_t d_latent) {
  if (check_latent(shape, d_latent) != MOE_OK) return 0;
  return layout_latent(*shape, d_latent, nullptr).total;
}

moe_status moe_forward_latent(const moe_shape* shape, int32_t d_latent, const void* x,
                              const float* w_router, const float* logit_add, const float* bias,
                              const void* w_down, const void* w_up, const void* w1,
                              const void* w2, const void* w1_shared, const void* w2_shared,
                              void* y, float* scores_out, int32_t* topk_idx, float* topk_w,
                              int32_t* counts, int32_t* offsets, int32_t* slot,
                              int32_t* n_kept_dropped, void* ws, size_t ws_bytes,
                              void* stream) {
  moe_status st = check_latent(shape, d_latent);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !w_down || !w_up || !w1 || !w2 || !y) return MOE_ERR_INVALID;
  if (shape->d_ff_shared > 0 && (!w1_shared || !w2_shared)) return MOE_ERR_INVALID;
  if (!aligned16({x, w_router, w_down, w_up, w1, w2, w1_shared, w2_shared, y}) ||
      !aligned4({logit_add, bias, scores_out, topk_idx, topk_w, counts, offsets, slot,
                 n_kept_dropped}))
    return MOE_ERR_INVALID;
  if (!ws || (reinterpret_cast<uintptr_t>(ws) % 256) != 0) return MOE_ERR_WORKSPACE;
  const LatentWorkspace L = layout_latent(*shape, d_latent, ws);
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  const Workspace& w = L.w;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const moe_shape& sh = *shape;
  const moe_shape se = latent_expert_shape(sh, d_latent);
  const int d = sh.d_model, l = d_latent, fs = sh.d_ff_shared;
  const bool shared = fs > 0;
  float* sc = scores_out ? scores_out : w.scores;
  int32_t* ti = topk_idx ? topk_idx : w.topk_idx;
  float* tw = topk_w ? topk_w : w.topk_w;
  int32_t* cn = counts ? counts : w.counts;
  int32_t* of = offsets ? offsets : w.offsets;
  int32_t* sl = slot ? slot : w.slot;
  int32_t* nk = n_kept_dropped ? n_kept_dropped : w.nkd;
  // routing and dispatch on the hidden state
  int np = 1;
  if (launch_router_gemm(sh, x, w_router, w.logits, w, s, &np) != hipSuccess) return MOE_ERR_HIP;
  if (launch_topk(sh, np > 1 ? w.router_part : w.logits, np, nullptr, logit_add, false, bias, sc,
                  ti, tw, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (launch_dispatch(sh, ti, cn, of, sl, w.perm, nk, w, s) != hipSuccess) return MOE_ERR_HIP;
  // work lists: the experts at the latent width, the dense products over T rows
  if (launch_plan(se, of, w, s) != hipSuccess) return MOE_ERR_HIP;
  hipError_t e = shared ? launch_dense_plan(sh, true, d, fs, L.plan_sh1, L.hdr_sh1, d, l,
                                            L.plan_down, L.hdr_down, s)
                        : launch_dense_plan(sh, false, d, l, L.plan_down, L.hdr_down, 0, 0,
                                            nullptr, nullptr, s);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (launch_dense_plan(sh, false, l, d, L.plan_up, L.hdr_up, 0, 0, nullptr, nullptr, s) !=
      hipSuccess)
    return MOE_ERR_HIP;
  // z = x W_down^T; the routed experts on z; their gated sum at the latent width
  if (launch_dense(sh, false, x, w_down, L.z, nullptr, d, l, L.plan_down, L.hdr_down,
                   L.cap_down, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (launch_gemm1(se, L.z, w.perm, w1, nullptr, w.h, nullptr, w, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (launch_gemm2(se, w.h, nullptr, w2, nullptr, w.y_perm, nullptr, w, s) != hipSuccess)
    return MOE_ERR_HIP;
  if (launch_combine(se, w.y_perm, nullptr, sl, tw, L.y_lat, s) != hipSuccess) return MOE_ERR_HIP;
  // the shared expert at full width, then y = y_lat W_up^T + shared
  if (shared) {
    if (launch_dense(sh, true, x, w1_shared, L.h_sh, nullptr, d, fs, L.plan_sh1, L.hdr_sh1,
                     L.cap_sh1, s) != hipSuccess)
      return MOE_ERR_HIP;
    if (launch_dense(sh, false, L.h_sh, w2_shared, L.y_sh, nullptr, fs, d, L.plan_up, L.hdr_up,
                     L.cap_up, s) != hipSuccess)
      return MOE_ERR_HIP;
  }
  return hip_status(launch_dense(sh, false, L.y_lat, w_up, y, shared ? L.y_sh : nullptr, l, d,
                                 L.plan_up, L.hdr_up, L.cap_up, s));
}

}  // extern "C"
