"""fp64 CPU oracle for the sparse MoE FFN layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use it.  It is deliberately plain and slow: NumPy in
float64, explicit rank counting and running counters instead of sorts, one
expert at a time.  It shares no code, table or helper with the HIP library.

What is computed, and the passage each step follows (page titles as printed
in the sources):

  [RM]  "MoE architecture in practice" (deepseekmodel.com blog), section
        "routing math: softmax, top-k and the small must-do steps" -- the
        TopKRouter: bias-free gate, additive jitter, softmax, top-k,
        renormalisation, capacity from the expected load, earliest-arrival
        keep rule.
  [LB]  same article, section "load-balancing loss" -- the f_i * P_i
        statistic and the BiasBalancedRouter (bias used for the choice
        only; sign update of the bias).
  [SE]  same article, section "shared expert" -- one always-on expert whose
        output is added.
  [EP]  same article, section "expert parallelism and all-to-all" -- flatten
        to [T*k] token-major, stable group-by-expert.
  [G]   llm-compass "MoE" page, section "sparse gating and top-k routing",
        gate equation g = softmax(TopK(x W_g, k)) and y = sum_i g_i E_i(x).
  [AF]  llm-compass "MoE" page, section "load balancing: from aux loss to
        aux-loss-free": T = TopK({s_i + b_i}), g_i proportional to s_i.
  [AUX] llm-compass "MoE" page, same section: L_aux = alpha*N*sum f_i P_i.
  [CAP] llm-compass "MoE" page, section "capacity factor and expert
        parallelism": capacity = capacity_factor * tokens / N, overflow
        dropped.
  [SG]  "MoE common taste of open models", section 7: sigmoid gating, an
        independent score per expert, then top-k and normalisation.
  [NL]  "MoE industrial evolution" (alishangtian.com), section 4
        (DeepSeek route): node-limited routing, each token's experts lie in
        at most M groups.
  [OBS] "MoE architecture in practice", section on scale drift between
        experts (its closing summary of the minimum MoE observability: drop
        ratio, per-expert load, per-expert output scale as mean / std / max,
        bias magnitude, gate entropy) and its implementation checklist (drop
        ratio logged per expert); "MoE landscape" (paper-daily-site topic
        page), TL;DR and recommendations: dead-expert count, usage CV, token
        drop and router bias norm as first-class indicators.
  [EC]  "MoE architecture in practice", routing-math section (expert
        choice routing: each expert takes its top-C tokens by its own
        capacity; perfectly balanced, no overflow, not causal); "MoE
        landscape" page (expert choice folds the capacity constraint into the
        routing).
  [FP8] "MoE common taste of open models", section 2 (FP8/MXFP8 expert
        compute listed as a strong candidate) and its closing recipe table
        (router kept in FP32, or at least protected, when the rest is
        quantised); "MoE architecture in practice", precision section (FP8
        for the forward matrix products with the gate GEMM kept at higher
        precision).  The number format is the one the name refers to: the
        OCP Microscaling Formats (MX) v1.0 specification, MXFP8 = E4M3
        elements sharing one E8M0 power-of-two scale per 32 consecutive
        values.
  [LAT] "MoE common taste of open models", section 10 (LatentMoE): the
        routed-expert path moves into a low-dimensional latent space -- the
        hidden state is first projected down, and the experts' compute,
        parameters and dispatch payload are paid in the latent width; the
        price is an extra down- and up-projection.
  [SEQ] "MoE architecture in practice", section "load-balancing loss"
        (update_bias from per-sequence loads, so that long sequences do not
        dominate), and its long-context section (sequence-level balancing).

Readings taken where the pages are silent or garbled are listed in the
repository's design notes; the ones that change arithmetic are restated at
the function that applies them.  Parity of the group score (sum of the best
k/topk_groups keys of a group) is unpinned by the pages: it is pinned only by
brute-force enumeration in the tests.
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Optional, Sequence, Tuple, Union

import numpy as np

f32 = np.float32

# ---------------------------------------------------------------------------
# router: affinity, scores
# ---------------------------------------------------------------------------


def router_logits(x: np.ndarray, w_router: np.ndarray,
                  logit_add: Optional[np.ndarray] = None) -> np.ndarray:
    """l = x W_g^T (+ additive logit term), fp64.

    [RM]: the gate is a linear layer with no bias; training-time jitter is
    added to the logits (read as l + noise, the noise drawn outside and passed
    in).  [G]: affinity x W_g.  x [T, d], w_router [N, d] -> [T, N].
    """
    l = np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T
    if logit_add is not None:
        l = l + np.asarray(logit_add, np.float64)
    return l


def scores_from_logits(l: np.ndarray, score_fn: str) -> np.ndarray:
    """softmax over the N experts of each token ([RM], [G]) or an
    independent logistic score per expert ([SG]).  fp64."""
    l = np.asarray(l, np.float64)
    if score_fn == "softmax":
        z = l - l.max(axis=1, keepdims=True)
        e = np.exp(z)
        return e / e.sum(axis=1, keepdims=True)
    if score_fn == "sigmoid":
        return 1.0 / (1.0 + np.exp(-l))
    raise ValueError(score_fn)


# ---------------------------------------------------------------------------
# selection
# ---------------------------------------------------------------------------


def selection_keys(s32: np.ndarray, bias: Optional[np.ndarray]) -> np.ndarray:
    """key_i = fl32(s_i + b_i): one IEEE fp32 addition ([AF]; [LB]
    BiasBalancedRouter adds the bias to the scores and selects on the sum).
    Weights never see the bias.  -0 is canonicalised to +0."""
    s32 = np.asarray(s32, f32)
    if bias is None:
        key = s32.copy()
    else:
        key = (s32 + np.asarray(bias, f32)[None, :]).astype(f32)
    key[key == 0] = f32(0.0)
    return key


def _beats(a_val, a_nan, b_val, b_nan):
    """a > b in the total order used for selection: numbers above NaN, NaN
    equal to NaN, otherwise the usual order."""
    return (~a_nan & b_nan) | (~a_nan & ~b_nan & (a_val > b_val))


def _ranks(keys: np.ndarray, cand: Optional[np.ndarray] = None,
           chunk: int = 64) -> np.ndarray:
    """rank_i = #{j candidate : key_j beats key_i, or key_j == key_i and j < i}
    for every candidate i of every row; non-candidates get a rank >= N."""
    T, N = keys.shape
    if cand is None:
        cand = np.ones((T, N), dtype=bool)
    out = np.empty((T, N), dtype=np.int64)
    idx = np.arange(N)
    lower = idx[None, :] < idx[:, None]  # [i, j] : j < i
    for t0 in range(0, T, chunk):
        k = keys[t0:t0 + chunk]
        c = cand[t0:t0 + chunk]
        nan = np.isnan(k)
        v = np.where(nan, 0.0, k).astype(np.float64)
        # [t, i, j]
        gt = _beats(v[:, None, :], nan[:, None, :], v[:, :, None], nan[:, :, None])
        eq = (nan[:, None, :] & nan[:, :, None]) | (
            ~nan[:, None, :] & ~nan[:, :, None] & (v[:, None, :] == v[:, :, None]))
        before = (gt | (eq & lower[None])) & c[:, None, :]
        r = before.sum(axis=2)
        out[t0:t0 + chunk] = np.where(c, r, N + r)
    return out


def group_candidates(keys: np.ndarray, n_groups: int, topk_groups: int,
                     per_group: int) -> np.ndarray:
    """Group-limited routing ([NL]): experts are split into n_groups
    contiguous groups; a group's score is fl32 sum of its best `per_group`
    keys (reading: per_group = k / topk_groups, summed in descending order);
    the topk_groups best groups (ties to the lower group index) stay
    candidates, all other experts are excluded.  Returns bool [T, N]."""
    T, N = keys.shape
    gs = N // n_groups
    gkeys = keys.reshape(T, n_groups, gs)
    gscore = np.empty((T, n_groups), dtype=f32)
    for g in range(n_groups):
        kg = gkeys[:, g, :]
        r = _ranks(kg)
        acc = np.zeros(T, dtype=f32)
        for m in range(per_group):
            pick = kg[np.arange(T), np.argmax(r == m, axis=1)]
            acc = (acc + pick).astype(f32)
        gscore[:, g] = acc
    grank = _ranks(gscore)
    chosen = grank < topk_groups  # [T, G]
    return np.repeat(chosen, gs, axis=1)


def topk_select(keys: np.ndarray, k: int, cand: Optional[np.ndarray] = None
                ) -> np.ndarray:
    """Token-choice top-k ([RM] probs.topk; [G] TopK): expert i is chosen iff
    its rank < k, and sits at column rank_i, i.e. columns in descending key
    order with ties to the lower expert index.  -> int64 [T, k]."""
    T, N = keys.shape
    r = _ranks(keys, cand)
    out = np.full((T, k), -1, dtype=np.int64)
    tt, ii = np.nonzero(r < k)
    out[tt, r[tt, ii]] = ii
    assert (out >= 0).all()
    return out


def gate_weights(s32: np.ndarray, topk_idx: np.ndarray,
                 renormalize: bool) -> np.ndarray:
    """g_tj = s_e / sum_{chosen} s (renormalised, [RM]; [G]; [AF] weights use
    the raw score) or g_tj = s_e.  fp64 from the fp32 scores."""
    s = np.asarray(s32, np.float64)
    g = np.take_along_axis(s, topk_idx, axis=1)
    if renormalize:
        g = g / g.sum(axis=1, keepdims=True)
    return g


# ---------------------------------------------------------------------------
# capacity and dispatch
# ---------------------------------------------------------------------------


def capacity(capacity_factor: float, T: int, N: int, k: int,
             rule: str = "tokens") -> Optional[int]:
    """Per-expert capacity, or None for dropless (capacity_factor <= 0).
    rule "tokens":      floor(cf * T / N)                       [CAP]
    rule "assignments": max(int(cf * k * T / N), k)             [RM]
    cf is taken as the fp32 value the caller passes."""
    cf = float(f32(capacity_factor))
    if cf <= 0:
        return None
    if rule == "tokens":
        return int(math.floor(cf * T / N))
    if rule == "assignments":
        return max(int(k * T / float(N) * cf), k)
    raise ValueError(rule)


def dispatch(topk_idx: np.ndarray, N: int, C: Optional[int]) -> Dict[str, np.ndarray]:
    """Flatten the [T, k] choices token-major into assignment ids a = t*k + j
    ([EP] reshape(-1)), number each expert's assignments in that order (the
    arrival position), keep an assignment iff its position < C ([RM]: the
    earliest arrivals keep the slot, no randomness; [CAP]: overflow dropped),
    and lay the kept ones out expert by expert, ascending a inside a segment
    ([EP] stable group-by-expert).

    Returns counts [N] (pre-drop), kept [N], offsets [N+1], pos [T*k],
    slot [T*k] (-1 = dropped), perm [R] (assignment id per slot), n_dropped.
    """
    flat = topk_idx.reshape(-1)
    A = flat.size
    pos = np.empty(A, dtype=np.int64)
    counts = np.zeros(N, dtype=np.int64)
    for e in range(N):
        where = np.nonzero(flat == e)[0]  # ascending assignment ids
        pos[where] = np.arange(where.size)
        counts[e] = where.size
    kept = counts.copy() if C is None else np.minimum(counts, C)
    offsets = np.zeros(N + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    keep = np.ones(A, dtype=bool) if C is None else pos < C
    slot = np.where(keep, offsets[flat] + pos, -1)
    R = int(offsets[-1])
    perm = np.full(R, -1, dtype=np.int64)
    perm[slot[keep]] = np.nonzero(keep)[0]
    n_dropped = int(A - R)
    return dict(counts=counts, kept=kept, offsets=offsets, pos=pos, slot=slot,
                perm=perm, n_dropped=n_dropped, keep=keep)


# ---------------------------------------------------------------------------
# experts and combine
# ---------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    return z / (1.0 + np.exp(-z))


def swiglu_ffn(x_rows: np.ndarray, w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """E(x) = W2 (silu(W_gate x) * (W_up x)); w1 = [W_gate; W_up] of shape
    [2*d_ff, d] (nn.Linear layout), w2 [d, d_ff].  fp64."""
    x = np.asarray(x_rows, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    f = w1.shape[0] // 2
    a = x @ w1[:f].T
    u = x @ w1[f:].T
    return (silu(a) * u) @ w2.T


# ---------------------------------------------------------------------------
# MXFP8 ([FP8]): E4M3 elements, one E8M0 scale per 32 consecutive values
# ---------------------------------------------------------------------------
MX_BLOCK = 32
E4M3_MAX = 448.0     # 1.75 * 2^8, the largest finite E4M3 magnitude
E4M3_EMAX = 8        # exponent of the largest normal binade


def e4m3_decode(codes) -> np.ndarray:
    """Value of each E4M3 code: sign bit, 4 exponent bits with bias 7, 3
    mantissa bits; exponent field 0 holds subnormals m * 2^-9; the two codes
    with all exponent and mantissa bits set are NaN (there is no infinity)."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where(c & 0x80, -mag, mag)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 code of each value, ties to the even mantissa; magnitudes
    beyond 448 saturate to 448; NaN gives the NaN code; the sign bit is kept
    (so -0 and negative values that round to zero give 0x80)."""
    v = np.asarray(v, np.float64)
    neg = np.signbit(v)
    nan = np.isnan(v)
    a = np.where(nan, 0.0, np.abs(v))
    # binade of a (subnormals share the lowest normal binade, 2^-6): the
    # spacing of E4M3 numbers there is 2^(binade - 3)
    _, e = np.frexp(a)                      # a = m 2^e, m in [0.5, 1)
    b = np.maximum(e - 1, -6)
    q = np.ldexp(np.rint(np.ldexp(a, 3 - b)), b - 3)   # exact scalings, RNE
    q = np.minimum(q, E4M3_MAX)
    # code of the rounded magnitude q (a rounding carry may have moved it up
    # one binade, so its binade is taken again)
    _, e2 = np.frexp(q)
    b2 = e2 - 1
    sub = q < 2.0 ** -6
    mant = np.where(sub, 0.0, np.ldexp(q, -b2) - 1.0) * 8.0
    code = np.where(sub, np.ldexp(q, 9), (b2 + 7) * 8 + mant)
    code = code.astype(np.int64)
    code = np.where(nan, 0x7F, code)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def mx_quantize(v) -> Tuple[np.ndarray, np.ndarray]:
    """MXFP8 quantisation along the last axis (length a multiple of 32), the
    OCP MX v1.0 conversion: each block of 32 gets the shared exponent
    X = floor(log2(max |v|)) - 8 (8 = exponent of the largest E4M3 binade),
    clamped to the E8M0 range [-127, 127]; each element becomes the E4M3
    code of v / 2^X (e4m3_encode: nearest, ties to even, saturating).
    Readings for the cases the definition leaves open: an all-zero block
    takes X = -127; NaN elements do not enter the maximum and give the NaN
    code; a block holding an infinity takes X = 127.  Returns (codes
    [..., K] uint8, scales [..., K/32] uint8 holding X + 127)."""
    v = np.asarray(v, np.float64)
    K = v.shape[-1]
    if K % MX_BLOCK:
        raise ValueError("MX blocks need a multiple of 32 values")
    blk = v.reshape(v.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    a = np.abs(blk)
    amax = np.max(np.where(np.isnan(a), 0.0, a), axis=-1)
    _, e = np.frexp(np.where(np.isfinite(amax), amax, 1.0))
    X = np.where(amax > 0, e - 1 - E4M3_EMAX, -127)
    X = np.where(np.isinf(amax), 127, X)
    X = np.clip(X, -127, 127).astype(np.int64)
    codes = e4m3_encode(np.ldexp(blk, -X[..., None]))
    return codes.reshape(v.shape), (X + 127).astype(np.uint8)


def mx_dequantize(codes, scales) -> np.ndarray:
    """Value of an MXFP8 tensor: code value * 2^(scale - 127), blocks of 32
    along the last axis."""
    c = np.asarray(codes, np.uint8)
    X = np.asarray(scales, np.int64) - 127
    K = c.shape[-1]
    vals = e4m3_decode(c).reshape(c.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    return np.ldexp(vals, X[..., None]).reshape(c.shape)


def mx_round(v) -> np.ndarray:
    """v rounded through MXFP8 (quantise, then dequantise)."""
    return mx_dequantize(*mx_quantize(v))


def swiglu_ffn_mx(x_rows: np.ndarray, w1: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """An MXFP8 expert ([FP8]): both operands of each matrix product are MXFP8
    with blocks along the reduction axis.  The weights arrive already rounded
    through MXFP8 (w1 [2*d_ff, d], w2 [d, d_ff]); the token rows are rounded
    here along d, the SwiGLU intermediate along d_ff; products, SiLU and sums
    in fp64."""
    x = mx_round(np.asarray(x_rows, np.float64))
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    f = w1.shape[0] // 2
    h = silu(x @ w1[:f].T) * (x @ w1[f:].T)
    return mx_round(h) @ w2.T


WeightSource = Union[Tuple[np.ndarray, np.ndarray],
                     Callable[[int], Tuple[np.ndarray, np.ndarray]]]


def _expert_weights(w1, w2, e):
    if callable(w1):
        return w1(e)
    return w1[e], w2[e]


def moe_layer(x: np.ndarray, w_router: np.ndarray, w1, w2, *, top_k: int,
              score_fn: str = "softmax", renormalize: bool = True,
              n_groups: int = 1, topk_groups: int = 1,
              capacity_factor: float = 0.0, capacity_rule: str = "tokens",
              bias: Optional[np.ndarray] = None,
              logit_add: Optional[np.ndarray] = None,
              w1_shared: Optional[np.ndarray] = None,
              w2_shared: Optional[np.ndarray] = None,
              scores_fp32: Optional[np.ndarray] = None,
              tokens: Optional[Sequence[int]] = None,
              compute_outputs: bool = True,
              ffn: Callable = swiglu_ffn) -> Dict[str, np.ndarray]:
    """One MoE FFN layer forward ([G] y = sum_i g_i E_i(x), [SE] plus the
    shared expert).  ``ffn`` is the expert function of the routed and shared
    experts: swiglu_ffn, or swiglu_ffn_mx for MXFP8 experts (with the router
    unchanged: fp32 scores from the unquantised x, [FP8]).

    x [T, d]; w_router [N, d]; w1 [N, 2*d_ff, d] and w2 [N, d, d_ff], or w1 a
    callable e -> (w1_e, w2_e) (w2 ignored) so that weights can be streamed one
    expert at a time.  ``scores_fp32`` replaces the fp32 scores that routing
    starts from (the scores are otherwise fl32 of the fp64 scores).
    ``tokens`` restricts the expert/combine stage to those token rows (routing
    and dispatch always cover all T tokens: capacity drops depend on every
    earlier token).  Dropped assignments contribute 0 ([RM] capacity section:
    the FFN branch output of a dropped token is zero).
    """
    x = np.asarray(x)
    T = x.shape[0]
    N = w_router.shape[0]
    out: Dict[str, np.ndarray] = {}
    if scores_fp32 is None:
        if tokens is not None:
            raise ValueError("routing needs the scores of every token")
        l = router_logits(x, w_router, logit_add)
        s = scores_from_logits(l, score_fn)
        out["logits"] = l
        out["scores"] = s
        s32 = s.astype(f32)
    else:
        s32 = np.asarray(scores_fp32, f32)
    keys = selection_keys(s32, bias)
    cand = None
    if n_groups > 1:
        if top_k % topk_groups:
            raise ValueError("top_k must be a multiple of topk_groups")
        cand = group_candidates(keys, n_groups, topk_groups, top_k // topk_groups)
    idx = topk_select(keys, top_k, cand)
    g = gate_weights(s32, idx, renormalize)
    C = capacity(capacity_factor, T, N, top_k, capacity_rule)
    dsp = dispatch(idx, N, C)
    out.update(topk_idx=idx, topk_w=g, capacity=C, **dsp)
    if not compute_outputs:
        return out

    rows = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    sel = np.zeros(T, dtype=bool)
    sel[rows] = True
    d = x.shape[1]
    y = np.zeros((T, d), dtype=np.float64)
    keep = dsp["keep"].reshape(T, top_k)
    for e in range(N):
        a = np.nonzero((idx.reshape(-1) == e) & dsp["keep"]
                       & np.repeat(sel, top_k))[0]
        if a.size == 0:
            continue
        t = a // top_k
        j = a % top_k
        w1e, w2e = _expert_weights(w1, w2, e)
        o = ffn(x[t], w1e, w2e)
        # accumulate in ascending-j order per token: add the j-th term of each
        # token one j at a time
        for jj in range(top_k):
            m = j == jj
            y[t[m]] += g[t[m], jj][:, None] * o[m]
    if w1_shared is not None:
        y[rows] += ffn(x[rows], w1_shared, w2_shared)
    out["y"] = y[rows]
    out["rows"] = rows
    out["keep2d"] = keep
    return out


# ---------------------------------------------------------------------------
# balancing step
# ---------------------------------------------------------------------------


def aux_statistic(scores: np.ndarray, counts: np.ndarray) -> float:
    """N * sum_i f_i P_i with P_i the mean score of expert i over the T tokens
    and f_i = count_i / T the share of tokens that chose i (pre-drop) ([AUX];
    [LB] load_balance_loss without its extra P^2 term).  Equals 1 for a
    perfectly uniform top-1 routing."""
    s = np.asarray(scores, np.float64)
    T, N = s.shape
    P = s.mean(axis=0)
    f = np.asarray(counts, np.float64) / T
    return float(N * np.sum(f * P))


def bias_update(bias: np.ndarray, counts: np.ndarray, T: int, k: int,
                step: float = 1e-3, clamp: float = 0.0) -> np.ndarray:
    """b_i <- fl32(b_i - fl32(step * sign(load_i - mean load))) with load_i the
    pre-drop count and mean load T*k/N; the sign is taken exactly in integers
    as sign(N*count_i - T*k) ([LB] update_bias: overloaded experts are pushed
    down, underloaded up, by a fixed step; [AF]).  Optional clamp to
    [-clamp, clamp] (clamp <= 0: off)."""
    b = np.asarray(bias, f32)
    N = b.size
    c = np.asarray(counts, np.int64)
    sg = np.sign(N * c - T * k).astype(f32)
    nb = (b - (f32(step) * sg).astype(f32)).astype(f32)
    if clamp > 0:
        nb = np.clip(nb, f32(-clamp), f32(clamp)).astype(f32)
    return nb


# ---------------------------------------------------------------------------
# router telemetry
# ---------------------------------------------------------------------------


def _entropy(p: np.ndarray) -> float:
    """-sum p ln p of a non-negative vector normalised to sum 1 (0 ln 0 = 0)."""
    p = np.asarray(p, np.float64)
    tot = p.sum()
    if not tot > 0:
        return 0.0
    q = p / tot
    nz = q > 0
    return float(-np.sum(q[nz] * np.log(q[nz])))


def router_stats(counts: np.ndarray, offsets: np.ndarray, topk_w: np.ndarray,
                 scores: Optional[np.ndarray], bias: Optional[np.ndarray],
                 y_perm: Optional[np.ndarray], y_shared: Optional[np.ndarray] = None
                 ) -> Dict[str, np.ndarray]:
    """The indicators [OBS] names, from what one forward already produced.

    Global:
      dropped       total dropped assignments, sum_e (load_e - kept_e)
      drop_fraction dropped / (T*k)
      usage_cv      population std / mean of the per-expert loads (pre-drop)
      dead          number of experts no token chose
      bias_norm     ||b||_2;  bias_absmax  max_i |b_i|   (0 without a bias)
      gate_entropy  mean over tokens of -sum_j p ln p, p = the k gates of the
                    token normalised to sum 1
      score_entropy mean over tokens of the entropy of the N scores normalised
                    to sum 1 (0 when no scores are given)
    Per expert e (rows 0..N-1; row N = shared expert when y_shared is given):
      load, kept, dropped, drop_ratio (dropped / load, 0 for an unused expert),
      and the mean, population std, max and max |.| of the expert's output
      rows (y_perm rows of its segment; all d columns), 0 for an empty one.
    """
    c = np.asarray(counts, np.int64)
    off = np.asarray(offsets, np.int64)
    N = c.size
    g = np.asarray(topk_w, np.float64)
    T, k = g.shape
    kept = off[1:] - off[:-1]
    dropped = c - kept
    load = c.astype(np.float64)
    mean = load.mean()
    cv = float(np.sqrt(np.mean((load - mean) ** 2)) / mean) if mean > 0 else 0.0
    glob = dict(dropped=int(dropped.sum()),
                drop_fraction=float(dropped.sum()) / float(T * k),
                usage_cv=cv, dead=int(np.sum(c == 0)))
    if bias is not None:
        b = np.asarray(bias, np.float64)
        glob["bias_norm"] = float(np.sqrt(np.sum(b * b)))
        glob["bias_absmax"] = float(np.max(np.abs(b)))
    else:
        glob["bias_norm"] = glob["bias_absmax"] = 0.0
    glob["gate_entropy"] = float(np.mean([_entropy(g[t]) for t in range(T)]))
    if scores is not None:
        s = np.asarray(scores, np.float64)
        glob["score_entropy"] = float(np.mean([_entropy(s[t]) for t in range(T)]))
    else:
        glob["score_entropy"] = 0.0
    rows = N + (1 if y_shared is not None else 0)
    per = np.zeros((rows, 8))
    per[:N, 0] = c
    per[:N, 1] = kept
    per[:N, 2] = dropped
    per[:N, 3] = np.where(c > 0, dropped / np.maximum(c, 1), 0.0)
    segs = [(int(off[e]), int(off[e + 1])) for e in range(N)]
    for e in range(rows):
        if e < N:
            if y_perm is None:
                continue
            blk = np.asarray(y_perm[segs[e][0]:segs[e][1]], np.float64)
        else:
            blk = np.asarray(y_shared, np.float64)
        if blk.size == 0:
            continue
        per[e, 4] = blk.mean()
        per[e, 5] = blk.std()
        per[e, 6] = blk.max()
        per[e, 7] = np.abs(blk).max()
    if y_shared is not None:
        T_ = np.asarray(y_shared).shape[0]
        per[N, 0] = per[N, 1] = T_
    glob["per_expert"] = per
    return glob


def bias_update_seq(bias: np.ndarray, topk_idx: np.ndarray, seq_lens: Sequence[int],
                    step: float = 1e-3, clamp: float = 0.0) -> np.ndarray:
    """Per-sequence balancing step ([SEQ]).  The article's update averages
    per-sequence loads over the sequences so that long sequences do not
    dominate; its code averages raw counts, which long sequences still
    dominate, so the load of expert i in sequence s is read as its share
    f_si = c_si / (k * L_s) (reading stated in the design notes).  Then
    score_i = sum_s f_si / S, mean = sum_i score_i / N, and
    b_i <- fl32(b_i + fl32(step * sign(mean - score_i))), clamped to
    [-clamp, clamp] when clamp > 0.

    The sign decides an integer, so the sums are taken in fp64 in a fixed
    order (s ascending, then i ascending), one IEEE operation at a time --
    the order the kernel uses."""
    b = np.asarray(bias, f32)
    N = b.size
    idx = np.asarray(topk_idx, np.int64)
    T, k = idx.shape
    L = [int(v) for v in seq_lens]
    assert sum(L) == T and all(v > 0 for v in L)
    S = len(L)
    score = [0.0] * N
    t0 = 0
    for s_ in range(S):
        cnt = [0] * N
        for t in range(t0, t0 + L[s_]):
            for j in range(k):
                cnt[int(idx[t, j])] += 1
        den = float(k * L[s_])
        for i in range(N):
            score[i] = score[i] + cnt[i] / den
        t0 += L[s_]
    for i in range(N):
        score[i] = score[i] / S
    tot = 0.0
    for i in range(N):
        tot = tot + score[i]
    mean = tot / N
    sg = np.array([(mean > score[i]) - (mean < score[i]) for i in range(N)], f32)
    nb = (b + (f32(step) * sg).astype(f32)).astype(f32)
    if clamp > 0:
        nb = np.clip(nb, f32(-clamp), f32(clamp)).astype(f32)
    return nb


# ---------------------------------------------------------------------------
# expert-choice routing
# ---------------------------------------------------------------------------


def expert_choice_select(s32: np.ndarray, C: int) -> np.ndarray:
    """[EC]: every expert e takes the min(C, T) tokens with the largest score
    s[t, e] (ties to the lower token index, NaN lowest, -0 == +0): the same
    total order as token choice, read down an expert's column.  Returns the
    [T, N] boolean choice matrix."""
    key = np.asarray(s32, f32).copy()
    key[key == 0] = f32(0.0)
    T = key.shape[0]
    # [N, T]: rank of t in column e (a few experts per pass: T x T pairs each)
    r = _ranks(np.ascontiguousarray(key.T), chunk=max(1, (1 << 24) // max(T * T, 1)))
    return (r < min(int(C), T)).T


def expert_choice_dispatch(chosen: np.ndarray, k: int) -> Dict[str, np.ndarray]:
    """Segments of the chosen tokens, expert by expert, tokens ascending in a
    segment (the stable grouping of [EP], one row per (token, expert) pair).
    perm holds t*k (the flat assignment id of slot 0 of the token, so the
    expert GEMMs find the token as perm // k); row_of[t, e] is the row of the
    pair or -1."""
    T, N = chosen.shape
    counts = chosen.sum(axis=0).astype(np.int64)
    offsets = np.zeros(N + 1, np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.zeros(int(offsets[-1]), np.int64)
    row_of = np.full((T, N), -1, np.int64)
    for e in range(N):
        r = int(offsets[e])
        for t in range(T):
            if chosen[t, e]:
                perm[r] = t * k
                row_of[t, e] = r
                r += 1
    return dict(counts=counts, offsets=offsets, perm=perm, row_of=row_of)


def moe_layer_ec(x: np.ndarray, w_router: np.ndarray, w1, w2, *, C: int, k: int,
                 score_fn: str = "softmax", logit_add: Optional[np.ndarray] = None,
                 w1_shared: Optional[np.ndarray] = None,
                 w2_shared: Optional[np.ndarray] = None,
                 scores_fp32: Optional[np.ndarray] = None,
                 compute_outputs: bool = True,
                 ffn: Callable = swiglu_ffn,
                 tokens: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """One expert-choice MoE layer forward ([EC]): scores as in token choice,
    each expert takes its top-C tokens, y_t = sum over the experts that took
    t of s[t, e] * E_e(x_t) (the raw score is the gate), plus the shared
    expert; a token no expert took gets only the shared term.  The sum over
    experts runs in ascending e.  ``tokens`` restricts the expert stage to
    those rows (the selection always covers all T tokens); out["y"] then
    holds those rows in the given order."""
    x = np.asarray(x)
    T = x.shape[0]
    N = w_router.shape[0]
    out: Dict[str, np.ndarray] = {}
    if scores_fp32 is None:
        l = router_logits(x, w_router, logit_add)
        s = scores_from_logits(l, score_fn)
        out["scores"] = s
        s32 = s.astype(f32)
    else:
        s32 = np.asarray(scores_fp32, f32)
    chosen = expert_choice_select(s32, C)
    out.update(chosen=chosen, **expert_choice_dispatch(chosen, k))
    if not compute_outputs:
        return out
    d = x.shape[1]
    y = np.zeros((T, d), np.float64)
    sel = np.ones(T, bool) if tokens is None else np.isin(np.arange(T), tokens)
    for e in range(N):
        t = np.nonzero(chosen[:, e] & sel)[0]
        if t.size == 0:
            continue
        w1e, w2e = _expert_weights(w1, w2, e)
        o = ffn(x[t], w1e, w2e)
        y[t] += s32[t, e].astype(np.float64)[:, None] * o
    rows = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    if w1_shared is not None:
        y[rows] += ffn(x[rows], w1_shared, w2_shared)
    out["y"] = y[rows]
    return out


# ---------------------------------------------------------------------------
# LatentMoE ([LAT])
# ---------------------------------------------------------------------------


def moe_layer_latent(x: np.ndarray, w_router: np.ndarray, w_down: np.ndarray,
                     w_up: np.ndarray, w1, w2, *, top_k: int,
                     w1_shared: Optional[np.ndarray] = None,
                     w2_shared: Optional[np.ndarray] = None,
                     scores_fp32: Optional[np.ndarray] = None,
                     tokens: Optional[Sequence[int]] = None,
                     compute_outputs: bool = True, **route_kw) -> Dict[str, np.ndarray]:
    """One LatentMoE layer forward ([LAT]).  The router, the selection and the
    dispatch are those of moe_layer, on the hidden state x [T, d]; the routed
    path runs in the latent width l: z = x W_down^T (W_down [l, d]), the
    experts E_e (w1 [N, 2*d_ff, l], w2 [N, l, d_ff]) act on z, their gated sum
    is formed in the latent space, y_lat = sum_j g_j E_j(z), and projected
    back, y = y_lat W_up^T (W_up [d, l]); the shared expert acts on x at full
    width and is added.  fp64."""
    x = np.asarray(x, np.float64)
    out = moe_layer(x, w_router, w1, w2, top_k=top_k, scores_fp32=scores_fp32,
                    compute_outputs=False, **route_kw)
    if not compute_outputs:
        return out
    s32 = out["scores"].astype(f32) if scores_fp32 is None else np.asarray(scores_fp32, f32)
    z = x @ np.asarray(w_down, np.float64).T
    lat = moe_layer(z, w_router, w1, w2, top_k=top_k, scores_fp32=s32, tokens=tokens,
                    **route_kw)
    rows = lat["rows"]
    y = lat["y"] @ np.asarray(w_up, np.float64).T
    if w1_shared is not None:
        y = y + swiglu_ffn(x[rows], w1_shared, w2_shared)
    out.update(z=z, y_latent=lat["y"], y=y, rows=rows)
    return out

