"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a worked
example printed on the pages, a closed form, an invariant, brute-force
enumeration on tiny inputs, or a textbook routine (scipy / explicit loops).
CPU only.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special

from oracle import moe_ref as R

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
f32 = np.float32


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- router ---

def test_router_logits_explicit_loops():
    r = rng(1)
    x = r.standard_normal((3, 5))
    w = r.standard_normal((4, 5))
    add = r.standard_normal((3, 4))
    l = R.router_logits(x, w, add)
    for t in range(3):
        for i in range(4):
            acc = 0.0
            for c in range(5):
                acc += x[t, c] * w[i, c]
            assert abs(l[t, i] - (acc + add[t, i])) < 1e-12


def test_scores_match_scipy():
    r = rng(2)
    l = r.standard_normal((7, 11)) * 3
    np.testing.assert_allclose(R.scores_from_logits(l, "softmax"),
                               scipy.special.softmax(l, axis=1), rtol=1e-13)
    np.testing.assert_allclose(R.scores_from_logits(l, "sigmoid"),
                               scipy.special.expit(l), rtol=1e-13)
    assert np.allclose(R.scores_from_logits(l, "softmax").sum(1), 1.0)


# ------------------------------------------------------------- selection ---

def _brute_topk_set(key, k, cand=None):
    """The unique k-subset S whose every member beats every non-member
    (higher key, or equal key and lower index), by enumeration."""
    N = len(key)
    idx = [i for i in range(N) if cand is None or cand[i]]

    def beats(i, j):
        return key[i] > key[j] or (key[i] == key[j] and i < j)

    found = [S for S in itertools.combinations(idx, k)
             if all(beats(i, j) for i in S for j in idx if j not in S)]
    assert len(found) == 1
    # order inside: descending key, ties to lower index (library sort)
    return sorted(found[0], key=lambda i: (-key[i], i))


def test_topk_bruteforce_all_pairs():
    r = rng(3)
    # every one of the C(8,2)=28 pairs must come out as the choice of some row
    seen = set()
    for a, b in itertools.combinations(range(8), 2):
        key = r.uniform(0, 0.5, 8).astype(f32)
        key[a], key[b] = f32(0.9), f32(0.7 + 0.1 * r.random())
        got = R.topk_select(key[None, :], 2)[0].tolist()
        assert got == _brute_topk_set(key, 2)
        seen.add(tuple(sorted(got)))
    assert len(seen) == 28


def test_topk_bruteforce_random_and_ties():
    r = rng(4)
    for trial in range(300):
        N = int(r.integers(2, 9))
        k = int(r.integers(1, N + 1))
        # values from a tiny set to force ties
        key = r.choice(np.array([0.0, 0.25, 0.5], f32), N)
        got = R.topk_select(key[None, :], k)[0].tolist()
        assert got == _brute_topk_set(key, k), (key, k)


def test_all_equal_row_picks_lowest_indices():
    key = np.full((2, 16), 0.125, f32)
    assert R.topk_select(key, 5).tolist() == [[0, 1, 2, 3, 4]] * 2


def test_nan_sorts_below_everything_and_negzero_equals_zero():
    key = np.array([[np.nan, -np.inf, -0.0, 0.0, np.nan]], f32)
    key = R.selection_keys(key, None)
    assert R.topk_select(key, 5)[0].tolist() == [2, 3, 1, 0, 4]


def test_group_limited_bruteforce_70_subsets():
    """N=16 experts in 8 groups of 2, keep 4 groups, k=8 (per_group 2 = all
    of a group): the chosen groups must be the unique 4-subset of groups whose
    every member beats every non-member on the group score, among all
    C(8,4)=70 subsets; each subset is reached by some row."""
    r = rng(5)
    seen = set()
    for G in itertools.combinations(range(8), 4):
        key = r.uniform(0, 0.3, 16).astype(f32)
        for g in G:
            key[2 * g: 2 * g + 2] += f32(0.5)
        key = key.astype(f32)
        cand = R.group_candidates(key[None], 8, 4, 2)[0]
        gsc = [float(f32(np.sort(key[2 * g:2 * g + 2])[::-1][0]
                         + np.sort(key[2 * g:2 * g + 2])[::-1][1])) for g in range(8)]
        subsets = [S for S in itertools.combinations(range(8), 4)
                   if all(gsc[a] > gsc[b] or (gsc[a] == gsc[b] and a < b)
                          for a in S for b in range(8) if b not in S)]
        assert len(subsets) == 1
        chosen = tuple(g for g in range(8) if cand[2 * g])
        assert chosen == subsets[0] == G
        idx = R.topk_select(key[None], 8, cand[None])[0].tolist()
        assert idx == _brute_topk_set(key, 8, cand)
        seen.add(chosen)
    assert len(seen) == 70


def test_group_score_uses_best_two_not_best_one():
    # group 0: (0.9, 0.0)  -> 0.9 ; group 1: (0.5, 0.5) -> 1.0 ; keep one group
    key = np.array([[0.9, 0.0, 0.5, 0.5]], f32)
    cand = R.group_candidates(key, 2, 1, 2)
    assert cand[0].tolist() == [False, False, True, True]
    assert R.topk_select(key, 2, cand)[0].tolist() == [2, 3]


def test_group_ties_go_to_lower_group():
    key = np.array([[0.5, 0.25, 0.25, 0.5, 0.75, 0.0]], f32)  # 3 groups of 2
    cand = R.group_candidates(key, 3, 1, 2)  # sums 0.75 0.75 0.75
    assert cand[0].tolist() == [True, True, False, False, False, False]


# ----------------------------------------------------------------- gates ---

def test_worked_example_renormalisation():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "renorm_worked_example.txt"))
            if l.strip() and not l.startswith("#")]
    for p1, p2, g1, g2 in rows:
        s = np.array([[float(p1), 0.01, float(p2), 0.02]], f32)
        idx = R.topk_select(R.selection_keys(s, None), 2)
        assert idx[0].tolist() == [0, 2]
        g = R.gate_weights(s, idx, True)[0]
        assert abs(g[0] - float(g1)) < 1e-7 and abs(g[1] - float(g2)) < 1e-7


def test_gates_sum_to_one():
    r = rng(6)
    s = scipy.special.softmax(r.standard_normal((50, 32)) * 2, axis=1).astype(f32)
    idx = R.topk_select(R.selection_keys(s, None), 6)
    g = R.gate_weights(s, idx, True)
    assert np.abs(g.sum(1) - 1).max() <= 4 * 6 * 2.0 ** -24


def test_softmax_of_topk_logits_equals_renormalised_topk_softmax():
    """llm-compass gate g = softmax(TopK(l)) (non-chosen logits -> -inf) vs
    the article's softmax -> topk -> renormalise."""
    r = rng(7)
    l = r.standard_normal((40, 12)) * 2
    s = R.scores_from_logits(l, "softmax")
    idx = R.topk_select(R.selection_keys(s.astype(f32), None), 3)
    g = R.gate_weights(s, idx, True)
    for t in range(40):
        top = np.argsort(-l[t], kind="stable")[:3]
        masked = np.full(12, -np.inf)
        masked[top] = l[t, top]
        ref = scipy.special.softmax(masked)
        assert sorted(top.tolist()) == sorted(idx[t].tolist())
        np.testing.assert_allclose(g[t], ref[idx[t]], rtol=1e-12)


def test_bias_changes_choice_not_weights():
    r = rng(8)
    s = scipy.special.expit(r.standard_normal((30, 16))).astype(f32)
    b = np.zeros(16, f32)
    b[5] = 10.0
    idx = R.topk_select(R.selection_keys(s, b), 4)
    assert (idx[:, 0] == 5).all()  # +10 forces expert 5 into every token
    g = R.gate_weights(s, idx, True)
    ref = np.take_along_axis(s.astype(np.float64), idx, 1)
    np.testing.assert_allclose(g, ref / ref.sum(1, keepdims=True), rtol=0, atol=0)
    # two biases giving the same choice give identical weights
    idx2 = R.topk_select(R.selection_keys(s, b * 2), 4)
    assert (idx2 == idx).all()
    assert (R.gate_weights(s, idx2, True) == g).all()


def test_selection_key_is_one_fp32_add():
    s = np.array([[1.0, 2.0 ** -24]], f32)
    b = np.array([2.0 ** -24, 1.0], f32)
    k = R.selection_keys(s, b)
    # 1 + 2^-24 rounds to 1 in fp32 (ties-to-even), same for the other
    assert k[0, 0] == f32(1.0) and k[0, 1] == f32(1.0)
    assert R.topk_select(k, 1)[0, 0] == 0


# -------------------------------------------------------------- capacity ---

def test_capacity_closed_forms():
    assert R.capacity(1.25, 64, 8, 2, "tokens") == 10
    assert R.capacity(1.25, 64, 8, 2, "assignments") == 20
    assert R.capacity(1.0, 16384, 64, 1, "tokens") == 256
    assert R.capacity(1.0, 16384, 64, 1, "assignments") == 256
    assert R.capacity(0.01, 10, 8, 2, "assignments") == 2  # floor of k
    assert R.capacity(0.0, 64, 8, 2) is None
    assert R.capacity(-1.0, 64, 8, 2) is None
    assert R.capacity(0.5, 7, 4, 1) == 0  # floor(0.875)


def _brute_pos(flat):
    pos = []
    for a in range(len(flat)):
        c = 0
        for b in range(a):
            if flat[b] == flat[a]:
                c += 1
        pos.append(c)
    return np.array(pos)


def test_dispatch_bruteforce_positions_tiny():
    r = rng(9)
    T, N, k = 64, 8, 2
    s = scipy.special.softmax(r.standard_normal((T, N)), axis=1).astype(f32)
    idx = R.topk_select(R.selection_keys(s, None), k)
    C = R.capacity(1.25, T, N, k)
    d = R.dispatch(idx, N, C)
    flat = idx.reshape(-1)
    pos = _brute_pos(flat.tolist())
    assert (d["pos"] == pos).all()
    assert (d["keep"] == (pos < C)).all()
    cnt = np.bincount(flat, minlength=N)
    assert (d["counts"] == cnt).all()
    assert d["n_dropped"] == int(np.maximum(cnt - C, 0).sum())
    _check_perm(d, flat, N)


def _check_perm(d, flat, N):
    R_ = int(d["offsets"][-1])
    perm = d["perm"]
    assert sorted(perm.tolist()) == sorted(np.nonzero(d["slot"] >= 0)[0].tolist())
    assert len(set(perm.tolist())) == R_
    for e in range(N):
        seg = perm[d["offsets"][e]:d["offsets"][e + 1]]
        assert (flat[seg] == e).all()
        assert (np.diff(seg) > 0).all()
    kept = np.nonzero(d["slot"] >= 0)[0]
    assert (perm[d["slot"][kept]] == kept).all()


def test_identical_tokens_drop_closed_form():
    T, N, k = 40, 8, 2
    C = R.capacity(1.25, T, N, k)  # floor(6.25) = 6
    s = np.tile(np.array([0.3, 0.1, 0.2, 0.05, 0.15, 0.1, 0.05, 0.05], f32), (T, 1))
    idx = R.topk_select(R.selection_keys(s, None), k)
    d = R.dispatch(idx, N, C)
    assert d["n_dropped"] == k * max(0, T - C)
    keep = d["keep"].reshape(T, k)
    assert keep[:C].all() and not keep[C:].any()


def test_dropless_keeps_everything():
    r = rng(10)
    idx = R.topk_select(R.selection_keys(r.random((100, 16)).astype(f32), None), 4)
    d = R.dispatch(idx, 16, None)
    assert d["n_dropped"] == 0 and d["offsets"][-1] == 400
    _check_perm(d, idx.reshape(-1), 16)


def test_capacity_zero_drops_all():
    idx = np.array([[0, 1], [1, 0]])
    d = R.dispatch(idx, 2, 0)
    assert d["n_dropped"] == 4 and (d["slot"] == -1).all() and d["perm"].size == 0


# --------------------------------------------------------------- experts ---

def _dense_swiglu_loops(x, w1, w2):
    T, d = x.shape
    f = w1.shape[0] // 2
    y = np.zeros((T, w2.shape[0]))
    for t in range(T):
        h = []
        for j in range(f):
            a = sum(x[t, c] * w1[j, c] for c in range(d))
            u = sum(x[t, c] * w1[f + j, c] for c in range(d))
            h.append(a / (1.0 + math.exp(-a)) * u)
        for o in range(w2.shape[0]):
            y[t, o] = sum(h[j] * w2[o, j] for j in range(f))
    return y


def _small_layer(seed, T=6, d=8, N=4, f=5):
    r = rng(seed)
    x = r.standard_normal((T, d))
    wr = r.standard_normal((N, d)) / math.sqrt(d)
    w1 = r.standard_normal((N, 2 * f, d)) / math.sqrt(d)
    w2 = r.standard_normal((N, d, f)) / math.sqrt(f)
    return x, wr, w1, w2


def test_identical_experts_collapse_to_dense():
    x, wr, w1, w2 = _small_layer(11)
    w1[:] = w1[0]
    w2[:] = w2[0]
    out = R.moe_layer(x, wr, w1, w2, top_k=2, renormalize=True)
    np.testing.assert_allclose(out["y"], _dense_swiglu_loops(x, w1[0], w2[0]),
                               rtol=1e-10, atol=1e-12)
    # with a shared expert: + its own dense FFN
    r = rng(12)
    ws1 = r.standard_normal((6, 8)) / math.sqrt(8)
    ws2 = r.standard_normal((8, 3)) / math.sqrt(3)
    out2 = R.moe_layer(x, wr, w1, w2, top_k=2, renormalize=True,
                       w1_shared=ws1, w2_shared=ws2)
    np.testing.assert_allclose(out2["y"], _dense_swiglu_loops(x, w1[0], w2[0])
                               + _dense_swiglu_loops(x, ws1, ws2), rtol=1e-10,
                               atol=1e-12)


def test_single_expert_top1_is_dense():
    x, wr, w1, w2 = _small_layer(13, N=1)
    out = R.moe_layer(x, wr, w1, w2, top_k=1, renormalize=True)
    assert (out["topk_w"] == 1).all()
    np.testing.assert_allclose(out["y"], _dense_swiglu_loops(x, w1[0], w2[0]),
                               rtol=1e-10, atol=1e-12)


def test_drops_scale_by_kept_gate_mass():
    T, d, N, f = 16, 8, 4, 5
    x, wr, w1, w2 = _small_layer(14, T=T, d=d, N=N, f=f)
    w1[:] = w1[0]
    w2[:] = w2[0]
    out = R.moe_layer(x, wr, w1, w2, top_k=2, renormalize=True,
                      capacity_factor=1.0)  # C = 4 of 8 expected per expert
    assert out["n_dropped"] > 0
    mass = (out["topk_w"] * out["keep2d"]).sum(1)
    dense = _dense_swiglu_loops(x, w1[0], w2[0])
    np.testing.assert_allclose(out["y"], mass[:, None] * dense, rtol=1e-10,
                               atol=1e-12)


def test_token_subset_matches_full():
    x, wr, w1, w2 = _small_layer(15, T=12)
    full = R.moe_layer(x, wr, w1, w2, top_k=2, capacity_factor=1.0)
    sub = R.moe_layer(x, wr, w1, w2, top_k=2, capacity_factor=1.0,
                      scores_fp32=full["scores"].astype(f32), tokens=[3, 7])
    np.testing.assert_allclose(sub["y"], full["y"][[3, 7]], rtol=1e-13)
    assert (sub["slot"] == full["slot"]).all()
    # streamed weights give the same answer
    sub2 = R.moe_layer(x, wr, lambda e: (w1[e], w2[e]), None, top_k=2,
                       capacity_factor=1.0, scores_fp32=full["scores"].astype(f32),
                       tokens=[3, 7])
    np.testing.assert_allclose(sub2["y"], sub["y"], rtol=0, atol=0)


def test_silu_matches_expit():
    z = np.linspace(-20, 20, 101)
    np.testing.assert_allclose(R.silu(z), z * scipy.special.expit(z), rtol=1e-13,
                               atol=1e-300)


# ------------------------------------------------------------- balancing ---

def test_aux_is_one_for_uniform_top1():
    N, T = 8, 32
    base = np.array([3.0, 1.0, 0.5, 0.2, 0.1, 0.0, -0.5, -1.0])
    l = np.stack([np.roll(base, t % N) for t in range(T)])
    s = R.scores_from_logits(l, "softmax")
    idx = R.topk_select(R.selection_keys(s.astype(f32), None), 1)
    counts = np.bincount(idx.reshape(-1), minlength=N)
    assert (counts == T // N).all()
    assert abs(R.aux_statistic(s, counts) - 1.0) < 1e-12


def test_aux_uniform_P_gives_k_and_uniform_f_gives_one():
    N, T, k = 8, 40, 3
    s = np.full((T, N), 1.0 / N)
    counts = np.array([30, 0, 20, 10, 15, 5, 20, 20])  # sums to T*k
    assert abs(R.aux_statistic(s, counts) - k) < 1e-12
    r = rng(16)
    s2 = scipy.special.softmax(r.standard_normal((T, N)), axis=1)
    assert abs(R.aux_statistic(s2, np.full(N, T // N)) - 1.0) < 1e-12


def test_bias_update_closed_form():
    N, T, k = 6, 30, 2  # mean load 10
    counts = np.array([10, 11, 9, 0, 30, 0])
    b = np.array([0.0, 0.005, -0.005, 0.0099, -0.0099, 1.0], f32)
    nb = R.bias_update(b, counts, T, k, 1e-3)
    expect_sign = [0, 1, -1, -1, 1, -1]
    for i in range(N):
        ref = np.float32(np.float32(b[i]) - np.float32(1e-3) * np.float32(expect_sign[i]))
        assert nb[i] == ref
        assert nb.dtype == np.float32
    assert nb[0] == b[0]
    nbc = R.bias_update(b, counts, T, k, 1e-3, clamp=1e-2)
    assert nbc[3] == np.float32(1e-2) and nbc[5] == np.float32(1e-2)
    # non-integer mean load: sign taken exactly, no rounding of T*k/N
    nb2 = R.bias_update(np.zeros(3, f32), np.array([3, 3, 4]), 5, 2, 1e-3)
    assert nb2.tolist() == [np.float32(1e-3), np.float32(1e-3), np.float32(-1e-3)]


# ------------------------------------------------------------- telemetry ---

def _segs(counts, C=None):
    """offsets of kept rows for per-expert loads under capacity C."""
    kept = np.minimum(counts, C) if C is not None else np.asarray(counts)
    return np.concatenate([[0], np.cumsum(kept)])


def test_stats_uniform_and_collapsed_loads():
    N, T, k = 8, 64, 2
    g = np.full((T, k), 0.5)
    st = R.router_stats(np.full(N, T * k // N), _segs(np.full(N, T * k // N)), g, None, None,
                        None)
    assert st["usage_cv"] == 0.0 and st["dead"] == 0 and st["dropped"] == 0
    # every assignment on expert 0 (k = 1): loads [T, 0, ...]: cv = sqrt(N-1)
    c = np.zeros(N, np.int64)
    c[0] = T
    st = R.router_stats(c, _segs(c), np.ones((T, 1)), None, None, None)
    assert abs(st["usage_cv"] - math.sqrt(N - 1)) < 1e-12 and st["dead"] == N - 1


def test_stats_drops_match_dispatch():
    r = rng(31)
    T, N, k = 64, 8, 2
    idx = np.stack([r.choice(N, k, replace=False) for _ in range(T)])
    C = R.capacity(1.25, T, N, k)
    d = R.dispatch(idx, N, C)
    st = R.router_stats(d["counts"], d["offsets"], np.full((T, k), 0.5), None, None, None)
    assert st["dropped"] == d["n_dropped"]
    assert abs(st["drop_fraction"] - d["n_dropped"] / (T * k)) < 1e-15
    per = st["per_expert"]
    for e in range(N):
        over = max(0, int(d["counts"][e]) - C)
        assert per[e, 2] == over
        assert abs(per[e, 3] - (over / d["counts"][e] if d["counts"][e] else 0.0)) < 1e-15


def test_stats_entropies_closed_forms():
    T, N, k = 5, 6, 4
    g = np.full((T, k), 0.25)
    st = R.router_stats(np.full(N, 1), _segs(np.full(N, 1)), g, np.full((T, N), 0.3), None,
                        None)
    assert abs(st["gate_entropy"] - math.log(k)) < 1e-12
    assert abs(st["score_entropy"] - math.log(N)) < 1e-12
    g1 = np.zeros((T, k))
    g1[:, 0] = 1.0
    s1 = np.zeros((T, N))
    s1[:, 2] = 0.9
    st = R.router_stats(np.full(N, 1), _segs(np.full(N, 1)), g1, s1, None, None)
    assert st["gate_entropy"] == 0.0 and st["score_entropy"] == 0.0
    # two gates p, 1-p
    p = 0.3
    g2 = np.tile([p, 1 - p], (T, 1))
    st = R.router_stats(np.full(N, 1), _segs(np.full(N, 1)), g2, None, None, None)
    assert abs(st["gate_entropy"] + p * math.log(p) + (1 - p) * math.log(1 - p)) < 1e-12


def test_stats_output_scale_and_bias_norm():
    N, d = 3, 4
    counts = np.array([2, 0, 3])
    off = _segs(counts)
    y = np.zeros((5, d))
    y[0:2] = 1.5                         # expert 0: constant rows
    y[2:5] = np.array([[2.0, -2.0, 2.0, -2.0]] * 3)   # expert 2: +-2
    b = np.array([3.0, 4.0, 0.0])
    st = R.router_stats(counts, off, np.full((5, 1), 1.0), None, b, y, y_shared=np.full((2, d), -1.0))
    per = st["per_expert"]
    assert per[0, 4:].tolist() == [1.5, 0.0, 1.5, 1.5]
    assert per[1, 4:].tolist() == [0.0, 0.0, 0.0, 0.0]  # no rows
    assert per[2, 4:].tolist() == [0.0, 2.0, 2.0, 2.0]
    assert per[3, 4:].tolist() == [-1.0, 0.0, -1.0, 1.0]  # shared expert row
    assert st["bias_norm"] == 5.0 and st["bias_absmax"] == 4.0


def test_seq_bias_update_equal_lengths_is_the_batch_rule():
    r = rng(32)
    N, k, L, S = 8, 2, 16, 4
    T = L * S
    idx = np.stack([r.choice(N, k, replace=False) for _ in range(T)])
    counts = np.bincount(idx.reshape(-1), minlength=N)
    b = r.uniform(-0.01, 0.01, N).astype(f32)
    # dyadic lengths: every fp64 share and sum is exact, ties stay ties
    assert np.array_equal(R.bias_update_seq(b, idx, [L] * S, 1e-3),
                          R.bias_update(b, counts, T, k, 1e-3))


def test_seq_bias_update_weights_sequences_equally():
    b = np.zeros(2, f32)
    # sequence 0: one token on expert 0; sequence 1: three tokens on expert 1.
    idx = np.array([[0], [1], [1], [1]])
    # per-sequence shares [1, 0] and [0, 1]: balanced, no change ...
    assert np.array_equal(R.bias_update_seq(b, idx, [1, 3], 1e-3), b)
    # ... while the batch rule (loads 1 vs 3) moves both
    assert R.bias_update(b, np.array([1, 3]), 4, 1, 1e-3).tolist() == \
        [np.float32(1e-3), np.float32(-1e-3)]
    # shares [1, 0] and [1/2, 1/2]: expert 0 overloaded
    idx2 = np.array([[0], [0], [0], [1]])
    nb = R.bias_update_seq(b, idx2, [2, 2], 1e-3, clamp=5e-4)
    assert nb.tolist() == [np.float32(-5e-4), np.float32(5e-4)]


# --------------------------------------------------------- expert choice ---

def test_expert_choice_bruteforce_and_balance():
    r = rng(41)
    T, N, C = 9, 5, 3
    for trial in range(20):
        s = r.integers(0, 4, size=(T, N)).astype(f32) / 4  # many ties
        ch = R.expert_choice_select(s, C)
        assert (ch.sum(axis=0) == C).all()          # perfectly balanced
        for e in range(N):
            # brute force: the chosen set is the lexicographically best C-subset
            # under (score desc, token asc)
            best = sorted(range(T), key=lambda t: (-float(s[t, e]), t))[:C]
            assert set(np.nonzero(ch[:, e])[0]) == set(best)


def test_expert_choice_nan_and_large_capacity():
    s = np.array([[np.nan, 0.1], [0.5, np.nan], [-0.0, 0.0]], f32)
    ch = R.expert_choice_select(s, 2)
    assert ch[:, 0].tolist() == [False, True, True]     # NaN lowest; -0 == +0 kept by index
    assert ch[:, 1].tolist() == [True, False, True]
    assert R.expert_choice_select(s, 10).all()           # C >= T: every token


def test_expert_choice_dispatch_segments():
    r = rng(42)
    T, N, C, k = 12, 4, 5, 2
    ch = R.expert_choice_select(r.random((T, N)).astype(f32), C)
    dsp = R.expert_choice_dispatch(ch, k)
    assert dsp["offsets"].tolist() == [0, 5, 10, 15, 20]
    for e in range(N):
        seg = dsp["perm"][dsp["offsets"][e]:dsp["offsets"][e + 1]] // k
        assert (np.diff(seg) > 0).all()                   # tokens ascending
        assert set(seg) == set(np.nonzero(ch[:, e])[0])
        for t in seg:
            assert dsp["perm"][dsp["row_of"][t, e]] == t * k
    assert (dsp["row_of"][~ch] == -1).all()


def test_expert_choice_full_capacity_identical_experts_is_dense():
    """C >= T with softmax scores: every expert takes every token and the
    gates of a token sum to 1, so identical experts give the dense FFN."""
    r = rng(43)
    T, d, N, f = 7, 12, 3, 10
    x = r.standard_normal((T, d))
    wr = r.standard_normal((N, d)) / math.sqrt(d)
    w1 = r.standard_normal((2 * f, d)) / math.sqrt(d)
    w2 = r.standard_normal((d, f)) / math.sqrt(f)
    out = R.moe_layer_ec(x, wr, np.stack([w1] * N), np.stack([w2] * N), C=T, k=1)
    dense = np.zeros((T, d))
    for t in range(T):
        for j in range(d):
            acc = 0.0
            for c in range(f):
                g = sum(x[t, i] * w1[c, i] for i in range(d))
                u = sum(x[t, i] * w1[f + c, i] for i in range(d))
                acc += w2[j, c] * g / (1.0 + math.exp(-g)) * u
            dense[t, j] = acc
    # the gates are fp32 scores: their sum is 1 to within a few fp32 ulps
    assert np.max(np.abs(out["y"] - dense)) <= 1e-6 * np.max(np.abs(dense))


def test_expert_choice_unchosen_token_gets_shared_only():
    T, d, N, f = 4, 8, 2, 6
    r = rng(44)
    x = r.standard_normal((T, d))
    wr = np.zeros((N, d))
    w1 = r.standard_normal((N, 2 * f, d))
    w2 = r.standard_normal((N, d, f))
    w1s = r.standard_normal((2 * f, d))
    w2s = r.standard_normal((d, f))
    # equal scores everywhere: each expert takes the first C tokens by index
    out = R.moe_layer_ec(x, wr, w1, w2, C=2, k=1, w1_shared=w1s, w2_shared=w2s)
    assert out["chosen"][:, 0].tolist() == [True, True, False, False]
    shared = R.swiglu_ffn(x, w1s, w2s)
    assert np.allclose(out["y"][2:], shared[2:], rtol=0, atol=1e-12)
    assert not np.allclose(out["y"][:2], shared[:2])


# ------------------------------------------------------------------ MXFP8 ---

def _torch():
    return pytest.importorskip("torch")


def test_e4m3_decode_matches_library_type():
    """All 256 codes against the library's float8 E4M3 (OCP 'fn') type."""
    torch = _torch()
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(R.e4m3_decode(c), ref, equal_nan=True)
    assert R.e4m3_decode(np.uint8(0x7E)) == 448.0 and R.e4m3_decode(np.uint8(0x01)) == 2.0 ** -9


def test_e4m3_encode_matches_library_cast_in_range():
    """Round to nearest, ties to even, against the library's cast, on random
    values of every binade and on every midpoint between neighbouring codes."""
    torch = _torch()
    r = rng(50)
    v = (r.standard_normal(100000) * np.exp2(r.integers(-14, 9, 100000))).astype(f32)
    vals = np.unique(R.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    mids = ((vals[1:] + vals[:-1]) / 2).astype(f32)
    assert np.array_equal(mids.astype(np.float64), (vals[1:] + vals[:-1]) / 2)
    v = np.concatenate([v, mids, -mids, vals.astype(f32)])
    v = v[np.abs(v) <= 448]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(R.e4m3_encode(v), ref)


def test_e4m3_encode_saturation_and_specials():
    v = np.array([1000.0, -449.0, 464.0, 479.0, np.nan, -np.nan, -0.0, 0.0, -1e-30,
                  2.0 ** -10, 3 * 2.0 ** -10])
    assert R.e4m3_encode(v).tolist() == [0x7E, 0xFE, 0x7E, 0x7E, 0x7F, 0xFF, 0x80, 0x00,
                                         0x80, 0x00, 0x02]


def test_mx_quantize_is_nearest_by_brute_force():
    """Every element's code is a nearest of the 254 finite codes times the
    block scale 2^X (ties to the even mantissa), or 448 when it lies beyond;
    X = floor(log2 max|v|) - 8 per block of 32 consecutive values."""
    r = rng(51)
    v = r.standard_normal((6, 128)) * np.exp2(r.integers(-20, 20, (6, 1)))
    v[0, :32] *= np.exp2(r.integers(-30, 0, 32))      # a block with a wide spread
    codes, scales = R.mx_quantize(v)
    fin = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    grid = R.e4m3_decode(fin)
    for i in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            blk = v[i, 32 * b:32 * b + 32]
            m, e = math.frexp(float(np.max(np.abs(blk))))
            X = e - 1 - 8
            assert int(scales[i, b]) == X + 127
            for j in range(32):
                s = blk[j] / 2.0 ** X
                got = R.e4m3_decode(codes[i, 32 * b + j])
                if abs(s) > 448:
                    assert got == math.copysign(448.0, s)
                    continue
                dist = np.abs(grid - s)
                best = dist.min()
                assert abs(got - s) == best
                ties = fin[dist == best]
                if len(set(R.e4m3_decode(ties).tolist())) > 1:  # a true tie: even mantissa
                    assert codes[i, 32 * b + j] % 2 == 0


def test_mx_quantize_closed_forms():
    # a power-of-two maximum 2^k: X = k - 8 and that element is 1.0 * 2^8
    blk = np.full(32, 0.001)
    blk[7] = 2.0 ** 5
    c, s = R.mx_quantize(blk)
    assert int(s[0]) == 127 + 5 - 8 and c[7] == 0x78
    # 448 * 2^j is exact; 480 * 2^j exceeds the top code after scaling and saturates
    blk[7] = 448.0 * 2.0 ** -3
    c, s = R.mx_quantize(blk)
    assert int(s[0]) == 127 - 3 and c[7] == 0x7E
    blk[7] = -480.0 * 2.0 ** -3
    c, s = R.mx_quantize(blk)
    assert int(s[0]) == 127 - 3 and c[7] == 0xFE
    # all zero (and negative zero): X = -127, codes keep the sign
    c, s = R.mx_quantize(np.array([0.0, -0.0] * 16))
    assert int(s[0]) == 0 and c.tolist() == [0x00, 0x80] * 16
    # NaN is left out of the maximum and keeps the NaN code; an infinity gives X = 127
    blk = np.linspace(-1, 1, 32)
    blk[3] = np.nan
    c, s = R.mx_quantize(blk)
    assert c[3] == 0x7F and int(s[0]) == 127 + 0 - 8
    blk[3] = -np.inf
    c, s = R.mx_quantize(blk)
    assert int(s[0]) == 254 and c[3] == 0xFE and (c[np.arange(32) != 3] & 0x7F == 0).all()


def test_mx_round_trip_of_representable_blocks():
    """Codes times 2^X, with one element in the top binade, quantise back to
    the same codes and scale."""
    r = rng(52)
    fin = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    for _ in range(50):
        c = r.choice(fin, 64)
        c[r.integers(0, 32)] = 0x78 | r.integers(0, 7)
        c[32 + r.integers(0, 32)] = 0xF8 | r.integers(0, 7)
        s = r.integers(1, 254, 2).astype(np.uint8)
        v = R.mx_dequantize(c, s)
        c2, s2 = R.mx_quantize(v)
        assert np.array_equal(s2, s)
        assert np.array_equal(R.e4m3_decode(c2), R.e4m3_decode(c))


def test_mx_error_bound():
    """|q - v| <= 2^-4 |v| in the normal range of the block, <= 2^(X-10) below."""
    r = rng(53)
    v = r.standard_normal((64, 256)) * np.exp2(r.integers(-8, 8, (64, 256)))
    c, s = R.mx_quantize(v)
    q = R.mx_dequantize(c, s)
    X = np.repeat(s.astype(np.int64) - 127, 32, axis=1)
    sc = np.abs(v) / np.exp2(X)
    normal = (sc >= 2.0 ** -6) & (sc <= 448)
    assert (np.abs(q - v)[normal] <= 2.0 ** -4 * np.abs(v)[normal]).all()
    assert (np.abs(q - v)[~normal & (sc < 1)] <= np.exp2(X - 10)[~normal & (sc < 1)]).all()


def test_swiglu_ffn_mx_explicit_loops():
    """The MXFP8 expert: token rows rounded along d, h along d_ff (each row
    quantised on its own here, in blocks of 32), products in loops."""
    r = rng(54)
    d, f, n = 64, 96, 3
    x = r.standard_normal((n, d))
    w1 = R.mx_round(r.standard_normal((2 * f, d)) / 8)
    w2 = R.mx_round(r.standard_normal((d, f)) / 8)
    got = R.swiglu_ffn_mx(x, w1, w2)
    for t in range(n):
        xq = R.mx_dequantize(*R.mx_quantize(x[t]))
        h = np.zeros(f)
        for c in range(f):
            a = sum(xq[i] * w1[c, i] for i in range(d))
            u = sum(xq[i] * w1[f + c, i] for i in range(d))
            h[c] = a / (1 + math.exp(-a)) * u
        hq = R.mx_dequantize(*R.mx_quantize(h))
        for j in range(d):
            ref = sum(hq[c] * w2[j, c] for c in range(f))
            assert abs(got[t, j] - ref) <= 1e-12 * (1 + abs(ref))


def test_moe_layer_mx_close_to_unquantised_layer():
    """MXFP8 experts change the output by the format's rounding only (a few
    per cent), and the routing not at all (the router stays fp32)."""
    r = rng(55)
    T, d, N, f, k = 40, 64, 6, 64, 2
    x = r.standard_normal((T, d))
    wr = r.standard_normal((N, d)) / 8
    w1 = R.mx_round(r.standard_normal((N, 2 * f, d)) / 8)
    w2 = R.mx_round(r.standard_normal((N, d, f)) / 8)
    a = R.moe_layer(x, wr, w1, w2, top_k=k)
    b = R.moe_layer(x, wr, w1, w2, top_k=k, ffn=R.swiglu_ffn_mx)
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    err = np.linalg.norm(a["y"] - b["y"]) / np.linalg.norm(a["y"])
    assert 1e-3 < err < 0.08


# -------------------------------------------------------------- LatentMoE ---

def _latent_case(seed, T=12, d=16, l=8, N=5, f=12, k=2, shared=True):
    r = rng(seed)
    x = r.standard_normal((T, d))
    wr = r.standard_normal((N, d)) / 4
    wd = r.standard_normal((l, d)) / 4
    wu = r.standard_normal((d, l)) / 3
    w1 = r.standard_normal((N, 2 * f, l)) / 3
    w2 = r.standard_normal((N, l, f)) / 3
    w1s = r.standard_normal((2 * f, d)) / 4 if shared else None
    w2s = r.standard_normal((d, f)) / 3 if shared else None
    return x, wr, wd, wu, w1, w2, w1s, w2s


def test_latent_identity_projections_give_the_plain_layer():
    """l = d and W_down = W_up = I: the LatentMoE layer is the plain layer."""
    x, wr, _, _, _, _, w1s, w2s = _latent_case(60, l=16)
    r = rng(61)
    w1 = r.standard_normal((5, 24, 16)) / 3
    w2 = r.standard_normal((5, 16, 12)) / 3
    eye = np.eye(16)
    a = R.moe_layer_latent(x, wr, eye, eye, w1, w2, top_k=2, w1_shared=w1s, w2_shared=w2s)
    b = R.moe_layer(x, wr, w1, w2, top_k=2, w1_shared=w1s, w2_shared=w2s)
    assert np.array_equal(a["topk_idx"], b["topk_idx"])
    assert np.allclose(a["y"], b["y"], rtol=0, atol=1e-12)


def test_latent_explicit_loops():
    """y_t = W_up (sum_j g_tj E_j(W_down x_t)) + S(x_t), written with loops;
    the routing does not depend on the projections."""
    x, wr, wd, wu, w1, w2, w1s, w2s = _latent_case(62)
    out = R.moe_layer_latent(x, wr, wd, wu, w1, w2, top_k=2, w1_shared=w1s, w2_shared=w2s)
    plain = R.moe_layer(x, wr, np.zeros((5, 24, 16)), np.zeros((5, 16, 12)), top_k=2,
                        compute_outputs=False)
    assert np.array_equal(out["topk_idx"], plain["topk_idx"])
    T, d, l, f = 12, 16, 8, 12
    for t in range(T):
        z = [sum(wd[a, i] * x[t, i] for i in range(d)) for a in range(l)]
        ylat = [0.0] * l
        for j in range(2):
            e = out["topk_idx"][t, j]
            g = out["topk_w"][t, j]
            h = []
            for c in range(f):
                a_ = sum(w1[e, c, i] * z[i] for i in range(l))
                u_ = sum(w1[e, f + c, i] * z[i] for i in range(l))
                h.append(a_ / (1 + math.exp(-a_)) * u_)
            for i in range(l):
                ylat[i] += g * sum(w2[e, i, c] * h[c] for c in range(f))
        for i in range(d):
            hs = []
            for c in range(f):
                a_ = sum(w1s[c, q] * x[t, q] for q in range(d))
                u_ = sum(w1s[f + c, q] * x[t, q] for q in range(d))
                hs.append(a_ / (1 + math.exp(-a_)) * u_)
            ref = sum(wu[i, a] * ylat[a] for a in range(l)) + sum(w2s[i, c] * hs[c] for c in range(f))
            assert abs(out["y"][t, i] - ref) <= 1e-10 * (1 + abs(ref))
