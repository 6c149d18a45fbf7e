"""GPU parity of the LatentMoE layer forward (moe_forward_latent) against
the fp64 oracle: routing bit for bit (same fp32 scores), output within the
layer tolerance (relative L2 2e-2 bf16, 1e-5 fp32).  With identity
projections at full width and no shared expert the latent layer must equal
moe_forward bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_18_amd as moe
import workloads as W
from gpu_util import check_routing_and_dispatch, host, oracle_kwargs, rel_l2, say, tol_for

pytestmark = pytest.mark.gpu


def run_latent(li, shape):
    inp = li.base
    T, N, k, d = shape.T, shape.n_experts, shape.top_k, shape.d_model
    dev = inp.x.device
    out = dict(
        y=torch.empty((T, d), dtype=shape.torch_dtype, device=dev),
        scores=torch.empty((T, N), dtype=torch.float32, device=dev),
        topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
        counts=torch.empty((N,), dtype=torch.int32, device=dev),
        offsets=torch.empty((N + 1,), dtype=torch.int32, device=dev),
        slot=torch.empty((T * k,), dtype=torch.int32, device=dev),
        n_kept_dropped=torch.empty((2,), dtype=torch.int32, device=dev))
    ws = moe.latent_workspace(shape, li.d_latent, dev)
    moe.moe_forward_latent(shape, li.d_latent, inp.x, inp.w_router, inp.logit_add, inp.bias,
                           li.w_down, li.w_up, li.w1, li.w2, inp.w1_shared, inp.w2_shared,
                           out["y"], out["scores"], out["topk_idx"], out["topk_w"],
                           out["counts"], out["offsets"], out["slot"], out["n_kept_dropped"], ws)
    torch.cuda.synchronize()
    return out


def oracle_latent(li, scores, tokens=None):
    inp = li.base
    return oracle.moe_layer_latent(
        host(inp.x), host(inp.w_router), host(li.w_down), host(li.w_up),
        lambda e: (host(li.w1[e]), host(li.w2[e])), None,
        w1_shared=None if inp.w1_shared is None else host(inp.w1_shared),
        w2_shared=None if inp.w2_shared is None else host(inp.w2_shared),
        scores_fp32=host(scores), tokens=tokens, **oracle_kwargs(inp))


def _small(name, **kw):
    base = dict(T=300, d_model=256, n_experts=8, top_k=2, d_ff=128)
    base.update(kw)
    return W.LayerConfig(name, **base)


CASES = [
    (_small("lat_small"), 128, None),
    (_small("lat_shared", T=513, n_experts=16, top_k=4, d_ff_shared=192, d_model=384), 64, None),
    (_small("lat_drop", T=257, n_experts=16, top_k=4, capacity_factor=1.1), 128, None),
    (_small("lat_f32", T=129, n_experts=6, top_k=3, dtype="f32", d_ff_shared=64), 96, None),
    (_small("lat_t1", T=1, n_experts=16, top_k=4, d_ff_shared=128), 128, None),
    (W.CONFIGS["decode"], 512, None),
    (W.CONFIGS["dsv3"].replace(T=512), 1792, 8),
    (W.CONFIGS["dsv3"], 1792, 3),
]


@pytest.mark.parametrize("cfg,l,n_sample", CASES,
                         ids=[f"{c.name}_T{c.T}_l{l}" for c, l, _ in CASES])
def test_latent_forward_matches_oracle(cfg, l, n_sample):
    say(f"[latent] {cfg.name} T={cfg.T} d={cfg.d_model} l={l} N={cfg.n_experts} k={cfg.top_k} "
        f"fs={cfg.d_ff_shared} {cfg.dtype}")
    li = W.make_latent_inputs(cfg, l, seed=21, device="cuda")
    shape = moe.MoeShape.from_config(cfg)
    out = run_latent(li, shape)
    T = cfg.T
    tokens = None
    if n_sample is not None and n_sample < T:
        r = np.random.default_rng(5)
        tokens = sorted(set([0, T - 1] + r.choice(T, n_sample - 2, replace=False).tolist()))
    ref = oracle_latent(li, out["scores"], tokens)
    check_routing_and_dispatch(out, ref, T, cfg.top_k)
    y = host(out["y"])[ref["rows"]]
    err = rel_l2(y, ref["y"])
    say(f"  rel L2 y = {err:.3e} over {len(ref['rows'])} tokens")
    assert err <= tol_for(cfg)


@pytest.mark.parametrize("name", ["decode", "small"])
def test_identity_projections_equal_the_plain_forward(name):
    """l = d, W_down = W_up = I, no shared expert: z = x exactly, the latent
    combine is the plain combine, and y_lat I = y_lat: bit for bit."""
    cfg = W.CONFIGS["decode"] if name == "decode" else _small("lat_id", T=300)
    d = cfg.d_model
    li = W.make_latent_inputs(cfg, d, seed=4, device="cuda")
    eye = torch.eye(d, dtype=torch.bfloat16, device="cuda")
    li.w_down, li.w_up = eye.contiguous(), eye.contiguous()
    shape = moe.MoeShape.from_config(cfg)
    out = run_latent(li, shape)
    plain = moe.forward(shape, li.base.x, li.base.w_router, li.w1, li.w2,
                        logit_add=li.base.logit_add, bias=li.base.bias)
    torch.cuda.synchronize()
    assert torch.equal(out["topk_idx"], plain["topk_idx"])
    assert torch.equal(out["y"], plain["y"])


def test_latent_rejects_unsupported():
    cfg = _small("lat_bad")
    shape = moe.MoeShape.from_config(cfg)
    assert moe.moe_latent_workspace_bytes(shape, 96) == 0
    mx = shape.replace(dtype=moe.MOE_DTYPE_MXFP8)
    assert moe.moe_latent_workspace_bytes(mx, 128) == 0


def test_latent_deterministic_and_graph_replay():
    """Two eager LatentMoE forwards are bitwise equal, and a HIP-graph replay
    of the forward gives the same bits (eager work between replays)."""
    cfg = _small("lat_graph", T=257, n_experts=16, top_k=4, d_ff_shared=128)
    li = W.make_latent_inputs(cfg, 128, seed=8, device="cuda")
    shape = moe.MoeShape.from_config(cfg)
    a = run_latent(li, shape)
    b = run_latent(li, shape)
    assert torch.equal(a["y"], b["y"])
    inp = li.base
    ws = moe.latent_workspace(shape, li.d_latent)
    y = torch.empty_like(a["y"])

    def step():
        moe.moe_forward_latent(shape, li.d_latent, inp.x, inp.w_router, inp.logit_add, inp.bias,
                               li.w_down, li.w_up, li.w1, li.w2, inp.w1_shared, inp.w2_shared,
                               y, None, None, None, None, None, None, None, ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        y.zero_()
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, a["y"]), rep
        assert float(junk) == float(junk)
