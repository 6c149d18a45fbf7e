"""MoE FFN layer forward benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config dsv3]
                    [--configs tiny,mixtral,decode,switch]

One step = one full layer forward (router GEMM, scores + top-k, dispatch,
grouped SwiGLU expert GEMMs incl. the shared expert, combine) over one batch
of synthetic, seeded inputs already resident in HBM.  The steps of the
headline workload (--config) are timed twice, launched eagerly and as replays
of one HIP graph of the step; the faster of the two is the reported rate
(both are in the line), and each replay is also timed on its own for the
median and the 10th/90th percentiles.  Prints ONE JSON line.

Extra fields beside the contract's:
  roofline      the dominant kernel, the gate/up grouped GEMM with the SwiGLU
                epilogue (every expert segment and the shared expert), timed
                live with HIP events on the stream it runs on, one launch per
                event pair.  Bound = the peak its algorithmic work reaches
                first: bytes (touched experts' W1, x once, h written) at the
                8 TB/s HBM peak, or FLOPs at the dense bf16 MFMA peak.
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload,
                timed on this host's cores
  mxfp8         the same layer with MXFP8 experts (weights quantised once,
                router unchanged): forward rate and the expert projections
                against the fp8 MFMA and HBM peaks
  expert_choice the same layer routed by expert choice at C = k*T/N
  latent        the LatentMoE variant of the layer at latent width d/4
  ep8_share     the expert FFNs at one GPU's share under 8-way expert
                parallelism (N/8 experts, k*T rows spread evenly over them)
  configs       the other workloads (--configs), each with the per-step
                median / p10 / p90 of its graph-replayed forward, tokens/s,
                TFLOP/s, the layer against its roofline, the same gate/up
                roofline object and a cpu_baseline of its own.  Decode and
                switch steps each follow a 512 MiB read that evicts the
                last-level cache (their expert weights would otherwise stay
                in it from one step to the next), and decode takes at least
                500 timed steps.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense fp8 MFMA
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
METRIC = "MoE layer fwd tokens/s + TFLOP/s (% bf16 MFMA peak), DeepSeek-V3 shape"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=30)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="dsv3")
    p.add_argument("--configs", default="tiny,mixtral,decode,switch",
                   help="comma list of further workloads measured after --config "
                        "('' for none)")
    p.add_argument("--cpu-sample-tokens", type=int, default=0,
                   help="tokens of the batch the oracle runs on (0: the workload's default, "
                        "about 10 s on the host)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--stage-iters", type=int, default=10)
    p.add_argument("--skip", default="",
                   help="comma list of extra sections to leave out: ec, mx, latent, telemetry, ep "
                        "(profiler runs use it to keep one kernel's dispatches apart)")
    return p.parse_args()


def algorithmic_flops(cfg, n_kept: int) -> dict:
    d, N, T = cfg.d_model, cfg.n_experts, cfg.T
    router = 2.0 * T * d * N
    experts = 6.0 * d * cfg.d_ff * n_kept
    shared = 6.0 * T * d * cfg.d_ff_shared
    return dict(router=router, experts=experts, shared=shared,
                total=router + experts + shared)


def committed_traffic(workload: str, proj: str = "gate_up"):
    """HBM bytes per launch of the gate/up (proj "gate_up", "gate_up_mxfp8")
    or down ("down") GEMM on this workload,
    from the committed rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE,
    each scaled by the same counter on a plain 1 GiB copy); None when there is
    none or the kernel source changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"gemm_{proj}_{workload}_hbm_traffic.md")
    src = os.path.join(ROOT, "sparse_mixture_experts_18_amd", "csrc", "grouped_gemm.hip")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("- "):
            k_, v_ = line.strip()[2:].split(":", 1)
            vals[k_.strip()] = v_.strip().strip("`")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if vals.get("grouped_gemm.hip sha256") != sha:
        return None
    try:
        return int(float(vals["hbm bytes per launch"]))
    except (KeyError, ValueError):
        return None


# tokens of each workload's batch the oracle runs on (run again until 10 s of host
# work have passed), the workloads whose steps follow a last-level-cache eviction,
# and the fewest timed steps per workload
CPU_SAMPLE = {"tiny": 64, "mixtral": 8, "decode": 64, "switch": 256, "dsv3": 64}
STEP_FLUSH = {"decode", "switch"}
MIN_STEPS = {"tiny": 500, "decode": 500, "switch": 200, "mixtral": 50}


def cpu_baseline(cfg, inp, n_tokens: int, min_seconds: float = 10.0) -> dict:
    """The fp64 oracle, as it stands, on the first n_tokens tokens of the
    batch: router, scores, selection, dispatch, expert FFNs of every expert
    those tokens touch, shared expert, combine (a capacity, if any, follows
    the sample's own token count).  Weights are copied to host before the
    clock starts (exact fp32 copies of the bf16 values); the layer is run
    again until min_seconds have passed."""
    import numpy as np
    import threadpoolctl
    import torch

    import oracle

    n_tokens = min(n_tokens, cfg.T)
    x = inp.x[:n_tokens].float().cpu().numpy()
    wr = inp.w_router.cpu().numpy()
    la = None if inp.logit_add is None else inp.logit_add[:n_tokens].cpu().numpy()
    bias = None if inp.bias is None else inp.bias.cpu().numpy()
    # experts the sample touches (routing is per token for dropless layers;
    # the oracle re-derives it below, this only decides what to prefetch)
    l = oracle.router_logits(x, wr, la)
    s = oracle.scores_from_logits(l, cfg.score_fn)
    keys = oracle.selection_keys(s.astype(np.float32), bias)
    cand = None
    if cfg.n_groups > 1:
        cand = oracle.group_candidates(keys, cfg.n_groups, cfg.topk_groups,
                                       cfg.top_k // cfg.topk_groups)
    touched = sorted(set(oracle.topk_select(keys, cfg.top_k, cand).reshape(-1).tolist()))
    # host copies in the layer's own dtype; each expert is widened when the
    # oracle asks for it (exact: bf16 -> fp32 is lossless)
    wcache = {e: (inp.w1[e].cpu(), inp.w2[e].cpu()) for e in touched}
    w1s = None if inp.w1_shared is None else inp.w1_shared.float().cpu().numpy()
    w2s = None if inp.w2_shared is None else inp.w2_shared.float().cpu().numpy()
    torch.cuda.synchronize()
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    runs = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_layer(x, wr, lambda e: (wcache[e][0].float().numpy(),
                                           wcache[e][1].float().numpy()), None,
                         top_k=cfg.top_k, score_fn=cfg.score_fn, renormalize=cfg.renormalize,
                         n_groups=cfg.n_groups, topk_groups=cfg.topk_groups,
                         capacity_factor=cfg.capacity_factor, capacity_rule=cfg.capacity_rule,
                         bias=bias, logit_add=la, w1_shared=w1s, w2_shared=w2s)
        runs += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(n_tokens * runs / dt, 3), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"first {n_tokens} tokens of the {cfg.name} batch, {runs} run(s): full "
                       f"fp64 layer (router over all {cfg.n_experts} experts, {len(touched)} "
                       f"touched experts{', shared expert' if cfg.d_ff_shared else ''}); "
                       f"{dt:.2f} s wall"),
            "blas": ",".join(sorted({i.get("internal_api", "?") for i in info}))}


def quantiles(ts) -> dict:
    t = sorted(ts)
    q = lambda f: t[min(len(t) - 1, int(round(f * (len(t) - 1))))]
    return {"median": round(q(0.5), 4), "p10": round(q(0.1), 4), "p90": round(q(0.9), 4)}


class Timer:
    """HIP-event timing on the stream the library launches on (torch's
    current stream).  evict() reads 512 MiB, twice the 256 MiB last-level
    cache (reads only: no dirty lines left to write back)."""

    def __init__(self, torch, dev):
        self.torch = torch
        self.stream = torch.cuda.current_stream()
        self.flush = torch.ones(64 << 20, dtype=torch.float64, device=dev)
        self.sink = torch.empty((), dtype=torch.float64, device=dev)

    def evict(self):
        self.torch.sum(self.flush, dim=0, out=self.sink)

    def each(self, fn, iters, evict=False, warm=2):
        """ms of each of `iters` calls, one event pair per call; the eviction
        (when asked) runs before each call, outside its events"""
        torch = self.torch
        evs = []
        for _ in range(warm + iters):
            if evict:
                self.evict()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(self.stream)
            fn()
            b.record(self.stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in evs[warm:]]

    def back_to_back(self, fn, iters):
        """mean ms of `iters` calls launched back to back"""
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(iters):
            fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters


def layer_roofline(cfg, touched: int, n_kept: int, ms: float) -> dict:
    """The whole layer against its roofline: the algorithmic bytes (router
    weights, the touched experts' and the shared expert's weights, x read
    and y written once) at the HBM peak, or the algorithmic FLOPs at the
    MFMA peak of the layer's dtype, whichever takes longer; frac = that
    time / the measured step."""
    d = cfg.d_model
    esz = 2 if cfg.dtype == "bf16" else 4
    nbytes = (4 * cfg.n_experts * d
              + esz * (3 * d * (touched * cfg.d_ff + cfg.d_ff_shared) + 2 * cfg.T * d))
    fl = algorithmic_flops(cfg, n_kept)["total"]
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9) * 1e3
    t_mfma = fl / (peak * 1e12) * 1e3
    bound = "hbm" if t_hbm >= t_mfma else "mfma"
    return {"bound": bound, "algorithmic_bytes": int(nbytes), "flops": fl,
            "min_ms_at_peaks": round(max(t_hbm, t_mfma), 4),
            "frac": round(max(t_hbm, t_mfma) / ms, 4),
            "hbm_frac": round(t_hbm / ms, 4), "mfma_frac": round(t_mfma / ms, 4)}


def expert_stages(moe, torch, tm, cfg, shape, inp, ws, n_kept, iters):
    """Route and dispatch once, build the work lists, then time the gate/up
    and the down grouped GEMMs alone (offsets=None launches the GEMM kernel
    only, so each event pair brackets one kernel), each call after a
    last-level-cache eviction.  Returns (roofline of gate/up, down-projection
    figures, the routing buffers)."""
    dev = inp.x.device
    T, N, k, d = cfg.T, cfg.n_experts, cfg.top_k, cfg.d_model
    b = dict(
        sc=torch.empty((T, N), dtype=torch.float32, device=dev),
        ti=torch.empty((T, k), dtype=torch.int32, device=dev),
        tw=torch.empty((T, k), dtype=torch.float32, device=dev),
        cn=torch.empty((N,), dtype=torch.int32, device=dev),
        of=torch.empty((N + 1,), dtype=torch.int32, device=dev),
        sl=torch.empty((T * k,), dtype=torch.int32, device=dev),
        pm=torch.empty((T * k,), dtype=torch.int32, device=dev),
        nkd=torch.empty((2,), dtype=torch.int32, device=dev),
    )
    dt = shape.torch_dtype
    b["h"] = torch.empty((T * k, cfg.d_ff), dtype=dt, device=dev)
    b["hs"] = (torch.empty((T, cfg.d_ff_shared), dtype=dt, device=dev)
               if cfg.d_ff_shared else None)
    b["yp"] = torch.empty((T * k, d), dtype=dt, device=dev)
    b["ysh"] = torch.empty((T, d), dtype=dt, device=dev) if cfg.d_ff_shared else None
    moe.moe_route(shape, inp.x, inp.w_router, inp.logit_add, None, inp.bias, None, b["sc"],
                  b["ti"], b["tw"], ws)
    moe.moe_dispatch(shape, b["ti"], b["cn"], b["of"], b["sl"], b["pm"], b["nkd"], ws)
    moe.moe_expert_plan(shape, b["of"], ws)
    t1 = tm.each(lambda: moe.moe_expert_gate_up(shape, inp.x, b["pm"], None, inp.w1,
                                                inp.w1_shared, b["h"], b["hs"], ws),
                 iters, evict=True)
    t2 = tm.each(lambda: moe.moe_expert_down(shape, b["h"], b["hs"], None, inp.w2,
                                             inp.w2_shared, b["yp"], b["ysh"], ws),
                 iters, evict=True)
    g1_ms, g2_ms = sum(t1) / len(t1), sum(t2) / len(t2)
    counts = b["cn"].cpu().numpy()
    g1_flops = 4.0 * d * cfg.d_ff * n_kept + 4.0 * T * d * cfg.d_ff_shared
    g2_flops = 2.0 * d * cfg.d_ff * n_kept + 2.0 * T * d * cfg.d_ff_shared
    touched = int((counts > 0).sum())
    esz = 2 if cfg.dtype == "bf16" else 4
    g1_bytes = esz * (touched * 2 * cfg.d_ff * d + 2 * cfg.d_ff_shared * d + T * d
                      + n_kept * cfg.d_ff + T * cfg.d_ff_shared)
    g2_bytes = esz * (touched * cfg.d_ff * d + cfg.d_ff_shared * d + n_kept * cfg.d_ff
                      + T * cfg.d_ff_shared + n_kept * d + (T * d if cfg.d_ff_shared else 0))
    traffic = committed_traffic(cfg.name)
    # the bound is whichever peak the kernel's algorithmic work would hit
    # first: its bytes at the HBM peak or its FLOPs at the MFMA peak
    peak_fl = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    t_hbm = g1_bytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = g1_flops / (peak_fl * 1e12)
    gbs = g1_bytes / (g1_ms * 1e-3) / 1e9
    tfs = g1_flops / (g1_ms * 1e-3) / 1e12
    if t_hbm >= t_mfma:
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "mfma_frac": round(tfs / peak_fl, 4)}
    else:
        roofline = {"bound": "mfma", "achieved": round(tfs, 2), "peak": peak_fl,
                    "unit": "TFLOP/s", "frac": round(tfs / peak_fl, 4), "traffic": traffic,
                    "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    if cfg.dtype == "bf16":
        kname = ("gemm_mfma_kernel<true, false, .> (bf16 gate/up projection + SwiGLU over "
                 "every expert segment and the shared expert; one launch per call, work "
                 "list prebuilt)")
        k2name = "gemm_mfma_kernel<false, false, .> (bf16 down projection)"
    else:
        kname = ("gemm_f32_kernel<true> (fp32 gate/up projection + SwiGLU over every "
                 "expert segment; one launch per call, work list prebuilt)")
        k2name = "gemm_f32_kernel<false> (fp32 down projection)"
    roofline.update({
        "kernel": kname,
        "avg_ms": round(g1_ms, 4),
        "median_ms": quantiles(t1)["median"],
        "flops_per_launch": g1_flops,
        "algorithmic_bytes_per_launch": g1_bytes,
        "touched_experts": touched,
        "min_ms_at_peaks": round(max(t_hbm, t_mfma) * 1e3, 4),
    })
    g2_gbs = g2_bytes / (g2_ms * 1e-3) / 1e9
    gemm2 = {"kernel": k2name, "avg_ms": round(g2_ms, 4),
             "tflops": round(g2_flops / (g2_ms * 1e-3) / 1e12, 2),
             "algorithmic_bytes_per_launch": g2_bytes, "GB/s": round(g2_gbs, 1),
             "hbm_frac": round(g2_gbs / PEAK_HBM_GBS, 4),
             "traffic": committed_traffic(cfg.name, "down")}
    b["touched"] = touched
    b["g1_flops"], b["g2_flops"] = g1_flops, g2_flops
    return roofline, gemm2, b


def workload_name(cfg) -> str:
    return (f"{cfg.name}: T={cfg.T} d_model={cfg.d_model} N={cfg.n_experts} top_k={cfg.top_k}"
            f" d_ff={cfg.d_ff} shared={cfg.d_ff_shared} score={cfg.score_fn}"
            f" groups={cfg.topk_groups}/{cfg.n_groups}"
            f" capacity_factor={cfg.capacity_factor}")


def measure_config(moe, W, torch, dev, cfg, args) -> dict:
    """One further workload: graph-replayed forwards timed one by one
    (median, p10, p90), the layer roofline, the gate/up kernel roofline and
    the oracle on a sample."""
    print(f"[bench] {cfg.name}: generating inputs", file=sys.stderr, flush=True)
    inp = W.make_inputs(cfg, seed=0, device=dev)
    shape = moe.MoeShape.from_config(cfg)
    ws = moe.workspace(shape, dev)
    y = torch.empty((cfg.T, cfg.d_model), dtype=shape.torch_dtype, device=dev)
    nkd = torch.empty(2, dtype=torch.int32, device=dev)
    tm = Timer(torch, dev)

    def step():
        moe.moe_forward(shape, inp.x, inp.w_router, inp.logit_add, inp.bias, inp.w1, inp.w2,
                        inp.w1_shared, inp.w2_shared, y, None, None, None, None, None, None,
                        nkd, ws)
    for _ in range(args.warmup):
        step()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    iters = max(args.steps, MIN_STEPS.get(cfg.name, 0))
    evict = cfg.name in STEP_FLUSH
    print(f"[bench] {cfg.name}: {iters} timed steps", file=sys.stderr, flush=True)
    ts = tm.each(graph.replay, iters, evict=evict, warm=max(2, args.warmup))
    del graph
    q = quantiles(ts)
    ms = q["median"]
    n_kept = int(nkd[0].item())
    fl = algorithmic_flops(cfg, n_kept)
    roofline, gemm2, b = expert_stages(moe, torch, tm, cfg, shape, inp, ws, n_kept,
                                       args.stage_iters)
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    tfl = fl["total"] / (ms * 1e-3) / 1e12
    ent = {
        "workload": workload_name(cfg),
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "launch": "hip graph replay, one event pair per step",
        "steps": iters,
        "step_preceded_by": ("a 512 MiB read evicting the last-level cache" if evict
                             else "the previous step"),
        "ms_per_step": ms,
        "ms_p10": q["p10"],
        "ms_p90": q["p90"],
        "tokens/s": round(cfg.T / (ms * 1e-3), 1),
        "tflops": round(tfl, 3),
        "peak_frac": round(tfl / peak, 4),
        "n_kept": n_kept,
        "layer_roofline": layer_roofline(cfg, b["touched"], n_kept, ms),
        "roofline": roofline,
        "gemm2": gemm2,
    }
    if not args.no_cpu_baseline:
        print(f"[bench] {cfg.name}: cpu baseline (oracle)", file=sys.stderr, flush=True)
        ent["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_tokens
                                           or CPU_SAMPLE.get(cfg.name, 64))
    del inp, ws, b
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return ent


def main():
    args = parse()
    skip = {t.strip() for t in args.skip.split(",") if t.strip()}
    bad = skip - {"ec", "mx", "latent", "telemetry", "ep"}
    if bad:
        raise SystemExit(f"--skip: unknown sections {sorted(bad)}")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build measures one GPU: the layer forward runs "
                                   "unsharded on a single MI355X; --gpus must be 1"}))
        sys.exit(2)

    import torch

    import sparse_mixture_experts_18_amd as moe
    import workloads as W

    moe.lib()  # fail loudly if the HIP library is missing
    cfg = W.CONFIGS[args.config]
    others = [c.strip() for c in args.configs.split(",") if c.strip() and c.strip() != cfg.name]
    unknown = [c for c in others if c not in W.CONFIGS]
    if unknown:
        raise SystemExit(f"--configs: unknown workloads {unknown}")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    res = headline(moe, W, torch, dev, cfg, args)
    # the headline workload's buffers are gone before the next inputs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    res["configs"] = {}
    for name in others:
        res["configs"][name] = measure_config(moe, W, torch, dev, W.CONFIGS[name], args)
    print(json.dumps(res), flush=True)


def headline(moe, W, torch, dev, cfg, args) -> dict:
    """The headline workload: eager and graph-replayed forwards, the expert
    GEMM stages, and the layer variants on the same inputs."""
    skip = {t.strip() for t in args.skip.split(",") if t.strip()}
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    inp = W.make_inputs(cfg, seed=0, device=dev)
    shape = moe.MoeShape.from_config(cfg)
    T, N, k, d = cfg.T, cfg.n_experts, cfg.top_k, cfg.d_model
    ws = moe.workspace(shape, dev)
    out = dict(
        y=torch.empty((T, d), dtype=shape.torch_dtype, device=dev),
        n_kept_dropped=torch.empty(2, dtype=torch.int32, device=dev),
    )
    tm = Timer(torch, dev)

    def step():
        moe.moe_forward(shape, inp.x, inp.w_router, inp.logit_add, inp.bias, inp.w1, inp.w2,
                        inp.w1_shared, inp.w2_shared, out["y"], None, None, None, None, None,
                        None, out["n_kept_dropped"], ws)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    eager_ms = tm.back_to_back(step, args.steps)

    # the same step captured once in a HIP graph (the library does no host
    # syncs, allocations or memsets), then replayed: every kernel still runs
    # every step, only the per-launch host overhead goes away
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(args.warmup):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = tm.back_to_back(graph.replay, args.steps)
    q = quantiles(tm.each(graph.replay, args.steps))
    del graph
    ms = min(eager_ms, graph_ms)
    n_kept = int(out["n_kept_dropped"][0].item())
    fl = algorithmic_flops(cfg, n_kept)
    tflops = fl["total"] / (ms * 1e-3) / 1e12
    print(f"[bench] {eager_ms:.3f} ms/step eager, {graph_ms:.3f} ms/step graph replay",
          file=sys.stderr, flush=True)

    # ---- per-kernel timing of the expert GEMMs, same stream, HIP events ----
    roofline, gemm2, b = expert_stages(moe, torch, tm, cfg, shape, inp, ws, n_kept,
                                       args.stage_iters)
    sc, ti, tw, cn, of = b["sc"], b["ti"], b["tw"], b["cn"], b["of"]
    sl, pm, nkd, yp, ysh = b["sl"], b["pm"], b["nkd"], b["yp"], b["ysh"]
    touched, g1_flops, g2_flops = b["touched"], b["g1_flops"], b["g2_flops"]
    esz = 2 if cfg.dtype == "bf16" else 4

    def timed(fn, iters):
        t = tm.each(fn, iters, evict=True)
        return sum(t) / len(t)
    # router telemetry over this forward's outputs (HBM-bound: it reads the
    # kept expert rows, the shared rows, the scores and the gates once)
    telemetry = None
    if "telemetry" not in skip:
        stats = torch.empty(moe.moe_router_stats_count(shape), dtype=torch.float64, device=dev)
        tl_ms = timed(lambda: moe.moe_router_stats(shape, cn, of, tw, sc, inp.bias, yp, ysh,
                                                   stats, ws), args.stage_iters)
        tl_bytes = esz * (n_kept + (T if cfg.d_ff_shared else 0)) * d + 4 * T * (N + k) + 8 * N
        tl_gbs = tl_bytes / (tl_ms * 1e-3) / 1e9
        telemetry = {"kernels": "row_stats, expert_stats, entropy, stats_final (moe_router_stats)",
                     "avg_ms": round(tl_ms, 4), "algorithmic_bytes": tl_bytes,
                     "GB/s": round(tl_gbs, 1), "hbm_frac": round(tl_gbs / PEAK_HBM_GBS, 4)}

    # expert-choice routing on the same layer: every expert takes its
    # C = k*T/N tokens (the same number of expert rows as token choice)
    ec_shape = shape.replace(capacity_factor=1.0, capacity_rule=moe.MOE_CAP_ASSIGNMENTS)
    expert_choice = None
    if "ec" not in skip and moe.moe_ec_capacity(ec_shape) * N <= T * k:
        y_ec = torch.empty_like(out["y"])
        ws_ec = moe.workspace(ec_shape, dev)

        def ec_step():
            moe.moe_forward_ec(ec_shape, inp.x, inp.w_router, inp.logit_add, inp.w1, inp.w2,
                               inp.w1_shared, inp.w2_shared, y_ec, None, None, None, ws_ec)
        for _ in range(2):
            ec_step()
        ec_ms = tm.back_to_back(ec_step, args.stage_iters)
        expert_choice = {"ms_per_step": round(ec_ms, 4), "tokens/s": round(T / (ec_ms * 1e-3), 1),
                         "capacity_per_expert": moe.moe_ec_capacity(ec_shape)}

    # MXFP8 experts on the same layer (router unchanged): the bf16 weights
    # quantised once by moe_quantize_mx, then the same forward and the two
    # expert projections timed as above
    mxfp8 = None
    if "mx" not in skip and cfg.dtype == "bf16" and d % 128 == 0 and cfg.d_ff % 128 == 0 and \
            cfg.d_ff_shared % 128 == 0:
        mx_shape = shape.replace(dtype=moe.MOE_DTYPE_MXFP8)
        ws_mx = moe.workspace(mx_shape, dev)
        w1q, w2q = moe.quantize_mx(inp.w1), moe.quantize_mx(inp.w2)
        w1sq = moe.quantize_mx(inp.w1_shared) if cfg.d_ff_shared else None
        w2sq = moe.quantize_mx(inp.w2_shared) if cfg.d_ff_shared else None
        y_mx = torch.empty_like(out["y"])

        def mx_step():
            moe.moe_forward(mx_shape, inp.x, inp.w_router, inp.logit_add, inp.bias, w1q, w2q,
                            w1sq, w2sq, y_mx, None, None, None, None, None, None, None, ws_mx)
        for _ in range(2):
            mx_step()
        g_mx = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_mx):
            mx_step()
        for _ in range(2):
            g_mx.replay()
        mx_ms = tm.back_to_back(g_mx.replay, args.steps)
        del g_mx
        hq = torch.empty(moe.mx_bytes(T * k * cfg.d_ff), dtype=torch.uint8, device=dev)
        hsq = (torch.empty(moe.mx_bytes(T * cfg.d_ff_shared), dtype=torch.uint8, device=dev)
               if cfg.d_ff_shared else None)
        moe.moe_expert_plan(mx_shape, of, ws_mx)
        m1_ms = timed(lambda: moe.moe_expert_gate_up(mx_shape, inp.x, pm, None, w1q, w1sq, hq,
                                                     hsq, ws_mx), args.stage_iters)
        m2_ms = timed(lambda: moe.moe_expert_down(mx_shape, hq, hsq, None, w2q, w2sq, yp, ysh,
                                                  ws_mx), args.stage_iters)
        mxb = 33.0 / 32.0  # bytes per MXFP8 value with its share of a scale
        m1_bytes = mxb * (touched * 2 * cfg.d_ff * d + 2 * cfg.d_ff_shared * d + T * d
                          + n_kept * cfg.d_ff + T * cfg.d_ff_shared)
        m1_gbs = m1_bytes / (m1_ms * 1e-3) / 1e9
        m1_tfs = g1_flops / (m1_ms * 1e-3) / 1e12
        mxfp8 = {
            "experts": "MXFP8 (E4M3 + E8M0 per 32), router fp32",
            "ms_per_step": round(mx_ms, 4), "tokens/s": round(T / (mx_ms * 1e-3), 1),
            "tflops": round(fl["total"] / (mx_ms * 1e-3) / 1e12, 2),
            "gate_up_ms": round(m1_ms, 4), "gate_up_note": "x quantisation + grouped GEMM",
            "gate_up_algorithmic_bytes": int(m1_bytes),
            "gate_up_traffic": committed_traffic(cfg.name, "gate_up_mxfp8"),
            "gate_up_GB/s": round(m1_gbs, 1), "gate_up_hbm_frac": round(m1_gbs / PEAK_HBM_GBS, 4),
            "gate_up_TFLOP/s": round(m1_tfs, 2),
            "gate_up_fp8_frac": round(m1_tfs / PEAK_FP8_TFLOPS, 4),
            "gate_up_min_ms_at_peaks": round(max(m1_bytes / (PEAK_HBM_GBS * 1e9),
                                                 g1_flops / (PEAK_FP8_TFLOPS * 1e12)) * 1e3, 4),
            "down_ms": round(m2_ms, 4),
            "down_TFLOP/s": round(g2_flops / (m2_ms * 1e-3) / 1e12, 2),
        }
        del w1q, w2q, w1sq, w2sq, ws_mx, hq, hsq

    # One GPU's share of the layer under 8-way expert parallelism: 32 of the
    # experts, each receiving the rows that 8 GPUs' batches (8 x T tokens,
    # top-k, balanced) send it -- k*T*8/N rows -- plus the shared expert on
    # the local T tokens.  The received rows are the local x rows (synthetic,
    # balanced routing: token t -> experts (t + (N/8/k) j) mod N/8), so the
    # expert kernels run at the per-GPU shape without any exchange.
    ep_share = None
    if "ep" not in skip and cfg.n_experts % 8 == 0 and cfg.n_experts // 8 >= k and \
            (cfg.n_experts // 8) % k == 0 and cfg.dtype == "bf16":
        n_loc = cfg.n_experts // 8
        ep_shape = shape.replace(n_experts=n_loc, n_groups=1, topk_groups=1)
        ws_ep = moe.workspace(ep_shape, dev)
        stride = n_loc // k
        tt = torch.arange(T, device=dev, dtype=torch.int32)[:, None]
        jj = torch.arange(k, device=dev, dtype=torch.int32)[None, :]
        ti_ep = ((tt + stride * jj) % n_loc).to(torch.int32).contiguous()
        cn_ep = torch.empty((n_loc,), dtype=torch.int32, device=dev)
        of_ep = torch.empty((n_loc + 1,), dtype=torch.int32, device=dev)
        moe.moe_dispatch(ep_shape, ti_ep, cn_ep, of_ep, sl, pm, nkd, ws_ep)
        w1_ep, w2_ep = inp.w1[:n_loc], inp.w2[:n_loc]
        moe.moe_expert_plan(ep_shape, of_ep, ws_ep)
        ep_ms = timed(lambda: moe.moe_expert_ffn(ep_shape, inp.x, pm, None, w1_ep, w2_ep,
                                                 inp.w1_shared, inp.w2_shared, yp, ysh, ws_ep),
                      args.stage_iters)
        ep_flops = 6.0 * d * cfg.d_ff * T * k + 6.0 * T * d * cfg.d_ff_shared
        ep_share = {"experts": n_loc, "rows_per_expert": T * k // n_loc,
                    "expert_ffn_ms": round(ep_ms, 4),
                    "TFLOP/s": round(ep_flops / (ep_ms * 1e-3) / 1e12, 2),
                    "mfma_frac": round(ep_flops / (ep_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "note": "both expert projections (+ shared expert) in one moe_expert_ffn "
                            "call; no all-to-all"}
        del ws_ep

    # LatentMoE on the same workload at latent width d/4: routing on x, the
    # experts (d_ff unchanged) on z = x W_down^T, y = y_lat W_up^T + shared
    latent = None
    l = d // 4
    if "latent" not in skip and cfg.dtype in ("bf16", "f32") and \
            l % (64 if cfg.dtype == "bf16" else 32) == 0:
        li = W.make_latent_inputs(cfg, l, seed=0, device=dev)
        ws_l = moe.latent_workspace(shape, l, dev)
        y_l = torch.empty_like(out["y"])

        def lat_step():
            moe.moe_forward_latent(shape, l, inp.x, inp.w_router, inp.logit_add, inp.bias,
                                   li.w_down, li.w_up, li.w1, li.w2, inp.w1_shared,
                                   inp.w2_shared, y_l, None, None, None, None, None, None,
                                   None, ws_l)
        for _ in range(2):
            lat_step()
        g_l = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_l):
            lat_step()
        for _ in range(2):
            g_l.replay()
        l_ms = tm.back_to_back(g_l.replay, args.steps)
        del g_l
        l_flops = (2.0 * T * d * N + 4.0 * T * d * l + 6.0 * l * cfg.d_ff * n_kept
                   + 6.0 * T * d * cfg.d_ff_shared)
        latent = {"d_latent": l, "ms_per_step": round(l_ms, 4),
                  "tokens/s": round(T / (l_ms * 1e-3), 1),
                  "tflops": round(l_flops / (l_ms * 1e-3) / 1e12, 2),
                  "expert_weight_bytes": int(li.w1.numel() + li.w2.numel()) * li.w1.element_size()}
        del li, ws_l, y_l

    res = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "launch": "hip graph replay" if graph_ms <= eager_ms else "eager stream launches",
        "eager_ms_per_step": round(eager_ms, 4),
        "graph_ms_per_step": round(graph_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": {"workload": workload_name(cfg), "global_batch": T,
                   "parallelism": "single GPU"},
        "ms_median": q["median"],
        "ms_p10": q["p10"],
        "ms_p90": q["p90"],
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "n_kept": n_kept,
        "layer_roofline": layer_roofline(cfg, touched, n_kept, ms),
        "roofline": roofline,
        "gemm2": gemm2,
        "telemetry": telemetry,
        "expert_choice": expert_choice,
        "mxfp8": mxfp8,
        "latent": latent,
        "ep8_share": ep_share,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample_tokens
                                           or CPU_SAMPLE.get(cfg.name, 64))
    return res


if __name__ == "__main__":
    main()
