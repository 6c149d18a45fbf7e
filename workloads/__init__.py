"""Seeded synthetic workloads for the sparse MoE FFN layer.

This module only *draws inputs*: shapes, random tensors and the per-token
logit offsets that the workloads prescribe.  It holds none of the layer's
arithmetic (no routing, no scoring, no expert math), so that both the fp64
oracle and the HIP path can be fed from it without sharing any code.

Every tensor is drawn from its own ``torch.Generator`` whose seed is a hash of
``(seed, workload, tensor tag, expert)``; regenerating one expert's weights
therefore never requires drawing the others.  Floating-point tensors are drawn
as float32 standard normals, scaled by ``1/sqrt(fan_in)`` and, for bf16
workloads, rounded to bf16 (round to nearest even) by ``Tensor.to``.

Workload recipe (shapes as given by the five layer configurations):
  tiny     T=64    d=128  N=8   k=2 d_ff=256   softmax+renorm, cf=1.25 drop, fp32
  mixtral  T=4096  d=4096 N=8   k=2 d_ff=14336 softmax+renorm, dropless, bf16
  dsv3     T=8192  d=7168 N=256 k=8 d_ff=2048  sigmoid + selection bias
                                               b~U(-0.1,0.1), group top-4 of 8,
                                               + 1 shared expert (d_ff 2048)
  decode   T=64    d=2048 N=128 k=8 d_ff=768   softmax+renorm, Zipf(1.1)
                                               logit offset -1.1*ln(i+1)
  switch   T=16384 d=1024 N=64  k=1 d_ff=4096  softmax (+ jitter N(0,0.01^2)
                                               on the logits), cf=1.0 drop
x ~ N(0,1); router W ~ N(0,1/d) fp32; W1 ~ N(0,1/d); W2 ~ N(0,1/d_ff).
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import torch

SOFTMAX = "softmax"
SIGMOID = "sigmoid"

# capacity rules: "tokens" = floor(cf * T / N)   (llm-compass MoE page,
# "capacity factor and expert parallelism" section);
# "assignments" = max(int(cf * k * T / N), k)   (deepseekmodel.com MoE
# engineering article, TopKRouter in the routing-math section).
CAP_TOKENS = "tokens"
CAP_ASSIGNMENTS = "assignments"


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    d_ff_shared: int = 0
    score_fn: str = SOFTMAX
    renormalize: bool = True
    n_groups: int = 1
    topk_groups: int = 1
    capacity_factor: float = 0.0  # <= 0: dropless
    capacity_rule: str = CAP_TOKENS
    dtype: str = "bf16"  # activations and expert weights; router is fp32
    # input recipe
    bias_range: float = 0.0  # b ~ U(-r, r); 0 and not bias_zero: no bias
    bias_zero: bool = False  # pass an all-zero bias tensor (balancing runs)
    zipf_s: float = 0.0  # logit offset -s*ln(i+1)
    jitter_std: float = 0.0  # additive Gaussian logit noise

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    @property
    def has_bias(self) -> bool:
        return self.bias_range > 0 or self.bias_zero

    @property
    def has_logit_add(self) -> bool:
        return self.zipf_s > 0 or self.jitter_std > 0


CONFIGS = {
    "tiny": LayerConfig("tiny", 64, 128, 8, 2, 256, capacity_factor=1.25,
                        dtype="f32"),
    "mixtral": LayerConfig("mixtral", 4096, 4096, 8, 2, 14336),
    "dsv3": LayerConfig("dsv3", 8192, 7168, 256, 8, 2048, d_ff_shared=2048,
                        score_fn=SIGMOID, n_groups=8, topk_groups=4,
                        bias_range=0.1),
    "decode": LayerConfig("decode", 64, 2048, 128, 8, 768, zipf_s=1.1),
    "switch": LayerConfig("switch", 16384, 1024, 64, 1, 4096,
                          capacity_factor=1.0, jitter_std=0.01,
                          bias_zero=True),
}
CONFIG_ORDER = ["tiny", "mixtral", "dsv3", "decode", "switch"]


def _seed(*parts) -> int:
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def torch_dtype(cfg: LayerConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def _normal(shape, scale, dtype, device, *parts) -> torch.Tensor:
    t = torch.randn(shape, generator=_gen(device, *parts), device=device,
                    dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(dtype)


@dataclasses.dataclass
class LayerInputs:
    cfg: LayerConfig
    x: torch.Tensor  # [T, d]
    w_router: torch.Tensor  # [N, d] fp32
    w1: torch.Tensor  # [N, 2*d_ff, d]  gate rows then up rows
    w2: torch.Tensor  # [N, d, d_ff]
    w1_shared: Optional[torch.Tensor] = None  # [2*d_ff_s, d]
    w2_shared: Optional[torch.Tensor] = None  # [d, d_ff_s]
    bias: Optional[torch.Tensor] = None  # [N] fp32
    logit_add: Optional[torch.Tensor] = None  # [T, N] fp32


def make_x(cfg: LayerConfig, seed: int = 0, device="cpu", T: Optional[int] = None):
    T = cfg.T if T is None else T
    return _normal((T, cfg.d_model), 1.0, torch_dtype(cfg), device,
                   seed, cfg.name, "x", T)


def make_expert_weights(cfg: LayerConfig, e: int, seed: int = 0, device="cpu"):
    """(W1_e [2*d_ff, d], W2_e [d, d_ff]) for routed expert e."""
    dt = torch_dtype(cfg)
    d, f = cfg.d_model, cfg.d_ff
    w1 = _normal((2 * f, d), 1.0 / math.sqrt(d), dt, device, seed, cfg.name, "w1", e)
    w2 = _normal((d, f), 1.0 / math.sqrt(f), dt, device, seed, cfg.name, "w2", e)
    return w1, w2


def make_inputs(cfg: LayerConfig, seed: int = 0, device="cpu",
                T: Optional[int] = None) -> LayerInputs:
    """Draw every input of one layer forward.  ``T`` overrides the token count
    (token rows are drawn from a T-specific stream; weights do not depend on T)."""
    T = cfg.T if T is None else T
    dt = torch_dtype(cfg)
    N, d, f = cfg.n_experts, cfg.d_model, cfg.d_ff
    x = make_x(cfg, seed, device, T)
    w_router = _normal((N, d), 1.0 / math.sqrt(d), torch.float32, device,
                       seed, cfg.name, "w_router")
    w1 = torch.empty((N, 2 * f, d), dtype=dt, device=device)
    w2 = torch.empty((N, d, f), dtype=dt, device=device)
    for e in range(N):
        a, b = make_expert_weights(cfg, e, seed, device)
        w1[e].copy_(a)
        w2[e].copy_(b)
        del a, b
    inp = LayerInputs(cfg, x, w_router, w1, w2)
    if cfg.d_ff_shared > 0:
        fs = cfg.d_ff_shared
        inp.w1_shared = _normal((2 * fs, d), 1.0 / math.sqrt(d), dt, device,
                                seed, cfg.name, "w1_shared")
        inp.w2_shared = _normal((d, fs), 1.0 / math.sqrt(fs), dt, device,
                                seed, cfg.name, "w2_shared")
    if cfg.bias_range > 0:
        u = torch.rand((N,), generator=_gen(device, seed, cfg.name, "bias"),
                       device=device, dtype=torch.float32)
        inp.bias = (u * 2.0 - 1.0) * cfg.bias_range
    elif cfg.bias_zero:
        inp.bias = torch.zeros((N,), dtype=torch.float32, device=device)
    if cfg.has_logit_add:
        la = torch.zeros((T, N), dtype=torch.float32, device=device)
        if cfg.zipf_s > 0:
            # expert i has Zipf rank i+1: softmax of this offset alone is Zipf(s)
            ranks = torch.arange(1, N + 1, dtype=torch.float64, device=device)
            la += (-cfg.zipf_s * torch.log(ranks)).to(torch.float32)[None, :]
        if cfg.jitter_std > 0:
            la += _normal((T, N), cfg.jitter_std, torch.float32, device,
                          seed, cfg.name, "jitter", T)
        inp.logit_add = la
    return inp


@dataclasses.dataclass
class LatentInputs:
    base: LayerInputs        # x, router, bias, logit offsets, shared expert (full width)
    d_latent: int
    w_down: torch.Tensor     # [d_latent, d]
    w_up: torch.Tensor       # [d, d_latent]
    w1: torch.Tensor         # [N, 2*d_ff, d_latent]
    w2: torch.Tensor         # [N, d_latent, d_ff]


def make_latent_inputs(cfg: LayerConfig, d_latent: int, seed: int = 0, device="cpu",
                       T: Optional[int] = None) -> LatentInputs:
    """Inputs of a LatentMoE layer of the same workload: the base layer's
    tokens, router, bias, logit offsets and shared expert, plus the two
    projections and routed experts of latent width d_latent (normals scaled
    by 1/sqrt(fan_in), like every other weight)."""
    T = cfg.T if T is None else T
    dt = torch_dtype(cfg)
    N, d, f, l = cfg.n_experts, cfg.d_model, cfg.d_ff, d_latent
    x = make_x(cfg, seed, device, T)
    w_router = _normal((N, d), 1.0 / math.sqrt(d), torch.float32, device,
                       seed, cfg.name, "w_router")
    inp = LayerInputs(cfg, x, w_router, torch.empty(0, device=device),
                      torch.empty(0, device=device))
    if cfg.d_ff_shared > 0:
        fs = cfg.d_ff_shared
        inp.w1_shared = _normal((2 * fs, d), 1.0 / math.sqrt(d), dt, device,
                                seed, cfg.name, "w1_shared")
        inp.w2_shared = _normal((d, fs), 1.0 / math.sqrt(fs), dt, device,
                                seed, cfg.name, "w2_shared")
    if cfg.bias_range > 0:
        u = torch.rand((N,), generator=_gen(device, seed, cfg.name, "bias"),
                       device=device, dtype=torch.float32)
        inp.bias = (u * 2.0 - 1.0) * cfg.bias_range
    elif cfg.bias_zero:
        inp.bias = torch.zeros((N,), dtype=torch.float32, device=device)
    if cfg.has_logit_add:
        la = torch.zeros((T, N), dtype=torch.float32, device=device)
        if cfg.zipf_s > 0:
            ranks = torch.arange(1, N + 1, dtype=torch.float64, device=device)
            la += (-cfg.zipf_s * torch.log(ranks)).to(torch.float32)[None, :]
        if cfg.jitter_std > 0:
            la += _normal((T, N), cfg.jitter_std, torch.float32, device,
                          seed, cfg.name, "jitter", T)
        inp.logit_add = la
    w_down = _normal((l, d), 1.0 / math.sqrt(d), dt, device, seed, cfg.name, "w_down", l)
    w_up = _normal((d, l), 1.0 / math.sqrt(l), dt, device, seed, cfg.name, "w_up", l)
    w1 = torch.empty((N, 2 * f, l), dtype=dt, device=device)
    w2 = torch.empty((N, l, f), dtype=dt, device=device)
    for e in range(N):
        w1[e].copy_(_normal((2 * f, l), 1.0 / math.sqrt(l), dt, device, seed, cfg.name,
                            "w1_latent", l, e))
        w2[e].copy_(_normal((l, f), 1.0 / math.sqrt(f), dt, device, seed, cfg.name,
                            "w2_latent", l, e))
    return LatentInputs(inp, l, w_down, w_up, w1, w2)


def to_f64(t: torch.Tensor):
    """Exact upcast of a (bf16 / fp32) tensor to a float64 NumPy array on host."""
    return t.detach().to("cpu", torch.float64).numpy()


def to_f32(t: torch.Tensor):
    return t.detach().to("cpu", torch.float32).numpy()
