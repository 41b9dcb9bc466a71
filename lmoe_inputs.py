"""Seeded synthetic inputs for the LatentMoE layer (shared by the tests, the
benchmark and the smoke check).

This module draws random tensors and nothing else: it holds none of the
layer's arithmetic.  Both the HIP library and the CPU oracle consume what it
produces; the HIP side gets device tensors, the oracle gets host copies of
the very same values (bfloat16 bit patterns as uint16, float32 as float32).

Recipe (each tensor has its own generator, seeded ``seed + i`` in the order
x, W1, Wg, beta, Wup, Wdn, W2, Wsu, Wsd, and gamma, the weight of the block's
pre-norm, which only the block-boundary runs use):

* x ~ N(0, 1); every weight ~ N(0, 0.02^2); beta ~ N(0, 0.01^2)
  (the second parameter is a variance: standard deviations 1, 0.02, 0.01);
* draws are float32, then rounded to bfloat16 (round-to-nearest-even) for
  x and every weight except the router gate and its correction bias, which
  stay float32 (the pages keep the gate and the bias in fp32);
* gamma = 1 + N(0, 0.1^2) per hidden unit, rounded to bfloat16;
* the "skewed" workload replaces beta by a bias that makes expert
  popularity follow a Zipf law (see ``zipf_bias``).

Values depend on the device the generators run on (CPU and GPU generators
differ); a test draws on one device and hands the same values to both sides.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, replace
from statistics import NormalDist

import numpy as np
import torch


@dataclass(frozen=True)
class LayerShape:
    hidden_size: int
    moe_latent_size: int
    n_routed_experts: int
    num_experts_per_tok: int
    moe_intermediate_size: int
    moe_shared_expert_intermediate_size: int
    routed_scaling_factor: float = 5.0
    n_group: int = 1
    topk_group: int = 1


@dataclass(frozen=True)
class Workload:
    name: str
    shape: LayerShape
    tokens: int
    seed: int = 0
    x_std: float = 1.0
    w_std: float = 0.02
    bias_std: float = 0.01
    bias_recipe: str = "normal"   # "normal" | "zipf"
    zipf_s: float = 1.2
    zipf_dead_frac: float = 0.1


FULL = LayerShape(8192, 2048, 512, 22, 5120, 10240, 5.0)
TINY = LayerShape(256, 64, 16, 4, 128, 512, 5.0)

WORKLOADS = {
    "tiny": Workload("tiny", TINY, 64),
    "decode": Workload("decode", FULL, 32),
    "mtp_verify": Workload("mtp_verify", FULL, 192),
    "prefill": Workload("prefill", FULL, 8192),
    "skewed": Workload("skewed", FULL, 8192, bias_recipe="zipf"),
    # the same decode batch with group-limited routing: 8 groups of 64 experts, 4 kept
    "decode_grouped": Workload("decode_grouped", replace(FULL, n_group=8, topk_group=4), 32),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **overrides) if overrides else w


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal_bf16(shape, std, gen, device, chunk_rows=None) -> torch.Tensor:
    """N(0, std^2) drawn in float32 and rounded to bfloat16, drawn in
    fixed-size chunks along dim 0 so large tensors need little scratch."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    rows = shape[0]
    step = rows if chunk_rows is None else max(1, chunk_rows)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        tmp = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen,
                          device=device, dtype=torch.float32)
        out[r0:r1] = (tmp * std).to(torch.bfloat16)
    return out


def zipf_bias(shape: LayerShape, seed: int, s: float = 1.2,
              dead_frac: float = 0.1, logit_std: float | None = None,
              x_std: float = 1.0, w_std: float = 0.02) -> np.ndarray:
    """Correction bias that makes expert popularity follow Zipf(s).

    Experts get Zipf ranks by a seeded random permutation.  The
    ``round(dead_frac * E)`` lowest ranks get bias -2: a sigmoid score lies
    in (0, 1), so they can never beat a live expert (live biases lie in
    (-1, 0]) and receive no tokens.  Live rank r targets selection
    probability p_r = min(1, a r^-s), with a chosen so that sum p_r = K.

    The bias is chosen from a model of the logits, not from the data: each
    logit is taken as N(0, sigma^2) with sigma the standard deviation the
    recipe implies (x_std * sqrt(D) * w_std * sqrt(R) * w_std), and a token
    is taken to keep the experts whose biased score exceeds a common
    threshold.  Expert e is then kept when its logit exceeds
    q_e = sigma * Phi^-1(1 - p_e), which the bias -1/(1 + e^-q_e) turns into
    a threshold of 0 on the biased score; the K-th largest biased score sits
    near 0 because the p_r sum to K.  The achieved histogram is measured,
    not assumed."""
    e = shape.n_routed_experts
    k = shape.num_experts_per_tok
    if logit_std is None:
        logit_std = (x_std * math.sqrt(shape.hidden_size) * w_std
                     * math.sqrt(shape.moe_latent_size) * w_std)
    rng = np.random.default_rng(seed)
    order = rng.permutation(e)           # order[rank-1] = expert id
    n_dead = int(round(dead_frac * e))
    n_live = e - n_dead
    ranks = np.arange(1, n_live + 1, dtype=np.float64)

    def total(a):
        return np.minimum(1.0, a * ranks ** (-s)).sum()

    lo, hi = 0.0, float(k) * 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if total(mid) < k:
            lo = mid
        else:
            hi = mid
    p = np.minimum(1.0, hi * ranks ** (-s))
    p = np.clip(p, 1e-6, 1.0 - 1e-6)
    nd = NormalDist()
    q = np.array([logit_std * nd.inv_cdf(1.0 - pi) for pi in p])
    bias = np.full(e, -2.0, dtype=np.float64)
    bias[order[:n_live]] = -1.0 / (1.0 + np.exp(-q))
    return bias.astype(np.float32)


@dataclass
class LayerInputs:
    """Device tensors of one workload (bf16 unless noted)."""
    workload: Workload
    x: torch.Tensor             # [T, D]
    fc1_latent: torch.Tensor    # [R, D]
    router: torch.Tensor        # [E, R] float32
    router_bias: torch.Tensor   # [E] float32
    expert_up: torch.Tensor     # [E, F, R]
    expert_down: torch.Tensor   # [E, R, F]
    fc2_latent: torch.Tensor    # [D, R]
    shared_up: torch.Tensor     # [S, D]
    shared_down: torch.Tensor   # [D, S]


def make_weights(wl: Workload, device="cpu") -> dict:
    sh = wl.shape
    D, R, E = sh.hidden_size, sh.moe_latent_size, sh.n_routed_experts
    F, S = sh.moe_intermediate_size, sh.moe_shared_expert_intermediate_size
    seed, ws = wl.seed, wl.w_std
    w = {}
    w["fc1_latent"] = _normal_bf16((R, D), ws, _gen(device, seed + 1), device)
    w["router"] = (torch.randn((E, R), generator=_gen(device, seed + 2),
                               device=device, dtype=torch.float32) * ws)
    if wl.bias_recipe == "zipf":
        w["router_bias"] = torch.from_numpy(
            zipf_bias(sh, seed + 3, wl.zipf_s, wl.zipf_dead_frac,
                      x_std=wl.x_std, w_std=ws)).to(device)
    else:
        w["router_bias"] = (torch.randn((E,), generator=_gen(device, seed + 3),
                                        device=device, dtype=torch.float32)
                            * wl.bias_std)
    w["expert_up"] = _normal_bf16((E, F, R), ws, _gen(device, seed + 4), device,
                                  chunk_rows=8)
    w["expert_down"] = _normal_bf16((E, R, F), ws, _gen(device, seed + 5), device,
                                    chunk_rows=8)
    w["fc2_latent"] = _normal_bf16((D, R), ws, _gen(device, seed + 6), device)
    w["shared_up"] = _normal_bf16((S, D), ws, _gen(device, seed + 7), device,
                                  chunk_rows=2048)
    w["shared_down"] = _normal_bf16((D, S), ws, _gen(device, seed + 8), device,
                                    chunk_rows=2048)
    return w


def make_norm_weight(wl: Workload, device="cpu") -> torch.Tensor:
    """gamma [D] bf16: the weight of the block's pre-norm RMSNorm."""
    g = torch.randn((wl.shape.hidden_size,), generator=_gen(device, wl.seed + 9),
                    device=device, dtype=torch.float32)
    return (1.0 + 0.1 * g).to(torch.bfloat16)


def make_x(wl: Workload, device="cpu", tokens: int | None = None) -> torch.Tensor:
    t = wl.tokens if tokens is None else tokens
    return _normal_bf16((t, wl.shape.hidden_size), wl.x_std,
                        _gen(device, wl.seed + 0), device, chunk_rows=4096)


def make_inputs(wl: Workload, device="cpu", weights: dict | None = None,
                tokens: int | None = None) -> LayerInputs:
    w = make_weights(wl, device) if weights is None else weights
    return LayerInputs(workload=wl, x=make_x(wl, device, tokens), **w)


# ---- host views for the oracle (bit copies, no arithmetic) -----------------

def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bfloat16 tensor, copied to the host."""
    assert t.dtype == torch.bfloat16
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class ExpertBits:
    """``obj[e]`` -> uint16 bits of expert e's weight matrix, copied to the
    host on demand (so a full-shape check never holds every expert at once)."""

    def __init__(self, t: torch.Tensor):
        self.t = t

    def __getitem__(self, e: int) -> np.ndarray:
        return bf16_bits(self.t[int(e)])

    def __len__(self):
        return self.t.shape[0]


class HostWeights:
    """Attribute view of a LayerInputs in the oracle's input form."""

    def __init__(self, li: LayerInputs, eager_experts: bool = False):
        self.fc1_latent = bf16_bits(li.fc1_latent)
        self.router = li.router.detach().cpu().numpy().astype(np.float32)
        self.router_bias = li.router_bias.detach().cpu().numpy().astype(np.float32)
        if eager_experts:
            self.expert_up = bf16_bits(li.expert_up)
            self.expert_down = bf16_bits(li.expert_down)
        else:
            self.expert_up = ExpertBits(li.expert_up)
            self.expert_down = ExpertBits(li.expert_down)
        self.fc2_latent = bf16_bits(li.fc2_latent)
        self.shared_up = bf16_bits(li.shared_up)
        self.shared_down = bf16_bits(li.shared_down)
