"""Plain, slow CPU oracle of the LatentMoE layer forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): the product path never
imports this module.

Definition followed (page "Nemotron 3 Ultra 架构深度拆解报告", CH5 §5.6,
"7 步数据流", Steps 1-7, with the router moved onto the latent as the
same page's summary (CH0) and the Super overview page ("NVIDIA Nemotron 3
Super 技术解读", §2.2) describe it):

    z      = x W1^T                                   fc1_latent_proj  (Step 5)
    l      = z Wg^T                     (float32)     router gate      (Step 1)
    s      = sigmoid(l)                 (float32)                      (Step 2)
    b      = s + beta                   (float32)     selection only   (Step 2)
    I_t    = the K largest b_t among the kept groups' experts         (Step 3, §5.5)
    w_t    = rho * s_t[I_t] / (sum s_t[I_t] + 1e-20)                   (Step 4)
    E_e(u) = relu(u Wup[e]^T)^2 Wdn[e]^T  (non-gated MLP)              (Step 6, §5.1)
    r_t    = sum_k w_t,k E_{I_t,k}(z_t)                                (Step 6)
    y_t    = r_t W2^T + relu(x_t Wsu^T)^2 Wsd^T                        (Step 7)

Weights are stored out x in, so ``linear(u, W) = u @ W.T`` (§5.1: expert
tensors are (num_experts, out_dim, in_dim)); no layer has a bias (§2.3.4).

Readings taken where the pages are silent or disagree:

* the router reads the float32 latent z (the gate upcasts its input to fp32,
  Step 1), not a bf16-rounded copy;
* relu^2(u) = max(u, 0)^2 for the experts and the shared expert;
* ties between equal biased scores go to the lower expert index, and the K
  selected experts are reported in ascending expert id (``topk`` is called
  with ``sorted=False``, so the order carries no meaning);
* the 1e-20 is added to the float32 sum before dividing, then the quotient is
  multiplied by rho (Step 4 order);
* routing groups (§5.5, used when n_group > 1): contiguous groups of
  E / n_group experts, a group's score is the float32 sum of its two largest
  biased scores, equal group scores go to the lower group index, and experts
  of the dropped groups are excluded from the top-K (not given a score of
  zero); with n_group = 1 the group step is a no-op.
* the block around the layer (``block_forward``; the same page, CH9 §9.3: each
  block applies a pre-norm RMSNorm, then the mixer, then adds the residual):
  RMSNorm(h) = gamma * h / sqrt(mean(h^2) + eps) with eps = 1e-5 unless
  given (the pages give no eps); the product gamma * h is rounded once to
  bfloat16 (it is the GEMM operand) and the per-token factor
  1 / sqrt(mean(h^2) + eps) is kept exact, so the normalised input is
  r_t * bf16(gamma * h_t); the block output is h + layer(RMSNorm(h)).

Parity pins (tests/test_oracle_pins.py): a hand-derived micro example
(tests/golden/worked_example_micro.json), brute-force subset enumeration for
the top-K, closed-form sigmoid values, exact integer GEMMs, the dense
"every expert on every token" formulation, and the invariants sum(w) = rho,
K = 1, K = E, x = 0, Wup = 0, identical experts, token-order equivariance and
the page's parameter/FLOP accounting; the MXFP4 quantiser by hand-worked
blocks (ties, saturation, zero blocks), exact round trips and its error
bound; the pre-norm by hand-worked rounding cases, the unit RMS of its
output, power-of-two scale invariance, and the block forward against the
plain forward on inputs that the norm maps exactly.  No function here is
unpinned.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32 = np.float32
F64 = np.float64


@dataclass(frozen=True)
class OracleConfig:
    """Layer sizes, named after the model's config keys (page
    "Nemotron-3-Labs-Ultra-Math-SFT" article, 核心配置速查表)."""

    hidden_size: int
    moe_latent_size: int
    n_routed_experts: int
    num_experts_per_tok: int
    moe_intermediate_size: int
    moe_shared_expert_intermediate_size: int
    routed_scaling_factor: float = 5.0
    n_group: int = 1
    topk_group: int = 1


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns (uint16) as float64.

    A bfloat16 is the upper 16 bits of an IEEE float32, so the value is the
    float32 whose high half is ``bits`` and whose low half is zero."""
    u = np.asarray(bits, dtype=np.uint16)
    return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(F64)


def f32_to_bf16_bits(v) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values, rounded to nearest
    with ties to the even pattern (finite inputs)."""
    u = np.asarray(v, F32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def rms_prenorm(h_bits, gamma_bits, eps: float = 1e-5):
    """The block's pre-norm RMSNorm (page "Nemotron 3 Ultra 架构深度拆解报告",
    CH9 §9.3: NemotronHRMSNorm before the mixer; one weight per hidden unit,
    §2.3.6), split into the GEMM operand and a per-token factor:

        xt_t = bf16(gamma * h_t)      the float32 product, rounded once
        r_t  = 1 / sqrt(mean_i h_t,i^2 + eps)        (float64)

    so that RMSNorm(h)_t = r_t * xt_t.  Returns (xt bits uint16 [T, D],
    r float64 [T])."""
    h = bf16_bits_to_f64(h_bits)
    g = bf16_bits_to_f64(gamma_bits)
    xt = f32_to_bf16_bits((h * g[None, :]).astype(F32))
    r = 1.0 / np.sqrt((h * h).mean(axis=1) + float(eps))
    return xt, r


# Magnitudes of the E2M1 (FP4) element format, by code 0..7 (page "Nemotron 3
# Ultra 架构深度拆解报告", CH8 §8.1, E2M1 格式: 0, ±0.5, ±1, ±1.5, ±2, ±3, ±4, ±6);
# code bit 3 is the sign.
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MX_BLOCK = 32


def mxfp4_quantize(w_bits):
    """Block-scaled FP4 (MXFP4) quantiser of a bf16 matrix [..., K] along its
    last (input) axis.  The pages fix the element format (E2M1, CH8 §8.1)
    but give two different block layouts, so the layout is defined here:
    blocks of 32 consecutive k, each with a power-of-two scale
    X = 2^e, e = floor(log2 max|w|) - 2 clipped to [-127, 127] (-127 for an
    all-zero block; 2 is the E2M1 exponent of 6), stored as the byte e + 127;
    each element is |w| / X rounded to the nearest E2M1 magnitude, ties to
    the code with a zero mantissa bit (even code), values above 6 clamped to
    6, with the sign of w unless the magnitude rounds to 0.  Codes pack two
    per byte, element 2i in the low nibble.  Returns (codes uint8
    [..., K/2], scales uint8 [..., K/32])."""
    w = bf16_bits_to_f64(w_bits)
    K = w.shape[-1]
    blocks = w.reshape(*w.shape[:-1], K // MX_BLOCK, MX_BLOCK)
    amax = np.abs(blocks).max(-1)
    _, ex = np.frexp(amax)                        # amax = m 2^ex, 0.5 <= m < 1
    e = np.where(amax > 0, ex - 1 - 2, -127).clip(-127, 127)
    a = np.abs(blocks) / np.ldexp(1.0, e)[..., None]
    dist = np.abs(a[..., None] - E2M1_MAGNITUDES)  # [..., 32, 8]
    nearest = dist == dist.min(-1, keepdims=True)
    even = nearest & (np.arange(8) % 2 == 0)
    mag = np.where(even.any(-1), even.argmax(-1), nearest.argmax(-1))
    code = mag + 8 * ((blocks < 0) & (mag > 0))
    flat = code.reshape(*w.shape[:-1], K)
    codes = (flat[..., 0::2] | (flat[..., 1::2] << 4)).astype(np.uint8)
    return codes, (e + 127).astype(np.uint8)


def mxfp4_dequantize(codes, scales) -> np.ndarray:
    """Values of MXFP4 codes (``mxfp4_quantize``'s layout), float64 [..., K]."""
    codes = np.asarray(codes, np.uint8)
    c = np.stack([codes & 15, codes >> 4], -1).reshape(*codes.shape[:-1], codes.shape[-1] * 2)
    mag = E2M1_MAGNITUDES[c & 7]
    val = np.where(c & 8, -mag, mag)
    K = c.shape[-1]
    x = np.ldexp(1.0, np.asarray(scales).astype(np.int64) - 127)
    return (val.reshape(*c.shape[:-1], K // MX_BLOCK, MX_BLOCK) * x[..., None]).reshape(val.shape)


def expert_matrix(a) -> np.ndarray:
    """An expert weight as float64: bf16 bit patterns (uint16) are upcast,
    float arrays (e.g. dequantised MXFP4 weights) are taken as they are."""
    a = np.asarray(a)
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(F64)


def latent_projection(x: np.ndarray, W1: np.ndarray) -> np.ndarray:
    """fc1_latent_proj: z = x W1^T, float64 (Step 5)."""
    return np.asarray(x, F64) @ np.asarray(W1, F64).T


def router_scores(z32: np.ndarray, Wg: np.ndarray):
    """Router gate and sigmoid (Steps 1-2), in float32 as the page fixes.

    The logits are the float64 dot products of the float32 latent with the
    float32 gate rows, rounded once to float32.  The sigmoid 1/(1+e^-l) is
    evaluated in float64 from that float32 logit and rounded once."""
    z32 = np.asarray(z32, F32)
    Wg = np.asarray(Wg, F32)
    logits = (z32.astype(F64) @ Wg.astype(F64).T).astype(F32)
    s = (1.0 / (1.0 + np.exp(-logits.astype(F64)))).astype(F32)
    return logits, s


def select_groups(b: np.ndarray, n_group: int, topk_group: int):
    """Group-limited routing, group step (page "Nemotron 3 Ultra 架构深度拆解
    报告", CH5 §5.5 items 1-2 and the group-score line of Step 3).

    The E experts are split into ``n_group`` contiguous groups of E/n_group;
    a group's score is the sum of its two largest biased scores (float32
    addition); the ``topk_group`` groups with the largest scores are kept,
    equal scores ranked by group index ascending.  Returns the mask of
    experts in kept groups [T, E] and the gap between the last kept and the
    first dropped group score (+inf if every group is kept)."""
    t, e = b.shape
    g = e // n_group
    bg = np.asarray(b, F32).reshape(t, n_group, g)
    top2 = -np.sort(-bg, axis=-1)[..., :2]
    gscore = (top2[..., 0] + top2[..., 1]).astype(F32)
    gids = np.broadcast_to(np.arange(n_group), gscore.shape)
    granked = np.lexsort((gids, -gscore), axis=-1)
    kept = np.zeros((t, n_group), bool)
    np.put_along_axis(kept, granked[:, :topk_group], True, axis=1)
    if topk_group < n_group:
        last = np.take_along_axis(gscore, granked[:, topk_group - 1:topk_group], 1)[:, 0]
        first_out = np.take_along_axis(gscore, granked[:, topk_group:topk_group + 1], 1)[:, 0]
        ggap = last.astype(F64) - first_out.astype(F64)
    else:
        ggap = np.full(t, np.inf)
    return np.repeat(kept, g, axis=1), ggap


def select_experts(s: np.ndarray, beta: np.ndarray, k: int, n_group: int = 1,
                   topk_group: int = 1):
    """Top-K selection on the biased score (Steps 2-3; §5.5 item 3).

    b = s + beta in float32.  For each token the experts of the kept groups
    (all experts when n_group = 1) are ranked by b descending, equal b ranked
    by expert index ascending; the first ``k`` are kept and returned in
    ascending expert id.  Experts of dropped groups cannot be selected.
    ``gap`` is the smaller of the group gap (``select_groups``) and the
    difference between the k-th and the (k+1)-th ranked biased scores among
    the eligible experts (+inf where there is no (k+1)-th), i.e. how close
    the token is to a different selection."""
    s = np.asarray(s, F32)
    b = (s + np.asarray(beta, F32)[None, :]).astype(F32)
    t, e = b.shape
    if n_group > 1:
        eligible, ggap = select_groups(b, n_group, topk_group)
    else:
        eligible, ggap = np.ones(b.shape, bool), np.full(t, np.inf)
    expert_ids = np.broadcast_to(np.arange(e), b.shape)
    ranked = np.lexsort((expert_ids, -b, ~eligible), axis=-1)
    idx = np.sort(ranked[:, :k], axis=1)
    n_eligible = eligible.sum(1)
    gap = np.full(t, np.inf)
    if k < e:
        bk = np.take_along_axis(b, ranked[:, k - 1:k], 1)[:, 0].astype(F64)
        bk1 = np.take_along_axis(b, ranked[:, k:k + 1], 1)[:, 0].astype(F64)
        gap = np.where(n_eligible > k, bk - bk1, np.inf)
    return idx, b, np.minimum(gap, ggap)


def renormalize(s: np.ndarray, idx: np.ndarray, rho: float) -> np.ndarray:
    """Routing weights (Step 4): gather the unbiased scores of the selected
    experts, divide by (their float32 sum + 1e-20), multiply by rho.

    The sum runs over the selected experts in ascending expert id, one
    float32 addition at a time."""
    sel = np.take_along_axis(np.asarray(s, F32), idx, 1).astype(F32)
    acc = np.zeros(sel.shape[0], F32)
    for j in range(sel.shape[1]):
        acc = (acc + sel[:, j]).astype(F32)
    denom = (acc + F32(1e-20)).astype(F32)
    return ((sel / denom[:, None]).astype(F32) * F32(rho)).astype(F32)


def expert_mlp(u: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """Non-gated relu^2 MLP, up -> act -> down (§5.1; Step 6), float64."""
    h = np.maximum(np.asarray(u, F64) @ np.asarray(w_up, F64).T, 0.0) ** 2
    return h @ np.asarray(w_down, F64).T


def routed_experts(z: np.ndarray, idx: np.ndarray, w: np.ndarray,
                   expert_up, expert_down) -> np.ndarray:
    """Step 6: loop over the experts that received tokens, run each on its
    tokens' latent rows, weight by the routing weight and add into the
    token's row.

    ``expert_up[e]`` / ``expert_down[e]`` return bfloat16 bit patterns
    (uint16) of shape [F, R] / [R, F], or float arrays (dequantised low-
    precision weights); they are upcast one expert at a time.
    Experts are visited in ascending id, so each token accumulates its
    contributions in ascending expert order."""
    z = np.asarray(z, F64)
    r = np.zeros_like(z)
    for e in np.unique(idx):
        tok, pos = np.nonzero(idx == e)
        o = expert_mlp(z[tok], expert_matrix(expert_up[int(e)]),
                       expert_matrix(expert_down[int(e)]))
        r[tok] += np.asarray(w, F64)[tok, pos][:, None] * o
    return r


def latent_up_projection(r: np.ndarray, W2: np.ndarray) -> np.ndarray:
    """fc2_latent_proj: r W2^T, float64 (Step 7)."""
    return np.asarray(r, F64) @ np.asarray(W2, F64).T


def shared_expert(x: np.ndarray, w_up: np.ndarray, w_down: np.ndarray) -> np.ndarray:
    """The shared expert on the un-projected input (Step 7), relu^2 MLP."""
    return expert_mlp(x, w_up, w_down)


def forward(x_bits, weights, cfg: OracleConfig, forced_idx=None) -> dict:
    """Whole layer forward for the rows of ``x_bits`` (bf16 bits, [T, D]).

    ``weights`` has attributes fc1_latent, router, router_bias, expert_up,
    expert_down, fc2_latent, shared_up, shared_down (bf16 bits except the
    float32 router and router_bias; expert_up/expert_down indexable by
    expert id).  ``forced_idx`` ([T, K] ascending ids) replaces the
    selection; it is used to re-evaluate tokens whose selection is within
    rounding of a tie.  Returns y (float64) and the intermediate values."""
    return layer(bf16_bits_to_f64(x_bits), weights, cfg, forced_idx)


def layer(x: np.ndarray, weights, cfg: OracleConfig, forced_idx=None) -> dict:
    """The layer (Steps 1-7) on a float64 input [T, D]; see ``forward``."""
    k = cfg.num_experts_per_tok
    x = np.asarray(x, F64)
    z = latent_projection(x, bf16_bits_to_f64(weights.fc1_latent))
    z32 = z.astype(F32)
    logits, s = router_scores(z32, weights.router)
    idx, b, gap = select_experts(s, weights.router_bias, k, cfg.n_group, cfg.topk_group)
    if forced_idx is not None:
        idx = np.sort(np.asarray(forced_idx, np.int64), axis=1)
    w = renormalize(s, idx, cfg.routed_scaling_factor)
    r = routed_experts(z, idx, w, weights.expert_up, weights.expert_down)
    y_routed = latent_up_projection(r, bf16_bits_to_f64(weights.fc2_latent))
    y_shared = shared_expert(x, bf16_bits_to_f64(weights.shared_up),
                             bf16_bits_to_f64(weights.shared_down))
    counts = np.bincount(idx.ravel(), minlength=cfg.n_routed_experts)
    return dict(y=y_routed + y_shared, y_routed=y_routed, y_shared=y_shared,
                z=z, z32=z32, logits=logits, s=s, b=b, idx=idx, w=w, gap=gap,
                r=r, counts=counts)


def block_forward(h_bits, gamma_bits, weights, cfg: OracleConfig, eps: float = 1e-5,
                  residual: bool = True, forced_idx=None) -> dict:
    """The layer inside its block (CH9 §9.3): pre-norm RMSNorm of the residual
    stream h (bf16 bits [T, D]) with weight ``gamma_bits`` (bf16 bits [D];
    None: no pre-norm, the layer reads h), the layer on the normalised rows
    r_t * bf16(gamma * h_t), and, if ``residual``, the residual added:
    y = h + layer(RMSNorm(h)).  Returns the layer's values with y replaced by
    the block output, plus xt and rnorm (``rms_prenorm``; absent without the
    pre-norm) and y_layer (the layer's own output)."""
    if gamma_bits is None:
        out = layer(bf16_bits_to_f64(h_bits), weights, cfg, forced_idx)
    else:
        xt, rn = rms_prenorm(h_bits, gamma_bits, eps)
        out = layer(rn[:, None] * bf16_bits_to_f64(xt), weights, cfg, forced_idx)
        out["xt"], out["rnorm"] = xt, rn
    out["y_layer"] = out["y"]
    if residual:
        out["y"] = bf16_bits_to_f64(h_bits) + out["y_layer"]
    return out
