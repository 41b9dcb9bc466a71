"""Pins of the CPU oracle to facts that do not come from the oracle itself:
a hand-derived worked example, brute-force enumeration, closed forms, exact
integer arithmetic, an independent (dense) formulation and invariants of
the definition.  CPU only."""

import itertools
import json
import math
import os
from types import SimpleNamespace

import numpy as np
import pytest
import torch

import lmoe_inputs as li
import oracle
from oracle import lmoe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def exact_bf16_bits(a) -> np.ndarray:
    """bf16 bit patterns of values that bfloat16 represents exactly."""
    f = np.asarray(a, np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bfloat16"
    return (u >> 16).astype(np.uint16)


def micro_case():
    g = json.load(open(os.path.join(GOLDEN, "worked_example_micro.json")))
    sh = g["shape"]
    cfg = O.OracleConfig(sh["hidden_size"], sh["moe_latent_size"], sh["n_routed_experts"],
                         sh["num_experts_per_tok"], sh["moe_intermediate_size"],
                         sh["moe_shared_expert_intermediate_size"], sh["routed_scaling_factor"])
    ln3 = math.log(3.0)
    w = SimpleNamespace(
        fc1_latent=exact_bf16_bits(g["fc1_latent"]),
        router=(np.asarray(g["router_ln3"], np.float64) * ln3).astype(np.float32),
        router_bias=np.asarray(g["router_bias"], np.float32),
        expert_up=exact_bf16_bits(g["expert_up"]),
        expert_down=exact_bf16_bits(g["expert_down"]),
        fc2_latent=exact_bf16_bits(g["fc2_latent"]),
        shared_up=exact_bf16_bits(g["shared_up"]),
        shared_down=exact_bf16_bits(g["shared_down"]),
    )
    return g, cfg, exact_bf16_bits(g["x"]), w


def check_micro(out, exp):
    np.testing.assert_allclose(out["z"], exp["z"], rtol=0, atol=0)
    np.testing.assert_allclose(out["s"], exp["s"], rtol=1e-6)
    np.testing.assert_array_equal(out["idx"], exp["idx"])
    np.testing.assert_allclose(out["gap"], exp["gap"], rtol=1e-5)
    np.testing.assert_allclose(out["w"], exp["w"], rtol=1e-6)
    np.testing.assert_allclose(out["r"], exp["r"], rtol=1e-6)
    np.testing.assert_allclose(out["y_shared"], exp["y_shared"], rtol=0, atol=0)
    np.testing.assert_allclose(out["y"], exp["y"], rtol=1e-6)


def test_worked_example_micro():
    g, cfg, x, w = micro_case()
    check_micro(O.forward(x, w, cfg), g["expected"])


# Plausible mistakes, planted in the oracle on the CPU: each must break the
# hand-derived example, which shows the example pins that part.
def _relu_not_squared(u, w_up, w_down):
    h = np.maximum(np.asarray(u, np.float64) @ np.asarray(w_up, np.float64).T, 0.0)
    return h @ np.asarray(w_down, np.float64).T


def _up_transposed(u, w_up, w_down):
    h = np.maximum(np.asarray(u, np.float64) @ np.asarray(w_up, np.float64), 0.0) ** 2
    return h @ np.asarray(w_down, np.float64).T


def _down_transposed(u, w_up, w_down):
    h = np.maximum(np.asarray(u, np.float64) @ np.asarray(w_up, np.float64).T, 0.0) ** 2
    return h @ np.asarray(w_down, np.float64)


def _no_renorm(s, idx, rho):
    sel = np.take_along_axis(np.asarray(s, np.float32), idx, 1)
    return (sel * np.float32(rho)).astype(np.float32)


_orig_renorm = O.renormalize


def _no_scale(s, idx, rho):
    return _orig_renorm(s, idx, 1.0)


_orig_select = O.select_experts


def _select_unbiased(s, beta, k, *groups):
    return _orig_select(s, np.zeros_like(np.asarray(beta)), k, *groups)


def _weights_from_biased(s, idx, rho):
    return _orig_renorm(np.asarray(s) + _BIAS[None, :], idx, rho)


_BIAS = None


@pytest.mark.parametrize("name,attr,fn", [
    ("relu not squared", "expert_mlp", _relu_not_squared),
    ("up weight transposed", "expert_mlp", _up_transposed),
    ("down weight transposed", "expert_mlp", _down_transposed),
    ("no renormalisation", "renormalize", _no_renorm),
    ("no routed scaling", "renormalize", _no_scale),
    ("bias ignored in selection", "select_experts", _select_unbiased),
    ("weights from biased score", "renormalize", _weights_from_biased),
    ("shared expert dropped", "shared_expert", lambda x, a, b: 0.0 * O.expert_mlp(x, a, b)),
    ("fc2_latent transposed", "latent_up_projection",
     lambda r, W2: np.asarray(r) @ np.asarray(W2, np.float64)),
])
def test_planted_mistakes_fail_worked_example(monkeypatch, name, attr, fn):
    global _BIAS
    g, cfg, x, w = micro_case()
    _BIAS = np.asarray(w.router_bias, np.float32)
    monkeypatch.setattr(O, attr, fn)
    # a wrong result or a shape error both count as caught
    with pytest.raises((AssertionError, ValueError)):
        check_micro(O.forward(x, w, cfg), g["expected"])


def test_bf16_upcast_exact():
    vals = np.array([0.0, -0.0, 1.0, -2.5, 3.140625, 1e-30, -65280.0, 2.0 ** -133], np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    back = O.bf16_bits_to_f64(bits)
    trunc = (vals.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(back, trunc)
    assert O.bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert O.bf16_bits_to_f64(np.array([0xC000], np.uint16))[0] == -2.0


def test_sigmoid_closed_forms():
    ln3 = math.log(3.0)
    wg = np.array([[0.0], [ln3], [-ln3], [100.0], [-100.0], [2.0], [-2.0]], np.float32)
    logits, s = O.router_scores(np.ones((1, 1), np.float32), wg)
    assert logits.dtype == np.float32 and s.dtype == np.float32
    assert s[0, 0] == np.float32(0.5)
    np.testing.assert_allclose(s[0, 1], 0.75, rtol=2e-7)
    np.testing.assert_allclose(s[0, 2], 0.25, rtol=2e-7)
    assert s[0, 3] == np.float32(1.0)
    # e^-100 is subnormal in float32: correct to within half a subnormal step
    assert abs(float(s[0, 4]) - math.exp(-100.0)) <= 0.5 * 2.0 ** -149
    # symmetry sigma(-l) = 1 - sigma(l), and the textbook value at 2
    assert abs(float(s[0, 5]) + float(s[0, 6]) - 1.0) < 1e-7
    np.testing.assert_allclose(s[0, 5], 1.0 / (1.0 + math.exp(-2.0)), rtol=1e-7)


def test_gemm_exact_on_integers():
    rng = np.random.default_rng(5)
    x = rng.integers(-8, 9, size=(5, 7))
    W = rng.integers(-8, 9, size=(3, 7))
    got = O.latent_projection(x, W)
    for t in range(5):
        for r in range(3):
            assert got[t, r] == sum(int(x[t, d]) * int(W[r, d]) for d in range(7))
    u = rng.integers(-3, 4, size=(4, 6))
    wu = rng.integers(-3, 4, size=(5, 6))
    wd = rng.integers(-3, 4, size=(6, 5))
    got = O.expert_mlp(u, wu, wd)
    for t in range(4):
        h = [max(0, sum(int(u[t, j]) * int(wu[f, j]) for j in range(6))) ** 2 for f in range(5)]
        for o in range(6):
            assert got[t, o] == sum(h[f] * int(wd[o, f]) for f in range(5))


def test_topk_matches_subset_enumeration():
    rng = np.random.default_rng(1)
    E, K, T = 16, 4, 40
    s = rng.uniform(0, 1, size=(T, E)).astype(np.float32)
    beta = rng.normal(0, 0.1, size=E).astype(np.float32)
    idx, b, gap = O.select_experts(s, beta, K)
    for t in range(T):
        best = max(itertools.combinations(range(E), K),
                   key=lambda c: sum(float(b[t, e]) for e in c))
        assert tuple(idx[t]) == best
        kept = sorted((float(b[t, e]) for e in best))
        rest = max(float(b[t, e]) for e in range(E) if e not in best)
        assert gap[t] == pytest.approx(kept[0] - rest, abs=0)


def test_topk_tie_break_lower_index():
    # x = 0 gives sigma(0) = 0.5 for every expert; the bias alone decides.
    s = np.full((1, 8), 0.5, np.float32)
    beta = np.array([0.1, 0.3, 0.3, 0.2, 0.3, 0.0, 0.2, 0.3], np.float32)
    idx, _, gap = O.select_experts(s, beta, 3)
    assert idx.tolist() == [[1, 2, 4]]
    assert gap[0] == 0.0
    idx, _, _ = O.select_experts(s, beta, 5)
    assert idx.tolist() == [[1, 2, 3, 4, 7]]
    # -0.0 and +0.0 compare equal: the lower index wins
    idx, _, _ = O.select_experts(np.zeros((1, 3), np.float32),
                                 np.array([0.0, -0.0, 0.0], np.float32), 1)
    assert idx.tolist() == [[0]]


def test_group_routing_worked_example():
    """§5.5 by hand: 8 experts in 4 groups of 2, keep 2 groups, top-3.
    Group scores (sum of the two best biased scores): 1.0, 1.0, 0.8, 0.6, so
    groups 0 and 1 stay and the top-3 of experts {0, 1, 2, 3} is {0, 2, 3}
    (2 and 3 tie at 0.5; both fit).  Ungrouped, expert 4 (0.8) would win a
    place; scoring groups by their single best expert would keep groups 0
    and 2 and select {0, 1, 4} -- so the example tells the three apart."""
    s = np.array([[0.9, 0.1, 0.5, 0.5, 0.8, 0.0, 0.3, 0.3]], np.float32)
    beta = np.zeros(8, np.float32)
    idx, _, gap = O.select_experts(s, beta, 3, n_group=4, topk_group=2)
    assert idx.tolist() == [[0, 2, 3]]
    # gap: groups 1.0 vs 0.8 (0.2) is closer than experts 0.5 vs 0.1 (0.4)
    assert gap[0] == pytest.approx(float(np.float32(0.5) + np.float32(0.5)) - 0.8, abs=1e-7)
    assert O.select_experts(s, beta, 3)[0].tolist() == [[0, 2, 4]]
    # equal group scores: the lower group index is kept
    s2 = np.array([[0.4, 0.4, 0.3, 0.5, 0.7, 0.1]], np.float32)   # groups of 2: 0.8, 0.8, 0.8
    idx2, _, gap2 = O.select_experts(s2, np.zeros(6, np.float32), 2, n_group=3, topk_group=1)
    assert idx2.tolist() == [[0, 1]] and gap2[0] == 0.0


def test_group_routing_matches_enumeration():
    """Group score as the best pair sum over the group, kept groups as the
    group subset with the largest score total, experts as the K-subset of
    eligible experts with the largest biased-score total: each by exhaustive
    enumeration, on random scores (no ties)."""
    rng = np.random.default_rng(7)
    E, T = 12, 12
    for n_group in (2, 3, 4, 6):
        G = E // n_group
        for topk_group in range(1, n_group + 1):
            K = min(3, topk_group * G)
            s = rng.uniform(0, 1, size=(T, E)).astype(np.float32)
            beta = rng.normal(0, 0.1, size=E).astype(np.float32)
            idx, b, _ = O.select_experts(s, beta, K, n_group, topk_group)
            for t in range(T):
                gs = [max(float(np.float32(b[t, i]) + np.float32(b[t, j]))
                          for i, j in itertools.combinations(range(g * G, g * G + G), 2))
                      for g in range(n_group)]
                kept = max(itertools.combinations(range(n_group), topk_group),
                           key=lambda c: sum(gs[g] for g in c))
                elig = [e for e in range(E) if e // G in kept]
                best = max(itertools.combinations(elig, K),
                           key=lambda c: sum(float(b[t, e]) for e in c))
                assert tuple(idx[t]) == best, (n_group, topk_group, t)


def test_group_routing_degenerate_cases():
    rng = np.random.default_rng(3)
    T, E, K = 20, 16, 4
    s = rng.uniform(0, 1, size=(T, E)).astype(np.float32)
    beta = rng.normal(0, 0.1, size=E).astype(np.float32)
    plain = O.select_experts(s, beta, K)
    # one group, or every group kept: the plain top-K
    for n_group, topk_group in [(1, 1), (4, 4), (8, 8)]:
        g = O.select_experts(s, beta, K, n_group, topk_group)
        assert np.array_equal(g[0], plain[0]) and np.array_equal(g[2], plain[2])
    # groups of two with K = 2 * kept groups: exactly the kept groups' experts
    idx, _, _ = O.select_experts(s, beta, 4, n_group=8, topk_group=2)
    groups = idx // 2
    assert np.all(groups[:, 0] == groups[:, 1]) and np.all(groups[:, 2] == groups[:, 3])
    # in general the selection spans at most topk_group groups
    idx, _, _ = O.select_experts(s, beta, 5, n_group=4, topk_group=2)
    assert all(len(set((idx[t] // 4).tolist())) <= 2 for t in range(T))


def _bf16(vals):
    """bf16 bit patterns of values that bf16 represents exactly."""
    v = np.asarray(vals, np.float32)
    b = (v.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(O.bf16_bits_to_f64(b), v.astype(np.float64))
    return b


def test_e2m1_magnitudes_are_the_pages_list():
    # Ultra teardown CH8 §8.1: 0, ±0.5, ±1, ±1.5, ±2, ±3, ±4, ±6
    assert O.E2M1_MAGNITUDES.tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_mxfp4_worked_block():
    """By hand: max |w| = 3 gives e = floor(log2 3) - 2 = -1, X = 0.5, scale
    byte 126; |w| / X = 6, 5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25, 0.5, 0.125:
    5, 3.5, 2.5, 1.75, 1.25, 0.75 and 0.25 are ties and go to the even code
    (4, 4, 2, 2, 1, 1, 0), -0.0625 rounds to an unsigned zero."""
    w = np.zeros(32, np.float32)
    w[:10] = [3.0, 2.5, 1.75, 1.25, 0.875, 0.625, 0.375, 0.125, -0.25, -0.0625]
    codes, scales = O.mxfp4_quantize(_bf16(w)[None])
    assert scales.tolist() == [[126]]
    assert codes[0, :5].tolist() == [7 | 6 << 4, 6 | 4 << 4, 4 | 2 << 4, 2 | 0 << 4, 9 | 0 << 4]
    assert not codes[0, 5:].any()
    assert O.mxfp4_dequantize(codes, scales)[0, :10].tolist() == [
        3.0, 2.0, 2.0, 1.0, 1.0, 0.5, 0.5, 0.0, -0.25, 0.0]


def test_mxfp4_saturation_zero_block_and_round_trip():
    # max |w| = 1.9375 < 2: e = -2, X = 0.25, 1.9375 / X = 7.75 clamps to 6 -> 1.5
    w = np.full(32, 0.5, np.float32)
    w[3] = -1.9375
    codes, scales = O.mxfp4_quantize(_bf16(w)[None])
    assert scales.tolist() == [[125]]
    back = O.mxfp4_dequantize(codes, scales)[0]
    assert back[3] == -1.5 and np.all(np.delete(back, 3) == 0.5)
    # all-zero block: smallest scale, zero codes
    codes, scales = O.mxfp4_quantize(np.zeros((2, 64), np.uint16))
    assert scales.tolist() == [[0, 0], [0, 0]] and not codes.any()
    assert not O.mxfp4_dequantize(codes, scales).any()
    # values already on the grid at the block's own scale come back exactly
    rng = np.random.default_rng(5)
    for e in (-9, -1, 0, 4):
        mags = O.E2M1_MAGNITUDES[rng.integers(0, 8, size=(3, 64))]
        mags[:, ::32] = 6.0                       # pin the block maximum
        v = (mags * rng.choice([-1, 1], size=mags.shape) * 2.0 ** e).astype(np.float32)
        c, sc = O.mxfp4_quantize(_bf16(v))
        assert np.all(sc == e + 127)
        assert np.array_equal(O.mxfp4_dequantize(c, sc), v.astype(np.float64))


def test_mxfp4_error_bound_and_monotone():
    """Random bf16 weights: within a block the error is at most X (half the
    widest grid spacing, 4 -> 6) below 6X and at most 2X above it, and the
    quantiser is monotone in w."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    b = (w.view(np.uint32) >> 16).astype(np.uint16)
    wv = O.bf16_bits_to_f64(b)
    codes, scales = O.mxfp4_quantize(b)
    back = O.mxfp4_dequantize(codes, scales)
    X = np.repeat(np.ldexp(1.0, scales.astype(int) - 127), 32, axis=1)
    a = np.abs(wv) / X
    err = np.abs(back - wv) / X
    assert np.all(err[a <= 6] <= 1.0) and np.all(err[a > 6] <= 2.0)
    assert np.all(a < 8)
    for r in range(4):
        for blk in range(8):
            sl = slice(32 * blk, 32 * blk + 32)
            order = np.argsort(wv[r, sl], kind="stable")
            assert np.all(np.diff(back[r, sl][order]) >= 0)


def test_mxfp4_planted_tie_rule_fails_worked_block(monkeypatch):
    """Ties to the lower magnitude instead of the even code: caught."""
    def lower_ties(w_bits):
        w = O.bf16_bits_to_f64(w_bits)
        K = w.shape[-1]
        blocks = w.reshape(*w.shape[:-1], K // 32, 32)
        amax = np.abs(blocks).max(-1)
        _, ex = np.frexp(amax)
        e = np.where(amax > 0, ex - 3, -127).clip(-127, 127)
        a = np.abs(blocks) / np.ldexp(1.0, e)[..., None]
        mag = np.abs(a[..., None] - O.E2M1_MAGNITUDES).argmin(-1)
        code = (mag + 8 * ((blocks < 0) & (mag > 0))).reshape(*w.shape[:-1], K)
        return (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8), (e + 127).astype(np.uint8)
    monkeypatch.setattr(O, "mxfp4_quantize", lower_ties)
    with pytest.raises(AssertionError):
        test_mxfp4_worked_block()


def test_float_expert_weights_equal_their_bf16_bits():
    """The forward takes expert weights as bf16 bits or as float arrays (the
    dequantised low-precision weights); the same values give the same
    layer output either way (worked example)."""
    g, cfg, x, w = micro_case()
    w2 = SimpleNamespace(**vars(w))
    w2.expert_up = [O.bf16_bits_to_f64(m) for m in w.expert_up]
    w2.expert_down = [O.bf16_bits_to_f64(m) for m in w.expert_down]
    check_micro(O.forward(x, w2, cfg), g["expected"])


def test_renormalisation_invariants():
    rng = np.random.default_rng(2)
    E, T = 64, 200
    s = rng.uniform(0.01, 1.0, size=(T, E)).astype(np.float32)
    for K in (1, 2, 7, 22):
        idx = np.sort(rng.permuted(np.tile(np.arange(E), (T, 1)), axis=1)[:, :K], axis=1)
        w = O.renormalize(s, idx, 5.0)
        assert w.dtype == np.float32
        tot = w.astype(np.float64).sum(1)
        assert np.all(np.abs(tot - 5.0) <= 32 * np.spacing(np.float32(5.0)))
        if K == 1:
            assert np.all(w == np.float32(5.0))
    idx = np.tile(np.arange(E), (T, 1))
    w = O.renormalize(s, idx, 5.0)
    ref = 5.0 * s.astype(np.float64) / np.array([math.fsum(r) for r in s.astype(np.float64)])[:, None]
    np.testing.assert_allclose(w, ref, rtol=3e-6)


def tiny_inputs(seed=0, **kw):
    wl = li.workload("tiny", seed=seed, **kw)
    inp = li.make_inputs(wl, "cpu")
    w = li.HostWeights(inp, eager_experts=True)
    sh = wl.shape
    cfg = O.OracleConfig(sh.hidden_size, sh.moe_latent_size, sh.n_routed_experts,
                         sh.num_experts_per_tok, sh.moe_intermediate_size,
                         sh.moe_shared_expert_intermediate_size, sh.routed_scaling_factor)
    return li.bf16_bits(inp.x), w, cfg


def test_dense_formulation_matches_sparse_dispatch():
    x, w, cfg = tiny_inputs()
    out = O.forward(x, w, cfg)
    z = out["z"]
    E = cfg.n_routed_experts
    gate = np.zeros((x.shape[0], E))
    for t in range(x.shape[0]):
        for k in range(cfg.num_experts_per_tok):
            gate[t, out["idx"][t, k]] = out["w"][t, k]
    r = np.zeros_like(z)
    for e in range(E):
        h = np.maximum(z @ O.bf16_bits_to_f64(w.expert_up[e]).T, 0) ** 2
        r += gate[:, e:e + 1] * (h @ O.bf16_bits_to_f64(w.expert_down[e]).T)
    np.testing.assert_allclose(out["r"], r, rtol=1e-12, atol=1e-12 * np.abs(r).max())
    assert out["counts"].sum() == x.shape[0] * cfg.num_experts_per_tok


def test_zero_input_gives_zero_output_and_bias_ranking():
    x, w, cfg = tiny_inputs()
    x0 = np.zeros_like(x)
    out = O.forward(x0, w, cfg)
    assert np.all(out["y"] == 0.0)
    assert np.all(out["s"] == np.float32(0.5))
    want = np.sort(np.argsort(-w.router_bias, kind="stable")[:cfg.num_experts_per_tok])
    assert np.all(out["idx"] == want[None, :])


def test_zero_expert_up_gives_shared_only():
    x, w, cfg = tiny_inputs()
    w.expert_up = np.zeros_like(w.expert_up)
    out = O.forward(x, w, cfg)
    assert np.all(out["y_routed"] == 0.0)
    np.testing.assert_array_equal(out["y"], out["y_shared"])


def test_identical_experts_give_rho_times_one_expert():
    x, w, cfg = tiny_inputs()
    w.expert_up = np.broadcast_to(w.expert_up[3], w.expert_up.shape).copy()
    w.expert_down = np.broadcast_to(w.expert_down[3], w.expert_down.shape).copy()
    out = O.forward(x, w, cfg)
    one = O.expert_mlp(out["z"], O.bf16_bits_to_f64(w.expert_up[3]),
                       O.bf16_bits_to_f64(w.expert_down[3]))
    np.testing.assert_allclose(out["r"], cfg.routed_scaling_factor * one,
                               rtol=1e-6, atol=1e-6 * np.abs(one).max())


def test_token_order_equivariance():
    x, w, cfg = tiny_inputs()
    out = O.forward(x, w, cfg)
    perm = np.random.default_rng(3).permutation(x.shape[0])
    outp = O.forward(x[perm], w, cfg)
    np.testing.assert_array_equal(outp["idx"], out["idx"][perm])
    np.testing.assert_array_equal(outp["w"], out["w"][perm])
    np.testing.assert_allclose(outp["y"], out["y"][perm], rtol=1e-12, atol=1e-12)


def test_forced_selection_is_used():
    x, w, cfg = tiny_inputs()
    out = O.forward(x, w, cfg)
    forced = np.tile(np.arange(cfg.num_experts_per_tok), (x.shape[0], 1))
    outf = O.forward(x, w, cfg, forced_idx=forced)
    assert np.all(outf["idx"] == forced)
    assert not np.allclose(outf["y"], out["y"])


def test_single_expert_and_all_experts():
    x, w, cfg = tiny_inputs()
    from dataclasses import replace
    c1 = replace(cfg, num_experts_per_tok=1)
    out = O.forward(x, w, c1)
    assert np.all(out["w"] == np.float32(5.0))
    cE = replace(cfg, num_experts_per_tok=cfg.n_routed_experts)
    out = O.forward(x, w, cE)
    assert np.all(out["idx"] == np.arange(cfg.n_routed_experts)[None, :])
    assert np.all(np.isinf(out["gap"]))


def test_page_parameter_and_flop_accounting():
    # "Nemotron 3 Ultra 架构深度拆解报告", §2.3.4 / §2.3.8 / §3.1.3: with the
    # gate on the 8192-d hidden state the page prints 10.94 B parameters per
    # MoE layer, 667.5 M active per token and about 1.33e9 FLOPs per token.
    sh = li.FULL
    D, R, E, K = sh.hidden_size, sh.moe_latent_size, sh.n_routed_experts, sh.num_experts_per_tok
    F, S = sh.moe_intermediate_size, sh.moe_shared_expert_intermediate_size
    params = E * D + E + 2 * D * R + E * 2 * F * R + 2 * D * S
    assert round(params / 1e9, 2) == 10.94
    # the page rounds one expert to 21 M before multiplying by 22
    per_expert_m = round(2 * F * R / 1e6)
    active_page = (E * D + 2 * D * R + 2 * D * S) / 1e6 + K * per_expert_m
    assert per_expert_m == 21 and round(active_page, 1) == 667.5
    flops = 2 * (E * D + 2 * D * R + K * 2 * F * R + 2 * D * S)
    assert round(flops / 1e9, 2) == 1.33
    # the page's single-expert size and the expert total
    assert 2 * F * R == 20_971_520 and E * 2 * F * R == 10_737_418_240


def test_zipf_bias_recipe_shape():
    b = li.zipf_bias(li.FULL, 3)
    assert b.dtype == np.float32 and b.shape == (512,)
    assert (b == np.float32(-2.0)).sum() == 51
    live = b[b > -1.5]
    assert np.all(live <= 0.0) and np.all(live > -1.0)


def test_tiny_generator_is_seeded():
    a = li.make_inputs(li.workload("tiny"), "cpu")
    b = li.make_inputs(li.workload("tiny"), "cpu")
    assert torch.equal(a.x, b.x) and torch.equal(a.expert_down, b.expert_down)
    assert a.x.dtype == torch.bfloat16 and a.router.dtype == torch.float32
    assert a.expert_up.shape == (16, 128, 64) and a.expert_down.shape == (16, 64, 128)


# ---- the block's pre-norm RMSNorm and residual (Ultra teardown CH9 §9.3) ----

def _prenorm_worked():
    """By hand (D = 4): gamma * h = 1.5 * 1.0078125 = 1.51171875 lies exactly
    half-way between the bf16 neighbours 1.5078125 and 1.515625 and goes to
    the even pattern 1.515625; 1.25 * 1.0078125 = 1.259765625 is below the
    half-way point of 1.2578125 and 1.265625 and rounds down; -1.51171875
    rounds like its magnitude; 2 * -4 = -8 is exact.  mean(h^2) =
    (3 * 1.0078125^2 + 16) / 4, r = 1 / sqrt(mean + eps)."""
    h = exact_bf16_bits([[1.0078125, 1.0078125, -1.0078125, -4.0]])
    g = exact_bf16_bits([1.5, 1.25, 1.5, 2.0])
    want_xt = [1.515625, 1.2578125, -1.515625, -8.0]
    mean = (3 * 1.0078125 ** 2 + 16.0) / 4
    return h, g, want_xt, mean


def test_prenorm_worked_rounding_and_factor():
    h, g, want_xt, mean = _prenorm_worked()
    for eps in (0.0, 1e-5, 0.25):
        xt, r = O.rms_prenorm(h, g, eps)
        assert O.bf16_bits_to_f64(xt)[0].tolist() == want_xt
        assert r[0] == pytest.approx(1.0 / math.sqrt(mean + eps), rel=1e-15)


def test_prenorm_unit_rms_and_eps_closed_form():
    rng = np.random.default_rng(7)
    h = li.bf16_bits(torch.from_numpy(rng.standard_normal((5, 96)).astype(np.float32)).to(torch.bfloat16))
    ones = exact_bf16_bits(np.ones(96))
    xt, r = O.rms_prenorm(h, ones, 0.0)
    assert np.array_equal(xt, h)                   # gamma = 1: the operand is h itself
    rms = np.sqrt(((r[:, None] * O.bf16_bits_to_f64(xt)) ** 2).mean(1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-14)
    # constant rows c: r = 1 / sqrt(c^2 + eps)
    c = np.array([0.5, 3.0, -2.0])
    hc = exact_bf16_bits(np.repeat(c[:, None], 96, 1))
    _, r = O.rms_prenorm(hc, ones, 0.75)
    np.testing.assert_allclose(r, 1.0 / np.sqrt(c ** 2 + 0.75), rtol=1e-15)


def test_prenorm_power_of_two_scale_invariance():
    rng = np.random.default_rng(8)
    h = li.bf16_bits(torch.from_numpy(rng.standard_normal((4, 64)).astype(np.float32)).to(torch.bfloat16))
    g = li.bf16_bits(torch.from_numpy((1 + 0.1 * rng.standard_normal(64)).astype(np.float32)).to(torch.bfloat16))
    xt, r = O.rms_prenorm(h, g, 0.0)
    base = r[:, None] * O.bf16_bits_to_f64(xt)
    for k in (-3, 2, 5):
        hk = exact_bf16_bits(O.bf16_bits_to_f64(h) * 2.0 ** k)
        xk, rk = O.rms_prenorm(hk, g, 0.0)
        assert np.array_equal(rk[:, None] * O.bf16_bits_to_f64(xk), base)


def test_block_forward_is_the_plain_forward_where_the_norm_is_exact():
    """h = +-2 everywhere: mean(h^2) = 4, so with eps = 0 r = 1/2 and
    bf16(gamma * h) = +-2 gamma exactly; the normalised rows are +-gamma,
    which bf16 holds.  The block output must be h plus the plain forward's
    output on those rows, bit for bit."""
    x, w, cfg = tiny_inputs()
    rng = np.random.default_rng(9)
    T, D = x.shape
    sign = rng.choice([-1.0, 1.0], size=(T, D))
    h = exact_bf16_bits(2.0 * sign)
    g = li.bf16_bits(torch.from_numpy((1 + 0.1 * rng.standard_normal(D)).astype(np.float32)).to(torch.bfloat16))
    plain = O.forward(exact_bf16_bits(sign * O.bf16_bits_to_f64(g)[None, :]), w, cfg)
    blk = O.block_forward(h, g, w, cfg, eps=0.0)
    assert np.all(blk["rnorm"] == 0.5)
    np.testing.assert_array_equal(blk["idx"], plain["idx"])
    assert np.array_equal(blk["y"], O.bf16_bits_to_f64(h) + plain["y"])
    assert np.array_equal(blk["y_layer"], plain["y"])
    nores = O.block_forward(h, g, w, cfg, eps=0.0, residual=False)
    assert np.array_equal(nores["y"], plain["y"])
    # no pre-norm: the layer reads h itself
    bare = O.block_forward(h, None, w, cfg)
    assert np.array_equal(bare["y_layer"], O.forward(h, w, cfg)["y"])
    assert np.array_equal(bare["y"], O.bf16_bits_to_f64(h) + bare["y_layer"])


def test_planted_prenorm_mistakes_fail_the_pins(monkeypatch):
    """Sum instead of mean, and truncation instead of round-to-nearest-even:
    each breaks the worked example."""
    real = O.rms_prenorm

    def by_sum(h_bits, gamma_bits, eps=1e-5):
        xt, _ = real(h_bits, gamma_bits, eps)
        hv = O.bf16_bits_to_f64(h_bits)
        return xt, 1.0 / np.sqrt((hv * hv).sum(axis=1) + eps)

    def truncated(h_bits, gamma_bits, eps=1e-5):
        _, r = real(h_bits, gamma_bits, eps)
        p = (O.bf16_bits_to_f64(h_bits) * O.bf16_bits_to_f64(gamma_bits)[None, :]).astype(np.float32)
        return (p.view(np.uint32) >> 16).astype(np.uint16), r

    for bad in (by_sum, truncated):
        monkeypatch.setattr(O, "rms_prenorm", bad)
        with pytest.raises(AssertionError):
            test_prenorm_worked_rounding_and_factor()
    monkeypatch.setattr(O, "rms_prenorm", real)


def _normalised_rows_are_scaled_not_rounded(block_forward):
    """The pre-norm reading: the layer reads r_t * bf16(gamma * h_t) with the
    factor r_t unrounded.  Both projections of the input are then exact
    rescalings of the plain layer run on xt = bf16(gamma * h): the latent is
    r_t times the plain latent (linear), and the shared expert's output is
    r_t^2 times the plain one (relu^2 is homogeneous of degree 2).  Rounding
    the normalised rows to bf16 instead perturbs both by up to 2^-9."""
    x, w, cfg = tiny_inputs()
    rng = np.random.default_rng(11)
    h = li.bf16_bits(torch.from_numpy(3.0 * rng.standard_normal(x.shape).astype(np.float32)).to(torch.bfloat16))
    g = li.bf16_bits(torch.from_numpy((1 + 0.1 * rng.standard_normal(x.shape[1])).astype(np.float32)).to(torch.bfloat16))
    blk = block_forward(h, g, w, cfg, eps=1e-5)
    rn = blk["rnorm"]
    assert not np.any(np.isclose(np.log2(rn), np.round(np.log2(rn))))  # r is not a power of two
    plain = O.forward(blk["xt"], w, cfg, forced_idx=blk["idx"])
    np.testing.assert_allclose(blk["z"], rn[:, None] * plain["z"], rtol=1e-12,
                               atol=1e-14 * np.abs(blk["z"]).max())
    np.testing.assert_allclose(blk["y_shared"], rn[:, None] ** 2 * plain["y_shared"],
                               rtol=1e-11, atol=1e-14 * np.abs(plain["y_shared"]).max())


def test_prenorm_reading_keeps_the_factor_exact():
    _normalised_rows_are_scaled_not_rounded(O.block_forward)


def test_planted_rounded_normalised_rows_fail_the_reading_pin():
    """The other reading (round r_t * gamma * h_t to bf16 before the layer)
    fails the pin above."""
    def rounded_rows(h_bits, gamma_bits, weights, cfg, eps=1e-5, residual=True, forced_idx=None):
        xt, rn = O.rms_prenorm(h_bits, gamma_bits, eps)
        rows = O.f32_to_bf16_bits((rn[:, None] * O.bf16_bits_to_f64(xt)).astype(np.float32))
        out = O.layer(O.bf16_bits_to_f64(rows), weights, cfg, forced_idx)
        out["xt"], out["rnorm"] = xt, rn
        return out

    with pytest.raises(AssertionError):
        _normalised_rows_are_scaled_not_rounded(rounded_rows)
