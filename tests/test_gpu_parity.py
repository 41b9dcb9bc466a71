"""GPU parity of the HIP LatentMoE layer against the CPU oracle, through the C
ABI, at sizes the oracle finishes in seconds (several tiles and ragged
tails), on both GEMM tilings, plus the edge cases of the method."""

import sys
from dataclasses import replace

import numpy as np
import pytest
import torch

import lmoe_inputs as li
import sparse_moe_layer_latentmoe_amd as pkg
from parity import (MEDIUM, assert_parity, check_properties, compare, medium, oracle_config,
                    run_gpu, weight_dict)
from oracle import lmoe_oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    return torch.device("cuda:0")


def layer_for(wl, inp, path=pkg.PATH_AUTO, max_tokens=None):
    return pkg.LatentMoE(wl.shape, weight_dict(inp), max_tokens or max(wl.tokens, 1), path)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("tokens", [64, 1, 17, 63])
def test_tiny_matches_oracle(dev, tokens):
    wl = li.workload("tiny", tokens=tokens)
    say(f"[tiny T={tokens}]")
    inp = li.make_inputs(wl, dev)
    g = run_gpu(layer_for(wl, inp), inp.x)
    check_properties(g, wl.shape, tokens)
    rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), wl.shape)
    say(rep)
    assert_parity(rep)


@pytest.mark.parametrize("path", [pkg.PATH_STREAM, pkg.PATH_TILED, pkg.PATH_AUTO])
@pytest.mark.parametrize("tokens", [300, 129])
def test_medium_both_tilings(dev, path, tokens):
    wl = medium(tokens)
    say(f"[medium T={tokens} path={path}]")
    inp = li.make_inputs(wl, dev)
    g = run_gpu(layer_for(wl, inp, path), inp.x)
    check_properties(g, wl.shape, tokens)
    rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), wl.shape)
    say(rep)
    assert_parity(rep)


# latent and expert widths of 1024: both bf16 expert GEMMs take 512 weight
# rows per tile (the up projection the two-stage LDS GEMM, which skips the
# copies of token rows past a tile's rows, the down projection the half-step
# pipelined one); both skip the MFMAs of 16-row token groups past them
DEEP = li.LayerShape(512, 1024, 16, 4, 1024, 512, 5.0)


@pytest.mark.parametrize("tokens", [150, 400, 600])
def test_expert_tiles_at_every_fill_level(dev, tokens):
    """Tiled path with ~37, ~100 and ~150 rows per expert: 128-row expert
    tiles whose row counts put the second wave row, and the last 16-row
    token group, at every fill level; every token compared."""
    wl = li.Workload("deep", DEEP, tokens)
    say(f"[deep T={tokens} tiled]")
    inp = li.make_inputs(wl, dev)
    g = run_gpu(layer_for(wl, inp, pkg.PATH_TILED), inp.x)
    check_properties(g, wl.shape, tokens)
    counts = np.bincount(g.idx.ravel(), minlength=DEEP.n_routed_experts) % 128
    say(f"  last-tile rows per expert: {sorted(set(counts.tolist()))}")
    rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), wl.shape)
    say(rep)
    assert_parity(rep)


# expert width 256 and latent 512: the down projection takes the half-step
# pipelined kernel with the shortest k range the tiled path allows (256, so
# eight half-steps: the three-unit prologue and both tail waits overlap)
SHORT_K = li.LayerShape(512, 512, 16, 4, 256, 512, 5.0)


@pytest.mark.parametrize("tokens", [150, 600])
def test_shortest_k_range_of_the_half_step_kernel(dev, tokens):
    """Tiled path, down projection over k = 256 in 512-row weight tiles
    (~37 rows per expert, where the second wave row only copies, and ~150,
    a full tile and a partly filled one); every token compared."""
    wl = li.Workload("short_k", SHORT_K, tokens)
    say(f"[short_k T={tokens} tiled]")
    inp = li.make_inputs(wl, dev)
    g = run_gpu(layer_for(wl, inp, pkg.PATH_TILED), inp.x)
    check_properties(g, wl.shape, tokens)
    rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), wl.shape)
    say(rep)
    assert_parity(rep)


# expert width 768 (a multiple of 256, not of 512) and latent 256: both
# expert GEMMs take the three-stage tiled kernel with 256 weight rows per
# tile, the up projection with gathered token rows
NARROW = li.LayerShape(512, 256, 16, 4, 768, 512, 5.0)


@pytest.mark.parametrize("tokens", [300, 700])
def test_expert_widths_off_the_wide_tiles(dev, tokens):
    """Tiled path where no expert width is a multiple of 512 (~75 and ~175
    rows per expert: one partly filled tile, then a full one and a partly
    filled one); every token compared."""
    wl = li.Workload("narrow", NARROW, tokens)
    say(f"[narrow T={tokens} tiled]")
    inp = li.make_inputs(wl, dev)
    g = run_gpu(layer_for(wl, inp, pkg.PATH_TILED), inp.x)
    check_properties(g, wl.shape, tokens)
    rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), wl.shape)
    say(rep)
    assert_parity(rep)


@pytest.mark.parametrize("tokens", [64, 65, 256, 257])
def test_dense_gemm_mode_boundaries(dev, tokens):
    """Automatic path at the token counts where the dense GEMMs switch from
    weight streaming (T <= 64) to split-k LDS tiles (T <= 256; at this shape
    the output projection's k range of 1280 splits into 4 ranges of 320, the
    first of which straddles the boundary between its two k segments at 256)
    and to whole-k LDS tiles (T > 256)."""
    wl = medium(tokens)
    say(f"[medium T={tokens} auto]")
    inp = li.make_inputs(wl, dev)
    g = run_gpu(layer_for(wl, inp), inp.x)
    check_properties(g, wl.shape, tokens)
    rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), wl.shape)
    say(rep)
    assert_parity(rep)


@pytest.mark.parametrize("tokens,experts,topk", [(100, 1024, 64), (400, 1024, 8)])
def test_largest_expert_count_and_top_k(dev, tokens, experts, topk):
    """The largest configuration the ABI accepts: 1024 experts (16 router
    slots per lane), top-64 (every lane of the selection wave holds a
    winner); at T = 400 the per-block masks no longer fit one work-group's
    LDS, so the three-kernel dispatch runs."""
    sh = li.LayerShape(256, 64, experts, topk, 128, 256, 5.0)
    wl = li.Workload("max", sh, tokens)
    say(f"[E={experts} K={topk} T={tokens}]")
    inp = li.make_inputs(wl, dev)
    g = run_gpu(layer_for(wl, inp), inp.x)
    check_properties(g, sh, tokens)
    rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), sh)
    say(rep)
    assert_parity(rep)


@pytest.mark.parametrize("shape,tokens", [
    # tiny: 8 groups of 2, keep 2, top-4 = exactly the kept groups' experts
    (replace(li.TINY, n_group=8, topk_group=2), 64),
    # medium: 4 groups of 8, keep 2, top-6; 8 groups of 4, keep 3, top-6
    (replace(MEDIUM, n_group=4, topk_group=2), 129),
    (replace(MEDIUM, n_group=8, topk_group=3), 300),
    # every group kept: the ungrouped selection
    (replace(MEDIUM, n_group=4, topk_group=4), 65),
])
def test_group_limited_routing(dev, shape, tokens):
    """Page §5.5: group score = sum of the group's two best biased scores,
    topk_group groups kept, top-K among their experts."""
    wl = li.Workload("grouped", shape, tokens)
    say(f"[groups n={shape.n_group} keep={shape.topk_group} E={shape.n_routed_experts} "
        f"K={shape.num_experts_per_tok} T={tokens}]")
    inp = li.make_inputs(wl, dev)
    g = run_gpu(layer_for(wl, inp), inp.x)
    check_properties(g, shape, tokens)
    rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), shape)
    say(rep)
    assert_parity(rep)


def test_paths_agree_on_routing(dev):
    wl = medium(300)
    inp = li.make_inputs(wl, dev)
    a = run_gpu(layer_for(wl, inp, pkg.PATH_STREAM), inp.x)
    b = run_gpu(layer_for(wl, inp, pkg.PATH_TILED), inp.x)
    assert np.array_equal(a.idx, b.idx)
    assert np.array_equal(a.z32, b.z32) or np.abs(a.z32 - b.z32).max() < 1e-4


def test_zero_input(dev):
    wl = li.workload("tiny")
    inp = li.make_inputs(wl, dev)
    inp.x.zero_()
    g = run_gpu(layer_for(wl, inp), inp.x)
    assert torch.count_nonzero(g.y) == 0
    beta = inp.router_bias.cpu().numpy()
    want = np.sort(np.argsort(-beta, kind="stable")[:wl.shape.num_experts_per_tok])
    assert np.all(g.idx == want[None, :])


def test_ties_go_to_lower_expert_index(dev):
    wl = li.workload("tiny")
    inp = li.make_inputs(wl, dev)
    inp.x.zero_()                       # every score is sigmoid(0) = 0.5
    bias = torch.zeros(wl.shape.n_routed_experts, dtype=torch.float32)
    bias[[3, 7, 9, 12, 15]] = 0.25      # five equal winners for K = 4
    inp.router_bias.copy_(bias.to(dev))
    g = run_gpu(layer_for(wl, inp), inp.x)
    assert np.all(g.idx == np.array([3, 7, 9, 12])[None, :])
    assert np.all(g.w == np.float32(1.25))


def test_one_expert_takes_every_token_and_empty_experts(dev):
    wl = medium(300)
    inp = li.make_inputs(wl, dev)
    bias = inp.router_bias.clone()
    bias[5] = 2.0                       # always selected
    bias[10:20] = -2.0                  # never selected
    inp.router_bias.copy_(bias)
    for path in (pkg.PATH_STREAM, pkg.PATH_TILED):
        g = run_gpu(layer_for(wl, inp, path), inp.x)
        check_properties(g, wl.shape, 300)
        assert g.counts[5] == 300 and np.all(g.counts[10:20] == 0)
        rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), wl.shape)
        say(path, rep)
        assert_parity(rep)


def test_single_expert_per_token_weight_is_rho(dev):
    base = li.workload("tiny")
    sh = li.LayerShape(256, 64, 16, 1, 128, 512, 5.0)
    wl = li.Workload("tiny_k1", sh, 64)
    inp = li.make_inputs(wl, dev)
    g = run_gpu(layer_for(wl, inp), inp.x)
    assert np.all(g.w == np.float32(5.0))
    rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), sh)
    assert_parity(rep)
    del base


def test_all_experts_per_token(dev):
    sh = li.LayerShape(256, 64, 16, 16, 128, 512, 5.0)
    wl = li.Workload("tiny_kE", sh, 40)
    inp = li.make_inputs(wl, dev)
    g = run_gpu(layer_for(wl, inp), inp.x)
    assert np.all(g.idx == np.arange(16)[None, :])
    rep = compare(g, li.bf16_bits(inp.x), li.HostWeights(inp, eager_experts=True), sh)
    assert_parity(rep)


def test_identical_experts_give_rho_times_one_expert(dev):
    wl = medium(200)
    inp = li.make_inputs(wl, dev)
    inp.expert_up.copy_(inp.expert_up[7:8].expand_as(inp.expert_up))
    inp.expert_down.copy_(inp.expert_down[7:8].expand_as(inp.expert_down))
    for path in (pkg.PATH_STREAM, pkg.PATH_TILED):
        g = run_gpu(layer_for(wl, inp, path), inp.x)
        z = g.z32.astype(np.float64)
        one = O.expert_mlp(z, O.bf16_bits_to_f64(li.bf16_bits(inp.expert_up[7])),
                           O.bf16_bits_to_f64(li.bf16_bits(inp.expert_down[7])))
        rel = np.abs(g.r - 5.0 * one).max() / np.abs(5.0 * one).max()
        say(path, "identical experts rel", rel)
        assert rel <= 2e-2


def test_zero_expert_up_gives_shared_only(dev):
    wl = medium(150)
    inp = li.make_inputs(wl, dev)
    inp.expert_up.zero_()
    g = run_gpu(layer_for(wl, inp), inp.x)
    assert np.count_nonzero(g.r) == 0
    cfg = oracle_config(wl.shape)
    hw = li.HostWeights(inp, eager_experts=True)
    ref = O.shared_expert(O.bf16_bits_to_f64(li.bf16_bits(inp.x)),
                          O.bf16_bits_to_f64(hw.shared_up), O.bf16_bits_to_f64(hw.shared_down))
    y = g.y.float().cpu().numpy()
    assert np.abs(y - ref).max() / np.abs(ref).max() <= 2e-2
    del cfg


@pytest.mark.parametrize("tokens", [300, 48])
def test_deterministic_and_token_order_equivariant(dev, tokens):
    # T = 48: the weight-streaming projections with the shared expert's down
    # projection on the auxiliary stream; T = 300: one concatenated GEMM
    wl = medium(tokens)
    inp = li.make_inputs(wl, dev)
    for path in (pkg.PATH_STREAM, pkg.PATH_TILED):
        layer = layer_for(wl, inp, path)
        a = run_gpu(layer, inp.x)
        b = run_gpu(layer, inp.x)
        assert torch.equal(a.y, b.y) and np.array_equal(a.idx, b.idx)
        perm = torch.randperm(tokens, generator=torch.Generator().manual_seed(4))
        c = run_gpu(layer, inp.x[perm.to(dev)].contiguous())
        assert torch.equal(c.y, a.y[perm.to(dev)])
        assert np.array_equal(c.idx, a.idx[perm.numpy()])


@pytest.mark.parametrize("fuse", [0, pkg.FUSE_BLOCK])
def test_debug_mode_gives_the_same_results(dev, monkeypatch, fuse):
    """LMOE_DEBUG set when the handle is created: every stage is waited for
    and checked; the forward (both tilings, with and without the block's
    pre-norm stage) and the router entry point give the same results bit for
    bit as a handle created without it."""
    wl = medium(300)
    inp = li.make_inputs(wl, dev)
    w = weight_dict(inp)
    if fuse:
        w["norm_weight"] = li.make_norm_weight(wl, dev)
    for path in (pkg.PATH_STREAM, pkg.PATH_TILED):
        say(f"[debug mode path={path} fuse={fuse}]")
        plain = pkg.LatentMoE(wl.shape, w, 300, path, fuse=fuse)
        monkeypatch.setenv("LMOE_DEBUG", "1")
        dbg = pkg.LatentMoE(wl.shape, w, 300, path, fuse=fuse)
        monkeypatch.delenv("LMOE_DEBUG")
        a, b = run_gpu(plain, inp.x), run_gpu(dbg, inp.x)
        assert torch.equal(a.y, b.y) and np.array_equal(a.idx, b.idx)
        assert np.array_equal(a.w, b.w) and np.array_equal(a.z32, b.z32)
        z = torch.from_numpy(a.z32).to(dev)
        ia, wa = plain.route(z)
        ib, wb = dbg.route(z)
        torch.cuda.synchronize()
        assert torch.equal(ia, ib) and torch.equal(wa, wb)


def test_smaller_batch_after_larger_on_one_handle(dev):
    # the workspace keeps the larger batch's contents; the smaller batch
    # (which may pick another tiling) must still match the oracle
    wl = medium(300)
    inp = li.make_inputs(wl, dev)
    layer = layer_for(wl, inp, max_tokens=300)
    run_gpu(layer, inp.x)
    x = inp.x[:37].contiguous()
    small = run_gpu(layer, x)
    check_properties(small, wl.shape, 37)
    rep = compare(small, li.bf16_bits(x), li.HostWeights(inp, eager_experts=True), wl.shape)
    say(rep)
    assert_parity(rep)


def test_route_entry_point_on_oracle_latent(dev):
    wl = medium(300)
    inp = li.make_inputs(wl, dev)
    cfg = oracle_config(wl.shape)
    hw = li.HostWeights(inp, eager_experts=True)
    ref = O.forward(li.bf16_bits(inp.x), hw, cfg)
    layer = layer_for(wl, inp)
    idx, w = layer.route(torch.from_numpy(ref["z32"]).to(dev))
    idx = idx.cpu().numpy()
    tie = ref["gap"] < 1e-6
    assert np.array_equal(idx[~tie], ref["idx"][~tie])
    assert np.abs(w.cpu().numpy()[~tie] - ref["w"][~tie]).max() <= 5e-5


def test_binding_refuses_mismatched_tensors_before_launching(dev):
    """Wrong width, dtype, layout or device of x, y, a tap or the router's
    latent raise in the binding (no launch); the handle then still gives the
    oracle-checked result of a correct call."""
    wl = li.workload("tiny", tokens=17)
    inp = li.make_inputs(wl, dev)
    layer = layer_for(wl, inp)
    ref = run_gpu(layer, inp.x)
    D, R = wl.shape.hidden_size, wl.shape.moe_latent_size
    y = torch.empty_like(inp.x)
    with pytest.raises(ValueError, match="shape"):
        layer.forward_into(inp.x[:, : D // 2].contiguous(), y)
    with pytest.raises(TypeError, match="dtype"):
        layer.forward_into(inp.x.float(), y)
    with pytest.raises(ValueError, match="contiguous"):
        layer.forward_into(inp.x, torch.empty(D, 17, dtype=torch.bfloat16, device=dev).t())
    with pytest.raises(ValueError, match="GPU"):
        layer.forward_into(inp.x.cpu(), y)
    with pytest.raises(ValueError, match="taps.topk_idx"):
        layer.forward_into(inp.x, y, pkg.Taps(topk_idx=torch.empty(17, 3, dtype=torch.int32,
                                                                   device=dev)))
    with pytest.raises(ValueError, match="shape"):
        layer.route(torch.zeros(17, R + 1, dtype=torch.float32, device=dev))
    again = run_gpu(layer, inp.x)
    assert torch.equal(again.y, ref.y)


def test_zero_tokens_is_a_noop(dev):
    wl = li.workload("tiny")
    inp = li.make_inputs(wl, dev)
    layer = layer_for(wl, inp)
    y = torch.full((0, 256), 1.0, dtype=torch.bfloat16, device=dev)
    layer.forward_into(inp.x[:0], y)
    torch.cuda.synchronize()


def test_profile_events_cover_every_stage(dev):
    wl = li.workload("tiny")
    inp = li.make_inputs(wl, dev)
    layer = layer_for(wl, inp)
    layer.profile_begin(3)
    for _ in range(3):
        layer.forward(inp.x)
    stages, n = layer.profile_end()
    assert n == 3 and set(stages) == set(pkg.stage_names())
    assert all(v >= 0 for v in stages.values())
