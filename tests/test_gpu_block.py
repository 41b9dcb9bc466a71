"""The layer with its block's pre-norm RMSNorm and residual add fused in
(lmoe_config.fuse), on the GPU through the C ABI, against the oracle's
block forward (page "Nemotron 3 Ultra 架构深度拆解报告", CH9 §9.3) on the same
seeded inputs: the residual stream h as the input, the pre-norm weight
gamma, and every combination of the two fused steps on both GEMM tilings."""

import sys

import numpy as np
import pytest
import torch

import lmoe_inputs as li
import sparse_moe_layer_latentmoe_amd as pkg
from parity import (MEDIUM, Block, assert_parity, assert_routing, check_properties, compare,
                    mxfp4_host_weights, route_every_token, run_gpu, weight_dict)

pytestmark = pytest.mark.gpu

MX_WIDE = li.LayerShape(512, 512, 16, 4, 1024, 512, 5.0)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def run_block(dev, shape, tokens, fuse, path=pkg.PATH_AUTO, eps=1e-5, rows=None,
              expert_format=pkg.EXPERTS_BF16, wl=None):
    wl = wl or li.Workload("block", shape, tokens)
    say(f"[block fuse={fuse} path={path} eps={eps} D={shape.hidden_size} "
        f"R={shape.moe_latent_size} E={shape.n_routed_experts} T={tokens} "
        f"format={expert_format}]")
    inp = li.make_inputs(wl, dev)
    gamma = li.make_norm_weight(wl, dev)
    w = weight_dict(inp)
    if fuse & pkg.FUSE_PRENORM:
        w["norm_weight"] = gamma
    if expert_format == pkg.EXPERTS_MXFP4:
        up_c, up_s = pkg.quantize_mxfp4(inp.expert_up)
        dn_c, dn_s = pkg.quantize_mxfp4(inp.expert_down)
        w.update(expert_up=None, expert_down=None, expert_up_mxfp4=up_c, expert_up_scale=up_s,
                 expert_down_mxfp4=dn_c, expert_down_scale=dn_s)
        hw = mxfp4_host_weights(inp, eager_experts=rows is None)
    else:
        hw = li.HostWeights(inp, eager_experts=rows is None)
    layer = pkg.LatentMoE(shape, w, tokens, path=path, expert_format=expert_format,
                          fuse=fuse, norm_eps=eps)
    g = run_gpu(layer, inp.x)
    check_properties(g, shape, tokens)
    block = Block(li.bf16_bits(gamma) if fuse & pkg.FUSE_PRENORM else None, eps,
                  bool(fuse & pkg.FUSE_RESIDUAL))
    x_bits = li.bf16_bits(inp.x)
    if rows is not None:
        # sampled outputs: every token's routing against the oracle's, and
        # the tie tokens added to the rows whose whole output is compared
        routing = route_every_token(g, x_bits, hw, shape, block=block)
        say(f"  {routing}")
        assert_routing(routing)
        rows = np.union1d(rows, routing.tie_rows)
    if rows is not None and expert_format == pkg.EXPERTS_MXFP4:
        used = np.unique(g.idx[rows])
        hw.expert_up.prefetch(used)
        hw.expert_down.prefetch(used)
    rep = compare(g, x_bits, hw, shape, rows=rows, block=block)
    say(f"  {rep}")
    assert_parity(rep)
    return g, inp


BOTH = pkg.FUSE_BLOCK


@pytest.mark.parametrize("shape,tokens,fuse,path,eps", [
    (li.TINY, 64, BOTH, pkg.PATH_AUTO, 1e-5),
    (li.TINY, 1, BOTH, pkg.PATH_AUTO, 1e-5),
    (li.TINY, 37, pkg.FUSE_PRENORM, pkg.PATH_AUTO, 0.5),
    (li.TINY, 64, pkg.FUSE_RESIDUAL, pkg.PATH_AUTO, 1e-5),
    (MEDIUM, 64, BOTH, pkg.PATH_STREAM, 1e-5),
    (MEDIUM, 129, BOTH, pkg.PATH_AUTO, 1e-5),       # split-k dense GEMMs
    (MEDIUM, 300, BOTH, pkg.PATH_AUTO, 1e-5),       # whole-k tiled dense GEMMs
    (MEDIUM, 300, pkg.FUSE_PRENORM, pkg.PATH_TILED, 1e-5),
    (MEDIUM, 37, pkg.FUSE_RESIDUAL, pkg.PATH_TILED, 1e-5),
])
def test_block_matches_oracle(dev, shape, tokens, fuse, path, eps):
    run_block(dev, shape, tokens, fuse, path, eps)


def test_block_with_mxfp4_experts(dev):
    run_block(dev, MX_WIDE, 37, BOTH, expert_format=pkg.EXPERTS_MXFP4)


@pytest.mark.parametrize("tokens,path", [(37, pkg.PATH_AUTO), (200, pkg.PATH_TILED)])
def test_every_option_at_once(dev, tokens, path):
    """Group-limited routing (4 groups of 4, keep 2), MXFP4 experts and both
    block steps in one layer, on the weight-streaming and the tiled path."""
    from dataclasses import replace
    shape = replace(MX_WIDE, n_group=4, topk_group=2)
    g, _ = run_block(dev, shape, tokens, BOTH, path=path, expert_format=pkg.EXPERTS_MXFP4)
    assert max(len(set((row // 4).tolist())) for row in g.idx) <= 2


def test_block_output_is_residual_plus_layer(dev):
    """The residual alone changes nothing but the add: y(fuse=RESIDUAL) is
    the bf16 rounding of h + the unfused layer's fp32 result, so it stays
    within two bf16 roundings of h + y(fuse=0)."""
    shape, T = MEDIUM, 64
    wl = li.Workload("block", shape, T)
    inp = li.make_inputs(wl, dev)
    w = weight_dict(inp)
    plain = pkg.LatentMoE(shape, w, T).forward(inp.x)
    res = pkg.LatentMoE(shape, w, T, fuse=pkg.FUSE_RESIDUAL).forward(inp.x)
    torch.cuda.synchronize()
    want = inp.x.float() + plain.float()
    err = (res.float() - want).abs()
    # two bf16 roundings, each within 2^-8 of its value: res's of h + acc and
    # plain's of acc (acc: the output GEMM's fp32 sum, the same in both runs),
    # so |res - (h + plain)| <= 2^-8 (|h + acc| + |acc|) <= 2^-8 (|h| + 2 |acc|)
    bound = 1.01 * 2.0 ** -8 * (inp.x.float().abs() + 2 * plain.float().abs()) + 1e-30
    assert bool((err <= bound).all()), float((err / bound).max())


@pytest.mark.fullshape
def test_block_decode_full_shape(dev):
    """Decode batch at full shape with both block steps fused: properties and
    routing on every token, the whole output on three sampled tokens (and
    any tie token)."""
    wl = li.workload("decode")
    run_block(dev, wl.shape, wl.tokens, BOTH, rows=np.array([0, 17, wl.tokens - 1]), wl=wl)
