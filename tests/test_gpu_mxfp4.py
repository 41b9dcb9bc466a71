"""MXFP4 (block-scaled FP4) expert weights on the GPU, through the C ABI:
the library's quantiser against the oracle's, bit for bit, and the layer
forward with MXFP4 experts against the oracle run on the same quantised
weights (its own quantisation of the bf16 weights), at small and full
shape."""

import sys

import numpy as np
import pytest
import torch

import lmoe_inputs as li
import sparse_moe_layer_latentmoe_amd as pkg
from parity import (MEDIUM, assert_parity, assert_routing, check_properties, compare, medium,
                    mxfp4_host_weights, route_every_token, run_gpu, weight_dict)
from oracle import lmoe_oracle as O

pytestmark = pytest.mark.gpu

MX_SMALL = li.LayerShape(256, 128, 16, 4, 256, 512, 5.0)
# latent and expert widths multiples of 512: both streaming expert GEMMs take
# the kernel with the codes copied into LDS (MX_SMALL takes the general one,
# MEDIUM one of each)
MX_WIDE = li.LayerShape(512, 512, 16, 4, 1024, 512, 5.0)
# expert width 4096: a long k range (16 stages) for the down projection
MX_LONG = li.LayerShape(512, 512, 16, 4, 4096, 512, 5.0)
# latent 1024 (two groups of four 128-k stages) and expert width 1024: on the
# tiled path the up projection takes the kernel with the codes staged in LDS
MX_DEEP = li.LayerShape(512, 1024, 16, 4, 1024, 512, 5.0)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def special_rows():
    """bf16 rows with the quantiser's corner cases, one 32-block each:
    all zero; exact ties at X = 0.5; saturation; signed and unsigned zeros;
    subnormal and huge magnitudes; a negative block maximum."""
    def bits(v):
        return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)
    rows = []
    rows.append(np.zeros(32, np.uint16))
    t = np.zeros(32, np.float32)
    t[:10] = [3.0, 2.5, 1.75, 1.25, 0.875, 0.625, 0.375, 0.125, -0.25, -0.0625]
    rows.append(bits(t))
    t = np.full(32, 0.5, np.float32)
    t[3] = -1.9375
    rows.append(bits(t))
    z = bits(np.linspace(-1, 1, 32))
    z[::4] = 0x8000                                  # -0.0
    rows.append(z)
    sub = np.full(32, 0x0001, np.uint16)             # smallest bf16 subnormal
    sub[5] = 0x0080                                  # smallest normal
    rows.append(sub)
    rows.append(bits(np.linspace(-3e38, 3e38, 32)))
    t = np.linspace(0.01, 0.3, 32).astype(np.float32)
    t[7] = -0.75
    rows.append(bits(t))
    return np.stack(rows)


def test_quantiser_matches_oracle_bit_for_bit(dev):
    rng = np.random.default_rng(2)
    cases = [special_rows(),
             (rng.standard_normal((64, 256)) * 0.02).astype(np.float32),
             (rng.standard_normal((8, 64)) * 100).astype(np.float32),
             (rng.standard_normal((1, 32)) * 1e-30).astype(np.float32)]
    for c in cases:
        b = c if c.dtype == np.uint16 else (c.view(np.uint32) >> 16).astype(np.uint16)
        say(f"[quantiser rows={b.shape[0]} cols={b.shape[1]}]")
        w = torch.from_numpy(b.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        codes, scales = pkg.quantize_mxfp4(w)
        torch.cuda.synchronize()
        oc, os_ = O.mxfp4_quantize(b)
        assert np.array_equal(scales.cpu().numpy(), os_)
        assert np.array_equal(codes.cpu().numpy(), oc)


def mx_weights(inp):
    w = weight_dict(inp)
    up_c, up_s = pkg.quantize_mxfp4(inp.expert_up)
    dn_c, dn_s = pkg.quantize_mxfp4(inp.expert_down)
    w.update(expert_up=None, expert_down=None, expert_up_mxfp4=up_c, expert_up_scale=up_s,
             expert_down_mxfp4=dn_c, expert_down_scale=dn_s)
    return w


# (shape, tokens, path): AUTO streams the experts for few tokens per expert
# and takes the LDS-tiled MXFP4 GEMMs for many (MEDIUM at T = 300: 1800 slots
# over 32 experts); TILED forces them wherever the widths allow it.
@pytest.mark.parametrize("shape,tokens,path", [
    (MX_SMALL, 64, pkg.PATH_AUTO), (MX_SMALL, 1, pkg.PATH_AUTO), (MX_SMALL, 37, pkg.PATH_AUTO),
    (MX_WIDE, 1, pkg.PATH_AUTO), (MX_WIDE, 37, pkg.PATH_AUTO), (MX_WIDE, 64, pkg.PATH_AUTO),
    (MX_WIDE, 200, pkg.PATH_AUTO), (MEDIUM, 129, pkg.PATH_AUTO), (MEDIUM, 300, pkg.PATH_AUTO),
    (MEDIUM, 1, pkg.PATH_TILED), (MEDIUM, 64, pkg.PATH_TILED), (MX_WIDE, 200, pkg.PATH_TILED),
    (MX_LONG, 1, pkg.PATH_AUTO), (MX_LONG, 37, pkg.PATH_AUTO),
    (MX_DEEP, 150, pkg.PATH_TILED), (MX_DEEP, 3, pkg.PATH_TILED),
    # ~100 and ~150 rows per expert: the LDS-staged kernel's partly filled
    # tiles take each of its four k-loop copies (quarter, half, three
    # quarters, all of the token groups)
    (MX_DEEP, 400, pkg.PATH_TILED), (MX_DEEP, 600, pkg.PATH_TILED),
])
def test_mxfp4_forward_matches_oracle(dev, shape, tokens, path):
    wl = li.Workload("mxfp4", shape, tokens)
    say(f"[mxfp4 forward E={shape.n_routed_experts} R={shape.moe_latent_size} "
        f"F={shape.moe_intermediate_size} T={tokens} path={path}]")
    inp = li.make_inputs(wl, dev)
    w = mx_weights(inp)
    layer = pkg.LatentMoE(shape, w, tokens, path=path, expert_format=pkg.EXPERTS_MXFP4)
    g = run_gpu(layer, inp.x)
    check_properties(g, shape, tokens)
    hw = mxfp4_host_weights(inp, eager_experts=True)
    rep = compare(g, li.bf16_bits(inp.x), hw, shape)
    say(rep)
    assert_parity(rep)
    # the library's codes are the oracle's codes for every expert touched
    for e in np.unique(g.idx):
        oc, os_ = hw.expert_up.coded[int(e)]
        assert np.array_equal(w["expert_up_mxfp4"][int(e)].cpu().numpy(), oc)
        assert np.array_equal(w["expert_up_scale"][int(e)].cpu().numpy(), os_)
        oc, os_ = hw.expert_down.coded[int(e)]
        assert np.array_equal(w["expert_down_mxfp4"][int(e)].cpu().numpy(), oc)
        assert np.array_equal(w["expert_down_scale"][int(e)].cpu().numpy(), os_)


@pytest.mark.fullshape
@pytest.mark.parametrize("name,tokens,rows", [("decode", None, [0, 13, 31]),
                                              ("prefill", None, [0, 4097, 8191]),
                                              ("prefill", 21504, [0, 10752, 21503])])
def test_mxfp4_full_shape(dev, name, tokens, rows):
    """The decode batch (weight streaming) and the prefill batch (LDS-tiled
    MXFP4 GEMMs) at full shape with MXFP4 experts, and a long prefill batch
    of 21504 tokens (more than 4096 expert tiles): properties on every
    token, every token's routing against the oracle's, the whole output on
    three sampled tokens plus any tie token (every expert they use quantised
    by the oracle and compared with the library's codes)."""
    wl = li.workload(name) if tokens is None else li.workload(name, tokens=tokens)
    say(f"[mxfp4 full {name} T={wl.tokens}]")
    inp = li.make_inputs(wl, dev)
    w = mx_weights(inp)
    layer = pkg.LatentMoE(wl.shape, w, wl.tokens, expert_format=pkg.EXPERTS_MXFP4)
    g = run_gpu(layer, inp.x)
    check_properties(g, wl.shape, wl.tokens)
    # the oracle quantises the touched experts itself, from the bf16 weights
    hw = mxfp4_host_weights(inp)
    x_bits = li.bf16_bits(inp.x)
    routing = route_every_token(g, x_bits, hw, wl.shape)
    say(f"  {routing}")
    assert_routing(routing)
    rows = np.union1d(np.array(rows), routing.tie_rows)
    used = np.unique(g.idx[rows])
    hw.expert_up.prefetch(used)
    hw.expert_down.prefetch(used)
    for e in used:
        assert np.array_equal(w["expert_up_mxfp4"][int(e)].cpu().numpy(), hw.expert_up.coded[int(e)][0])
        assert np.array_equal(w["expert_down_scale"][int(e)].cpu().numpy(), hw.expert_down.coded[int(e)][1])
    rep = compare(g, x_bits, hw, wl.shape, rows=rows)
    say(f"  sampled and tie rows {rows.tolist()}: {rep}")
    assert_parity(rep)
