"""lmoe_forward_noalloc, the allocation-free entry point, against
lmoe_forward (the handle and workspace entry point) through the C ABI: two
calls in a row on one shape, the second with fewer tokens, each equal to
the handle's forward on the same input bit for bit (the same kernels in the
same order; only the shared expert's stream and the scratch differ).  The
shapes cover the weight-streaming and the split-k tiled dense paths and the
full-shape decode batch; a forward that needs more than the static scratch
is refused before any launch."""

import sys

import pytest
import torch

import lmoe_inputs as li
import sparse_moe_layer_latentmoe_amd as pkg
from parity import MEDIUM, weight_dict

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    return torch.device("cuda:0")


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("shape,tokens,path", [
    (li.TINY, (64, 13), pkg.PATH_AUTO),        # weight-streaming GEMMs
    (MEDIUM, (200, 70), pkg.PATH_AUTO),        # split-k dense GEMMs, tiled experts
    (MEDIUM, (48, 1), pkg.PATH_TILED),         # every GEMM LDS-tiled
    (li.FULL, (32, 5), pkg.PATH_AUTO),         # the full-shape decode batch
])
def test_noalloc_matches_the_handle_forward(dev, shape, tokens, path):
    T0 = tokens[0]
    say(f"[noalloc D={shape.hidden_size} E={shape.n_routed_experts} T={tokens} path={path}]")
    wl = li.Workload("noalloc", shape, T0)
    inp = li.make_inputs(wl, dev)
    layer = pkg.LatentMoE(shape, weight_dict(inp), T0, path=path)
    for T in tokens:                     # two calls in a row, the second smaller
        x = inp.x[:T].contiguous() if T < T0 else inp.x
        want = layer.forward(x)
        got = torch.full_like(x, float("nan"))
        layer.forward_noalloc_into(x, got)
        torch.cuda.synchronize()
        say(f"  T={T}: equal {torch.equal(got, want)}")
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), T
    layer.close()


# latent and expert widths multiples of 512: the MXFP4 streaming kernel that
# copies the codes into LDS; MEDIUM at 200 tokens: the LDS-tiled MXFP4 GEMMs
MX_WIDE = li.LayerShape(512, 512, 16, 4, 1024, 512, 5.0)


@pytest.mark.parametrize("shape,tokens", [(MX_WIDE, (64, 13)), (MEDIUM, (200, 70))])
def test_noalloc_matches_the_handle_forward_mxfp4(dev, shape, tokens):
    T0 = tokens[0]
    say(f"[noalloc mxfp4 D={shape.hidden_size} E={shape.n_routed_experts} T={tokens}]")
    wl = li.Workload("noalloc", shape, T0)
    inp = li.make_inputs(wl, dev)
    w = weight_dict(inp)
    up_c, up_s = pkg.quantize_mxfp4(inp.expert_up)
    dn_c, dn_s = pkg.quantize_mxfp4(inp.expert_down)
    w.update(expert_up=None, expert_down=None, expert_up_mxfp4=up_c, expert_up_scale=up_s,
             expert_down_mxfp4=dn_c, expert_down_scale=dn_s)
    layer = pkg.LatentMoE(shape, w, T0, expert_format=pkg.EXPERTS_MXFP4)
    for T in tokens:
        x = inp.x[:T].contiguous() if T < T0 else inp.x
        want = layer.forward(x)
        got = torch.full_like(x, float("nan"))
        layer.forward_noalloc_into(x, got)
        torch.cuda.synchronize()
        say(f"  T={T}: equal {torch.equal(got, want)}")
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), T
    layer.close()


def test_noalloc_refuses_forwards_beyond_its_scratch(dev):
    """A full-shape forward of 192 tokens needs ~130 MB of scratch: refused
    with LMOE_ERR_SCRATCH, nothing launched (y keeps its contents)."""
    shape = li.TINY
    wl = li.Workload("noalloc", shape, 4)
    inp = li.make_inputs(wl, dev)
    layer = pkg.LatentMoE(shape, weight_dict(inp), 4)
    # a config whose 192-token workspace exceeds the array; the weights are
    # never read (the check comes first)
    big = pkg.make_config(li.FULL, 192)
    x = torch.zeros(192, li.FULL.hidden_size, dtype=torch.bfloat16, device=dev)
    y = torch.ones_like(x)
    st = layer.lib.lmoe_forward_noalloc(big, layer.wstruct, x.data_ptr(), 192, y.data_ptr(), None)
    assert st == pkg.LMOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((y == 1).all())
    layer.close()
