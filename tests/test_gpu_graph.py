"""lmoe_forward under HIP graph capture: one forward captured (its
auxiliary-stream fork and join included), then replayed several times with
the input changed, eager forwards and host synchronisations in between;
every replay must equal an eager forward on the same input, bit for bit
(the kernels are deterministic).  The forward enqueues no memset and no host
synchronisation, which is what makes it capturable."""

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


# warm: one eager forward on a side stream before the capture; cold: the
# handle's first forward is the captured one (the auxiliary stream and its
# events already exist, created with the handle)
@pytest.mark.parametrize("shape,tokens,path,warm", [
    (li.TINY, 64, pkg.PATH_AUTO, False),        # weight-streaming GEMMs
    (MEDIUM, 300, pkg.PATH_AUTO, False),        # LDS-tiled GEMMs
    (MEDIUM, 300, pkg.PATH_AUTO, True),
])
def test_captured_forward_replays_match_eager(dev, shape, tokens, path, warm):
    print(f"[graph D={shape.hidden_size} T={tokens} path={path} warm={warm}]", flush=True)
    sys.stdout.flush()
    wl = li.Workload("graph", shape, tokens)
    inp = li.make_inputs(wl, dev)
    layer = pkg.LatentMoE(shape, weight_dict(inp), tokens, path=path)
    x = inp.x.clone()
    y = torch.empty_like(x)
    if warm:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            layer.forward_into(x, y)
        torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward_into(x, y)
    torch.cuda.synchronize()
    gen = torch.Generator(device=dev)
    for r in range(3):
        gen.manual_seed(100 + r)
        x.copy_(torch.randn(x.shape, generator=gen, device=dev).to(torch.bfloat16))
        want = layer.forward(x)           # eager, same input
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want), f"replay {r} differs from the eager forward"
