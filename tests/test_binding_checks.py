"""The Python binding's argument checks, on the CPU: the C ABI takes bare
device pointers, so the binding refuses tensors whose dtype, shape or
layout would make the kernels read or write out of bounds."""

import pytest
import torch

import lmoe_inputs as li
import sparse_moe_layer_latentmoe_amd as pkg


def test_weight_specs_follow_the_header_layouts():
    spec = pkg.weight_specs(li.FULL)
    assert spec["fc1_latent"] == ((2048, 8192), torch.bfloat16)
    assert spec["router"] == ((512, 2048), torch.float32)
    assert spec["router_bias"] == ((512,), torch.float32)
    assert spec["expert_up"] == ((512, 5120, 2048), torch.bfloat16)
    assert spec["expert_down"] == ((512, 2048, 5120), torch.bfloat16)
    assert spec["fc2_latent"] == ((8192, 2048), torch.bfloat16)
    assert spec["shared_up"] == ((10240, 8192), torch.bfloat16)
    assert spec["shared_down"] == ((8192, 10240), torch.bfloat16)
    assert "norm_weight" not in spec and "expert_up_mxfp4" not in spec
    mx = pkg.weight_specs(li.FULL, pkg.EXPERTS_MXFP4, pkg.FUSE_BLOCK)
    assert "expert_up" not in mx and mx["norm_weight"] == ((8192,), torch.bfloat16)
    assert mx["expert_up_mxfp4"] == ((512, 5120, 1024), torch.uint8)
    assert mx["expert_up_scale"] == ((512, 5120, 64), torch.uint8)
    assert mx["expert_down_mxfp4"] == ((512, 2048, 2560), torch.uint8)
    assert mx["expert_down_scale"] == ((512, 2048, 160), torch.uint8)


def test_tensor_checks_name_the_problem():
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(TypeError, match="dtype"):
        pkg._expect(x.float(), (4, 8), torch.bfloat16, "x")
    with pytest.raises(ValueError, match="shape"):
        pkg._expect(x, (4, 16), torch.bfloat16, "x")
    with pytest.raises(ValueError, match="contiguous"):
        pkg._expect(torch.zeros(8, 4, dtype=torch.bfloat16).t(), (4, 8), torch.bfloat16, "x")
    with pytest.raises(ValueError, match="GPU"):
        pkg._expect(x, (4, 8), torch.bfloat16, "x")
    with pytest.raises(TypeError, match="torch.Tensor"):
        pkg._expect([0], (4, 8), torch.bfloat16, "x")


def test_missing_or_misshapen_weights_are_refused():
    sh = li.workload("tiny").shape
    spec = pkg.weight_specs(sh)
    w = {k: torch.zeros(shp, dtype=dt) for k, (shp, dt) in spec.items()}
    with pytest.raises(ValueError, match="GPU"):           # everything right but the device
        pkg.check_weights(sh, w)
    bad = dict(w, expert_up=torch.zeros(3, 3, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="expert_up"):
        pkg.check_weights(sh, bad)
    del w["router_bias"]
    with pytest.raises(ValueError, match="router_bias"):
        pkg.check_weights(sh, w)


def test_quantiser_input_is_checked():
    with pytest.raises(TypeError, match="dtype"):
        pkg.quantize_mxfp4(torch.zeros(4, 32, dtype=torch.float32))
    with pytest.raises(ValueError, match="GPU"):
        pkg.quantize_mxfp4(torch.zeros(4, 32, dtype=torch.bfloat16))
