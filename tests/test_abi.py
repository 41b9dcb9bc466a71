"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments before any HIP call (so these run
without a GPU).  A valid lmoe_create makes its HIP calls (the auxiliary
stream and events): without a GPU it must return LMOE_ERR_HIP and leave no
handle, with one LMOE_OK.  The forward's own argument checks need a handle,
so that test runs where a GPU is present (it launches nothing)."""

import ctypes
import os
import re
import subprocess

import pytest

import lmoe_inputs as li
import sparse_moe_layer_latentmoe_amd as pkg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmoe.h")

FAKE = 0x10000  # 256-byte aligned host-side stand-in; never dereferenced


def have_gpu():
    import torch
    return torch.cuda.is_available()


def created(st, h):
    """A valid lmoe_create: a handle with a GPU; LMOE_ERR_HIP and none without."""
    if have_gpu():
        return st == pkg.LMOE_OK and bool(h.value)
    return st == pkg.LMOE_ERR_HIP and not h.value


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pkg.LIB_PATH):
        pytest.fail("liblmoe.so not built (run __graft_entry__.build())")
    return pkg.load_library()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lmoe_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = header_functions()
    for n in ("lmoe_workspace_size", "lmoe_create", "lmoe_forward", "lmoe_route",
              "lmoe_destroy", "lmoe_status_string"):
        assert n in names
    assert set(names) == set(pkg.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", pkg.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(lmoe_\w+)", out))
    for n in header_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def cfg(**kw):
    c = pkg.make_config(li.TINY, 64)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def weights(**kw):
    w = pkg.LmoeWeights(*([FAKE] * 8))
    for k, v in kw.items():
        setattr(w, k, v)
    return w


def create(lib, c, w=None, ws=FAKE, nbytes=None):
    h = ctypes.c_void_p()
    if nbytes is None:
        nbytes = lib.lmoe_workspace_size(ctypes.byref(c)) or 1
    st = lib.lmoe_create(ctypes.byref(c), ctypes.byref(w or weights()), ws, nbytes,
                         ctypes.byref(h))
    return st, h


def test_workspace_size_and_config_checks(lib):
    assert lib.lmoe_workspace_size(ctypes.byref(cfg())) > 0
    full = pkg.make_config(li.FULL, 8192)
    # at least the expert hidden and output buffers
    assert lib.lmoe_workspace_size(ctypes.byref(full)) > 8192 * 22 * (5120 + 2048) * 2
    assert lib.lmoe_workspace_size(None) == 0
    # group-limited routing is accepted (4 groups of 4, keep 2, top-4)
    assert lib.lmoe_workspace_size(ctypes.byref(cfg(n_group=4, topk_group=2))) > 0
    for bad, status in [
        (dict(hidden_size=0), pkg.LMOE_ERR_INVALID_ARG),
        (dict(max_tokens=0), pkg.LMOE_ERR_INVALID_ARG),
        (dict(routed_scaling_factor=float("inf")), pkg.LMOE_ERR_INVALID_ARG),
        (dict(path=7), pkg.LMOE_ERR_INVALID_ARG),
        # routing groups: equal groups of >= 2 experts, 1 <= topk_group <= n_group,
        # K <= experts in the kept groups, at most 64 groups
        (dict(n_group=0), pkg.LMOE_ERR_INVALID_ARG),
        (dict(topk_group=2), pkg.LMOE_ERR_INVALID_ARG),            # > n_group = 1
        (dict(n_group=3), pkg.LMOE_ERR_INVALID_ARG),               # 16 experts
        (dict(n_group=16, topk_group=4), pkg.LMOE_ERR_INVALID_ARG),  # groups of one
        (dict(n_group=8, topk_group=1), pkg.LMOE_ERR_INVALID_ARG),   # K = 4 > 2 eligible
        (dict(n_routed_experts=256, n_group=128, topk_group=2), pkg.LMOE_ERR_UNSUPPORTED),
        (dict(hidden_size=200), pkg.LMOE_ERR_UNSUPPORTED),
        (dict(moe_intermediate_size=96), pkg.LMOE_ERR_UNSUPPORTED),
        (dict(n_routed_experts=2048), pkg.LMOE_ERR_UNSUPPORTED),
        (dict(n_routed_experts=24), pkg.LMOE_ERR_UNSUPPORTED),
        (dict(num_experts_per_tok=17), pkg.LMOE_ERR_UNSUPPORTED),
        (dict(num_experts_per_tok=0), pkg.LMOE_ERR_INVALID_ARG),
        (dict(path=pkg.PATH_TILED), pkg.LMOE_ERR_UNSUPPORTED),  # tiny R=64 < tile
    ]:
        c = cfg(**bad)
        assert lib.lmoe_workspace_size(ctypes.byref(c)) == 0, bad
        st, h = create(lib, c, nbytes=1 << 30)
        assert st == status, (bad, st)
        assert not h.value


def test_create_argument_errors(lib):
    c = cfg()
    need = lib.lmoe_workspace_size(ctypes.byref(c))
    assert create(lib, c, weights(expert_up=None))[0] == pkg.LMOE_ERR_INVALID_ARG
    assert create(lib, c, weights(router=FAKE + 4))[0] == pkg.LMOE_ERR_INVALID_ARG
    assert create(lib, c, ws=None)[0] == pkg.LMOE_ERR_WORKSPACE
    assert create(lib, c, nbytes=need - 1)[0] == pkg.LMOE_ERR_WORKSPACE
    assert create(lib, c, ws=FAKE + 16)[0] == pkg.LMOE_ERR_WORKSPACE
    assert lib.lmoe_create(ctypes.byref(c), ctypes.byref(weights()), FAKE, need,
                           None) == pkg.LMOE_ERR_INVALID_ARG
    st, h = create(lib, c)
    assert created(st, h)
    lib.lmoe_destroy(h)
    lib.lmoe_destroy(None)


def test_mxfp4_config_weights_and_quantiser_argument_errors(lib):
    # expert format: a known value, and (MXFP4) latent / expert widths multiple of 128
    st, _ = create(lib, cfg(expert_format=7))
    assert st == pkg.LMOE_ERR_INVALID_ARG
    assert lib.lmoe_workspace_size(ctypes.byref(cfg(expert_format=pkg.EXPERTS_MXFP4))) == 0
    mx_shape = li.LayerShape(256, 128, 16, 4, 256, 512, 5.0)
    c = pkg.make_config(mx_shape, 64, expert_format=pkg.EXPERTS_MXFP4)
    assert lib.lmoe_workspace_size(ctypes.byref(c)) > 0
    # MXFP4: the code and scale pointers are required (codes 16-byte aligned),
    # the bf16 expert pointers are not
    mx = dict(expert_up=None, expert_down=None, expert_up_mxfp4=FAKE, expert_up_scale=FAKE + 1,
              expert_down_mxfp4=FAKE, expert_down_scale=FAKE + 3)
    st, h = create(lib, c, weights(**mx))
    assert created(st, h)
    lib.lmoe_destroy(h)
    for bad in (dict(expert_up_mxfp4=None), dict(expert_down_scale=None),
                dict(expert_down_mxfp4=FAKE + 8)):
        assert create(lib, c, weights(**{**mx, **bad}))[0] == pkg.LMOE_ERR_INVALID_ARG
    # quantiser: cols a positive multiple of 32, rows >= 0, aligned pointers
    q = lib.lmoe_quantize_mxfp4
    assert q(FAKE, 4, 48, FAKE, FAKE, None) == pkg.LMOE_ERR_INVALID_ARG
    assert q(FAKE, 4, 0, FAKE, FAKE, None) == pkg.LMOE_ERR_INVALID_ARG
    assert q(FAKE, -1, 64, FAKE, FAKE, None) == pkg.LMOE_ERR_INVALID_ARG
    assert q(FAKE, 0, 64, None, None, None) == pkg.LMOE_OK      # no rows, no launch
    assert q(None, 4, 64, FAKE, FAKE, None) == pkg.LMOE_ERR_INVALID_ARG
    assert q(FAKE + 2, 4, 64, FAKE, FAKE, None) == pkg.LMOE_ERR_INVALID_ARG
    assert q(FAKE, 4, 64, FAKE + 8, FAKE, None) == pkg.LMOE_ERR_INVALID_ARG
    assert q(FAKE, 4, 64, FAKE, None, None) == pkg.LMOE_ERR_INVALID_ARG


def test_block_fusion_config_and_weights(lib):
    # fuse bits: PRENORM (needs a finite eps >= 0 and the norm weight) and RESIDUAL
    base = lib.lmoe_workspace_size(ctypes.byref(cfg()))
    pre = lib.lmoe_workspace_size(ctypes.byref(cfg(fuse=pkg.FUSE_BLOCK)))
    assert pre > base                                       # xt [T, D] and 1/rms [T]
    assert lib.lmoe_workspace_size(ctypes.byref(cfg(fuse=pkg.FUSE_RESIDUAL))) == base
    for bad in (dict(fuse=4), dict(fuse=-1), dict(fuse=pkg.FUSE_PRENORM, norm_eps=-1.0),
                dict(fuse=pkg.FUSE_PRENORM, norm_eps=float("inf")),
                dict(fuse=pkg.FUSE_PRENORM, norm_eps=float("nan"))):
        c = cfg(**bad)
        assert lib.lmoe_workspace_size(ctypes.byref(c)) == 0, bad
        assert create(lib, c, nbytes=1 << 30)[0] == pkg.LMOE_ERR_INVALID_ARG, bad
    # a negative eps is fine when the pre-norm is not fused (the field is unused)
    assert lib.lmoe_workspace_size(ctypes.byref(cfg(fuse=pkg.FUSE_RESIDUAL, norm_eps=-1.0))) > 0
    c = cfg(fuse=pkg.FUSE_BLOCK, norm_eps=0.0)
    assert create(lib, c)[0] == pkg.LMOE_ERR_INVALID_ARG             # no norm weight
    assert create(lib, c, weights(norm_weight=FAKE + 2))[0] == pkg.LMOE_ERR_INVALID_ARG
    st, h = create(lib, c, weights(norm_weight=FAKE))
    assert created(st, h)
    lib.lmoe_destroy(h)
    st, h = create(lib, cfg(fuse=pkg.FUSE_RESIDUAL))           # residual alone: no weight needed
    assert created(st, h)
    lib.lmoe_destroy(h)


@pytest.mark.gpu
def test_forward_and_route_argument_errors(lib):
    c = cfg()
    st, h = create(lib, c)
    assert st == pkg.LMOE_OK
    D = c.hidden_size
    x, y = FAKE, FAKE + 64 * D * 2 + 4096
    f = lib.lmoe_forward
    assert f(None, x, 4, y, None, None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(h, x, -1, y, None, None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(h, x, 65, y, None, None) == pkg.LMOE_ERR_TOO_MANY_TOKENS
    assert f(h, x, 0, y, None, None) == pkg.LMOE_OK          # no-op, no launch
    assert f(h, None, 4, y, None, None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(h, x, 4, None, None, None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(h, x, 4, x, None, None) == pkg.LMOE_ERR_INVALID_ARG      # y == x
    assert f(h, x, 4, x + 2 * D, None, None) == pkg.LMOE_ERR_INVALID_ARG  # overlap
    assert f(h, x + 2, 4, y, None, None) == pkg.LMOE_ERR_INVALID_ARG  # misaligned
    bad_taps = pkg.LmoeTaps(None, FAKE + 8, None, None, None)
    assert f(h, x, 4, y, None, ctypes.byref(bad_taps)) == pkg.LMOE_ERR_INVALID_ARG
    r = lib.lmoe_route
    assert r(None, FAKE, 4, FAKE, FAKE, None) == pkg.LMOE_ERR_INVALID_ARG
    assert r(h, FAKE, 65, FAKE, FAKE, None) == pkg.LMOE_ERR_TOO_MANY_TOKENS
    assert r(h, FAKE, 0, FAKE, FAKE, None) == pkg.LMOE_OK
    assert r(h, None, 4, FAKE, FAKE, None) == pkg.LMOE_ERR_INVALID_ARG
    assert r(h, FAKE, 4, FAKE + 4, FAKE, None) == pkg.LMOE_ERR_INVALID_ARG
    lib.lmoe_destroy(h)


def test_noalloc_forward_argument_errors(lib):
    """lmoe_forward_noalloc checks cfg, weights, T, x and y on the host, and
    rejects a forward whose scratch exceeds the static array, before any HIP
    call (the full-shape layer at T = 192 needs ~130 MB against 64 MiB)."""
    f = lib.lmoe_forward_noalloc
    c = cfg()
    w = weights()
    D = c.hidden_size
    x, y = FAKE, FAKE + 64 * D * 2 + 4096
    assert f(None, ctypes.byref(w), x, 4, y, None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(cfg(path=7)), ctypes.byref(w), x, 4, y, None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(c), None, x, 4, y, None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(c), ctypes.byref(weights(router=None)), x, 4, y,
             None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(c), ctypes.byref(w), x, -1, y, None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(c), ctypes.byref(w), x, 65, y, None) == pkg.LMOE_ERR_TOO_MANY_TOKENS
    assert f(ctypes.byref(c), ctypes.byref(w), x, 0, y, None) == pkg.LMOE_OK   # no-op
    assert f(ctypes.byref(c), ctypes.byref(w), None, 4, y, None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(c), ctypes.byref(w), x + 2, 4, y, None) == pkg.LMOE_ERR_INVALID_ARG
    assert f(ctypes.byref(c), ctypes.byref(w), x, 4, x + 2 * D, None) == pkg.LMOE_ERR_INVALID_ARG
    full = pkg.make_config(li.FULL, 256)
    fx, fy = FAKE, FAKE + (1 << 30)
    assert f(ctypes.byref(full), ctypes.byref(w), fx, 192, fy, None) == pkg.LMOE_ERR_SCRATCH
    # the limit is the workspace a handle for exactly T tokens would need
    for T, fits in ((32, True), (192, False)):
        need = lib.lmoe_workspace_size(ctypes.byref(pkg.make_config(li.FULL, T)))
        assert (need <= pkg.NOALLOC_SCRATCH_BYTES) == fits


def test_status_strings_and_stages(lib):
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert lib.lmoe_status_string(s)
    assert lib.lmoe_status_string(99) == b"unknown status"
    names = pkg.stage_names()
    assert names[0] == "proj_latent" and "expert_up" in names and "shared_up" in names and len(names) == lib.lmoe_num_stages()
    assert lib.lmoe_stage_name(-1) is None
    assert lib.lmoe_profile_begin(None, 4) == pkg.LMOE_ERR_INVALID_ARG
    ms = (ctypes.c_float * 16)()
    n = ctypes.c_int32()
    assert lib.lmoe_profile_end(None, ms, 16, ctypes.byref(n)) == pkg.LMOE_ERR_INVALID_ARG


def test_product_path_does_not_reach_the_oracle():
    for dirpath, _, files in os.walk(os.path.join(ROOT, "sparse_moe_layer_latentmoe_amd")):
        for fn in files:
            if fn.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(dirpath, fn), encoding="utf-8").read()
                assert "oracle" not in text.replace("no oracle", ""), fn
