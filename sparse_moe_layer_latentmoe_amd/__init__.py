"""LatentMoE feed-forward layer (forward pass) for AMD MI355X (gfx950).

A thin ctypes binding over the C ABI of ``liblmoe.so`` (declared in
``include/lmoe.h``).  The binding only marshals arguments: every step of the
layer runs in the library's HIP kernels.  PyTorch is used to own device
memory (weights, workspace, inputs, outputs) and to name the HIP stream.

The library must have been built (``python -m
sparse_moe_layer_latentmoe_amd._build`` or ``__graft_entry__.build()``);
loading fails loudly if it is missing -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblmoe.so")

LMOE_OK = 0
LMOE_ERR_INVALID_ARG = -1
LMOE_ERR_UNSUPPORTED = -2
LMOE_ERR_TOO_MANY_TOKENS = -3
LMOE_ERR_WORKSPACE = -4
LMOE_ERR_HIP = -5
LMOE_ERR_SCRATCH = -6
NOALLOC_SCRATCH_BYTES = 64 << 20      # LMOE_NOALLOC_SCRATCH_BYTES

PATH_AUTO, PATH_STREAM, PATH_TILED = 0, 1, 2
EXPERTS_BF16, EXPERTS_MXFP4 = 0, 1
FUSE_PRENORM, FUSE_RESIDUAL = 1, 2      # lmoe_fuse bits
FUSE_BLOCK = FUSE_PRENORM | FUSE_RESIDUAL

EXPORTED = (
    "lmoe_workspace_size", "lmoe_create", "lmoe_forward", "lmoe_route", "lmoe_destroy",
    "lmoe_status_string", "lmoe_num_stages", "lmoe_stage_name", "lmoe_profile_begin",
    "lmoe_profile_end", "lmoe_quantize_mxfp4", "lmoe_forward_noalloc",
)


class LmoeConfig(ctypes.Structure):
    _fields_ = [
        ("hidden_size", ctypes.c_int32),
        ("moe_latent_size", ctypes.c_int32),
        ("n_routed_experts", ctypes.c_int32),
        ("num_experts_per_tok", ctypes.c_int32),
        ("moe_intermediate_size", ctypes.c_int32),
        ("moe_shared_expert_intermediate_size", ctypes.c_int32),
        ("n_group", ctypes.c_int32),
        ("topk_group", ctypes.c_int32),
        ("routed_scaling_factor", ctypes.c_float),
        ("max_tokens", ctypes.c_int32),
        ("path", ctypes.c_int32),
        ("expert_format", ctypes.c_int32),
        ("fuse", ctypes.c_int32),
        ("norm_eps", ctypes.c_float),
    ]


class LmoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "fc1_latent", "router", "router_bias", "expert_up", "expert_down",
        "fc2_latent", "shared_up", "shared_down", "expert_up_mxfp4", "expert_up_scale",
        "expert_down_mxfp4", "expert_down_scale", "norm_weight")]


class LmoeTaps(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "z_f32", "topk_idx", "topk_w", "expert_counts", "r_latent")]


class LmoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblmoe.so and declare its C signatures (raises if it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m sparse_moe_layer_latentmoe_amd._build)")
    # torch ships its own HIP runtime under the same soname as the system's;
    # whichever is loaded first serves the whole process.  Importing torch
    # first keeps torch on the runtime it was built with (loading this
    # library first made torch's allocations unusable for its launches).
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.lmoe_workspace_size.argtypes = [ctypes.POINTER(LmoeConfig)]
    lib.lmoe_workspace_size.restype = ctypes.c_size_t
    lib.lmoe_create.argtypes = [ctypes.POINTER(LmoeConfig), ctypes.POINTER(LmoeWeights), P,
                                ctypes.c_size_t, ctypes.POINTER(P)]
    lib.lmoe_create.restype = ctypes.c_int
    lib.lmoe_forward.argtypes = [P, P, ctypes.c_int32, P, P, ctypes.POINTER(LmoeTaps)]
    lib.lmoe_forward.restype = ctypes.c_int
    lib.lmoe_route.argtypes = [P, P, ctypes.c_int32, P, P, P]
    lib.lmoe_route.restype = ctypes.c_int
    lib.lmoe_destroy.argtypes = [P]
    lib.lmoe_destroy.restype = None
    lib.lmoe_status_string.argtypes = [ctypes.c_int]
    lib.lmoe_status_string.restype = ctypes.c_char_p
    lib.lmoe_num_stages.argtypes = []
    lib.lmoe_num_stages.restype = ctypes.c_int32
    lib.lmoe_stage_name.argtypes = [ctypes.c_int32]
    lib.lmoe_stage_name.restype = ctypes.c_char_p
    lib.lmoe_profile_begin.argtypes = [P, ctypes.c_int32]
    lib.lmoe_profile_begin.restype = ctypes.c_int
    lib.lmoe_profile_end.argtypes = [P, ctypes.POINTER(ctypes.c_float), ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_int32)]
    lib.lmoe_profile_end.restype = ctypes.c_int
    lib.lmoe_quantize_mxfp4.argtypes = [P, ctypes.c_int64, ctypes.c_int32, P, P, P]
    lib.lmoe_quantize_mxfp4.restype = ctypes.c_int
    lib.lmoe_forward_noalloc.argtypes = [ctypes.POINTER(LmoeConfig), ctypes.POINTER(LmoeWeights),
                                         P, ctypes.c_int32, P, P]
    lib.lmoe_forward_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().lmoe_status_string(status).decode()


def stage_names() -> list:
    lib = load_library()
    return [lib.lmoe_stage_name(i).decode() for i in range(lib.lmoe_num_stages())]


def make_config(shape, max_tokens: int, path: int = PATH_AUTO,
                expert_format: int = EXPERTS_BF16, fuse: int = 0,
                norm_eps: float = 1e-5) -> LmoeConfig:
    """Config struct from any object with the model's config-key attributes."""
    return LmoeConfig(
        shape.hidden_size, shape.moe_latent_size, shape.n_routed_experts,
        shape.num_experts_per_tok, shape.moe_intermediate_size,
        shape.moe_shared_expert_intermediate_size, int(getattr(shape, "n_group", 1)),
        int(getattr(shape, "topk_group", 1)),
        float(shape.routed_scaling_factor), int(max_tokens), int(path), int(expert_format),
        int(fuse), float(norm_eps))


def workspace_size(cfg: LmoeConfig) -> int:
    return int(load_library().lmoe_workspace_size(ctypes.byref(cfg)))


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _stream_handle(stream) -> int | None:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    return int(getattr(stream, "cuda_stream", stream))


@dataclass
class Taps:
    """Optional device outputs (torch tensors) of one forward."""
    z_f32: object = None
    topk_idx: object = None
    topk_w: object = None
    expert_counts: object = None
    r_latent: object = None

    def as_struct(self) -> LmoeTaps:
        return LmoeTaps(_ptr(self.z_f32), _ptr(self.topk_idx), _ptr(self.topk_w),
                        _ptr(self.expert_counts), _ptr(self.r_latent))


def quantize_mxfp4(w, stream=None):
    """MXFP4 codes and block scales of a bf16 matrix [..., K] (K a multiple
    of 32), quantised along its last axis by the library's kernel:
    (codes uint8 [..., K/2], scales uint8 [..., K/32]) on w's device."""
    import torch
    if getattr(w, "dim", lambda: 0)() < 1:
        raise ValueError("w: expected a tensor of at least one dimension")
    _expect(w, tuple(w.shape), torch.bfloat16, "w", contiguous=False)
    w = w.contiguous()
    K = int(w.shape[-1])
    rows = w.numel() // K if K else 0
    codes = torch.empty(*w.shape[:-1], K // 2, dtype=torch.uint8, device=w.device)
    scales = torch.empty(*w.shape[:-1], K // 32, dtype=torch.uint8, device=w.device)
    st = load_library().lmoe_quantize_mxfp4(_ptr(w), rows, K, _ptr(codes), _ptr(scales),
                                            _stream_handle(stream))
    if st != LMOE_OK:
        raise LmoeError(st, "lmoe_quantize_mxfp4")
    return codes, scales


def _expect(t, shape, dtype, what: str, contiguous: bool = True, device=None,
            on_gpu: bool = True) -> None:
    """Raise unless ``t`` is a GPU tensor of this dtype and shape (and
    contiguous, and on ``device``, when asked): the C ABI takes bare
    pointers, so a tensor of the wrong size or type would be read or written
    out of bounds on the device."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{what}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{what}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{what}: must be contiguous")
    if on_gpu and t.device.type != "cuda":
        raise ValueError(f"{what}: must be a GPU tensor, got one on {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{what}: on {t.device}, the layer is on {device}")


def weight_specs(shape, expert_format: int = EXPERTS_BF16, fuse: int = 0) -> dict:
    """{lmoe_weights field: (shape, torch dtype)} of the weights a layer with
    this shape, expert format and fusion needs (the layouts of lmoe.h)."""
    import torch
    D, R, E = shape.hidden_size, shape.moe_latent_size, shape.n_routed_experts
    F, S = shape.moe_intermediate_size, shape.moe_shared_expert_intermediate_size
    bf16, f32, u8 = torch.bfloat16, torch.float32, torch.uint8
    spec = {"fc1_latent": ((R, D), bf16), "router": ((E, R), f32), "router_bias": ((E,), f32),
            "fc2_latent": ((D, R), bf16), "shared_up": ((S, D), bf16),
            "shared_down": ((D, S), bf16)}
    if expert_format == EXPERTS_MXFP4:
        spec.update(expert_up_mxfp4=((E, F, R // 2), u8), expert_up_scale=((E, F, R // 32), u8),
                    expert_down_mxfp4=((E, R, F // 2), u8),
                    expert_down_scale=((E, R, F // 32), u8))
    else:
        spec.update(expert_up=((E, F, R), bf16), expert_down=((E, R, F), bf16))
    if fuse & FUSE_PRENORM:
        spec["norm_weight"] = ((D,), bf16)
    return spec


def check_weights(shape, weights: dict, expert_format: int = EXPERTS_BF16, fuse: int = 0,
                  device=None) -> None:
    """Raise unless ``weights`` holds every tensor the layer needs with the
    right shape and dtype, on one GPU (non-contiguous ones are copied by the
    layer)."""
    spec = weight_specs(shape, expert_format, fuse)
    for name, (shp, dt) in spec.items():        # presence, dtype and shape first
        if weights.get(name) is None:
            raise ValueError(f"weights[{name!r}] is required")
        _expect(weights[name], shp, dt, f"weights[{name!r}]", contiguous=False, on_gpu=False)
    for name, (shp, dt) in spec.items():        # then where they live
        _expect(weights[name], shp, dt, f"weights[{name!r}]", contiguous=False, device=device)


class LatentMoE:
    """One LatentMoE layer bound to caller-owned device weights.

    ``weights`` maps the lmoe_weights field names to contiguous device
    tensors (bf16, the router and its bias fp32).  The workspace is a
    uint8 device tensor allocated here with torch; the library itself never
    allocates.  ``fuse`` (FUSE_PRENORM | FUSE_RESIDUAL bits) makes the
    forward take the block's residual stream h and return h + layer(
    RMSNorm(h)); the pre-norm needs ``weights["norm_weight"]`` (bf16 [D])."""

    def __init__(self, shape, weights: dict, max_tokens: int, path: int = PATH_AUTO,
                 device=None, expert_format: int = EXPERTS_BF16, fuse: int = 0,
                 norm_eps: float = 1e-5):
        import torch
        self.lib = load_library()
        self.shape = shape
        self.cfg = make_config(shape, max_tokens, path, expert_format, fuse, norm_eps)
        ws_bytes = workspace_size(self.cfg)
        if ws_bytes == 0:
            raise LmoeError(LMOE_ERR_UNSUPPORTED, "lmoe_workspace_size")
        if device is None:
            check_weights(shape, weights, expert_format, fuse)
            dev = weights["fc1_latent"].device
        else:
            dev = torch.device(device)
            if dev.index is None:
                dev = torch.device(dev.type, torch.cuda.current_device())
        check_weights(shape, weights, expert_format, fuse, dev)
        self.device = dev
        self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        self.weights = {k: v.contiguous() for k, v in weights.items() if v is not None}
        self.wstruct = LmoeWeights(*[_ptr(self.weights.get(n)) for n, _ in LmoeWeights._fields_])
        h = ctypes.c_void_p()
        st = self.lib.lmoe_create(ctypes.byref(self.cfg), ctypes.byref(self.wstruct),
                                  _ptr(self.workspace), ws_bytes, ctypes.byref(h))
        if st != LMOE_OK:
            raise LmoeError(st, "lmoe_create")
        self.handle = h

    def close(self):
        if getattr(self, "handle", None):
            self.lib.lmoe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def forward_into(self, x, y, taps: Taps | None = None, stream=None) -> None:
        """y <- LatentMoE(x); x, y bf16 [T, D] device tensors."""
        import torch
        sh = self.shape
        T = int(x.shape[0]) if getattr(x, "dim", lambda: 0)() == 2 else -1
        D, R, K = sh.hidden_size, sh.moe_latent_size, sh.num_experts_per_tok
        _expect(x, (T, D), torch.bfloat16, "x", device=self.device)
        _expect(y, (T, D), torch.bfloat16, "y", device=self.device)
        if taps is not None:
            for name, shp, dt in (("z_f32", (T, R), torch.float32),
                                  ("topk_idx", (T, K), torch.int32),
                                  ("topk_w", (T, K), torch.float32),
                                  ("expert_counts", (sh.n_routed_experts,), torch.int32),
                                  ("r_latent", (T, R), torch.float32)):
                t = getattr(taps, name)
                if t is not None:
                    _expect(t, shp, dt, f"taps.{name}", device=self.device)
        ts = taps.as_struct() if taps is not None else None
        st = self.lib.lmoe_forward(self.handle, _ptr(x), int(x.shape[0]), _ptr(y),
                                   _stream_handle(stream),
                                   ctypes.byref(ts) if ts is not None else None)
        if st != LMOE_OK:
            raise LmoeError(st, "lmoe_forward")

    def forward_noalloc_into(self, x, y, stream=None) -> None:
        """y <- LatentMoE(x) through lmoe_forward_noalloc: the same forward
        without the handle's workspace or auxiliary stream, its scratch in the
        library's static device array (raises LmoeError with LMOE_ERR_SCRATCH
        when T tokens need more than NOALLOC_SCRATCH_BYTES)."""
        import torch
        sh = self.shape
        T = int(x.shape[0]) if getattr(x, "dim", lambda: 0)() == 2 else -1
        _expect(x, (T, sh.hidden_size), torch.bfloat16, "x", device=self.device)
        _expect(y, (T, sh.hidden_size), torch.bfloat16, "y", device=self.device)
        st = self.lib.lmoe_forward_noalloc(ctypes.byref(self.cfg), ctypes.byref(self.wstruct),
                                           _ptr(x), T, _ptr(y), _stream_handle(stream))
        if st != LMOE_OK:
            raise LmoeError(st, "lmoe_forward_noalloc")

    def forward(self, x, taps: Taps | None = None, stream=None):
        import torch
        y = torch.empty_like(x)
        self.forward_into(x, y, taps, stream)
        return y

    __call__ = forward

    def route(self, z_f32, stream=None):
        """(topk_idx int32 [T, K], topk_w fp32 [T, K]) from a given fp32 latent."""
        import torch
        T = int(z_f32.shape[0]) if getattr(z_f32, "dim", lambda: 0)() == 2 else -1
        K = self.shape.num_experts_per_tok
        _expect(z_f32, (T, self.shape.moe_latent_size), torch.float32, "z_f32",
                device=self.device)
        idx = torch.empty((T, K), dtype=torch.int32, device=z_f32.device)
        w = torch.empty((T, K), dtype=torch.float32, device=z_f32.device)
        st = self.lib.lmoe_route(self.handle, _ptr(z_f32), T, _ptr(idx), _ptr(w),
                                 _stream_handle(stream))
        if st != LMOE_OK:
            raise LmoeError(st, "lmoe_route")
        return idx, w

    def profile_begin(self, max_forwards: int) -> None:
        st = self.lib.lmoe_profile_begin(self.handle, int(max_forwards))
        if st != LMOE_OK:
            raise LmoeError(st, "lmoe_profile_begin")

    def profile_end(self):
        """{stage name: summed ms}, number of forwards recorded."""
        n = self.lib.lmoe_num_stages()
        ms = (ctypes.c_float * n)()
        nf = ctypes.c_int32()
        st = self.lib.lmoe_profile_end(self.handle, ms, n, ctypes.byref(nf))
        if st != LMOE_OK:
            raise LmoeError(st, "lmoe_profile_end")
        return dict(zip(stage_names(), list(ms))), int(nf.value)
