"""ctypes binding of libst_block.so (declared in include/st_block.h).

Argument marshalling only: every step of the block runs in the library's HIP
kernels.  PyTorch supplies device memory (tensor data pointers) and streams
(``torch.cuda.current_stream().cuda_stream``, a hipStream_t under ROCm).  If
the shared library is missing, every entry point raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libst_block.so")

ST_OK, ST_ERR_INVALID, ST_ERR_UNSUPPORTED, ST_ERR_OUT_OF_MEMORY, ST_ERR_DEVICE = range(5)
ST_DTYPE_BF16, ST_DTYPE_F32 = 0, 1
STATUS_NAMES = {0: "ST_OK", 1: "ST_ERR_INVALID", 2: "ST_ERR_UNSUPPORTED",
                3: "ST_ERR_OUT_OF_MEMORY", 4: "ST_ERR_DEVICE"}

KERNEL_KINDS = ("gn_stats", "proj_in", "layernorm", "qkv", "self_attn",
                "attn_out", "cross_q", "ctx_kv", "cross_attn", "ff1_geglu",
                "ff2", "proj_out")
K_SELF_ATTN = KERNEL_KINDS.index("self_attn")

LAYER_FIELDS = ("ln1_w", "ln1_b", "q1_w", "k1_w", "v1_w", "q1_b", "k1_b",
                "v1_b", "o1_w", "o1_b", "ln2_w", "ln2_b", "q2_w", "q2_b",
                "k2_w", "v2_w", "k2_b", "v2_b", "o2_w", "o2_b", "ln3_w",
                "ln3_b", "ff1_w", "ff1_b", "ff2_w", "ff2_b")
BLOCK_FIELDS = ("gn_w", "gn_b", "proj_in_w", "proj_in_b", "proj_out_w",
                "proj_out_b")

# Every function include/st_block.h declares.
EXPORTS = ("st_block_create", "st_block_forward", "st_block_forward_stage",
           "st_block_destroy", "st_last_error", "st_block_set_timing",
           "st_block_read_timing")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BLOCK_FIELDS] + [
        ("layers", ctypes.POINTER(LayerWeights))]


class Timing(ctypes.Structure):
    _fields_ = [("ms", ctypes.c_double * len(KERNEL_KINDS)),
                ("launches", ctypes.c_longlong * len(KERNEL_KINDS))]


class STError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libst_block.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build the HIP library first "
            "(python -m latent_diffusion_net_amd.build)")
    # torch ships its own HIP runtime; load it first so that the library binds
    # to that one instead of bringing a second runtime into the process.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    vp, i, u = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint
    lib.st_block_create.argtypes = [i, i, i, i, i, i, i, i,
                                    ctypes.POINTER(BlockWeights), vp,
                                    ctypes.POINTER(vp)]
    lib.st_block_create.restype = i
    lib.st_block_forward.argtypes = [vp, vp, vp, vp, vp]
    lib.st_block_forward.restype = i
    lib.st_block_forward_stage.argtypes = [vp, vp, vp, i, vp, vp]
    lib.st_block_forward_stage.restype = i
    lib.st_block_destroy.argtypes = [vp]
    lib.st_block_destroy.restype = None
    lib.st_last_error.argtypes = []
    lib.st_last_error.restype = ctypes.c_char_p
    lib.st_block_set_timing.argtypes = [vp, u]
    lib.st_block_set_timing.restype = i
    lib.st_block_read_timing.argtypes = [vp, ctypes.POINTER(Timing)]
    lib.st_block_read_timing.restype = i
    _lib = lib
    return lib


def last_error() -> str:
    return load_library().st_last_error().decode()


def _check(status: int):
    if status != ST_OK:
        raise STError(status, last_error())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return int(t.data_ptr())


def _stream_handle(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    h = getattr(stream, "cuda_stream", stream)
    return int(h) if h else None


class STBlock:
    """One Spatial-Transformer block instance (owns a library handle).

    ``params`` holds device tensors of the handle's dtype (torch.bfloat16 or
    torch.float32) with the names of ``BLOCK_FIELDS`` plus ``layers``, a list
    of dicts with the names of ``LAYER_FIELDS``; missing biases, gammas and
    betas are passed as NULL.  The library copies the weights.
    """

    def __init__(self, B, C, H, W, heads, D_ctx, depth, dtype: str,
                 params: Dict, stream=None):
        self._lib = load_library()
        self._h = None
        self.shape = (B, C, H, W)
        self.heads, self.D_ctx, self.depth, self.dtype = heads, D_ctx, depth, dtype
        layers = (LayerWeights * max(depth, 1))()
        for li in range(min(depth, len(params.get("layers", [])))):
            lw = params["layers"][li]
            for n in LAYER_FIELDS:
                setattr(layers[li], n, _ptr(lw.get(n)))
        bw = BlockWeights()
        for n in BLOCK_FIELDS:
            setattr(bw, n, _ptr(params.get(n)))
        bw.layers = ctypes.cast(layers, ctypes.POINTER(LayerWeights))
        handle = ctypes.c_void_p()
        dt = ST_DTYPE_BF16 if dtype == "bf16" else ST_DTYPE_F32
        st = self._lib.st_block_create(B, C, H, W, heads, D_ctx, depth, dt,
                                       ctypes.byref(bw), _stream_handle(stream),
                                       ctypes.byref(handle))
        _check(st)
        self._h = handle

    @property
    def handle(self):
        return self._h

    def forward(self, x, ctx, y=None, stream=None):
        """Enqueue y = block(x, ctx) on ``stream`` (default: torch's current)."""
        import torch
        if y is None:
            y = torch.empty_like(x)
        _check(self._lib.st_block_forward(self._h, _ptr(x), _ptr(ctx), _ptr(y),
                                          _stream_handle(stream)))
        return y

    def forward_stage(self, x, ctx, stage: int, stream=None):
        """fp32 residual stream [B*H*W, C] after ``stage`` (0 = proj_in)."""
        import torch
        B, C, H, W = self.shape
        h = torch.empty((B * H * W, C), dtype=torch.float32, device=x.device)
        _check(self._lib.st_block_forward_stage(self._h, _ptr(x), _ptr(ctx),
                                                stage, _ptr(h),
                                                _stream_handle(stream)))
        return h

    def set_timing(self, kinds=()):
        mask = 0
        for k in kinds:
            mask |= 1 << (KERNEL_KINDS.index(k) if isinstance(k, str) else int(k))
        _check(self._lib.st_block_set_timing(self._h, mask))

    def read_timing(self) -> Dict[str, Dict[str, float]]:
        t = Timing()
        _check(self._lib.st_block_read_timing(self._h, ctypes.byref(t)))
        return {k: {"ms": t.ms[i], "launches": t.launches[i]}
                for i, k in enumerate(KERNEL_KINDS) if t.launches[i]}

    def close(self):
        if self._h is not None:
            self._lib.st_block_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def params_to_device(params: Dict, dtype: str, device="cuda"):
    """Copy a NumPy parameter tree (float32 arrays) to device tensors."""
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32

    def conv(a):
        return torch.from_numpy(a).to(device=device).to(tdt).contiguous()

    out = {k: conv(v) for k, v in params.items() if k != "layers"}
    out["layers"] = [{k: conv(v) for k, v in lw.items()} for lw in params["layers"]]
    return out


def array_to_device(a, dtype: str, device="cuda"):
    import torch
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    return torch.from_numpy(a).to(device=device).to(tdt).contiguous()
