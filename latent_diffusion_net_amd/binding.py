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

(ST_OK, ST_ERR_INVALID, ST_ERR_UNSUPPORTED, ST_ERR_OUT_OF_MEMORY, ST_ERR_DEVICE,
 ST_ERR_RANGE) = range(6)
ST_DTYPE_BF16, ST_DTYPE_F32 = 0, 1
STATUS_NAMES = {0: "ST_OK", 1: "ST_ERR_INVALID", 2: "ST_ERR_UNSUPPORTED",
                3: "ST_ERR_OUT_OF_MEMORY", 4: "ST_ERR_DEVICE", 5: "ST_ERR_RANGE"}

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

# Every function include/st_block.h and include/st_ops.h declare.
EXPORTS = ("st_block_create", "st_block_forward", "st_block_forward_masked",
           "st_block_forward_stage",
           "st_block_destroy", "st_block_check_range", "st_last_error",
           "st_block_set_timing", "st_block_set_timing_layers", "st_block_read_timing",
           "st_block_read_timing_launches", "st_measure_mfma_bf16",
           "st_group_norm_workspace_bytes", "st_group_norm", "st_group_norm_noalloc",
           "st_guided_ddpm_step", "st_resnet_create", "st_resnet_forward",
           "st_resnet_check_range", "st_resnet_destroy", "st_unet_create",
           "st_unet_forward", "st_unet_device_bytes", "st_unet_check_range",
           "st_unet_destroy")


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in LAYER_FIELDS]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BLOCK_FIELDS] + [
        ("layers", ctypes.POINTER(LayerWeights))]


RESNET_FIELDS = ("gn1_w", "gn1_b", "conv1_w", "conv1_b", "temb_w", "temb_b", "gn2_w",
                 "gn2_b", "conv2_w", "conv2_b", "sc_w", "sc_b")


class ResnetWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in RESNET_FIELDS]


class UNetConfigC(ctypes.Structure):
    _fields_ = [("in_channels", ctypes.c_int), ("out_channels", ctypes.c_int),
                ("levels", ctypes.c_int), ("channels", ctypes.c_int * 4),
                ("depths", ctypes.c_int * 4), ("mid_depth", ctypes.c_int),
                ("layers_per_block", ctypes.c_int), ("ctx_dim", ctypes.c_int),
                ("add_in", ctypes.c_int)]


class UNetWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "time1_w", "time1_b", "time2_w", "time2_b", "add1_w", "add1_b", "add2_w", "add2_b",
        "conv_in_w", "conv_in_b")] + [
        ("resnets", ctypes.POINTER(ResnetWeights)), ("blocks", ctypes.POINTER(BlockWeights)),
        ("down_w", ctypes.POINTER(ctypes.c_void_p)), ("down_b", ctypes.POINTER(ctypes.c_void_p)),
        ("up_w", ctypes.POINTER(ctypes.c_void_p)), ("up_b", ctypes.POINTER(ctypes.c_void_p))] + [
        (n, ctypes.c_void_p) for n in ("norm_out_w", "norm_out_b", "conv_out_w", "conv_out_b")]


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
    lib.st_block_forward_masked.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.st_block_forward_masked.restype = i
    lib.st_block_forward_stage.argtypes = [vp, vp, vp, i, vp, vp]
    lib.st_block_forward_stage.restype = i
    lib.st_block_destroy.argtypes = [vp]
    lib.st_block_destroy.restype = None
    lib.st_last_error.argtypes = []
    lib.st_last_error.restype = ctypes.c_char_p
    lib.st_block_set_timing.argtypes = [vp, u]
    lib.st_block_set_timing.restype = i
    lib.st_block_set_timing_layers.argtypes = [vp, i]
    lib.st_block_set_timing_layers.restype = i
    lib.st_block_read_timing.argtypes = [vp, ctypes.POINTER(Timing)]
    lib.st_block_read_timing.restype = i
    ll, dbl = ctypes.c_longlong, ctypes.c_double
    lib.st_block_check_range.argtypes = [vp, vp]
    lib.st_block_check_range.restype = i
    lib.st_block_read_timing_launches.argtypes = [vp, ctypes.POINTER(i), ctypes.POINTER(dbl),
                                                  ll, ctypes.POINTER(ll)]
    lib.st_block_read_timing_launches.restype = i
    lib.st_measure_mfma_bf16.argtypes = [i, vp, ctypes.POINTER(dbl), ctypes.POINTER(dbl)]
    lib.st_measure_mfma_bf16.restype = i
    f32, sz = ctypes.c_float, ctypes.c_size_t
    lib.st_group_norm_workspace_bytes.argtypes = [i]
    lib.st_group_norm_workspace_bytes.restype = sz
    lib.st_group_norm.argtypes = [vp, vp, vp, vp, i, i, i, i, f32, i, i, vp, sz, vp]
    lib.st_group_norm.restype = i
    lib.st_resnet_create.argtypes = [i, i, i, i, i, i, f32, i, ctypes.POINTER(ResnetWeights), vp,
                                     ctypes.POINTER(vp)]
    lib.st_resnet_create.restype = i
    lib.st_resnet_forward.argtypes = [vp, vp, vp, vp, vp]
    lib.st_resnet_forward.restype = i
    lib.st_resnet_check_range.argtypes = [vp, vp]
    lib.st_resnet_check_range.restype = i
    lib.st_resnet_destroy.argtypes = [vp]
    lib.st_resnet_destroy.restype = None
    lib.st_unet_create.argtypes = [ctypes.POINTER(UNetConfigC), i, i, i, ctypes.POINTER(UNetWeights),
                                   vp, ctypes.POINTER(vp)]
    lib.st_unet_create.restype = i
    lib.st_unet_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.st_unet_forward.restype = i
    lib.st_unet_device_bytes.argtypes = [vp, ctypes.POINTER(ctypes.c_ulonglong)]
    lib.st_unet_device_bytes.restype = i
    lib.st_unet_check_range.argtypes = [vp, vp]
    lib.st_unet_check_range.restype = i
    lib.st_unet_destroy.argtypes = [vp]
    lib.st_unet_destroy.restype = None
    lib.st_group_norm_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, f32, i, i, vp]
    lib.st_group_norm_noalloc.restype = i
    lib.st_guided_ddpm_step.argtypes = [vp, i, vp, vp, vp, ll, f32, i, i, dbl, dbl, vp]
    lib.st_guided_ddpm_step.restype = i
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

    def forward_masked(self, x, ctx, ctx_mask, y=None, stream=None):
        """y = block(x, ctx) with the context key padding mask ``ctx_mask``
        ([B, 77] uint8 device tensor, nonzero = attend; None = no mask)."""
        import torch
        if y is None:
            y = torch.empty_like(x)
        _check(self._lib.st_block_forward_masked(self._h, _ptr(x), _ptr(ctx), _ptr(ctx_mask),
                                                 _ptr(y), _stream_handle(stream)))
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

    def set_timing(self, kinds=(), layers=0):
        """Time the launches of ``kinds``; the per-layer kinds only in the
        first ``layers`` layers of each forward (0 = every layer)."""
        mask = 0
        for k in kinds:
            mask |= 1 << (KERNEL_KINDS.index(k) if isinstance(k, str) else int(k))
        _check(self._lib.st_block_set_timing(self._h, mask))
        _check(self._lib.st_block_set_timing_layers(self._h, int(layers)))

    def read_timing(self) -> Dict[str, Dict[str, float]]:
        t = Timing()
        _check(self._lib.st_block_read_timing(self._h, ctypes.byref(t)))
        return {k: {"ms": t.ms[i], "launches": t.launches[i]}
                for i, k in enumerate(KERNEL_KINDS) if t.launches[i]}

    def check_range(self, stream=None):
        """Raise STError(ST_ERR_RANGE) if an fp16 intermediate of a forward
        since the last check left the fp16 range (waits for ``stream``)."""
        _check(self._lib.st_block_check_range(self._h, _stream_handle(stream)))

    def read_timing_launches(self, capacity: int = 4096):
        """[(kind name, ms)] of every recorded launch, in launch order."""
        kinds = (ctypes.c_int * capacity)()
        ms = (ctypes.c_double * capacity)()
        n = ctypes.c_longlong()
        _check(self._lib.st_block_read_timing_launches(self._h, kinds, ms, capacity,
                                                       ctypes.byref(n)))
        return [(KERNEL_KINDS[kinds[i]], ms[i]) for i in range(min(n.value, capacity))]

    def close(self):
        if self._h is not None:
            self._lib.st_block_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class STResnet:
    """One ResnetBlock2D (owns a library handle).  ``params``: device bf16
    tensors named as ``RESNET_FIELDS`` (biases, gammas and betas optional;
    sc_w / sc_b only when Cin != Cout).  The library copies the weights."""

    def __init__(self, B, Cin, Cout, H, W, Dt, params: Dict, eps: float = 1e-5, stream=None):
        self._lib = load_library()
        self._h = None
        self.shape = (B, Cin, Cout, H, W, Dt)
        w = ResnetWeights()
        for n in RESNET_FIELDS:
            setattr(w, n, _ptr(params.get(n)))
        handle = ctypes.c_void_p()
        _check(self._lib.st_resnet_create(B, Cin, Cout, H, W, Dt, eps, ST_DTYPE_BF16,
                                          ctypes.byref(w), _stream_handle(stream),
                                          ctypes.byref(handle)))
        self._h = handle

    def forward(self, x, temb, y=None, stream=None):
        import torch
        B, Cin, Cout, H, W, Dt = self.shape
        if y is None:
            y = torch.empty((B, Cout, H, W), dtype=x.dtype, device=x.device)
        _check(self._lib.st_resnet_forward(self._h, _ptr(x), _ptr(temb), _ptr(y),
                                           _stream_handle(stream)))
        return y

    def check_range(self, stream=None):
        _check(self._lib.st_resnet_check_range(self._h, _stream_handle(stream)))

    def close(self):
        if self._h is not None:
            self._lib.st_resnet_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _block_struct(bp, keep):
    layers = (LayerWeights * max(len(bp["layers"]), 1))()
    for li, lw in enumerate(bp["layers"]):
        for n in LAYER_FIELDS:
            setattr(layers[li], n, _ptr(lw.get(n)))
    keep.append(layers)
    bw = BlockWeights()
    for n in BLOCK_FIELDS:
        setattr(bw, n, _ptr(bp.get(n)))
    bw.layers = ctypes.cast(layers, ctypes.POINTER(LayerWeights))
    return bw


class STUNet:
    """One U-Net denoiser timestep (st_unet_*).  ``cfg``: a
    ``synth.UNetConfig``; ``params``: the nested tree of
    ``synth.unet_param_shapes`` holding device bf16 tensors.  The library
    copies the weights."""

    def __init__(self, cfg, B, H, W, params: Dict, stream=None):
        self._lib = load_library()
        self._h = None
        self.cfg, self.shape = cfg, (B, H, W)
        L = len(cfg.channels)
        c = UNetConfigC()
        c.in_channels, c.out_channels, c.levels = cfg.in_channels, cfg.out_channels, L
        for i in range(L):
            c.channels[i], c.depths[i] = cfg.channels[i], cfg.depths[i]
        c.mid_depth, c.layers_per_block = cfg.mid_depth, cfg.layers_per_block
        c.ctx_dim, c.add_in = cfg.ctx_dim, cfg.add_in
        keep = []
        res = [r for lv in params["down"] for r in lv["res"]] + params["mid"]["res"] + \
              [r for lv in params["up"] for r in lv["res"]]
        blk = [b for lv in params["down"] for b in lv["attn"]] + params["mid"]["attn"] + \
              [b for lv in params["up"] for b in lv["attn"]]
        rarr = (ResnetWeights * len(res))()
        for i, r in enumerate(res):
            for n in RESNET_FIELDS:
                setattr(rarr[i], n, _ptr(r.get(n)))
        barr = (BlockWeights * max(len(blk), 1))()
        for i, b in enumerate(blk):
            barr[i] = _block_struct(b, keep)
        ptrs = lambda vals: (ctypes.c_void_p * max(len(vals), 1))(*[_ptr(v) for v in vals])
        dw = ptrs([lv["down_w"] for lv in params["down"] if "down_w" in lv])
        db = ptrs([lv["down_b"] for lv in params["down"] if "down_w" in lv])
        uw = ptrs([lv["up_w"] for lv in params["up"] if "up_w" in lv])
        ub = ptrs([lv["up_b"] for lv in params["up"] if "up_w" in lv])
        w = UNetWeights()
        for n in ("time1_w", "time1_b", "time2_w", "time2_b", "add1_w", "add1_b", "add2_w",
                  "add2_b", "conv_in_w", "conv_in_b", "norm_out_w", "norm_out_b", "conv_out_w",
                  "conv_out_b"):
            setattr(w, n, _ptr(params.get(n)))
        w.resnets = ctypes.cast(rarr, ctypes.POINTER(ResnetWeights))
        w.blocks = ctypes.cast(barr, ctypes.POINTER(BlockWeights))
        cv = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_void_p))
        w.down_w, w.down_b, w.up_w, w.up_b = cv(dw), cv(db), cv(uw), cv(ub)
        handle = ctypes.c_void_p()
        _check(self._lib.st_unet_create(ctypes.byref(c), B, H, W, ctypes.byref(w),
                                        _stream_handle(stream), ctypes.byref(handle)))
        self._h = handle

    def forward(self, x, t, ctx, add=None, y=None, stream=None):
        import torch
        B, H, W = self.shape
        if y is None:
            y = torch.empty((B, self.cfg.out_channels, H, W), dtype=torch.bfloat16, device=x.device)
        _check(self._lib.st_unet_forward(self._h, _ptr(x), _ptr(t), _ptr(ctx), _ptr(add), _ptr(y),
                                         _stream_handle(stream)))
        return y

    def device_bytes(self) -> int:
        n = ctypes.c_ulonglong()
        _check(self._lib.st_unet_device_bytes(self._h, ctypes.byref(n)))
        return n.value

    def check_range(self, stream=None):
        _check(self._lib.st_unet_check_range(self._h, _stream_handle(stream)))

    def close(self):
        if self._h is not None:
            self._lib.st_unet_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def tree_to_device(tree, device="cuda"):
    """A nested dict / list of float32 arrays (None kept) -> device bf16 tensors."""
    import torch
    if isinstance(tree, dict):
        return {k: tree_to_device(v, device) for k, v in tree.items()}
    if isinstance(tree, list):
        return [tree_to_device(v, device) for v in tree]
    if tree is None:
        return None
    return torch.from_numpy(tree).to(device=device).to(torch.bfloat16).contiguous()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return ST_DTYPE_BF16
    if t.dtype == torch.float32:
        return ST_DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def group_norm(x, gamma=None, beta=None, eps: float = 1e-5, silu: bool = False,
               y=None, workspace=None, stream=None):
    """y = [SiLU](GroupNorm_32(x)) on an NCHW device tensor (st_group_norm).
    ``workspace``: a device tensor of at least st_group_norm_workspace_bytes(B)
    bytes (allocated here when None)."""
    import torch
    lib = load_library()
    B, C, H, W = x.shape
    if y is None:
        y = torch.empty_like(x)
    need = lib.st_group_norm_workspace_bytes(B)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.st_group_norm(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), B, C, H, W, eps,
                             1 if silu else 0, _dtype_code(x), _ptr(workspace), nbytes,
                             _stream_handle(stream)))
    return y


def group_norm_noalloc(x, y, gamma=None, beta=None, eps: float = 1e-5, silu: bool = False,
                       stream=None):
    """st_group_norm_noalloc: as group_norm, partial sums in the library's
    static device array (no allocation; ``y`` must be given)."""
    lib = load_library()
    B, C, H, W = x.shape
    _check(lib.st_group_norm_noalloc(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(y), B, C, H, W, eps,
                                     1 if silu else 0, _dtype_code(x), _stream_handle(stream)))
    return y


def guided_ddpm_step(eps_pair, x_t, t: int, guidance_scale: float, noise=None, x_prev=None,
                     T: int = 1000, beta_start: float = 1e-4, beta_end: float = 0.02,
                     stream=None):
    """x_{t-1} from x_t (fp32) and the pair's noise predictions [2, ...]
    (unconditional first), with guidance and the linear DDPM schedule."""
    import torch
    lib = load_library()
    if x_prev is None:
        x_prev = torch.empty_like(x_t)
    n = x_t.numel()
    _check(lib.st_guided_ddpm_step(_ptr(eps_pair), _dtype_code(eps_pair), _ptr(x_t), _ptr(noise),
                                   _ptr(x_prev), n, guidance_scale, t, T, beta_start, beta_end,
                                   _stream_handle(stream)))
    return x_prev


def measure_mfma_bf16(iters: int = 16384, stream=None):
    """(TFLOP/s, shader MHz) of a dense bf16 MFMA loop on the current device."""
    lib = load_library()
    tf, mhz = ctypes.c_double(), ctypes.c_double()
    _check(lib.st_measure_mfma_bf16(iters, _stream_handle(stream), ctypes.byref(tf),
                                    ctypes.byref(mhz)))
    return tf.value, mhz.value


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
