"""The C ABI on the CPU: the library loads, exports exactly what the header
declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

from latent_diffusion_net_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def _declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(st_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def _lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail("libst_block.so is not built (run __graft_entry__.build())")
    return binding.load_library()


def test_header_declares_binding_exports():
    assert _declared_functions() == sorted(binding.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         stdout=subprocess.PIPE, text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines()
                       if l.split() and l.split()[-1].startswith("st_")})
    assert exported == _declared_functions()


def _create(lib, B=1, C=64, H=2, W=2, heads=1, D=64, depth=1, dtype=0, w=None):
    handle = ctypes.c_void_p()
    st = lib.st_block_create(B, C, H, W, heads, D, depth, dtype,
                             ctypes.byref(w) if w is not None else None, None,
                             ctypes.byref(handle))
    return st, handle


def _fake_weights(depth=1, ptr=0x10000):
    layers = (binding.LayerWeights * depth)()
    for i in range(depth):
        for n in binding.LAYER_FIELDS:
            if n.endswith("_w") and not n.startswith("ln"):
                setattr(layers[i], n, ptr)
    bw = binding.BlockWeights()
    bw.proj_in_w = ptr
    bw.proj_out_w = ptr
    bw.layers = ctypes.cast(layers, ctypes.POINTER(binding.LayerWeights))
    return bw, layers


@pytest.mark.parametrize("kw,why", [
    (dict(B=0), "B"), (dict(H=0), "H"), (dict(W=-1), "W"),
    (dict(C=96, heads=1), "C"), (dict(C=128, heads=1), "heads"),
    (dict(D=100), "D_ctx"), (dict(D=0), "D_ctx"), (dict(depth=0), "depth"),
    (dict(dtype=7), "dtype"),
])
def test_create_rejects_bad_shapes(kw, why):
    lib = _lib()
    bw, _keep = _fake_weights()
    st, h = _create(lib, w=bw, **kw)
    assert st == binding.ST_ERR_INVALID
    assert h.value is None
    assert why in binding.last_error()


def test_create_rejects_null_and_misaligned_weights():
    lib = _lib()
    st, h = _create(lib, w=None)
    assert st == binding.ST_ERR_INVALID and h.value is None
    bw, _keep = _fake_weights()
    bw.proj_in_w = None
    st, h = _create(lib, w=bw)
    assert st == binding.ST_ERR_INVALID and "proj_in_w" in binding.last_error()
    bw, layers = _fake_weights()
    layers[0].ff2_w = 0x10008  # not 16-byte aligned
    st, h = _create(lib, w=bw)
    assert st == binding.ST_ERR_INVALID and "aligned" in binding.last_error()
    bw, _keep = _fake_weights()
    bw.layers = None
    st, h = _create(lib, w=bw)
    assert st == binding.ST_ERR_INVALID


def test_null_out_pointer():
    lib = _lib()
    bw, _keep = _fake_weights()
    st = lib.st_block_create(1, 64, 2, 2, 1, 64, 1, 0, ctypes.byref(bw), None, None)
    assert st == binding.ST_ERR_INVALID


def test_null_handle_calls():
    lib = _lib()
    assert lib.st_block_forward(None, 16, 16, 16, None) == binding.ST_ERR_INVALID
    assert lib.st_block_forward_stage(None, 16, 16, 0, 16, None) == binding.ST_ERR_INVALID
    assert lib.st_block_set_timing(None, 1) == binding.ST_ERR_INVALID
    t = binding.Timing()
    assert lib.st_block_read_timing(None, ctypes.byref(t)) == binding.ST_ERR_INVALID
    lib.st_block_destroy(None)  # NULL-safe
    assert isinstance(binding.last_error(), str)


def test_no_device_is_reported():
    """Valid arguments on a host without a GPU: ST_ERR_DEVICE, no handle.

    Only meaningful where no GPU is visible (the fake weight pointers would
    be dereferenced by a real device), so it is skipped elsewhere.
    """
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible")
    lib = _lib()
    bw, _keep = _fake_weights()
    st, h = _create(lib, w=bw)
    assert st == binding.ST_ERR_DEVICE
    assert h.value is None
    assert binding.last_error()


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        binding.load_library.__wrapped__(str(tmp_path / "nope.so")) \
            if hasattr(binding.load_library, "__wrapped__") else \
            _load_fresh(str(tmp_path / "nope.so"))


def _load_fresh(path):
    saved = binding._lib
    binding._lib = None
    try:
        return binding.load_library(path)
    finally:
        binding._lib = saved


def test_create_rejects_shapes_beyond_32bit_offsets():
    """The GEMMs address each operand with 32-bit byte offsets; create
    refuses every shape whose operands reach 2^31 bytes, before any device
    call, so that a forward on a created handle never fails half-way."""
    lib = _lib()
    bw, _keep = _fake_weights()
    # 1 x 1024 x 1024 tokens x 4*1280 = 5.4e9 elements
    st, h = _create(lib, B=1, C=1280, H=1024, W=1024, heads=20, w=bw)
    assert st == binding.ST_ERR_UNSUPPORTED
    assert h.value is None
    assert "2^30" in binding.last_error()
    # 2^31 elements exactly
    st, h = _create(lib, B=2, C=64, H=2048, W=2048, heads=1, w=bw)
    assert st == binding.ST_ERR_UNSUPPORTED and h.value is None
    # just above 2^30 elements of the GEGLU output (2^31 bytes of FF2's A
    # operand): B=4, C=1280, 256 x 256 -> T*4C = 1.34e9
    st, h = _create(lib, B=4, C=1280, H=256, W=256, heads=20, w=bw)
    assert st == binding.ST_ERR_UNSUPPORTED and h.value is None
    assert "FF2" in binding.last_error()
    # T*4C = 2^30 exactly: 2^31 bytes, refused; one token fewer per sample
    # reaches the device (no GPU here: ST_ERR_DEVICE, or a handle with one)
    st, h = _create(lib, B=1, C=64, H=2048, W=2048, heads=1, w=bw)
    assert st == binding.ST_ERR_UNSUPPORTED and h.value is None


@pytest.mark.parametrize("kw,what", [
    # FF1 weights [8C][C] in 16-bit: 16*C^2 bytes >= 2^31 from C = 11648
    (dict(C=11648, heads=182, H=1, W=1), "FF1"),
    # context K/V weights [2C*depth][D] in 16-bit: 4*C*depth*D >= 2^31
    (dict(C=1280, heads=20, depth=10, D=41984, H=1, W=1), "context K/V"),
])
def test_create_rejects_large_weight_operands(kw, what):
    lib = _lib()
    bw, _keep = _fake_weights(depth=kw.get("depth", 1))
    st, h = _create(lib, w=bw, **kw)
    assert st == binding.ST_ERR_UNSUPPORTED and h.value is None
    assert what in binding.last_error()


def test_null_handle_new_entry_points():
    lib = _lib()
    assert lib.st_block_check_range(None, None) == binding.ST_ERR_INVALID
    n = ctypes.c_longlong()
    assert lib.st_block_read_timing_launches(None, None, None, 0, ctypes.byref(n)) \
        == binding.ST_ERR_INVALID
    d = ctypes.c_double()
    assert lib.st_measure_mfma_bf16(0, None, ctypes.byref(d), ctypes.byref(d)) \
        == binding.ST_ERR_INVALID
    assert lib.st_block_set_timing_layers(None, 1) == binding.ST_ERR_INVALID


def test_ops_validate_before_any_device_call():
    """st_group_norm and st_guided_ddpm_step reject bad arguments with
    ST_ERR_INVALID (no device needed: nothing is enqueued)."""
    lib = _lib()
    P = 0x10000
    ws = lib.st_group_norm_workspace_bytes(2)
    assert ws == 2 * 32 * 64 * 8
    assert lib.st_group_norm_workspace_bytes(0) == 0
    ok = dict(x=P, g=None, b=None, y=P + (1 << 30), B=2, C=64, H=4, W=4, eps=1e-5, silu=1,
              dt=0, ws=P + (1 << 31), wsb=ws)

    def gn(**kw):
        a = dict(ok, **kw)
        return lib.st_group_norm(a["x"], a["g"], a["b"], a["y"], a["B"], a["C"], a["H"], a["W"],
                                 a["eps"], a["silu"], a["dt"], a["ws"], a["wsb"], None)
    for kw, why in [(dict(x=None), "non-NULL"), (dict(B=0), "B"), (dict(C=48), "multiple of 32"),
                    (dict(eps=0.0), "eps"), (dict(dt=5), "dtype"), (dict(x=P + 8), "aligned"),
                    (dict(y=P + 64), "overlaps"), (dict(wsb=ws - 1), "workspace"),
                    (dict(ws=None), "workspace")]:
        assert gn(**kw) == binding.ST_ERR_INVALID, kw
        assert why in binding.last_error(), (kw, binding.last_error())

    def dd(**kw):
        a = dict(eps=P, dt=0, xt=P, z=None, xp=P, n=16, s=7.5, t=10, T=1000, b0=1e-4, b1=0.02)
        a.update(kw)
        return lib.st_guided_ddpm_step(a["eps"], a["dt"], a["xt"], a["z"], a["xp"], a["n"], a["s"],
                                       a["t"], a["T"], a["b0"], a["b1"], None)
    for kw in [dict(t=0), dict(t=1001), dict(T=0), dict(n=-1), dict(b0=0.0), dict(b1=1.0),
               dict(dt=3), dict(eps=None), dict(s=float("inf"))]:
        assert dd(**kw) == binding.ST_ERR_INVALID, kw
    assert dd(n=0, eps=None, xt=None, xp=None) == binding.ST_OK  # nothing to do


def test_resnet_create_validates_before_any_device_call():
    lib = _lib()
    P = 0x10000
    w = binding.ResnetWeights()
    w.conv1_w = w.conv2_w = w.temb_w = w.sc_w = P

    def create(B=2, Ci=64, Co=64, H=8, W=8, Dt=32, eps=1e-5, dt=0, ww=w):
        h = ctypes.c_void_p()
        st = lib.st_resnet_create(B, Ci, Co, H, W, Dt, eps, dt,
                                  ctypes.byref(ww) if ww is not None else None, None, ctypes.byref(h))
        assert h.value is None
        return st
    assert create(B=0) == binding.ST_ERR_INVALID
    assert create(Ci=96) == binding.ST_ERR_INVALID
    assert create(Co=0) == binding.ST_ERR_INVALID
    assert create(eps=0.0) == binding.ST_ERR_INVALID
    assert create(dt=4) == binding.ST_ERR_INVALID
    assert create(dt=1) == binding.ST_ERR_UNSUPPORTED      # fp32 storage
    assert create(B=17) == binding.ST_ERR_UNSUPPORTED      # time-embedding batch limit
    assert create(W=6) == binding.ST_ERR_UNSUPPORTED       # width not a multiple of 4
    assert create(ww=None) == binding.ST_ERR_INVALID
    nosc = binding.ResnetWeights()
    nosc.conv1_w = nosc.conv2_w = nosc.temb_w = P
    assert create(Co=128, ww=nosc) == binding.ST_ERR_INVALID  # projection needs sc_w
    assert create(H=4096, W=4096, Ci=640, Co=640) == binding.ST_ERR_UNSUPPORTED
    assert lib.st_resnet_forward(None, P, P, P, None) == binding.ST_ERR_INVALID
    assert lib.st_resnet_check_range(None, None) == binding.ST_ERR_INVALID
    lib.st_resnet_destroy(None)


def test_unet_create_validates_before_any_device_call():
    lib = _lib()
    c = binding.UNetConfigC()
    c.in_channels, c.out_channels, c.levels = 4, 4, 2
    c.channels[0], c.channels[1] = 64, 128
    c.depths[0], c.depths[1] = 1, 1
    c.mid_depth, c.layers_per_block, c.ctx_dim = 1, 2, 64
    w = binding.UNetWeights()

    def create(B=2, H=16, W=16, cc=c, ww=w):
        h = ctypes.c_void_p()
        st = lib.st_unet_create(ctypes.byref(cc) if cc is not None else None, B, H, W,
                                ctypes.byref(ww) if ww is not None else None, None, ctypes.byref(h))
        assert h.value is None
        return st
    assert create(cc=None) == binding.ST_ERR_INVALID
    assert create(ww=None) == binding.ST_ERR_INVALID
    assert create(B=5) == binding.ST_ERR_UNSUPPORTED
    assert create(W=12) == binding.ST_ERR_UNSUPPORTED   # 12 / 2 = 6, not a multiple of 4
    assert create() == binding.ST_ERR_INVALID            # weights missing
    c.levels = 5
    assert create() == binding.ST_ERR_INVALID
    c.levels = 2
    c.channels[1] = 100
    assert create() == binding.ST_ERR_INVALID
    c.channels[1] = 128
    assert lib.st_unet_forward(None, 16, 16, 16, None, 16, None) == binding.ST_ERR_INVALID
    n = ctypes.c_ulonglong()
    assert lib.st_unet_device_bytes(None, ctypes.byref(n)) == binding.ST_ERR_INVALID
    assert lib.st_unet_check_range(None, None) == binding.ST_ERR_INVALID
    lib.st_unet_destroy(None)
