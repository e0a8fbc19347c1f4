"""The C ABI on the CPU: the library loads, exports exactly what the header
declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

from latent_diffusion_net_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "st_block.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(st_[a-z_]+)\s*\(", src)))


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
    """The kernels index activations with 32-bit element offsets; the
    largest buffer, the GEGLU output [B*H*W][4C], must stay below 2^31
    elements.  Checked before any device call."""
    lib = _lib()
    bw, _keep = _fake_weights()
    # 1 x 1024 x 1024 tokens x 4*1280 = 5.4e9 elements
    st, h = _create(lib, B=1, C=1280, H=1024, W=1024, heads=20, w=bw)
    assert st == binding.ST_ERR_UNSUPPORTED
    assert h.value is None
    assert "2^31" in binding.last_error()
    # just past the limit: 2^31 elements exactly
    st, h = _create(lib, B=2, C=64, H=2048, W=2048, heads=1, w=bw)
    assert st == binding.ST_ERR_UNSUPPORTED and h.value is None
