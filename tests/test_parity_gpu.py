"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Tolerances.
* bf16 storage (inputs, weights, output; 16-bit GEMM/attention operands with
  fp32 accumulation): max-abs <= 3e-2 and rel-L2 <= 1e-2 on y.
  The block's update Delta = y - x is far smaller than x (weights
  N(0, 0.02^2)), so the update is checked as well, against a bound derived
  from the arithmetic: storing y in bf16 (unit roundoff u = 2^-8) alone moves
  Delta by up to u*|y| per element, and the 16-bit operands on the way to
  Delta (about six roundings of relative size <= u each, partly cancelling)
  add a few u of Delta itself, so
      ||Delta_gpu - Delta_oracle|| <= u * (||y|| + 5 ||Delta||).
* fp32 storage: rel-L2 <= 1e-5 on y; on Delta, fp32 sums of K <= 5120 terms
  (u = 2^-24) give well under 1e-4.
"""
import gc
import os
import sys

import numpy as np
import pytest

import oracle.block as ob
from latent_diffusion_net_amd import synth

pytestmark = pytest.mark.gpu

BF16_MAX_ABS = 3e-2
BF16_REL_L2 = 1e-2
U_BF16 = 2.0 ** -8
F32_REL_L2 = 1e-5
F32_DELTA_REL_L2 = 1e-4


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def run_gpu(cfg, inp, stages=()):
    import torch
    from latent_diffusion_net_amd import STBlock, array_to_device, params_to_device
    _say(f"[gpu] {cfg.name}: B={cfg.B} C={cfg.C} H={cfg.H} W={cfg.W} heads={cfg.heads} "
         f"D_ctx={cfg.D_ctx} depth={cfg.depth} dtype={cfg.dtype}")
    p = params_to_device(inp["params"], cfg.dtype)
    x = array_to_device(inp["x"], cfg.dtype)
    ctx = array_to_device(inp["ctx"], cfg.dtype)
    blk = STBlock(cfg.B, cfg.C, cfg.H, cfg.W, cfg.heads, cfg.D_ctx, cfg.depth,
                  cfg.dtype, p)
    del p
    y = blk.forward(x, ctx)
    hs = {s: blk.forward_stage(x, ctx, s) for s in stages}
    torch.cuda.synchronize()
    out = y.float().cpu().numpy().astype(np.float64)
    hs = {s: h.cpu().numpy().astype(np.float64) for s, h in hs.items()}
    blk.close()
    return out, hs


def check(cfg, inp, y, yo):
    x = np.asarray(inp["x"], np.float64)
    err = float(np.max(np.abs(y - yo)))
    r = rel_l2(y, yo)
    rd = rel_l2(y - x, yo - x)
    _say(f"    max_abs={err:.3e} rel_l2={r:.3e} delta_rel_l2={rd:.3e}")
    assert np.isfinite(y).all()
    if cfg.dtype == "bf16":
        assert err <= BF16_MAX_ABS, err
        assert r <= BF16_REL_L2, r
        bound = U_BF16 * (np.linalg.norm(yo) / np.linalg.norm(yo - x) + 5.0)
        assert rd <= bound, (rd, bound)
    else:
        assert r <= F32_REL_L2, r
        assert rd <= F32_DELTA_REL_L2, rd


SMALL = [
    # several 128-query tiles with a ragged tail (225 tokens), two layers
    dict(name="b2_c128_15x15_d2", B=2, C=128, H=15, W=15, heads=2, D_ctx=128, depth=2),
    # non-square map, three heads, wide context, ragged everything
    dict(name="b1_c192_17x13_d1", B=1, C=192, H=17, W=13, heads=3, D_ctx=192, depth=1),
    # one head, tokens a multiple of the tiles
    dict(name="b2_c64_16x16_d1", B=2, C=64, H=16, W=16, heads=1, D_ctx=64, depth=1),
    # degenerate: a single token (self-attention over one key)
    dict(name="b1_c64_1x1_d2", B=1, C=64, H=1, W=1, heads=1, D_ctx=64, depth=2),
    # C=320 (GEMM tiles ragged along N), 3 sublayers deep stack
    dict(name="b1_c320_12x12_d3", B=1, C=320, H=12, W=12, heads=5, D_ctx=768, depth=3),
    # few output tiles and F=2048: FF2 split over K (bf16 storage), its row
    # sums feeding the next layer's folded LayerNorm; ragged rows
    dict(name="b1_c512_9x11_d2", B=1, C=512, H=9, W=11, heads=8, D_ctx=256, depth=2),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("spec", SMALL, ids=lambda s: s["name"])
def test_small_stress(spec, dtype):
    """Biases, norm affines and weights all drawn (every term matters)."""
    spec = dict(spec)
    cfg = synth.BlockConfig(spec.pop("name") + "_" + dtype, dtype=dtype, **spec)
    inp = synth.make_inputs(cfg, 77, bias_std=0.05, norm_std=0.2)
    yo = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    y, _ = run_gpu(cfg, inp)
    check(cfg, inp, y, yo)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("grid", [(1, 20, 20), (2, 8, 8), (1, 24, 24)],
                         ids=["b1_20x20", "b2_8x8", "b1_24x24"])
def test_sharp_softmax(dtype, grid):
    """Large weights: logits spread over tens of units, so the online softmax
    rescales often and the row maxima matter.  400 tokens run the
    cross-attention as its own kernel; 2 x 64 tokens (a multiple of 64 per
    sample) run it inside the Q projection's epilogue, with GEMM tiles that
    span both samples; 576 tokens too, ending half-way into a 128-row tile."""
    B, H, W = grid
    cfg = synth.BlockConfig(f"sharp_{B}x{H}x{W}_" + dtype, B, 128, H, W, 2, 128, 1, dtype)
    inp = synth.make_inputs(cfg, 5, weight_std=0.12)
    yo, inter = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads,
                                 intermediates=True)
    y, hs = run_gpu(cfg, inp, stages=(1, 2))
    tol = 2e-2 if dtype == "bf16" else 1e-5
    for s, key in ((1, "l0_sa"), (2, "l0_ca")):
        # the sublayer's own contribution, relative
        prev = inter["h0"] if s == 1 else inter["l0_sa"]
        r = rel_l2(hs[s].reshape(prev.shape) - prev, inter[key] - prev)
        _say(f"    stage {s}: update rel_l2={r:.3e}")
        assert r <= (tol if dtype == "bf16" else 1e-4), r
    assert rel_l2(y, yo) <= (1e-2 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("shape", [
    (2, 128, 15, 15, 2, 128),
    # F = 2048 over few output tiles: FF2 takes the split-K path, so the
    # stream after each feed-forward comes from the ordered slice sum
    (1, 512, 9, 11, 8, 256),
    # 144 tokens per sample: the 128-row tiles of every product straddle the
    # two samples, and 288 rows leave a ragged last tile
    (2, 128, 12, 12, 2, 128),
    # 320 channels: five K stages (an odd count) and output columns ragged
    # over 128-wide tiles; 80 rows, one partial tile
    (1, 320, 8, 10, 5, 128),
], ids=["b2_c128", "b1_c512_splitk", "b2_c128_straddle", "b1_c320_odd_stages"])
def test_stages_bf16(shape):
    """Residual stream after proj_in and after every sublayer."""
    B, C, H, W, heads, D_ctx = shape
    cfg = synth.BlockConfig("stages", B, C, H, W, heads, D_ctx, 2, "bf16")
    inp = synth.make_inputs(cfg, 9, bias_std=0.05, norm_std=0.2)
    _, inter = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads,
                                intermediates=True)
    keys = ["h0"] + [f"l{l}_{s}" for l in range(2) for s in ("sa", "ca", "ff")]
    _, hs = run_gpu(cfg, inp, stages=range(len(keys)))
    for s, key in enumerate(keys):
        h = hs[s].reshape(inter[key].shape)
        r = rel_l2(h, inter[key])
        _say(f"    stage {s} ({key}): rel_l2={r:.3e}")
        assert r <= 1e-2, (key, r)


def test_groupnorm_offsets_and_scales():
    """GroupNorm on an input whose channels carry offsets up to 30 and
    spreads from 0.05 to 8 (the groups' means and variances differ widely):
    h after proj_in against the oracle within what fp16 rounding of the
    normalised operand and of h allows (each ~2^-12 relative, rel-L2 well
    under 2e-3)."""
    cfg = synth.BlockConfig("gn_offsets_c256_16x16", 2, 256, 16, 16, 4, 128, 1, "bf16")
    inp = synth.make_inputs(cfg, 21, bias_std=0.05, norm_std=0.2)
    rng = np.random.default_rng(22)
    C = cfg.C
    offset = rng.uniform(-30.0, 30.0, size=(1, C, 1, 1))
    spread = np.exp(rng.uniform(np.log(0.05), np.log(8.0), size=(1, C, 1, 1)))
    inp["x"] = synth.round_bf16((offset + spread * inp["x"]).astype(np.float32))
    _, inter = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads,
                                intermediates=True)
    _, hs = run_gpu(cfg, inp, stages=[0])
    h0 = inter["h0"]
    r = rel_l2(hs[0].reshape(h0.shape), h0)
    _say(f"    h0 rel_l2={r:.3e}")
    assert r <= 2e-3, r


def test_f32_tiny_config_exact():
    """The tiny fp32 workload at its full size, rel-L2 <= 1e-5."""
    cfg = synth.CONFIGS[0]
    inp = synth.make_inputs(cfg, synth.config_seed(0))
    yo = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    y, _ = run_gpu(cfg, inp)
    check(cfg, inp, y, yo)


def test_tiny_config_on_bf16_path():
    """The tiny workload rounded to bf16 runs through the bf16 kernels too."""
    c0 = synth.CONFIGS[0]
    cfg = synth.BlockConfig(c0.name + "_as_bf16", c0.B, c0.C, c0.H, c0.W, c0.heads,
                            c0.D_ctx, c0.depth, "bf16")
    inp = synth.make_inputs(cfg, synth.config_seed(0))
    yo = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    y, _ = run_gpu(cfg, inp)
    check(cfg, inp, y, yo)


@pytest.mark.parametrize("index", [1, 2, 3, 4])
def test_full_config(index):
    """The workloads at their full sizes, every output element compared."""
    cfg = synth.CONFIGS[index]
    inp = synth.make_inputs(cfg, synth.config_seed(index))
    y, _ = run_gpu(cfg, inp)
    _say("    oracle ...")
    yo = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    check(cfg, inp, y, yo)
    del inp, yo, y
    gc.collect()


def test_unet_level_1024_tokens_batch1():
    """A transformer block at the shape of the SDXL-Inpaint U-Net's 1024-token
    levels at batch 1 (32x32, C = 1280, 20 heads): FF1 + GEGLU on 256x256
    tiles that cover the product exactly (160 of them, fewer than the
    general threshold), the out-projections and FF2 split over K (80 output
    tiles), and proj_in on the three-stage ring; every output element
    against the oracle."""
    cfg = synth.BlockConfig("b1_c1280_32x32_d1", 1, 1280, 32, 32, 20, 2048, 1, "bf16")
    inp = synth.make_inputs(cfg, 17)
    y, _ = run_gpu(cfg, inp)
    _say("    oracle ...")
    yo = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    check(cfg, inp, y, yo)


def test_deterministic_and_timing():
    import torch
    from latent_diffusion_net_amd import STBlock, array_to_device, params_to_device
    cfg = synth.BlockConfig("det", 2, 128, 15, 15, 2, 128, 2, "bf16")
    inp = synth.make_inputs(cfg, 3)
    p = params_to_device(inp["params"], "bf16")
    x = array_to_device(inp["x"], "bf16")
    ctx = array_to_device(inp["ctx"], "bf16")
    blk = STBlock(cfg.B, cfg.C, cfg.H, cfg.W, cfg.heads, cfg.D_ctx, cfg.depth, "bf16", p)
    blk.set_timing(["self_attn", "cross_attn", "ff1_geglu"])
    y1 = blk.forward(x, ctx)
    y2 = blk.forward(x, ctx)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    t = blk.read_timing()
    assert t["self_attn"]["launches"] == 2 * cfg.depth
    assert t["cross_attn"]["launches"] == 2 * cfg.depth
    assert t["self_attn"]["ms"] > 0
    assert "qkv" not in t
    assert blk.read_timing() == {}
    # the per-layer kinds timed in the first layer only; the block-level
    # kinds (proj_out) in every forward; outputs unchanged
    blk.set_timing(["self_attn", "ff2", "proj_out"], layers=1)
    y3 = blk.forward(x, ctx)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))
    t = blk.read_timing()
    assert t["self_attn"]["launches"] == 1 and t["ff2"]["launches"] == 1
    assert t["proj_out"]["launches"] == 1
    blk.set_timing([])
    blk.close()


def test_forward_rejects_aliasing_on_device():
    import torch
    from latent_diffusion_net_amd import STBlock, STError, array_to_device, params_to_device
    cfg = synth.BlockConfig("alias", 1, 64, 4, 4, 1, 64, 1, "bf16")
    inp = synth.make_inputs(cfg, 4)
    p = params_to_device(inp["params"], "bf16")
    x = array_to_device(inp["x"], "bf16")
    ctx = array_to_device(inp["ctx"], "bf16")
    blk = STBlock(1, 64, 4, 4, 1, 64, 1, "bf16", p)
    with pytest.raises(STError, match="overlaps"):
        blk.forward(x, ctx, y=x)
    with pytest.raises(STError, match="stage"):
        blk.forward_stage(x, ctx, 99)
    torch.cuda.synchronize()
    blk.close()


def test_create_respects_device_memory_cap(monkeypatch):
    """ST_MAX_DEVICE_BYTES (read at create): a handle that needs more device
    memory is refused with ST_ERR_OUT_OF_MEMORY and keeps nothing; a cap
    above the need changes nothing (bitwise)."""
    import torch
    from latent_diffusion_net_amd import STBlock, array_to_device, params_to_device
    from latent_diffusion_net_amd.binding import ST_ERR_OUT_OF_MEMORY, STError
    cfg = synth.BlockConfig("cap", dtype="bf16", B=1, C=64, H=8, W=8, heads=1, D_ctx=64, depth=1)
    inp = synth.make_inputs(cfg, 31)
    _say("[gpu] device memory cap")
    p = params_to_device(inp["params"], "bf16")
    x = array_to_device(inp["x"], "bf16")
    ctx = array_to_device(inp["ctx"], "bf16")
    blk = STBlock(cfg.B, cfg.C, cfg.H, cfg.W, cfg.heads, cfg.D_ctx, cfg.depth, "bf16", p)
    y0 = blk.forward(x, ctx)
    torch.cuda.synchronize()
    blk.close()
    free0, _ = torch.cuda.mem_get_info()
    monkeypatch.setenv("ST_MAX_DEVICE_BYTES", "65536")
    with pytest.raises(STError) as e:
        STBlock(cfg.B, cfg.C, cfg.H, cfg.W, cfg.heads, cfg.D_ctx, cfg.depth, "bf16", p)
    assert e.value.status == ST_ERR_OUT_OF_MEMORY
    free1, _ = torch.cuda.mem_get_info()
    assert abs(free1 - free0) <= 4 << 20, (free0, free1)
    monkeypatch.setenv("ST_MAX_DEVICE_BYTES", str(1 << 40))
    blk = STBlock(cfg.B, cfg.C, cfg.H, cfg.W, cfg.heads, cfg.D_ctx, cfg.depth, "bf16", p)
    y1 = blk.forward(x, ctx)
    torch.cuda.synchronize()
    blk.close()
    assert torch.equal(y0.view(torch.int16), y1.view(torch.int16))


@pytest.mark.parametrize("cus,spec", [
    # 32 query tiles over 12 CUs: 24 whole, 8 split in 2 over 64 key tiles
    (12, dict(name="split2", B=1, C=64, H=64, W=64, heads=1, D_ctx=64, depth=1)),
    # ragged keys (3969 = 62 tiles of 64 + 1): 31 whole, 1 split in 3 pieces,
    # the last of which holds the ragged tile
    (31, dict(name="split3_ragged", B=1, C=64, H=63, W=63, heads=1, D_ctx=64, depth=1)),
    # every tile split in 2, two layers
    (64, dict(name="split2_all", B=1, C=64, H=64, W=64, heads=1, D_ctx=64, depth=2)),
], ids=lambda v: v if isinstance(v, int) else v["name"])
def test_self_attention_split_over_keys(cus, spec, monkeypatch):
    """Self-attention with query tiles split over key ranges (the load
    balance used when tiles do not fill the CUs evenly), forced at a small
    size by planning for fewer CUs: parity with the oracle, and repeated
    forwards bitwise equal (the pieces are merged in a fixed order)."""
    import torch
    from latent_diffusion_net_amd import STBlock, array_to_device, params_to_device
    monkeypatch.setenv("ST_ATTN_CUS", str(cus))
    spec = dict(spec)
    cfg = synth.BlockConfig(spec.pop("name"), dtype="bf16", **spec)
    inp = synth.make_inputs(cfg, 21, bias_std=0.05, norm_std=0.2)
    yo = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    _say(f"[gpu] {cfg.name}: planned for {cus} CUs")
    p = params_to_device(inp["params"], "bf16")
    x = array_to_device(inp["x"], "bf16")
    ctx = array_to_device(inp["ctx"], "bf16")
    blk = STBlock(cfg.B, cfg.C, cfg.H, cfg.W, cfg.heads, cfg.D_ctx, cfg.depth, "bf16", p)
    y1 = blk.forward(x, ctx)
    y2 = blk.forward(x, ctx)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    y = y1.float().cpu().numpy().astype(np.float64)
    blk.close()
    check(cfg, inp, y, yo)


@pytest.mark.parametrize("spec", __import__("sa_stage").SHAPES, ids=lambda s: s["name"])
def test_self_attention_sharp(spec, monkeypatch):
    """The self-attention path the workloads time, with a softmax far from
    flat (logit std about 3): the 128-query kernel at the full SDXL Down1
    shape (whole tiles, key-split pieces and their merge), with ragged
    queries and keys, and the forced key-split plans.  The sublayer's update
    (stage 1 minus stage 0 of the GPU's own stream) against the oracle's
    l0_sa - h0, element by element; bounds and the mutations they reject in
    tests/sa_stage.py and tests/test_sa_stage_pins.py."""
    import torch
    import sa_stage as sa
    from latent_diffusion_net_amd import STBlock, array_to_device, params_to_device
    if spec["cus"] is not None:
        monkeypatch.setenv("ST_ATTN_CUS", str(spec["cus"]))
    cfg, inp = sa.inputs(spec)
    _say(f"[gpu] sharp self-attention {cfg.name}: B={cfg.B} C={cfg.C} N={cfg.N} "
         f"planned CUs={spec['cus']}")
    p = params_to_device(inp["params"], "bf16")
    x = array_to_device(inp["x"], "bf16")
    ctx = array_to_device(inp["ctx"], "bf16")
    blk = STBlock(cfg.B, cfg.C, cfg.H, cfg.W, cfg.heads, cfg.D_ctx, cfg.depth, "bf16", p)
    del p
    g0 = blk.forward_stage(x, ctx, 0)
    g1 = blk.forward_stage(x, ctx, 1)
    g1b = blk.forward_stage(x, ctx, 1)
    blk.check_range()
    torch.cuda.synchronize()
    assert torch.equal(g1, g1b)  # pieces merged in a fixed order
    d_gpu = (g1 - g0).cpu().numpy().astype(np.float64)
    blk.close()
    del g0, g1, g1b
    h0, h1 = sa.oracle_stage1(inp, cfg.heads)
    d_ref = (h1 - h0).reshape(d_gpu.shape)
    rel, mx = sa.update_errors(d_gpu, d_ref)
    _say(f"    update rel_l2={rel:.3e} max_abs/max|update|={mx:.3e}")
    assert np.isfinite(d_gpu).all()
    assert rel <= sa.UPDATE_REL_L2, rel
    assert mx <= sa.UPDATE_MAX_ABS_REL, mx


def _offset_stream_inputs(cfg, seed, offset):
    """Headline draws, with proj_in's bias = offset on every channel, so each
    row of the residual stream h has mean ~offset and std ~0.02 sqrt(C);
    proj_out's bias cancels the offset's image in y (b_out = -offset *
    row sums of W_out, rounded to bf16: the same values on both sides), so y
    keeps its usual scale."""
    inp = synth.make_inputs(cfg, seed)
    p = inp["params"]
    C = cfg.C
    p["proj_in_b"] = synth.round_bf16(np.full(C, offset, np.float32))
    rs = np.asarray(p["proj_out_w"], np.float64).sum(axis=1)
    p["proj_out_b"] = synth.round_bf16((-float(p["proj_in_b"][0]) * rs).astype(np.float32))
    return inp


def test_fp16_stream_large_row_mean():
    """Rows of h whose mean is ~30 standard deviations away from zero (h0 =
    15 + N(0, 0.51^2) at C = 640): the fp16 stream rounds them with an
    absolute error ~30x larger relative to their spread than usual, and the
    folded LayerNorm subtracts the mean after the product.  The output still
    meets the bf16 gate and no range error is raised."""
    cfg = synth.BlockConfig("offset15_c640_32x32_d2", 1, 640, 32, 32, 10, 256, 2, "bf16")
    inp = _offset_stream_inputs(cfg, 13, 15.0)
    _, inter = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads,
                                intermediates=True)
    h0 = inter["h0"]
    ratio = np.abs(h0.mean(axis=-1)) / h0.std(axis=-1)
    _say(f"    |mean|/std of the rows of h0: median {np.median(ratio):.1f}")
    assert np.median(ratio) > 25
    yo = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    y, _ = run_gpu(cfg, inp)
    check(cfg, inp, y, yo)


def test_fp16_stream_overflow_is_reported():
    """A proj_in bias of 70144 puts every value of h beyond the fp16 range:
    st_block_check_range reports ST_ERR_RANGE (then the flag is clear);
    the same block with an in-range bias reports nothing."""
    import torch
    from latent_diffusion_net_amd import STBlock, STError, array_to_device, params_to_device
    from latent_diffusion_net_amd.binding import ST_ERR_RANGE
    cfg = synth.BlockConfig("overflow_c128", 1, 128, 8, 8, 2, 128, 1, "bf16")
    _say("[gpu] fp16 range flag")
    for offset, expect in ((70144.0, True), (15.0, False)):
        inp = _offset_stream_inputs(cfg, 17, offset)
        p = params_to_device(inp["params"], "bf16")
        x = array_to_device(inp["x"], "bf16")
        ctx = array_to_device(inp["ctx"], "bf16")
        blk = STBlock(cfg.B, cfg.C, cfg.H, cfg.W, cfg.heads, cfg.D_ctx, cfg.depth, "bf16", p)
        y = blk.forward(x, ctx)
        if expect:
            with pytest.raises(STError) as e:
                blk.check_range()
            assert e.value.status == ST_ERR_RANGE
        blk.check_range()  # clear (or never set)
        torch.cuda.synchronize()
        if not expect:
            assert torch.isfinite(y.float()).all()
        blk.close()


def _masks(B, kind):
    m = np.ones((B, 77), np.uint8)
    if kind == "padded":        # tokenizer padding: real tokens first
        for b in range(B):
            m[b, 12 + 9 * b:] = 0
    elif kind == "scattered":
        m[:, 3::4] = 0
        m[-1, :70] = 0
    elif kind == "first_tile_masked":  # every key of the first 64 masked
        m[:, :64] = 0
    elif kind == "one_sample_empty":   # the last sample has no real token
        m[0, 40:] = 0
        m[-1, :] = 0
    return m


MASK_CASES = [
    # bf16, H*W % 64 == 0: cross-attention in the cross-Q epilogue
    ("fused", synth.BlockConfig("mask_fused", 2, 128, 8, 8, 2, 128, 2, "bf16")),
    # bf16, H*W = 225: the separate 77-key attention kernel (128-query tiles)
    ("kernel", synth.BlockConfig("mask_kernel", 2, 128, 15, 15, 2, 128, 2, "bf16")),
    # fp32 path
    ("f32", synth.BlockConfig("mask_f32", 2, 128, 15, 15, 2, 128, 2, "f32")),
]


@pytest.mark.parametrize("kind", ["padded", "scattered", "first_tile_masked", "one_sample_empty"])
@pytest.mark.parametrize("path,cfg", MASK_CASES, ids=[c[0] for c in MASK_CASES])
def test_cross_attention_key_mask(path, cfg, kind):
    """st_block_forward_masked against the oracle with the same key padding
    mask (anatomy article §5.5), on every cross-attention path; a softmax
    far from flat (logit std ~3 in both attentions), so that the mask
    visibly matters; an all-ones mask equals the unmasked forward bitwise."""
    import math
    import torch
    from latent_diffusion_net_amd import STBlock, array_to_device, params_to_device
    inp = synth.make_inputs(cfg, 61, bias_std=0.05, norm_std=0.2, qk_std=math.sqrt(3.0 / cfg.C))
    m = _masks(cfg.B, kind)
    _say(f"[gpu] key mask {path} {kind}: B={cfg.B} C={cfg.C} N={cfg.N} dtype={cfg.dtype}")
    p = params_to_device(inp["params"], cfg.dtype)
    x = array_to_device(inp["x"], cfg.dtype)
    ctx = array_to_device(inp["ctx"], cfg.dtype)
    blk = STBlock(cfg.B, cfg.C, cfg.H, cfg.W, cfg.heads, cfg.D_ctx, cfg.depth, cfg.dtype, p)
    md = torch.from_numpy(m).cuda()
    y = blk.forward_masked(x, ctx, md)
    y1 = blk.forward_masked(x, ctx, torch.ones_like(md))
    y0 = blk.forward(x, ctx)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16 if cfg.dtype == "bf16" else torch.int32),
                       y0.view(torch.int16 if cfg.dtype == "bf16" else torch.int32))
    y = y.float().cpu().numpy().astype(np.float64)
    blk.close()
    yo = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads, ctx_mask=m)
    yu = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    x64 = np.asarray(inp["x"], np.float64)
    moved = rel_l2(yo - x64, yu - x64)
    _say(f"    the mask moves the oracle's update by {moved:.3e} (rel-L2)")
    assert moved > 0.05
    check(cfg, inp, y, yo)


def test_refiner_depth_four():
    """Depth 4 (the SDXL Refiner's transformer depth) at a Refiner-like stage:
    C = 768, 32 x 32, context width 1280 (OpenCLIP ViT-bigG)."""
    cfg = synth.BlockConfig("refiner_c768_32x32_d4", 2, 768, 32, 32, 12, 1280, 4, "bf16")
    inp = synth.make_inputs(cfg, 71, bias_std=0.02, norm_std=0.1)
    yo = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    y, _ = run_gpu(cfg, inp)
    check(cfg, inp, y, yo)
