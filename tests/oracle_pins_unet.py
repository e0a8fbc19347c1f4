"""Pins of the fp64 oracle's U-Net parts (oracle/unet.py) and of the
cross-attention key mask (oracle/block.py) against facts that do not come
from the oracle: independent library routines (torch fp64 conv2d,
interpolate, silu, scaled_dot_product_attention with a boolean mask),
closed forms, textbook identities, the scalar brute force and values the
pages print.  ``tests/test_oracle.py`` runs every pin;
``tests/test_oracle_unet_mutations.py`` plants mistakes and checks that
some pin fails for each.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
import torch.nn.functional as Fnn

import oracle.block as ob
import oracle.brute as brute
import oracle.unet as ou
from latent_diffusion_net_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


def resnet_params(rng, Ci, Co, Dt, scale=0.1):
    p = {"gn1_w": 1 + scale * rng.standard_normal(Ci), "gn1_b": scale * rng.standard_normal(Ci),
         "conv1_w": scale * rng.standard_normal((Co, Ci, 3, 3)), "conv1_b": scale * rng.standard_normal(Co),
         "temb_w": 2 * scale * rng.standard_normal((Co, Dt)), "temb_b": scale * rng.standard_normal(Co),
         "gn2_w": 1 + scale * rng.standard_normal(Co), "gn2_b": scale * rng.standard_normal(Co),
         "conv2_w": scale * rng.standard_normal((Co, Co, 3, 3)), "conv2_b": scale * rng.standard_normal(Co)}
    if Ci != Co:
        p["sc_w"] = scale * rng.standard_normal((Co, Ci))
        p["sc_b"] = scale * rng.standard_normal(Co)
    return p


# ------------------------------------------------------------------ SiLU
def pin_silu_identity_and_library():
    """silu(x) - silu(-x) = x (x sigma(x) + x sigma(-x) = x), silu(0) = 0,
    silu(x) -> x for large x; torch fp64 silu."""
    x = np.linspace(-30, 30, 601)
    _close(ou.silu(x) - ou.silu(-x), x, 1e-12, "silu odd part")
    assert ou.silu(np.array([0.0]))[0] == 0.0
    _close(ou.silu(np.array([40.0])), [40.0], 1e-12, "silu large")
    _close(ou.silu(x), Fnn.silu(_t(x)).numpy(), 1e-14, "silu vs torch")


# ------------------------------------------------------------ convolution
def pin_conv2d_library():
    """torch fp64 conv2d: 3x3 stride 1 and 2 (padding 1), 1x1 (padding 0)."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 5, 9, 8))
    for (kh, stride, pad) in ((3, 1, 1), (3, 2, 1), (1, 1, 0)):
        w = rng.standard_normal((7, 5, kh, kh))
        b = rng.standard_normal(7)
        ref = Fnn.conv2d(_t(x), _t(w), _t(b), stride=stride, padding=pad).numpy()
        _close(ou.conv2d(x, w, b, stride=stride, padding=pad), ref, 1e-12,
               f"conv {kh}x{kh} stride {stride}")


def pin_conv2d_orientation():
    """A kernel whose only tap is (0, 0) reads pixel (i-1, j-1) (zero at the
    border): the kernel is applied unflipped; the centre tap is the identity."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((1, 3, 6, 5))
    w = np.zeros((3, 3, 3, 3))
    for c in range(3):
        w[c, c, 1, 1] = 1.0
    _close(ou.conv2d(x, w), x, 0.0, "centre tap identity")
    w = np.zeros((3, 3, 3, 3))
    for c in range(3):
        w[c, c, 0, 0] = 1.0
    ref = np.zeros_like(x)
    ref[:, :, 1:, 1:] = x[:, :, :-1, :-1]
    _close(ou.conv2d(x, w), ref, 0.0, "tap (0,0) reads (i-1, j-1)")


def pin_downsample_shape():
    """DownSample: Conv 3x3, stride 2, padding 1 halves even sizes (the
    tutorial page's DownSample module; 64 x 64 -> 32 x 32 between SDXL's
    Down1 and Down2 stages)."""
    x = np.zeros((1, 2, 64, 64))
    assert ou.conv2d(x, np.zeros((2, 2, 3, 3)), stride=2).shape == (1, 2, 32, 32)


def pin_conv2d_brute():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((1, 3, 5, 4))
    w = rng.standard_normal((2, 3, 3, 3))
    b = rng.standard_normal(2)
    for s in (1, 2):
        _close(ou.conv2d(x, w, b, stride=s), np.array(brute.conv2d(x, w, b, stride=s)), 1e-12,
               f"conv brute stride {s}")


def pin_upsample_library():
    rng = np.random.default_rng(24)
    x = rng.standard_normal((2, 3, 4, 5))
    ref = Fnn.interpolate(_t(x), scale_factor=2, mode="nearest").numpy()
    _close(ou.upsample_nearest2x(x), ref, 0.0, "nearest upsample vs torch")


# ------------------------------------------------------------ ResnetBlock2D
def pin_resnet_zero_conv2_is_shortcut():
    """conv2 weights and bias zero => y = shortcut(x): x itself when the
    channel counts match, the 1x1 projection otherwise."""
    rng = np.random.default_rng(25)
    x = rng.standard_normal((2, 64, 5, 6))
    temb = rng.standard_normal((2, 16))
    p = resnet_params(rng, 64, 64, 16)
    p["conv2_w"] = np.zeros_like(p["conv2_w"])
    p["conv2_b"] = np.zeros_like(p["conv2_b"])
    _close(ou.resnet_block(x, temb, p), x, 0.0, "identity shortcut")
    p = resnet_params(rng, 64, 96, 16)
    p["conv2_w"] = np.zeros_like(p["conv2_w"])
    p["conv2_b"] = np.zeros_like(p["conv2_b"])
    ref = np.einsum("oc,bchw->bohw", p["sc_w"], x) + p["sc_b"][None, :, None, None]
    _close(ou.resnet_block(x, temb, p), ref, 1e-12, "1x1 shortcut")


def pin_resnet_time_embedding_closed_form():
    """conv1 weights zero => h1 = conv1_b + Linear(SiLU(temb)), constant over
    each (sample, channel) plane; GroupNorm2 of such a field normalises the
    plane constants a_c within each group; at interior pixels conv2 of the
    constant field SiLU(a) is sum over ci of (sum of the 9 taps) * SiLU(a_ci)
    + conv2_b; y = x + that (identity shortcut)."""
    rng = np.random.default_rng(26)
    B, C, H, W, Dt, eps = 2, 64, 5, 6, 16, 1e-5
    x = rng.standard_normal((B, C, H, W))
    temb = rng.standard_normal((B, Dt))
    p = resnet_params(rng, C, C, Dt, scale=0.3)
    p["conv1_w"] = np.zeros_like(p["conv1_w"])
    y = ou.resnet_block(x, temb, p, eps=eps)
    sig = lambda v: v / (1.0 + np.exp(-v))
    for b in range(B):
        a = p["conv1_b"] + p["temb_w"] @ sig(temb[b]) + p["temb_b"]
        g = a.reshape(32, C // 32)
        m = g.mean(axis=1, keepdims=True)
        v = ((g - m) ** 2).mean(axis=1, keepdims=True)
        n = ((g - m) / np.sqrt(v + eps)).reshape(C) * p["gn2_w"] + p["gn2_b"]
        ref = p["conv2_w"].sum(axis=(2, 3)) @ sig(n) + p["conv2_b"]
        _close(y[b, :, 1:H - 1, 1:W - 1] - x[b, :, 1:H - 1, 1:W - 1],
               np.broadcast_to(ref[:, None, None], (C, H - 2, W - 2)), 1e-12,
               "time-embedding closed form")


def pin_resnet_brute():
    rng = np.random.default_rng(27)
    for Ci, Co in ((64, 64), (64, 96)):
        x = rng.standard_normal((2, Ci, 4, 3))
        temb = rng.standard_normal((2, 8))
        p = resnet_params(rng, Ci, Co, 8, scale=0.2)
        _close(ou.resnet_block(x, temb, p), np.array(brute.resnet_block(x, temb, p)), 1e-11,
               f"resnet brute {Ci}->{Co}")


def pin_resnet_library_composition():
    """The same block composed from torch fp64 library routines (group_norm,
    silu, conv2d, linear) in the order the pages give."""
    rng = np.random.default_rng(28)
    x = rng.standard_normal((2, 64, 6, 5))
    temb = rng.standard_normal((2, 32))
    p = resnet_params(rng, 64, 128, 32, scale=0.2)
    T = {k: _t(v) for k, v in p.items()}
    h = Fnn.conv2d(Fnn.silu(Fnn.group_norm(_t(x), 32, T["gn1_w"], T["gn1_b"], 1e-5)),
                   T["conv1_w"], T["conv1_b"], padding=1)
    h = h + Fnn.linear(Fnn.silu(_t(temb)), T["temb_w"], T["temb_b"])[:, :, None, None]
    h = Fnn.conv2d(Fnn.silu(Fnn.group_norm(h, 32, T["gn2_w"], T["gn2_b"], 1e-5)),
                   T["conv2_w"], T["conv2_b"], padding=1)
    ref = Fnn.conv2d(_t(x), T["sc_w"][:, :, None, None], T["sc_b"]) + h
    _close(ou.resnet_block(x, temb, p), ref.numpy(), 1e-12, "resnet vs torch composition")


# ------------------------------------------------------------ guidance, DDPM
def pin_cfg_special_scales():
    rng = np.random.default_rng(29)
    eu, ec = rng.standard_normal((2, 4, 3, 3))
    _close(ou.cfg_combine(eu, ec, 0.0), eu, 0.0, "scale 0 = unconditional")
    _close(ou.cfg_combine(eu, ec, 1.0), ec, 1e-15, "scale 1 = conditional")
    a, b = ou.cfg_combine(eu, ec, 2.0), ou.cfg_combine(eu, ec, 7.5)
    _close(b - a, 5.5 * (ec - eu), 1e-13, "linear in the scale")


def pin_ddpm_schedule_from_the_page():
    """beta_1 = 0.0001, beta_T = 0.02, T = 1000, linear (tutorial page);
    alphabar_t = prod alpha_i = exp(sum log alpha_i)."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "ddpm_schedule.txt"))
            if l.strip() and not l.startswith("#")]
    T, b1, bT = int(rows[0][0]), float(rows[0][1]), float(rows[0][2])
    beta, alpha, ab = ou.linear_schedule(T, b1, bT)
    assert len(beta) == T
    _close([beta[0], beta[-1]], [b1, bT], 1e-18, "schedule ends")
    _close(np.diff(beta), np.full(T - 1, (bT - b1) / (T - 1)), 1e-15, "linear steps")
    _close(alpha, 1.0 - beta, 0.0, "alpha = 1 - beta")
    _close(ab, np.exp(np.cumsum(np.log(alpha))), 1e-15, "alphabar")


def pin_ddpm_step_is_posterior_mean():
    """With the true noise as the prediction (x_t = sqrt(ab_t) x0 +
    sqrt(1 - ab_t) eps), the noise-free step equals the mean of the forward
    process posterior q(x_{t-1} | x_t, x0) = sqrt(ab_{t-1}) beta_t / (1 -
    ab_t) x0 + sqrt(alpha_t) (1 - ab_{t-1}) / (1 - ab_t) x_t (ab_0 = 1), an
    identity of the Gaussian forward process; and the noise enters as
    sqrt(beta_t) z."""
    rng = np.random.default_rng(30)
    sched = ou.linear_schedule()
    beta, alpha, ab = sched
    x0 = rng.standard_normal((1, 4, 3, 3))
    eps = rng.standard_normal(x0.shape)
    z = rng.standard_normal(x0.shape)
    for t in (1, 2, 17, 500, 999, 1000):
        abt = ab[t - 1]
        abp = ab[t - 2] if t > 1 else 1.0
        xt = math.sqrt(abt) * x0 + math.sqrt(1 - abt) * eps
        mean = (math.sqrt(abp) * beta[t - 1] / (1 - abt)) * x0 \
            + (math.sqrt(alpha[t - 1]) * (1 - abp) / (1 - abt)) * xt
        _close(ou.ddpm_step(xt, eps, t, sched), mean, 1e-12 * max(1.0, np.abs(mean).max()),
               f"posterior mean t={t}")
        _close(ou.ddpm_step(xt, eps, t, sched, z) - ou.ddpm_step(xt, eps, t, sched),
               math.sqrt(beta[t - 1]) * z, 1e-12, f"noise term t={t}")


def pin_guided_step_halves():
    """The pair's first half is the unconditional prediction."""
    rng = np.random.default_rng(31)
    sched = ou.linear_schedule()
    x = rng.standard_normal((1, 4, 2, 2))
    eu, ec = rng.standard_normal((2, 1, 4, 2, 2))
    pair = np.concatenate([eu, ec])
    _close(ou.guided_ddpm_step(x, pair, 10, 1.0, sched), ou.ddpm_step(x, ec, 10, sched), 1e-15,
           "scale 1 uses the conditional half")
    _close(ou.guided_ddpm_step(x, pair, 10, 0.0, sched), ou.ddpm_step(x, eu, 10, sched), 1e-15,
           "scale 0 uses the unconditional half")


# ------------------------------------------------------------ key mask
def pin_mask_equals_deleting_keys():
    """Masking keys equals removing them: attention over the kept keys only,
    per sample; all keys kept = no mask; a single kept key gives its V; no
    key kept gives 0."""
    rng = np.random.default_rng(32)
    q = rng.standard_normal((3, 7, 128)) * 2
    k = rng.standard_normal((3, 77, 128)) * 2
    v = rng.standard_normal((3, 77, 128))
    m = np.ones((3, 77), np.int32)
    m[0, 50:] = 0
    m[1, ::3] = 0
    m[2, :] = 0
    m[2, 11] = 1
    o = ob.attention(q, k, v, 2, key_mask=m)
    for b in range(3):
        keep = m[b] != 0
        ref = ob.attention(q[b:b + 1], k[b:b + 1, keep], v[b:b + 1, keep], 2)
        _close(o[b:b + 1], ref, 1e-13, f"mask = deletion, sample {b}")
    _close(o[2], np.broadcast_to(v[2, 11], (7, 128)), 1e-13, "single kept key")
    _close(ob.attention(q, k, v, 2, key_mask=np.ones((3, 77))), ob.attention(q, k, v, 2), 0.0,
           "all-ones mask")
    _close(ob.attention(q, k, v, 2, key_mask=np.zeros((3, 77))), np.zeros_like(q), 0.0,
           "nothing kept")


def pin_mask_library():
    """torch scaled_dot_product_attention with a boolean key mask, fp64."""
    rng = np.random.default_rng(33)
    B, Nq, Nk, heads = 2, 9, 77, 2
    q = rng.standard_normal((B, Nq, 64 * heads)) * 2
    k = rng.standard_normal((B, Nk, 64 * heads)) * 2
    v = rng.standard_normal((B, Nk, 64 * heads))
    m = rng.random((B, Nk)) > 0.4

    def split(a):
        return _t(a).view(a.shape[0], a.shape[1], heads, 64).transpose(1, 2)

    am = torch.from_numpy(m)[:, None, None, :].expand(B, heads, Nq, Nk)
    ref = Fnn.scaled_dot_product_attention(split(q), split(k), split(v), attn_mask=am)
    ref = ref.transpose(1, 2).reshape(B, Nq, 64 * heads).numpy()
    _close(ob.attention(q, k, v, heads, key_mask=m), ref, 1e-12, "masked attention vs SDPA")


def pin_mask_brute_whole_block():
    cfg = synth.BlockConfig("mask_pin", 2, 64, 3, 3, 1, 64, 2, "f32")
    inp = synth.make_inputs(cfg, 34, weight_std=0.15, bias_std=0.1, norm_std=0.2)
    m = np.ones((2, 77), np.int32)
    m[0, 30:] = 0
    m[1, 5:9] = 0
    y = ob.block_forward(inp["x"], inp["ctx"], inp["params"], 1, ctx_mask=m)
    yb = brute.block_forward(inp["x"], inp["ctx"], inp["params"], 1, ctx_mask=m.tolist())
    _close(y, np.array(yb), 1e-11, "masked block vs brute force")



# ------------------------------------------------------------------ U-Net
def _golden(name):
    return [l.split() for l in open(os.path.join(GOLDEN, name))
            if l.strip() and not l.startswith("#")]


def pin_unet_parameter_counts_from_the_pages():
    """The U-Net structure reproduces the parameter counts the pages print:
    SD1.5 (the SD2.1 topology with a 768-wide context) about 860M, SDXL
    Base (4 input channels) 5.14G in FP16 = 2.57e9."""
    import dataclasses
    cfgs = {"sd15": dataclasses.replace(synth.UNET_CONFIGS["sd21"], ctx_dim=768),
            "sdxl_base": dataclasses.replace(synth.UNET_CONFIGS["sdxl_inpaint"], in_channels=4)}
    for name, n, tol in _golden("unet_params.txt"):
        got = synth.unet_param_count(cfgs[name])
        assert abs(got / float(n) - 1.0) <= float(tol), (name, got, n)


def _zero_params(cfg):
    # read-only zero views of the real shapes: the wiring is exercised at the
    # full widths without holding the weights in memory
    return synth._walk(synth.unet_param_shapes(cfg), lambda p, s: np.broadcast_to(np.float32(0), s))


def pin_unet_topology_from_the_pages():
    """Every stage output of the oracle's U-Net has the channels and size of
    the pages' topology diagrams (batch 0: shapes only)."""
    rows = _golden("unet_topology.txt")
    for key in ("sdxl_inpaint", "sd21"):
        cfg = synth.UNET_CONFIGS[key]
        want = {r[1]: tuple(int(v) for v in r[2:]) for r in rows if r[0] == key}
        Cin, H, W = want["input"]
        assert Cin == cfg.in_channels
        rec = []
        x = np.zeros((0, Cin, H, W))
        ctx = np.zeros((0, 77, cfg.ctx_dim))
        add = np.zeros((0, cfg.add_in)) if cfg.add_in else None
        ou.unet_forward(x, np.zeros(0), ctx, _zero_params(cfg), cfg, add, rec)
        got = {name: shape[1:] for name, shape in rec}
        L = len(cfg.channels)
        for lvl in range(L):
            assert got[f"down{lvl}.{cfg.layers_per_block - 1}"] == want[f"down{lvl}"], (key, lvl)
            assert got[f"up{lvl}"] == want[f"up{lvl}"], (key, lvl)
        assert got["mid"] == want["mid"]
        assert got["conv_out"] == want["output"]
        # the skips the diagrams list: the last output kept at each level
        for lvl in range(L):
            assert got[f"down{lvl}.0"][0] == want[f"down{lvl}"][0]


def pin_timestep_embedding():
    """Sinusoidal embedding: t = 0 gives cosines 1 and sines 0; the first
    frequency is 1 (entries cos t, sin t); e(t1) . e(t2) = sum_i cos((t1 -
    t2) f_i) with f_i = 10000^(-i / half), so |e(t)|^2 = half."""
    dim, half = 320, 160
    e = ou.timestep_embedding(np.array([0.0, 1.0, 999.0, 500.5]), dim)
    _close(e[0], np.r_[np.ones(half), np.zeros(half)], 0.0, "t = 0")
    _close([e[2, 0], e[2, half]], [math.cos(999.0), math.sin(999.0)], 1e-12, "first frequency")
    f = 10000.0 ** (-np.arange(half) / half)
    _close(e[2] @ e[3], np.cos((999.0 - 500.5) * f).sum(), 1e-9, "shift identity")
    _close((e * e).sum(axis=1), np.full(4, float(half)), 1e-9, "norm")


def pin_unet_batch_independence():
    cfg = synth.UNetConfig("pin_tiny", 4, 4, (64, 128), (1, 1), 1, 2, 64, add_in=32)
    inp = synth.make_unet_inputs(cfg, 3, 2, 8, 8, weight_std=0.08, t=(999.0, 17.0))
    y = ou.unet_forward(inp["x"], inp["t"], inp["ctx"], inp["params"], cfg, inp["add"])
    for b in range(2):
        yb = ou.unet_forward(inp["x"][b:b + 1], inp["t"][b:b + 1], inp["ctx"][b:b + 1],
                             inp["params"], cfg, inp["add"][b:b + 1])
        _close(y[b:b + 1], yb, 1e-12, f"sample {b} alone")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
