"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages, a closed form, an invariant, an independent library routine or
the scalar brute force fixes.  ``tests/test_oracle.py`` runs every pin;
``tests/test_oracle_mutations.py`` plants plausible mistakes in the oracle and
checks that some pin fails for each of them.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch
import torch.nn.functional as Fnn

import oracle.block as ob
import oracle.brute as brute
from latent_diffusion_net_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs diff {err:.3e} > {tol:.1e}"


def _tiny_cfg(**kw):
    base = dict(B=2, C=64, H=3, W=3, heads=1, D_ctx=64, depth=2, dtype="f32")
    base.update(kw)
    return synth.BlockConfig("tiny_pin", **base)


def _stress_inputs(cfg, seed):
    # nonzero biases and norm affines so that every term of the block matters
    return synth.make_inputs(cfg, seed, weight_std=0.15, bias_std=0.1,
                             norm_std=0.2)


# ---------------------------------------------------------------- GroupNorm
def pin_group_norm_invariant():
    """gamma=1, beta=0: each (sample, group) has mean 0, variance s2/(s2+eps)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 64, 5, 4)) * 3.0 + 1.5
    z = ob.group_norm(x, np.ones(64), np.zeros(64))
    g = z.reshape(2, 32, 2, 5, 4)
    xg = x.reshape(2, 32, 2, 5, 4)
    s2 = xg.var(axis=(2, 3, 4))
    _close(g.mean(axis=(2, 3, 4)), np.zeros((2, 32)), 1e-12, "GN group mean")
    _close(g.var(axis=(2, 3, 4)), s2 / (s2 + 1e-6), 1e-12, "GN group variance")


def pin_group_norm_groups_contiguous():
    """Closed form: channel c belongs to group c // (C/32).

    x[c] = c at every pixel, one pixel, C = 64: group g holds the values
    {2g, 2g+1}, so the normalised values are -+ 0.5/sqrt(0.25 + eps).
    """
    x = np.arange(64, dtype=np.float64).reshape(1, 64, 1, 1)
    z = ob.group_norm(x, np.ones(64), np.zeros(64))[0, :, 0, 0]
    a = 0.5 / math.sqrt(0.25 + 1e-6)
    _close(z, np.tile([-a, a], 32), 1e-13, "GN contiguous groups")


def pin_group_norm_library():
    """torch.nn.functional.group_norm in float64 (independent library)."""
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 128, 6, 7))
    g = rng.standard_normal(128)
    b = rng.standard_normal(128)
    ref = Fnn.group_norm(_t(x), 32, _t(g), _t(b), eps=1e-6).numpy()
    _close(ob.group_norm(x, g, b), ref, 1e-12, "GN vs torch")


# ------------------------------------------------------------- token layout
def pin_token_order():
    """Tutorial page reshape (C,H,W)->(C,HW)->(HW,C) and back (golden)."""
    for C, H, W, N in _golden_rows("token_reshape.txt"):
        C, H, W, N = int(C), int(H), int(W), int(N)
        z = np.arange(C * H * W, dtype=np.float64).reshape(1, C, H, W)
        t = ob.to_tokens(z)
        assert t.shape == (1, N, C), "token shape"
        for (i, j) in [(0, 0), (0, W - 1), (1, 0), (H - 1, 2), (H - 1, W - 1)]:
            _close(t[0, i * W + j], z[0, :, i, j], 0.0, "token n = i*W + j")
        _close(ob.from_tokens(t, H, W), z, 0.0, "tokens -> NCHW inverse")


def pin_linear_library():
    """y = x W^T + b with W as (out, in): torch.nn.functional.linear."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 5, 7))
    w = rng.standard_normal((3, 7))
    b = rng.standard_normal(3)
    _close(ob.linear(x, w, b), Fnn.linear(_t(x), _t(w), _t(b)).numpy(), 1e-12,
           "linear vs torch")


def pin_weight_shapes():
    """Cross-attention q/k/v parameter count at C=320, D_ctx=768 (golden)."""
    for C, D, count in _golden_rows("cross_attn_qkv_params.txt"):
        cfg = synth.BlockConfig("pin", 1, int(C), 2, 2, int(C) // 64, int(D), 1, "f32")
        lw = synth.make_inputs(cfg, 0)["params"]["layers"][0]
        n = lw["q2_w"].size + lw["k2_w"].size + lw["v2_w"].size
        assert n == int(count), f"cross q/k/v params {n} != {count}"
        # and the oracle accepts exactly these shapes: Q from C, K/V from D
        h = np.zeros((1, 4, int(C)))
        ctx = np.ones((1, 77, int(D)))
        ob.cross_attention_sublayer(h, ctx, lw, int(C) // 64)


def pin_stage_shapes():
    """The workload table matches the pages' stage shapes and depths (golden)."""
    byname = {c.name: c for c in synth.CONFIGS}
    for name, C, H, W, D, depth in _golden_rows("stage_shapes.txt"):
        c = byname[name]
        assert (c.C, c.H, c.W, c.D_ctx, c.depth) == (int(C), int(H), int(W), int(D), int(depth)), name
        assert c.heads * 64 == c.C


# ---------------------------------------------------------------- LayerNorm
def pin_layer_norm():
    rng = np.random.default_rng(4)
    h = rng.standard_normal((3, 9, 96)) * 2 + 0.7
    u = ob.layer_norm(h, np.ones(96), np.zeros(96))
    s2 = h.var(axis=-1)
    _close(u.mean(axis=-1), np.zeros((3, 9)), 1e-12, "LN mean")
    _close(u.var(axis=-1), s2 / (s2 + 1e-5), 1e-12, "LN variance")
    g = rng.standard_normal(96)
    b = rng.standard_normal(96)
    ref = Fnn.layer_norm(_t(h), (96,), _t(g), _t(b), eps=1e-5).numpy()
    _close(ob.layer_norm(h, g, b), ref, 1e-12, "LN vs torch")


# ---------------------------------------------------------------- attention
def pin_attention_rows_sum_to_one():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 11, 128)) * 3
    k = rng.standard_normal((2, 13, 128)) * 3
    v = rng.standard_normal((2, 13, 128))
    _, p = ob.attention(q, k, v, 2, return_probs=True)
    _close(p.sum(axis=-1), np.ones((2, 2, 11)), 1e-12, "softmax rows sum to 1")
    assert (p >= 0).all()


def pin_attention_uniform():
    """Q = 0 => uniform weights => O is the mean of V over keys, per head."""
    rng = np.random.default_rng(6)
    k = rng.standard_normal((1, 17, 128))
    v = rng.standard_normal((1, 17, 128))
    o = ob.attention(np.zeros((1, 5, 128)), k, v, 2)
    _close(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), 1e-13,
           "uniform attention")


def pin_attention_library():
    """torch scaled_dot_product_attention (default scale 1/sqrt(64)), fp64."""
    rng = np.random.default_rng(7)
    B, Nq, Nk, heads = 2, 19, 23, 3
    q = rng.standard_normal((B, Nq, 64 * heads)) * 2
    k = rng.standard_normal((B, Nk, 64 * heads)) * 2
    v = rng.standard_normal((B, Nk, 64 * heads))

    def split(a):
        return _t(a).view(a.shape[0], a.shape[1], heads, 64).transpose(1, 2)

    ref = Fnn.scaled_dot_product_attention(split(q), split(k), split(v))
    ref = ref.transpose(1, 2).reshape(B, Nq, 64 * heads).numpy()
    _close(ob.attention(q, k, v, heads, row_block=4), ref, 1e-12, "attention vs SDPA")


def pin_cross_attention_context_permutation():
    """Permuting the 77 context tokens leaves cross-attention unchanged."""
    cfg = _tiny_cfg(C=128, heads=2, D_ctx=64, depth=1)
    inp = _stress_inputs(cfg, 11)
    lw = inp["params"]["layers"][0]
    rng = np.random.default_rng(8)
    h = rng.standard_normal((2, 9, 128))
    perm = rng.permutation(77)
    a = ob.cross_attention_sublayer(h, inp["ctx"], lw, 2)
    b = ob.cross_attention_sublayer(h, inp["ctx"][:, perm, :], lw, 2)
    _close(a, b, 1e-12, "context permutation invariance")


def pin_cross_attention_equal_context():
    """All context rows equal => O = that row's V, whatever the queries."""
    cfg = _tiny_cfg(C=128, heads=2, D_ctx=64, depth=1)
    lw = _stress_inputs(cfg, 12)["params"]["layers"][0]
    rng = np.random.default_rng(9)
    row = rng.standard_normal(64)
    ctx = np.broadcast_to(row, (1, 77, 64)).copy()
    h = rng.standard_normal((1, 6, 128))
    u = ob.layer_norm(h, lw["ln2_w"], lw["ln2_b"])
    vrow = ob.linear(row[None, None, :], lw["v2_w"], lw["v2_b"])
    o = ob.attention(ob.linear(u, lw["q2_w"], lw["q2_b"]),
                     ob.linear(ctx, lw["k2_w"], lw["k2_b"]),
                     ob.linear(ctx, lw["v2_w"], lw["v2_b"]), 2)
    _close(o, np.broadcast_to(vrow, o.shape), 1e-12, "equal-context attention")


# -------------------------------------------------------------------- GEGLU
def pin_gelu_values():
    for x, g in _golden_rows("gelu_values.txt"):
        _close(ob.gelu_erf(np.array([float(x)])), [float(g)], 1e-15, f"GELU({x})")
    xs = np.linspace(-6, 6, 101)
    _close(ob.gelu_erf(xs), Fnn.gelu(_t(xs), approximate="none").numpy(), 1e-14,
           "GELU vs torch")


def pin_geglu_halves():
    """Reading: z = [value | gate], out = value * GELU(gate)."""
    z = np.array([[1.0, 2.0, -3.0, 0.0, 1.0, -1.0]])
    want = [0.0, 2.0 * 0.8413447460685429, -3.0 * -0.15865525393145707]
    _close(ob.geglu(z, 3), [want], 1e-15, "GEGLU value/gate halves")


# ------------------------------------------------------- residuals / depth
def pin_zero_sublayers_identity():
    """Zeroed o1, o2, ff2 weights and biases: the layer stack is the identity,
    so y = proj_out(proj_in(GN(x))) + x; with W_out = 0, b_out = 0, y = x."""
    cfg = _tiny_cfg(C=128, heads=2, H=4, W=5, depth=2)
    inp = _stress_inputs(cfg, 13)
    p = synth.map_params(inp["params"], np.array)
    for lw in p["layers"]:
        for k in ("o1_w", "o1_b", "o2_w", "o2_b", "ff2_w", "ff2_b"):
            lw[k] = np.zeros_like(lw[k])
    x = inp["x"]
    y = ob.block_forward(x, inp["ctx"], p, 2)
    z = ob.group_norm(x, p["gn_w"], p["gn_b"])
    h = ob.to_tokens(z) @ np.asarray(p["proj_in_w"], np.float64).T + p["proj_in_b"]
    o = h @ np.asarray(p["proj_out_w"], np.float64).T + p["proj_out_b"]
    _close(y, ob.from_tokens(o, 4, 5) + x, 1e-12, "identity stack")
    p["proj_out_w"] = np.zeros_like(p["proj_out_w"])
    p["proj_out_b"] = np.zeros_like(p["proj_out_b"])
    _close(ob.block_forward(x, inp["ctx"], p, 2), x, 0.0, "y = x")


def pin_spatial_permutation_equivariance():
    """No positional encoding: permuting pixels permutes the output."""
    cfg = _tiny_cfg(C=128, heads=2, H=3, W=4, depth=2)
    inp = _stress_inputs(cfg, 14)
    rng = np.random.default_rng(10)
    perm = rng.permutation(12)
    x = inp["x"]
    xp = x.reshape(2, 128, 12)[:, :, perm].reshape(2, 128, 3, 4)
    y = ob.block_forward(x, inp["ctx"], inp["params"], 2)
    yp = ob.block_forward(xp, inp["ctx"], inp["params"], 2)
    _close(yp, y.reshape(2, 128, 12)[:, :, perm].reshape(2, 128, 3, 4), 1e-12,
           "spatial permutation equivariance")


def pin_batch_independence():
    cfg = _tiny_cfg(C=128, heads=2, H=3, W=3, depth=1)
    inp = _stress_inputs(cfg, 15)
    y = ob.block_forward(inp["x"], inp["ctx"], inp["params"], 2)
    y1 = ob.block_forward(inp["x"][1:], inp["ctx"][1:], inp["params"], 2)
    _close(y[1:], y1, 1e-12, "batch independence")


def pin_brute_force_whole_block():
    """Scalar-loop oracle vs vectorised oracle on a tiny block, depth 2."""
    cfg = _tiny_cfg()
    inp = _stress_inputs(cfg, 16)
    y = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    yb = np.array(brute.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads))
    _close(y, yb, 1e-11, "brute force vs vectorised")


def pin_brute_force_two_heads():
    """Brute force with 2 heads, non-square map, 1 layer."""
    cfg = _tiny_cfg(B=1, C=128, heads=2, H=2, W=3, depth=1)
    inp = _stress_inputs(cfg, 17)
    y = ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    yb = np.array(brute.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads))
    _close(y, yb, 1e-11, "brute force, 2 heads")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
