"""Scalar-loop oracle of the Spatial-Transformer block, for tiny shapes.

TEST INFRASTRUCTURE ONLY.  Written independently of ``oracle.block``: Python
floats (IEEE double), nested lists and explicit loops, stdlib ``math`` only.
It exists to cross-check the vectorised oracle element by element.  Same
definition and readings as ``oracle.block`` (pages cited there): GroupNorm(32
contiguous channel groups, eps 1e-6, population variance) -> tokens n = i*W+j
-> proj_in -> depth x [LN -> self-attn -> +, LN -> cross-attn over the
un-normalised context -> +, LN -> GEGLU(value = first half, gate = second
half, exact-erf GELU) -> Linear -> +] -> proj_out -> NCHW -> + x.
"""
from __future__ import annotations

import math


def _mean(vals):
    s = 0.0
    for v in vals:
        s += v
    return s / len(vals)


def _lin(vec, w, b):
    """One output row: out[o] = sum_i vec[i] * w[o][i] + b[o]."""
    out = []
    for o in range(len(w)):
        acc = 0.0
        row = w[o]
        for i in range(len(vec)):
            acc += vec[i] * row[i]
        out.append(acc + (b[o] if b is not None else 0.0))
    return out


def _ln(vec, g, bt, eps=1e-5):
    m = _mean(vec)
    var = _mean([(v - m) * (v - m) for v in vec])
    r = 1.0 / math.sqrt(var + eps)
    return [(vec[c] - m) * r * g[c] + bt[c] for c in range(len(vec))]


def _attend(qrow, keys, vals, heads):
    """Attention of one query row against lists of key/value rows."""
    C = len(qrow)
    d = C // heads
    out = [0.0] * C
    for hd in range(heads):
        lo = hd * d
        scores = []
        for kr in keys:
            s = 0.0
            for j in range(d):
                s += qrow[lo + j] * kr[lo + j]
            scores.append(s / math.sqrt(d))
        mx = max(scores)
        ex = [math.exp(s - mx) for s in scores]
        tot = sum(ex)
        for j in range(d):
            acc = 0.0
            for n in range(len(keys)):
                acc += ex[n] / tot * vals[n][lo + j]
            out[lo + j] = acc
    return out


def _gelu(g):
    return 0.5 * g * (1.0 + math.erf(g / math.sqrt(2.0)))


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def block_forward(x, ctx, params, heads, groups=32, gn_eps=1e-6, ctx_mask=None):
    """Return y as nested lists [B][C][H][W].

    ``ctx_mask`` [B][77] (nonzero = real token): the cross-attention of
    sample b attends over the unmasked context tokens only (none: its output
    is 0)."""
    x = _tolist(x)
    ctx = _tolist(ctx)
    P = {k: _tolist(v) for k, v in params.items() if k != "layers"}
    layers = [{k: _tolist(v) for k, v in lw.items()} for lw in params["layers"]]
    B, C, H, W = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0])
    cg = C // groups
    y = []
    for b in range(B):
        # GroupNorm
        z = [[[0.0] * W for _ in range(H)] for _ in range(C)]
        for g in range(groups):
            vals = [x[b][c][i][j] for c in range(g * cg, (g + 1) * cg)
                    for i in range(H) for j in range(W)]
            m = _mean(vals)
            var = _mean([(v - m) * (v - m) for v in vals])
            r = 1.0 / math.sqrt(var + gn_eps)
            for c in range(g * cg, (g + 1) * cg):
                for i in range(H):
                    for j in range(W):
                        z[c][i][j] = (x[b][c][i][j] - m) * r * P["gn_w"][c] + P["gn_b"][c]
        # tokens in row-major pixel order, then proj_in
        tok = []
        for i in range(H):
            for j in range(W):
                tok.append(_lin([z[c][i][j] for c in range(C)],
                                P["proj_in_w"], P.get("proj_in_b")))
        ctx_b = ctx[b]
        if ctx_mask is not None:
            ctx_b = [ctx_b[n] for n in range(len(ctx_b)) if ctx_mask[b][n]]
        for lw in layers:
            u = [_ln(t, lw["ln1_w"], lw["ln1_b"]) for t in tok]
            qs = [_lin(r, lw["q1_w"], lw.get("q1_b")) for r in u]
            ks = [_lin(r, lw["k1_w"], lw.get("k1_b")) for r in u]
            vs = [_lin(r, lw["v1_w"], lw.get("v1_b")) for r in u]
            new = []
            for n in range(len(tok)):
                o = _lin(_attend(qs[n], ks, vs, heads), lw["o1_w"], lw.get("o1_b"))
                new.append([tok[n][c] + o[c] for c in range(C)])
            tok = new
            u = [_ln(t, lw["ln2_w"], lw["ln2_b"]) for t in tok]
            qs = [_lin(r, lw["q2_w"], lw.get("q2_b")) for r in u]
            ks = [_lin(r, lw["k2_w"], lw.get("k2_b")) for r in ctx_b]
            vs = [_lin(r, lw["v2_w"], lw.get("v2_b")) for r in ctx_b]
            new = []
            for n in range(len(tok)):
                att = _attend(qs[n], ks, vs, heads) if ks else [0.0] * C
                o = _lin(att, lw["o2_w"], lw.get("o2_b"))
                new.append([tok[n][c] + o[c] for c in range(C)])
            tok = new
            new = []
            for t in tok:
                u = _ln(t, lw["ln3_w"], lw["ln3_b"])
                zz = _lin(u, lw["ff1_w"], lw.get("ff1_b"))
                F = len(zz) // 2
                f = [zz[k] * _gelu(zz[F + k]) for k in range(F)]
                o = _lin(f, lw["ff2_w"], lw.get("ff2_b"))
                new.append([t[c] + o[c] for c in range(C)])
            tok = new
        out = [_lin(t, P["proj_out_w"], P.get("proj_out_b")) for t in tok]
        yb = [[[out[i * W + j][c] + x[b][c][i][j] for j in range(W)]
               for i in range(H)] for c in range(C)]
        y.append(yb)
    return y


# ------------------------------------------------------------ U-Net parts
def _silu(v):
    return v / (1.0 + math.exp(-v)) if v > -700.0 else 0.0


def conv2d(x, w, b=None, stride=1, padding=1):
    """Cross-correlation with zero padding, scalar loops: [B][Ci][H][W] ->
    [B][Co][Ho][Wo]."""
    x = _tolist(x)
    w = _tolist(w)
    b = _tolist(b) if b is not None else None
    B, Ci, H, W = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0])
    Co, kh, kw = len(w), len(w[0][0]), len(w[0][0][0])
    Ho = (H + 2 * padding - kh) // stride + 1
    Wo = (W + 2 * padding - kw) // stride + 1
    out = []
    for bb in range(B):
        ob_ = []
        for co in range(Co):
            plane = []
            for i in range(Ho):
                row = []
                for j in range(Wo):
                    acc = b[co] if b is not None else 0.0
                    for ci in range(Ci):
                        for di in range(kh):
                            ii = i * stride + di - padding
                            if ii < 0 or ii >= H:
                                continue
                            for dj in range(kw):
                                jj = j * stride + dj - padding
                                if jj < 0 or jj >= W:
                                    continue
                                acc += w[co][ci][di][dj] * x[bb][ci][ii][jj]
                    row.append(acc)
                plane.append(row)
            ob_.append(plane)
        out.append(ob_)
    return out


def _group_norm(x, g, bt, groups, eps):
    B, C, H, W = len(x), len(x[0]), len(x[0][0]), len(x[0][0][0])
    cg = C // groups
    z = [[[[0.0] * W for _ in range(H)] for _ in range(C)] for _ in range(B)]
    for b in range(B):
        for gr in range(groups):
            vals = [x[b][c][i][j] for c in range(gr * cg, (gr + 1) * cg)
                    for i in range(H) for j in range(W)]
            m = _mean(vals)
            var = _mean([(v - m) * (v - m) for v in vals])
            r = 1.0 / math.sqrt(var + eps)
            for c in range(gr * cg, (gr + 1) * cg):
                for i in range(H):
                    for j in range(W):
                        z[b][c][i][j] = (x[b][c][i][j] - m) * r * g[c] + bt[c]
    return z


def _map4(x, f):
    return [[[[f(v) for v in row] for row in plane] for plane in s] for s in x]


def resnet_block(x, temb, p, groups=32, eps=1e-5):
    """ResnetBlock2D (same definition and readings as oracle.unet), scalar
    loops; returns [B][Co][H][W]."""
    x = _tolist(x)
    temb = _tolist(temb)
    P = {k: _tolist(v) for k, v in p.items()}
    B, Ci = len(x), len(x[0])
    h = conv2d(_map4(_group_norm(x, P["gn1_w"], P["gn1_b"], groups, eps), _silu),
               P["conv1_w"], P.get("conv1_b"))
    Co = len(h[0])
    for b in range(B):
        t = _lin([_silu(v) for v in temb[b]], P["temb_w"], P.get("temb_b"))
        for c in range(Co):
            h[b][c] = [[v + t[c] for v in row] for row in h[b][c]]
    h = conv2d(_map4(_group_norm(h, P["gn2_w"], P["gn2_b"], groups, eps), _silu),
               P["conv2_w"], P.get("conv2_b"))
    if Ci != Co:
        w11 = [[[[P["sc_w"][co][ci]]] for ci in range(Ci)] for co in range(Co)]
        sc = conv2d(x, w11, P.get("sc_b"), padding=0)
    else:
        sc = x
    return [[[[sc[b][c][i][j] + h[b][c][i][j] for j in range(len(h[b][c][i]))]
              for i in range(len(h[b][c]))] for c in range(Co)] for b in range(B)]
