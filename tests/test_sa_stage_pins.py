"""CPU: the bounds of the non-flat self-attention parity tests catch the
mistakes they are meant to catch.

Each mistake is planted in the oracle's attention (never in the GPU path)
and its self-attention update is compared with the oracle's own under the
bounds that tests/test_parity_gpu.py::test_self_attention_sharp applies to
the GPU; every mutation must exceed them by a wide margin.  The mutations
are what a wrong K tile, rescale or merge in the kernel would produce:
  * flat     -- scores ignored: every query gets the mean of V;
  * half     -- the keys of the second half dropped (a missing key piece);
  * unweighted merge -- two key pieces each normalised on its own and
                averaged, without their maxima and row sums;
  * no scale -- softmax(Q K^T) without the 1/sqrt(64);
  * no rescale -- keys taken in tiles of 64 against a lazy reference max
                (raised when a tile's max exceeds it by more than 8 in base
                2, as both kernels do), with the row sums rescaled but the
                accumulated output not.
A further check counts, on the oracle's own scores, how many queries take
at least one such lazy rescale, so that the GPU tests are known to reach
that path.
"""
import numpy as np
import pytest

import oracle.block as ob
import sa_stage as sa

MARGIN = 3.0  # every mutation must exceed the bound at least this much
_attention = ob.attention  # the oracle's own, captured before any patching


def _flat(q, k, v, heads, **kw):
    q = np.asarray(q, np.float64)
    v = np.asarray(v, np.float64)
    return np.broadcast_to(v.mean(axis=1, keepdims=True), q.shape[:2] + (v.shape[2],)).copy()


def _half(q, k, v, heads, **kw):
    n = (np.asarray(k).shape[1] + 1) // 2
    return _attention(q, np.asarray(k)[:, :n], np.asarray(v)[:, :n], heads)


def _unweighted_merge(q, k, v, heads, **kw):
    k = np.asarray(k)
    v = np.asarray(v)
    n = (k.shape[1] + 1) // 2
    a = _attention(q, k[:, :n], v[:, :n], heads)
    b = _attention(q, k[:, n:], v[:, n:], heads)
    return 0.5 * (a + b)


def _no_scale(q, k, v, heads, **kw):
    return _attention(8.0 * np.asarray(q, np.float64), k, v, heads)


LAZY_BOUND = 8.0  # base-2 excess over the reference max that forces a rescale


def _lazy_events(s2):
    """Rescale events per row of base-2 scores s2 [rows, keys] under the
    lazy rule (tile 0 sets the reference max exactly)."""
    nt = (s2.shape[1] + 63) // 64
    m = s2[:, :64].max(axis=1)
    ev = np.zeros(s2.shape[0], np.int64)
    for t in range(1, nt):
        mt = s2[:, 64 * t:64 * t + 64].max(axis=1)
        big = mt > m + LAZY_BOUND
        ev += big
        m = np.where(big, mt, m)
    return ev


def _no_rescale(q, k, v, heads, **kw):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Nq, C = q.shape
    Nk = k.shape[1]
    out = np.empty((B, Nq, C))
    for b in range(B):
        for hd in range(heads):
            sl = slice(64 * hd, 64 * hd + 64)
            s2 = (q[b, :, sl] @ k[b, :, sl].T) / 8.0 * np.log2(np.e)
            m = s2[:, :64].max(axis=1)
            e = np.exp2(s2[:, :64] - m[:, None])
            o = e @ v[b, :64, sl]
            l = e.sum(axis=1)
            for t in range(1, (Nk + 63) // 64):
                st = s2[:, 64 * t:64 * t + 64]
                mt = st.max(axis=1)
                big = mt > m + LAZY_BOUND
                m_new = np.where(big, mt, m)
                l = l * np.exp2(m - m_new)  # the output is (wrongly) not rescaled
                m = m_new
                e = np.exp2(st - m[:, None])
                o = o + e @ v[b, 64 * t:64 * t + 64, sl]
                l = l + e.sum(axis=1)
            out[b, :, sl] = o / l[:, None]
    return out


MUTATIONS = {"flat": _flat, "half": _half, "unweighted_merge": _unweighted_merge,
             "no_scale": _no_scale, "no_rescale": _no_rescale}

# the forced split plans and the ragged C=640 shape every time; the full
# SDXL Down1 shape too (about 90 GFLOP of fp64 attention per evaluation)
SPECS = [s for s in sa.SHAPES if s.get("pins", True)]


@pytest.mark.parametrize("spec", SPECS, ids=lambda s: s["name"])
def test_mutations_exceed_update_bounds(spec):
    cfg, inp = sa.inputs(spec)
    h0, h1 = sa.oracle_stage1(inp, cfg.heads)
    d_ref = h1 - h0
    # the softmax is far from flat: the largest probability of a row is
    # well above 1/N for most rows (checked on a few rows of head 0)
    p = inp["params"]["layers"][0]
    u = ob.layer_norm(h0[:1, :64], p["ln1_w"], p["ln1_b"])
    q = ob.linear(u, p["q1_w"], p.get("q1_b"))
    uk = ob.layer_norm(h0[:1], p["ln1_w"], p["ln1_b"])
    kk = ob.linear(uk, p["k1_w"], p.get("k1_b"))
    s = (q[0, :, :64] @ kk[0, :, :64].T) / 8.0
    pr = np.exp(s - s.max(axis=1, keepdims=True))
    pr /= pr.sum(axis=1, keepdims=True)
    assert np.median(pr.max(axis=1)) > 20.0 / cfg.N
    for name, fn in MUTATIONS.items():
        _, hm = sa.oracle_stage1(inp, cfg.heads, attention=fn)
        rel, mx = sa.update_errors(hm - h0, d_ref)
        print(f"{spec['name']} {name}: rel_l2={rel:.3e} max_abs/max={mx:.3e}")
        assert rel > MARGIN * sa.UPDATE_REL_L2, (name, rel)


@pytest.mark.parametrize("spec", [s for s in SPECS if s["cus"] is None], ids=lambda s: s["name"])
def test_sharp_inputs_reach_the_lazy_rescale(spec):
    """At the full-size sharp shapes a good share of the queries see a key
    tile whose maximum exceeds the running reference by more than 8 (base
    2), so the kernels' rescale path runs in the GPU tests (head 0, every
    8th query of sample 0)."""
    cfg, inp = sa.inputs(spec)
    p = inp["params"]
    lw = p["layers"][0]
    z = ob.group_norm(inp["x"][:1], p["gn_w"], p["gn_b"])
    h0 = ob.linear(ob.to_tokens(z), p["proj_in_w"], p.get("proj_in_b"))
    u = ob.layer_norm(h0, lw["ln1_w"], lw["ln1_b"])
    q = ob.linear(u[:, ::8], lw["q1_w"][:64], None if lw.get("q1_b") is None else lw["q1_b"][:64])
    k = ob.linear(u, lw["k1_w"][:64], None if lw.get("k1_b") is None else lw["k1_b"][:64])
    ev = _lazy_events((q[0] @ k[0].T) / 8.0 * np.log2(np.e))
    share = float((ev > 0).mean())
    print(f"{spec['name']}: {share:.2f} of the queries take a lazy rescale")
    assert share >= 0.1, share
