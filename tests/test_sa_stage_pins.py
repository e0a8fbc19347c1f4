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
  * no scale -- softmax(Q K^T) without the 1/sqrt(64).
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


MUTATIONS = {"flat": _flat, "half": _half, "unweighted_merge": _unweighted_merge,
             "no_scale": _no_scale}

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
