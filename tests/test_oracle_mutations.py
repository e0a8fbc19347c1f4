"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch each of them: a pin suite that a dropped term, a wrong sign, a wrong
index or a transposed operand can pass is no pin at all."""
import math

import numpy as np
import pytest
from scipy.special import erf

import oracle.block as ob
import oracle_pins


def _gn_interleaved(x, gamma, beta, groups=32, eps=1e-6):
    x = np.asarray(x, np.float64)
    B, C, H, W = x.shape
    g = x.reshape(B, C // groups, groups, H, W)          # channel c -> group c % G
    m = g.mean(axis=(1, 3, 4), keepdims=True)
    v = ((g - m) ** 2).mean(axis=(1, 3, 4), keepdims=True)
    z = ((g - m) / np.sqrt(v + eps)).reshape(B, C, H, W)
    return z * np.asarray(gamma)[None, :, None, None] + np.asarray(beta)[None, :, None, None]


def _gn_sample_var(x, gamma, beta, groups=32, eps=1e-6):
    x = np.asarray(x, np.float64)
    B, C, H, W = x.shape
    g = x.reshape(B, groups, C // groups, H, W)
    m = g.mean(axis=(2, 3, 4), keepdims=True)
    n = g[0, 0].size
    v = ((g - m) ** 2).sum(axis=(2, 3, 4), keepdims=True) / (n - 1)
    z = ((g - m) / np.sqrt(v + eps)).reshape(B, C, H, W)
    return z * np.asarray(gamma)[None, :, None, None] + np.asarray(beta)[None, :, None, None]


def _tokens_colmajor(z):
    z = np.asarray(z, np.float64)
    B, C, H, W = z.shape
    return z.transpose(0, 1, 3, 2).reshape(B, C, H * W).transpose(0, 2, 1)


def _linear_no_transpose(t, w, b=None):
    # square W used as (in, out): a transposed operand that still has the
    # right shape (non-square W stay correct, so only numbers can catch it)
    w = np.asarray(w, np.float64)
    y = np.asarray(t, np.float64) @ (w if w.shape[0] == w.shape[1] else w.T)
    return y + (np.asarray(b) if b is not None else 0.0)


def _ln_no_gamma(h, gamma, beta, eps=1e-5):
    h = np.asarray(h, np.float64)
    m = h.mean(axis=-1, keepdims=True)
    v = ((h - m) ** 2).mean(axis=-1, keepdims=True)
    return (h - m) / np.sqrt(v + eps) + np.asarray(beta)


def _attention_scale_1_over_d(q, k, v, heads, row_block=2048, return_probs=False, rows=None):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    return _generic_attention(q, k, v, heads, 1.0 / 64, axis=1, return_probs=return_probs)


def _attention_softmax_over_queries(q, k, v, heads, row_block=2048, return_probs=False, rows=None):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    return _generic_attention(q, k, v, heads, 0.125, axis=0, return_probs=return_probs)


def _attention_interleaved_heads(q, k, v, heads, row_block=2048, return_probs=False, rows=None):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    C = q.shape[-1]
    perm = np.arange(C).reshape(C // heads, heads).T.reshape(-1)  # head = c % heads
    out = _generic_attention(q[..., perm], k[..., perm], v[..., perm], heads, 0.125,
                             axis=1, return_probs=return_probs)
    inv = np.argsort(perm)
    if return_probs:
        return out[0][..., inv], out[1]
    return out[..., inv]


def _generic_attention(q, k, v, heads, scale, axis, return_probs):
    B, Nq, C = q.shape
    d = C // heads
    out = np.empty((B, Nq, C))
    probs = np.empty((B, heads, Nq, k.shape[1]))
    for b in range(B):
        for hd in range(heads):
            sl = slice(hd * d, (hd + 1) * d)
            s = q[b, :, sl] @ k[b, :, sl].T * scale
            e = np.exp(s - s.max(axis=axis, keepdims=True))
            p = e / e.sum(axis=axis, keepdims=True)
            probs[b, hd] = p
            out[b, :, sl] = p @ v[b, :, sl]
    return (out, probs) if return_probs else out


def _gelu_tanh(g):
    g = np.asarray(g, np.float64)
    return 0.5 * g * (1 + np.tanh(math.sqrt(2 / math.pi) * (g + 0.044715 * g ** 3)))


def _geglu_swapped(z, F):
    z = np.asarray(z, np.float64)
    return z[..., F:] * ob.gelu_erf(z[..., :F])


def _sa_no_residual(h, lw, heads):
    u = ob.layer_norm(h, lw["ln1_w"], lw["ln1_b"])
    q = ob.linear(u, lw["q1_w"], lw.get("q1_b"))
    k = ob.linear(u, lw["k1_w"], lw.get("k1_b"))
    v = ob.linear(u, lw["v1_w"], lw.get("v1_b"))
    return ob.linear(ob.attention(q, k, v, heads), lw["o1_w"], lw.get("o1_b"))


def _ca_normalised_context(h, ctx, lw, heads, ctx_mask=None):
    u = ob.layer_norm(h, lw["ln2_w"], lw["ln2_b"])
    c = ob.layer_norm(ctx, np.ones(ctx.shape[-1]), np.zeros(ctx.shape[-1]))
    q = ob.linear(u, lw["q2_w"], lw.get("q2_b"))
    o = ob.attention(q, ob.linear(c, lw["k2_w"], lw.get("k2_b")),
                     ob.linear(c, lw["v2_w"], lw.get("v2_b")), heads, key_mask=ctx_mask)
    return h + ob.linear(o, lw["o2_w"], lw.get("o2_b"))


def _ff_sign_flip(h, lw):
    u = ob.layer_norm(h, lw["ln3_w"], lw["ln3_b"])
    z = ob.linear(u, lw["ff1_w"], lw.get("ff1_b"))
    F = z.shape[-1] // 2
    return h - ob.linear(ob.geglu(z, F), lw["ff2_w"], lw.get("ff2_b"))


def _ff_dropped_bias(h, lw):
    u = ob.layer_norm(h, lw["ln3_w"], lw["ln3_b"])
    z = ob.linear(u, lw["ff1_w"], None)
    F = z.shape[-1] // 2
    return h + ob.linear(ob.geglu(z, F), lw["ff2_w"], lw.get("ff2_b"))


def _from_tokens_transposed(t, H, W):
    t = np.asarray(t, np.float64)
    B, N, C = t.shape
    return t.transpose(0, 2, 1).reshape(B, C, W, H).transpose(0, 1, 3, 2)


MUTATIONS = {
    "gn_interleaved_groups": ("group_norm", _gn_interleaved),
    "gn_sample_variance": ("group_norm", _gn_sample_var),
    "tokens_column_major": ("to_tokens", _tokens_colmajor),
    "untokens_transposed": ("from_tokens", _from_tokens_transposed),
    "linear_no_transpose": ("linear", _linear_no_transpose),
    "ln_missing_gamma": ("layer_norm", _ln_no_gamma),
    "attention_scale_1_over_d": ("attention", _attention_scale_1_over_d),
    "softmax_over_queries": ("attention", _attention_softmax_over_queries),
    "heads_interleaved": ("attention", _attention_interleaved_heads),
    "gelu_tanh_approx": ("gelu_erf", _gelu_tanh),
    "geglu_halves_swapped": ("geglu", _geglu_swapped),
    "self_attn_residual_dropped": ("self_attention_sublayer", _sa_no_residual),
    "context_normalised": ("cross_attention_sublayer", _ca_normalised_context),
    "ff_residual_sign": ("feed_forward_sublayer", _ff_sign_flip),
    "ff1_bias_dropped": ("feed_forward_sublayer", _ff_dropped_bias),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(ob, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"mutation {name} passed every pin"
