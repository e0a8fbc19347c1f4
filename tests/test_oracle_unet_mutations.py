"""Plant plausible mistakes in the oracle's U-Net parts and in its key mask
(on the CPU) and check that some pin of tests/oracle_pins_unet.py catches
each of them."""
import math

import numpy as np
import pytest

import oracle.block as ob
import oracle.unet as ou
import oracle_pins_unet

_conv = ou.conv2d
_attention = ob.attention
_emb = ou.timestep_embedding
_gn = ou.group_norm
_linear = ou.linear


def _relu(x):
    return np.maximum(np.asarray(x, np.float64), 0.0)


def _silu_sigmoid_only(x):
    x = np.asarray(x, np.float64)
    return 1.0 / (1.0 + np.exp(-x))


def _conv_flipped(x, w, b=None, stride=1, padding=1):
    return _conv(x, np.asarray(w)[:, :, ::-1, ::-1], b, stride, padding)


def _conv_no_bias(x, w, b=None, stride=1, padding=1):
    return _conv(x, w, None, stride, padding)


def _conv_transposed_channels(x, w, b=None, stride=1, padding=1):
    w = np.asarray(w)
    if w.shape[0] == w.shape[1]:
        w = w.transpose(1, 0, 2, 3)
    return _conv(x, w, b, stride, padding)


def _upsample_bilinearish(x):
    x = np.asarray(x, np.float64)
    up = np.repeat(np.repeat(x, 2, axis=2), 2, axis=3)
    up[:, :, 1:-1:2, :] = 0.5 * (up[:, :, 1:-1:2, :] + up[:, :, 2::2, :])
    return up


def _resnet(variant):
    def f(x, temb, p, groups=32, eps=1e-5):
        x = np.asarray(x, np.float64)
        h = _conv(ou.silu(_gn(x, p["gn1_w"], p["gn1_b"], groups, eps)), p["conv1_w"], p.get("conv1_b"))
        t = _linear(temb if variant == "temb_no_silu" else ou.silu(temb), p["temb_w"], p.get("temb_b"))
        if variant != "temb_after_norm2":
            h = h + t[:, :, None, None]
        g = _gn(h, p["gn2_w"], p["gn2_b"], groups, eps)
        if variant == "temb_after_norm2":
            g = g + t[:, :, None, None]
        g = g if variant == "no_silu2" else ou.silu(g)
        h = _conv(g, p["conv2_w"], p.get("conv2_b"))
        if variant == "no_shortcut":
            return h
        if x.shape[1] != h.shape[1]:
            sc = _conv(x, np.asarray(p["sc_w"])[:, :, None, None], p.get("sc_b"), padding=0)
        else:
            sc = x
        return sc + h
    return f


def _cfg_reversed(eu, ec, scale):
    eu, ec = np.asarray(eu, np.float64), np.asarray(ec, np.float64)
    return ec + scale * (eu - ec)


def _schedule_off_by_one(T=1000, beta_start=1e-4, beta_end=0.02):
    beta = np.linspace(beta_start, beta_end, T + 1)[1:]
    alpha = 1.0 - beta
    return beta, alpha, np.cumprod(alpha)


def _ddpm(variant):
    def f(x_t, eps, t, schedule, noise=None):
        beta, alpha, ab = schedule
        bt, at, abt = beta[t - 1], alpha[t - 1], ab[t - 1]
        c = bt / math.sqrt(1.0 - abt) if variant != "sqrt_alphabar" else bt / math.sqrt(abt)
        out = np.asarray(x_t, np.float64) - c * np.asarray(eps, np.float64)
        if variant != "no_inv_sqrt_alpha":
            out = out / math.sqrt(at)
        if noise is not None:
            out = out + (bt if variant == "sigma_beta" else math.sqrt(bt)) * np.asarray(noise)
        return out
    return f


def _mask_ignored(q, k, v, heads, row_block=2048, return_probs=False, rows=None, key_mask=None):
    return _attention(q, k, v, heads, row_block, return_probs, rows)


def _mask_inverted(q, k, v, heads, row_block=2048, return_probs=False, rows=None, key_mask=None):
    if key_mask is not None:
        key_mask = (np.asarray(key_mask) == 0).astype(np.int32)
    return _attention(q, k, v, heads, row_block, return_probs, rows, key_mask)


def _mask_zero_value(q, k, v, heads, row_block=2048, return_probs=False, rows=None, key_mask=None):
    # masked keys keep their weight but contribute V = 0
    if key_mask is None:
        return _attention(q, k, v, heads, row_block, return_probs, rows)
    v = np.asarray(v, np.float64) * (np.asarray(key_mask) != 0)[:, :, None]
    return _attention(q, k, v, heads, row_block, return_probs, rows)


def _emb_sin_first(t, dim):
    e = _emb(t, dim)
    h = dim // 2
    return np.concatenate([e[:, h:], e[:, :h]], axis=1)


def _emb_freq_per_dim(t, dim):
    t = np.asarray(t, np.float64).reshape(-1)
    half = dim // 2
    f = np.exp(-math.log(10000.0) * np.arange(half) / dim)  # exponent over dim, not half
    a = t[:, None] * f[None, :]
    return np.concatenate([np.cos(a), np.sin(a)], axis=1)


def _no_upsample(x):
    return np.asarray(x, np.float64)


MUTATIONS = {
    "silu_is_relu": (ou, "silu", _relu),
    "silu_sigmoid_only": (ou, "silu", _silu_sigmoid_only),
    "conv_kernel_flipped": (ou, "conv2d", _conv_flipped),
    "conv_bias_dropped": (ou, "conv2d", _conv_no_bias),
    "conv_channels_transposed": (ou, "conv2d", _conv_transposed_channels),
    "upsample_interpolated": (ou, "upsample_nearest2x", _upsample_bilinearish),
    "resnet_temb_after_norm2": (ou, "resnet_block", _resnet("temb_after_norm2")),
    "resnet_temb_without_silu": (ou, "resnet_block", _resnet("temb_no_silu")),
    "resnet_no_silu_after_norm2": (ou, "resnet_block", _resnet("no_silu2")),
    "resnet_shortcut_dropped": (ou, "resnet_block", _resnet("no_shortcut")),
    "cfg_halves_swapped": (ou, "cfg_combine", _cfg_reversed),
    "schedule_off_by_one": (ou, "linear_schedule", _schedule_off_by_one),
    "ddpm_sqrt_alphabar": (ou, "ddpm_step", _ddpm("sqrt_alphabar")),
    "ddpm_no_inv_sqrt_alpha": (ou, "ddpm_step", _ddpm("no_inv_sqrt_alpha")),
    "ddpm_sigma_beta": (ou, "ddpm_step", _ddpm("sigma_beta")),
    "embedding_sines_first": (ou, "timestep_embedding", _emb_sin_first),
    "embedding_frequencies_over_dim": (ou, "timestep_embedding", _emb_freq_per_dim),
    "unet_upsampling_dropped": (ou, "upsample_nearest2x", _no_upsample),
    "mask_ignored": (ob, "attention", _mask_ignored),
    "mask_inverted": (ob, "attention", _mask_inverted),
    "mask_zero_value": (ob, "attention", _mask_zero_value),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_unet_pin_catches(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in oracle_pins_unet.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
            break  # one pin that fails is enough
    assert caught, f"mutation {name} passed every pin"
