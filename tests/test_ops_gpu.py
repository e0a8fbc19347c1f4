"""Standalone operations on the GPU against the fp64 oracle, through the C
ABI: GroupNorm (+SiLU) on NCHW maps and the guided DDPM step.

Tolerances.  GroupNorm with bf16 storage: statistics in fp32/fp64, one
rounding of the output to bf16 (u = 2^-8), so max-abs <= 3e-2 and rel-L2 <=
1e-2 (the block's bf16 gate); fp32 storage: rel-L2 <= 1e-5.  DDPM step: the
update runs in fp32 on exactly the oracle's inputs (a bf16 prediction is
exact in fp64), a handful of roundings of u = 2^-24 each: rel-L2 <= 1e-6 and
max-abs <= 1e-5 * max(1, max |x_prev|).
"""
import numpy as np
import pytest

import oracle.block as ob
import oracle.unet as ou
from latent_diffusion_net_amd import synth

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


def _rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


GN_CASES = [
    # ResnetBlock2D norms at the SDXL Down1 and SD2.1 Down0 stage shapes
    dict(B=2, C=640, H=64, W=64, silu=True, eps=1e-5, affine=True, dtype="bf16"),
    dict(B=2, C=320, H=96, W=96, silu=True, eps=1e-5, affine=False, dtype="bf16"),
    # concatenated up-block input (1920 channels: 60 per group), no SiLU
    dict(B=2, C=1920, H=16, W=16, silu=False, eps=1e-6, affine=True, dtype="bf16"),
    # ragged planes (35 pixels: the scalar path), fp32 storage
    dict(B=1, C=64, H=5, W=7, silu=True, eps=1e-5, affine=True, dtype="f32"),
    dict(B=3, C=96, H=17, W=9, silu=False, eps=1e-6, affine=True, dtype="f32"),
    dict(B=1, C=32, H=1, W=1, silu=True, eps=1e-5, affine=True, dtype="bf16"),
]


@pytest.mark.parametrize("case", GN_CASES, ids=lambda c: f"b{c['B']}_c{c['C']}_{c['H']}x{c['W']}_{c['dtype']}")
def test_group_norm_op(case):
    import torch
    from latent_diffusion_net_amd.binding import group_norm
    B, C, H, W = case["B"], case["C"], case["H"], case["W"]
    rng = np.random.default_rng(B * 1000 + C + H)
    x = (rng.standard_normal((B, C, H, W)) * 2.0 + 0.5).astype(np.float32)
    g = (1 + 0.2 * rng.standard_normal(C)).astype(np.float32) if case["affine"] else None
    bt = (0.2 * rng.standard_normal(C)).astype(np.float32) if case["affine"] else None
    if case["dtype"] == "bf16":
        x = synth.round_bf16(x)
        g = synth.round_bf16(g) if g is not None else None
        bt = synth.round_bf16(bt) if bt is not None else None
    tdt = torch.bfloat16 if case["dtype"] == "bf16" else torch.float32
    dev = lambda a: None if a is None else torch.from_numpy(a).to("cuda").to(tdt)
    _say(f"[gpu] group_norm {case}")
    y = group_norm(dev(x), dev(g), dev(bt), eps=case["eps"], silu=case["silu"])
    torch.cuda.synchronize()
    y = y.float().cpu().numpy().astype(np.float64)
    ref = ob.group_norm(x, g if g is not None else np.ones(C), bt if bt is not None else np.zeros(C),
                        eps=case["eps"])
    if case["silu"]:
        ref = ou.silu(ref)
    err, rel = float(np.abs(y - ref).max()), _rel(y, ref)
    _say(f"    max_abs={err:.3e} rel_l2={rel:.3e}")
    if case["dtype"] == "bf16":
        assert err <= 3e-2 and rel <= 1e-2
    else:
        assert rel <= 1e-5


DDPM_CASES = [
    # SDXL latent pair (4 x 128 x 128), bf16 prediction, first, middle and last step
    dict(n=4 * 128 * 128, t=1000, scale=7.5, noise=True, dtype="bf16"),
    dict(n=4 * 128 * 128, t=500, scale=5.0, noise=True, dtype="bf16"),
    dict(n=4 * 128 * 128, t=1, scale=7.5, noise=False, dtype="bf16"),
    # fp32 prediction, ragged length, no guidance (scale 1)
    dict(n=1001, t=37, scale=1.0, noise=True, dtype="f32"),
    dict(n=1, t=2, scale=0.0, noise=True, dtype="f32"),
]


@pytest.mark.parametrize("case", DDPM_CASES, ids=lambda c: f"n{c['n']}_t{c['t']}_{c['dtype']}")
def test_guided_ddpm_step(case):
    import torch
    from latent_diffusion_net_amd.binding import guided_ddpm_step
    n, t = case["n"], case["t"]
    rng = np.random.default_rng(n + t)
    eps = rng.standard_normal((2, n)).astype(np.float32)
    if case["dtype"] == "bf16":
        eps = synth.round_bf16(eps)
    x = rng.standard_normal(n).astype(np.float32)
    z = rng.standard_normal(n).astype(np.float32) if case["noise"] else None
    tdt = torch.bfloat16 if case["dtype"] == "bf16" else torch.float32
    _say(f"[gpu] guided DDPM step {case}")
    xp = guided_ddpm_step(torch.from_numpy(eps).cuda().to(tdt), torch.from_numpy(x).cuda(), t,
                          case["scale"], None if z is None else torch.from_numpy(z).cuda())
    torch.cuda.synchronize()
    xp = xp.cpu().numpy().astype(np.float64)
    ref = ou.guided_ddpm_step(x, eps, t, case["scale"], ou.linear_schedule(), z).reshape(n)
    err, rel = float(np.abs(xp - ref).max()), _rel(xp, ref)
    _say(f"    max_abs={err:.3e} rel_l2={rel:.3e}")
    assert rel <= 1e-6
    assert err <= 1e-5 * max(1.0, float(np.abs(ref).max()))
