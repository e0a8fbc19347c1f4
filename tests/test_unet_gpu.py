"""One U-Net denoiser timestep on the GPU (st_unet_*) against the fp64
oracle (oracle.unet.unet_forward), every output element, through the C ABI.

Tolerance.  Each part meets its own bf16 gate; the U-Net chains them: every
ResNet, transformer block and convolution output is stored in bf16 (unit
roundoff u = 2^-8), so the output carries the accumulated relative error of
S such roundings, partly cancelling: rel-L2 <= u sqrt(S) c with c = 2 (the
parts' own errors are about one u each, measured), and max-abs <= 8 u
max |y| (a few roundings of the largest values line up).  S counts the
stored stages of the configuration (parts + skip copies).
"""
import math

import numpy as np
import pytest

import oracle.unet as ou
from latent_diffusion_net_amd import synth

pytestmark = pytest.mark.gpu
U = 2.0 ** -8


def _say(msg):
    print(msg, flush=True)


def stages(cfg):
    L = len(cfg.channels)
    n = 1 + 1 + 2 + (1 if cfg.mid_depth else 0)  # conv_in, conv_out, mid
    for l in range(L):
        per = 2 if cfg.depths[l] else 1
        n += cfg.layers_per_block * per + (cfg.layers_per_block + 1) * per
    return n + 2 * (L - 1)


def run_unet(cfg, inp, B, H, W):
    import torch
    from latent_diffusion_net_amd import STUNet, tree_to_device
    p = tree_to_device(inp["params"])
    bf = lambda a: torch.from_numpy(a).to("cuda").to(torch.bfloat16).contiguous()
    x, ctx = bf(inp["x"]), bf(inp["ctx"])
    add = bf(inp["add"]) if inp["add"] is not None else None
    t = torch.from_numpy(inp["t"]).cuda()
    u = STUNet(cfg, B, H, W, p)
    del p
    y = u.forward(x, t, ctx, add)
    y2 = u.forward(x, t, ctx, add)
    u.check_range()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    _say(f"    device bytes held by the handle: {u.device_bytes() / 2**30:.2f} GiB")
    u.close()
    return y.float().cpu().numpy().astype(np.float64)


CASES = [
    # two levels, ResNet + transformer everywhere, extra embedding
    (synth.UNetConfig("tiny2", 4, 4, (64, 128), (1, 1), 1, 2, 64, add_in=32), 2, 16, 16, 0.05),
    # three levels, a ResNet-only level, depth 2 in the middle of the down path
    (synth.UNetConfig("tiny3", 9, 4, (64, 128, 192), (0, 2, 1), 1, 2, 128, add_in=64), 2, 16, 16, 0.05),
    # the real SD2.1-base and SDXL-Inpaint widths and depths at a 32 x 32 latent
    (synth.UNET_CONFIGS["sd21"], 2, 32, 32, 0.02),
    (synth.UNET_CONFIGS["sdxl_inpaint"], 1, 32, 32, 0.02),
]


@pytest.mark.parametrize("cfg,B,H,W,std", CASES, ids=[f"{c[0].name}_{c[2]}x{c[3]}_b{c[1]}" for c in CASES])
def test_unet_timestep(cfg, B, H, W, std):
    inp = synth.make_unet_inputs(cfg, 900 + H, B, H, W, weight_std=std, t=(999.0, 431.0))
    _say(f"[gpu] unet {cfg.name} B={B} {H}x{W}")
    y = run_unet(cfg, inp, B, H, W)
    _say("    oracle ...")
    yo = ou.unet_forward(inp["x"], inp["t"], inp["ctx"], inp["params"], cfg, inp["add"])
    check(cfg, y, yo)


def check(cfg, y, yo):
    err = float(np.abs(y - yo).max())
    rel = float(np.linalg.norm(y - yo) / np.linalg.norm(yo))
    S = stages(cfg)
    rb = 2.0 * U * math.sqrt(S)
    mb = 8.0 * U * float(np.abs(yo).max())
    _say(f"    max_abs={err:.3e} (bound {mb:.3e}) rel_l2={rel:.3e} (bound {rb:.3e}, {S} stages)")
    assert np.isfinite(y).all()
    assert rel <= rb
    assert err <= mb


def test_unet_sd21_full_size():
    """SD2.1-base at its full latent size (96 x 96, the page's [1, 4, 96, 96]),
    a classifier-free-guidance pair (B = 2)."""
    cfg = synth.UNET_CONFIGS["sd21"]
    inp = synth.make_unet_inputs(cfg, 21, 2, 96, 96, t=(999.0, 999.0))
    _say("[gpu] unet sd21 full size B=2 96x96")
    y = run_unet(cfg, inp, 2, 96, 96)
    _say("    oracle ...")
    yo = ou.unet_forward(inp["x"], inp["t"], inp["ctx"], inp["params"], cfg, inp["add"])
    check(cfg, y, yo)
