"""ResnetBlock2D on the GPU (st_resnet_*) against the fp64 oracle
(oracle.unet.resnet_block), every output element, through the C ABI.

Tolerance: bf16 storage (x, temb, weights, y, the intermediate h) with fp16
convolution operands and fp32 accumulation -- the block's bf16 gate,
max-abs <= 3e-2 and rel-L2 <= 1e-2 on y; and on the residual branch
Delta = y - shortcut(x) (shortcut computed by the oracle) the bound
derived from the roundings: ||Delta_gpu - Delta_oracle|| <= u (||y|| +
5 ||Delta||), u = 2^-8 (y's own bf16 rounding plus a few roundings of the
branch).
"""
import numpy as np
import pytest

import oracle.unet as ou
from latent_diffusion_net_amd import synth

pytestmark = pytest.mark.gpu
U = 2.0 ** -8


def _say(msg):
    print(msg, flush=True)


def run_resnet(cfg, inp, eps=1e-5):
    import torch
    from latent_diffusion_net_amd import STResnet
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(torch.bfloat16)
    p = {k: dev(v) for k, v in inp["params"].items()}
    x, temb = dev(inp["x"]), dev(inp["temb"])
    r = STResnet(cfg.B, cfg.Cin, cfg.Cout, cfg.H, cfg.W, cfg.Dt, p, eps=eps)
    y = r.forward(x, temb)
    y2 = r.forward(x, temb)
    r.check_range()
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    r.close()
    return y.float().cpu().numpy().astype(np.float64)


def check(cfg, inp, y, eps=1e-5):
    yo = ou.resnet_block(inp["x"], inp["temb"], inp["params"], eps=eps)
    x = np.asarray(inp["x"], np.float64)
    p = inp["params"]
    sc = x if cfg.Cin == cfg.Cout else ou.conv2d(x, np.asarray(p["sc_w"], np.float64)[:, :, None, None],
                                                  p.get("sc_b"), padding=0)
    err = float(np.abs(y - yo).max())
    rel = float(np.linalg.norm(y - yo) / np.linalg.norm(yo))
    rd = float(np.linalg.norm((y - sc) - (yo - sc)) / np.linalg.norm(yo - sc))
    bound = U * (np.linalg.norm(yo) / np.linalg.norm(yo - sc) + 5.0)
    _say(f"    max_abs={err:.3e} rel_l2={rel:.3e} branch_rel_l2={rd:.3e} (bound {bound:.3e})")
    assert np.isfinite(y).all()
    assert err <= 3e-2 and rel <= 1e-2
    assert rd <= bound


CASES = [
    # SDXL Down1: the first ResNet (320 -> 640, 1x1 shortcut as a tenth tap) and the second
    (synth.ResnetConfig("sdxl_down1_320to640_64x64", 2, 320, 640, 64, 64), {}),
    (synth.ResnetConfig("sdxl_down1_640_64x64", 2, 640, 640, 64, 64), {}),
    # SD2.1 Down0 (96 x 96 latent stage, 320 channels)
    (synth.ResnetConfig("sd21_down0_320_96x96", 2, 320, 320, 96, 96), {}),
    # SDXL Up1's first ResNet: skip concatenated (1280 + 640 -> 640)
    (synth.ResnetConfig("sdxl_up1_1920to640_64x64", 2, 1920, 640, 64, 64), {}),
    # SD2.1's 12 x 12 level at B = 1: 20 output tiles, the convolutions split
    # over K (10 and 11 slices; the second product's slices reach into the
    # 1x1-shortcut segment, 2560 -> 1280 channels)
    (synth.ResnetConfig("sd21_up0_1280_12x12_b1", 1, 1280, 1280, 12, 12), {}),
    (synth.ResnetConfig("sd21_up0_2560to1280_12x12_b1", 1, 2560, 1280, 12, 12), {}),
    # small and ragged: every bias, gamma and beta drawn; 5 rows, 8 columns
    (synth.ResnetConfig("b1_64to128_5x8", 1, 64, 128, 5, 8, Dt=32),
     dict(bias_std=0.1, norm_std=0.2, weight_std=0.05)),
    (synth.ResnetConfig("b3_128_7x4", 3, 128, 128, 7, 4, Dt=64),
     dict(bias_std=0.1, norm_std=0.2, weight_std=0.05)),
]


@pytest.mark.parametrize("cfg,kw", CASES, ids=[c[0].name for c in CASES])
def test_resnet_block(cfg, kw):
    inp = synth.make_resnet_inputs(cfg, 500 + cfg.Cin + cfg.H, **kw)
    _say(f"[gpu] resnet {cfg}")
    y = run_resnet(cfg, inp)
    check(cfg, inp, y)
