"""st_group_norm_noalloc (the allocation-free variant, partial sums in the
library's static device array) against st_group_norm (caller workspace),
through the C ABI: two calls in a row, the second with a smaller input,
bitwise equal outputs (same kernels, same order of every sum), and both
within the bf16 gate of the fp64 oracle."""
import numpy as np
import pytest

import oracle.block as ob
import oracle.unet as ou
from latent_diffusion_net_amd import synth

pytestmark = pytest.mark.gpu


def _inputs(B, C, H, W, seed):
    rng = np.random.default_rng(seed)
    x = synth.round_bf16((rng.standard_normal((B, C, H, W)) * 1.5 - 0.3).astype(np.float32))
    g = synth.round_bf16((1 + 0.2 * rng.standard_normal(C)).astype(np.float32))
    b = synth.round_bf16((0.2 * rng.standard_normal(C)).astype(np.float32))
    return x, g, b


def test_group_norm_noalloc_matches_workspace_entry_point():
    import torch
    from latent_diffusion_net_amd.binding import (ST_ERR_UNSUPPORTED, STError, group_norm,
                                                  group_norm_noalloc)
    dev = lambda a: torch.from_numpy(a).to("cuda").to(torch.bfloat16)
    # SDXL Down1 ResnetBlock2D norm, then a smaller ragged map
    for (B, C, H, W), seed in (((2, 640, 64, 64), 1), ((1, 64, 5, 7), 2)):
        print(f"[gpu] no-alloc GroupNorm B={B} C={C} {H}x{W}", flush=True)
        x, g, b = _inputs(B, C, H, W, seed)
        xd, gd, bd = dev(x), dev(g), dev(b)
        y_ws = group_norm(xd, gd, bd, eps=1e-5, silu=True)
        y_na = torch.full_like(xd, float("nan"))
        group_norm_noalloc(xd, y_na, gd, bd, eps=1e-5, silu=True)
        torch.cuda.synchronize()
        assert torch.equal(y_ws.view(torch.int16), y_na.view(torch.int16))
        ref = ou.silu(ob.group_norm(x, g, b, eps=1e-5))
        y = y_na.float().cpu().numpy().astype(np.float64)
        err = float(np.abs(y - ref).max())
        rel = float(np.linalg.norm(y - ref) / np.linalg.norm(ref))
        print(f"    max_abs={err:.3e} rel_l2={rel:.3e}", flush=True)
        assert err <= 3e-2 and rel <= 1e-2
    # beyond the static array: refused before anything is enqueued
    x = torch.zeros((65, 32, 1, 1), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(STError) as e:
        group_norm_noalloc(x, torch.empty_like(x))
    assert e.value.status == ST_ERR_UNSUPPORTED
