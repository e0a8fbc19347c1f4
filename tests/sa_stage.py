"""Self-attention sublayer checks with a non-flat softmax (shared by the GPU
parity tests and the CPU mutation checks of their bounds).

The shapes reach every variant of the bf16 self-attention that the
workloads run: the 128-query kernel at the full SDXL Down1 shape (B=2,
C=640, 64x64 tokens, 10 heads: 640 query tiles on 256 CUs, so whole tiles
plus tiles split over their keys into pieces and merged), the same kernel
with ragged queries and keys (63x63 = 3969 tokens: the last query tile has
one query, the last key tile one key), the key-split plans forced at a
small size by planning for fewer CUs (``cus``), and the overlapped kernel
that takes plans without a key split (the SD2.1 Down0 shape, 9216 tokens,
and the ragged shape planned so that nothing is split).  ``pins=False``
leaves a shape out of the CPU mutation checks (the oracle's cost there).

The query and key weights are drawn with std sqrt(3 / C), so the logits
have a standard deviation of about 3 (a softmax far from flat: at 4096 keys
the largest probability of a row is typically 0.05-0.2); every other weight
keeps the headline N(0, 0.02^2), the norms' gamma and beta are drawn
(N(1, 0.2^2), N(0, 0.2^2)) and the biases stay zero, so that the update is
the attention's output alone.  The checked quantity is the
sublayer's update, Delta = h(after self-attention) - h(after proj_in), per
element; the GPU's update is its own stage-1 stream minus its own stage-0
stream, the oracle's is l0_sa - h0.

Bounds (bf16 operands, fp32 accumulation and softmax): Q, K, V, P and O are
each rounded once to bf16 (unit roundoff u = 2^-8), the LayerNorm output and
the out-projection's result meet fp16 roundings; the update's relative
error is a few u, so
    rel-L2(Delta_gpu, Delta_oracle) <= 1e-2            (2.6 u)
    max |Delta_gpu - Delta_oracle| <= 3e-2 * max |Delta_oracle|
The CPU tests in test_sa_stage_pins.py show that plausible mistakes in the
attention (scores ignored, half of the keys dropped, pieces merged without
their weights, the 1/sqrt(d) scale missing) exceed these bounds many times.
"""
import math

import numpy as np

import oracle.block as ob
from latent_diffusion_net_amd import synth

UPDATE_REL_L2 = 1e-2
UPDATE_MAX_ABS_REL = 3e-2

SHAPES = [
    dict(name="sdxl_down1_b2_c640_64x64", B=2, C=640, H=64, W=64, D_ctx=2048, cus=None),
    dict(name="b2_c640_63x63_ragged", B=2, C=640, H=63, W=63, D_ctx=128, cus=None),
    dict(name="split2", B=1, C=64, H=64, W=64, D_ctx=64, cus=12),
    dict(name="split3_ragged", B=1, C=64, H=63, W=63, D_ctx=64, cus=31),
    dict(name="split2_all", B=1, C=64, H=64, W=64, D_ctx=64, cus=64),
    # whole query tiles only (no key split): the overlapped kernel, at the
    # SD2.1 Down0 shape (720 tiles on 512 persistent workgroups, so some take
    # two) and with ragged queries and keys (planned for 320 CUs: 640 tiles,
    # no remainder to split)
    dict(name="sd21_down0_b2_c320_96x96", B=2, C=320, H=96, W=96, D_ctx=1024, cus=None, pins=False),
    dict(name="b2_c640_63x63_ragged_whole", B=2, C=640, H=63, W=63, D_ctx=128, cus=320),
    # the overlapped kernel on few key tiles (many samples and heads, so
    # that the plan still has at least two query tiles per CU): four key
    # tiles (its loop's tail iterations only) and a single one; left out of
    # the CPU mutation checks, which need several key tiles to mean anything
    # (a single tile takes no lazy rescale)
    dict(name="b32_c1024_16x16_four_key_tiles", B=32, C=1024, H=16, W=16, D_ctx=64, cus=None, pins=False),
    dict(name="b32_c1024_8x8_one_key_tile", B=32, C=1024, H=8, W=8, D_ctx=64, cus=None, pins=False),
]


def config(spec):
    return synth.BlockConfig(spec["name"], spec["B"], spec["C"], spec["H"], spec["W"],
                             spec["C"] // 64, spec["D_ctx"], 1, "bf16")


def inputs(spec, seed=41):
    cfg = config(spec)
    return cfg, synth.make_inputs(cfg, seed, norm_std=0.2, qk_std=math.sqrt(3.0 / cfg.C))


def oracle_stage1(inp, heads, attention=None):
    """(h0, h after the first self-attention sublayer), fp64, [B, N, C].

    ``attention`` replaces the oracle's attention in the sublayer (the CPU
    mutation checks plant their mistakes this way)."""
    p = inp["params"]
    z = ob.group_norm(inp["x"], p["gn_w"], p["gn_b"])
    h0 = ob.linear(ob.to_tokens(z), p["proj_in_w"], p.get("proj_in_b"))
    if attention is None:
        h1 = ob.self_attention_sublayer(h0, p["layers"][0], heads)
    else:
        saved = ob.attention
        ob.attention = attention
        try:
            h1 = ob.self_attention_sublayer(h0, p["layers"][0], heads)
        finally:
            ob.attention = saved
    return h0, h1


def update_errors(d_test, d_ref):
    d_test = np.asarray(d_test, np.float64)
    d_ref = np.asarray(d_ref, np.float64)
    rel = float(np.linalg.norm(d_test - d_ref) / np.linalg.norm(d_ref))
    mx = float(np.abs(d_test - d_ref).max() / np.abs(d_ref).max())
    return rel, mx
