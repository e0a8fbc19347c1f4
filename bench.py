"""Benchmark of the Spatial-Transformer block on one MI355X.

One step = one st_block_forward of the whole block (GroupNorm, proj_in, every
layer's self-attention, cross-attention and GEGLU feed-forward, proj_out) on
the SDXL Down1 workload: B=2, C=640, 64x64 latent (4096 tokens per sample),
10 heads of 64, context [2, 77, 2048], depth 2, bf16 storage, seeded
random-init weights (N(0, 0.02^2)) and N(0, 1) inputs already resident in HBM.

Prints one JSON line: block tokens/s as `value` (wall clock over the timed
steps), the median and minimum of the same forwards each bracketed by its
own pair of HIP events, the self-attention kernel's achieved TFLOP/s against
the bf16 MFMA peak as `roofline` (its duration from HIP events recorded by
the library around each self-attention launch, on the stream it runs on,
during the timed region: mean, median and minimum per launch), the same rate
against a measured MFMA-loop ceiling with the shader clock observed during
that loop, and the fp64 CPU oracle timed on the host as `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import platform
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "spatial-transformer block tokens/s + attention TFLOP/s (% bf16 MFMA peak)"
ATTN_SRC = os.path.join(ROOT, "latent_diffusion_net_amd", "csrc", "k_attn.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "self_attn_sdxl_down1_hbm_traffic.md")
COPY_BYTES = 256 << 20      # calibration copy: 256 MiB read + 256 MiB written
SELF_ATTN_KERNEL = "attn_bf16_kernel<0,"   # kernel-name prefix of self-attention
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E
DEFAULT_WORKLOAD = 3       # index into synth.CONFIGS: SDXL Down1, 64x64, depth 2


def attention_flops(cfg) -> float:
    """QK^T and PV of one self-attention launch: 4 * B * heads * N^2 * 64."""
    return 4.0 * cfg.B * cfg.heads * float(cfg.N) ** 2 * 64


def block_flops(cfg) -> float:
    """All GEMM and attention FLOPs of one forward (2 per multiply-add)."""
    T, C, D, depth, B, N = cfg.T, cfg.C, cfg.D_ctx, cfg.depth, cfg.B, cfg.N
    per_layer = 36.0 * T * C * C + attention_flops(cfg) + 4.0 * B * N * 77 * C \
        + 4.0 * B * 77 * D * C
    return 4.0 * T * C * C + depth * per_layer


# Algorithmic work per launch of each timed kernel kind, and the roofline
# that bounds it: (row(s) of the method, bound, work per launch).  Flops count
# 2 per multiply-add; bytes count what the step must read and write at least
# once (bf16 storage).  proj_in's time also holds the GroupNorm apply.  On
# the bf16 path the LayerNorms have no launch of their own (statistics in the
# epilogues of the GEMMs that write h, normalisation folded into Q/K/V,
# cross Q and FF1), so their row is absent and their cost sits in those rows;
# likewise the cross-attention when it runs in the cross Q epilogue (its
# time is in A8, whose rate is still computed on the projection's flops).
def fused_cross(cfg) -> bool:
    """The cross-attention runs in the epilogue of its Q projection."""
    return getattr(cfg, "dtype", "bf16") == "bf16" and cfg.N % 64 == 0


def row_work(cfg):
    T, C, B, N, D, F, h = cfg.T, cfg.C, cfg.B, cfg.N, cfg.D_ctx, cfg.F, cfg.heads
    return {
        "gn_stats": ("A1 GroupNorm statistics", "hbm", 2.0 * T * C),
        "proj_in": ("A2 GroupNorm apply + proj_in", "mfma", 2.0 * T * C * C),
        "layernorm": ("A3/A7/A12 LayerNorm", "hbm", T * C * (4.0 + 2.0)),
        "qkv": ("A4 Q/K/V projection", "mfma", 6.0 * T * C * C),
        "self_attn": ("A5 self-attention", "mfma", attention_flops(cfg)),
        "attn_out": ("A6/A11 out-projections + residual", "mfma", 2.0 * T * C * C),
        # with the cross-attention in its epilogue (bf16, H*W % 64 == 0) the
        # launch also does the 77-key attention: QK^T and PV flops counted
        "cross_q": ("A8 cross-attention Q", "mfma",
                    2.0 * T * C * C + (4.0 * B * N * 77 * C if fused_cross(cfg) else 0.0)),
        # B*77 rows: 154 flop/B at most, below the ridge (about 312 flop/B at
        # 2.5 PFLOP/s and 8 TB/s): rated on its bytes -- the weights of all
        # layers, the context and the K/V it writes, each moved once
        "ctx_kv": ("A9 context K/V (all layers)", "hbm",
                   2.0 * (2 * C * cfg.depth * D + B * 77 * D + 2 * B * 77 * C * cfg.depth)),
        "cross_attn": ("A10 cross-attention", "hbm", 2.0 * T * C * 2 + 2.0 * B * h * 77 * 64 * 2),
        "ff1_geglu": ("A13 FF1 + GEGLU", "mfma", 16.0 * T * C * C),
        "ff2": ("A14 FF2 + residual", "mfma", 8.0 * T * C * C),
        "proj_out": ("A15 proj_out + NCHW + residual", "mfma", 2.0 * T * C * C),
    }


def copy_ceiling_gbs(torch, dev):
    """Device-to-device copy rate of a 256 MiB buffer (read + write bytes)."""
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    del src, dst
    return 2.0 * COPY_BYTES / (ms * 1e-3) / 1e9


LAYERNORM_FOLDED = ("no launch of its own: per-row sums in the epilogues of the GEMMs that "
                    "write h, normalisation folded into Q/K/V, cross-attention Q and FF1")


CROSS_ATTN_FUSED = ("no launch of its own: computed in the epilogue of the cross-attention Q "
                    "projection (row A8, whose time includes it) when H*W is a multiple of 64")


def row_rates(cfg, timing, copy_gbs):
    rows = {}
    if getattr(cfg, "dtype", "bf16") == "bf16" and not (timing.get("layernorm") or {}).get("launches"):
        rows["A3/A7/A12 LayerNorm"] = {"fused": LAYERNORM_FOLDED}
    if getattr(cfg, "dtype", "bf16") == "bf16" and not (timing.get("cross_attn") or {}).get("launches"):
        rows["A10 cross-attention"] = {"fused": CROSS_ATTN_FUSED}
    for kind, (name, bound, work) in row_work(cfg).items():
        t = timing.get(kind)
        if not t or not t["launches"]:
            continue
        s = t["ms"] / 1e3 / t["launches"]
        if bound == "hbm":
            a = work / s / 1e9
            rows[name] = {"bound": "hbm", "achieved": round(a, 1), "unit": "GB/s",
                          "peak": HBM_PEAK_GBS, "frac": round(a / HBM_PEAK_GBS, 3),
                          "frac_of_copy": round(a / copy_gbs, 3), "us_per_launch": round(s * 1e6, 2)}
        else:
            a = work / s / 1e12
            rows[name] = {"bound": "mfma", "achieved": round(a, 1), "unit": "TFLOP/s",
                          "peak": BF16_PEAK_TFLOPS, "frac": round(a / BF16_PEAK_TFLOPS, 3),
                          "us_per_launch": round(s * 1e6, 2)}
    return rows


def source_hash() -> str:
    with open(ATTN_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per self-attention launch from the committed counter summary,
    or None when that summary was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    txt = open(TRAFFIC_FILE).read()
    h = re.search(r"kernel source sha256\[:16\]: ([0-9a-f]{16})", txt)
    b = re.search(r"traffic_bytes_per_launch: ([0-9.eE+]+)", txt)
    if not h or not b or h.group(1) != source_hash():
        return None
    return float(b.group(1))


def summarize_pmc(fetch_csv, write_csv):
    """Counter CSVs of two rocprofv3 --pmc passes over `bench.py --pmc-pass`
    -> per-launch HBM bytes of self-attention, scaled by the copy kernel."""
    def vals(path, counter, pred):
        return [float(r["Counter_Value"]) for r in csv.DictReader(open(path))
                if r["Counter_Name"] == counter and pred(r["Kernel_Name"])]

    def avg(v):
        return (sum(v) / len(v), len(v)) if v else (float("nan"), 0)
    is_attn = lambda k: SELF_ATTN_KERNEL in k
    # the calibration copy is by far the largest copyBuffer dispatch (the
    # others copy weights while the block is created)
    is_copy = lambda k: "copyBuffer" in k
    fa, na = avg(vals(fetch_csv, "FETCH_SIZE", is_attn))
    fc, nc = max(vals(fetch_csv, "FETCH_SIZE", is_copy) or [float("nan")]), 1
    wa, _ = avg(vals(write_csv, "WRITE_SIZE", is_attn))
    wc = max(vals(write_csv, "WRITE_SIZE", is_copy) or [float("nan")])
    kf = COPY_BYTES / (fc * 1024.0)  # counters are in KiB
    kw = COPY_BYTES / (wc * 1024.0)
    fetch_b = fa * 1024.0 * kf
    write_b = wa * 1024.0 * kw
    return {"attn_fetch_kib": fa, "attn_write_kib": wa, "copy_fetch_kib": fc,
            "copy_write_kib": wc, "fetch_scale": kf, "write_scale": kw,
            "attn_launches": na, "copy_launches": nc,
            "traffic_bytes_per_launch": fetch_b + write_b,
            "fetch_bytes": fetch_b, "write_bytes": write_b}


def summarize_pmc_kernels(fetch_csv, write_csv, tcc_csv=None):
    """Per kernel name: dispatches, mean FETCH_SIZE / WRITE_SIZE bytes per
    dispatch scaled by the calibration copy, and (third CSV, a TCC_HIT_sum /
    TCC_MISS_sum pass) the L2 hit rate."""
    def rows(path):
        return list(csv.DictReader(open(path)))

    def per_kernel(path, counter):
        acc = {}
        for r in rows(path):
            if r["Counter_Name"] == counter:
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc
    fetch = per_kernel(fetch_csv, "FETCH_SIZE")
    write = per_kernel(write_csv, "WRITE_SIZE")
    fc = max((max(v) for k, v in fetch.items() if "copyBuffer" in k), default=float("nan"))
    wc = max((max(v) for k, v in write.items() if "copyBuffer" in k), default=float("nan"))
    kf, kw = COPY_BYTES / (fc * 1024.0), COPY_BYTES / (wc * 1024.0)
    hit = per_kernel(tcc_csv, "TCC_HIT_sum") if tcc_csv else {}
    miss = per_kernel(tcc_csv, "TCC_MISS_sum") if tcc_csv else {}
    out = {"fetch_scale": kf, "write_scale": kw, "kernels": {}}
    for k, v in fetch.items():
        if "copyBuffer" in k:
            continue
        w = write.get(k, [])
        e = {"dispatches": len(v),
             "fetch_mb": sum(v) / len(v) * 1024.0 * kf / 1e6,
             "write_mb": (sum(w) / len(w) * 1024.0 * kw / 1e6) if w else None}
        if k in hit and k in miss:
            h, m = sum(hit[k]), sum(miss[k])
            e["l2_hit_rate"] = h / (h + m) if h + m > 0 else None
        out["kernels"][k] = e
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(cfg, inp):
    """The fp64 oracle as it stands: one full forward of the same workload."""
    import oracle.block as ob
    threads, blas = None, "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = [p for p in threadpool_info() if p.get("user_api") == "blas"] or threadpool_info()
        threads = max((p.get("num_threads") or 0) for p in info) or None
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '?')}"
    except Exception:
        pass
    t0 = time.perf_counter()
    ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    dt = time.perf_counter() - t0
    return {"value": cfg.T / dt, "unit": "tokens/s",
            "cores": threads or os.cpu_count(), "kind": "oracle",
            "cpu": cpu_model(), "blas": blas,
            "fp64_gflops": round(block_flops(cfg) / dt / 1e9, 2),
            "sample": f"one full fp64 forward of the same workload ({cfg.T} tokens), {dt:.1f} s"}


def _event_times(torch, fn, reps, stream):
    """Per-call milliseconds of ``fn`` (one HIP event pair each, on ``stream``)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def _rate(ms_list, work, unit, peak):
    med = statistics.median(ms_list)
    a = work / (med * 1e-3) / (1e12 if unit == "TFLOP/s" else 1e9)
    return {"us_median": round(med * 1e3, 2), "us_min": round(min(ms_list) * 1e3, 2),
            "achieved": round(a, 1), "unit": unit, "peak": peak, "frac": round(a / peak, 3)}


def resnet_flops(cfg) -> float:
    """Both 3x3 convolutions (and a 1x1 shortcut) of one ResnetBlock2D."""
    n = cfg.B * cfg.H * cfg.W
    f = 2.0 * n * cfg.Cout * 9 * cfg.Cin + 2.0 * n * cfg.Cout * 9 * cfg.Cout
    if cfg.Cin != cfg.Cout:
        f += 2.0 * n * cfg.Cout * cfg.Cin
    return f


def unet_flops(ucfg, B, H, W) -> float:
    """Every convolution, ResnetBlock2D and transformer block of one U-Net
    timestep (2 flops per multiply-add; the embedding MLPs left out)."""
    from latent_diffusion_net_amd import synth
    conv = lambda ci, co, h, w: 2.0 * B * h * w * co * 9 * ci
    res = lambda ci, co, h, w: resnet_flops(synth.ResnetConfig("r", B, ci, co, h, w))
    blk = lambda c, h, w, d: block_flops(synth.BlockConfig("b", B, c, h, w, c // 64, ucfg.ctx_dim, d, "bf16"))
    L = len(ucfg.channels)
    f = conv(ucfg.in_channels, ucfg.channels[0], H, W) + conv(ucfg.channels[0], ucfg.out_channels, H, W)
    skips = synth.unet_skip_channels(ucfg)
    ch, h, w = ucfg.channels[0], H, W
    for l, c in enumerate(ucfg.channels):
        for _ in range(ucfg.layers_per_block):
            f += res(ch, c, h, w) + (blk(c, h, w, ucfg.depths[l]) if ucfg.depths[l] else 0.0)
            ch = c
        if l < L - 1:
            f += conv(c, c, h // 2, w // 2)
            h, w = h // 2, w // 2
    f += 2 * res(ch, ch, h, w) + (blk(ch, h, w, ucfg.mid_depth) if ucfg.mid_depth else 0.0)
    for l in reversed(range(L)):
        c = ucfg.channels[l]
        for _ in range(ucfg.layers_per_block + 1):
            f += res(ch + skips.pop(), c, h, w) + (blk(c, h, w, ucfg.depths[l]) if ucfg.depths[l] else 0.0)
            ch = c
        if l > 0:
            h, w = 2 * h, 2 * w
            f += conv(c, c, h, w)
    return f


def unet_params_on_device(torch, ucfg, seed, dev):
    """Random-init U-Net weights drawn on the GPU (N(0, 0.02^2) weights, zero
    biases, unit norm gammas): for timing only, nothing is compared."""
    from latent_diffusion_net_amd import synth
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    norm_w = ("gn1_w", "gn2_w", "gn_w", "norm_out_w", "ln1_w", "ln2_w", "ln3_w")

    def draw(path, shape):
        n = path[-1]
        if n in norm_w:
            return torch.ones(shape, dtype=torch.bfloat16, device=dev)
        if n.endswith("_w"):
            return (torch.randn(shape, generator=g, device=dev) * 0.02).to(torch.bfloat16)
        return torch.zeros(shape, dtype=torch.bfloat16, device=dev)
    return synth._walk(synth.unet_param_shapes(ucfg), draw)


# The pages' run evidence: peak CUDA memory allocated for one denoiser
# timestep at batch 1 (section 5 of each architecture page).
PAGE_PEAK_GIB = {"sd21": 1.78, "sdxl_inpaint": 5.17}
PAGE_LATENT = {"sd21": 96, "sdxl_inpaint": 128}


def unet_row(torch, key, B, stream, reps=5):
    from latent_diffusion_net_amd import STUNet, synth
    dev = "cuda:0"
    ucfg = synth.UNET_CONFIGS[key]
    S = PAGE_LATENT[key]
    p = unet_params_on_device(torch, ucfg, 7, dev)
    weight_bytes = 2 * synth.unet_param_count(ucfg)
    u = STUNet(ucfg, B, S, S, p)
    del p
    torch.cuda.empty_cache()
    x = torch.randn(B, ucfg.in_channels, S, S, device=dev).to(torch.bfloat16)
    ctx = torch.randn(B, 77, ucfg.ctx_dim, device=dev).to(torch.bfloat16)
    add = torch.randn(B, ucfg.add_in, device=dev).to(torch.bfloat16) if ucfg.add_in else None
    t = torch.full((B,), 999.0, device=dev)
    y = torch.empty(B, ucfg.out_channels, S, S, device=dev, dtype=torch.bfloat16)
    for _ in range(2):
        u.forward(x, t, ctx, add, y, stream)
    ms = _event_times(torch, lambda: u.forward(x, t, ctx, add, y, stream), reps, stream)
    held = u.device_bytes()
    u.close()
    fl = unet_flops(ucfg, B, S, S)
    r = _rate(ms, fl, "TFLOP/s", BF16_PEAK_TFLOPS)
    r.update({"flops": fl, "bound": "mfma (convolutions, attention and GEMMs of every part)",
              "device_gib_held": round(held / 2**30, 2),
              "weights_gib_bf16": round(weight_bytes / 2**30, 2)})
    if B == 1:
        r["page_peak_allocated_gib_batch1"] = PAGE_PEAK_GIB[key]
    return r


def resnet_row(torch, stream, reps=20):
    """ResnetBlock2D at the SDXL Down1 stage (640 channels, 64 x 64, B = 2)."""
    from latent_diffusion_net_amd import STResnet, synth
    dev = "cuda:0"
    rc = synth.ResnetConfig("sdxl_down1_640_64x64", 2, 640, 640, 64, 64)
    ri = synth.make_resnet_inputs(rc, 1)
    bf = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16).contiguous()
    rp = {k: bf(v) for k, v in ri["params"].items()}
    rx, rt = bf(ri["x"]), bf(ri["temb"])
    ry = torch.empty_like(rx)
    res = STResnet(rc.B, rc.Cin, rc.Cout, rc.H, rc.W, rc.Dt, rp)
    for _ in range(3):
        res.forward(rx, rt, ry, stream)
    ms = _event_times(torch, lambda: res.forward(rx, rt, ry, stream), reps, stream)
    res.close()
    return dict(_rate(ms, resnet_flops(rc), "TFLOP/s", BF16_PEAK_TFLOPS), flops=resnet_flops(rc),
                bound="mfma (the two 3x3 convolutions; GroupNorm passes and the time embedding inside)")


def next_rows(torch, cfg_block, blk_inputs, stream, reps=20):
    """Measured rates of the parts built around the block: a ResnetBlock2D at
    the bench stage, the GroupNorm(+SiLU) op, the guided DDPM step and the
    block forward with a context key padding mask."""
    from latent_diffusion_net_amd import synth
    from latent_diffusion_net_amd.binding import group_norm, guided_ddpm_step
    out = {}
    dev = "cuda:0"
    out["F1 ResnetBlock2D (SDXL Down1, 640 ch, 64x64, B=2)"] = resnet_row(torch, stream, reps)
    bf = lambda a: torch.from_numpy(a).to(dev).to(torch.bfloat16).contiguous()
    rx = bf(synth.make_resnet_inputs(synth.ResnetConfig("gn", 2, 640, 640, 64, 64), 1)["x"])
    # GroupNorm + SiLU op on the same map: read once, write once at least
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    gy = torch.empty_like(rx)
    group_norm(rx, None, None, 1e-5, True, gy, ws, stream)
    ms = _event_times(torch, lambda: group_norm(rx, None, None, 1e-5, True, gy, ws, stream), reps, stream)
    out["GroupNorm + SiLU op (2 x 640 x 64 x 64 bf16)"] = dict(
        _rate(ms, 2.0 * rx.numel() * 2, "GB/s", HBM_PEAK_GBS), bytes=2.0 * rx.numel() * 2,
        bound="hbm (algorithmic: x read once, y written once; the kernels read x twice)")
    # guided DDPM step on an SDXL latent (4 x 128 x 128)
    n = 4 * 128 * 128
    eps = torch.randn(2, n, device=dev).to(torch.bfloat16)
    xt = torch.randn(n, device=dev)
    z = torch.randn(n, device=dev)
    xp = torch.empty_like(xt)
    guided_ddpm_step(eps, xt, 500, 7.5, z, xp, stream=stream)
    ms = _event_times(torch, lambda: guided_ddpm_step(eps, xt, 500, 7.5, z, xp, stream=stream), reps, stream)
    out["F4 guidance + DDPM step (4 x 128 x 128 latent)"] = dict(
        _rate(ms, 2.0 * 2 * n + 4.0 * 3 * n, "GB/s", HBM_PEAK_GBS), bytes=2.0 * 2 * n + 4.0 * 3 * n,
        bound="hbm (a 1 MB step: launch latency dominates)")
    # block forward with a padded context mask (the first 20 tokens real)
    blk, x, ctx, y = blk_inputs
    m = torch.zeros((cfg_block.B, 77), dtype=torch.uint8, device=dev)
    m[:, :20] = 1
    blk.forward_masked(x, ctx, m, y, stream)
    ms = _event_times(torch, lambda: blk.forward_masked(x, ctx, m, y, stream), reps, stream)
    ms0 = _event_times(torch, lambda: blk.forward(x, ctx, y, stream), reps, stream)
    out["F2 U-Net timestep, SD2.1-base (96x96 latent, B=2 guidance pair)"] = unet_row(torch, "sd21", 2, stream)
    out["F2 U-Net timestep, SD2.1-base (96x96 latent, B=1)"] = unet_row(torch, "sd21", 1, stream)
    out["F2 U-Net timestep, SDXL-Inpaint (128x128 latent, B=1)"] = unet_row(torch, "sdxl_inpaint", 1, stream)
    out["F3 block forward with a context key mask (bench workload)"] = {
        "us_median": round(statistics.median(ms) * 1e3, 2),
        "us_median_unmasked_same_run": round(statistics.median(ms0) * 1e3, 2),
        "tokens_per_s": cfg_block.T / (statistics.median(ms) * 1e-3)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=DEFAULT_WORKLOAD,
                    help="workload index (default: the SDXL Down1 block)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--part", choices=["resnet", "unet_sd21", "unet_sd21_b1", "unet_sdxl"],
                    help="time only this part (for kernel traces) and print its row")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the ResnetBlock2D / GroupNorm / DDPM / masked-forward measurements")
    ap.add_argument("--kernels", action="store_true",
                    help="also print the per-step microseconds of every kernel kind")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="counter-collection run: a 256 MiB device copy (the "
                         "calibration kernel) then a few forwards; no JSON")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the self-attention HBM traffic from two "
                         "counter CSVs of --pmc-pass runs")
    ap.add_argument("--summarize-pmc-kernels", nargs="+", metavar="CSV",
                    help="per-kernel HBM bytes (and L2 hit rate) from the FETCH_SIZE "
                         "and WRITE_SIZE (and TCC_HIT_sum/TCC_MISS_sum) CSVs of "
                         "--pmc-pass runs")
    args = ap.parse_args()
    if args.summarize_pmc_kernels:
        if len(args.summarize_pmc_kernels) not in (2, 3):
            ap.error("--summarize-pmc-kernels takes FETCH_CSV WRITE_CSV [TCC_CSV]")
        print(json.dumps(summarize_pmc_kernels(*args.summarize_pmc_kernels), indent=1))
        return
    if args.summarize_pmc:
        r = summarize_pmc(*args.summarize_pmc)
        r["kernel_source_sha256_16"] = source_hash()
        print(json.dumps(r, indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the block runs on one GPU and is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)

    import torch
    from latent_diffusion_net_amd import (STBlock, array_to_device,
                                          params_to_device, synth)
    if args.part:
        stream = torch.cuda.current_stream()
        if args.part == "resnet":
            row = resnet_row(torch, stream)
        else:
            key, B = {"unet_sd21": ("sd21", 2), "unet_sd21_b1": ("sd21", 1),
                      "unet_sdxl": ("sdxl_inpaint", 1)}[args.part]
            row = unet_row(torch, key, B, stream)
        print(json.dumps({"part": args.part, **row}), flush=True)
        return

    cfg = synth.CONFIGS[args.config]
    inp = synth.make_inputs(cfg, synth.config_seed(args.config))
    dev = "cuda:0"
    p = params_to_device(inp["params"], cfg.dtype, dev)
    x = array_to_device(inp["x"], cfg.dtype, dev)
    ctx = array_to_device(inp["ctx"], cfg.dtype, dev)
    y = torch.empty_like(x)
    blk = STBlock(cfg.B, cfg.C, cfg.H, cfg.W, cfg.heads, cfg.D_ctx, cfg.depth,
                  cfg.dtype, p)
    del p
    stream = torch.cuda.current_stream()

    for _ in range(args.warmup):
        blk.forward(x, ctx, y, stream)
    torch.cuda.synchronize()
    if args.pmc_pass:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        for _ in range(3):
            blk.forward(x, ctx, y, stream)
        torch.cuda.synchronize()
        blk.close()
        print("pmc pass done", flush=True)
        return
    blk.read_timing()
    # Live self-attention timing inside the timed forwards: an event pair
    # around the first layer's launch (kernel + merge) of every forward.
    # Each pair leaves a bubble of ~5 us between two kernels, so the other
    # layers' launches (the same kernel at the same shape) go untimed.
    blk.set_timing(["self_attn"], layers=1)
    # one event pair around each forward, on the stream the forward runs on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        blk.forward(x, ctx, y, stream)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    launches = blk.read_timing_launches()
    blk.set_timing([])

    fwd_ms = [a.elapsed_time(b) for a, b in ev]
    ms_per_step = dt * 1e3 / args.steps
    tokens_per_s = cfg.T / (dt / args.steps)
    attn_ms = [ms for k, ms in launches if k == "self_attn"] or [float("nan")]
    attn_s = statistics.fmean(attn_ms) / 1e3
    attn_tflops = attention_flops(cfg) / attn_s / 1e12

    # Every kernel kind against its roofline, from a few more forwards after
    # the timed region (events around every launch perturb the block rate,
    # so they stay out of it).
    from latent_diffusion_net_amd.binding import KERNEL_KINDS
    blk.set_timing(KERNEL_KINDS)
    for _ in range(5):
        blk.forward(x, ctx, y, stream)
    torch.cuda.synchronize()
    kt = blk.read_timing()
    blk.set_timing([])
    kernels = {k: round(v["ms"] / 5 * 1e3, 2) for k, v in kt.items()} if args.kernels else None
    nxt = None if args.no_next_rows else next_rows(torch, cfg, (blk, x, ctx, y), stream)
    blk.close()
    copy_gbs = copy_ceiling_gbs(torch, dev)
    rows = row_rates(cfg, kt, copy_gbs)
    from latent_diffusion_net_amd.binding import measure_mfma_bf16
    mfma_tflops, sclk = measure_mfma_bf16(stream=stream)
    attn_med_s = statistics.median(attn_ms) / 1e3
    attn_min_s = min(attn_ms) / 1e3

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded random-init weights N(0,0.02^2), x and ctx N(0,1))",
        "config": {"workload": cfg.name, "B": cfg.B, "C": cfg.C, "H": cfg.H,
                   "W": cfg.W, "heads": cfg.heads, "D_ctx": cfg.D_ctx,
                   "depth": cfg.depth, "tokens_per_step": cfg.T},
        "roofline": {"bound": "mfma", "achieved": attn_tflops,
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": attn_tflops / BF16_PEAK_TFLOPS,
                     "traffic": measured_traffic(),
                     "kernel": "attn_bf16_kernel (self-attention)",
                     "us_per_launch": attn_s * 1e6,
                     "us_per_launch_median": attn_med_s * 1e6,
                     "us_per_launch_min": attn_min_s * 1e6,
                     "launches_timed": len(attn_ms),
                     "achieved_median": attention_flops(cfg) / attn_med_s / 1e12,
                     "flops_per_launch": attention_flops(cfg),
                     "measured_mfma_ceiling_tflops": round(mfma_tflops, 1),
                     "frac_of_measured_ceiling": attn_tflops / mfma_tflops,
                     "sclk_mhz_during_ceiling": round(sclk, 1)},
        "forward_ms": {"median": statistics.median(fwd_ms), "min": min(fwd_ms),
                       "mean": statistics.fmean(fwd_ms), "timed_by": "HIP events, one pair per forward"},
        "tokens_per_s_median_forward": cfg.T / (statistics.median(fwd_ms) * 1e-3),
        "block_tflops": block_flops(cfg) / (dt / args.steps) / 1e12,
        "copy_ceiling_gbs": round(copy_gbs, 1),
        "rows": rows,
    }
    if kernels is not None:
        result["kernel_us_per_step"] = kernels
    if nxt is not None:
        result["next_rows"] = nxt
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
