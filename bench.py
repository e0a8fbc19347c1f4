"""Benchmark of the Spatial-Transformer block on one MI355X.

One step = one st_block_forward of the whole block (GroupNorm, proj_in, every
layer's self-attention, cross-attention and GEGLU feed-forward, proj_out) on
the SDXL Down1 workload: B=2, C=640, 64x64 latent (4096 tokens per sample),
10 heads of 64, context [2, 77, 2048], depth 2, bf16 storage, seeded
random-init weights (N(0, 0.02^2)) and N(0, 1) inputs already resident in HBM.

Prints one JSON line: block tokens/s as `value`, the self-attention kernel's
achieved TFLOP/s against the bf16 MFMA peak as `roofline` (its duration from
HIP events recorded by the library around each self-attention launch, on the
stream it runs on, during the timed region), and the fp64 CPU oracle timed on
the host as `cpu_baseline`.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
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
def row_work(cfg):
    T, C, B, N, D, F, h = cfg.T, cfg.C, cfg.B, cfg.N, cfg.D_ctx, cfg.F, cfg.heads
    return {
        "gn_stats": ("A1 GroupNorm statistics", "hbm", 2.0 * T * C),
        "proj_in": ("A2 GroupNorm apply + proj_in", "mfma", 2.0 * T * C * C),
        "layernorm": ("A3/A7/A12 LayerNorm", "hbm", T * C * (4.0 + 2.0)),
        "qkv": ("A4 Q/K/V projection", "mfma", 6.0 * T * C * C),
        "self_attn": ("A5 self-attention", "mfma", attention_flops(cfg)),
        "attn_out": ("A6/A11 out-projections + residual", "mfma", 2.0 * T * C * C),
        "cross_q": ("A8 cross-attention Q", "mfma", 2.0 * T * C * C),
        "ctx_kv": ("A9 context K/V (all layers)", "mfma", 2.0 * B * 77 * 2 * C * cfg.depth * D),
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


def cpu_baseline(cfg, inp):
    """The fp64 oracle as it stands: one full forward of the same workload."""
    import oracle.block as ob
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((p.get("num_threads") or 0) for p in threadpool_info()) or None
    except Exception:
        pass
    t0 = time.perf_counter()
    ob.block_forward(inp["x"], inp["ctx"], inp["params"], cfg.heads)
    dt = time.perf_counter() - t0
    return {"value": cfg.T / dt, "unit": "tokens/s",
            "cores": threads or os.cpu_count(), "kind": "oracle",
            "sample": f"one full fp64 forward of the same workload ({cfg.T} tokens), {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=DEFAULT_WORKLOAD,
                    help="workload index (default: the SDXL Down1 block)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernels", action="store_true",
                    help="also print the per-step microseconds of every kernel kind")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="counter-collection run: a 256 MiB device copy (the "
                         "calibration kernel) then a few forwards; no JSON")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the self-attention HBM traffic from two "
                         "counter CSVs of --pmc-pass runs")
    args = ap.parse_args()
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
    blk.set_timing(["self_attn"])

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        blk.forward(x, ctx, y, stream)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    timing = blk.read_timing()
    blk.set_timing([])

    ms_per_step = dt * 1e3 / args.steps
    tokens_per_s = cfg.T / (dt / args.steps)
    attn = timing.get("self_attn", {"ms": float("nan"), "launches": 1})
    attn_s = attn["ms"] / 1e3 / attn["launches"]
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
    blk.close()
    copy_gbs = copy_ceiling_gbs(torch, dev)
    rows = row_rates(cfg, kt, copy_gbs)

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
                     "flops_per_launch": attention_flops(cfg)},
        "block_tflops": block_flops(cfg) / (dt / args.steps) / 1e12,
        "copy_ceiling_gbs": round(copy_gbs, 1),
        "rows": rows,
    }
    if kernels is not None:
        result["kernel_us_per_step"] = kernels
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
