"""Benchmark: Switch FFN layer forward (route, dispatch, experts, combine, aux
loss) on one MI355X, with the fp64 oracle timed on the host beside it.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

Prints one JSON line.  A step is one switch_layer_fwd over the whole batch of
seeded synthetic inputs (already in HBM when timing starts).  The default
workload is the Switch-Base-shaped layer: T=16384 tokens, d=768, d_ff=3072,
E=128 experts, capacity factor 1.0 (C=128).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Switch FFN layer fwd tokens/s (E=128,d=768) + % bf16 MFMA peak + dispatch GB/s"
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--config", type=int, default=2, help="layer configuration 1..5 (2 = Switch-Base shape)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-variants", action="store_true",
                   help="skip the timing of the layer variants (z-loss, routing groups, top-2)")
    p.add_argument("--cpu-sample-tokens", type=int, default=0,
                   help="tokens in the oracle's timed sample (0 = the whole batch)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                   help="only run the plain copy kernel on BYTES bytes (hardware-counter calibration)")
    return p.parse_args()


def copy_calibration(nbytes: int, reps: int):
    """Runs the library's plain 16-byte-vector copy kernel `reps` times on
    `nbytes` bytes; its counter readings calibrate FETCH_SIZE / WRITE_SIZE."""
    import torch

    import sparse_mixture_experts_order_amd as sw
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sw.switch_stream_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        sw.switch_stream_copy(dst, src, nbytes)
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / reps
    print(json.dumps({"copy_bytes": nbytes, "reps": reps, "ms": ms, "GBps_read_plus_write": 2 * nbytes / ms / 1e6}))


def kernel_source_sha() -> str:
    src = os.path.join(ROOT, "sparse_mixture_experts_order_amd", "csrc", "expert_ffn.hip")
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` (FETCH_SIZE + WRITE_SIZE, each scaled by
    the same counter's reading on a plain copy of known size) from the committed
    counter summary, or None when the summary is missing or was taken on a
    different expert-kernel source."""
    path = os.path.join(PROFILES, f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != kernel_source_sha():
        return None
    f, w = vals.get(f"{kernel}_fetch_bytes_per_launch"), vals.get(f"{kernel}_write_bytes_per_launch")
    return float(f) + float(w) if f and w else None


def cpu_baseline(inp, cfg, sample_tokens):
    """The oracle, untuned, on the host cores: the whole layer (router,
    softmax/top-1, scan, dispatch, experts, combine, aux loss and gradient)
    on the first `sample_tokens` tokens of the batch."""
    from threadpoolctl import threadpool_info

    from oracle import switch_oracle as so
    n = sample_tokens or cfg.T
    x = inp.x[:n]
    dt = float("inf")
    for _ in range(3):      # best of three
        t0 = time.perf_counter()
        L = so.layer_forward(x, inp.w_r, inp.b_r, inp.w1, inp.w2, cfg.c, cfg.alpha)
        dt = min(dt, time.perf_counter() - t0)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    del L
    return n / dt, dt, threads, n


def time_variants(sw, torch, cfg, x, w_r, b_r, w1, w2, stream, steps, warmup):
    """The same layer with the rows beyond the Switch forward switched on: the
    router z-loss, routing groups of 64 tokens (capacity per group), and top-2
    choices in groups of 2048 tokens.  Each variant: warm-up, then `steps`
    timed steps between events on the launch stream."""
    out = {}
    variants = [
        ("z_loss", dict(k=1, group=0, z=True)),
        ("groups_of_64", dict(k=1, group=64, z=False)),
        ("top2_groups_of_2048", dict(k=2, group=2048, z=False)),
        ("top2_one_group", dict(k=2, group=0, z=False)),
    ]
    for name, v in variants:
        G = v["group"] or cfg.T
        if cfg.T % G:
            continue
        C = sw.switch_capacity(v["k"] * G, cfg.E, cfg.c)
        t = sw.layer_tensors(cfg.T, cfg.d, cfg.d_ff, cfg.E, C, dlogits=cfg.want_grad, z_loss=v["z"], k=v["k"],
                             group=v["group"])
        la = sw.make_layer_args(x, w_r, b_r, w1, w2, t, cfg.T, cfg.d, cfg.d_ff, cfg.E, C, cfg.alpha, residual=True,
                                z_beta=1e-3 if v["z"] else 0.0, k=v["k"], group=v["group"])
        for _ in range(warmup):
            sw.switch_layer_fwd(la, t["ws"], stream)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(steps):
            sw.switch_layer_fwd(la, t["ws"], stream)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        keep = t["keep"].cpu().numpy()
        out[name] = {"k": v["k"], "group": G, "C_per_group": C, "ms_per_step": ms,
                     "tokens_per_s": cfg.T / (ms / 1000.0), "kept_choices": float(keep.mean())}
        del t, la
    out["backward"] = time_backward(sw, torch, cfg, x, w_r, b_r, w1, w2, stream, steps, warmup)
    return out


def time_backward(sw, torch, cfg, x, w_r, b_r, w1, w2, stream, steps, warmup):
    """The layer backward (switch_layer_bwd) after a forward that keeps what it
    needs (logits, hidden activations, dispatch buffer, expert outputs); a
    step is one backward.  Per-kernel times from the library's events."""
    T, d, F, E = cfg.T, cfg.d, cfg.d_ff, cfg.E
    C = sw.switch_capacity(T, E, cfg.c)
    t = sw.layer_tensors(T, d, F, E, C, for_backward=True)
    la = sw.make_layer_args(x, w_r, b_r, w1, w2, t, T, d, F, E, C, cfg.alpha, residual=True)
    sw.switch_layer_fwd(la, t["ws"], stream)
    dout = torch.randn((T, d), device=x.device, generator=torch.Generator(device=x.device).manual_seed(7)).to(
        torch.bfloat16)
    g = sw.layer_bwd_tensors(T, d, F, E, C)
    ba = sw.make_layer_bwd_args(t, x, w_r, w1, w2, dout, g, T, d, F, E, C, cfg.alpha)
    for _ in range(warmup):
        sw.switch_layer_bwd(ba, g["ws"], stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        sw.switch_layer_bwd(ba, g["ws"], stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    sw.switch_profile_enable(True)
    for _ in range(steps):
        sw.switch_layer_bwd(ba, g["ws"], stream)
    torch.cuda.synchronize()
    recs = sw.switch_profile_collect()
    sw.switch_profile_enable(False)
    per = {}
    for name, kms in recs:
        per[name] = per.get(name, 0.0) + kms
    kern = {k: round(1000.0 * v / steps, 2) for k, v in sorted(per.items(), key=lambda kv: -kv[1])}
    wbytes = 2 * E * F * d
    return {"ms_per_step": ms, "tokens_per_s": T / (ms / 1000.0), "kernels_us_per_step": kern,
            "weight_grad_bytes_fp32": 2 * wbytes}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build runs every expert on a single MI355X "
              "(no all-to-all, no sharding); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, max(1, args.steps))
        return

    import torch

    import sparse_mixture_experts_order_amd as sw
    import workloads

    cfg = workloads.CONFIGS[args.config]
    inp = workloads.make_layer_inputs(cfg)
    dev = "cuda"
    to_bf16 = lambda bits: torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(dev)
    x, w1, w2 = to_bf16(inp.x_bits), to_bf16(inp.w1_bits), to_bf16(inp.w2_bits)
    w_r, b_r = torch.from_numpy(inp.w_r).to(dev), torch.from_numpy(inp.b_r).to(dev)
    C = sw.switch_capacity(cfg.T, cfg.E, cfg.c)
    t = sw.layer_tensors(cfg.T, cfg.d, cfg.d_ff, cfg.E, C, device=dev, dlogits=cfg.want_grad)
    la = sw.make_layer_args(x, w_r, b_r, w1, w2, t, cfg.T, cfg.d, cfg.d_ff, cfg.E, C, cfg.alpha, residual=True)
    stream = torch.cuda.current_stream()

    def step():
        sw.switch_layer_fwd(la, t["ws"], stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K whole-layer steps, events on the launch stream
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = start.elapsed_time(stop)
    ms_per_step = ms_total / args.steps

    # per-kernel durations: the same K steps again with an event pair around
    # every launch (recorded on the launch stream by the library)
    sw.switch_profile_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    recs = sw.switch_profile_collect()
    sw.switch_profile_enable(False)
    per = {}
    for name, ms in recs:
        per.setdefault(name, []).append(ms)
    kern_us = {k: 1000.0 * float(np.mean(v)) for k, v in per.items()}

    accepted = t["accepted"].cpu().numpy().astype(np.int64)
    A = int(accepted.sum())
    T, d, F, E = cfg.T, cfg.d, cfg.d_ff, cfg.E
    # algorithmic bytes and flops per launch (padding rows excluded).  Without a
    # combine launch the second GEMM wrote the kept tokens' output rows itself
    # (residual row read, bf16 row written, slot_token and gate read) and the
    # gather copied the dropped tokens' residual rows.
    fused = "combine" not in kern_us
    w_bytes = 2 * E * F * d
    alg = {
        "expert_gemm1": dict(bytes=w_bytes + 2 * A * d + 2 * A * F, flops=2 * A * d * F),
        "expert_gemm2": dict(bytes=w_bytes + 2 * A * F + (4 * A * d + 8 * A if fused else 4 * A * d),
                             flops=2 * A * d * F),
        "gather": dict(bytes=2 * A * d + 2 * E * C * d + 9 * T + 8 * E + 4 * E * C + (4 * (T - A) * d if fused else 0),
                       flops=0),
        "combine": dict(bytes=4 * A * d + 2 * T * d + 2 * T * d + 13 * T, flops=0),
        "router_gemm": dict(bytes=2 * T * d + 6 * d * E + 4 * T * E, flops=2 * T * d * E),
        "router_fused": dict(bytes=2 * T * d + 6 * d * E + 12 * T + 4 * E * ((T + 63) // 64), flops=2 * T * d * E),
    }
    dominant = max((k for k in kern_us if k in alg), key=lambda k: kern_us[k])
    dur_s = kern_us[dominant] * 1e-6
    achieved = alg[dominant]["bytes"] / dur_s / 1e9
    ffn_us = kern_us.get("expert_gemm1", 0) + kern_us.get("expert_gemm2", 0)
    ffn_flops = 4 * A * d * F
    ffn_bytes = alg["expert_gemm1"]["bytes"] + alg["expert_gemm2"]["bytes"]
    dispatch_us = sum(kern_us.get(k, 0) for k in ("scan_local", "scan_offsets", "gather"))
    traffic = read_traffic(dominant, cfg.name)

    result = {
        "metric": METRIC,
        "value": cfg.T * args.steps / (ms_total / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: x ~ N(0,1) in bf16, router N(0, 0.1/d) fp32, experts truncated normal "
                "0.1/sqrt(fan_in) in bf16)",
        "config": {"workload": cfg.name, "T": T, "d_model": d, "d_ff": F, "E": E, "capacity_factor": cfg.c,
                   "C": C, "alpha": cfg.alpha, "aux_grad": bool(cfg.want_grad), "parallelism": "none (1 GPU)"},
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": achieved,
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS,
            "traffic": traffic,
            "algorithmic_bytes": alg[dominant]["bytes"],
            "avg_launch_us": kern_us[dominant],
        },
        "ffn": {
            "mfma_pct_of_bf16_peak": 100.0 * ffn_flops / (ffn_us * 1e-6) / (PEAK_BF16_TFLOPS * 1e12),
            "hbm_GBps": ffn_bytes / (ffn_us * 1e-6) / 1e9,
            "us": ffn_us,
            "algorithmic_flops": ffn_flops,
        },
        "dispatch": {
            "GBps": alg["gather"]["bytes"] / (dispatch_us * 1e-6) / 1e9 if dispatch_us else None,
            "gather_GBps": alg["gather"]["bytes"] / (kern_us["gather"] * 1e-6) / 1e9,
            "us": dispatch_us,
        },
        "combine": ({"fused": True, "into": "expert_gemm2 epilogue"} if fused else
                    {"fused": False, "GBps": alg["combine"]["bytes"] / (kern_us["combine"] * 1e-6) / 1e9}),
        "kernels_us": {k: round(v, 2) for k, v in sorted(kern_us.items(), key=lambda kv: -kv[1])},
        "routing": {"accepted": A, "drop_rate": 1 - A / T,
                    "empty_slot_ratio": 1 - A / (E * C) if C else None},
        "wall_s_timed": wall,
    }

    if not args.no_variants:
        result["variants"] = time_variants(sw, torch, cfg, x, w_r, b_r, w1, w2, stream, min(args.steps, 20),
                                           min(args.warmup, 5))

    if not args.no_cpu_baseline:
        rate, dt, threads, n = cpu_baseline(inp, cfg, args.cpu_sample_tokens)
        result["cpu_baseline"] = {
            "value": rate, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"whole fp64 oracle layer on {n} of {cfg.T} tokens, best of 3 ({dt:.1f} s each, "
                      f"{platform.processor() or platform.machine()})",
        }
    print(json.dumps(result))


if __name__ == "__main__":
    main()
