"""Benchmark: decoded frames/s of the Wan-style VAE decoder on one MI355X.

One step = one whole wvd_decode of the workload (every layer of the decoder,
all passes) with the latents already resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config NAME] [--frames-per-pass P]
                  [--no-cpu-baseline] [--gpus 1]

The conv roofline comes from HIP-event timing of every launch inside the
library (same stream as the kernels), summed per kernel class; the CPU
baseline is the oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 / bf16 MFMA
HBM_PEAK_GBS = 8000.0
CONV_SRC = os.path.join(ROOT, "video_diffusion_vae_amd", "csrc", "wvd_conv.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv3x3x3_main_c256_T49_704x1248_traffic.json")
# Direct 3x3x3 multiply-adds per Winograd-domain multiply-add: F(6,3) along x
# replaces 6 outputs x 27 taps by 8 planes x 9 (t, y) taps.
WINO_DIRECT_PER_EXECUTED = (6 * 27) / (8 * 9)


def conv_src_hash() -> str:
    import hashlib
    with open(CONV_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic():
    """HBM bytes per launch of the dominant conv kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, or None when that summary was
    taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("conv_src_sha256") != conv_src_hash():
        return None
    return t.get("hbm_bytes_per_launch")
METRIC = "decoded frames/s at 704x1248, T=49, 1 GPU; Conv3d MFMA % of bf16 peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--config", default="c256_T49_704x1248")
    ap.add_argument("--frames-per-pass", type=int, default=None)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--T", type=int, default=None, help="override the latent frame count (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration-copy", action="store_true",
                    help="skip the cold 1 GiB copy that calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--cpu-sample-frames", type=int, default=1,
                    help="latent frames of the causal prefix the oracle decodes")
    ap.add_argument("--sweep", default=None,
                    help="comma-separated frames_per_pass values: print one JSON line per value with time "
                         "and peak HBM (the 481-frame workload sweeps 2,4,8,16)")
    return ap.parse_args()


def run_sweep(args):
    """frames_per_pass sweep: time per decode and peak allocated HBM for each
    value; outputs must be bit-identical across the sweep."""
    import torch

    from video_diffusion_vae_amd import synth, wvd

    cfg = synth.config_by_name(args.config)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(0)
    W = synth.make_weights(cfg.c, seed=args.seed, bf16=cfg.weights_bf16, deep=cfg.deep)
    dec = wvd.Decoder({k: torch.from_numpy(v).to(torch.bfloat16) for k, v in W.items()}, cfg.c, cfg.h, cfg.w,
                      device=dev)
    z = torch.from_numpy(synth.make_latents(cfg.T, cfg.h, cfg.w, seed=args.seed)).to(dev).to(torch.bfloat16)
    ref = None
    for P in [int(p) for p in args.sweep.split(",")]:
        dec.release_workspace()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats(dev)
        base = torch.cuda.memory_allocated(dev)
        out = torch.empty(cfg.video_shape, dtype=torch.bfloat16, device=dev)
        ws = torch.empty(dec.workspace_bytes(cfg.T, P), dtype=torch.uint8, device=dev)
        for _ in range(args.warmup):
            dec.decode(z, P, out=out, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            dec.decode(z, P, out=out, workspace=ws)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        same = True if ref is None else bool(torch.equal(out, ref))
        if ref is None:
            ref = out.clone()
        print(json.dumps({"workload": cfg.name, "frames_per_pass": P, "ms_per_decode": ms,
                          "frames_per_s": (4 * cfg.T - 3) / (ms / 1e3),
                          "peak_hbm_gib": torch.cuda.max_memory_allocated(dev) / 2 ** 30,
                          "workspace_gib": ws.numel() / 2 ** 30, "video_gib": out.numel() * 2 / 2 ** 30,
                          "resident_before_gib": base / 2 ** 30,
                          "bit_identical_to_first": same}), flush=True)
        del out, ws


def cpu_baseline(cfg, W, seed, T_sample):
    """The oracle on the exact causal prefix of T_sample latent frames."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import decoder as O
    from video_diffusion_vae_amd import synth

    z = synth.make_latents(T_sample, cfg.h, cfg.w, seed=seed, bf16=cfg.weights_bf16)
    t0 = time.perf_counter()
    v = O.decode(z, W, cfg.c)
    dt = time.perf_counter() - t0
    frames = v.shape[2]
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {
        "value": frames / dt,
        "unit": "frames/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"exact causal prefix: {T_sample} latent frame(s) -> {frames} video frame(s) of "
                  f"{cfg.name}, full decoder, numpy fp32 ({dt:.1f} s)",
        "seconds": dt,
        "gflops": O.conv_flops(cfg.c, T_sample, cfg.h, cfg.w, cfg.deep) / dt / 1e9,
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the decoder has no multi-GPU path "
              "(one GPU per process, no collectives); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        run_sweep(args)
        return
    import numpy as np
    import torch

    from video_diffusion_vae_amd import synth, wvd
    from oracle import decoder as O

    cfg = synth.config_by_name(args.config)
    if args.T:
        import dataclasses
        cfg = dataclasses.replace(cfg, T=args.T, name=f"{cfg.name}_prefixT{args.T}")
    P = args.frames_per_pass or cfg.passes[0]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    W = synth.make_weights(cfg.c, seed=args.seed, bf16=cfg.weights_bf16, deep=cfg.deep)
    wt = {k: torch.from_numpy(v) for k, v in W.items()}
    if cfg.weights_bf16:
        wt = {k: v.to(torch.bfloat16) for k, v in wt.items()}
    dec = wvd.Decoder(wt, cfg.c, cfg.h, cfg.w, device=dev)
    del wt
    z = synth.make_latents(cfg.T, cfg.h, cfg.w, seed=args.seed, bf16=cfg.weights_bf16)
    zt = torch.from_numpy(z).to(dev)
    if cfg.weights_bf16:
        zt = zt.to(torch.bfloat16)
    out = torch.empty(cfg.video_shape, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(dec.workspace_bytes(cfg.T, P), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    if not args.no_calibration_copy:
        # A plain copy of known size over a buffer larger than the last-level
        # cache: the reference that scales the HBM byte counters of a profile.
        src = torch.empty(1 << 28, dtype=torch.int32, device=dev)  # 1 GiB read, 1 GiB written
        dst = torch.empty_like(src)
        torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        dec.decode(zt, P, out=out, workspace=ws)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    dec.profile(True)
    dec.profile_read()  # clear
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        dec.decode(zt, P, out=out, workspace=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    prof = dec.profile_read()
    dec.profile(False)
    peak_alloc = torch.cuda.max_memory_allocated(dev)
    vid = out.float()
    finite = bool(torch.isfinite(vid).all().item())
    in_range = bool((vid.abs() <= 1.0).all().item())
    del vid

    frames = 4 * cfg.T - 3
    fps = frames / (ms / 1e3)
    total_flops = O.conv_flops(cfg.c, cfg.T, cfg.h, cfg.w, cfg.deep)  # nominal (9-tap up-convs)
    alg_flops = sum(v["flops"] for v in prof.values()) / args.steps
    conv = prof["conv3x3x3_main"]
    launches = max(conv["launches"], 1)
    avg_launch_ms = conv["ms"] / launches
    # The library counts the multiply-adds each launch performs; the roofline
    # uses algorithmic FLOPs (the direct 3x3x3 count these launches replace).
    avg_launch_exec = conv["flops"] / launches
    avg_launch_flops = avg_launch_exec * WINO_DIRECT_PER_EXECUTED
    exec_tflops = avg_launch_exec / (avg_launch_ms / 1e3) / 1e12 if conv["ms"] > 0 else 0.0
    conv_tflops = exec_tflops * WINO_DIRECT_PER_EXECUTED
    all_conv_ms = sum(prof[k]["ms"] for k in ("conv3x3x3_main", "conv_other", "attention_gemm", "wino_transforms"))
    all_conv_fl = (prof["conv3x3x3_main"]["flops"] * WINO_DIRECT_PER_EXECUTED +
                   sum(prof[k]["flops"] for k in ("conv_other", "attention_gemm")))
    res = {
        "metric": METRIC,
        "value": fps,
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic: seeded random-init weights (uniform +-1/sqrt(fan_in)), latents N(0,1), bf16-exact",
        "config": {"workload": cfg.name, "latents": [1, 48, cfg.T, cfg.h, cfg.w],
                   "video": list(cfg.video_shape), "frames_per_pass": P, "c": cfg.c},
        "roofline": {"bound": "mfma", "achieved": conv_tflops, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": conv_tflops / MFMA_PEAK_TFLOPS, "traffic": measured_traffic(),
                     "kernel": "conv_persist<256, 2, 4, 0, 4, *>: Winograd-domain GEMM of the norm-SiLU "
                               "3x3x3 convs (F(6,3) along x, eight xi planes, causal (t,y) 3x3 taps), 256x256 "
                               "tiles of frames x rows x column groups (2x8x16 up to 8x8x4, chosen per "
                               "launch) on 4 waves, one persistent workgroup per CU; all tile shapes together",
                     "flops": "algorithmic: the direct 3x3x3 convolution FLOPs of the launches; the kernel "
                              "performs 4/9 as many multiply-adds (F(6,3))",
                     "executed_mfma_tflops": exec_tflops, "executed_mfma_frac": exec_tflops / MFMA_PEAK_TFLOPS,
                     "avg_launch_ms": avg_launch_ms, "avg_launch_tflop": avg_launch_flops / 1e12,
                     "launches_per_step": conv["launches"] / args.steps},
        "conv_all_algorithmic_tflops": all_conv_fl / (all_conv_ms / 1e3) / 1e12 if all_conv_ms > 0 else 0.0,
        "executed_tflop_per_step": alg_flops / 1e12,
        "nominal_tflop_per_step": total_flops / 1e12,
        "end_to_end_direct_equivalent_tflops": total_flops / (ms / 1e3) / 1e12,
        "time_split_ms_per_step": {k: v["ms"] / args.steps for k, v in prof.items()},
        "launches_per_step": {k: v["launches"] / args.steps for k, v in prof.items()},
        "peak_hbm_gib": peak_alloc / 2 ** 30,
        "output_finite_in_range": finite and in_range,
        "wall_s": t_wall,
    }
    if not args.no_cpu_baseline:
        del out, ws, zt
        torch.cuda.empty_cache()
        cb = cpu_baseline(cfg, W, args.seed, args.cpu_sample_frames)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        res["cpu_baseline"]["gflops"] = cb["gflops"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
