"""Benchmark: decoded frames/s of the Wan-style VAE decoder on one MI355X.

One step = one whole wvd_decode of the workload (every layer of the decoder,
all passes) with the latents already resident in HBM.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--config NAME] [--frames-per-pass P]
                  [--profile-steps N] [--no-cpu-baseline] [--gpus 1]
  python bench.py --config enc_c256_T13_704x1248    (the encoder)

The headline `value` is timed over K decodes with nothing else recorded on
the stream.  A separate pass of N decodes with HIP-event timing around every
launch inside the library (same stream as the kernels) gives the per-class
split and the dominant kernel's average launch time, from which the roofline
is computed.  The CPU baseline is the oracle timed on the exact causal prefix
of the same workload (the first two latent frames: five video frames), and
those five frames of the GPU's video are compared with it.
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
# The dominant kernel's sources: its file and the device helpers it inlines.
CONV_SRCS = [os.path.join(ROOT, "video_diffusion_vae_amd", "csrc", n) for n in ("wvd_conv.hip", "wvd_common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv3x3x3_main_c256_T49_704x1248_traffic.json")
# Direct 3x3x3 multiply-adds per Winograd-domain multiply-add: F(6,3) along x
# replaces 6 outputs x 27 taps by 8 planes x 9 (t, y) taps.  Reported only as
# a separate direct-equivalent rate; the roofline counts the multiply-adds the
# Winograd algorithm performs.
WINO_DIRECT_PER_EXECUTED = (6 * 27) / (8 * 9)


def conv_src_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for p in CONV_SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


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
    ap.add_argument("--cpu-sample-frames", type=int, default=2,
                    help="latent frames of the causal prefix the oracle decodes (2: five video frames)")
    ap.add_argument("--profile-steps", type=int, default=2,
                    help="decodes of the separate pass with per-launch HIP-event timing")
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
        # the first video is kept in host memory, so it does not count in the
        # next values' peak HBM
        host = out.cpu()
        same = True if ref is None else bool(torch.equal(host, ref))
        if ref is None:
            ref = host
        print(json.dumps({"workload": cfg.name, "frames_per_pass": P, "ms_per_decode": ms,
                          "frames_per_s": (4 * cfg.T - 3) / (ms / 1e3),
                          "peak_hbm_gib": torch.cuda.max_memory_allocated(dev) / 2 ** 30,
                          "peak_hbm_reserved_gib": torch.cuda.max_memory_reserved(dev) / 2 ** 30,
                          "workspace_gib": ws.numel() / 2 ** 30, "video_gib": out.numel() * 2 / 2 ** 30,
                          "resident_before_gib": base / 2 ** 30,
                          "bit_identical_to_first": same,
                          "fp16_range_flags": wvd.range_flags(clear=True)}), flush=True)
        del out, ws


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg, W, seed, T_sample):
    """The oracle on the exact causal prefix of T_sample latent frames, its
    BLAS threads limited to the cores this process may run on."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import decoder as O
    from video_diffusion_vae_amd import synth

    cores = len(os.sched_getaffinity(0))
    z = synth.make_latents(T_sample, cfg.h, cfg.w, seed=seed, bf16=cfg.weights_bf16)
    with threadpool_limits(limits=cores):
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        t0 = time.perf_counter()
        v = O.decode(z, W, cfg.c)
        dt = time.perf_counter() - t0
    frames = v.shape[2]
    return {
        "value": frames / dt,
        "unit": "frames/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"exact causal prefix: {T_sample} latent frame(s) -> {frames} video frame(s) of "
                  f"{cfg.name}, full decoder, numpy fp32 ({dt:.1f} s)",
        "seconds": dt,
        "gflops": O.conv_flops(cfg.c, T_sample, cfg.h, cfg.w, cfg.deep) / dt / 1e9,
        "cpu_model": cpu_model(),
        "affinity_cores": cores,
        "video": v,
    }


def run_encoder(args):
    """The encoder (the decoder's mirror image): encoded video frames/s of
    the clip, the dominant kernel's roofline from a separate profiled pass,
    and the encoder oracle on the first five video frames beside it."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import encoder as OE
    from video_diffusion_vae_amd import synth_encoder as SE
    from video_diffusion_vae_amd import wvd

    cfg = SE.encoder_config_by_name(args.config)
    P = args.frames_per_pass or cfg.passes[0]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    W = SE.make_encoder_weights(cfg.c, seed=args.seed, bf16=cfg.weights_bf16)
    dt = torch.bfloat16 if cfg.weights_bf16 else torch.float32
    enc = wvd.Encoder({k: torch.from_numpy(v).to(dt) for k, v in W.items()}, cfg.c, cfg.h, cfg.w, device=dev)
    v = torch.from_numpy(SE.make_video(cfg.T, cfg.h, cfg.w, seed=args.seed, bf16=cfg.weights_bf16)).to(dev).to(dt)
    out = torch.empty(cfg.latent_shape, dtype=torch.float32, device=dev)
    ws = torch.empty(enc.workspace_bytes(cfg.T, P), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        enc.encode(v, P, out=out, workspace=ws)
    torch.cuda.synchronize()
    wvd.range_flags(clear=True)
    torch.cuda.reset_peak_memory_stats(dev)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        enc.encode(v, P, out=out, workspace=ws)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    peak_alloc, peak_res = torch.cuda.max_memory_allocated(dev), torch.cuda.max_memory_reserved(dev)
    nprof = max(1, args.profile_steps)
    enc.profile(True)
    enc.profile_read()
    for _ in range(nprof):
        enc.encode(v, P, out=out, workspace=ws)
    torch.cuda.synchronize()
    prof = enc.profile_read()
    enc.profile(False)
    flags = wvd.range_flags(clear=True)
    frames = 4 * cfg.T - 3
    conv = prof["conv3x3x3_main"]
    launches = max(conv["launches"], 1)
    avg_ms = conv["ms"] / launches
    exec_tflops = conv["flops"] / launches / (avg_ms / 1e3) / 1e12 if conv["ms"] > 0 else 0.0
    res = {
        "metric": "encoded video frames/s at 704x1248 (the decoder's mirror-image encoder), 1 GPU",
        "value": frames / (ms / 1e3), "unit": "frames/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16",
        "data": "synthetic: seeded random-init weights (uniform +-1/sqrt(fan_in)), video uniform(-1,1), bf16-exact",
        "config": {"workload": cfg.name, "video": list(cfg.video_shape), "latents": list(cfg.latent_shape),
                   "frames_per_pass": P, "c": cfg.c},
        "roofline": {"bound": "mfma", "achieved": exec_tflops, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": exec_tflops / MFMA_PEAK_TFLOPS, "traffic": None,
                     "kernel": "conv_persist<256, 2, 4, 0, 4, *>: Winograd-domain GEMM of the norm-SiLU 3x3x3 "
                               "convs, all tile shapes",
                     "flops": "the Winograd-domain multiply-adds the kernel performs",
                     "avg_launch_ms": avg_ms, "launches_per_step": conv["launches"] / nprof},
        "executed_tflop_per_step": sum(x["flops"] for x in prof.values()) / nprof / 1e12,
        "nominal_tflop_per_step": OE.encoder_flops(cfg.c, cfg.T, cfg.h, cfg.w) / 1e12,
        "time_split_ms_per_step": {k: x["ms"] / nprof for k, x in prof.items()},
        "peak_hbm_gib": peak_alloc / 2 ** 30, "peak_hbm_reserved_gib": peak_res / 2 ** 30,
        "fp16_range_flags": flags,
    }
    if not args.no_cpu_baseline:
        Ts = args.cpu_sample_frames
        head = out[:, :, :Ts].cpu().numpy()
        del out, ws, v
        torch.cuda.empty_cache()
        vs = SE.make_video(Ts, cfg.h, cfg.w, seed=args.seed, bf16=cfg.weights_bf16)
        cores = len(os.sched_getaffinity(0))
        with threadpool_limits(limits=cores):
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
            t0 = time.perf_counter()
            ref = OE.encode(vs, W, cfg.c)
            dt_cpu = time.perf_counter() - t0
        res["cpu_baseline"] = {
            "value": vs.shape[2] / dt_cpu, "unit": "frames/s", "cores": int(threads), "kind": "oracle",
            "sample": f"exact causal prefix: {vs.shape[2]} video frame(s) -> {Ts} latent frame(s) of {cfg.name}, "
                      f"full encoder, numpy fp32 ({dt_cpu:.1f} s)",
            "gflops": OE.encoder_flops(cfg.c, Ts, cfg.h, cfg.w) / dt_cpu / 1e9, "cpu_model": cpu_model(),
            "affinity_cores": cores}
        d = np.abs(head.astype(np.float64) - ref)
        res["parity_vs_oracle_prefix"] = {
            "latent_frames": Ts, "max_abs": float(d.max()),
            "rel_l2": float(np.linalg.norm(head.astype(np.float64) - ref) / np.linalg.norm(ref)),
            "tolerance": {"max_abs": 3e-2, "rel_l2": 1e-2}}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the decoder has no multi-GPU path "
              "(one GPU per process, no collectives); rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        run_sweep(args)
        return
    if args.config.startswith("enc_"):
        run_encoder(args)
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
    wvd.range_flags(clear=True)
    torch.cuda.reset_peak_memory_stats(dev)

    # Headline: K decodes, nothing but the decoder's own launches on the stream.
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
    peak_alloc = torch.cuda.max_memory_allocated(dev)
    peak_reserved = torch.cuda.max_memory_reserved(dev)
    range_flags = wvd.range_flags(clear=True)

    # Separate pass: HIP events around every launch (per-class split, and the
    # dominant kernel's average launch time for the roofline).
    nprof = max(1, args.profile_steps)
    dec.profile(True)
    dec.profile_read()  # clear
    pe0 = torch.cuda.Event(enable_timing=True)
    pe1 = torch.cuda.Event(enable_timing=True)
    pe0.record(stream)
    for _ in range(nprof):
        dec.decode(zt, P, out=out, workspace=ws)
    pe1.record(stream)
    torch.cuda.synchronize()
    prof = dec.profile_read()
    dec.profile(False)
    ms_profiled = pe0.elapsed_time(pe1) / nprof
    range_flags |= wvd.range_flags(clear=True)
    vid = out.float()
    finite = bool(torch.isfinite(vid).all().item())
    in_range = bool((vid.abs() <= 1.0).all().item())
    del vid

    frames = 4 * cfg.T - 3
    fps = frames / (ms / 1e3)
    total_flops = O.conv_flops(cfg.c, cfg.T, cfg.h, cfg.w, cfg.deep)  # nominal (9-tap up-convs)
    exec_flops = sum(v["flops"] for v in prof.values()) / nprof
    conv = prof["conv3x3x3_main"]
    launches = max(conv["launches"], 1)
    avg_launch_ms = conv["ms"] / launches
    # FLOPs the dominant kernel performs per launch: 2 per Winograd-domain
    # multiply-add (F(6,3): 8 planes x 9 (t, y) taps per 6 output columns).
    avg_launch_exec = conv["flops"] / launches
    exec_tflops = avg_launch_exec / (avg_launch_ms / 1e3) / 1e12 if conv["ms"] > 0 else 0.0
    direct_tflops = exec_tflops * WINO_DIRECT_PER_EXECUTED
    gemm_ms = sum(prof[k]["ms"] for k in ("conv3x3x3_main", "conv_other", "attention_gemm"))
    gemm_fl = sum(prof[k]["flops"] for k in ("conv3x3x3_main", "conv_other", "attention_gemm"))
    all_ms = gemm_ms + prof["wino_transforms"]["ms"]
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
        "roofline": {"bound": "mfma", "achieved": exec_tflops, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": exec_tflops / MFMA_PEAK_TFLOPS, "traffic": measured_traffic(),
                     "kernel": "conv_persist<256, 2, 4, 0, 4, *>: Winograd-domain GEMM of the norm-SiLU "
                               "3x3x3 convs (F(6,3) along x, eight xi planes, causal (t,y) 3x3 taps), 256x256 "
                               "tiles of frames x rows x column groups (2x8x16 up to 8x8x4, chosen per "
                               "launch) on 4 waves, one persistent workgroup per CU; all tile shapes together",
                     "flops": "the multiply-adds the kernel's algorithm performs (Winograd-domain GEMM: "
                              "2 x 8 planes x 9 (t,y) taps x Cin x Cout per 6 output columns), 4/9 of the "
                              "direct 3x3x3 count",
                     "direct_equivalent_tflops": direct_tflops,
                     "avg_launch_ms": avg_launch_ms, "avg_launch_tflop": avg_launch_exec / 1e12,
                     "launches_per_step": conv["launches"] / nprof,
                     "timing": f"HIP events around each launch on the decode stream, {nprof} separate "
                               f"decode(s) after the timed ones"},
        "gemm_kernels_tflops": gemm_fl / (gemm_ms / 1e3) / 1e12 if gemm_ms > 0 else 0.0,
        "gemm_kernels_frac": gemm_fl / (gemm_ms / 1e3) / 1e12 / MFMA_PEAK_TFLOPS if gemm_ms > 0 else 0.0,
        "executed_tflop_per_step": exec_flops / 1e12,
        "executed_tflops_over_conv_time": exec_flops / (all_ms / 1e3) / 1e12 if all_ms > 0 else 0.0,
        "nominal_tflop_per_step": total_flops / 1e12,
        "end_to_end_direct_equivalent_tflops": total_flops / (ms / 1e3) / 1e12,
        "ms_per_step_profiled": ms_profiled,
        "time_split_ms_per_step": {k: v["ms"] / nprof for k, v in prof.items()},
        "launches_per_step": {k: v["launches"] / nprof for k, v in prof.items()},
        "peak_hbm_gib": peak_alloc / 2 ** 30,
        "peak_hbm_reserved_gib": peak_reserved / 2 ** 30,
        "output_finite_in_range": finite and in_range,
        "fp16_range_flags": range_flags,
        "wall_s": t_wall,
    }
    if not args.no_cpu_baseline:
        head = out[:, :, :4 * args.cpu_sample_frames - 3].float().cpu().numpy()
        del out, ws, zt
        torch.cuda.empty_cache()
        cb = cpu_baseline(cfg, W, args.seed, args.cpu_sample_frames)
        res["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        for k in ("gflops", "cpu_model", "affinity_cores"):
            res["cpu_baseline"][k] = cb[k]
        ref = cb["video"]
        d = np.abs(head.astype(np.float64) - ref)
        res["parity_vs_oracle_prefix"] = {
            "frames": int(ref.shape[2]), "max_abs": float(d.max()),
            "rel_l2": float(np.linalg.norm(head.astype(np.float64) - ref) / np.linalg.norm(ref)),
            "tolerance": {"max_abs": 3e-2, "rel_l2": 1e-2}}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
