"""Benchmark: the streaming 5 s video decode at 704x1248 on one MI355X.

One step = one whole decode of the synthetic Wan2.2-style decoder (48 -> 384 channels, 2 mid
residual blocks, 4 up stages of 384/384/192/96 channels, 2 of them temporal): latents
[1, 48, 31, 44, 78] in passes of 4 latent frames with the causal caches carried between passes,
121 bf16 frames of 704x1248 out. Inputs (latents, packed weights, cache, workspace) are resident
in HBM before the timed region starts; the timed region holds exactly `--steps` decodes.

Prints one JSON line: frames/s (value), ms per decode, the matrix-core conv kernels' achieved
TFLOP/s against the bf16 dense peak (measured with HIP events around every conv launch in the
timed region), peak HBM, and the CPU oracle timed on a bounded sample of the same decode.
"""
import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import causal_convolution_causalconv3d_amd as wvd  # noqa: E402
import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0

from causal_convolution_causalconv3d_amd import profiling  # noqa: E402


def algorithmic_conv_flops(spec: wl.DecoderSpec, latent_frames: int, fpp: int, hw=(wl.LATENT_H, wl.LATENT_W)) -> float:
    """2*M*N*K of every conv of the decode, with the spatial x2 conv in its four-phase form
    (4 taps of C per phase at the low resolution), real (unpadded) channel counts."""
    total = 0.0
    start = 0
    n_st = len(spec.stage_channels)
    spatial = getattr(spec, "spatial", (True,) * n_st)
    while start < latent_frames:
        n = min(fpp, latent_frames - start)
        first = start == 0
        T = n
        H, W = hw
        c = spec.base_channels
        P = T * H * W
        if getattr(spec, "post_quant", False):
            total += 2.0 * P * spec.z_channels * spec.z_channels
        total += 2.0 * P * c * 27 * spec.z_channels
        for i in range(spec.mid_resblocks):
            total += 2.0 * P * c * 27 * c * 2
            if i == 0 and getattr(spec, "mid_attention", False):
                hw_ = H * W  # qkv, scores, values, proj
                total += 2.0 * P * 3 * c * c + T * (2.0 * hw_ * hw_ * c * 2) + 2.0 * P * c * c
        for s, cs in enumerate(spec.stage_channels):
            P = T * H * W
            for j in range(spec.stage_resblocks):
                cin = c if j == 0 else cs
                total += 2.0 * P * cs * 27 * cin + 2.0 * P * cs * 27 * cs
                if cin != cs:
                    total += 2.0 * P * cs * cin
            c = cs
            if spec.temporal[s]:
                Tc = T - 1 if first else T
                total += 2.0 * Tc * H * W * (2 * c) * 3 * c
                T = 2 * T - 1 if first else 2 * T
            if spatial[s]:
                total += 2.0 * (4 * T * H * W) * c * (4 * c)
                H, W = 2 * H, 2 * W
        total += 2.0 * T * H * W * spec.out_channels * 27 * c
        start += n
    return total


def achievable_peaks():
    """What this chip sustains, as context for the spec peaks: a large bf16 library GEMM (torch.matmul,
    8192^3, random data) in TFLOP/s and a plain device copy (2 GiB) in GB/s. Run after the timed
    region; not part of any step."""
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(0)
    a = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
    b = torch.randn((n, n), device="cuda", generator=g).to(torch.bfloat16)
    c = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    nbytes = 2 << 30
    x = torch.empty(nbytes // 4, device="cuda", dtype=torch.float32).normal_(generator=g)
    y = torch.empty_like(x)
    y.copy_(x)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2.0 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return {"bf16_gemm_tflops": round(gemm_tflops, 1), "copy_gbs": round(copy_gbs, 1),
            "what": "torch.matmul bf16 8192^3 (hipBLASLt) and a 2 GiB device copy, 20 reps each, after the timed region"}


def cpu_baseline(seconds_hint: float = 15.0):
    """The oracle (as it stands) on a bounded sample of the same decode: a 20x28 latent crop,
    one pass of 2 latent frames (8 video frames of 320x448), scaled to full-frame frames/s by the
    crop's share of the 44x78 latent frame (about 10 s on 16 host cores)."""
    import oracle  # CPU baseline leg only

    crop = (20, 28)
    z, params = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=2, latent_hw=crop)
    p = oracle.as_numpy_params(params)
    zz = oracle._f32(z[0])
    t0 = time.perf_counter()
    video = oracle.decode(zz, p, wl.FULL_DECODER, frames_per_pass=2, first_frame_rule=False)
    dt = time.perf_counter() - t0
    share = (crop[0] * crop[1]) / float(wl.LATENT_H * wl.LATENT_W)
    frames_equiv = video.shape[1] * share
    return {"value": frames_equiv / dt, "unit": "frames/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"oracle decode of a {crop[0]}x{crop[1]} latent crop, 2 latent frames (one pass, {video.shape[1]} "
                      f"frames of {crop[0] * 16}x{crop[1] * 16}) in {dt:.1f} s, scaled by the crop's share "
                      f"{share:.4f} of the 44x78 latent frame"}


def conv_launch_bytes(sh) -> float:
    """Algorithmic HBM bytes of one conv launch: the input frames it reads (with up to kt - 1 history
    frames) once, the packed weights once, the bf16 output once, the residual once when it adds
    one, and the cache frames it copies as side work (read and written once)."""
    kt = 3 if sh["taps"] in (27, 3) else 1
    frames_in = sh["T"] + min(sh["Th"], kt - 1)
    hw = sh["H"] * sh["W"]
    out = sh["T"] * hw * sh["phases"] * sh["N"]
    return 2.0 * (frames_in * hw * sh["Ci"] + sh["phases"] * sh["N"] * sh["taps"] * sh["Ci"]
                  + out * (2 if sh.get("res", 0) else 1) + 2 * sh.get("copied", 0) * hw * sh["Ci"])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--frames-per-pass", type=int, default=4)
    ap.add_argument("--early-frames-per-pass", type=int, default=0, metavar="N",
                    help="latent frames per pass through the stages up to the last temporal upsample "
                         "(per-level pass sizes; the later stages keep --frames-per-pass); 0: same")
    ap.add_argument("--latent-frames", type=int, default=31)
    ap.add_argument("--topology", choices=("synthetic", "real"), default="synthetic",
                    help="synthetic: the configured 384/384/192/96 decoder (the headline); real: the Wan2.2 "
                         "TI2V-5B topology (1024/1024/512/256, mid attention, DupUp3D, 12-channel head, "
                         "unpatchify, clamp) with random weights, no CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain copy kernel over MIB MiB (calibrates the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the decode is not sharded here.",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        profiling.copy_calibration_run(args.copy_calibration)
        return

    real = args.topology == "real"
    spec = wl.REAL_DECODER if real else wl.FULL_DECODER
    _, params = wl.decoder_weights(spec, seed=4, latent_frames=4)
    z = wl.streaming_latents(seed=5, latent_frames=args.latent_frames).to(torch.bfloat16).cuda()
    dec = wvd.Decoder(wvd.desc_from_spec(spec), params)
    del params
    fpp = args.frames_per_pass
    early = max(args.early_frames_per_pass, fpp)
    F = dec.video_frames(args.latent_frames, fpp)
    video = torch.empty(wvd.video_shape(dec.desc, F), dtype=torch.bfloat16, device="cuda")
    assert video.shape[3:] == (wl.VIDEO_H, wl.VIDEO_W)
    dec.workspace(fpp, early)
    torch.cuda.synchronize()

    for _ in range(args.warmup):
        dec.decode(z, frames_per_pass=fpp, out=video, early_frames_per_pass=early)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()

    wvd.timing_reset()
    wvd.timing_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dec.decode(z, frames_per_pass=fpp, out=video, early_frames_per_pass=early)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wvd.timing_enable(False)
    per_cfg = wvd.timing_read()
    per_mem = wvd.timing_read_mem()
    launches = wvd.timing_launches()
    peak_alloc = torch.cuda.max_memory_allocated() / 2 ** 30
    peak_reserved = torch.cuda.max_memory_reserved() / 2 ** 30

    elapsed = t1 - t0
    ms_per_step = 1000.0 * elapsed / args.steps
    fps = F * args.steps / elapsed
    conv_ms = sum(v[1] for v in per_cfg.values())
    conv_flops = sum(v[2] for v in per_cfg.values())
    # the dominant kernel: the conv configuration with the most time
    dom_name, (dom_n, dom_ms, dom_flops) = max(per_cfg.items(), key=lambda kv: kv[1][1])
    dom_tflops = (dom_flops / dom_n) / (dom_ms / dom_n * 1e-3) / 1e12
    algo = algorithmic_conv_flops(spec, args.latent_frames, fpp)
    dom_bytes = [conv_launch_bytes(sh) for (nm, _, _, sh) in launches if nm == dom_name]

    line = {
        "metric": "decoded frames/s at 704x1248 + conv TFLOP/s vs bf16 MFMA peak; peak HBM GiB",
        "value": round(fps, 3),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"streaming decode: latents [1,48,{args.latent_frames},44,78] -> video "
                               f"[1,3,{F},704,1248], "
                               f"{fpp} latent frames per pass"
                               + (f" ({early} per pass through conv_in, the middle blocks and the two temporal "
                                  f"stages)" if early > fpp else "")
                               + (", the Wan2.2 TI2V-5B decoder topology: post_quant_conv, conv_in 48->1024, mid "
                                  "resblock + single-head attention + resblock, up blocks 1024/1024/512/256 (3 "
                                  "resblocks each; time x2 on the first two, spatial x2 and DupUp3D on the first "
                                  "three), conv_out 256->12, unpatchify, clamp; random Kaiming weights" if real else
                                  ", decoder 48->384, 2 mid resblocks, stages "
                                  "384/384/192/96 (2 resblocks each, time x2 on the first two), random Kaiming weights"),
                   "topology": args.topology,
                   "latent_frames": args.latent_frames, "video_frames": F, "frames_per_pass": fpp,
                   "early_frames_per_pass": early,
                   "global_batch": 1, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "kernel": dom_name, "achieved": round(dom_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(dom_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": profiling.committed_traffic(dom_name), "traffic_unit": "HBM bytes per launch",
                     "launches_per_step": dom_n // args.steps,
                     "avg_launch_us": round(1000.0 * dom_ms / dom_n, 2),
                     "flops_per_launch": dom_flops / dom_n,
                     "algorithmic_bytes_per_launch": round(sum(dom_bytes) / max(len(dom_bytes), 1))},
        "conv": {"tflops": round(conv_flops / (conv_ms * 1e-3) / 1e12, 2),
                 "frac_of_peak": round(conv_flops / (conv_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                 "conv_ms_per_step": round(conv_ms / args.steps, 3),
                 "algorithmic_tflop_per_step": round(algo / 1e12, 3),
                 "timed_tflop_per_step": round(conv_flops / args.steps / 1e12, 3),
                 "per_config": {k: {"launches": v[0], "ms": round(v[1], 3), "tflops": round(v[2] / (v[1] * 1e-3) / 1e12, 2)}
                                for k, v in per_cfg.items()}},
        "epilogues": {k: {"launches_per_step": v[0] // args.steps, "avg_launch_us": round(1000.0 * v[1] / v[0], 2),
                          "gbs": round(v[2] / (v[1] * 1e-3) / 1e9, 1),
                          "frac_of_hbm": round(v[2] / (v[1] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "ms_per_step": round(v[1] / args.steps, 3)}
                      for k, v in per_mem.items()},
        "achievable": achievable_peaks(),
        "peak_hbm_gib": round(peak_alloc, 3),
        "peak_hbm_reserved_gib": round(peak_reserved, 3),
    }
    if not args.no_cpu_baseline and not real:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
