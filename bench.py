"""Benchmark: the streaming 5 s video decode at 704x1248 on one MI355X.

One step = one whole decode of the synthetic Wan2.2-style decoder (48 -> 384 channels, 2 mid
residual blocks, 4 up stages of 384/384/192/96 channels, 2 of them temporal): latents
[1, 48, 31, 44, 78] in passes of 4 latent frames with the causal caches carried between passes,
121 bf16 frames of 704x1248 out. Inputs (latents, packed weights, cache, workspace) are resident
in HBM before the timed region starts; the timed region holds exactly `--steps` decodes.

Prints one JSON line:
  * value / ms_per_step: frames/s and ms per decode from a timed loop with no instrumentation;
  * roofline, conv, epilogues: from a second, instrumented loop of the same `--steps` decodes
    (HIP events around every conv and memory-bound launch, on the stream it runs on): the
    dominant conv configuration's achieved TFLOP/s against the bf16 dense peak, all convs'
    TFLOP/s, the memory-bound kernels' GB/s against the HBM peak;
  * peak HBM of the decode;
  * configs: the other workloads measured on their own (the fp32 single conv, the residual
    block, the upsample stage, the one-pass decode), each with its conv TFLOP/s, memory-bound
    GB/s, and the oracle's time on the host cores for the same workload or a bounded sample;
  * cpu_baseline: the oracle on a bounded sample of the streaming decode, timed here, beside
    the recorded wall time of the oracle's whole 121-frame decode (the stored samples' run).
"""
import argparse
import json
import math
import os
import platform
import subprocess
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import causal_convolution_causalconv3d_amd as wvd  # noqa: E402
import workloads as wl  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix-core peak
PEAK_HBM_GBS = 8000.0
GOLDEN = os.path.join(ROOT, "tests", "golden")

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


def host_info():
    """The host the CPU baseline runs on: logical CPUs, CPU model, OMP_NUM_THREADS."""
    model = platform.processor() or "unknown"
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, check=True).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model, "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def _oracle():
    import oracle  # CPU baseline leg only

    return oracle


def _timed(fn):
    t0 = time.perf_counter()
    out = fn()
    return out, time.perf_counter() - t0


def cpu_stream_sample():
    """The oracle on a bounded sample of the streaming decode: a 20x28 latent crop of the same
    latents, their first 3 latent frames in one pass with the first-frame rule (9 video frames of
    320x448), scaled to full-frame frames/s by the crop's share of the 44x78 latent frame."""
    oracle = _oracle()
    crop, nf = (20, 28), 3
    _, params = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=4)
    z = wl.streaming_latents(seed=5, latent_frames=31)[0, :, :nf, :crop[0], :crop[1]]
    p = oracle.as_numpy_params(params)
    video, dt = _timed(lambda: oracle.decode(oracle._f32(z), p, wl.FULL_DECODER, frames_per_pass=nf,
                                             first_frame_rule=True))
    share = (crop[0] * crop[1]) / float(wl.LATENT_H * wl.LATENT_W)
    return {"value": video.shape[1] * share / dt, "unit": "frames/s", "cores": oracle.num_threads(), "kind": "oracle",
            "seconds": round(dt, 2),
            "sample": f"oracle decode of a {crop[0]}x{crop[1]} crop of the streaming latents, their first {nf} "
                      f"latent frames in one pass with the first-frame rule ({video.shape[1]} frames of "
                      f"{crop[0] * 16}x{crop[1] * 16}) in {dt:.1f} s, scaled by the crop's share {share:.4f} of "
                      f"the 44x78 latent frame"}


def recorded_stream_oracle():
    """The wall time of the oracle's whole 121-frame streaming decode, from the stored samples'
    run (tests/golden/make_stream_golden.py), with the host it ran on; None if not stored."""
    path = os.path.join(GOLDEN, "stream_decode_samples.npz")
    if not os.path.exists(path):
        return None
    g = np.load(path)
    sec = float(g["oracle_seconds"])
    return {"value": 121.0 / sec, "unit": "frames/s", "seconds": round(sec, 1), "cores": int(g["threads"]),
            "cpu_model": str(g["cpu_model"]), "nproc": int(g["nproc"]),
            "what": f"the oracle's full 121-frame decode (passes of {int(g['oracle_pass'])} latent frames, "
                    f"bitwise the one-shot decode), timed once when the stored samples were written; "
                    f"not on this host"}


def timed_calls(fn, reps):
    """Median ms of `reps` calls of fn (each bracketed by events on the current stream)."""
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return float(np.median(ts))


def instrumented(fn, reps):
    """Per-config conv and memory-bound kernel figures over `reps` instrumented calls of fn."""
    wvd.timing_reset()
    wvd.timing_enable(True)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    wvd.timing_enable(False)
    per_cfg = wvd.timing_read()
    per_mem = wvd.timing_read_mem()
    launches = wvd.timing_launches()
    conv_ms = sum(v[1] for v in per_cfg.values())
    conv_flops = sum(v[2] for v in per_cfg.values())
    conv_bytes = sum(conv_launch_bytes(sh) for (_, _, _, sh) in launches)
    out = {}
    if per_cfg:
        tf = conv_flops / (conv_ms * 1e-3) / 1e12
        out["conv"] = {"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                       "gbs_algorithmic": round(conv_bytes / (conv_ms * 1e-3) / 1e9, 1),
                       "ms_per_call": round(conv_ms / reps, 4),
                       "per_config": {k: {"launches_per_call": v[0] // reps, "us_per_launch": round(1000 * v[1] / v[0], 1),
                                          "tflops": round(v[2] / (v[1] * 1e-3) / 1e12, 1),
                                          "frac_of_peak": round(v[2] / (v[1] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
                                      for k, v in per_cfg.items()}}
    if per_mem:
        out["memory_bound"] = {k: {"launches_per_call": v[0] // reps, "us_per_launch": round(1000 * v[1] / v[0], 1),
                                   "gbs": round(v[2] / (v[1] * 1e-3) / 1e9, 1),
                                   "frac_of_hbm": round(v[2] / (v[1] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
                               for k, v in per_mem.items()}
    return out


def bench_single_conv(reps, cpu):
    """The fp32 single causal conv [1,16,5,16,16] (latency bound: no roofline claim)."""
    cfg = wl.single_conv_fp32()
    x = cfg["x"].cuda()
    w = cfg["weight"].cuda()
    b = cfg["bias"].cuda()
    y = torch.empty_like(x)
    call = lambda: wvd.causal_conv3d(x, w, 16, bias=b, out=y, layout="NCTHW")  # noqa: E731
    call()
    ms = timed_calls(call, reps)
    r = {"workload": "single causal conv, fp32: x [1,16,5,16,16], weight [16,16,3,3,3], bias, 2 causal zero frames",
         "ms_per_call": round(ms, 4), "gflop": 2 * 1280 * 16 * 432 / 1e9}
    if cpu:
        oracle = _oracle()
        _, dt = _timed(lambda: oracle.causal_conv3d(cfg["x"][0], cfg["weight"], cfg["bias"]))
        r["cpu_oracle_seconds"] = round(dt, 4)
    return r


def bench_resblock(reps, cpu):
    """The residual block [1,384,4,44,78] with its given 2-frame history (bf16, fp32 accumulation)."""
    cfg = wl.resblock_bf16()
    wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
    x = cfg["x"].permute(0, 2, 3, 4, 1).contiguous().to(torch.bfloat16).cuda()
    hd = cfg["hist"].permute(0, 2, 3, 4, 1).contiguous().to(torch.bfloat16).cuda()
    y = torch.empty_like(x)
    call = lambda: wvd.resblock(x, wts, 1e-6, hist1=hd, hist2=hd, out=y)  # noqa: E731
    call()
    ms = timed_calls(call, reps)
    flops = 2 * (2.0 * 4 * 44 * 78 * 384 * 27 * 384)
    r = {"workload": "residual block, bf16 / fp32 acc: x [1,384,4,44,78] + 2-frame history, norm1 + SiLU, conv "
                     "384->384, norm2 + SiLU, conv 384->384, + x",
         "ms_per_call": round(ms, 4), "tflops_whole_block": round(flops / (ms * 1e-3) / 1e12, 1),
         "algorithmic_tflop": round(flops / 1e12, 4)}
    r.update(instrumented(call, reps))
    if cpu:
        oracle = _oracle()
        p = oracle.as_numpy_params(cfg["params"])
        _, dt = _timed(lambda: oracle.resblock(cfg["x"][0], p, "res", {}, 1e-6, given_hist=oracle._f32(cfg["hist"][0])))
        r["cpu_oracle_seconds"] = round(dt, 2)
    return r


def bench_upsample(reps, cpu):
    """The upsample stage [1,192,4,176,312] -> [1,192,8,352,624], spatial x2 first, then the time conv."""
    cfg = wl.upsample_stage_bf16()
    x = cfg["x"].permute(0, 2, 3, 4, 1).contiguous().to(torch.bfloat16).cuda()
    ws = wvd.conv_pack(cfg["spatial.weight"].cuda(), wvd.WVD_PACK_PHASE2X)
    wt = wvd.conv_pack(cfg["time.weight"].cuda())
    bs, bt = cfg["spatial.bias"].cuda(), cfg["time.bias"].cuda()
    y = torch.empty((1, 8, 352, 624, 192), dtype=torch.bfloat16, device="cuda")
    call = lambda: wvd.upsample(x, spatial=ws, spatial_bias=bs, temporal=wt, temporal_bias=bt,  # noqa: E731
                                order=wvd.WVD_SPATIAL_FIRST, out=y)
    call()
    ms = timed_calls(call, reps)
    flops = 2.0 * (4 * 4 * 176 * 312) * 192 * (4 * 192) + 2.0 * 4 * 352 * 624 * 384 * 3 * 192
    r = {"workload": "upsample stage, bf16: x [1,192,4,176,312] -> nearest x2 + 3x3 conv 192->192 (four 2x2 phase "
                     "convs) -> causal (3,1,1) conv 192->384 into 8 frames -> [1,192,8,352,624]",
         "ms_per_call": round(ms, 4), "tflops_whole_stage": round(flops / (ms * 1e-3) / 1e12, 1),
         "algorithmic_tflop": round(flops / 1e12, 4),
         "gbs_output": round(y.numel() * 2 / (ms * 1e-3) / 1e9, 1)}
    r.update(instrumented(call, reps))
    if cpu:
        oracle = _oracle()
        p = {k: oracle._f32(v) for k, v in cfg.items() if k != "x"}
        _, dt = _timed(lambda: oracle.upsample_stage(cfg["x"][0], p))
        r["cpu_oracle_seconds"] = round(dt, 2)
    return r


def bench_one_pass(dec, reps, cpu):
    """The one-pass decode [1,48,4,44,78] -> [1,3,16,704,1248] (the decoder's weights, seed 4, a
    non-first pass with empty caches), with PSNR against the oracle's stored samples."""
    z, _ = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=4)
    zd = z.to(torch.bfloat16).cuda()
    video = torch.empty((1, 3, 16, 704, 1248), dtype=torch.bfloat16, device="cuda")
    call = lambda: dec.decode(zd, frames_per_pass=4, first_frame_rule=False, out=video)  # noqa: E731
    call()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    call()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() / 2 ** 30
    ms = timed_calls(call, reps)
    r = {"workload": "one-pass decode: latents [1,48,4,44,78] -> video [1,3,16,704,1248], empty caches, "
                     "first-frame rule off",
         "ms_per_call": round(ms, 3), "frames_per_s": round(16 / (ms * 1e-3), 1), "peak_hbm_gib": round(peak, 3),
         "algorithmic_tflop": round(algorithmic_conv_flops(wl.FULL_DECODER, 4, 4) / 1e12, 3)}
    gp = os.path.join(GOLDEN, "decoder_onepass_samples.npz")
    if os.path.exists(gp):
        g = np.load(gp)
        got = video[0].float().cpu().reshape(-1).numpy()[g["index"]].astype(np.float64)
        mse = float(((got - g["value"]) ** 2).mean())
        rng = float(g["vmax"] - g["vmin"])
        r["psnr_db_vs_oracle_samples"] = round(10 * math.log10(rng * rng / mse), 2) if mse > 0 else None
    r.update(instrumented(call, reps))
    del video
    if cpu:
        oracle = _oracle()
        crop = (20, 28)
        zc, params = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=2, latent_hw=crop)
        p = oracle.as_numpy_params(params)
        v, dt = _timed(lambda: oracle.decode(oracle._f32(zc[0]), p, wl.FULL_DECODER, frames_per_pass=2,
                                             first_frame_rule=False))
        share = (crop[0] * crop[1]) / float(wl.LATENT_H * wl.LATENT_W)
        r["cpu_oracle"] = {"frames_per_s": v.shape[1] * share / dt, "seconds": round(dt, 2),
                           "sample": f"a {crop[0]}x{crop[1]} latent crop, 2 latent frames in one pass "
                                     f"({v.shape[1]} frames), scaled by the crop's share {share:.4f}"}
        if os.path.exists(gp):
            sec = float(np.load(gp)["oracle_seconds"])
            r["cpu_oracle"]["recorded_full_seconds"] = round(sec, 1)
            r["cpu_oracle"]["recorded_full_threads"] = int(np.load(gp)["threads"])
    return r


def bench_winograd(reps):
    """Same-box A/B of one causal 3x3x3 conv, direct (the decoder's kernel) against the Winograd
    F(2x2, 3x3) prototype, at the real topology's 512-channel 176x312 and 256-channel 352x624
    levels (16 frames, a 2-frame history, bias): median ms of each, the algorithmic (direct) conv
    TFLOP/s both reach, the Winograd time split into its products and transforms, and the largest
    difference between the two outputs relative to the direct one's largest value."""
    out = {}
    for C, T, H, W in ((512, 16, 176, 312), (256, 16, 352, 624)):
        g = torch.Generator().manual_seed(C)
        x = torch.nn.functional.silu(torch.randn((1, T, H, W, C), generator=g)).to(torch.bfloat16).cuda()
        h = torch.randn((1, 2, H, W, C), generator=g).to(torch.bfloat16).cuda()
        w = wl.kaiming(g, (C, C, 3, 3, 3)).cuda()
        b = (0.1 * torch.randn((C,), generator=g)).cuda()
        wd, ww = wvd.conv_pack(w), wvd.winograd_pack(w)
        yd, yw = torch.empty_like(x), torch.empty_like(x)
        ws = torch.empty(wvd.lib().wvd_winograd_workspace_bytes(C, C, T, 2, H, W), dtype=torch.uint8, device="cuda")
        direct = lambda: wvd.causal_conv3d(x, wd, C, bias=b, hist=h, out=yd)  # noqa: E731
        wino = lambda: wvd.causal_conv3d_winograd(x, ww, C, bias=b, hist=h, out=yw, ws=ws)  # noqa: E731
        direct()
        wino()
        torch.cuda.synchronize()
        diff = float((yw.float() - yd.float()).abs().max() / yd.float().abs().max())
        md, mw = timed_calls(direct, reps), timed_calls(wino, reps)
        flops = 2.0 * T * H * W * C * 27 * C
        inst = instrumented(wino, reps)
        key = f"{C}ch_{T}x{H}x{W}"
        out[key] = {"direct_ms": round(md, 3), "winograd_ms": round(mw, 3), "speedup": round(md / mw, 3),
                    "direct_tflops": round(flops / (md * 1e-3) / 1e12, 1),
                    "winograd_effective_tflops": round(flops / (mw * 1e-3) / 1e12, 1),
                    "winograd_products_ms": inst.get("conv", {}).get("ms_per_call"),
                    "winograd_products_tflops": inst.get("conv", {}).get("tflops"),
                    "winograd_transforms": inst.get("memory_bound"),
                    "workspace_gib": round(ws.numel() / 2 ** 30, 2),
                    "max_rel_diff_vs_direct": round(diff, 5)}
        del x, h, yd, yw, ws
        torch.cuda.empty_cache()
    return {"workload": "one causal 3x3x3 conv C->C, bias, 2-frame history: direct vs Winograd F(2x2,3x3)",
            "ms_per_call": None, "levels": out}


def conv_by_shape(launches, steps):
    """Conv launches grouped by configuration and problem shape: launches per step, average us,
    TFLOP/s (the kernel time of each layer of the decode)."""
    groups = {}
    for name, ms, fl, sh in launches:
        key = (f"{name} T{sh['T']} {sh['H']}x{sh['W']} {sh['Ci']}->{sh['N']} taps{sh['taps']} ph{sh['phases']}"
               + (" +res" if sh.get("res") else ""))
        g = groups.setdefault(key, [0, 0.0, 0.0])
        g[0] += 1
        g[1] += ms
        g[2] += fl
    return {k: {"per_step": v[0] // steps, "avg_us": round(1000.0 * v[1] / v[0], 1),
                "tflops": round(v[2] / (v[1] * 1e-3) / 1e12, 1)}
            for k, v in sorted(groups.items(), key=lambda kv: -kv[1][1])}


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
    ap.add_argument("--frames-per-pass", type=int, default=None,
                    help="latent frames per pass (default 4; with --topology real 2 through the late stages, "
                         "4 through the early ones: the same speed at 16.9 instead of 22.9 GiB)")
    ap.add_argument("--early-frames-per-pass", type=int, default=0, metavar="N",
                    help="latent frames per pass through the stages up to the last temporal upsample "
                         "(per-level pass sizes; the later stages keep --frames-per-pass); 0: same")
    ap.add_argument("--latent-frames", type=int, default=31)
    ap.add_argument("--topology", choices=("synthetic", "real"), default="synthetic",
                    help="synthetic: the configured 384/384/192/96 decoder (the headline); real: the Wan2.2 "
                         "TI2V-5B topology (1024/1024/512/256, mid attention, DupUp3D, 12-channel head, "
                         "unpatchify, clamp) with random weights, no CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--head", choices=("fused", "separate"), default="separate",
                    help="the last x2 upsample, norm_out + SiLU and the head as one kernel where the decoder allows "
                         "it (less memory, slower) or through the activated tensor (the default; "
                         "wvd_decode_fuse_head)")
    ap.add_argument("--norm1", choices=("fused", "separate"), default="fused",
                    help="each residual block's norm1 + SiLU in the producing conv's epilogue (the default) or as "
                         "a separate pass (wvd_decode_fuse_norm1)")
    ap.add_argument("--shortcut", choices=("fused", "separate"), default="fused",
                    help="a 192 -> 96 block's 1x1 shortcut in the epilogue of the x2 upsample that produces its "
                         "input (the default) or as a separate pass (wvd_decode_fuse_shortcut)")
    ap.add_argument("--no-configs", action="store_true", help="skip the other workloads' measurements")
    ap.add_argument("--config-reps", type=int, default=10, help="timed calls per other workload (median)")
    ap.add_argument("--workload", default="stream",
                    choices=("stream", "single_conv_fp32", "resblock", "upsample_stage", "one_pass_decode",
                             "winograd"),
                    help="stream: the headline decode (default); otherwise only that workload's measurement "
                         "(--config-reps calls after a warm-up one), printed as one JSON line (for profiling)")
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

    if args.workload != "stream":
        cpu = not args.no_cpu_baseline
        if args.workload == "winograd":
            r = bench_winograd(args.config_reps)
            print(json.dumps({"workload_key": args.workload, **r}), flush=True)
            return
        if args.workload == "one_pass_decode":
            _, params = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=4)
            dec = wvd.Decoder(wvd.desc_from_spec(wl.FULL_DECODER), params)
            r = bench_one_pass(dec, args.config_reps, cpu)
        else:
            fn = {"single_conv_fp32": bench_single_conv, "resblock": bench_resblock,
                  "upsample_stage": bench_upsample}[args.workload]
            r = fn(args.config_reps, cpu)
        if cpu:
            r["host"] = host_info()
        print(json.dumps({"workload_key": args.workload, **r}), flush=True)
        return

    real = args.topology == "real"
    spec = wl.REAL_DECODER if real else wl.FULL_DECODER
    wvd.decode_fuse_norm1(args.norm1 == "fused")
    wvd.decode_fuse_head(args.head == "fused")
    wvd.decode_fuse_shortcut(args.shortcut == "fused")
    _, params = wl.decoder_weights(spec, seed=4, latent_frames=4)
    z = wl.streaming_latents(seed=5, latent_frames=args.latent_frames).to(torch.bfloat16).cuda()
    dec = wvd.Decoder(wvd.desc_from_spec(spec), params)
    del params
    fpp = args.frames_per_pass
    if fpp is None:
        fpp = 2 if real else 4
        if real and args.early_frames_per_pass == 0:
            args.early_frames_per_pass = 4
    early = max(args.early_frames_per_pass, fpp)
    F = dec.video_frames(args.latent_frames, fpp)
    video = torch.empty(wvd.video_shape(dec.desc, F), dtype=torch.bfloat16, device="cuda")
    assert video.shape[3:] == (wl.VIDEO_H, wl.VIDEO_W)
    dec.workspace(fpp, early)
    torch.cuda.synchronize()
    step = lambda: dec.decode(z, frames_per_pass=fpp, out=video, early_frames_per_pass=early)  # noqa: E731

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()

    # the headline: no instrumentation inside the timed region
    wvd.timing_enable(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    peak_alloc = torch.cuda.max_memory_allocated() / 2 ** 30
    peak_reserved = torch.cuda.max_memory_reserved() / 2 ** 30
    elapsed = t1 - t0
    ms_per_step = 1000.0 * elapsed / args.steps
    fps = F * args.steps / elapsed
    print(f"headline: {ms_per_step:.2f} ms per decode, {fps:.1f} frames/s", file=sys.stderr, flush=True)

    # the breakdown: the same steps again with HIP events around every launch
    wvd.timing_reset()
    wvd.timing_enable(True)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    wvd.timing_enable(False)
    per_cfg = wvd.timing_read()
    per_mem = wvd.timing_read_mem()
    launches = wvd.timing_launches()
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
        "ms_per_step_instrumented": round(1000.0 * (t3 - t2) / args.steps, 3),
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
                   "early_frames_per_pass": early, "norm1": args.norm1, "head": args.head,
                   "shortcut": args.shortcut,
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
        "conv_by_shape": conv_by_shape(launches, args.steps),
        "epilogues": {k: {"launches_per_step": v[0] // args.steps, "avg_launch_us": round(1000.0 * v[1] / v[0], 2),
                          "gbs": round(v[2] / (v[1] * 1e-3) / 1e9, 1),
                          "frac_of_hbm": round(v[2] / (v[1] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "ms_per_step": round(v[1] / args.steps, 3)}
                      for k, v in per_mem.items()},
        "peak_hbm_gib": round(peak_alloc, 3),
        "peak_hbm_reserved_gib": round(peak_reserved, 3),
    }
    cpu = not args.no_cpu_baseline and not real
    if not args.no_configs and not real:
        del video
        dec._ws = None
        torch.cuda.empty_cache()
        configs = {}
        for key, fn in (("single_conv_fp32", lambda: bench_single_conv(args.config_reps, cpu)),
                        ("resblock", lambda: bench_resblock(args.config_reps, cpu)),
                        ("upsample_stage", lambda: bench_upsample(args.config_reps, cpu)),
                        ("one_pass_decode", lambda: bench_one_pass(dec, args.config_reps, cpu))):
            configs[key] = fn()
            torch.cuda.empty_cache()
            print(f"{key}: {configs[key]['ms_per_call']} ms", file=sys.stderr, flush=True)
        line["configs"] = configs
    line["achievable"] = achievable_peaks()
    # context for the roofline fraction: the dominant conv against what the chip's own library GEMM
    # sustains here (the bf16 figure assumes a clock that matrix work with random operands does
    # not hold under the power limit)
    line["roofline"]["frac_of_library_gemm"] = round(line["roofline"]["achieved"] /
                                                     line["achievable"]["bf16_gemm_tflops"], 4)
    if cpu:
        cb = cpu_stream_sample()
        cb["host"] = host_info()
        rec = recorded_stream_oracle()
        if rec is not None:
            cb["recorded_full_decode"] = rec
        line["cpu_baseline"] = cb
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
