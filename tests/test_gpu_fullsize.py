"""GPU parity at the workloads' full sizes, in the launch configuration the bench times.

  * residual block [1,384,4,44,78] with its 2-frame cache: every output against the oracle, and
    the histories it hands on (the last two frames of conv1's and conv2's activated inputs); its
    conv2 alone, in the block's tile configuration, on the oracle's bf16-rounded input, every
    output within the bf16 elementwise bound;
  * upsample stage [1,192,4,176,312] -> [1,192,8,352,624]: windows (corners, edges, centre)
    against the oracle run on the matching input crop plus a one-pixel halo (a conv is
    translation-equivariant, so the crop's interior equals the full-size result);
  * one-pass decode [1,48,4,44,78] -> [1,3,16,704,1248]: against the oracle's values at 32768
    seeded positions (tests/golden/decoder_onepass_samples.npz, written by make_decoder_golden.py
    from the oracle alone), bitwise pass-size invariance, and the same bits from channels-last
    latents;
  * streaming 5 s decode [1,48,31,44,78] -> 121 frames: bitwise equal for 4 frames per pass, 3,
    all 31 in one pass (the one-shot form), and per-level pass sizes (8 or 16 latent frames
    through the early stages, sub-passes of 4 through the late ones);
  * the same streaming decode (4 latent frames per pass) against the oracle's decode of the whole
    clip (tests/golden/stream_decode_samples.npz, written by make_stream_golden.py from the oracle
    alone, in passes of 5 latent frames, bitwise its one-shot decode): PSNR over the samples and
    on each sampled frame (frame 0, both sides of the GPU's and the oracle's first pass
    boundaries, a later boundary, frame 120), and each frame's mean and mean square over all of
    its pixels;
  * the Wan2.2 TI2V-5B topology at 704x1248 (random weights, 2 latent frames -> 5 frames, clamp
    off): against the oracle's decode in two passes of one latent frame
    (tests/golden/real_decode_samples.npz, written by make_real_golden.py from the oracle alone),
    the GPU decoding both latent frames in one pass, so the oracle's pass boundary is not one of
    the GPU's.
"""
import dataclasses
import math
import os

import numpy as np
import pytest
import torch

import causal_convolution_causalconv3d_amd as wvd
import oracle
import workloads as wl
from gpu_util import bf16_elementwise_ok, from_dev_nthwc, log, psnr, rel_max, to_dev_nthwc

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "decoder_onepass_samples.npz")
STREAM_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "stream_decode_samples.npz")
REAL_GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "real_decode_samples.npz")


def test_resblock_full_size():
    """The block's output, and each step inside it: the histories it hands on are the last two
    frames of norm1's activation (conv1's input) and of norm2's activation of conv1's output
    (conv2's input), so both intermediate tensors are checked at full size too."""
    cfg = wl.resblock_bf16()  # [1,384,4,44,78] + [1,384,2,44,78] cache, seed 2
    p = oracle.as_numpy_params(cfg["params"])
    hist = oracle._f32(cfg["hist"][0])
    x = oracle._f32(cfg["x"][0])
    a1 = oracle.norm_silu(x, p["res.norm1.gamma"], 1e-6)
    h = oracle.causal_conv3d(a1, p["res.conv1.weight"], p.get("res.conv1.bias"), hist)
    a2 = oracle.norm_silu(h, p["res.norm2.gamma"], 1e-6)
    ref = oracle.resblock(x, p, "res", {}, 1e-6, given_hist=hist)
    wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
    hd = to_dev_nthwc(cfg["hist"])
    C, T, H, W = x.shape
    h1o = torch.empty((1, 2, H, W, C), dtype=torch.bfloat16, device="cuda")
    h2o = torch.empty_like(h1o)
    y = wvd.resblock(to_dev_nthwc(cfg["x"]), wts, 1e-6, hist1=hd, hist2=hd, hist1_out=h1o, hist2_out=h2o)
    torch.cuda.synchronize()
    for name, got, want in (("norm1 activation", from_dev_nthwc(h1o), a1[:, T - 2:]),
                            ("conv1 + norm2 activation", from_dev_nthwc(h2o), a2[:, T - 2:])):
        r = rel_max(got, want)
        log(f"resblock full size, {name} (frames {T - 2}, {T - 1}): rel {r:.3e}, psnr {psnr(got, want):.2f} dB")
        assert r <= 2e-2
    got = from_dev_nthwc(y)
    r = rel_max(got, ref)
    log(f"resblock full size: rel {r:.3e}, psnr {psnr(got, ref):.2f} dB")
    assert r <= 2e-2


def test_resblock_conv2_full_size_alone():
    """conv2 of the full-size block by itself, on the oracle's conv2 input rounded to bf16 (so the
    kernel's error is not mixed with that of the steps before it), with the block's residual, in
    the same tile configuration the block launches: every output against the oracle."""
    cfg = wl.resblock_bf16()
    p = oracle.as_numpy_params(cfg["params"])
    hist = oracle._f32(cfg["hist"][0])
    x = oracle._f32(cfg["x"][0])
    a1 = oracle.norm_silu(x, p["res.norm1.gamma"], 1e-6)
    h = oracle.causal_conv3d(a1, p["res.conv1.weight"], p.get("res.conv1.bias"), hist)
    a2 = torch.from_numpy(oracle.norm_silu(h, p["res.norm2.gamma"], 1e-6)).to(torch.bfloat16)
    ref = oracle.add(oracle.causal_conv3d(a2.float().numpy(), p["res.conv2.weight"], p.get("res.conv2.bias"), hist), x)
    wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
    hd = to_dev_nthwc(cfg["hist"])
    xd = to_dev_nthwc(cfg["x"])
    wvd.timing_enable(True)
    try:
        wvd.timing_reset()
        wvd.resblock(xd, wts, 1e-6, hist1=hd, hist2=hd)
        torch.cuda.synchronize()
        in_block = wvd.timing_read()
        wvd.timing_reset()
        y = wvd.causal_conv3d(to_dev_nthwc(a2[None]), wts["conv2"], wts["cout"], bias=wts["bias2"], hist=hd,
                              residual=xd)
        torch.cuda.synchronize()
        alone = wvd.timing_read()
    finally:
        wvd.timing_enable(False)
    log(f"block convs {sorted(in_block)}, conv2 alone {sorted(alone)}")
    assert len(alone) == 1 and next(iter(alone.values()))[0] == 1 and set(alone) <= set(in_block)
    got = from_dev_nthwc(y)
    ok, worst = bf16_elementwise_ok(got, ref)
    log(f"resblock conv2 alone, full size: rel {rel_max(got, ref):.3e}, worst bf16 bound ratio {worst:.3f}")
    assert ok


def test_upsample_stage_full_size_windows():
    cfg = wl.upsample_stage_bf16()  # [1,192,4,176,312], seed 3
    x = cfg["x"]
    _, C, T, H, W = x.shape
    p = {k: oracle._f32(v) for k, v in cfg.items() if k != "x"}
    y = wvd.upsample(to_dev_nthwc(x), spatial=wvd.conv_pack(cfg["spatial.weight"].cuda(), wvd.WVD_PACK_PHASE2X),
                     spatial_bias=cfg["spatial.bias"].cuda(), temporal=wvd.conv_pack(cfg["time.weight"].cuda()),
                     temporal_bias=cfg["time.bias"].cuda(), order=wvd.WVD_SPATIAL_FIRST)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (1, 2 * T, 2 * H, 2 * W, C)
    S = 12
    windows = [(0, 0), (H - S, W - S), (H // 2, W // 2), (0, W // 3), (H // 3, 0), (H - S, 0)]
    for r0, c0 in windows:
        r1, c1 = r0 + S, c0 + S
        a0, a1 = max(r0 - 1, 0), min(r1 + 1, H)
        b0, b1 = max(c0 - 1, 0), min(c1 + 1, W)
        ref = oracle.upsample_stage(x[0, :, :, a0:a1, b0:b1], p)
        ref = ref[:, :, 2 * (r0 - a0):2 * (r0 - a0) + 2 * S, 2 * (c0 - b0):2 * (c0 - b0) + 2 * S]
        got = y[0, :, 2 * r0:2 * r1, 2 * c0:2 * c1].float().cpu().permute(3, 0, 1, 2).numpy()
        r = rel_max(got, ref)
        log(f"upsample window ({r0},{c0}): rel {r:.3e}")
        assert r <= 2e-2


def _full_decoder(params):
    return wvd.Decoder(wvd.make_desc(), params)


def test_one_pass_decode_full_size_against_oracle_samples():
    z, params = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=4)
    dec = _full_decoder(params)
    zd = z.to(torch.bfloat16).cuda()
    v4 = dec.decode(zd, frames_per_pass=4, first_frame_rule=False)
    torch.cuda.synchronize()
    assert tuple(v4.shape) == (1, 3, 16, 704, 1248)
    assert bool(torch.isfinite(v4.float()).all())
    for fpp in (1, 3):
        assert torch.equal(dec.decode(zd, frames_per_pass=fpp, first_frame_rule=False), v4), fpp
    z_cl = zd.permute(0, 2, 3, 4, 1).contiguous()
    assert torch.equal(dec.decode(z_cl, frames_per_pass=4, first_frame_rule=False, z_layout="NTHWC"), v4)
    if not os.path.exists(GOLDEN):
        pytest.skip("golden samples not generated (tests/golden/make_decoder_golden.py)")
    g = np.load(GOLDEN)
    flat = v4[0].float().cpu().reshape(-1).numpy()
    got, ref = flat[g["index"]], g["value"]
    mse = float(((got.astype(np.float64) - ref) ** 2).mean())
    rng = float(g["vmax"] - g["vmin"])
    q = math.inf if mse == 0 else 10 * math.log10(rng * rng / mse)
    log(f"one-pass decode vs oracle samples: psnr {q:.2f} dB, max abs {np.abs(got - ref).max():.3e}, range {rng:.3f}")
    assert q >= 55.0


def test_streaming_decode_full_size_pass_size_invariant():
    _, params = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=4)
    z = wl.streaming_latents(seed=5, latent_frames=31).to(torch.bfloat16).cuda()
    dec = _full_decoder(params)
    v4 = dec.decode(z, frames_per_pass=4).clone()
    torch.cuda.synchronize()
    assert tuple(v4.shape) == (1, 3, 121, 704, 1248)
    assert bool(torch.isfinite(v4.float()).all())
    for fpp, early in ((3, None), (31, None), (4, 8), (4, 16)):
        log(f"streaming decode fpp={fpp} early={early}")
        v = dec.decode(z, frames_per_pass=fpp, early_frames_per_pass=early)
        torch.cuda.synchronize()
        assert torch.equal(v, v4), (fpp, early)
        del v
        dec._ws = None
        torch.cuda.empty_cache()


def _check_stream_golden(v, g, label):
    """The 121-frame 704x1248 video against the one-shot oracle's stored samples: PSNR over the
    samples and at the first frame, pass boundaries and the last frame, and every frame's mean
    and mean square over all its pixels."""
    assert tuple(v.shape) == (1, 3, 121, 704, 1248)
    video = v[0].float()
    flat = video.reshape(-1)
    idx = torch.from_numpy(g["index"]).cuda()
    got = flat[idx].cpu().numpy().astype(np.float64)
    ref = g["value"].astype(np.float64)
    rng = float(g["vmax"] - g["vmin"])
    err = got - ref
    q = 10 * math.log10(rng * rng / float((err ** 2).mean()))
    log(f"{label} vs one-shot oracle: psnr {q:.2f} dB over {ref.size} samples, max abs {np.abs(err).max():.3e}, "
        f"range {rng:.3f}")
    assert q >= 55.0
    frame = (g["index"] // (704 * 1248)) % 121
    for f in (0, 12, 13, 14, 16, 17, 60, 61, 120):
        e = err[frame == f]
        qf = 10 * math.log10(rng * rng / float((e ** 2).mean()))
        log(f"  frame {f}: psnr {qf:.2f} dB over {e.size} samples, max abs {np.abs(e).max():.3e}")
        assert qf >= 55.0, f
    # every frame's mean and mean square over all its pixels
    per_frame = video.permute(1, 0, 2, 3).reshape(121, -1).double()
    mean = per_frame.mean(dim=1).cpu().numpy()
    meansq = (per_frame ** 2).mean(dim=1).cpu().numpy()
    dm = np.abs(mean - g["frame_mean"]).max() / rng
    dq = np.abs(meansq / g["frame_meansq"] - 1.0).max()
    log(f"  per-frame mean: max |diff| {dm:.2e} of the range; mean square: max rel diff {dq:.2e}")
    assert dm <= 1e-3 and dq <= 1e-2


def test_streaming_decode_full_size_against_the_one_shot_oracle():
    if not os.path.exists(STREAM_GOLDEN):
        pytest.skip("stream golden samples not generated (tests/golden/make_stream_golden.py)")
    g = np.load(STREAM_GOLDEN)
    _, params = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=4)
    z = wl.streaming_latents(seed=5, latent_frames=31)
    dec = _full_decoder(params)
    v = dec.decode(z.to(torch.bfloat16).cuda(), frames_per_pass=4)
    torch.cuda.synchronize()
    _check_stream_golden(v, g, "streaming decode")


def test_fused_tail_streaming_decode_full_size_against_the_one_shot_oracle():
    """The same decode with the last upsample, norm_out and the head as one kernel
    (wvd_decode_fuse_head): against the one-shot oracle's samples, and bitwise the same for 4 and
    3 latent frames per pass (the head's partial sums carried across every pass boundary)."""
    if not os.path.exists(STREAM_GOLDEN):
        pytest.skip("stream golden samples not generated (tests/golden/make_stream_golden.py)")
    g = np.load(STREAM_GOLDEN)
    _, params = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=4)
    z = wl.streaming_latents(seed=5, latent_frames=31).to(torch.bfloat16).cuda()
    try:
        wvd.decode_fuse_head(True)
        dec = _full_decoder(params)
        wvd.timing_reset()
        wvd.timing_enable(True)
        v4 = dec.decode(z, frames_per_pass=4).clone()
        torch.cuda.synchronize()
        wvd.timing_enable(False)
        ran = wvd.timing_read()
        log(f"fused tail launches: {ran.get('conv_tail_phase_head_n3_m1_w8')}")
        assert "conv_tail_phase_head_n3_m1_w8" in ran and "conv_phase_halo_dma_n3_m1_w8" not in ran
        _check_stream_golden(v4, g, "fused-tail streaming decode")
        log("fused tail, 3 latent frames per pass")
        v3 = dec.decode(z, frames_per_pass=3)
        torch.cuda.synchronize()
        assert torch.equal(v3, v4)
    finally:
        wvd.decode_fuse_head(False)
        wvd.timing_enable(False)


def test_real_topology_full_size_streaming_properties():
    """The Wan2.2 TI2V-5B topology at 704x1248 (random weights): 9 latent frames give 33 frames
    in [-1, 1] (the clamp), every pass size and the per-level pass sizes give the same bits, and
    latent frames after the first pass leave the first pass's video frames untouched."""
    spec = wl.REAL_DECODER
    _, params = wl.decoder_weights(spec, seed=4, latent_frames=4)
    z = wl.streaming_latents(seed=5, latent_frames=9).to(torch.bfloat16).cuda()
    dec = wvd.Decoder(wvd.desc_from_spec(spec), params)
    del params
    log("real topology full size, 9 latent frames")
    v4 = dec.decode(z, frames_per_pass=4).clone()
    torch.cuda.synchronize()
    assert tuple(v4.shape) == (1, 3, 33, 704, 1248)
    assert bool(torch.isfinite(v4.float()).all()) and float(v4.float().abs().max()) <= 1.0
    for fpp, early in ((3, None), (4, 9)):
        log(f"real topology fpp={fpp} early={early}")
        v = dec.decode(z, frames_per_pass=fpp, early_frames_per_pass=early)
        torch.cuda.synchronize()
        assert torch.equal(v, v4), (fpp, early)
        del v
        dec._ws = None
        torch.cuda.empty_cache()
    z2 = z.clone()
    z2[:, :, 4:] = 0
    v = dec.decode(z2, frames_per_pass=4)
    torch.cuda.synchronize()
    assert torch.equal(v[:, :, :13], v4[:, :, :13])  # latent frames 0..3 -> video frames 0..12
    assert not torch.equal(v[:, :, 13:], v4[:, :, 13:])


def test_real_topology_full_size_against_oracle_samples():
    """The real topology without the clamp (random weights put most values outside [-1, 1]; the
    clamp is pinned as clamped == clip(unclamped) on small decoders): 2 latent frames -> 5 frames
    at 704x1248, one GPU pass against the oracle's two, PSNR over the stored samples and on each
    frame, and each frame's mean and mean square."""
    if not os.path.exists(REAL_GOLDEN):
        pytest.skip("real-topology golden samples not generated (tests/golden/make_real_golden.py)")
    g = np.load(REAL_GOLDEN)
    spec = dataclasses.replace(wl.REAL_DECODER, clamp=False)
    z, params = wl.decoder_weights(spec, seed=4, latent_frames=2)
    dec = wvd.Decoder(wvd.desc_from_spec(spec), params)
    del params
    v = dec.decode(z.to(torch.bfloat16).cuda(), frames_per_pass=2)
    torch.cuda.synchronize()
    assert tuple(v.shape) == (1, 3, 5, 704, 1248)
    video = v[0].float()
    flat = video.reshape(-1)
    got = flat[torch.from_numpy(g["index"]).cuda()].cpu().numpy().astype(np.float64)
    ref = g["value"].astype(np.float64)
    rng = float(g["vmax"] - g["vmin"])
    err = got - ref
    q = 10 * math.log10(rng * rng / float((err ** 2).mean()))
    log(f"real topology vs oracle: psnr {q:.2f} dB over {ref.size} samples, max abs {np.abs(err).max():.3e}, "
        f"range {rng:.3f}")
    assert q >= 55.0
    frame = (g["index"] // (704 * 1248)) % 5
    for f in range(5):
        e = err[frame == f]
        qf = 10 * math.log10(rng * rng / float((e ** 2).mean()))
        log(f"  frame {f}: psnr {qf:.2f} dB over {e.size} samples, max abs {np.abs(e).max():.3e}")
        assert qf >= 55.0, f
    per_frame = video.permute(1, 0, 2, 3).reshape(5, -1).double()
    mean = per_frame.mean(dim=1).cpu().numpy()
    meansq = (per_frame ** 2).mean(dim=1).cpu().numpy()
    dm = np.abs(mean - g["frame_mean"]).max() / rng
    dq = np.abs(meansq / g["frame_meansq"] - 1.0).max()
    log(f"  per-frame mean: max |diff| {dm:.2e} of the range; mean square: max rel diff {dq:.2e}")
    assert dm <= 1e-3 and dq <= 1e-2
