"""GPU parity: the HIP path (through the C ABI) against the oracle, element by element, on the
same seeded inputs. Sizes span several tiles and ragged tails; the full-size workload cases follow in
test_gpu_fullsize.py.

Tolerances. fp32 path: max abs error <= 1e-4 (fp32 accumulation of <= 27*Ci products against the
oracle's double sums). bf16 single ops (one conv, one norm): elementwise
|d| <= 2 * 2^-9 * |ref| + 1e-4 * max|ref| (one bf16 rounding of the result, a flipped rounding,
and fp32 summation error), on identical bf16 inputs. Composite layers (residual block, upsample
stage), whose bf16 path rounds its intermediates: normwise max relative error <= 2e-2. Whole
decodes: PSNR >= 55 dB against the fp32 oracle.
"""
import numpy as np
import pytest
import torch

import causal_convolution_causalconv3d_amd as wvd
import oracle
import workloads as wl
from gpu_util import bf16_elementwise_ok, from_dev_nthwc, log, psnr, rel_max, to_dev_nthwc

pytestmark = pytest.mark.gpu


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g) * scale


# ---------------------------------------------------------------------------------------------
# fp32 path (the single-conv fp32 workload)
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("layout", ["NCTHW", "NTHWC"])
@pytest.mark.parametrize("Th", [0, 1, 2])
def test_fp32_single_conv(layout, Th):
    log(f"fp32 conv layout={layout} Th={Th}")
    cfg = wl.single_conv_fp32()
    x, w, b = cfg["x"], cfg["weight"], cfg["bias"]
    hist = _rand((1, 16, Th, 16, 16), 11) if Th else None
    ref = oracle.causal_conv3d(x[0], w, b, None if hist is None else hist[0])
    dev = lambda t: (t.contiguous() if layout == "NCTHW" else t.permute(0, 2, 3, 4, 1).contiguous()).cuda()
    xd, wd, bd = dev(x), w.contiguous().cuda(), b.cuda()
    hd = dev(hist) if hist is not None else None
    hout = None
    if layout == "NTHWC":
        hout = torch.empty((1, 2, 16, 16, 16), device="cuda")
    y = wvd.causal_conv3d(xd, wd, 16, bias=bd, hist=hd, hist_out=hout, layout=layout)
    torch.cuda.synchronize()
    got = y[0].cpu().numpy() if layout == "NCTHW" else y[0].cpu().permute(3, 0, 1, 2).numpy()
    assert got.shape == ref.shape
    err = float(np.abs(got - ref).max())
    log(f"  max abs err {err:.3e}")
    assert err <= 1e-4
    if hout is not None:
        assert torch.equal(hout.cpu(), xd[:, -2:].cpu())


# ---------------------------------------------------------------------------------------------
# bf16 matrix-core conv
# ---------------------------------------------------------------------------------------------
CONV_CASES = [
    # Ci, Co, T, H, W, kernel, Th
    (96, 96, 3, 13, 17, (3, 3, 3), 2),
    (384, 384, 2, 9, 11, (3, 3, 3), 1),
    (48, 384, 3, 7, 9, (3, 3, 3), 0),     # conv_in: a partial 32-channel chunk
    (192, 96, 2, 11, 21, (3, 3, 3), 2),
    (384, 192, 2, 10, 13, (3, 3, 3), 0),
    (96, 32, 3, 12, 37, (3, 3, 3), 1),    # a narrow output (one 32-channel block)
    (64, 64, 2, 5, 7, (3, 3, 3), 2),
    (384, 192, 3, 9, 10, (1, 1, 1), 0),   # residual-block shortcut
    (192, 384, 4, 6, 9, (3, 1, 1), 2),    # time conv, plain layout
    (96, 96, 1, 3, 3, (1, 3, 3), 0),      # a per-frame 2-D conv, tiny
    (1024, 1024, 2, 9, 13, (3, 3, 3), 2), # the real topology's width: 11 channel tiles, the last partial
    (1024, 512, 2, 5, 7, (1, 1, 1), 0),   # its shortcut (128-wide linear tiles)
    (256, 12, 2, 7, 9, (3, 3, 3), 2),     # its 12-channel head (32-wide halo tiles)
]


@pytest.mark.parametrize("case", CONV_CASES, ids=lambda c: "x".join(map(str, c[:5])) + f"_k{''.join(map(str, c[5]))}_h{c[6]}")
def test_bf16_conv_matches_oracle(case):
    Ci, Co, T, H, W, k, Th = case
    log(f"bf16 conv {case}")
    seed = Ci * 7 + Co * 3 + T * 11 + H * 13 + W * 17 + Th
    x = wl.bf16_values(_rand((1, Ci, T, H, W), seed))
    w = wl.bf16_values(wl.kaiming(torch.Generator().manual_seed(seed + 1), (Co, Ci) + k))
    b = 0.1 * _rand((Co,), seed + 2)
    hist = wl.bf16_values(_rand((1, Ci, Th, H, W), seed + 3)) if Th else None
    ref = oracle.causal_conv3d(x[0], w, b, None if hist is None else hist[0])
    y = wvd.causal_conv3d(to_dev_nthwc(x), wvd.conv_pack(w.cuda()), Co, kernel=k, bias=b.cuda(),
                          hist=None if hist is None else to_dev_nthwc(hist))
    torch.cuda.synchronize()
    got = from_dev_nthwc(y)
    ok, worst = bf16_elementwise_ok(got, ref)
    log(f"  rel {rel_max(got, ref):.3e} worst/bound {worst:.3f}")
    assert ok, worst


SPATIAL3_CASES = [c for c in CONV_CASES if c[5][1:] == (3, 3)]


@pytest.mark.parametrize("case", SPATIAL3_CASES, ids=lambda c: "x".join(map(str, c[:5])) + f"_k{''.join(map(str, c[5]))}_h{c[6]}")
def test_bf16_conv_every_config_matches_oracle(case):
    """Every kernel configuration (linear tiles and halo tiles), forced, on ragged 3x3-tap convs."""
    Ci, Co, T, H, W, k, Th = case
    seed = Ci * 5 + Co * 7 + T * 3 + H * 19 + W * 23 + Th
    x = wl.bf16_values(_rand((1, Ci, T, H, W), seed))
    w = wl.bf16_values(wl.kaiming(torch.Generator().manual_seed(seed + 1), (Co, Ci) + k))
    b = 0.1 * _rand((Co,), seed + 2)
    hist = wl.bf16_values(_rand((1, Ci, Th, H, W), seed + 3)) if Th else None
    ref = oracle.causal_conv3d(x[0], w, b, None if hist is None else hist[0])
    xd, wp, bd = to_dev_nthwc(x), wvd.conv_pack(w.cuda()), b.cuda()
    hd = None if hist is None else to_dev_nthwc(hist)
    names = wvd.conv_config_names()
    assert any(n.startswith("conv_halo") for n in names)
    ran = 0
    try:
        for i, name in enumerate(names):
            log(f"bf16 conv {case} forced {name}")
            wvd.conv_force_config(i)
            try:
                y = wvd.causal_conv3d(xd, wp, Co, kernel=k, bias=bd, hist=hd)
            except wvd.WvdError as e:
                # (phase tiles, the fused tail, which runs only with the head attached, and the GEMM
                # tiles, which take convs without spatial taps only)
                assert e.status == 8 and name.startswith(("conv_phase_halo", "conv_tail", "conv_gemm")), (name, str(e))
                assert not (name.startswith("conv_gemm") and k[1:] == (1, 1)), (name, str(e))
                continue
            torch.cuda.synchronize()
            ok, worst = bf16_elementwise_ok(from_dev_nthwc(y), ref)
            assert ok, (name, worst)
            ran += 1
    finally:
        wvd.conv_force_config(None)
    tapless = k[1:] == (1, 1)
    assert ran == len([n for n in names if not n.startswith(("conv_phase_halo", "conv_tail"))
                       and (tapless or not n.startswith("conv_gemm"))])


GEMM_CASES = [
    # Ci, Co, T, H, W, kernel, Th, residual
    (384, 768, 2, 44, 78, (3, 1, 1), 2, False),  # the first level's time conv (a ragged last tile per frame)
    (192, 200, 3, 11, 13, (3, 1, 1), 1, True),   # a partial channel tile, one history frame, a residual
    (48, 256, 2, 7, 9, (1, 1, 1), 0, False),     # a partial 32-channel chunk (Ci 48)
    (1024, 512, 2, 5, 7, (1, 1, 1), 0, True),    # the real topology's shortcut width, a residual
    (96, 384, 1, 16, 16, (3, 1, 1), 2, False),   # one frame, its first two taps in the history; 256 positions
    (256, 128, 5, 3, 5, (3, 1, 1), 0, False),    # no history (the first frames' early taps read zeros), tiny frames
]


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: "x".join(map(str, c[:5])) + f"_k{''.join(map(str, c[5]))}_h{c[6]}"
                         + ("_res" if c[7] else ""))
def test_gemm_tiles_same_bits_as_linear_kernel(case):
    """The LDS-DMA GEMM tiles of the convs without spatial taps keep the linear kernel's K order and
    per-lane operand layout, so all three tile shapes (4 and 8 waves, 128 to 256 channels) give its
    bits; the automatic choice too; and against the oracle (below a size the oracle finishes
    quickly) the single-op bar."""
    Ci, Co, T, H, W, k, Th, with_res = case
    log(f"gemm tiles {case}")
    seed = Ci * 3 + Co * 5 + T * 7 + H * 11 + W * 13 + Th
    x = wl.bf16_values(_rand((1, Ci, T, H, W), seed))
    w = wl.bf16_values(wl.kaiming(torch.Generator().manual_seed(seed + 1), (Co, Ci) + k))
    b = 0.1 * _rand((Co,), seed + 2)
    hist = wl.bf16_values(_rand((1, Ci, Th, H, W), seed + 3)) if Th else None
    res = wl.bf16_values(_rand((1, Co, T, H, W), seed + 4)) if with_res else None
    xd, wp, bd = to_dev_nthwc(x), wvd.conv_pack(w.cuda()), b.cuda()
    hd = None if hist is None else to_dev_nthwc(hist)
    rd = None if res is None else to_dev_nthwc(res)
    names = wvd.conv_config_names()
    outs = {}
    try:
        for name in ("conv_mfma_n3_m1_w8", "conv_gemm_dma_n3_m2_w2x2", "conv_gemm_dma_n2_m2_w2x2",
                     "conv_gemm_dma_n4_m2_w4x2", None):
            wvd.conv_force_config(None if name is None else names.index(name))
            outs[name] = wvd.causal_conv3d(xd, wp, Co, kernel=k, bias=bd, hist=hd, residual=rd)
        torch.cuda.synchronize()
    finally:
        wvd.conv_force_config(None)
    base = outs["conv_mfma_n3_m1_w8"]
    for name, y in outs.items():
        assert torch.equal(y, base), name
    if not with_res and Ci * Co * k[0] * T * H * W < 1e9:
        ref = oracle.causal_conv3d(x[0], w, b, None if hist is None else hist[0])
        ok, worst = bf16_elementwise_ok(from_dev_nthwc(base), ref)
        assert ok, worst


@pytest.mark.parametrize("C,T,H,W", [(96, 2, 19, 37), (192, 1, 9, 40), (384, 2, 5, 7)])
def test_spatial_upsample_every_config_matches_oracle(C, T, H, W):
    """Nearest x2 + 3x3 conv as four phase convs, under every configuration that runs them.
    The phase weights are bf16 sums of up to four bf16 taps (a second rounding), so the bar is
    the per-layer normwise one; all configurations share the K order and agree bit for bit."""
    g = torch.Generator().manual_seed(C + 7 * H + W)
    x = wl.bf16_values(torch.randn((1, C, T, H, W), generator=g))
    w = wl.bf16_values(wl.kaiming(g, (C, C, 3, 3)))
    b = 0.1 * torch.randn((C,), generator=g)
    ref = oracle.spatial_upsample(x[0], w, b)
    xd, wp, bd = to_dev_nthwc(x), wvd.conv_pack(w.cuda(), wvd.WVD_PACK_PHASE2X), b.cuda()
    auto = wvd.upsample(xd, spatial=wp, spatial_bias=bd)
    torch.cuda.synchronize()
    r = rel_max(from_dev_nthwc(auto), ref)
    log(f"spatial upsample C={C} rel {r:.3e}")
    assert r <= 2e-2
    ran = []
    try:
        for i, name in enumerate(wvd.conv_config_names()):
            wvd.conv_force_config(i)
            try:
                y = wvd.upsample(xd, spatial=wp, spatial_bias=bd)
            except wvd.WvdError as e:
                # (3x3 halo tiles; the fused tail and the shortcut-product tile, which run only
                # with the head or the shortcut attached; the GEMM tiles of convs without spatial taps)
                assert e.status == 8 and name.startswith(("conv_halo", "conv_tail", "conv_phase_halo_dma_sc",
                                                          "conv_gemm")), (name, str(e))
                continue
            torch.cuda.synchronize()
            assert torch.equal(y, auto), name
            ran.append(name)
    finally:
        wvd.conv_force_config(None)
    assert any(n.startswith("conv_phase_halo") for n in ran)


def test_forced_halo_config_rejects_other_taps():
    x = to_dev_nthwc(wl.bf16_values(_rand((1, 96, 2, 5, 6), 41)))
    wp = wvd.conv_pack(wl.kaiming(torch.Generator().manual_seed(42), (96, 96, 3, 1, 1)).cuda())
    try:
        wvd.conv_force_config("conv_halo_n3_m2_w8")
        with pytest.raises(wvd.WvdError):
            wvd.causal_conv3d(x, wp, 96, kernel=(3, 1, 1))
    finally:
        wvd.conv_force_config(None)


def test_bf16_conv_residual_and_hist_out():
    Ci, Co, T, H, W = 96, 96, 3, 10, 12
    x = wl.bf16_values(_rand((1, Ci, T, H, W), 21))
    res = wl.bf16_values(_rand((1, Co, T, H, W), 22))
    w = wl.bf16_values(wl.kaiming(torch.Generator().manual_seed(23), (Co, Ci, 3, 3, 3)))
    hist = wl.bf16_values(_rand((1, Ci, 1, H, W), 24))
    ref = oracle.add(oracle.causal_conv3d(x[0], w, None, hist[0]), res[0])
    xd, hd = to_dev_nthwc(x), to_dev_nthwc(hist)
    hout = torch.empty((1, 2, H, W, Ci), dtype=torch.bfloat16, device="cuda")
    y = wvd.causal_conv3d(xd, wvd.conv_pack(w.cuda()), Co, hist=hd, residual=to_dev_nthwc(res), hist_out=hout)
    torch.cuda.synchronize()
    ok, worst = bf16_elementwise_ok(from_dev_nthwc(y), ref)
    assert ok, worst
    assert torch.equal(hout[:, :], xd[:, -2:])
    # a one-frame input keeps the old last history frame in front of it
    hout1 = torch.empty((1, 2, H, W, Ci), dtype=torch.bfloat16, device="cuda")
    wvd.causal_conv3d(xd[:, :1].contiguous(), wvd.conv_pack(w.cuda()), Co, hist=hd, hist_out=hout1)
    torch.cuda.synchronize()
    assert torch.equal(hout1[:, 0], hd[:, 0]) and torch.equal(hout1[:, 1], xd[:, 0])


WALK_CASES = [
    # Ci, Co, T, H, W, Th: 3x3x3 convs with enough tiles that 8 workgroups each walk several
    (96, 96, 3, 40, 70, 2),    # an odd number of K stages (3 chunks x 3 temporal taps)
    (64, 192, 2, 35, 66, 1),   # an even number of stages, two 96-channel tiles
    (48, 96, 2, 33, 40, 0),    # a partial 32-channel chunk
]


@pytest.mark.parametrize("case", WALK_CASES, ids=lambda c: "x".join(map(str, c)))
def test_conv_tile_walk_matches_one_tile_per_workgroup_and_oracle(case):
    """Halo-tile convs whose workgroups each walk a run of tiles (capped at 8 workgroups) give the
    same bits as the default launch, and match the oracle (with a residual added)."""
    Ci, Co, T, H, W, Th = case
    seed = Ci + 3 * Co + 5 * T + 7 * H + 11 * W + Th
    x = wl.bf16_values(_rand((1, Ci, T, H, W), seed))
    res = wl.bf16_values(_rand((1, Co, T, H, W), seed + 1))
    w = wl.bf16_values(wl.kaiming(torch.Generator().manual_seed(seed + 2), (Co, Ci, 3, 3, 3)))
    b = 0.1 * _rand((Co,), seed + 3)
    hist = wl.bf16_values(_rand((1, Ci, Th, H, W), seed + 4)) if Th else None
    ref = oracle.add(oracle.causal_conv3d(x[0], w, b, None if hist is None else hist[0]), res[0])
    xd, wp, bd, rd = to_dev_nthwc(x), wvd.conv_pack(w.cuda()), b.cuda(), to_dev_nthwc(res)
    hd = None if hist is None else to_dev_nthwc(hist)
    base = wvd.causal_conv3d(xd, wp, Co, bias=bd, hist=hd, residual=rd)
    try:
        for cap in (8, 16):
            log(f"conv tile walk {case} cap {cap}")
            wvd.conv_max_workgroups(cap)
            y = wvd.causal_conv3d(xd, wp, Co, bias=bd, hist=hd, residual=rd)
            torch.cuda.synchronize()
            assert torch.equal(y, base), cap
    finally:
        wvd.conv_max_workgroups(0)
    ok, worst = bf16_elementwise_ok(from_dev_nthwc(base), ref)
    assert ok, worst


def test_wide_channel_tiles_same_bits_as_96_wide():
    """256 output channels (a multiple of 128, not of 96) on a grid where the 128-wide halo tiles'
    rounds over the chip take no longer: the automatic choice takes them; the K order is that of
    the 96-wide tiles (compared with the oracle above, as is the forced 128-wide configuration on
    the ragged cases), so the bits are the same, with and without a residual, also with 8
    workgroups walking all tiles. The 128-wide configuration has no fused-norm form and refuses a
    norm."""
    Ci, Co, T, H, W = 256, 256, 2, 160, 320
    log(f"wide tiles {Ci}->{Co} {T}x{H}x{W}")
    x = to_dev_nthwc(wl.bf16_values(_rand((1, Ci, T, H, W), 91)))
    wp = wvd.conv_pack(wl.kaiming(torch.Generator().manual_seed(92), (Co, Ci, 3, 3, 3)).cuda())
    b = (0.1 * _rand((Co,), 93)).cuda()
    hd = to_dev_nthwc(wl.bf16_values(_rand((1, Ci, 2, H, W), 94)))
    rd = to_dev_nthwc(wl.bf16_values(_rand((1, Co, T, H, W), 96)))
    try:
        for res in (None, rd):
            wvd.timing_reset()
            wvd.timing_enable(True)
            y = wvd.causal_conv3d(x, wp, Co, bias=b, hist=hd, residual=res)
            torch.cuda.synchronize()
            wvd.timing_enable(False)
            assert list(wvd.timing_read()) == ["conv_halo_dma_n4_m2_w8"]
            wvd.conv_force_config("conv_halo_dma_n3_m2_w8")
            y3 = wvd.causal_conv3d(x, wp, Co, bias=b, hist=hd, residual=res)
            wvd.conv_force_config(None)
            wvd.conv_max_workgroups(8)
            yw = wvd.causal_conv3d(x, wp, Co, bias=b, hist=hd, residual=res)
            torch.cuda.synchronize()
            wvd.conv_max_workgroups(0)
            assert torch.equal(y, y3) and torch.equal(y, yw), res is None
        cfg = wl.resblock_bf16(seed=95, C=96, T=2, H=5, W=7)
        wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
        wvd.conv_force_config("conv_halo_dma_n4_m2_w8")
        with pytest.raises(wvd.WvdError):
            wvd.resblock(to_dev_nthwc(cfg["x"]), wts, 1e-6)
    finally:
        wvd.timing_enable(False)
        wvd.conv_force_config(None)
        wvd.conv_max_workgroups(0)


@pytest.mark.parametrize("C,T,H,W", [(96, 2, 21, 45), (192, 2, 18, 40), (384, 1, 11, 35)])
def test_upsample_tile_walk_matches_one_tile_per_workgroup(C, T, H, W):
    """The x2 phase convs (phases dealt as the fastest tile index) with 8 workgroups walking all
    tiles give the same bits as the default launch."""
    g = torch.Generator().manual_seed(5 * C + H)
    x = wl.bf16_values(torch.randn((1, C, T, H, W), generator=g))
    w = wl.bf16_values(wl.kaiming(g, (C, C, 3, 3)))
    b = 0.1 * torch.randn((C,), generator=g)
    xd, wp, bd = to_dev_nthwc(x), wvd.conv_pack(w.cuda(), wvd.WVD_PACK_PHASE2X), b.cuda()
    base = wvd.upsample(xd, spatial=wp, spatial_bias=bd)
    try:
        wvd.conv_max_workgroups(8)
        y = wvd.upsample(xd, spatial=wp, spatial_bias=bd)
        torch.cuda.synchronize()
    finally:
        wvd.conv_max_workgroups(0)
    assert torch.equal(y, base)
    r = rel_max(from_dev_nthwc(base), oracle.spatial_upsample(x[0], w, b))
    assert r <= 2e-2, r


def test_bf16_conv_chunked_equals_one_shot_bitwise():
    """Carrying the history between chunks gives the very same bits as one conv over all frames."""
    Ci, Co, T, H, W = 96, 96, 5, 9, 14
    x = to_dev_nthwc(_rand((1, Ci, T, H, W), 31))
    wp = wvd.conv_pack(wl.kaiming(torch.Generator().manual_seed(32), (Co, Ci, 3, 3, 3)).cuda())
    whole = wvd.causal_conv3d(x, wp, Co)
    for splits in ([1, 4], [2, 3], [1, 1, 1, 1, 1], [4, 1]):
        parts, start, hist = [], 0, None
        for n in splits:
            xc = x[:, start:start + n].contiguous()
            th = 0 if hist is None else hist.shape[1]
            hout = torch.empty((1, wvd.history_frames_after(n, th), H, W, Ci), dtype=torch.bfloat16, device="cuda")
            parts.append(wvd.causal_conv3d(xc, wp, Co, hist=hist, hist_out=hout))
            hist = hout
            start += n
        assert torch.equal(torch.cat(parts, dim=1), whole), splits


# ---------------------------------------------------------------------------------------------
# RMS norm + SiLU
# ---------------------------------------------------------------------------------------------
@pytest.mark.parametrize("C", [48, 96, 192, 384, 520, 1024, 1536, 2048])
def test_norm_silu_matches_oracle(C):
    """Up to 512 channels one 16-byte chunk per lane; beyond, two to four per lane."""
    log(f"norm C={C}")
    x = wl.bf16_values(_rand((1, C, 3, 7, 11), C) * 3.0)
    gamma = 1.0 + 0.1 * _rand((C,), C + 1)
    ref = oracle.silu(oracle.rms_norm(x[0], gamma, 1e-6))
    y = wvd.rmsnorm_silu(to_dev_nthwc(x), gamma.cuda(), 1e-6)
    torch.cuda.synchronize()
    ok, worst = bf16_elementwise_ok(from_dev_nthwc(y), ref, floor=1e-6)
    assert ok, worst
    # the norm alone (no SiLU)
    ref2 = oracle.rms_norm(x[0], gamma, 1e-6)
    y2 = wvd.rmsnorm_silu(to_dev_nthwc(x), gamma.cuda(), 1e-6, silu=False)
    torch.cuda.synchronize()
    ok, worst = bf16_elementwise_ok(from_dev_nthwc(y2), ref2, floor=1e-6)
    assert ok, worst


# ---------------------------------------------------------------------------------------------
# Residual block
# ---------------------------------------------------------------------------------------------
def test_resblock_given_history_matches_oracle():
    cfg = wl.resblock_bf16(seed=2, C=384, T=4, H=6, W=10)
    p = oracle.as_numpy_params(cfg["params"])
    ref = oracle.resblock(cfg["x"][0], p, "res", {}, 1e-6, given_hist=oracle._f32(cfg["hist"][0]))
    wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
    hd = to_dev_nthwc(cfg["hist"])
    y = wvd.resblock(to_dev_nthwc(cfg["x"]), wts, 1e-6, hist1=hd, hist2=hd)
    torch.cuda.synchronize()
    r = rel_max(from_dev_nthwc(y), ref)
    log(f"resblock rel {r:.3e}")
    assert r <= 2e-2


@pytest.mark.parametrize("C", [96, 192])
def test_resblock_widths_match_oracle(C):
    """Widths whose conv1 carries the second norm in its epilogue (one channel tile)."""
    cfg = wl.resblock_bf16(seed=20 + C, C=C, T=3, H=9, W=13)
    p = oracle.as_numpy_params(cfg["params"])
    ref = oracle.resblock(cfg["x"][0], p, "res", {}, 1e-6, given_hist=oracle._f32(cfg["hist"][0]))
    wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
    hd = to_dev_nthwc(cfg["hist"])
    y = wvd.resblock(to_dev_nthwc(cfg["x"]), wts, 1e-6, hist1=hd, hist2=hd)
    torch.cuda.synchronize()
    r = rel_max(from_dev_nthwc(y), ref)
    log(f"resblock C={C} rel {r:.3e}")
    assert r <= 2e-2


@pytest.mark.parametrize("C", [96, 192])
def test_resblock_halo_configs_match_oracle(C):
    """The halo-tile kernels with the fused norm (conv1) and the residual add (conv2)."""
    cfg = wl.resblock_bf16(seed=30 + C, C=C, T=3, H=19, W=45)
    p = oracle.as_numpy_params(cfg["params"])
    ref = oracle.resblock(cfg["x"][0], p, "res", {}, 1e-6, given_hist=oracle._f32(cfg["hist"][0]))
    wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
    hd = to_dev_nthwc(cfg["hist"])
    xd = to_dev_nthwc(cfg["x"])
    try:
        for name in ("conv_halo_n6_m1_w8", "conv_halo_n3_m2_w8", "conv_halo_dma_n6_m1_w8", "conv_halo_dma_n3_m2_w8"):
            if C > 96 and "n3_m2" in name:
                continue  # a 96-wide tile cannot hold a 192-channel norm
            wvd.conv_force_config(name)
            y = wvd.resblock(xd, wts, 1e-6, hist1=hd, hist2=hd)
            torch.cuda.synchronize()
            r = rel_max(from_dev_nthwc(y), ref)
            log(f"resblock C={C} {name} rel {r:.3e}")
            assert r <= 2e-2
    finally:
        wvd.conv_force_config(None)


def test_resblock_shortcut_and_histories_match_oracle():
    cfg = wl.resblock_bf16(seed=12, C=384, T=3, H=7, W=9, Cout=192, hist_frames=0)
    p = oracle.as_numpy_params(cfg["params"])
    h1 = wl.bf16_values(_rand((1, 384, 2, 7, 9), 13))
    h2 = wl.bf16_values(_rand((1, 192, 1, 7, 9), 14))
    x = oracle._f32(cfg["x"][0])
    a1 = oracle.norm_silu(x, p["res.norm1.gamma"], 1e-6)
    h = oracle.causal_conv3d(a1, p["res.conv1.weight"], p["res.conv1.bias"], h1[0].numpy())
    a2 = oracle.norm_silu(h, p["res.norm2.gamma"], 1e-6)
    h2o = oracle.causal_conv3d(a2, p["res.conv2.weight"], p["res.conv2.bias"], h2[0].numpy())
    ref = oracle.add(h2o, oracle.causal_conv3d(x, p["res.shortcut.weight"], p["res.shortcut.bias"]))
    wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
    o1 = torch.empty((1, 2, 7, 9, 384), dtype=torch.bfloat16, device="cuda")
    o2 = torch.empty((1, 2, 7, 9, 192), dtype=torch.bfloat16, device="cuda")
    y = wvd.resblock(to_dev_nthwc(cfg["x"]), wts, 1e-6, hist1=to_dev_nthwc(h1), hist2=to_dev_nthwc(h2), hist1_out=o1,
                     hist2_out=o2)
    torch.cuda.synchronize()
    r = rel_max(from_dev_nthwc(y), ref)
    log(f"resblock 384->192 rel {r:.3e}")
    assert r <= 2e-2
    # the saved histories are the activated conv inputs' last two frames
    a1_last = from_dev_nthwc(o1)
    assert rel_max(a1_last, a1[:, -2:]) <= 2e-2


@pytest.mark.parametrize("cout", [192, 160, 96])
def test_norm_shortcut_pass_same_bits_as_separate_passes(cout):
    """wvd_fuse_norm_shortcut: a 384 -> cout block's norm1 + SiLU and 1x1 shortcut from one read of
    its input give the same bits as the separate norm and 1x1 conv passes (several 256-position
    tiles and a ragged tail; product passes of 96 and 64 outputs; the activated input checked
    through conv1's saved history)."""
    cfg = wl.resblock_bf16(seed=15, C=384, T=3, H=19, W=45, Cout=cout, hist_frames=0)
    wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
    xd = to_dev_nthwc(cfg["x"])
    outs = {}
    try:
        for fused in (False, True):
            wvd.fuse_norm_shortcut(fused)
            o1 = torch.empty((1, 2, 19, 45, 384), dtype=torch.bfloat16, device="cuda")
            y = wvd.resblock(xd, wts, 1e-6, hist1_out=o1)
            torch.cuda.synchronize()
            outs[fused] = (y.clone(), o1.clone())
    finally:
        wvd.fuse_norm_shortcut(True)
    assert torch.equal(outs[True][1], outs[False][1])
    assert torch.equal(outs[True][0], outs[False][0])
    log(f"norm + shortcut pass 384 -> {cout}: same bits as the separate passes")


def test_full_channel_decoder_norm_shortcut_same_bits():
    """The decoder's 384 -> 192 block with norm1 and the shortcut in one pass (default) against
    the separate passes: the same video."""
    spec = wl.FULL_DECODER
    hw = (3, 5)
    z, params = wl.decoder_weights(spec, seed=51, latent_frames=2, latent_hw=hw)
    zd = z.to(torch.bfloat16).cuda()
    vids = {}
    try:
        for fused in (False, True):
            wvd.fuse_norm_shortcut(fused)
            dec = _gpu_decoder(spec, params, hw)
            vids[fused] = dec.decode(zd, frames_per_pass=1).clone()
            torch.cuda.synchronize()
    finally:
        wvd.fuse_norm_shortcut(True)
    assert torch.equal(vids[True], vids[False])


# ---------------------------------------------------------------------------------------------
# Upsampling
# ---------------------------------------------------------------------------------------------
def test_upsample_stage_spatial_first_matches_oracle():
    cfg = wl.upsample_stage_bf16(seed=3, C=192, T=3, H=10, W=14)
    p = {k: oracle._f32(v) for k, v in cfg.items() if k != "x"}
    ref = oracle.upsample_stage(cfg["x"][0], p)
    y = wvd.upsample(to_dev_nthwc(cfg["x"]), spatial=wvd.conv_pack(cfg["spatial.weight"].cuda(), wvd.WVD_PACK_PHASE2X),
                     spatial_bias=cfg["spatial.bias"].cuda(), temporal=wvd.conv_pack(cfg["time.weight"].cuda()),
                     temporal_bias=cfg["time.bias"].cuda(), order=wvd.WVD_SPATIAL_FIRST)
    torch.cuda.synchronize()
    got = from_dev_nthwc(y)
    assert got.shape == ref.shape == (192, 6, 20, 28)
    r = rel_max(got, ref)
    log(f"upsample stage rel {r:.3e}")
    assert r <= 2e-2


@pytest.mark.parametrize("first", [False, True])
def test_upsample_time_first_with_history(first):
    C, T, H, W = 96, 3, 9, 11
    x = wl.bf16_values(_rand((1, C, T, H, W), 41))
    ws = wl.bf16_values(wl.kaiming(torch.Generator().manual_seed(42), (C, C, 3, 3)))
    wt = wl.bf16_values(wl.kaiming(torch.Generator().manual_seed(43), (2 * C, C, 3, 1, 1)))
    bs, bt = 0.1 * _rand((C,), 44), 0.1 * _rand((2 * C,), 45)
    hist = None if first else wl.bf16_values(_rand((1, C, 2, H, W), 46))
    cache = {} if first else {"t": oracle._f32(hist[0])}
    xt = oracle.time_upsample_first(x[0], wt, bt, cache, "t") if first else oracle.time_upsample(x[0], wt, bt, cache, "t")
    ref = oracle.spatial_upsample(xt, ws, bs)
    hout = torch.empty((1, 2, H, W, C), dtype=torch.bfloat16, device="cuda")
    y = wvd.upsample(to_dev_nthwc(x), spatial=wvd.conv_pack(ws.cuda(), wvd.WVD_PACK_PHASE2X), spatial_bias=bs.cuda(),
                     temporal=wvd.conv_pack(wt.cuda()), temporal_bias=bt.cuda(), order=wvd.WVD_TIME_FIRST, first=first,
                     time_hist=None if hist is None else to_dev_nthwc(hist), time_hist_out=hout)
    torch.cuda.synchronize()
    got = from_dev_nthwc(y)
    assert got.shape == ref.shape
    r = rel_max(got, ref)
    log(f"upsample time-first first={first} rel {r:.3e}")
    assert r <= 2e-2
    assert np.array_equal(from_dev_nthwc(hout), cache["t"])
    if first:  # frame 0 passes through, spatially upsampled only
        ref0 = oracle.spatial_upsample(x[0][:, :1], ws, bs)
        assert rel_max(got[:, :1], ref0) <= 2e-2


def test_empty_inputs_pass_histories_through():
    """Zero-frame inputs launch nothing, give empty outputs and leave every history as it was (a
    conv over no frames keeps its cache); a chunk after an empty one gives the same bits as
    without it. The history outputs start as NaN so that a missed copy shows."""
    log("empty inputs")
    C, H, W = 96, 9, 14
    nan = float("nan")
    x = to_dev_nthwc(_rand((1, C, 4, H, W), 81))
    empty = torch.empty((1, 0, H, W, C), dtype=torch.bfloat16, device="cuda")
    # conv
    wp = wvd.conv_pack(wl.kaiming(torch.Generator().manual_seed(82), (C, C, 3, 3, 3)).cuda())
    h1 = torch.empty((1, 2, H, W, C), dtype=torch.bfloat16, device="cuda")
    a = wvd.causal_conv3d(x[:, :2].contiguous(), wp, C, hist_out=h1)
    h2 = torch.full_like(h1, nan)
    e = wvd.causal_conv3d(empty, wp, C, hist=h1, hist_out=h2)
    b = wvd.causal_conv3d(x[:, 2:].contiguous(), wp, C, hist=h2)
    torch.cuda.synchronize()
    assert e.shape == (1, 0, H, W, C)
    assert torch.equal(h2, h1)
    assert torch.equal(torch.cat([a, b], 1), wvd.causal_conv3d(x, wp, C))
    # norm
    assert wvd.rmsnorm_silu(empty, torch.ones(C, device="cuda"), 1e-6).shape == (1, 0, H, W, C)
    # residual block: both convs' histories
    cfg = wl.resblock_bf16(seed=83, C=C, T=4, H=H, W=W)
    wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
    xr = to_dev_nthwc(cfg["x"])

    def res_chunks(parts):
        ys, g1, g2, start = [], None, None, 0
        for n in parts:
            t = wvd.history_frames_after(n, 0 if g1 is None else g1.shape[1])
            o1 = torch.full((1, t, H, W, C), nan, dtype=torch.bfloat16, device="cuda")
            o2 = torch.full_like(o1, nan)
            ys.append(wvd.resblock(xr[:, start:start + n].contiguous(), wts, 1e-6, hist1=g1, hist2=g2, hist1_out=o1,
                                   hist2_out=o2))
            g1, g2, start = o1, o2, start + n
        torch.cuda.synchronize()
        return torch.cat(ys, 1), g1, g2

    y0, a1, a2 = res_chunks([2, 2])
    y1, b1, b2 = res_chunks([2, 0, 2])
    assert torch.equal(y0, y1) and torch.equal(a1, b1) and torch.equal(a2, b2)
    # upsample with a time step (not the first chunk): the time conv's history
    wt = wvd.conv_pack(wl.kaiming(torch.Generator().manual_seed(84), (2 * C, C, 3, 1, 1)).cuda())
    wsp = wvd.conv_pack(wl.kaiming(torch.Generator().manual_seed(85), (C, C, 3, 3)).cuda(), wvd.WVD_PACK_PHASE2X)

    def up_chunks(parts):
        ys, g, start = [], None, 0
        for n in parts:
            o = torch.full((1, wvd.history_frames_after(n, 0 if g is None else g.shape[1]), H, W, C), nan,
                           dtype=torch.bfloat16, device="cuda")
            ys.append(wvd.upsample(x[:, start:start + n].contiguous(), spatial=wsp, temporal=wt,
                                   order=wvd.WVD_TIME_FIRST, time_hist=g, time_hist_out=o))
            g, start = o, start + n
        torch.cuda.synchronize()
        return torch.cat(ys, 1), g

    u0, g0 = up_chunks([2, 2])
    u1, g1 = up_chunks([2, 0, 2])
    assert u1.shape == (1, 8, 2 * H, 2 * W, C)
    assert torch.equal(u0, u1) and torch.equal(g0, g1)


# ---------------------------------------------------------------------------------------------
# Whole decodes at reduced size
# ---------------------------------------------------------------------------------------------
SMALL_GPU = wl.DecoderSpec(z_channels=16, base_channels=64, stage_channels=(64, 64, 32, 32))


def _gpu_decoder(spec, params, latent_hw):
    desc = wvd.make_desc(z_channels=spec.z_channels, base_channels=spec.base_channels,
                         stage_channels=spec.stage_channels, stage_temporal=spec.temporal,
                         mid_resblocks=spec.mid_resblocks, stage_resblocks=spec.stage_resblocks,
                         out_channels=spec.out_channels, eps=spec.eps, latent_h=latent_hw[0], latent_w=latent_hw[1])
    return wvd.Decoder(desc, params)


@pytest.mark.parametrize("rule", [True, False])
def test_small_decoder_matches_oracle_and_is_pass_size_invariant(rule):
    hw = (5, 7)
    z, params = wl.decoder_weights(SMALL_GPU, seed=50, latent_frames=3, latent_hw=hw)
    ref = oracle.decode(z[0], oracle.as_numpy_params(params), SMALL_GPU, frames_per_pass=3, first_frame_rule=rule)
    dec = _gpu_decoder(SMALL_GPU, params, hw)
    zd = z.to(torch.bfloat16).cuda()
    videos = [dec.decode(zd, frames_per_pass=f, first_frame_rule=rule) for f in (3, 1, 2)]
    # the same latents handed over channels-last ([1, T, h, w, C]): the same bits
    z_cl = zd.permute(0, 2, 3, 4, 1).contiguous()
    videos += [dec.decode(z_cl, frames_per_pass=f, first_frame_rule=rule, z_layout="NTHWC") for f in (3, 2)]
    torch.cuda.synchronize()
    for v in videos[1:]:
        assert torch.equal(v, videos[0])
    got = videos[0][0].float().cpu().numpy()
    assert got.shape == ref.shape
    q = psnr(got, ref)
    log(f"small decoder rule={rule} psnr {q:.2f} dB rel {rel_max(got, ref):.3e}")
    assert q >= 55.0


@pytest.mark.parametrize("rule", [True, False])
def test_small_decoder_per_level_pass_sizes_same_bits(rule):
    """Early stages over many latent frames per pass, the late ones in sub-passes
    (wvd_decode_chunk_split): the same bits as plain passes, for sub-passes that divide the chunk
    or not, with and without the first-frame rule."""
    hw = (5, 7)
    z, params = wl.decoder_weights(SMALL_GPU, seed=51, latent_frames=7, latent_hw=hw)
    dec = _gpu_decoder(SMALL_GPU, params, hw)
    zd = z.to(torch.bfloat16).cuda()
    base = dec.decode(zd, frames_per_pass=2, first_frame_rule=rule).clone()
    for fpp, early in ((2, 4), (2, 7), (1, 3), (3, 5), (2, 2)):
        log(f"split decode rule={rule} frames_per_pass={fpp} early={early}")
        v = dec.decode(zd, frames_per_pass=fpp, first_frame_rule=rule, early_frames_per_pass=early)
        torch.cuda.synchronize()
        assert torch.equal(v, base), (fpp, early)


# widths that reach every place the norm1 fusion applies: conv2 of up to 96 and of 97-192
# channels, and an x2 upsample of 128 channels (no time step) feeding a residual block
FUSE_GPU = wl.DecoderSpec(z_channels=16, base_channels=64, stage_channels=(64, 160, 128, 96))


@pytest.mark.parametrize("rule", [True, False])
def test_decoder_with_norm1_fused_matches_oracle_and_is_pass_size_invariant(rule):
    """wvd_decode_fuse_norm1: each block's norm1 + SiLU in the producing conv's epilogue (the
    previous conv2's, or the x2 upsample's, which then stores two outputs; the default) or a
    separate pass. Both against the oracle, each with the same bits for every pass size and
    per-level sub-passes, and within rounding of each other."""
    hw = (5, 7)
    z, params = wl.decoder_weights(FUSE_GPU, seed=52, latent_frames=3, latent_hw=hw)
    ref = oracle.decode(z[0], oracle.as_numpy_params(params), FUSE_GPU, frames_per_pass=3, first_frame_rule=rule)
    dec = _gpu_decoder(FUSE_GPU, params, hw)
    zd = z.to(torch.bfloat16).cuda()
    got = {}
    try:
        for fused in (False, True):
            wvd.decode_fuse_norm1(fused)
            videos = [dec.decode(zd, frames_per_pass=f, first_frame_rule=rule).clone() for f in (3, 1, 2)]
            videos.append(dec.decode(zd, frames_per_pass=1, first_frame_rule=rule, early_frames_per_pass=3))
            torch.cuda.synchronize()
            for v in videos[1:]:
                assert torch.equal(v, videos[0]), fused
            got[fused] = videos[0][0].float().cpu().numpy()
            log(f"norm1 {'fused' if fused else 'separate'} rule={rule}: psnr {psnr(got[fused], ref):.2f} dB vs oracle")
            assert psnr(got[fused], ref) >= 55.0
    finally:
        wvd.decode_fuse_norm1(True)
    assert not np.array_equal(got[True], got[False])  # the fused path did run
    assert psnr(got[True], got[False]) >= 55.0


# a 192 -> 96 stage change after a 192-channel x2 upsample with the dual store: the first block's
# shortcut in that upsample's epilogue (the full decoder's 176x312 -> 352x624 step)
SC_GPU = wl.DecoderSpec(z_channels=16, base_channels=64, stage_channels=(64, 64, 192, 96))


@pytest.mark.parametrize("rule,hw", [(True, (5, 7)), (False, (3, 9))])
def test_decoder_with_shortcut_in_upsample_matches_oracle_and_is_pass_size_invariant(rule, hw):
    """wvd_decode_fuse_shortcut: the 192 -> 96 block's 1x1 shortcut applied in the epilogue of the
    x2 upsample that produces its input (the default), or as its own pass. Both against the
    oracle, each with the same bits for every pass size and per-level sub-passes, within rounding
    of each other, and the fused launch seen in the timing records only when on."""
    z, params = wl.decoder_weights(SC_GPU, seed=56, latent_frames=3, latent_hw=hw)
    ref = oracle.decode(z[0], oracle.as_numpy_params(params), SC_GPU, frames_per_pass=3, first_frame_rule=rule)
    dec = _gpu_decoder(SC_GPU, params, hw)
    zd = z.to(torch.bfloat16).cuda()
    got = {}
    wvd.timing_enable(True)
    try:
        for fused in (False, True):
            wvd.decode_fuse_shortcut(fused)
            wvd.timing_reset()
            videos = [dec.decode(zd, frames_per_pass=f, first_frame_rule=rule).clone() for f in (3, 1, 2)]
            videos.append(dec.decode(zd, frames_per_pass=1, first_frame_rule=rule, early_frames_per_pass=3))
            torch.cuda.synchronize()
            ran = wvd.timing_read()
            assert ("conv_phase_halo_dma_sc_n6_m1_w8" in ran) == fused, sorted(ran)
            for v in videos[1:]:
                assert torch.equal(v, videos[0]), fused
            got[fused] = videos[0][0].float().cpu().numpy()
            log(f"shortcut {'in the upsample' if fused else 'separate'} rule={rule} hw={hw}: "
                f"psnr {psnr(got[fused], ref):.2f} dB vs oracle")
            assert psnr(got[fused], ref) >= 55.0
    finally:
        wvd.decode_fuse_shortcut(True)
        wvd.timing_enable(False)
    assert not np.array_equal(got[True], got[False])
    assert psnr(got[True], got[False]) >= 55.0


# last stages the fused tail kernel takes (65-96 channels, at most 3 colours)
TAIL_GPU = wl.DecoderSpec(z_channels=16, base_channels=64, stage_channels=(64, 64, 32, 96))
TAIL72_GPU = wl.DecoderSpec(z_channels=16, base_channels=64, stage_channels=(64, 64, 32, 72), out_channels=2)


@pytest.mark.parametrize("spec,rule,hw", [(TAIL_GPU, True, (5, 7)), (TAIL_GPU, False, (2, 9)),
                                          (TAIL72_GPU, True, (3, 4))], ids=["c96_rule", "c96", "c72_2colours"])
def test_fused_tail_matches_oracle_and_unfused_and_is_pass_size_invariant(spec, rule, hw):
    """wvd_decode_fuse_head: the last x2 upsample, norm_out + SiLU and the head in one kernel
    (the head's temporal taps carried between passes as partial sums) against the path through the
    activated tensor. Frame sizes that leave partial blocks (14 x 62 output pixels each) on both
    edges; each mode against the oracle, with the same bits for every pass size and per-level
    sub-passes (the carry), the two modes within rounding of each other."""
    z, params = wl.decoder_weights(spec, seed=55, latent_frames=4, latent_hw=hw)
    ref = oracle.decode(z[0], oracle.as_numpy_params(params), spec, frames_per_pass=4, first_frame_rule=rule)
    zd = z.to(torch.bfloat16).cuda()
    got = {}
    try:
        for fused in (False, True):
            wvd.decode_fuse_head(fused)
            dec = _gpu_decoder(spec, params, hw)  # (its cache and workspace follow the switch)
            wvd.timing_reset()
            wvd.timing_enable(True)
            videos = [dec.decode(zd, frames_per_pass=f, first_frame_rule=rule).clone() for f in (4, 1, 3)]
            videos.append(dec.decode(zd, frames_per_pass=1, first_frame_rule=rule, early_frames_per_pass=4))
            torch.cuda.synchronize()
            wvd.timing_enable(False)
            ran = "conv_tail_phase_head_n3_m1_w8" in wvd.timing_read()
            assert ran == fused
            for v in videos[1:]:
                assert torch.equal(v, videos[0]), fused
            got[fused] = videos[0][0].float().cpu().numpy()
            assert got[fused].shape == ref.shape
            q = psnr(got[fused], ref)
            log(f"tail {'fused' if fused else 'through memory'} {spec.stage_channels[-1]} ch rule={rule} {hw}: "
                f"psnr {q:.2f} dB vs oracle, rel {rel_max(got[fused], ref):.3e}")
            assert q >= 55.0
    finally:
        wvd.decode_fuse_head(False)
        wvd.timing_enable(False)
    assert not np.array_equal(got[True], got[False])
    assert psnr(got[True], got[False]) >= 55.0


WIDE_TAIL_GPU = wl.DecoderSpec(z_channels=16, base_channels=64, stage_channels=(64, 64, 32, 224))


MID_TAIL_GPU = wl.DecoderSpec(z_channels=16, base_channels=64, stage_channels=(64, 64, 32, 160))


@pytest.mark.parametrize("spec", [WIDE_TAIL_GPU, MID_TAIL_GPU], ids=["tail224", "tail160"])
def test_wide_last_stage_decoder_matches_oracle(spec):
    """Last stages wider than the input-stationary head takes (96 channels): 160 channels run
    the frame-tiled fused head; 224 channels, wider than one fused-epilogue tile, run norm_out as
    its own pass and the head as the tap-plane conv + stencil kernels (the fused paths' fallbacks)."""
    hw = (2, 3)
    z, params = wl.decoder_weights(spec, seed=54, latent_frames=3, latent_hw=hw)
    ref = oracle.decode(z[0], oracle.as_numpy_params(params), spec, frames_per_pass=3)
    dec = _gpu_decoder(spec, params, hw)
    zd = z.to(torch.bfloat16).cuda()
    v3 = dec.decode(zd, frames_per_pass=3)
    v1 = dec.decode(zd, frames_per_pass=1)
    torch.cuda.synchronize()
    assert torch.equal(v1, v3)
    got = v3[0].float().cpu().numpy()
    assert got.shape == ref.shape
    q = psnr(got, ref)
    log(f"wide-tail decoder {spec.stage_channels} psnr {q:.2f} dB")
    assert q >= 55.0


def test_full_channel_decoder_small_latent_matches_oracle():
    spec = wl.FULL_DECODER
    hw = (3, 5)
    z, params = wl.decoder_weights(spec, seed=51, latent_frames=2, latent_hw=hw)
    ref = oracle.decode(z[0], oracle.as_numpy_params(params), spec, frames_per_pass=2)
    dec = _gpu_decoder(spec, params, hw)
    v = dec.decode(z.to(torch.bfloat16).cuda(), frames_per_pass=1)
    torch.cuda.synchronize()
    got = v[0].float().cpu().numpy()
    assert got.shape == ref.shape == (3, 5, 48, 80)
    q = psnr(got, ref)
    log(f"full-channel decoder psnr {q:.2f} dB")
    assert q >= 55.0


def test_decoder_causality_and_independence_on_gpu():
    hw = (4, 6)
    z, params = wl.decoder_weights(SMALL_GPU, seed=52, latent_frames=4, latent_hw=hw)
    dec = _gpu_decoder(SMALL_GPU, params, hw)
    zd = z.to(torch.bfloat16).cuda()
    base = dec.decode(zd, frames_per_pass=2).clone()
    other = wl.streaming_latents(seed=53, latent_frames=3, spec=SMALL_GPU, latent_hw=hw).to(torch.bfloat16).cuda()
    dec.decode(other, frames_per_pass=3)
    again = dec.decode(zd, frames_per_pass=2)
    assert torch.equal(again, base)
    for k in (1, 3):
        z2 = zd.clone()
        z2[:, :, k] += 1.0
        v2 = dec.decode(z2, frames_per_pass=2)
        keep = 4 * k - 3
        assert torch.equal(v2[:, :, :keep], base[:, :, :keep])
        assert not torch.equal(v2[:, :, keep], base[:, :, keep])
