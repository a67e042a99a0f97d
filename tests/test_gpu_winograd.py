"""GPU parity of wvd_causal_conv3d_winograd (Winograd F(2x2, 3x3) in space, causal 3-tap time
conv) against the oracle's direct causal convolution, to the per-layer bar max |y - ref| /
max |ref| <= 2e-2 (the bf16 transformed operands cost about 4e-3, tests/test_winograd_precision.py):
odd frame sizes (partial 2x2 tiles), 0-2 history frames, ragged channel chunks, a residual,
one-frame inputs, the real topology's 512 channels, an empty input, and windows of a full-size
512-channel 176x312 layer against the oracle on the matching crops."""
import numpy as np
import pytest
import torch

import causal_convolution_causalconv3d_amd as wvd
import oracle
import workloads as wl
from gpu_util import from_dev_nthwc, log, rel_max, to_dev_nthwc

pytestmark = pytest.mark.gpu


def _case(seed, C, Co, T, H, W, Th, bias=True, residual=False):
    g = torch.Generator().manual_seed(seed)
    x = wl.bf16_values(torch.nn.functional.silu(torch.randn((1, C, T, H, W), generator=g)))
    h = wl.bf16_values(torch.randn((1, C, Th, H, W), generator=g)) if Th else None
    w = wl.bf16_values(wl.kaiming(g, (Co, C, 3, 3, 3)))
    b = 0.1 * torch.randn((Co,), generator=g) if bias else None
    r = wl.bf16_values(torch.randn((1, Co, T, H, W), generator=g)) if residual else None
    return x, h, w, b, r


@pytest.mark.parametrize("C,Co,T,H,W,Th,res", [
    (64, 32, 3, 9, 13, 2, False),    # odd height and width: partial tiles on both edges
    (48, 20, 2, 8, 10, 1, True),     # ragged 32-channel chunk, one history frame, residual
    (32, 64, 1, 7, 6, 2, False),     # one frame after a full history
    (32, 32, 4, 6, 6, 0, True),      # no history (causal zeros)
    (512, 512, 2, 12, 20, 2, False), # the real topology's 512-channel width
])
def test_winograd_conv_matches_oracle(C, Co, T, H, W, Th, res):
    x, h, w, b, r = _case(C + Co + T, C, Co, T, H, W, Th, residual=res)
    ref = oracle.causal_conv3d(x[0], w, b, None if h is None else h[0])
    if r is not None:
        ref = oracle.add(ref, r[0])
    wp = wvd.winograd_pack(w.cuda())
    y = wvd.causal_conv3d_winograd(to_dev_nthwc(x), wp, Co, bias=None if b is None else b.cuda(),
                                   hist=None if h is None else to_dev_nthwc(h),
                                   residual=None if r is None else to_dev_nthwc(r))
    torch.cuda.synchronize()
    got = from_dev_nthwc(y)
    # the direct kernel on the same inputs, for scale
    direct = from_dev_nthwc(wvd.causal_conv3d(to_dev_nthwc(x), wvd.conv_pack(w.cuda()), Co,
                                              bias=None if b is None else b.cuda(),
                                              hist=None if h is None else to_dev_nthwc(h),
                                              residual=None if r is None else to_dev_nthwc(r)))
    e, ed = rel_max(got, ref), rel_max(direct, ref)
    log(f"winograd C {C}->{Co} T {T} {H}x{W} hist {Th}: rel {e:.3e} (direct kernel {ed:.3e})")
    assert e <= 2e-2


def test_winograd_conv_empty_input():
    x = torch.empty((1, 0, 6, 6, 32), dtype=torch.bfloat16, device="cuda")
    w = torch.randn((32, 32, 3, 3, 3), device="cuda")
    y = wvd.causal_conv3d_winograd(x, wvd.winograd_pack(w), 32)
    assert tuple(y.shape) == (1, 0, 6, 6, 32)


def test_winograd_conv_full_size_windows():
    """A 512-channel 3x3x3 conv over 4 frames of 176x312 with a 2-frame history (the real
    topology's 512-channel level): windows against the oracle run on the matching input crop plus
    a one-pixel halo (the conv is translation-equivariant, and the Winograd tiling does not change
    the function)."""
    C = Co = 512
    T, H, W, Th = 4, 176, 312, 2
    x, h, w, b, _ = _case(7, C, Co, T, H, W, Th)
    y = wvd.causal_conv3d_winograd(to_dev_nthwc(x), wvd.winograd_pack(w.cuda()), Co, bias=b.cuda(),
                                   hist=to_dev_nthwc(h))
    torch.cuda.synchronize()
    S = 10
    for r0, c0 in ((0, 0), (H - S, W - S), (H // 2 + 1, W // 2 + 1), (0, W - S), (H - S, 1)):
        a0, a1 = max(r0 - 1, 0), min(r0 + S + 1, H)
        b0, b1 = max(c0 - 1, 0), min(c0 + S + 1, W)
        ref = oracle.causal_conv3d(x[0, :, :, a0:a1, b0:b1], w, b, h[0, :, :, a0:a1, b0:b1])
        ref = ref[:, :, r0 - a0:r0 - a0 + S, c0 - b0:c0 - b0 + S]
        got = y[0, :, r0:r0 + S, c0:c0 + S].float().cpu().permute(3, 0, 1, 2).numpy()
        e = rel_max(got, ref)
        log(f"winograd full size window ({r0},{c0}): rel {e:.3e}")
        assert e <= 2e-2
