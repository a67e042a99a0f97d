"""GPU test of wvd_resblock_noalloc, the residual block that takes no workspace argument (its
workspace is the library's built-in per-GPU scratch): through the C ABI, its outputs and
histories equal wvd_resblock's (a caller workspace, the same kernels) bit for bit, on two calls
in a row, the second with a smaller input and a channel change (so the second call runs on the
scratch the first one left behind)."""
import pytest
import torch

import causal_convolution_causalconv3d_amd as wvd
import workloads as wl
from gpu_util import log, to_dev_nthwc

pytestmark = pytest.mark.gpu


def _case(seed, C, Cout, T, H, W):
    cfg = wl.resblock_bf16(seed=seed, C=C, T=T, H=H, W=W, Cout=Cout)
    wts = wvd.pack_resblock(cfg["params"], "res", "cuda")
    x = to_dev_nthwc(cfg["x"])
    h1 = to_dev_nthwc(cfg["hist"])
    h2 = to_dev_nthwc(torch.randn((1, Cout, 2, H, W), generator=torch.Generator().manual_seed(seed + 100)))
    return wts, x, h1, h2


def _both(wts, x, h1, h2):
    _, T, H, W, _ = x.shape
    cin, cout = wts["cin"], wts["cout"]
    outs = []
    for fn in ("resblock", "resblock_noalloc"):
        y = torch.full((1, T, H, W, cout), float("nan"), dtype=torch.bfloat16, device="cuda")
        ho1 = torch.full((1, min(T, 2), H, W, cin), float("nan"), dtype=torch.bfloat16, device="cuda")
        ho2 = torch.full((1, min(T, 2), H, W, cout), float("nan"), dtype=torch.bfloat16, device="cuda")
        if fn == "resblock":
            wvd.resblock(x, wts, 1e-6, hist1=h1, hist2=h2, out=y, hist1_out=ho1, hist2_out=ho2)
        else:
            wvd.resblock_noalloc(x, wts, 1e-6, y, hist1=h1, hist2=h2, hist1_out=ho1, hist2_out=ho2)
        torch.cuda.synchronize()
        outs.append((y, ho1, ho2))
    return outs


def test_resblock_noalloc_matches_resblock_on_two_calls():
    # first call: the residual-block workload's size (384 channels, 4 frames of 44x78, 21.1 MB of
    # workspace); second call: smaller, with a 1x1x1 shortcut (96 -> 192 channels)
    for seed, C, Cout, T, H, W in ((2, 384, 384, 4, 44, 78), (12, 96, 192, 3, 20, 36)):
        log(f"resblock_noalloc vs resblock: C {C} -> {Cout}, T {T}, {H}x{W}")
        wts, x, h1, h2 = _case(seed, C, Cout, T, H, W)
        assert wvd.lib().wvd_resblock_workspace_bytes(C, Cout, T, H, W) <= wvd.lib().wvd_resblock_noalloc_max_bytes()
        (y_ref, a_ref, b_ref), (y, a, b) = _both(wts, x, h1, h2)
        assert bool(torch.isfinite(y_ref.float()).all())
        assert torch.equal(y, y_ref)
        assert torch.equal(a, a_ref) and torch.equal(b, b_ref)


def test_resblock_noalloc_refuses_an_input_beyond_its_scratch():
    wts, x, h1, h2 = _case(2, 384, 384, 8, 44, 78)
    y = torch.empty_like(x)
    with pytest.raises(wvd.WvdError) as e:
        wvd.resblock_noalloc(x, wts, 1e-6, y, hist1=h1, hist2=h2)
    assert "scratch" in str(e.value)
