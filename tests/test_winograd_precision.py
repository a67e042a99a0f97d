"""Winograd F(2x2, 3x3) in space for the causal 3x3x3 conv, simulated on the CPU (no GPU, no
library code): the transform matrices are checked against the oracle's direct convolution in
float64 (exact up to rounding), and the precision of the GPU form (transformed inputs U and
weights V rounded to bf16, products summed in fp32) is measured against the oracle at the real
topology's channel counts. The per-layer bar is the one the GPU layers meet: max |y - ref| /
max |ref| <= 2e-2.

Matrices (F(2,3), cross-correlation; the page's decoder uses F(4x4, 3x3) for its up blocks,
"How the decoder got here", "The design"):
  B^T = [1 0 -1 0; 0 1 1 0; 0 -1 1 0; 0 1 0 -1], G = [1 0 0; .5 .5 .5; .5 -.5 .5; 0 0 1],
  A^T = [1 1 1 0; 0 1 -1 -1].
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl

BT = np.array([[1, 0, -1, 0], [0, 1, 1, 0], [0, -1, 1, 0], [0, 1, 0, -1]], dtype=np.float64)
G = np.array([[1, 0, 0], [0.5, 0.5, 0.5], [0.5, -0.5, 0.5], [0, 0, 1]], dtype=np.float64)
AT = np.array([[1, 1, 1, 0], [0, 1, -1, -1]], dtype=np.float64)


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def winograd_conv(x, w, hist=None, round_bf16=False):
    """Causal 3x3x3 conv of x [C, T, H, W] with w [Co, C, 3, 3, 3] (history frames hist
    [C, Th, H, W] before x, zeros before those), through F(2x2, 3x3) in space. With round_bf16,
    U and V are rounded to bf16 and the products summed in fp32, as the GPU form does."""
    C, T, H, W = x.shape
    Co = w.shape[0]
    Th = 0 if hist is None else hist.shape[1]
    frames = np.zeros((C, 2 + T, H, W), dtype=np.float64)  # frame j holds input frame j - 2
    if Th:
        frames[:, 2 - Th:2] = hist
    frames[:, 2:] = x
    tH, tW = (H + 1) // 2, (W + 1) // 2
    pad = np.zeros((C, 2 + T, 2 * tH + 2, 2 * tW + 2))
    pad[:, :, 1:H + 1, 1:W + 1] = frames
    # U[a, b, c, f, ty, tx] = (B^T d B)[a, b] with d the 4x4 tile at rows 2ty-1.., cols 2tx-1..
    d = np.stack([np.stack([pad[:, :, r:r + 2 * tH:2, s:s + 2 * tW:2] for s in range(4)], 0) for r in range(4)], 0)
    U = np.einsum("ar,rscfyx,bs->abcfyx", BT, d, BT)
    V = np.einsum("ar,ocirs,bs->aboci", G, w.astype(np.float64), G)  # [a, b, o, c, i]
    if round_bf16:
        U, V = bf16(U).astype(np.float64), bf16(V).astype(np.float64)
    M = np.zeros((4, 4, Co, T, tH, tW))
    for i in range(3):
        # tap i meets frame t - 2 + i, i.e. frames[t + i]
        M += np.einsum("aboc,abcfyx->abofyx", V[:, :, :, :, i], U[:, :, :, i:i + T])
    if round_bf16:
        M = M.astype(np.float32).astype(np.float64)
    Y = np.einsum("pa,abofyx,qb->ofypxq", AT, M, AT).reshape(Co, T, 2 * tH, 2 * tW)
    return Y[:, :, :H, :W]


def test_transforms_reproduce_the_direct_conv_in_float64():
    g = torch.Generator().manual_seed(71)
    for C, Co, T, H, W, Th in ((3, 2, 2, 5, 7, 0), (4, 3, 3, 6, 4, 2), (2, 5, 1, 3, 3, 1)):
        x = torch.randn((C, T, H, W), generator=g).double().numpy()
        w = torch.randn((Co, C, 3, 3, 3), generator=g).double().numpy()
        h = torch.randn((C, Th, H, W), generator=g).double().numpy() if Th else None
        ref = oracle.causal_conv3d(x, w, None, h)  # fp32 storage, double sums
        got = winograd_conv(x.astype(np.float32), w.astype(np.float32), None if h is None else h.astype(np.float32))
        assert np.abs(got - ref).max() <= 1e-5 * max(np.abs(ref).max(), 1.0), (C, Co, T, H, W, Th)


@pytest.mark.slow
@pytest.mark.parametrize("C,act", [(256, "silu"), (512, "silu"), (512, "normal")])
def test_bf16_transformed_operands_meet_the_layer_bar(C, act):
    """The GPU form's roundings (U and V in bf16, fp32 products) against the oracle's direct conv at
    the real topology's widths; the direct bf16 kernel's error (operands rounded once) is logged
    for comparison."""
    g = torch.Generator().manual_seed(72 + C)
    T, H, W = 2, 10, 12
    x = torch.randn((C, T, H, W), generator=g)
    hist = torch.randn((C, 2, H, W), generator=g)
    if act == "silu":
        x, hist = torch.nn.functional.silu(x), torch.nn.functional.silu(hist)
    w = wl.kaiming(g, (C, C, 3, 3, 3))
    xb, hb, wb = bf16(x.numpy()), bf16(hist.numpy()), bf16(w.numpy())
    ref = oracle.causal_conv3d(xb, wb, None, hb)
    got = winograd_conv(xb, wb, hb, round_bf16=True)
    scale = np.abs(ref).max()
    rel_max = np.abs(got - ref).max() / scale
    rel_rms = np.sqrt(((got - ref) ** 2).mean()) / np.sqrt((ref ** 2).mean())
    direct = bf16(ref)  # the direct kernel's one rounding of the output
    print(f"C={C} {act}: winograd rel max {rel_max:.3e}, rel rms {rel_rms:.3e}; direct output rounding rel max "
          f"{np.abs(direct - ref).max() / scale:.3e}")
    assert rel_max <= 2e-2
    assert rel_rms <= 1e-2
