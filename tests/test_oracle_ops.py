"""Pins of the oracle's single ops against library routines, closed forms and invariants (CPU)."""
import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).numpy()


def _torch_causal_conv64(x, w, b=None, hist=None):
    """torch float64 F.conv3d after explicit padding: a library routine, not the oracle's loop."""
    xt = torch.from_numpy(np.ascontiguousarray(x)).double()
    wt = torch.from_numpy(np.ascontiguousarray(w)).double()
    kt, kh, kw = wt.shape[2:]
    front = 2 * (kt // 2)
    if hist is not None and hist.shape[1] > 0:
        xt = torch.cat([torch.from_numpy(hist).double(), xt], dim=1)
        front -= hist.shape[1]
    xt = F.pad(xt, [kw // 2, kw // 2, kh // 2, kh // 2, front, 0])
    bt = None if b is None else torch.from_numpy(b).double()
    return F.conv3d(xt[None], wt, bt)[0].numpy()


def _scalar_conv(x, w, b, hist):
    """Brute force, one output element at a time, straight from the definition."""
    C, T, H, W = x.shape
    Co, _, kt, kh, kw = w.shape
    P = 2 * (kt // 2)
    Th = 0 if hist is None else hist.shape[1]

    def xt(c, u, h, ww):
        if h < 0 or h >= H or ww < 0 or ww >= W:
            return 0.0
        if u >= P:
            return float(x[c, u - P, h, ww])
        if u >= P - Th:
            return float(hist[c, u - (P - Th), h, ww])
        return 0.0

    y = np.zeros((Co, T, H, W))
    for o, t, h, ww in itertools.product(range(Co), range(T), range(H), range(W)):
        s = 0.0 if b is None else float(b[o])
        for c, i, j, k in itertools.product(range(C), range(kt), range(kh), range(kw)):
            s += float(w[o, c, i, j, k]) * xt(c, t + i, h + j - kh // 2, ww + k - kw // 2)
        y[o, t, h, ww] = s
    return y


@pytest.mark.parametrize("kt,kh,kw,Th", [(3, 3, 3, 0), (3, 3, 3, 1), (3, 3, 3, 2), (3, 1, 1, 2), (1, 3, 3, 0),
                                          (1, 1, 1, 0), (3, 1, 3, 1)])
def test_conv3d_matches_torch_float64(kt, kh, kw, Th):
    C, T, H, W, Co = 3, 4, 5, 7, 4
    x = _rand((C, T, H, W), 1)
    w = _rand((Co, C, kt, kh, kw), 2)
    b = _rand((Co,), 3)
    hist = _rand((C, Th, H, W), 4) if Th else None
    y = oracle.causal_conv3d(x, w, b, hist)
    ref = _torch_causal_conv64(x, w, b, hist)
    # the oracle sums in double and rounds once: within one fp32 rounding of the exact value
    assert np.abs(y - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max())
    assert y.dtype == np.float32 and y.shape == (Co, T, H, W)


def test_conv3d_matches_scalar_brute_force():
    x = _rand((2, 3, 4, 3), 5)
    w = _rand((2, 2, 3, 3, 3), 6)
    b = _rand((2,), 7)
    hist = _rand((2, 1, 4, 3), 8)
    y = oracle.causal_conv3d(x, w, b, hist)
    ref = _scalar_conv(x, w, b, hist)
    assert np.abs(y - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max())


def test_conv3d_delta_kernel_is_identity_bitwise():
    C = 5
    x = _rand((C, 4, 6, 9), 9)
    w = np.zeros((C, C, 3, 3, 3), np.float32)
    for c in range(C):
        w[c, c, 2, 1, 1] = 1.0  # tap (2,1,1) meets the current frame at the same position
    y = oracle.causal_conv3d(x, w, None, _rand((C, 2, 6, 9), 10))
    assert np.array_equal(y, x)


def test_conv3d_time_shift_with_history_and_zeros():
    C, T = 2, 5
    x = _rand((C, T, 4, 4), 11)
    hist = _rand((C, 1, 4, 4), 12)
    w = np.zeros((C, C, 3, 3, 3), np.float32)
    for c in range(C):
        w[c, c, 0, 1, 1] = 1.0  # tap 0 meets frame t-2
    y = oracle.causal_conv3d(x, w, None, hist)
    # padded sequence: [zero, hist0, x0, x1, ...]; y[t] = padded[t]
    assert np.all(y[:, 0] == 0)
    assert np.array_equal(y[:, 1], hist[:, 0])
    assert np.array_equal(y[:, 2:], x[:, :T - 2])
    w2 = np.zeros_like(w)
    for c in range(C):
        w2[c, c, 1, 1, 1] = 1.0  # tap 1 meets frame t-1
    y2 = oracle.causal_conv3d(x, w2, None, hist)
    assert np.array_equal(y2[:, 0], hist[:, 0]) and np.array_equal(y2[:, 1:], x[:, :T - 1])


def test_conv3d_row_and_column_shift_with_zero_padding():
    C = 2
    x = _rand((C, 2, 5, 6), 13)
    w = np.zeros((C, C, 3, 3, 3), np.float32)
    for c in range(C):
        w[c, c, 2, 0, 1] = 1.0  # row offset -1
    y = oracle.causal_conv3d(x, w, None)
    assert np.all(y[:, :, 0] == 0) and np.array_equal(y[:, :, 1:], x[:, :, :-1])
    w = np.zeros_like(w)
    for c in range(C):
        w[c, c, 2, 1, 2] = 1.0  # column offset +1
    y = oracle.causal_conv3d(x, w, None)
    assert np.all(y[:, :, :, -1] == 0) and np.array_equal(y[:, :, :, :-1], x[:, :, :, 1:])


def test_conv3d_weight_index_order():
    """A single nonzero weight W[o,c,i,j,k] moves channel c to channel o only."""
    x = _rand((3, 3, 4, 4), 14)
    w = np.zeros((2, 3, 3, 3, 3), np.float32)
    w[1, 2, 2, 1, 1] = 2.0
    y = oracle.causal_conv3d(x, w, np.array([0.5, -0.25], np.float32))
    assert np.all(y[0] == 0.5)
    assert np.array_equal(y[1], (2.0 * x[2].astype(np.float64) - 0.25).astype(np.float32))


def test_conv3d_linearity():
    x1, x2 = _rand((3, 3, 5, 5), 15), _rand((3, 3, 5, 5), 16)
    w = _rand((2, 3, 3, 3, 3), 17)
    a = 0.75
    lhs = oracle.causal_conv3d(a * x1 + x2, w)
    rhs = a * oracle.causal_conv3d(x1, w) + oracle.causal_conv3d(x2, w)
    assert np.abs(lhs - rhs).max() <= 1e-5 * np.abs(rhs).max()


@pytest.mark.parametrize("tp", [1, 2, 4])
def test_conv3d_causality(tp):
    x = _rand((3, 5, 4, 6), 18)
    w = _rand((2, 3, 3, 3, 3), 19)
    y = oracle.causal_conv3d(x, w)
    x2 = x.copy()
    x2[:, tp] += 1.0
    y2 = oracle.causal_conv3d(x2, w)
    assert np.array_equal(y[:, :tp], y2[:, :tp])
    assert not np.array_equal(y[:, tp], y2[:, tp])


def test_conv3d_rejects_bad_history():
    with pytest.raises(ValueError):
        oracle.causal_conv3d(_rand((2, 2, 3, 3), 1), _rand((2, 2, 3, 3, 3), 2), None, _rand((2, 3, 3, 3), 3))


def test_rms_norm_closed_form():
    # one position, C = 2, x = (3, 4): mean of squares 12.5
    x = np.array([3.0, 4.0], np.float32).reshape(2, 1, 1, 1)
    eps = 1e-6
    y = oracle.rms_norm(x, np.ones(2, np.float32), eps)
    r = 1.0 / math.sqrt(12.5 + eps)
    assert np.allclose(y.ravel(), [3 * r, 4 * r], rtol=1e-7, atol=0)
    # gains act per channel
    y2 = oracle.rms_norm(x, np.array([2.0, -0.5], np.float32), eps)
    assert np.allclose(y2.ravel(), [6 * r, -2 * r], rtol=1e-7, atol=0)


def test_rms_norm_mean_square_identity_and_scale_invariance():
    x = _rand((16, 3, 4, 5), 20)
    eps = 1e-6
    y = oracle.rms_norm(x, np.ones(16, np.float32), eps).astype(np.float64)
    m = (x.astype(np.float64) ** 2).mean(axis=0)
    assert np.allclose((y ** 2).mean(axis=0), m / (m + eps), rtol=1e-6)
    ys = oracle.rms_norm(8.0 * x, np.ones(16, np.float32), 0.0)
    y0 = oracle.rms_norm(x, np.ones(16, np.float32), 0.0)
    assert np.allclose(ys, y0, rtol=1e-6, atol=1e-7)


def test_rms_norm_normalizes_over_channels_not_positions():
    x = np.zeros((2, 1, 1, 2), np.float32)
    x[:, 0, 0, 0] = [1.0, 1.0]
    x[:, 0, 0, 1] = [10.0, 0.0]
    y = oracle.rms_norm(x, np.ones(2, np.float32), 0.0)
    assert np.allclose(y[:, 0, 0, 0], [1.0, 1.0])
    assert np.allclose(y[:, 0, 0, 1], [math.sqrt(2.0), 0.0])


def test_silu_identities():
    x = np.linspace(-30, 30, 1001).astype(np.float32)
    y = oracle.silu(x).astype(np.float64)
    xd = x.astype(np.float64)
    assert oracle.silu(np.zeros(3, np.float32)).tolist() == [0.0, 0.0, 0.0]
    assert np.allclose(y, 0.5 * xd * (1.0 + np.tanh(0.5 * xd)), rtol=1e-6, atol=1e-12)
    assert np.allclose(y - oracle.silu(-x).astype(np.float64), xd, rtol=1e-6, atol=1e-6)
    assert abs(y[-1] - 30.0) < 1e-6 and abs(y[0]) < 1e-11


def test_keep_frames_cases():
    a3 = _rand((2, 3, 2, 2), 21)
    a1 = _rand((2, 1, 2, 2), 22)
    assert oracle.keep_frames(None, a3).shape[1] == 2 and np.array_equal(oracle.keep_frames(None, a3), a3[:, 1:])
    assert np.array_equal(oracle.keep_frames(None, a1), a1)                    # no history: one frame
    k = oracle.keep_frames(a3[:, 1:], a1)
    assert np.array_equal(k, np.concatenate([a3[:, 2:], a1], axis=1))         # old last frame + new
    assert oracle.keep_frames(a3, a3[:, :0]) is a3                              # zero frames: unchanged


@pytest.mark.parametrize("splits", [[5], [1, 4], [2, 3], [1, 1, 1, 1, 1], [3, 2], [4, 1]])
def test_cached_conv_chunked_equals_one_shot(splits):
    x = _rand((3, 5, 4, 5), 23)
    w = _rand((2, 3, 3, 3, 3), 24)
    b = _rand((2,), 25)
    whole = oracle.causal_conv3d(x, w, b)
    cache = {}
    parts, s = [], 0
    for n in splits:
        parts.append(oracle.cached_conv(x[:, s:s + n], w, b, cache, "c"))
        s += n
    assert np.array_equal(np.concatenate(parts, axis=1), whole)


def test_time_upsample_channel_halves_to_even_and_odd_frames():
    C = 3
    x = _rand((C, 4, 3, 3), 26)
    w = np.zeros((2 * C, C, 3, 1, 1), np.float32)
    for c in range(C):
        w[c, c, 2] = 1.0          # first half: current frame
        w[C + c, c, 1] = -1.0     # second half: minus the previous frame
    y = oracle.time_upsample(x, w, None, {}, "t")
    assert y.shape == (C, 8, 3, 3)
    assert np.array_equal(y[:, 0::2], x)
    assert np.all(y[:, 1] == 0) and np.array_equal(y[:, 3::2], -x[:, :-1])


def test_time_upsample_first_frame_rule():
    C = 2
    x = _rand((C, 3, 2, 2), 27)
    w = _rand((2 * C, C, 3, 1, 1), 28)
    cache = {}
    y = oracle.time_upsample_first(x, w, None, cache, "t")
    assert y.shape[1] == 2 * 3 - 1
    assert np.array_equal(y[:, 0], x[:, 0])
    # the conv never sees frame 0: its output equals a fresh time conv of frames 1.. alone
    assert np.array_equal(y[:, 1:], oracle.time_upsample(x[:, 1:], w, None, {}, "t"))
    assert np.array_equal(cache["t"], x[:, 1:])
    # a one-frame first pass: the conv is skipped and its history stays empty
    cache = {}
    y1 = oracle.time_upsample_first(x[:, :1], w, None, cache, "t")
    assert np.array_equal(y1, x[:, :1]) and "t" not in cache


def test_spatial_upsample_matches_torch_float64():
    x = _rand((3, 2, 4, 5), 29)
    w = _rand((4, 3, 3, 3), 30)
    b = _rand((4,), 31)
    y = oracle.spatial_upsample(x, w, b)
    xt = torch.from_numpy(x).double().permute(1, 0, 2, 3)  # frames as batch
    u = F.interpolate(xt, scale_factor=2.0, mode="nearest-exact")
    ref = F.conv2d(u, torch.from_numpy(w).double(), torch.from_numpy(b).double(), padding=1).permute(1, 0, 2, 3)
    assert y.shape == (4, 2, 8, 10)
    assert np.abs(y - ref.numpy()).max() <= 1e-6 * np.abs(ref.numpy()).max()


def test_spatial_upsample_four_phase_identity():
    """Nearest x2 then 3x3 equals, per output parity (a, b), a 2x2 conv at low resolution whose
    taps are sums of the 3x3 taps (the kernel README's upsampler design)."""
    C, H, W = 2, 4, 5
    x = _rand((C, 1, H, W), 32)
    w = _rand((C, C, 3, 3), 33)
    y = oracle.spatial_upsample(x, w, None).astype(np.float64)
    xd = np.pad(x[:, 0].astype(np.float64), ((0, 0), (1, 1), (1, 1)))
    wd = w.astype(np.float64)
    # row taps of phase a: a=0 -> offsets (-1: r0, 0: r1+r2); a=1 -> (0: r0+r1, +1: r2)
    groups = {0: [(-1, [0]), (0, [1, 2])], 1: [(0, [0, 1]), (1, [2])]}
    for a, bb in itertools.product((0, 1), (0, 1)):
        out = np.zeros((C, H, W))
        for (dy, rs), (dx, cs) in itertools.product(groups[a], groups[bb]):
            wp = sum(wd[:, :, r, c] for r in rs for c in cs)
            patch = xd[:, 1 + dy:1 + dy + H, 1 + dx:1 + dx + W]
            out += np.einsum("oc,chw->ohw", wp, patch)
        assert np.abs(y[:, 0, a::2, bb::2] - out).max() <= 1e-5


def test_spatial_upsample_all_ones_kernel_on_constant():
    v = 1.5
    x = np.full((1, 1, 3, 4), v, np.float32)
    y = oracle.spatial_upsample(x, np.ones((1, 1, 3, 3), np.float32), None)[0, 0]
    assert y[3, 3] == 9 * v and y[0, 3] == 6 * v and y[3, 0] == 6 * v and y[0, 0] == 4 * v and y[-1, -1] == 4 * v


def test_upsample_stage_shape_and_order():
    C = 2
    x = _rand((C, 3, 2, 3), 34)
    p = {"spatial.weight": _rand((C, C, 3, 3), 35), "time.weight": _rand((2 * C, C, 3, 1, 1), 36)}
    y = oracle.upsample_stage(x, p)
    assert y.shape == (C, 6, 4, 6)
    ref = oracle.time_upsample(oracle.spatial_upsample(x, p["spatial.weight"], None), p["time.weight"], None, {}, "t")
    assert np.array_equal(y, ref)
