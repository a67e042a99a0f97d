"""Pins of the oracle's parts of the real Wan2.2 topology (the FastVideo compare page's part list:
attention, DupUp3D, unpatchify, clamp, the L2 form of the RMS norm, post_quant_conv) and of a
small decoder built from them: hand values, closed forms, brute-force loops, torch float64
library ops, and the chunking invariants (CPU)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl

SMALL_REAL = wl.DecoderSpec(z_channels=4, base_channels=8, stage_channels=(8, 8, 4, 4), stage_resblocks=3,
                            out_channels=12, eps=1e-27, post_quant=True, mid_attention=True,
                            spatial=(True, True, True, False), dup=(True, True, True, False), patch=2, clamp=True,
                            norm_l2=True)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).double()


def test_real_topology_has_the_pages_110_parameters():
    names = [n for n, _, _ in wl.decoder_param_list(wl.REAL_DECODER)]
    assert len(names) == 110
    assert names[0] == "post_quant.weight" and names[-1] == "conv_out.bias"


def test_rms_norm_l2_hand_values_and_zero():
    x = np.array([[[[3.0]]], [[[4.0]]]], dtype=np.float32)  # C = 2, one position
    y = oracle.rms_norm_l2(x, np.array([1.0, 2.0], dtype=np.float32))
    assert np.allclose(y.ravel(), [3 / 5 * math.sqrt(2), 2 * 4 / 5 * math.sqrt(2)], rtol=1e-7)
    assert np.all(oracle.rms_norm_l2(np.zeros((3, 1, 2, 2), np.float32), np.ones(3, np.float32)) == 0)
    # equals gamma * x / sqrt(mean x^2) away from zero
    x = _rand((6, 2, 3, 4), 1)
    g = _rand((6,), 2)
    assert np.allclose(oracle.rms_norm_l2(x, g), oracle.rms_norm(x, g, 0.0), rtol=2e-6, atol=1e-6)


def _attn_params(C, seed, zero_q=False):
    g = torch.Generator().manual_seed(seed)
    p = {"a.norm.gamma": wl.gain(g, C).numpy(),
         "a.qkv.weight": wl.kaiming(g, (3 * C, C, 1, 1, 1)).numpy(),
         "a.qkv.bias": (0.1 * wl.randn(g, (3 * C,))).numpy(),
         "a.proj.weight": wl.kaiming(g, (C, C, 1, 1, 1)).numpy(),
         "a.proj.bias": (0.1 * wl.randn(g, (C,))).numpy()}
    if zero_q:
        p["a.qkv.weight"][:C] = 0
        p["a.qkv.bias"][:C] = 0
    return p


def test_attention_with_vanishing_queries_averages_the_values():
    C, T, H, W = 4, 2, 3, 5
    x = _rand((C, T, H, W), 3)
    p = _attn_params(C, 4, zero_q=True)
    y = oracle.attention(x, p, "a", 1e-6)
    # every score is 0: each query takes the plain mean of the frame's values
    n = oracle.rms_norm(x, p["a.norm.gamma"], 1e-6).astype(np.float64)
    wv = p["a.qkv.weight"][2 * C:, :, 0, 0, 0].astype(np.float64)
    v = np.einsum("oc,cthw->othw", wv, n) + p["a.qkv.bias"][2 * C:, None, None, None]
    mean_v = v.mean(axis=(2, 3), keepdims=True) * np.ones((1, 1, H, W))
    wp = p["a.proj.weight"][:, :, 0, 0, 0].astype(np.float64)
    ref = np.einsum("oc,cthw->othw", wp, mean_v) + p["a.proj.bias"][:, None, None, None] + x
    assert np.abs(y - ref).max() <= 1e-5 * np.abs(ref).max()


def test_attention_matches_scalar_loops():
    C, T, H, W = 2, 2, 2, 3
    x = _rand((C, T, H, W), 5)
    p = _attn_params(C, 6)
    y = oracle.attention(x, p, "a", 1e-6)
    n = oracle.rms_norm(x, p["a.norm.gamma"], 1e-6)
    wq, bq = p["a.qkv.weight"][:, :, 0, 0, 0], p["a.qkv.bias"]
    wp, bp = p["a.proj.weight"][:, :, 0, 0, 0], p["a.proj.bias"]
    pos = [(h, w) for h in range(H) for w in range(W)]
    for t in range(T):
        proj = {}
        for (h, w) in pos:
            proj[(h, w)] = [sum(float(wq[o, c]) * float(n[c, t, h, w]) for c in range(C)) + float(bq[o])
                            for o in range(3 * C)]
        for (h, w) in pos:
            q = proj[(h, w)][:C]
            scores = [sum(q[c] * proj[key][C + c] for c in range(C)) / math.sqrt(C) for key in pos]
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            tot = sum(e)
            o = [sum(e[k] / tot * proj[key][2 * C + c] for k, key in enumerate(pos)) for c in range(C)]
            for co in range(C):
                ref = sum(float(wp[co, c]) * o[c] for c in range(C)) + float(bp[co]) + float(x[co, t, h, w])
                assert abs(float(y[co, t, h, w]) - ref) <= 1e-5 * max(1.0, abs(ref))


def test_attention_matches_torch_sdpa_float64():
    C, T, H, W = 8, 2, 4, 5
    x = _rand((C, T, H, W), 7)
    p = _attn_params(C, 8)
    y = oracle.attention(x, p, "a", 0.0, l2=True)
    xt = _t(x)
    n = F.normalize(xt, dim=0) * math.sqrt(C) * _t(p["a.norm.gamma"])[:, None, None, None]
    qkv = torch.einsum("oc,cthw->othw", _t(p["a.qkv.weight"][:, :, 0, 0, 0]), n) + _t(p["a.qkv.bias"])[:, None, None, None]
    q, k, v = (qkv[i * C:(i + 1) * C].permute(1, 2, 3, 0).reshape(T, 1, H * W, C) for i in range(3))
    o = F.scaled_dot_product_attention(q, k, v).reshape(T, H, W, C).permute(3, 0, 1, 2)
    ref = torch.einsum("oc,cthw->othw", _t(p["a.proj.weight"][:, :, 0, 0, 0]), o) + _t(p["a.proj.bias"])[:, None, None, None] + xt
    assert np.abs(y - ref.numpy()).max() <= 1e-5 * float(ref.abs().max())


def test_attention_is_equivariant_to_position_permutations():
    C, T, H, W = 4, 2, 3, 4
    x = _rand((C, T, H, W), 9)
    p = _attn_params(C, 10)
    perm = np.random.default_rng(11).permutation(H * W)
    xp = x.reshape(C, T, H * W)[:, :, perm].reshape(C, T, H, W)
    y = oracle.attention(x, p, "a", 1e-6)
    yp = oracle.attention(xp, p, "a", 1e-6)
    assert np.abs(yp - y.reshape(C, T, H * W)[:, :, perm].reshape(C, T, H, W)).max() <= 1e-5 * np.abs(y).max()


def test_dup_up_ratio_8_is_nearest_x2_in_time_rows_and_columns():
    x = _rand((4, 3, 2, 3), 12)
    ref = np.repeat(np.repeat(np.repeat(x, 2, axis=1), 2, axis=2), 2, axis=3)
    assert np.array_equal(oracle.dup_up(x, 4, 2, first=False), ref)
    assert np.array_equal(oracle.dup_up(x, 4, 2, first=True), ref[:, 1:])


def test_dup_up_ratio_2_turns_channel_pairs_into_row_pairs():
    x = _rand((8, 2, 2, 3), 13)
    y = oracle.dup_up(x, 4, 1, first=False)
    assert y.shape == (4, 2, 4, 6)
    for c in range(4):
        for t in range(2):
            for yy in range(2):
                for xx in range(3):
                    for i in range(2):
                        for j in range(2):
                            assert y[c, t, 2 * yy + i, 2 * xx + j] == x[2 * c + i, t, yy, xx]
    assert np.array_equal(oracle.dup_up(x, 4, 1, first=True), y)  # one time copy: nothing dropped


@pytest.mark.parametrize("cin,cout,ft", [(4, 4, 2), (8, 4, 1), (8, 8, 1), (4, 2, 2), (2, 4, 1)])
def test_dup_up_matches_torch_repeat_interleave(cin, cout, ft):
    x = _rand((cin, 3, 2, 3), 14 + cin + cout + ft)
    t = torch.from_numpy(x)[None]
    r = cout * ft * 4 // cin
    d = t.repeat_interleave(r, dim=1).view(1, cout, ft, 2, 2, 3, 2, 3)
    d = d.permute(0, 1, 5, 2, 6, 3, 7, 4).reshape(1, cout, 3 * ft, 4, 6)[0].numpy()
    assert np.array_equal(oracle.dup_up(x, cout, ft, first=False), d)


def test_unpatchify_scalar_loops_and_inverse():
    x = _rand((12, 2, 3, 4), 15)
    v = oracle.unpatchify(x, 2)
    assert v.shape == (3, 2, 6, 8)
    for k in range(3):
        for f in range(2):
            for y in range(3):
                for xx in range(4):
                    for i in range(2):
                        for j in range(2):
                            assert v[k, f, 2 * y + i, 2 * xx + j] == x[4 * k + 2 * j + i, f, y, xx]
    # space-to-depth with the channel order (colour, column offset, row offset) undoes it
    back = v.reshape(3, 2, 3, 2, 4, 2).transpose(0, 5, 3, 1, 2, 4).reshape(12, 2, 3, 4)
    assert np.array_equal(back, x)
    assert np.array_equal(oracle.unpatchify(x, 1), x)


def test_clamp():
    x = np.array([-3.0, -1.0, -0.25, 0.0, 0.5, 1.0, 7.0], dtype=np.float32)
    assert np.array_equal(oracle.clamp(x), np.array([-1, -1, -0.25, 0, 0.5, 1, 1], dtype=np.float32))


def _small_real(seed=50, T=4, hw=(3, 4), spec=SMALL_REAL):
    z, p = wl.decoder_weights(spec, seed=seed, latent_frames=T, latent_hw=hw)
    return oracle._f32(z[0]), oracle.as_numpy_params(p)


def test_real_topology_frame_counts_and_size():
    z, p = _small_real(T=3)
    y = oracle.decode(z, p, SMALL_REAL, frames_per_pass=2)
    assert y.shape == (3, 4 * 3 - 3, 3 * 8 * 2, 4 * 8 * 2)
    assert np.abs(y).max() <= 1.0


@pytest.mark.parametrize("fpp", [1, 2, 3])
def test_real_topology_chunked_equals_one_shot_bitwise(fpp):
    z, p = _small_real(T=4)
    one = oracle.decode(z, p, SMALL_REAL, frames_per_pass=4)
    assert np.array_equal(oracle.decode(z, p, SMALL_REAL, frames_per_pass=fpp), one)


def test_real_topology_video_causality():
    z, p = _small_real(T=3)
    y = oracle.decode(z, p, SMALL_REAL, frames_per_pass=1)
    z2 = z.copy()
    z2[:, 2] += 1.0
    y2 = oracle.decode(z2, p, SMALL_REAL, frames_per_pass=1)
    assert np.array_equal(y[:, :5], y2[:, :5])  # latent frames 0, 1 -> video frames 0 .. 4
    assert not np.array_equal(y[:, 5:], y2[:, 5:])


# ---- the composition against torch float64 library ops (one-shot, without the clamp) ---------
def _conv64(x, w, b):
    kt, kh, kw = w.shape[2:]
    xp = F.pad(x[None], [kw // 2, kw // 2, kh // 2, kh // 2, 2 * (kt // 2), 0])
    return F.conv3d(xp, _t(w), None if b is None else _t(b))[0]


def _norm64(x, g):
    return F.normalize(x, dim=0) * math.sqrt(x.shape[0]) * _t(g)[:, None, None, None]


def _res64(x, p, pre):
    h = _conv64(F.silu(_norm64(x, p[f"{pre}.norm1.gamma"])), p[f"{pre}.conv1.weight"], p[f"{pre}.conv1.bias"])
    h = _conv64(F.silu(_norm64(h, p[f"{pre}.norm2.gamma"])), p[f"{pre}.conv2.weight"], p[f"{pre}.conv2.bias"])
    sc = _conv64(x, p[f"{pre}.shortcut.weight"], p[f"{pre}.shortcut.bias"]) if f"{pre}.shortcut.weight" in p else x
    return h + sc


def _attn64(x, p):
    C, T, H, W = x.shape
    n = _norm64(x, p["mid.attn.norm.gamma"])
    qkv = _conv64(n, p["mid.attn.qkv.weight"], p["mid.attn.qkv.bias"])
    q, k, v = (qkv[i * C:(i + 1) * C].permute(1, 2, 3, 0).reshape(T, 1, H * W, C) for i in range(3))
    o = F.scaled_dot_product_attention(q, k, v).reshape(T, H, W, C).permute(3, 0, 1, 2)
    return _conv64(o, p["mid.attn.proj.weight"], p["mid.attn.proj.bias"]) + x


def _decode64(z, p, spec):
    x = _conv64(_conv64(_t(z), p["post_quant.weight"], p["post_quant.bias"]), p["conv_in.weight"], p["conv_in.bias"])
    x = _res64(x, p, "mid.0")
    x = _attn64(x, p)
    x = _res64(x, p, "mid.1")
    for s, cs in enumerate(spec.stage_channels):
        block_input = x
        for j in range(spec.stage_resblocks):
            x = _res64(x, p, f"up.{s}.res.{j}")
        ft = 2 if spec.temporal[s] else 1
        if spec.temporal[s]:
            C = x.shape[0]
            y = _conv64(x[:, 1:], p[f"up.{s}.time.weight"], p[f"up.{s}.time.bias"])
            up = torch.stack([y[:C], y[C:]], dim=2).reshape(C, 2 * (x.shape[1] - 1), *x.shape[2:])
            x = torch.cat([x[:, :1], up], dim=1)
        if spec.spatial[s]:
            u = F.interpolate(x.permute(1, 0, 2, 3), scale_factor=2.0, mode="nearest-exact")
            x = F.conv2d(u, _t(p[f"up.{s}.spatial.weight"]), _t(p[f"up.{s}.spatial.bias"]), padding=1)
            x = x.permute(1, 0, 2, 3)
        if spec.dup[s]:
            cin, T, H, W = block_input.shape
            r = cs * ft * 4 // cin
            d = block_input.repeat_interleave(r, dim=0).view(cs, ft, 2, 2, T, H, W)
            d = d.permute(0, 4, 1, 5, 2, 6, 3).reshape(cs, T * ft, 2 * H, 2 * W)[:, ft - 1:]
            x = x + d
    x = F.silu(_norm64(x, p["norm_out.gamma"]))
    y = _conv64(x, p["conv_out.weight"], p["conv_out.bias"])
    c12, Fr, h, w = y.shape
    return y.view(3, 2, 2, Fr, h, w).permute(0, 3, 4, 2, 5, 1).reshape(3, Fr, 2 * h, 2 * w).numpy()


def test_real_decoder_composition_matches_torch_float64():
    spec = SMALL_REAL.__class__(**{**SMALL_REAL.__dict__, "clamp": False})
    z, p = _small_real(T=3, spec=spec)
    y = oracle.decode(z, p, spec, frames_per_pass=2)
    ref = _decode64(z, p, spec)
    assert y.shape == ref.shape
    assert np.abs(y - ref).max() <= 5e-5 * np.abs(ref).max()
    yc = oracle.decode(z, p, SMALL_REAL, frames_per_pass=2)
    assert np.array_equal(yc, np.clip(y, -1, 1))
