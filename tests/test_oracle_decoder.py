"""Pins of the oracle's decoder composition: the page's frame counts, chunked == one-shot, video
causality, and the composition against torch float64 library ops (CPU)."""
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "frame_counts.txt")
SMALL = wl.DecoderSpec(z_channels=4, base_channels=8, stage_channels=(8, 8, 4, 4))
TINY = wl.DecoderSpec(z_channels=2, base_channels=2, stage_channels=(2, 2, 2, 2), mid_resblocks=1,
                      stage_resblocks=1)


def _small(seed=40, T=5, hw=(3, 4), spec=SMALL):
    z, p = wl.decoder_weights(spec, seed=seed, latent_frames=T, latent_hw=hw)
    return oracle._f32(z[0]), oracle.as_numpy_params(p)


def _golden_counts():
    rows = []
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            t, f = line.split()
            rows.append((int(t), int(f)))
    return rows


def test_frame_counts_match_the_pages():
    rows = _golden_counts()
    assert len(rows) >= 8
    for T, frames in rows:
        z, p = _small(seed=41, T=T, hw=(1, 1), spec=TINY)
        y = oracle.decode(z, p, TINY, frames_per_pass=4)
        assert y.shape == (3, frames, 16, 16), (T, y.shape)


def test_one_pass_without_first_frame_rule_quadruples_frames():
    z, p = _small(T=4)
    y = oracle.decode(z, p, SMALL, frames_per_pass=4, first_frame_rule=False)
    assert y.shape == (3, 16, 48, 64)


@pytest.mark.parametrize("rule", [True, False])
def test_chunked_equals_one_shot_bitwise_for_every_pass_size(rule):
    z, p = _small(T=5)
    whole = oracle.decode(z, p, SMALL, frames_per_pass=5, first_frame_rule=rule)
    for fpp in (1, 2, 3, 4):
        assert np.array_equal(oracle.decode(z, p, SMALL, frames_per_pass=fpp, first_frame_rule=rule), whole), fpp


def test_video_causality():
    z, p = _small(T=4)
    y = oracle.decode(z, p, SMALL, frames_per_pass=2)
    for k in (1, 2, 3):
        z2 = z.copy()
        z2[:, k] += 1.0
        y2 = oracle.decode(z2, p, SMALL, frames_per_pass=2)
        # with the first-frame rule, video frame f depends on latents <= ceil(f / 4)
        unchanged = 4 * k - 3
        assert np.array_equal(y[:, :unchanged], y2[:, :unchanged])
        assert not np.array_equal(y[:, unchanged], y2[:, unchanged])


def test_decodes_are_independent():
    z, p = _small(T=2)
    first = oracle.decode(z, p, SMALL, frames_per_pass=1)
    oracle.decode(_small(seed=43, T=3)[0], p, SMALL, frames_per_pass=2)
    assert np.array_equal(oracle.decode(z, p, SMALL, frames_per_pass=1), first)


# ---- the composition against torch float64 library ops (one-shot form of the decode) ----------
def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).double()


def _conv64(x, w, b):
    kt, kh, kw = w.shape[2:]
    xp = F.pad(x[None], [kw // 2, kw // 2, kh // 2, kh // 2, 2 * (kt // 2), 0])
    return F.conv3d(xp, _t(w), None if b is None else _t(b))[0]


def _norm_silu64(x, g, eps):
    y = x * _t(g)[:, None, None, None] / torch.sqrt((x * x).mean(dim=0, keepdim=True) + eps)
    return F.silu(y)


def _res64(x, p, pre, eps):
    h = _conv64(_norm_silu64(x, p[f"{pre}.norm1.gamma"], eps), p[f"{pre}.conv1.weight"], p[f"{pre}.conv1.bias"])
    h = _conv64(_norm_silu64(h, p[f"{pre}.norm2.gamma"], eps), p[f"{pre}.conv2.weight"], p[f"{pre}.conv2.bias"])
    sc = _conv64(x, p[f"{pre}.shortcut.weight"], p[f"{pre}.shortcut.bias"]) if f"{pre}.shortcut.weight" in p else x
    return h + sc


def _decode64(z, p, spec, rule):
    x = _conv64(_t(z), p["conv_in.weight"], p["conv_in.bias"])
    for i in range(spec.mid_resblocks):
        x = _res64(x, p, f"mid.{i}", spec.eps)
    for s in range(len(spec.stage_channels)):
        for j in range(spec.stage_resblocks):
            x = _res64(x, p, f"up.{s}.res.{j}", spec.eps)
        if spec.temporal[s]:
            C = x.shape[0]
            src = x[:, 1:] if rule else x
            y = _conv64(src, p[f"up.{s}.time.weight"], p[f"up.{s}.time.bias"])
            up = torch.stack([y[:C], y[C:]], dim=2).reshape(C, 2 * src.shape[1], *src.shape[2:])
            x = torch.cat([x[:, :1], up], dim=1) if rule else up
        u = F.interpolate(x.permute(1, 0, 2, 3), scale_factor=2.0, mode="nearest")
        x = F.conv2d(u, _t(p[f"up.{s}.spatial.weight"]), _t(p[f"up.{s}.spatial.bias"]), padding=1).permute(1, 0, 2, 3)
    x = _norm_silu64(x, p["norm_out.gamma"], spec.eps)
    return _conv64(x, p["conv_out.weight"], p["conv_out.bias"]).numpy()


@pytest.mark.parametrize("rule", [True, False])
def test_decoder_composition_matches_torch_float64(rule):
    z, p = _small(T=3)
    y = oracle.decode(z, p, SMALL, frames_per_pass=2, first_frame_rule=rule)
    ref = _decode64(z, p, SMALL, rule)
    assert y.shape == ref.shape
    assert np.abs(y - ref).max() <= 2e-5 * np.abs(ref).max()


def _conv64_hist(x, w, hist):
    """Causal conv with `hist` frames placed in front (zeros for the ones missing)."""
    kt, kh, kw = w.shape[2:]
    xp = torch.cat([_t(hist), x], 1)
    xp = F.pad(xp[None], [kw // 2, kw // 2, kh // 2, kh // 2, 2 * (kt // 2) - hist.shape[1], 0])
    return F.conv3d(xp, _t(w))[0]


def test_resblock_with_given_history_matches_torch_float64():
    eps = 1e-6
    cfg = wl.resblock_bf16(seed=45, C=6, T=3, H=5, W=4)
    p = oracle.as_numpy_params(cfg["params"])
    x, hist = oracle._f32(cfg["x"][0]), oracle._f32(cfg["hist"][0])
    y = oracle.resblock(x, p, "res", {}, eps, given_hist=hist)
    a1 = _norm_silu64(_t(x), p["res.norm1.gamma"], eps)
    h = _conv64_hist(a1, p["res.conv1.weight"], hist)
    a2 = _norm_silu64(h, p["res.norm2.gamma"], eps)
    h2 = _conv64_hist(a2, p["res.conv2.weight"], hist)
    ref = (h2 + _t(x)).numpy()
    assert y.shape == ref.shape
    assert np.abs(y - ref).max() <= 2e-5 * np.abs(ref).max()
    # a one-frame history: one zero frame in front of it
    y1 = oracle.resblock(x, p, "res", {}, eps, given_hist=hist[:, 1:])
    h = _conv64_hist(a1, p["res.conv1.weight"], hist[:, 1:])
    h2 = _conv64_hist(_norm_silu64(h, p["res.norm2.gamma"], eps), p["res.conv2.weight"], hist[:, 1:])
    assert np.abs(y1 - (h2 + _t(x)).numpy()).max() <= 2e-5 * np.abs(ref).max()


def test_resblock_shortcut_matches_torch_float64():
    eps = 1e-6
    cfg = wl.resblock_bf16(seed=46, C=8, T=3, H=5, W=6, Cout=4, hist_frames=0)
    p = oracle.as_numpy_params(cfg["params"])
    x = oracle._f32(cfg["x"][0])
    y = oracle.resblock(x, p, "res", {}, eps)
    ref = _res64(_t(x), p, "res", eps).numpy()
    assert y.shape == (4, 3, 5, 6)
    assert np.abs(y - ref).max() <= 2e-5 * np.abs(ref).max()
