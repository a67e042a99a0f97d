"""GPU parity of the real Wan2.2 topology's parts (post_quant_conv, mid-block attention, DupUp3D,
stages without the spatial step, the 12-channel head with unpatchify and clamp) through the C
ABI, against the oracle on the same seeded inputs: small decoders over several passes (with and
without the first-frame rule, clamp on and off), the attention at the full 44x78 latent frame,
and the per-level pass sizes. Bars as in test_gpu_parity.py: PSNR >= 55 dB for whole decodes."""
import numpy as np
import pytest
import torch

import causal_convolution_causalconv3d_amd as wvd
import oracle
import workloads as wl
from gpu_util import log, psnr, rel_max

pytestmark = pytest.mark.gpu

# base channels a multiple of 32 and latent h*w a multiple of 8 (the attention's GEMM shapes)
SMALL_REAL_GPU = wl.DecoderSpec(z_channels=16, base_channels=64, stage_channels=(64, 64, 32, 16), stage_resblocks=3,
                                out_channels=12, eps=1e-27, post_quant=True, mid_attention=True,
                                spatial=(True, True, True, False), dup=(True, True, True, False), patch=2,
                                clamp=False, norm_l2=True)


def _spec(**kw):
    return SMALL_REAL_GPU.__class__(**{**SMALL_REAL_GPU.__dict__, **kw})


def _decoder(spec, params, hw):
    return wvd.Decoder(wvd.desc_from_spec(spec, latent_h=hw[0], latent_w=hw[1]), params)


@pytest.mark.parametrize("rule", [True, False])
def test_small_real_decoder_matches_oracle_and_is_pass_size_invariant(rule):
    spec = _spec()
    hw = (4, 6)
    z, params = wl.decoder_weights(spec, seed=60, latent_frames=3, latent_hw=hw)
    ref = oracle.decode(z[0], oracle.as_numpy_params(params), spec, frames_per_pass=3, first_frame_rule=rule)
    dec = _decoder(spec, params, hw)
    zd = z.to(torch.bfloat16).cuda()
    log(f"small real decoder rule={rule}")
    videos = [dec.decode(zd, frames_per_pass=f, first_frame_rule=rule) for f in (3, 1, 2)]
    torch.cuda.synchronize()
    for v in videos[1:]:
        assert torch.equal(v, videos[0])
    got = videos[0][0].float().cpu().numpy()
    assert got.shape == ref.shape == (3, 4 * 3 - 3 if rule else 12, 4 * 8 * 2, 6 * 8 * 2)
    q = psnr(got, ref)
    log(f"small real decoder rule={rule} psnr {q:.2f} dB rel {rel_max(got, ref):.3e}")
    assert q >= 55.0
    # the clamp is exact in bf16: the clamped decode is the unclamped one clipped to [-1, 1]
    # (random weights put most values far outside it, so an error bar on the clipped video
    # would measure the few pixels near the bounds, not the path)
    dec_c = _decoder(_spec(clamp=True), params, hw)
    vc = dec_c.decode(zd, frames_per_pass=2, first_frame_rule=rule)
    torch.cuda.synchronize()
    assert torch.equal(vc, videos[0].clamp(-1.0, 1.0))
    assert 0.0 < float((videos[0].abs() < 1).float().mean()) < 1.0


def test_dup_up_of_every_ratio_matches_oracle():
    """DupUp3D ratios 8 (nearest copies, time x2), 4 with time x2 (channel halving: the general
    gather), 4 without (nearest copies) and 2 (channel pairs to row pairs)."""
    spec = _spec(stage_channels=(64, 32, 32, 16), dup=(True, True, True, False), clamp=False)
    hw = (4, 6)
    z, params = wl.decoder_weights(spec, seed=63, latent_frames=3, latent_hw=hw)
    for rule in (True, False):
        ref = oracle.decode(z[0], oracle.as_numpy_params(params), spec, frames_per_pass=2, first_frame_rule=rule)
        dec = _decoder(spec, params, hw)
        got = dec.decode(z.to(torch.bfloat16).cuda(), frames_per_pass=2, first_frame_rule=rule)[0].float().cpu().numpy()
        q = psnr(got, ref)
        log(f"dup ratios rule={rule} psnr {q:.2f} dB")
        assert got.shape == ref.shape
        assert q >= 55.0


@pytest.mark.parametrize("rule", [True, False])
def test_small_real_decoder_per_level_pass_sizes_same_bits(rule):
    spec = _spec()
    hw = (4, 6)
    z, params = wl.decoder_weights(spec, seed=61, latent_frames=6, latent_hw=hw)
    dec = _decoder(spec, params, hw)
    zd = z.to(torch.bfloat16).cuda()
    base = dec.decode(zd, frames_per_pass=2, first_frame_rule=rule).clone()
    for fpp, early in ((2, 4), (1, 3), (2, 6)):
        log(f"real split decode rule={rule} frames_per_pass={fpp} early={early}")
        v = dec.decode(zd, frames_per_pass=fpp, first_frame_rule=rule, early_frames_per_pass=early)
        torch.cuda.synchronize()
        assert torch.equal(v, base), (fpp, early)


def test_attention_at_the_full_latent_frame_matches_oracle():
    """conv_in, one mid block, the attention over all 3,432 positions of a 44x78 frame (scores
    3432 x 3432, values 256 wide), the head; two latent frames in one pass."""
    spec = wl.DecoderSpec(z_channels=16, base_channels=256, stage_channels=(), temporal=(), mid_resblocks=1,
                          stage_resblocks=0, out_channels=12, eps=1e-27, post_quant=False, mid_attention=True,
                          spatial=(), dup=(), patch=2, clamp=False, norm_l2=True)
    hw = (44, 78)
    z, params = wl.decoder_weights(spec, seed=62, latent_frames=2, latent_hw=hw)
    ref = oracle.decode(z[0], oracle.as_numpy_params(params), spec, frames_per_pass=2, first_frame_rule=False)
    dec = _decoder(spec, params, hw)
    log("attention decoder 44x78, 256 channels")
    got = dec.decode(z.to(torch.bfloat16).cuda(), frames_per_pass=2, first_frame_rule=False)[0].float().cpu().numpy()
    assert got.shape == ref.shape == (3, 2, 88, 156)
    q = psnr(got, ref)
    log(f"attention decoder psnr {q:.2f} dB rel {rel_max(got, ref):.3e}")
    assert q >= 55.0


def _random_spec(rng):
    """A small decoder with random switches, kept inside the descriptor's bounds."""
    base = int(rng.choice([32, 64]))
    n_st = int(rng.integers(1, 4))
    chans, temporal, spatial, dup = [], [], [], []
    c = base
    for s in range(n_st):
        co = int(rng.choice([c, max(16, c // 2)]))
        sp = bool(rng.random() < 0.8) or s == 0
        t = sp and bool(rng.random() < 0.5)
        ft = 2 if t else 1
        d = sp and (co * ft * 4) % c == 0 and bool(rng.random() < 0.6)
        chans.append(co), temporal.append(t), spatial.append(sp), dup.append(d)
        c = co
    patch = int(rng.choice([1, 2]))
    return wl.DecoderSpec(z_channels=int(rng.choice([8, 16])), base_channels=base, stage_channels=tuple(chans),
                          temporal=tuple(temporal), mid_resblocks=int(rng.integers(1, 3)),
                          stage_resblocks=int(rng.integers(1, 3)), out_channels=3 * patch * patch, eps=1e-27,
                          post_quant=bool(rng.random() < 0.5), mid_attention=bool(rng.random() < 0.5),
                          spatial=tuple(spatial), dup=tuple(dup), patch=patch, clamp=False, norm_l2=True)


@pytest.mark.parametrize("seed", range(6))
def test_random_small_decoders_match_oracle(seed):
    """Seeded random topologies (stage counts, channel changes, time and spatial steps, DupUp3D,
    post_quant_conv, attention, patch 1 or 2) and random pass sizes: PSNR >= 55 dB against the
    oracle and the same bits for every pass size."""
    rng = np.random.default_rng(100 + seed)
    spec = _random_spec(rng)
    hw = (4, 6) if seed % 2 else (2, 4)
    T = int(rng.integers(2, 5))
    rule = bool(seed % 3)
    log(f"random decoder seed={seed} {spec} T={T} rule={rule}")
    z, params = wl.decoder_weights(spec, seed=200 + seed, latent_frames=T, latent_hw=hw)
    ref = oracle.decode(z[0], oracle.as_numpy_params(params), spec, frames_per_pass=T, first_frame_rule=rule)
    dec = _decoder(spec, params, hw)
    zd = z.to(torch.bfloat16).cuda()
    videos = [dec.decode(zd, frames_per_pass=f, first_frame_rule=rule) for f in (T, 1, 2)]
    torch.cuda.synchronize()
    for v in videos[1:]:
        assert torch.equal(v, videos[0])
    got = videos[0][0].float().cpu().numpy()
    assert got.shape == ref.shape
    q = psnr(got, ref)
    log(f"random decoder seed={seed} psnr {q:.2f} dB")
    assert q >= 55.0


@pytest.mark.parametrize("real", [False, True])
def test_decodes_are_independent_bitwise(real):
    """The same latents give the same bits after another clip (of another length, so the cache
    slots' halves end in another state) went through the same decoder (the pages' independence
    test)."""
    spec = _spec() if real else wl.DecoderSpec(z_channels=16, base_channels=64, stage_channels=(64, 64, 32, 32))
    hw = (4, 6)
    za, params = wl.decoder_weights(spec, seed=64, latent_frames=5, latent_hw=hw)
    zb, _ = wl.decoder_weights(spec, seed=65, latent_frames=4, latent_hw=hw)
    dec = _decoder(spec, params, hw)
    a1 = dec.decode(za.to(torch.bfloat16).cuda(), frames_per_pass=2).clone()
    dec.decode(zb[:, :, :3].to(torch.bfloat16).cuda(), frames_per_pass=2)
    a2 = dec.decode(za.to(torch.bfloat16).cuda(), frames_per_pass=2)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2)
