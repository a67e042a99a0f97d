"""Writes tests/golden/real_decode_samples.npz: the oracle's decode of the Wan2.2 TI2V-5B topology
(random weights from seed 4 for 2 latent frames, latents [1,48,2,44,78] from the same draw) in two
passes of one latent frame with the first-frame rule, video [1,3,5,704,1248], at 32768 seeded
sample positions, plus the whole video's min / max / mean / mean square. The decode is taken
without the final clamp: with random weights most values lie far outside [-1, 1], so clamped
samples would compare little more than signs; the clamp itself is pinned as the exact identity
clamped == clip(unclamped) on the GPU. Two passes reach the mid
attention over the whole 44x78 frame, the first-frame rule of every temporal upsample, and the
histories handed from the first pass to the second. The GPU test compares its full-size decode
against these samples (PSNR over the samples and per frame). Calls only oracle/ and workloads/;
takes about an hour on 6 cores.

Usage: OMP_NUM_THREADS=6 python tests/golden/make_real_golden.py
"""
import os
import sys
import time

import dataclasses

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
from make_decoder_golden import input_digest, sample_indices  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "real_decode_samples.npz")
LATENT_FRAMES = 2
FRAMES_PER_PASS = 1
SPEC = dataclasses.replace(wl.REAL_DECODER, clamp=False)


def main():
    z, params = wl.decoder_weights(SPEC, seed=4, latent_frames=LATENT_FRAMES)
    digest = input_digest(z, params)
    p = oracle.as_numpy_params(params)
    del params
    t0 = time.time()
    video = oracle.decode(z[0], p, SPEC, frames_per_pass=FRAMES_PER_PASS, first_frame_rule=True)
    dt = time.time() - t0
    assert video.shape == (3, 5, 704, 1248), video.shape
    idx = sample_indices(video.shape)
    flat = video.reshape(-1)
    v64 = video.astype(np.float64)
    frame_mean = v64.mean(axis=(0, 2, 3))
    frame_meansq = (v64 ** 2).mean(axis=(0, 2, 3))
    np.savez_compressed(OUT, index=idx.astype(np.int64), value=flat[idx].astype(np.float32),
                        vmin=np.float64(v64.min()), vmax=np.float64(v64.max()), mean=np.float64(v64.mean()),
                        meansq=np.float64((v64 ** 2).mean()), frame_mean=frame_mean, frame_meansq=frame_meansq,
                        digest=np.array(digest), oracle_seconds=np.float64(dt),
                        threads=np.int64(oracle.num_threads()))
    print(f"wrote {OUT}: oracle {dt:.0f} s on {oracle.num_threads()} threads, range [{v64.min():.4f}, {v64.max():.4f}]")


if __name__ == "__main__":
    main()
