"""Writes tests/golden/decoder_onepass_samples.npz: the oracle's one-pass decode of the full
synthetic decoder (latents [1,48,4,44,78] from seed 4, the same seed's weights, every latent frame
doubled twice: video [1,3,16,704,1248]) at 32768 seeded sample positions, plus the whole video's
min / max / mean / mean square. The GPU test compares its full-size decode against these samples
(PSNR over the samples). Calls only oracle/ and workloads/; takes ~15 minutes on 8 cores.

Usage: python tests/golden/make_decoder_golden.py
"""
import hashlib
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as wl  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "decoder_onepass_samples.npz")
N_SAMPLES = 32768
SAMPLE_SEED = 1234


def sample_indices(shape, n=N_SAMPLES, seed=SAMPLE_SEED):
    rng = np.random.default_rng(seed)
    total = int(np.prod(shape))
    return np.sort(rng.choice(total, size=n, replace=False)).astype(np.int64)


def input_digest(z, params) -> str:
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(z.numpy()).tobytes())
    for name in sorted(params):
        h.update(name.encode())
        h.update(np.ascontiguousarray(params[name].numpy()).tobytes())
    return h.hexdigest()


def main():
    z, params = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=4)
    digest = input_digest(z, params)
    t0 = time.time()
    video = oracle.decode(z[0], oracle.as_numpy_params(params), wl.FULL_DECODER, frames_per_pass=4,
                          first_frame_rule=False)
    dt = time.time() - t0
    assert video.shape == (3, 16, 704, 1248), video.shape
    idx = sample_indices(video.shape)
    flat = video.reshape(-1)
    v64 = video.astype(np.float64)
    np.savez_compressed(OUT, index=idx.astype(np.int64), value=flat[idx].astype(np.float32),
                        vmin=np.float64(v64.min()), vmax=np.float64(v64.max()), mean=np.float64(v64.mean()),
                        meansq=np.float64((v64 ** 2).mean()), digest=np.array(digest),
                        oracle_seconds=np.float64(dt), threads=np.int64(oracle.num_threads()))
    print(f"wrote {OUT}: oracle {dt:.0f} s on {oracle.num_threads()} threads, range [{v64.min():.4f}, {v64.max():.4f}]")


if __name__ == "__main__":
    main()
