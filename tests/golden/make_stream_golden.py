"""Writes tests/golden/stream_decode_samples.npz: the oracle's decode of the 5 s streaming workload
(latents [1,48,31,44,78] from seed 5, the full synthetic decoder's weights from seed 4, first-frame
rule on: video [1,3,121,704,1248]) at seeded sample positions, plus per-frame statistics of the
whole video. The GPU test compares its 4-latent-frame streaming decode against these values.

The oracle decodes in passes of 5 latent frames ([5,5,5,5,5,5,1]). Its chunked decode equals its
one-shot decode bit for bit (every output element sums the same operands in the same order; the
CPU tests check this for every split of small decoders), so these are the one-shot decode's
values; the one-shot form itself would hold ~150 GB of fp32 activations at once. The pass
boundaries (latent frames 5, 10, ...) differ from the GPU's (4, 8, ...), so a cache-carry or
first-frame mistake on the GPU side cannot cancel against the same mistake here.

Sample positions: 32768 uniform over the video, plus 1024 per frame on frame 0, the GPU's first
pass boundary (frames 12, 13, 14), a later GPU boundary (frames 60, 61), the oracle's own first
boundary (frames 16, 17) and the last frame (120).

Calls only oracle/ and workloads/. Takes about 80 minutes on 8 cores.

Usage: python tests/golden/make_stream_golden.py
"""
import hashlib
import os
import platform
import subprocess
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as wl  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "stream_decode_samples.npz")
SHAPE = (3, 121, 704, 1248)
N_UNIFORM = 32768
PER_FRAME = 1024
FOCUS_FRAMES = (0, 12, 13, 14, 16, 17, 60, 61, 120)
SAMPLE_SEED = 4321
ORACLE_PASS = 5


def sample_indices():
    rng = np.random.default_rng(SAMPLE_SEED)
    C, F, H, W = SHAPE
    total = C * F * H * W
    idx = [rng.choice(total, size=N_UNIFORM, replace=False)]
    frame_size = H * W
    for f in FOCUS_FRAMES:
        c = rng.integers(0, C, size=PER_FRAME)
        pos = rng.choice(frame_size, size=PER_FRAME, replace=False)
        idx.append((c * F + f) * frame_size + pos)
    return np.unique(np.concatenate(idx)).astype(np.int64)


def input_digest(z, params) -> str:
    h = hashlib.sha256()
    h.update(np.ascontiguousarray(z.numpy()).tobytes())
    for name in sorted(params):
        h.update(name.encode())
        h.update(np.ascontiguousarray(params[name].numpy()).tobytes())
    return h.hexdigest()


def cpu_model() -> str:
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, check=True).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except Exception:
        pass
    return platform.processor() or "unknown"


def main():
    _, params = wl.decoder_weights(wl.FULL_DECODER, seed=4, latent_frames=4)
    z = wl.streaming_latents(seed=5, latent_frames=31)
    digest = input_digest(z, params)
    p = oracle.as_numpy_params(params)
    del params
    t0 = time.time()
    video = oracle.decode(z[0], p, wl.FULL_DECODER, frames_per_pass=ORACLE_PASS, first_frame_rule=True)
    dt = time.time() - t0
    assert video.shape == SHAPE, video.shape
    idx = sample_indices()
    flat = video.reshape(-1)
    per_frame = video.transpose(1, 0, 2, 3).reshape(SHAPE[1], -1).astype(np.float64)
    v64 = video.astype(np.float64)
    np.savez_compressed(
        OUT, index=idx, value=flat[idx].astype(np.float32),
        vmin=np.float64(v64.min()), vmax=np.float64(v64.max()), mean=np.float64(v64.mean()),
        meansq=np.float64((v64 ** 2).mean()),
        frame_min=per_frame.min(axis=1), frame_max=per_frame.max(axis=1),
        frame_mean=per_frame.mean(axis=1), frame_meansq=(per_frame ** 2).mean(axis=1),
        digest=np.array(digest), oracle_pass=np.int64(ORACLE_PASS),
        oracle_seconds=np.float64(dt), threads=np.int64(oracle.num_threads()),
        nproc=np.int64(os.cpu_count() or 0), cpu_model=np.array(cpu_model()),
        omp_num_threads=np.array(os.environ.get("OMP_NUM_THREADS", "")))
    print(f"wrote {OUT}: {idx.size} samples, oracle {dt:.0f} s on {oracle.num_threads()} threads, "
          f"range [{v64.min():.4f}, {v64.max():.4f}]", flush=True)


if __name__ == "__main__":
    main()
