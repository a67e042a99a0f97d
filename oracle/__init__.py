"""Oracle of the chunked causal-conv video decoder. TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this package. It shares no code with the GPU path (``causal_convolution_causalconv3d_amd``)
and imports nothing from it.

It is a plain, slow CPU decoder: fp32 tensors in [C, T, H, W] order (batch 1), every sum in
double in a fixed order, rounded to fp32 once per op (the C primitives in ``oracle.c``); the
composition below follows the parts of the reference decoder printed on the FastVideo compare
page "[perf] PAN2 sampling: Wan2.2 VAE decode kernel, split decode, fused DiT kernels"
(reference.py: its docstring's part list, "The first latent frame yields one frame", "Causal
caches", and the functions cached_conv, causal_conv, residual_block, time_upsample,
spatial_upsample, rms_norm, decode_chunk). bf16 workloads hand the oracle bf16-rounded values;
inside the oracle nothing is rounded to bf16.

Readings taken where the page is silent or the workload text differs:
  * RMS norm is gamma * x / sqrt(mean_c x^2 + eps), eps = 1e-6 (the workload's explicit eps),
    not the page's x / max(||x||, 1e-12) * sqrt(C) form; they differ by <= eps / (2 mean x^2).
  * The synthetic decoder has no post_quant_conv, attention, DupUp3D shortcut, unpatchify or
    clamp: conv_in -> mid residual blocks -> up stages (residual blocks, time conv on the
    temporal stages, spatial x2 conv) -> norm_out + SiLU -> conv_out. A spec with the real
    topology's switches (workloads.REAL_DECODER and smaller ones) adds them in the page's order:
    post_quant_conv before conv_in (a 1x1x1 conv: per pass is the same as over all frames);
    attention after the first mid block; per stage an optional spatial step and DupUp3D of the
    stage's input added after it; unpatchify, then clamp. With norm_l2 the RMS norm is the
    page's x / max(||x||, 1e-12) * sqrt(C) * gamma (rms_norm_l2).
  * Each stage's first residual block changes channels (with a 1x1x1 shortcut when they differ).
  * The upsample-stage workload runs the spatial step first, then the time conv.
  * A conv whose input has zero frames is skipped and leaves its history unchanged.

Pins (tests/test_oracle_*.py, ``-m "not gpu"``), chosen so that a dropped term, a wrong sign or
index, or a transposed operand fails one of them:
  conv3d        torch float64 F.conv3d(F.pad(...)) and a pure-Python scalar loop on tiny
                tensors; delta-kernel identity (bitwise); time and row shifts; linearity;
                causality under perturbation of later frames; history placement.
  rms_norm      hand vectors with closed forms; mean_c y^2 = m / (m + eps) with gamma = 1;
                scale invariance; gamma per channel.
  silu          silu(0) = 0; x*sigmoid(x) == (x/2)(1 + tanh(x/2)); odd/even decomposition
                silu(x) - silu(-x) = x; limits.
  cache rule    the frame-keeping cases of the page's cached_conv, and chunked == one-shot
                bitwise for every split of T (causal caches part of the docstring).
  time upsample identity-tap weights duplicate frames; channel halves land on even/odd frames;
                first-frame rule gives 2T-1 frames with frame 0 passed through bit for bit.
  spatial up    torch float64 F.conv2d(F.interpolate(nearest)); the four-phase 2x2 identity;
                all-ones kernel on a constant frame gives 9v/6v/4v interior/edge/corner.
  decoder       frame counts 4T-3 (tests/golden/frame_counts.txt, the page's numbers); chunked ==
                one-shot bitwise for every pass size; video causality; decode independence;
                and the composition against torch float64 library ops.
  real parts    (tests/test_oracle_real.py) rms_norm_l2 hand values, zero vector, and equality
                with rms_norm(eps=0); attention: vanishing queries give the frame's mean value,
                scalar loops, torch float64 scaled_dot_product_attention, equivariance under
                position permutations; dup_up: ratio 8 is nearest x2 in t, h, w, ratio 2 maps
                channel pairs to row pairs (loops), torch repeat_interleave/permute for five
                shapes; unpatchify: loops and an inverse space-to-depth; clamp; the real
                topology's 110 parameters (the page's count); a small real-topology decoder:
                frame counts, chunked == one-shot bitwise, causality, and its composition
                against torch float64 library ops.
No absolute value of the synthetic decoder is printed on the pages: the decoder's output values
are pinned only through the identities above (parity of absolute values: pinned by op, the
composition by invariants).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()

# Portable x86-64 (AVX2/FMA) so that a build made on one host also runs on another.
CFLAGS = ["-O3", "-march=x86-64-v3", "-mtune=generic", "-fopenmp", "-fPIC", "-shared", "-std=c11",
          "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (fast; done on first use when missing)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB_PATH)
            fp = ctypes.POINTER(ctypes.c_float)
            lib.orc_causal_conv3d.argtypes = [fp, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, fp,
                                              ctypes.c_int, fp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, fp, fp]
            lib.orc_causal_conv3d.restype = ctypes.c_int
            lib.orc_rms_norm.argtypes = [fp, ctypes.c_int, ctypes.c_int64, fp, ctypes.c_double, fp]
            lib.orc_rms_norm.restype = ctypes.c_int
            lib.orc_silu.argtypes = [fp, ctypes.c_int64, fp]
            lib.orc_silu.restype = ctypes.c_int
            lib.orc_num_threads.argtypes = []
            lib.orc_num_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    if hasattr(a, "detach"):  # a torch tensor
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_float)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def num_threads() -> int:
    return int(_load().orc_num_threads())


# ----------------------------------------------------------------------------------------------
# Single ops (tensors [C, T, H, W])
# ----------------------------------------------------------------------------------------------
def causal_conv3d(x, w, b=None, hist=None) -> np.ndarray:
    """Causal conv: zero pad kh//2, kw//2 in space; 2*(kt//2) frames in front in time (the
    history, oldest first, after zeros for the frames it lacks); cross-correlation, stride 1.
    Follows the page's causal conv part and causal_conv function."""
    x = _f32(x)
    w = _f32(w)
    C, T, H, W = x.shape
    Co, Cw, kt, kh, kw = w.shape
    if Cw != C:
        raise ValueError(f"weight has {Cw} input channels, x has {C}")
    b = None if b is None else _f32(b)
    h = None
    Th = 0
    if hist is not None:
        h = _f32(hist)
        Th = h.shape[1]
        if Th == 0:
            h = None
        elif h.shape[0] != C or h.shape[2:] != (H, W):
            raise ValueError("history shape does not match x")
    y = np.empty((Co, T, H, W), dtype=np.float32)
    rc = _load().orc_causal_conv3d(_ptr(x), C, T, H, W, _ptr(h), Th, _ptr(w), Co, kt, kh, kw, _ptr(b), _ptr(y))
    if rc != 0:
        raise ValueError("orc_causal_conv3d rejected its arguments")
    return y


def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """gamma[c] * x / sqrt(mean over channels of x^2 + eps), at every position."""
    x = _f32(x)
    g = _f32(gamma)
    y = np.empty_like(x)
    P = int(np.prod(x.shape[1:]))
    if _load().orc_rms_norm(_ptr(x), x.shape[0], P, _ptr(g), float(eps), _ptr(y)) != 0:
        raise ValueError("orc_rms_norm rejected its arguments")
    return y


def silu(x) -> np.ndarray:
    """x / (1 + exp(-x))."""
    x = _f32(x)
    y = np.empty_like(x)
    if _load().orc_silu(_ptr(x), x.size, _ptr(y)) != 0:
        raise ValueError("orc_silu rejected its arguments")
    return y


def add(a, b) -> np.ndarray:
    """Elementwise fp32 sum (correctly rounded: the exact sum rounded once)."""
    return (_f32(a) + _f32(b)).astype(np.float32)


# ----------------------------------------------------------------------------------------------
# Causal caches (the page's "Causal caches" part and its cached_conv function)
# ----------------------------------------------------------------------------------------------
CACHE_T = 2


def keep_frames(old: Optional[np.ndarray], a: np.ndarray) -> Optional[np.ndarray]:
    """The history a conv keeps after consuming input `a` (frames on axis 1): its last two
    frames; after a one-frame input, the previous history's last frame and that frame. An input
    with no frames leaves the history as it was."""
    Ta = a.shape[1]
    if Ta == 0:
        return old
    keep = a[:, max(0, Ta - CACHE_T):]
    if keep.shape[1] < CACHE_T and old is not None and old.shape[1] > 0:
        keep = np.concatenate([old[:, -1:], keep], axis=1)
    return np.ascontiguousarray(keep)


def cached_conv(x, w, b, cache: Dict[str, np.ndarray], name: str) -> np.ndarray:
    x = _f32(x)
    if x.shape[1] == 0:
        return np.zeros((w.shape[0], 0) + x.shape[2:], dtype=np.float32)
    hist = cache.get(name)
    cache[name] = keep_frames(hist, x)
    return causal_conv3d(x, w, b, hist)


# ----------------------------------------------------------------------------------------------
# Blocks
# ----------------------------------------------------------------------------------------------
def norm_silu(x, gamma, eps) -> np.ndarray:
    return silu(rms_norm(x, gamma, eps))


def resblock(x, p: Dict[str, np.ndarray], prefix: str, cache: Dict[str, np.ndarray], eps: float,
             given_hist: Optional[np.ndarray] = None, l2: bool = False) -> np.ndarray:
    """Residual block: conv2(SiLU(norm2(conv1(SiLU(norm1(x)))))) + shortcut, the shortcut being x
    or a 1x1x1 conv of x when the channel count changes (the page's residual block part).

    `given_hist`, when set, is the activated history placed in front of both convs' inputs (the
    single-block workload's given cache); otherwise each conv uses its own entry of `cache`."""
    x = _f32(x)
    a1 = silu(_norm(x, p[f"{prefix}.norm1.gamma"], eps, l2))
    if given_hist is not None:
        h = causal_conv3d(a1, p[f"{prefix}.conv1.weight"], p.get(f"{prefix}.conv1.bias"), given_hist)
    else:
        h = cached_conv(a1, p[f"{prefix}.conv1.weight"], p.get(f"{prefix}.conv1.bias"), cache, f"{prefix}.conv1")
    a2 = silu(_norm(h, p[f"{prefix}.norm2.gamma"], eps, l2))
    if given_hist is not None:
        h2 = causal_conv3d(a2, p[f"{prefix}.conv2.weight"], p.get(f"{prefix}.conv2.bias"), given_hist)
    else:
        h2 = cached_conv(a2, p[f"{prefix}.conv2.weight"], p.get(f"{prefix}.conv2.bias"), cache, f"{prefix}.conv2")
    if f"{prefix}.shortcut.weight" in p:
        sc = causal_conv3d(x, p[f"{prefix}.shortcut.weight"], p.get(f"{prefix}.shortcut.bias"))
    else:
        sc = x
    return add(h2, sc)


def time_upsample(x, w, b, cache: Dict[str, np.ndarray], name: str) -> np.ndarray:
    """Causal 3x1x1 conv C -> 2C; output channel c goes to frame 2t, channel C + c to frame 2t+1
    (the page's upsample3d time conv and time_upsample function)."""
    x = _f32(x)
    C, T, H, W = x.shape
    y = cached_conv(x, w, b, cache, name)
    out = np.empty((C, 2 * T, H, W), dtype=np.float32)
    out[:, 0::2] = y[:C]
    out[:, 1::2] = y[C:]
    return out


def time_upsample_first(x, w, b, cache: Dict[str, np.ndarray], name: str) -> np.ndarray:
    """The pass holding latent frame 0: that frame passes through unchanged, the time conv runs on
    the frames after it (its history starting empty) - "The first latent frame yields one frame"."""
    x = _f32(x)
    rest = time_upsample(x[:, 1:], w, b, cache, name)
    return np.concatenate([x[:, :1], rest], axis=1)


def nearest2x(x) -> np.ndarray:
    """Nearest x2 in rows and columns: u[c, t, 2y+a, 2x+b] = x[c, t, y, x]."""
    x = _f32(x)
    return np.ascontiguousarray(np.repeat(np.repeat(x, 2, axis=2), 2, axis=3))


def spatial_upsample(x, w2d, b) -> np.ndarray:
    """Per frame: nearest x2, then a 3x3 conv2d with zero padding 1 (the page's upsample2d part;
    the 2-D conv is the causal conv with a one-frame kernel, which has no temporal padding)."""
    w2d = _f32(w2d)
    return causal_conv3d(nearest2x(x), w2d[:, :, None], b)


def upsample_stage(x, p: Dict[str, np.ndarray], prefix: str = "", cache=None) -> np.ndarray:
    """The upsample-stage workload: nearest x2 + 3x3 conv per frame, then the time conv into 2T
    frames (spatial first, as that workload states), zero history."""
    pre = f"{prefix}." if prefix else ""
    cache = {} if cache is None else cache
    u = spatial_upsample(x, p[f"{pre}spatial.weight"], p.get(f"{pre}spatial.bias"))
    return time_upsample(u, p[f"{pre}time.weight"], p.get(f"{pre}time.bias"), cache, f"{pre}time")


# ----------------------------------------------------------------------------------------------
# Parts of the real topology (the page's attention, dup_up, unpatchify and rms_norm functions and
# its part list): mid-block attention, DupUp3D, unpatchify, clamp, the L2 form of the RMS norm
# ----------------------------------------------------------------------------------------------
def rms_norm_l2(x, gamma) -> np.ndarray:
    """The page's WanRMS_norm: x / max(||x||_2 over channels, 1e-12) * sqrt(C) * gamma[c], in
    double, rounded to fp32 once."""
    x64 = _f32(x).astype(np.float64)
    C = x64.shape[0]
    nrm = np.sqrt((x64 * x64).sum(axis=0, keepdims=True))
    g = _f32(gamma).astype(np.float64).reshape((C,) + (1,) * (x64.ndim - 1))
    return (x64 / np.maximum(nrm, 1e-12) * np.sqrt(C) * g).astype(np.float32)


def _norm(x, gamma, spec_or_eps, l2: bool = False) -> np.ndarray:
    return rms_norm_l2(x, gamma) if l2 else rms_norm(x, gamma, spec_or_eps)


def attention(x, p: Dict[str, np.ndarray], prefix: str, eps: float, l2: bool = False) -> np.ndarray:
    """The page's attention part, per frame: n = RMS norm of x (no SiLU); q, k, v = channels
    [0, C), [C, 2C), [2C, 3C) of a 1x1 conv C -> 3C of n; softmax(q k^T / sqrt(C)) v over the
    frame's h*w positions (one head of dim C, no mask); a 1x1 conv C -> C; plus x. The products
    and the softmax in double (numpy matmul as the library step), each conv through conv3d."""
    x = _f32(x)
    C, T, H, W = x.shape
    n = _norm(x, p[f"{prefix}.norm.gamma"], eps, l2)
    qkv = causal_conv3d(n, p[f"{prefix}.qkv.weight"], p.get(f"{prefix}.qkv.bias"))
    o = np.empty((C, T, H, W), dtype=np.float32)
    for t in range(T):
        q = qkv[:C, t].reshape(C, H * W).T.astype(np.float64)          # [positions, C]
        k = qkv[C:2 * C, t].reshape(C, H * W).T.astype(np.float64)
        v = qkv[2 * C:, t].reshape(C, H * W).T.astype(np.float64)
        s = (q @ k.T) / np.sqrt(C)                                      # [query, key]
        s -= s.max(axis=1, keepdims=True)
        e = np.exp(s)
        a = e / e.sum(axis=1, keepdims=True)
        o[:, t] = (a @ v).T.reshape(C, H, W).astype(np.float32)
    y = causal_conv3d(o, p[f"{prefix}.proj.weight"], p.get(f"{prefix}.proj.bias"))
    return add(y, x)


def dup_up(x, out_channels: int, ft: int, first: bool) -> np.ndarray:
    """DupUp3D (the page's part list): with r = out * ft * 4 / in,
    dup[c, ft*t + a, 2y + i, 2x + j] = x[(4*ft*c + 4a + 2i + j) // r, t, y, x]; on the pass
    holding latent frame 0 only the last of that frame's ft time copies is kept."""
    x = _f32(x)
    Cin, T, H, W = x.shape
    if (out_channels * ft * 4) % Cin:
        raise ValueError("DupUp3D needs out * ft * 4 to be a multiple of the input channels")
    r = out_channels * ft * 4 // Cin
    out = np.empty((out_channels, ft * T, 2 * H, 2 * W), dtype=np.float32)
    c = np.arange(out_channels)
    for a in range(ft):
        for i in range(2):
            for j in range(2):
                out[:, a::ft, i::2, j::2] = x[(4 * ft * c + 4 * a + 2 * i + j) // r]
    return np.ascontiguousarray(out[:, ft - 1:]) if first else out


def unpatchify(x, patch: int) -> np.ndarray:
    """[3 * p^2, F, h, w] -> [3, F, p*h, p*w]: channel (k*p + j)*p + i is colour k at row offset i,
    column offset j (the page's unpatchify)."""
    x = _f32(x)
    Cp, Fr, h, w = x.shape
    if patch == 1:
        return x
    k_n = Cp // (patch * patch)
    out = np.empty((k_n, Fr, patch * h, patch * w), dtype=np.float32)
    for k in range(k_n):
        for j in range(patch):
            for i in range(patch):
                out[k, :, i::patch, j::patch] = x[(k * patch + j) * patch + i]
    return out


def clamp(x, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    return np.minimum(np.maximum(_f32(x), np.float32(lo)), np.float32(hi))


# ----------------------------------------------------------------------------------------------
# The decoder
# ----------------------------------------------------------------------------------------------
def decoder_pass(z, p: Dict[str, np.ndarray], spec, cache: Dict[str, np.ndarray], first: bool) -> np.ndarray:
    """One pass of the synthetic decoder over latents z [Cz, n, h, w] (the page's decode_chunk,
    minus the parts the synthetic decoder leaves out). `cache` carries every causal conv's history
    from the previous pass and is updated; `first` marks the pass holding latent frame 0."""
    eps = spec.eps
    l2 = getattr(spec, "norm_l2", False)
    z = _f32(z)
    if getattr(spec, "post_quant", False):
        z = causal_conv3d(z, p["post_quant.weight"], p.get("post_quant.bias"))
    x = cached_conv(z, p["conv_in.weight"], p.get("conv_in.bias"), cache, "conv_in")
    for i in range(spec.mid_resblocks):
        x = resblock(x, p, f"mid.{i}", cache, eps, l2=l2)
        if i == 0 and getattr(spec, "mid_attention", False):
            x = attention(x, p, "mid.attn", eps, l2)
    n_st = len(spec.stage_channels)
    spatial = getattr(spec, "spatial", (True,) * n_st)
    dup = getattr(spec, "dup", (False,) * n_st)
    for s in range(n_st):
        block_input = x
        for j in range(spec.stage_resblocks):
            x = resblock(x, p, f"up.{s}.res.{j}", cache, eps, l2=l2)
        if spec.temporal[s]:
            tw, tb = p[f"up.{s}.time.weight"], p.get(f"up.{s}.time.bias")
            if first:
                x = time_upsample_first(x, tw, tb, cache, f"up.{s}.time")
            else:
                x = time_upsample(x, tw, tb, cache, f"up.{s}.time")
        if spatial[s]:
            x = spatial_upsample(x, p[f"up.{s}.spatial.weight"], p.get(f"up.{s}.spatial.bias"))
        if dup[s]:
            x = add(x, dup_up(block_input, spec.stage_channels[s], 2 if spec.temporal[s] else 1, first))
    x = silu(_norm(x, p["norm_out.gamma"], eps, l2))
    y = cached_conv(x, p["conv_out.weight"], p.get("conv_out.bias"), cache, "conv_out")
    y = unpatchify(y, getattr(spec, "patch", 1))
    return clamp(y) if getattr(spec, "clamp", False) else y


def split_passes(latent_frames: int, frames_per_pass: int) -> List[int]:
    if frames_per_pass < 1:
        raise ValueError("frames_per_pass must be at least 1")
    sizes = []
    left = latent_frames
    while left > 0:
        sizes.append(min(frames_per_pass, left))
        left -= sizes[-1]
    return sizes


def decode(z, p: Dict[str, np.ndarray], spec, frames_per_pass: int, first_frame_rule: bool = True) -> np.ndarray:
    """Streaming decode: passes of `frames_per_pass` latent frames, one cache set carried across
    them, the outputs concatenated in time. With first_frame_rule the first pass holds latent
    frame 0 (4T-3 frames in all); without it every pass doubles every frame (the one-pass decoder
    workload). frames_per_pass >= T is the one-shot decode."""
    z = _f32(z)
    if z.ndim == 5:
        z = z[0]
    cache: Dict[str, np.ndarray] = {}
    outs = []
    start = 0
    for n in split_passes(z.shape[1], frames_per_pass):
        outs.append(decoder_pass(z[:, start:start + n], p, spec, cache, first=first_frame_rule and start == 0))
        start += n
    return np.concatenate(outs, axis=1)


def as_numpy_params(params) -> Dict[str, np.ndarray]:
    return {k: _f32(v) for k, v in params.items()}
