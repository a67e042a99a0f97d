"""Python binding of libwvd, the MI355X (gfx950) causal-conv video decoder.

Argument marshalling only: every step of the decode runs in the library's HIP kernels; PyTorch
provides device memory (tensors, workspaces) and the stream (``torch.cuda.current_stream()``).
The names mirror the C ABI in ``include/wvd.h``.

Tensor conventions of this binding:
  * bf16 activations are torch tensors of shape [1, T, H, W, C] (NTHWC, contiguous);
  * the fp32 path also accepts [1, C, T, H, W] tensors (NCTHW, contiguous): pass layout="NCTHW";
  * the decoded video is [1, C_out, F, H, W] bf16 (NCTHW).
There is no fallback: if libwvd.so is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwvd.so")

WVD_F32, WVD_BF16 = 0, 1
WVD_NCTHW, WVD_NTHWC = 0, 1
WVD_PACK_CONV, WVD_PACK_PHASE2X = 0, 1
WVD_TIME_FIRST, WVD_SPATIAL_FIRST = 0, 1
MAX_STAGES = 8

STATUS_NAMES = {0: "OK", 1: "ERR_ARG", 2: "ERR_SHAPE", 3: "ERR_DTYPE", 4: "ERR_LAYOUT", 5: "ERR_ALIGN",
                6: "ERR_STATE", 7: "ERR_WORKSPACE", 8: "ERR_UNSUPPORTED", 9: "ERR_HIP"}


class WvdError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("n", ctypes.c_int64), ("c", ctypes.c_int64), ("t", ctypes.c_int64), ("h", ctypes.c_int64),
                ("w", ctypes.c_int64)]


class ResblockWeights(ctypes.Structure):
    _fields_ = [("cin", ctypes.c_int), ("cout", ctypes.c_int), ("gamma1", ctypes.c_void_p), ("conv1", ctypes.c_void_p),
                ("bias1", ctypes.c_void_p), ("gamma2", ctypes.c_void_p), ("conv2", ctypes.c_void_p),
                ("bias2", ctypes.c_void_p), ("shortcut", ctypes.c_void_p), ("shortcut_bias", ctypes.c_void_p)]


class DecoderDesc(ctypes.Structure):
    _fields_ = [("z_channels", ctypes.c_int), ("base_channels", ctypes.c_int), ("n_stages", ctypes.c_int),
                ("stage_channels", ctypes.c_int * MAX_STAGES), ("stage_temporal", ctypes.c_int * MAX_STAGES),
                ("mid_resblocks", ctypes.c_int), ("stage_resblocks", ctypes.c_int), ("out_channels", ctypes.c_int),
                ("eps", ctypes.c_float), ("latent_h", ctypes.c_int), ("latent_w", ctypes.c_int),
                ("post_quant", ctypes.c_int), ("mid_attention", ctypes.c_int),
                ("stage_no_spatial", ctypes.c_int * MAX_STAGES), ("stage_dup", ctypes.c_int * MAX_STAGES),
                ("patch", ctypes.c_int), ("clamp", ctypes.c_int)]


_lib = None
_P = ctypes.c_void_p
_T = ctypes.POINTER(Tensor)


def lib():
    """The loaded libwvd.so (raises if it is not built or does not load)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libwvd.so is not built ({LIB_PATH}); run python -m causal_convolution_causalconv3d_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        sigs = {
            "wvd_last_error": ([], ctypes.c_char_p),
            "wvd_abi_version": ([], ctypes.c_int),
            "wvd_convert": ([_T, _T, _P], ctypes.c_int),
            "wvd_conv_packed_bytes": ([ctypes.c_int] * 6, ctypes.c_size_t),
            "wvd_conv_pack": ([_P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, _P, _P], ctypes.c_int),
            "wvd_causal_conv3d": ([_T, _P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _T, _T, _T, _T, _P],
                                  ctypes.c_int),
            "wvd_rmsnorm_silu": ([_T, _P, ctypes.c_float, ctypes.c_int, _T, _P], ctypes.c_int),
            "wvd_resblock_workspace_bytes": ([ctypes.c_int] * 5, ctypes.c_size_t),
            "wvd_resblock": ([_T, ctypes.POINTER(ResblockWeights), ctypes.c_float, _T, _T, _T, _T, _T, _P, ctypes.c_size_t,
                              _P], ctypes.c_int),
            "wvd_resblock_noalloc_max_bytes": ([], ctypes.c_size_t),
            "wvd_resblock_noalloc": ([_T, ctypes.POINTER(ResblockWeights), ctypes.c_float, _T, _T, _T, _T, _T, _P],
                                     ctypes.c_int),
            "wvd_upsample_workspace_bytes": ([ctypes.c_int] * 7, ctypes.c_size_t),
            "wvd_upsample": ([_T, _P, _P, _P, _P, ctypes.c_int, ctypes.c_int, _T, _T, _T, _P, ctypes.c_size_t, _P],
                             ctypes.c_int),
            "wvd_decoder_param_count": ([ctypes.POINTER(DecoderDesc)], ctypes.c_int),
            "wvd_decoder_param_info": ([ctypes.POINTER(DecoderDesc), ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                        ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
            "wvd_decoder_packed_bytes": ([ctypes.POINTER(DecoderDesc)], ctypes.c_size_t),
            "wvd_decoder_pack": ([ctypes.POINTER(DecoderDesc), ctypes.POINTER(ctypes.c_void_p), _P, _P], ctypes.c_int),
            "wvd_cache_bytes": ([ctypes.POINTER(DecoderDesc)], ctypes.c_size_t),
            "wvd_cache_init": ([ctypes.POINTER(DecoderDesc), _P, ctypes.POINTER(ctypes.c_void_p)], ctypes.c_int),
            "wvd_cache_reset": ([_P], ctypes.c_int),
            "wvd_cache_destroy": ([_P], None),
            "wvd_cache_next_latent": ([_P], ctypes.c_int64),
            "wvd_decode_workspace_bytes": ([ctypes.POINTER(DecoderDesc), ctypes.c_int], ctypes.c_size_t),
            "wvd_decode_chunk": ([ctypes.POINTER(DecoderDesc), _P, _P, _T, ctypes.c_int, ctypes.c_int, _T, ctypes.c_int64,
                                  _P, ctypes.c_size_t, _P], ctypes.c_int),
            "wvd_chunk_video_frames": ([ctypes.POINTER(DecoderDesc), ctypes.c_int64, ctypes.c_int, ctypes.c_int],
                                       ctypes.c_int64),
            "wvd_decode_workspace_bytes_split": ([ctypes.POINTER(DecoderDesc), ctypes.c_int, ctypes.c_int],
                                                 ctypes.c_size_t),
            "wvd_decode_chunk_split": ([ctypes.POINTER(DecoderDesc), _P, _P, _T, ctypes.c_int, ctypes.c_int, _T,
                                        ctypes.c_int64, ctypes.c_int, _P, ctypes.c_size_t, _P], ctypes.c_int),
            "wvd_timing_enable": ([ctypes.c_int], ctypes.c_int),
            "wvd_timing_reset": ([], ctypes.c_int),
            "wvd_timing_read": ([ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int64),
                                 ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
            "wvd_timing_launch": ([ctypes.c_int, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_double),
                                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
            "wvd_conv_force_config": ([ctypes.c_int], ctypes.c_int),
            "wvd_conv_max_workgroups": ([ctypes.c_int], ctypes.c_int),
            "wvd_calib_dma_copy": ([_P, _P, ctypes.c_size_t, _P], ctypes.c_int),
            "wvd_decode_fuse_norm1": ([ctypes.c_int], ctypes.c_int),
            "wvd_decode_fuse_head": ([ctypes.c_int], ctypes.c_int),
            "wvd_decode_fuse_shortcut": ([ctypes.c_int], ctypes.c_int),
            "wvd_fuse_norm_shortcut": ([ctypes.c_int], ctypes.c_int),
            "wvd_winograd_packed_bytes": ([ctypes.c_int, ctypes.c_int], ctypes.c_size_t),
            "wvd_winograd_pack": ([_P, ctypes.c_int, ctypes.c_int, ctypes.c_int, _P, _P], ctypes.c_int),
            "wvd_winograd_workspace_bytes": ([ctypes.c_int] * 6, ctypes.c_size_t),
            "wvd_causal_conv3d_winograd": ([_T, _P, ctypes.c_int, _P, _T, _T, _T, _P, ctypes.c_size_t, _P], ctypes.c_int),
            "wvd_timing_read_mem": ([ctypes.c_int, ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_int64),
                                     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
        }
        for name, (args, res) in sigs.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def exported_symbols() -> Sequence[str]:
    """Names of the C ABI this binding declares (all must be exported by libwvd.so)."""
    lib()
    return ["wvd_last_error", "wvd_abi_version", "wvd_convert", "wvd_conv_packed_bytes", "wvd_conv_pack",
            "wvd_causal_conv3d", "wvd_rmsnorm_silu", "wvd_resblock_workspace_bytes", "wvd_resblock",
            "wvd_resblock_noalloc_max_bytes", "wvd_resblock_noalloc",
            "wvd_upsample_workspace_bytes", "wvd_upsample", "wvd_decoder_param_count", "wvd_decoder_param_info",
            "wvd_decoder_packed_bytes", "wvd_decoder_pack", "wvd_cache_bytes", "wvd_cache_init", "wvd_cache_reset",
            "wvd_cache_destroy", "wvd_cache_next_latent", "wvd_decode_workspace_bytes", "wvd_decode_chunk",
            "wvd_decode_workspace_bytes_split", "wvd_decode_chunk_split",
            "wvd_chunk_video_frames", "wvd_timing_enable", "wvd_timing_reset", "wvd_timing_read",
            "wvd_timing_launch", "wvd_conv_force_config", "wvd_timing_read_mem", "wvd_conv_max_workgroups",
            "wvd_calib_dma_copy", "wvd_winograd_packed_bytes", "wvd_winograd_pack", "wvd_winograd_workspace_bytes",
            "wvd_causal_conv3d_winograd", "wvd_decode_fuse_norm1", "wvd_decode_fuse_head",
            "wvd_decode_fuse_shortcut", "wvd_fuse_norm_shortcut"]


def _check(status: int):
    if status != 0:
        raise WvdError(status, lib().wvd_last_error().decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def nthwc(t: torch.Tensor) -> Tensor:
    """Descriptor of a [1, T, H, W, C] contiguous tensor (NTHWC)."""
    if t.dim() != 5 or not t.is_contiguous():
        raise ValueError("expected a contiguous [1, T, H, W, C] tensor")
    dt = {torch.bfloat16: WVD_BF16, torch.float32: WVD_F32}[t.dtype]
    n, T, H, W, C = t.shape
    return Tensor(t.data_ptr() if t.numel() else None, dt, WVD_NTHWC, n, C, T, H, W)


def ncthw(t: torch.Tensor) -> Tensor:
    """Descriptor of a [1, C, T, H, W] contiguous tensor (NCTHW)."""
    if t.dim() != 5 or not t.is_contiguous():
        raise ValueError("expected a contiguous [1, C, T, H, W] tensor")
    dt = {torch.bfloat16: WVD_BF16, torch.float32: WVD_F32}[t.dtype]
    n, C, T, H, W = t.shape
    return Tensor(t.data_ptr() if t.numel() else None, dt, WVD_NCTHW, n, C, T, H, W)


def _desc(t: Optional[torch.Tensor], layout: str):
    if t is None:
        return None
    return ctypes.byref(nthwc(t) if layout == "NTHWC" else ncthw(t))


def history_frames_after(T: int, Th: int) -> int:
    """Frames a conv's history holds after an input of T frames (the page's cached_conv rule)."""
    if T >= 2:
        return 2
    if T == 1:
        return 2 if Th >= 1 else 1
    return Th


# ------------------------------------------------------------------------------------------------
# Single ops
# ------------------------------------------------------------------------------------------------
def convert(x: torch.Tensor, x_layout: str, y: torch.Tensor, y_layout: str):
    _check(lib().wvd_convert(_desc(x, x_layout), _desc(y, y_layout), _stream()))
    return y


def conv_pack(w: torch.Tensor, mode: int = WVD_PACK_CONV) -> torch.Tensor:
    """Pack a raw conv weight (device, fp32 or bf16) for the bf16 kernels."""
    w = w.contiguous()
    if mode == WVD_PACK_PHASE2X:
        co, ci, kh, kw = w.shape
        kt = 1
    else:
        co, ci, kt, kh, kw = w.shape
    nbytes = lib().wvd_conv_packed_bytes(co, ci, kt, kh, kw, mode)
    if nbytes == 0:
        raise WvdError(1, "unsupported weight shape")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    dt = WVD_BF16 if w.dtype == torch.bfloat16 else WVD_F32
    _check(lib().wvd_conv_pack(_ptr(w), dt, co, ci, kt, kh, kw, mode, _ptr(out), _stream()))
    return out


def causal_conv3d(x, w, co, kernel=(3, 3, 3), bias=None, hist=None, residual=None, out=None, hist_out=None,
                  layout="NTHWC"):
    """wvd_causal_conv3d. bf16: `w` packed (conv_pack); fp32: `w` the raw fp32 weight."""
    kt, kh, kw = kernel
    if out is None:
        if layout == "NTHWC":
            out = torch.empty(x.shape[:4] + (co,), dtype=x.dtype, device=x.device)
        else:
            out = torch.empty((x.shape[0], co) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device)
    _check(lib().wvd_causal_conv3d(_desc(x, layout), _ptr(w), co, kt, kh, kw, _ptr(bias), _desc(hist, layout),
                                   _desc(residual, layout), _desc(out, layout), _desc(hist_out, layout), _stream()))
    return out


def winograd_pack(w: torch.Tensor) -> torch.Tensor:
    """wvd_winograd_pack: the raw 3x3x3 weight [co, ci, 3, 3, 3] (fp32 or bf16, device) -> its 16
    transformed component weights, packed."""
    co, ci = w.shape[:2]
    if tuple(w.shape[2:]) != (3, 3, 3):
        raise WvdError(2, "winograd_pack needs a 3x3x3 weight")
    out = torch.empty(lib().wvd_winograd_packed_bytes(co, ci), dtype=torch.uint8, device=w.device)
    dt = WVD_BF16 if w.dtype == torch.bfloat16 else WVD_F32
    _check(lib().wvd_winograd_pack(_ptr(w.contiguous()), dt, co, ci, _ptr(out), _stream()))
    return out


def causal_conv3d_winograd(x, w_packed, co, bias=None, hist=None, residual=None, out=None, ws=None):
    """wvd_causal_conv3d_winograd on a [1, T, H, W, ci] bf16 tensor (NTHWC)."""
    _, T, H, W, ci = x.shape
    th = 0 if hist is None else hist.shape[1]
    if out is None:
        out = torch.empty(x.shape[:4] + (co,), dtype=x.dtype, device=x.device)
    nbytes = lib().wvd_winograd_workspace_bytes(ci, co, T, th, H, W)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _check(lib().wvd_causal_conv3d_winograd(_desc(x, "NTHWC"), _ptr(w_packed), co, _ptr(bias), _desc(hist, "NTHWC"),
                                            _desc(residual, "NTHWC"), _desc(out, "NTHWC"), _ptr(ws), ws.numel(),
                                            _stream()))
    return out


def rmsnorm_silu(x, gamma, eps, silu=True, out=None):
    out = torch.empty_like(x) if out is None else out
    _check(lib().wvd_rmsnorm_silu(_desc(x, "NTHWC"), _ptr(gamma), eps, int(silu), _desc(out, "NTHWC"), _stream()))
    return out


def pack_resblock(params: Dict[str, torch.Tensor], prefix: str, device) -> dict:
    """Packed weights of a residual block from its raw parameters (names '<prefix>.conv1.weight', ...)."""
    g = lambda k: params[f"{prefix}.{k}"].to(device=device, dtype=torch.float32).contiguous()
    cout, cin = params[f"{prefix}.conv1.weight"].shape[:2]
    d = {"cin": int(cin), "cout": int(cout), "gamma1": g("norm1.gamma"), "conv1": conv_pack(g("conv1.weight")),
         "bias1": g("conv1.bias") if f"{prefix}.conv1.bias" in params else None, "gamma2": g("norm2.gamma"),
         "conv2": conv_pack(g("conv2.weight")),
         "bias2": g("conv2.bias") if f"{prefix}.conv2.bias" in params else None, "shortcut": None,
         "shortcut_bias": None}
    if f"{prefix}.shortcut.weight" in params:
        d["shortcut"] = conv_pack(g("shortcut.weight"))
        d["shortcut_bias"] = g("shortcut.bias") if f"{prefix}.shortcut.bias" in params else None
    return d


def resblock(x, wts: dict, eps, hist1=None, hist2=None, out=None, hist1_out=None, hist2_out=None):
    """wvd_resblock on a [1, T, H, W, cin] bf16 tensor."""
    _, T, H, W, _ = x.shape
    if out is None:
        out = torch.empty((1, T, H, W, wts["cout"]), dtype=torch.bfloat16, device=x.device)
    rw = ResblockWeights(wts["cin"], wts["cout"], *[wts[k].data_ptr() if wts[k] is not None else None for k in (
        "gamma1", "conv1", "bias1", "gamma2", "conv2", "bias2", "shortcut", "shortcut_bias")])
    nbytes = lib().wvd_resblock_workspace_bytes(wts["cin"], wts["cout"], T, H, W)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _check(lib().wvd_resblock(_desc(x, "NTHWC"), ctypes.byref(rw), eps, _desc(hist1, "NTHWC"), _desc(hist2, "NTHWC"),
                              _desc(out, "NTHWC"), _desc(hist1_out, "NTHWC"), _desc(hist2_out, "NTHWC"), _ptr(ws), nbytes,
                              _stream()))
    return out


def resblock_noalloc(x, wts: dict, eps, out, hist1=None, hist2=None, hist1_out=None, hist2_out=None):
    """wvd_resblock_noalloc: wvd_resblock with the library's built-in scratch as its workspace
    (no device allocation inside the call; `out` must be given)."""
    rw = ResblockWeights(wts["cin"], wts["cout"], *[wts[k].data_ptr() if wts[k] is not None else None for k in (
        "gamma1", "conv1", "bias1", "gamma2", "conv2", "bias2", "shortcut", "shortcut_bias")])
    _check(lib().wvd_resblock_noalloc(_desc(x, "NTHWC"), ctypes.byref(rw), eps, _desc(hist1, "NTHWC"),
                                      _desc(hist2, "NTHWC"), _desc(out, "NTHWC"), _desc(hist1_out, "NTHWC"),
                                      _desc(hist2_out, "NTHWC"), _stream()))
    return out


def upsample(x, spatial=None, spatial_bias=None, temporal=None, temporal_bias=None, order=WVD_TIME_FIRST, first=False,
             time_hist=None, out=None, time_hist_out=None):
    """wvd_upsample on a [1, T, H, W, C] bf16 tensor; `spatial` / `temporal` are packed weights."""
    _, T, H, W, C = x.shape
    To = (2 * T - 1 if (first and T > 0) else 2 * T) if temporal is not None else T
    Ho, Wo = (2 * H, 2 * W) if spatial is not None else (H, W)
    if out is None:
        out = torch.empty((1, To, Ho, Wo, C), dtype=torch.bfloat16, device=x.device)
    nbytes = lib().wvd_upsample_workspace_bytes(C, T, H, W, int(spatial is not None), int(temporal is not None), order)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    _check(lib().wvd_upsample(_desc(x, "NTHWC"), _ptr(spatial), _ptr(spatial_bias), _ptr(temporal), _ptr(temporal_bias),
                              order, int(first), _desc(time_hist, "NTHWC"), _desc(out, "NTHWC"),
                              _desc(time_hist_out, "NTHWC"), _ptr(ws), nbytes, _stream()))
    return out


# ------------------------------------------------------------------------------------------------
# The decoder
# ------------------------------------------------------------------------------------------------
def make_desc(z_channels=48, base_channels=384, stage_channels=(384, 384, 192, 96), stage_temporal=(1, 1, 0, 0),
              mid_resblocks=2, stage_resblocks=2, out_channels=3, eps=1e-6, latent_h=44, latent_w=78,
              post_quant=False, mid_attention=False, stage_spatial=None, stage_dup=None, patch=1,
              clamp=False) -> DecoderDesc:
    """The decoder descriptor; the defaults are the synthetic decoder, the keyword arguments from
    post_quant on switch on the real Wan2.2 decoder's parts (see desc_from_spec)."""
    d = DecoderDesc()
    d.z_channels, d.base_channels, d.n_stages = z_channels, base_channels, len(stage_channels)
    n = len(stage_channels)
    spatial = (1,) * n if stage_spatial is None else stage_spatial
    dup = (0,) * n if stage_dup is None else stage_dup
    for i, (c, t) in enumerate(zip(stage_channels, stage_temporal)):
        d.stage_channels[i] = c
        d.stage_temporal[i] = int(bool(t))
        d.stage_no_spatial[i] = int(not spatial[i])
        d.stage_dup[i] = int(bool(dup[i]))
    d.mid_resblocks, d.stage_resblocks, d.out_channels = mid_resblocks, stage_resblocks, out_channels
    d.eps, d.latent_h, d.latent_w = eps, latent_h, latent_w
    d.post_quant, d.mid_attention = int(bool(post_quant)), int(bool(mid_attention))
    d.patch, d.clamp = int(patch), int(bool(clamp))
    return d


def desc_from_spec(spec, latent_h=44, latent_w=78) -> DecoderDesc:
    """The descriptor of a workloads.DecoderSpec-like object (attribute names as there)."""
    n = len(spec.stage_channels)
    return make_desc(z_channels=spec.z_channels, base_channels=spec.base_channels,
                     stage_channels=tuple(spec.stage_channels), stage_temporal=tuple(spec.temporal),
                     mid_resblocks=spec.mid_resblocks, stage_resblocks=spec.stage_resblocks,
                     out_channels=spec.out_channels, eps=spec.eps, latent_h=latent_h, latent_w=latent_w,
                     post_quant=getattr(spec, "post_quant", False), mid_attention=getattr(spec, "mid_attention", False),
                     stage_spatial=tuple(getattr(spec, "spatial", (True,) * n)),
                     stage_dup=tuple(getattr(spec, "dup", (False,) * n)), patch=getattr(spec, "patch", 1),
                     clamp=getattr(spec, "clamp", False))


def video_shape(desc: DecoderDesc, frames: int):
    """[1, colours, frames, H, W] of a decode with this descriptor."""
    levels = sum(1 for i in range(desc.n_stages) if not desc.stage_no_spatial[i])
    p = desc.patch if desc.patch >= 2 else 1
    return (1, desc.out_channels // (p * p), frames, (desc.latent_h << levels) * p, (desc.latent_w << levels) * p)


def param_names(desc: DecoderDesc):
    n = lib().wvd_decoder_param_count(ctypes.byref(desc))
    if n < 0:
        raise WvdError(1, lib().wvd_last_error().decode())
    out = []
    for i in range(n):
        name = ctypes.c_char_p()
        nd = ctypes.c_int()
        shape = (ctypes.c_int64 * 5)()
        _check(lib().wvd_decoder_param_info(ctypes.byref(desc), i, ctypes.byref(name), ctypes.byref(nd), shape))
        out.append((name.value.decode(), tuple(shape[: nd.value])))
    return out


class Decoder:
    """The packed decoder on one device; decode() streams latents through wvd_decode_chunk."""

    def __init__(self, desc: DecoderDesc, params: Dict[str, torch.Tensor], device="cuda"):
        self.desc = desc
        self.device = torch.device(device)
        names = param_names(desc)
        dev = [params[n].to(device=self.device, dtype=torch.float32).contiguous() for n, _ in names]
        for (n, shape), t in zip(names, dev):
            if tuple(t.shape) != shape:
                raise ValueError(f"{n}: shape {tuple(t.shape)}, expected {shape}")
        self.packed = torch.empty(lib().wvd_decoder_packed_bytes(ctypes.byref(desc)), dtype=torch.uint8,
                                  device=self.device)
        ptrs = (ctypes.c_void_p * len(dev))(*[t.data_ptr() for t in dev])
        _check(lib().wvd_decoder_pack(ctypes.byref(desc), ptrs, _ptr(self.packed), _stream()))
        torch.cuda.current_stream().synchronize()  # the raw fp32 copies may go now
        self.cache_storage = torch.empty(lib().wvd_cache_bytes(ctypes.byref(desc)), dtype=torch.uint8,
                                         device=self.device)
        h = ctypes.c_void_p()
        _check(lib().wvd_cache_init(ctypes.byref(desc), _ptr(self.cache_storage), ctypes.byref(h)))
        self.cache = h
        self._ws = None
        self._ws_frames = None

    def __del__(self):
        try:
            if getattr(self, "cache", None):
                lib().wvd_cache_destroy(self.cache)
                self.cache = None
        except Exception:
            pass

    def video_frames(self, latent_frames: int, frames_per_pass: int, first_frame_rule: bool = True) -> int:
        total, start = 0, 0
        while start < latent_frames:
            n = min(frames_per_pass, latent_frames - start)
            total += lib().wvd_chunk_video_frames(ctypes.byref(self.desc), n, int(start == 0), int(first_frame_rule))
            start += n
        return total

    def workspace(self, frames_per_pass: int, early_frames_per_pass: Optional[int] = None) -> torch.Tensor:
        early = max(early_frames_per_pass or frames_per_pass, frames_per_pass)
        key = (early, frames_per_pass if early > frames_per_pass else 0)
        if self._ws is None or self._ws_frames != key:
            if key[1]:
                nbytes = lib().wvd_decode_workspace_bytes_split(ctypes.byref(self.desc), key[0], key[1])
            else:
                nbytes = lib().wvd_decode_workspace_bytes(ctypes.byref(self.desc), key[0])
            self._ws = None
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self._ws_frames = key
        return self._ws

    def decode(self, z: torch.Tensor, frames_per_pass: int = 4, first_frame_rule: bool = True,
               out: Optional[torch.Tensor] = None, z_layout: str = "NCTHW",
               early_frames_per_pass: Optional[int] = None) -> torch.Tensor:
        """z: bf16 latents [1, C, T, h, w] (NCTHW, default) or [1, T, h, w, C] (NTHWC).
        early_frames_per_pass > frames_per_pass: the stages up to the last temporal upsample take
        that many latent frames per pass, the later ones (and the memory they need) still
        frames_per_pass (wvd_decode_chunk_split); the video is the same bits."""
        if frames_per_pass < 1:
            raise ValueError("frames_per_pass must be at least 1")
        early = max(early_frames_per_pass or frames_per_pass, frames_per_pass)
        T = z.shape[2] if z_layout == "NCTHW" else z.shape[1]
        F = self.video_frames(T, frames_per_pass, first_frame_rule)
        if out is None:
            out = torch.empty(video_shape(self.desc, F), dtype=torch.bfloat16, device=self.device)
        ws = self.workspace(frames_per_pass, early)
        _check(lib().wvd_cache_reset(self.cache))
        start, offset = 0, 0
        while start < T:
            n = min(early, T - start)
            zc = z[:, :, start:start + n] if z_layout == "NCTHW" else z[:, start:start + n]
            zc = zc.contiguous()
            first = int(start == 0)
            if early > frames_per_pass:
                _check(lib().wvd_decode_chunk_split(ctypes.byref(self.desc), _ptr(self.packed), self.cache,
                                                    _desc(zc, z_layout), first, int(first_frame_rule),
                                                    ctypes.byref(ncthw(out)), offset, frames_per_pass, _ptr(ws),
                                                    ws.numel(), _stream()))
            else:
                _check(lib().wvd_decode_chunk(ctypes.byref(self.desc), _ptr(self.packed), self.cache,
                                              _desc(zc, z_layout), first, int(first_frame_rule),
                                              ctypes.byref(ncthw(out)), offset, _ptr(ws), ws.numel(), _stream()))
            offset += lib().wvd_chunk_video_frames(ctypes.byref(self.desc), n, first, int(first_frame_rule))
            start += n
        return out


# ------------------------------------------------------------------------------------------------
# Timing
# ------------------------------------------------------------------------------------------------
def timing_enable(on: bool = True):
    _check(lib().wvd_timing_enable(int(on)))


def timing_reset():
    _check(lib().wvd_timing_reset())


def timing_read():
    """{config name: (launches, total ms, total algorithmic flops)} of the matrix-core conv kernel."""
    L = lib()
    n = L.wvd_timing_read(-1, None, None, None, None)
    out = {}
    for i in range(n):
        name = ctypes.c_char_p()
        launches = ctypes.c_int64()
        ms = ctypes.c_double()
        flops = ctypes.c_double()
        L.wvd_timing_read(i, ctypes.byref(name), ctypes.byref(launches), ctypes.byref(ms), ctypes.byref(flops))
        if launches.value:
            out[name.value.decode()] = (launches.value, ms.value, flops.value)
    return out


def timing_read_mem():
    """{kernel kind: (launches, total ms, total algorithmic bytes)} of the memory-bound kernels."""
    L = lib()
    n = L.wvd_timing_read_mem(-1, None, None, None, None)
    out = {}
    for i in range(n):
        name = ctypes.c_char_p()
        launches = ctypes.c_int64()
        ms = ctypes.c_double()
        nbytes = ctypes.c_double()
        L.wvd_timing_read_mem(i, ctypes.byref(name), ctypes.byref(launches), ctypes.byref(ms), ctypes.byref(nbytes))
        if launches.value:
            out[name.value.decode()] = (launches.value, ms.value, nbytes.value)
    return out


def conv_config_names():
    """Names of the matrix-core conv configurations, by index."""
    L = lib()
    out = []
    for i in range(L.wvd_timing_read(-1, None, None, None, None)):
        nm = ctypes.c_char_p()
        L.wvd_timing_read(i, ctypes.byref(nm), None, None, None)
        out.append(nm.value.decode())
    return out


def conv_force_config(config):
    """Run every following conv launch with configuration `config` (index or name), or with the
    automatic choice when config is None or -1 (testing and tuning)."""
    if config is None:
        config = -1
    elif isinstance(config, str):
        config = conv_config_names().index(config)
    _check(lib().wvd_conv_force_config(int(config)))


def decode_fuse_norm1(on: bool):
    """wvd_decode_fuse_norm1: apply each residual block's norm1 + SiLU in the producing conv's
    epilogue (two outputs; the default) or, with False, as a separate pass."""
    _check(lib().wvd_decode_fuse_norm1(int(on)))


def decode_fuse_shortcut(on: bool):
    """wvd_decode_fuse_shortcut: apply a 192 -> 96 residual block's 1x1 shortcut in the epilogue
    of the x2 upsample that produces its input (default on)."""
    _check(lib().wvd_decode_fuse_shortcut(int(on)))


def fuse_norm_shortcut(on: bool):
    """wvd_fuse_norm_shortcut: run a 384 -> (up to) 192 residual block's norm1 + SiLU and its 1x1
    shortcut as one pass over its input (default on; the same bits either way)."""
    _check(lib().wvd_fuse_norm_shortcut(int(on)))


def decode_fuse_head(on: bool):
    """wvd_decode_fuse_head: run the last x2 upsample, norm_out + SiLU and the head as one kernel
    where the decoder allows it (less memory, slower) or, with False (the default), through the
    activated tensor. Caches and workspaces follow the switch: make them after setting it."""
    _check(lib().wvd_decode_fuse_head(int(on)))


def calib_dma_copy(src: torch.Tensor, dst: torch.Tensor):
    """wvd_calib_dma_copy: copy src into dst (same byte size) through the conv kernels' load path."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst sizes differ")
    _check(lib().wvd_calib_dma_copy(_ptr(src), _ptr(dst), n, _stream()))
    return dst


def conv_max_workgroups(n):
    """Cap the workgroups of the following multi-tile halo conv launches at n (0 or None: default);
    every workgroup then walks a longer run of tiles (testing)."""
    _check(lib().wvd_conv_max_workgroups(int(n or 0)))


def timing_launches():
    """Every timed conv launch since the last reset: (config name, ms, flops, shape dict)."""
    L = lib()
    n = L.wvd_timing_launch(-1, None, None, None, None)
    names = {}
    for i in range(L.wvd_timing_read(-1, None, None, None, None)):
        nm = ctypes.c_char_p()
        L.wvd_timing_read(i, ctypes.byref(nm), None, None, None)
        names[i] = nm.value.decode()
    out = []
    for i in range(n):
        cfg = ctypes.c_int()
        ms = ctypes.c_double()
        fl = ctypes.c_double()
        sh = (ctypes.c_int * 10)()
        L.wvd_timing_launch(i, ctypes.byref(cfg), ctypes.byref(ms), ctypes.byref(fl), sh)
        out.append((names.get(cfg.value, "?"), ms.value, fl.value,
                    dict(zip(("T", "H", "W", "Ci", "N", "taps", "phases", "Th", "copied", "res"), list(sh)))))
    return out
