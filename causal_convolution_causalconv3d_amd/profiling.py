"""Measurement support: rocprofv3 summaries and the HBM traffic of the conv kernels.

* ``copy_calibration_run(mib)`` runs a plain elementwise copy (y = -x, fp32) over ``mib`` MiB three
  times. Under ``rocprofv3 --pmc FETCH_SIZE`` (then ``--pmc WRITE_SIZE``) its per-dispatch
  counters give the factor between what the counters report and the bytes really moved, which
  then scales the counters of the conv kernel.
* ``kernel_sources_sha256()`` hashes the conv kernels' sources; a traffic figure is only valid
  for the sources it was measured on.
* ``committed_traffic(config)`` returns the HBM bytes per launch recorded for a conv
  configuration in ``profiles/<config>_hbm_traffic_*.md`` when the recorded source hash matches
  the current sources, else None.

Command line (prints markdown):
  python -m causal_convolution_causalconv3d_amd.profiling stats <rocprof kernel_stats.csv> [--command CMD]
  python -m causal_convolution_causalconv3d_amd.profiling traffic --config NAME --fetch DIR --write DIR
      --copy-fetch DIR --copy-write DIR --copy-mib N [--copy-kernel neg|dma_copy] [--workload TEXT]
      [--command CMD ...]
  python -m causal_convolution_causalconv3d_amd.profiling mfma <rocprof counter_collection.csv> [--command CMD]
  python -m causal_convolution_causalconv3d_amd.profiling calib --fetch DIR --write DIR --copy-mib N [--command CMD ...]
  python -m causal_convolution_causalconv3d_amd.profiling lds <rocprof counter_collection.csv> [--command CMD]
  python -m causal_convolution_causalconv3d_amd.profiling hbm [--topology real] [--frames-per-pass N]
      [--early-frames-per-pass N]   (host only: the peak's items from the library's size queries)
"""
import argparse
import csv
import glob
import hashlib
import os
import re
import sys
from typing import Dict, List, Optional

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
KERNEL_SOURCES = ("conv_mfma.hip", "conv_epilogue.h", "common.h")


def kernel_sources_sha256() -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def _keyvals(path: str) -> Dict[str, str]:
    out = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^\s*[-*]?\s*`?([a-z_0-9]+)`?\s*:\s*`?([^`\s]+)`?\s*$", line)
            if m:
                out[m.group(1)] = m.group(2)
    return out


def committed_traffic(config: str) -> Optional[int]:
    """HBM bytes per launch of `config` from its committed traffic summary, if still valid."""
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"{config}_hbm_traffic_*.md"))):
        kv = _keyvals(path)
        if kv.get("config") == config and kv.get("kernel_sources_sha256") == kernel_sources_sha256():
            try:
                return int(float(kv["hbm_bytes_per_launch"]))
            except (KeyError, ValueError):
                return None
    return None


def copy_calibration_run(mib: int) -> None:
    import torch

    n = mib * (1 << 20) // 4
    x = torch.randn(n, device="cuda")
    y = torch.empty_like(x)
    torch.neg(x, out=y)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(f"copy calibration: 3 dispatches of y = -x over {mib} MiB ({n * 4} bytes read and written each)", flush=True)
    # the same bytes through the conv kernels' 16-byte buffer-load-to-LDS path
    import causal_convolution_causalconv3d_amd as wvd

    wvd.calib_dma_copy(x, y)
    torch.cuda.synchronize()
    assert torch.equal(x, y), "DMA copy mismatch"
    for _ in range(3):
        wvd.calib_dma_copy(x, y)
    torch.cuda.synchronize()
    print(f"copy calibration: 3 dispatches of dma_copy_kernel over {mib} MiB ({n * 4} bytes read and written each)",
          flush=True)


def kernel_symbol(config: str) -> str:
    """The demangled name prefix shared by a configuration's kernels (its plain and fused-norm
    epilogue instantiations)."""
    m = re.fullmatch(r"conv_(mfma|halo|phase_halo|halo_dma|phase_halo_dma)_n(\d+)_m(\d+)_w(\d+)", config)
    if not m:
        raise ValueError(f"unknown conv configuration {config}")
    kind, nb, mb, w = m.groups()
    if kind == "mfma":
        return f"conv_mfma_kernel<{nb}, {mb}, {w}, "
    ks = 2 if kind.startswith("phase") else 3
    base = "conv_halo_dma_kernel" if kind.endswith("dma") else "conv_halo_kernel"
    return f"{base}<{nb}, {mb}, {w}, {ks}, "


def _counter_rows(d: str) -> List[dict]:
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(d: str, counter: str, match) -> List[float]:
    acc: Dict[str, float] = {}
    for r in _counter_rows(d):
        if r["Counter_Name"] != counter or not match(r["Kernel_Name"]):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    return list(acc.values())


COPY_KERNELS = {"neg": "y = -x, fp32, a plain elementwise copy",
                "dma_copy": "dma_copy_kernel: 16-byte buffer loads into LDS, the conv kernels' load path"}


def calib_summary(fetch: str, write: str, copy_mib: int, commands: List[str]) -> str:
    """The counter-to-bytes factors of the two calibration copies side by side."""
    copy_bytes = copy_mib * (1 << 20)
    lines = ["# Counter calibration: FETCH_SIZE / WRITE_SIZE of copies of known size", "",
             f"Each copy reads and writes {copy_mib} MiB per dispatch; the factor turns the counter into bytes",
             "(true bytes / counted bytes, mean of the last 3 dispatches of each copy).", "", "Commands:", ""]
    lines += [f"    {c}" for c in commands]
    lines += ["", "| copy | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch factor | write factor |", "|---|---:|---:|---:|---:|"]
    for key, what in COPY_KERNELS.items():
        cf = _per_dispatch(fetch, "FETCH_SIZE", lambda n, k=key: k in n)
        cw = _per_dispatch(write, "WRITE_SIZE", lambda n, k=key: k in n)
        if not (cf and cw):
            raise RuntimeError(f"no dispatches of {key} in the counter files")
        f_kib, w_kib = sum(cf[-3:]) / len(cf[-3:]), sum(cw[-3:]) / len(cw[-3:])
        lines.append(f"| {what} | {f_kib:.1f} | {w_kib:.1f} | {copy_bytes / (f_kib * 1024):.4f} | "
                     f"{copy_bytes / (w_kib * 1024):.4f} |")
    return "\n".join(lines) + "\n"


STREAM_DECODE = "the streaming decode (704x1248, 4 latent frames per pass)"


def traffic_summary(config: str, fetch: str, write: str, copy_fetch: str, copy_write: str, copy_mib: int,
                    commands: List[str], copy_kernel: str = "neg", workload: str = STREAM_DECODE) -> str:
    sym = kernel_symbol(config)
    is_kernel = lambda name: sym in name  # noqa: E731
    is_copy = lambda name: copy_kernel in name  # noqa: E731
    kf = _per_dispatch(fetch, "FETCH_SIZE", is_kernel)
    kw = _per_dispatch(write, "WRITE_SIZE", is_kernel)
    cf = _per_dispatch(copy_fetch, "FETCH_SIZE", is_copy)
    cw = _per_dispatch(copy_write, "WRITE_SIZE", is_copy)
    if not (kf and kw and cf and cw):
        raise RuntimeError("missing dispatches in the counter files")
    copy_bytes = copy_mib * (1 << 20)
    # the copy's last dispatches (after the warm-up one)
    cf_kib, cw_kib = sum(cf[-3:]) / len(cf[-3:]), sum(cw[-3:]) / len(cw[-3:])
    f_scale = copy_bytes / (cf_kib * 1024.0)
    w_scale = copy_bytes / (cw_kib * 1024.0)
    kf_kib, kw_kib = sum(kf) / len(kf), sum(kw) / len(kw)
    fetch_b = kf_kib * 1024.0 * f_scale
    write_b = kw_kib * 1024.0 * w_scale
    lines = [
        f"# HBM traffic of {config} in {workload}",
        "",
        "Counters: rocprofv3 `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE` (KiB per dispatch), one run each,",
        "averaged over every dispatch of the kernel; scaled by the same counters on a copy kernel",
        f"({COPY_KERNELS[copy_kernel]}; {copy_mib} MiB read and written per dispatch, mean of its last 3 dispatches).",
        "",
        "Commands:",
        "",
    ]
    lines += [f"    {c}" for c in commands]
    lines += [
        "",
        "| quantity | value |",
        "|---|---|",
        f"| kernel dispatches (fetch run / write run) | {len(kf)} / {len(kw)} |",
        f"| FETCH_SIZE per dispatch (KiB, raw) | {kf_kib:.1f} |",
        f"| WRITE_SIZE per dispatch (KiB, raw) | {kw_kib:.1f} |",
        f"| copy FETCH_SIZE per dispatch (KiB) / true | {cf_kib:.1f} / {copy_bytes / 1024:.1f} |",
        f"| copy WRITE_SIZE per dispatch (KiB) / true | {cw_kib:.1f} / {copy_bytes / 1024:.1f} |",
        f"| fetch scale / write scale | {f_scale:.4f} / {w_scale:.4f} |",
        f"| HBM read per launch (bytes, scaled) | {fetch_b:.4g} |",
        f"| HBM write per launch (bytes, scaled) | {write_b:.4g} |",
        "",
        f"- config: `{config}`",
        f"- kernel_sources_sha256: `{kernel_sources_sha256()}`",
        f"- hbm_bytes_per_launch: `{int(round(fetch_b + write_b))}`",
        "",
    ]
    return "\n".join(lines)


def stats_summary(path: str, command: str, top: int = 25) -> str:
    with open(path) as f:
        rows = list(csv.DictReader(f))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = ["Command:", "", f"    {command}", "",
           "| kernel | calls | total ms | avg us | share |", "|---|---:|---:|---:|---:|"]
    for r in rows[:top]:
        name = r["Name"]
        name = re.sub(r"\(wvd::ConvProblem\)$", "", name)
        name = name.replace("void wvd::(anonymous namespace)::", "")
        if len(name) > 90:
            name = name[:87] + "..."
        t = float(r["TotalDurationNs"])
        out.append(f"| `{name}` | {r['Calls']} | {t / 1e6:.2f} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{100.0 * t / total:.1f}% |")
    out.append(f"| all kernels | {sum(int(r['Calls']) for r in rows)} | {total / 1e6:.2f} | | 100% |")
    return "\n".join(out) + "\n"


def mfma_summary(path: str, command: str, top: int = 12, simds: int = 1024, xcds: int = 8) -> str:
    """MFMA-busy share per kernel from one `--pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES ...`
    run: SQ_VALU_MFMA_BUSY_CYCLES / (kernel cycles x SIMDs), the kernel cycles being
    GRBM_GUI_ACTIVE (summed over the XCDs) / XCDs; also the clock those cycles imply over the
    dispatches' durations."""
    acc: Dict[str, Dict[str, float]] = {}
    dur: Dict[str, float] = {}
    seen = set()
    with open(path) as f:
        for r in csv.DictReader(f):
            name = re.sub(r"\(wvd::ConvProblem\)$", "", r["Kernel_Name"]).replace("void wvd::(anonymous namespace)::", "")
            name = name if len(name) <= 70 else name[:67] + "..."
            c = acc.setdefault(name, {})
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if r["Dispatch_Id"] not in seen:
                seen.add(r["Dispatch_Id"])
                dur[name] = dur.get(name, 0.0) + (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    rows = sorted(acc.items(), key=lambda kv: -dur[kv[0]])[:top]
    out = ["Command:", "", f"    {command}", "",
           "| kernel | ms | clock GHz | MFMA busy |", "|---|---:|---:|---:|"]
    for name, c in rows:
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        busy = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / max(cyc * simds, 1.0)
        out.append(f"| `{name}` | {1e3 * dur[name]:.2f} | {cyc / max(dur[name], 1e-12) / 1e9:.2f} | {100 * busy:.1f}% |")
    return "\n".join(out) + "\n"


def lds_summary(path: str, command: str, top: int = 12) -> str:
    """LDS bank-conflict share per kernel from one `--pmc SQ_LDS_BANK_CONFLICT SQ_LDS_IDX_ACTIVE ...`
    run: bank-conflict cycles / LDS-active (indexed) cycles, summed over the kernel's dispatches."""
    acc: Dict[str, Dict[str, float]] = {}
    dur: Dict[str, float] = {}
    seen = set()
    with open(path) as f:
        for r in csv.DictReader(f):
            name = re.sub(r"\(wvd::ConvProblem\)$", "", r["Kernel_Name"]).replace("void wvd::(anonymous namespace)::", "")
            name = name if len(name) <= 70 else name[:67] + "..."
            c = acc.setdefault(name, {})
            c[r["Counter_Name"]] = c.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if r["Dispatch_Id"] not in seen:
                seen.add(r["Dispatch_Id"])
                dur[name] = dur.get(name, 0.0) + (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    rows = sorted(acc.items(), key=lambda kv: -dur[kv[0]])[:top]
    out = ["Command:", "", f"    {command}", "",
           "| kernel | ms | LDS bank-conflict cycles / LDS-active cycles |", "|---|---:|---:|"]
    for name, c in rows:
        act = c.get("SQ_LDS_IDX_ACTIVE", 0.0)
        out.append(f"| `{name}` | {1e3 * dur[name]:.2f} | "
                   f"{(100 * c.get('SQ_LDS_BANK_CONFLICT', 0.0) / act) if act else 0.0:.1f}% |")
    return "\n".join(out) + "\n"


def hbm_summary(topology: str, latent_frames: int, fpp: int, early: int) -> str:
    """Device memory a streaming decode holds at its peak, item by item, from the library's own
    size queries (host only): packed weights, the double-buffered cache, the workspace (split into
    the buffers the layout sizes), the whole video and the latents."""
    import ctypes

    import causal_convolution_causalconv3d_amd as wvd
    import workloads as wl

    spec = wl.REAL_DECODER if topology == "real" else wl.FULL_DECODER
    d = wvd.desc_from_spec(spec)
    L = wvd.lib()
    dec_frames = 0
    start = 0
    while start < latent_frames:
        n = min(fpp, latent_frames - start)
        dec_frames += L.wvd_chunk_video_frames(ctypes.byref(d), n, int(start == 0), 1)
        start += n
    early = max(early, fpp)
    ws = (L.wvd_decode_workspace_bytes_split(ctypes.byref(d), early, fpp) if early > fpp
          else L.wvd_decode_workspace_bytes(ctypes.byref(d), fpp))
    items = [("packed weights (bf16, channel-padded)", L.wvd_decoder_packed_bytes(ctypes.byref(d))),
             ("cache (one slot per causal conv, two halves of two frames)", L.wvd_cache_bytes(ctypes.byref(d))),
             (f"workspace ({early} latent frames per pass through the early stages, {fpp} through the late ones)", ws),
             (f"video [1,3,{dec_frames},704,1248] bf16", 3 * dec_frames * 704 * 1248 * 2),
             (f"latents [1,48,{latent_frames},44,78] bf16", 48 * latent_frames * 44 * 78 * 2)]
    total = sum(b for _, b in items)
    out = ["| item | GiB |", "|---|---:|"]
    out += [f"| {k} | {b / 2 ** 30:.3f} |" for k, b in items]
    out.append(f"| sum | {total / 2 ** 30:.3f} |")
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m causal_convolution_causalconv3d_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    st = sub.add_parser("stats")
    st.add_argument("csv")
    st.add_argument("--command", default="")
    tr = sub.add_parser("traffic")
    tr.add_argument("--config", required=True)
    for k in ("fetch", "write", "copy-fetch", "copy-write"):
        tr.add_argument(f"--{k}", required=True)
    tr.add_argument("--copy-mib", type=int, required=True)
    tr.add_argument("--copy-kernel", choices=sorted(COPY_KERNELS), default="neg")
    tr.add_argument("--workload", default=STREAM_DECODE, help="what the counted run decoded (the title)")
    tr.add_argument("--command", action="append", default=[])
    ca = sub.add_parser("calib")
    ca.add_argument("--fetch", required=True)
    ca.add_argument("--write", required=True)
    ca.add_argument("--copy-mib", type=int, required=True)
    ca.add_argument("--command", action="append", default=[])
    mf = sub.add_parser("mfma")
    mf.add_argument("csv")
    mf.add_argument("--command", default="")
    hb = sub.add_parser("hbm")
    hb.add_argument("--topology", choices=("synthetic", "real"), default="synthetic")
    hb.add_argument("--latent-frames", type=int, default=31)
    hb.add_argument("--frames-per-pass", type=int, default=4)
    hb.add_argument("--early-frames-per-pass", type=int, default=0)
    ld = sub.add_parser("lds")
    ld.add_argument("csv")
    ld.add_argument("--command", default="")
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        sys.stdout.write(stats_summary(a.csv, a.command))
    elif a.cmd == "mfma":
        sys.stdout.write(mfma_summary(a.csv, a.command))
    elif a.cmd == "hbm":
        sys.stdout.write(hbm_summary(a.topology, a.latent_frames, a.frames_per_pass, a.early_frames_per_pass))
    elif a.cmd == "lds":
        sys.stdout.write(lds_summary(a.csv, a.command))
    elif a.cmd == "calib":
        sys.stdout.write(calib_summary(a.fetch, a.write, a.copy_mib, a.command))
    else:
        sys.stdout.write(traffic_summary(a.config, a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_mib, a.command,
                                         a.copy_kernel, a.workload))


if __name__ == "__main__":
    main()
