#!/usr/bin/env python3
"""Benchmark: chunked prefill of recurrent mixers on one MI355X.

One step = one pass of the whole hot path over the batched mixed workload:
16 prompts of U{1..4096} rows (seeded), each prefilled in 64-row chunks with
its state carried between chunks, through
  1. the Mamba short conv   (K=4, 5120 fp32 channels)
  2. the Mamba selective scan (d_inner 5120 x d_state 16, fp32)
  3. RWKV-4 WKV             (hidden 2560, fp32)
  4. the DeltaNet short conv (K=4, 2*16*128 + 32*128 = 8192 bf16 channels)
  5. the Gated DeltaNet chunk (32 value heads on 16 key heads, 128 x 128, bf16 in, fp32 state)
Inputs are synthetic and already resident in HBM when timing starts.

Prints ONE JSON line.  `value` is prompt rows per second through the whole
step.  Per-kernel times come from HIP events on the stream the kernels run
on; `roofline` covers the kernel with the largest share of the step.
`cpu_baseline` times the float64 oracle (test infrastructure) on a bounded
sample of the same workload on the host cores, and on one core.
`per_config` repeats the measurement for every kernel at each workload of the
metric (Mamba tiny, RWKV-4 169M-like, DeltaNet small, DeltaNet 9B-like, and
the mixed step itself): time, rows/s and roofline fraction on the GPU, and, in
the oracle leg, max rel err of every output and state tensor against the
float64 oracle run from the same incoming state, plus the oracle's own rows/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
MFMA_FP32_PEAK_TFS = 157.3  # MI355X dense fp32 MFMA, TFLOP/s
FP32_VEC_PEAK_TFS = 157.3    # MI355X fp32 vector, TFLOP/s


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing on the host")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="target seconds of oracle work")
    ap.add_argument("--only", default="", help="comma list of kernels to run (profiling aid)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-config table (cfg1..cfg4)")
    ap.add_argument("--no-extra-legs", action="store_true",
                    help="time only the step's own launches: no split-form or FP32-input DeltaNet legs, "
                         "no rows beyond the step (profiling aid)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 4 GiB device copy (for scaling HBM counters) and exit")
    return ap.parse_args()


# ----------------------------------------------------------------------------- workload
def make_workload(dev):
    import torch

    from linear_recurrence_chunked_amd import inputs, lrc

    lens = inputs.mixed_lengths()
    sh = inputs.MIXED_SHAPES
    m = inputs.mixed_mamba(lens, dev)
    r = inputs.mixed_rwkv(lens, dev)
    g = inputs.mixed_gdn(lens, dev)
    R = sum(lens)
    D, N = sh["mamba_d_inner"], sh["mamba_d_state"]
    W = {
        "lens": lens, "R": R,
        # Mamba conv + scan
        "xm": m["conv_x"], "ym": torch.empty_like(m["conv_x"]), "sm": m["conv_state"], "wm": m["conv_w"],
        "a": m["a"].view(R, D, N), "b": m["b"].view(R, D, N), "h": torch.empty((R, D, N), device=dev),
        "hs": m["h0"].view(len(lens), D, N),
        # the tiled scan's completion flags (zero-filled once, reused by every step)
        "scan_ws": torch.zeros(lrc.scan_workspace_size(len(lens), D, N), dtype=torch.uint8, device=dev),
        # RWKV-4
        "k": r["k"], "v": r["v"], "w": r["w"], "u": r["u"], "wkv": torch.empty_like(r["k"]),
        "num": r["num"], "den": r["den"], "max": r["max"],
        # DeltaNet conv + chunk
        "xg": g["conv_x"], "yg": torch.empty_like(g["conv_x"]), "sg": g["conv_state"], "wg": g["conv_w"],
        "q": g["q"], "gk": g["k"], "gv": g["v"], "beta": g["beta"], "g": g["g"],
        "o": torch.empty((R, sh["gdn_hv"], sh["gdn_dv"]), device=dev), "S": g["S0"],
    }
    return W


KERNELS = ["conv_mamba", "scan", "wkv4", "conv_gdn", "gdn"]
# Oracle sample for the CPU baseline: every prompt and row; every n-th channel or
# state element per kernel (every DeltaNet head); about 10 s of float64 work
# on 16 threads, bounded by the host memory the scan's float64 copies take.
SAMPLE_STRIDE = {"conv_mamba": 1, "scan": 2, "wkv4": 1, "conv_gdn": 1}
# HIP source of each kernel (its hash ties a stored counter measurement to the code measured)
KERNEL_SOURCE = {"conv_mamba": "conv.hip", "scan": "scan.hip", "wkv4": "wkv4.hip", "conv_gdn": "conv.hip",
                 "gdn": "gdn_mfma.hip"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_mixed_prefill.md")


def source_sha(kernel: str) -> str:
    """Hash of the kernel's HIP source with comments and whitespace removed, so
    that only a change to the code itself invalidates a stored measurement."""
    path = os.path.join(ROOT, "linear_recurrence_chunked_amd", "csrc", KERNEL_SOURCE[kernel])
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()


def stored_traffic(kernel: str):
    """HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a plain
    copy's reading), from the committed summary; None if absent or if the kernel's source
    changed since the counters were taken."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    if not m:
        return None
    rec = json.loads(m.group(1)).get(kernel)
    if not rec or rec.get("source_sha256") != source_sha(kernel):
        return None
    return rec.get("traffic_bytes_per_launch")


def measure_copy_gbps(dev, nbytes=4 << 30, reps=5):
    """Read+write bandwidth of a plain device-to-device copy on this GPU (GB/s)."""
    import torch

    src = torch.empty(nbytes // 4, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * nbytes / (ms * 1e-3) / 1e9


def measure_add_gbps(dev, nbytes=2 << 30, reps=5):
    """Bandwidth of torch's elementwise add c = a + b (two reads per write, the scan's mix; GB/s)."""
    import torch

    a = torch.empty(nbytes // 4, device=dev)
    b, c = torch.empty_like(a), torch.empty_like(a)
    torch.add(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.add(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return 3 * nbytes / (ms * 1e-3) / 1e9


def run_kernel(lrc, W, name):
    lens = W["lens"]
    if name == "conv_mamba":
        lrc.conv_prefill(W["xm"], W["ym"], W["sm"], W["wm"], lens)
    elif name == "scan":
        lrc.scan_prefill_ws(W["a"], W["b"], W["h"], W["hs"], lens, W["scan_ws"])
    elif name == "wkv4":
        lrc.wkv4_prefill(W["k"], W["v"], W["w"], W["u"], W["wkv"], W["num"], W["den"], W["max"], lens)
    elif name == "conv_gdn":
        lrc.conv_prefill(W["xg"], W["yg"], W["sg"], W["wg"], lens)
    elif name == "gdn":
        lrc.gdn_prefill(W["q"], W["gk"], W["gv"], W["beta"], W["g"], W["o"], W["S"], lens)
    else:
        raise KeyError(name)


def algorithmic_work(W):
    """Bytes (and flops for the DeltaNet chunk) one launch of each kernel must move/do."""
    from linear_recurrence_chunked_amd import inputs

    sh = inputs.MIXED_SHAPES
    lens, R, P = W["lens"], W["R"], len(W["lens"])
    K = sh["conv_k"]
    Cm, Cg, Cr = sh["mamba_conv_c"], sh["gdn_conv_c"], sh["rwkv_c"]
    E = sh["mamba_d_inner"] * sh["mamba_d_state"]
    Hk, Hv, dk, dv = sh["gdn_hk"], sh["gdn_hv"], sh["gdn_dk"], sh["gdn_dv"]
    grp = Hv // Hk
    work = {
        # rows in + rows out, state rows read + written, taps once
        "conv_mamba": {"bytes": R * Cm * 8 + P * 2 * (K - 1) * Cm * 4 + Cm * K * 4},
        "scan": {"bytes": R * E * 12 + P * E * 8},
        "wkv4": {"bytes": R * Cr * 12 + P * Cr * 24 + Cr * 8},
        "conv_gdn": {"bytes": R * Cg * 4 + P * 2 * (K - 1) * Cg * 2 + Cg * K * 4},
        "gdn": {"bytes": R * (2 * Hk * dk * 2 + Hv * dv * 2 + Hv * 8 + Hv * dv * 4) + P * Hv * dk * dv * 8},
    }
    # Dense-contraction flops the chunk form prescribes, per value head and
    # chunk of r rows: K K^T and Q K^T (shared by the value heads of a key
    # head), K S0, Q S0, the state update, T (I+A)^-1 applied to the right-
    # hand side, P U, plus the 64-row block inverse.
    inv = 8 * 4 * 2 * 8 ** 3 + sum((64 // (2 * s)) * 2 * 2 * s ** 3 for s in (8, 16, 32))
    fl = 0
    for L in lens:
        for c0 in range(0, L, 64):
            r = min(64, L - c0)
            per_head = (2 * 2 * r * r * dk) / grp + 3 * 2 * r * dk * dv + 2 * 2 * r * r * dv + inv
            fl += per_head * Hv
    work["gdn"]["flops"] = fl
    return work


# ----------------------------------------------------------------------------- oracle sample
def cpu_baseline(W, lrc_outputs_fresh, budget_s):
    """Time the float64 oracle on a bounded sample of the workload (every prompt,
    a strided subset of channels / state elements / heads of each kernel), scale
    each kernel's time by its sampled fraction, and report rows/s for the whole
    step.  Also returns the GPU's max rel err on the same sample."""
    import numpy as np
    import torch

    import oracle

    from linear_recurrence_chunked_amd import inputs

    oracle.build(force=False)
    sh = inputs.MIXED_SHAPES
    lens, R = W["lens"], W["R"]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    fresh = lrc_outputs_fresh
    # sample fractions (fraction of the kernel's independent units)
    Cm, Cg, Cr = sh["mamba_conv_c"], sh["gdn_conv_c"], sh["rwkv_c"]
    E = sh["mamba_d_inner"] * sh["mamba_d_state"]
    Hk, Hv = sh["gdn_hk"], sh["gdn_hv"]
    sel = {
        "conv_mamba": np.arange(0, Cm, SAMPLE_STRIDE["conv_mamba"]),
        "scan": np.arange(0, E, SAMPLE_STRIDE["scan"]),
        "wkv4": np.arange(0, Cr, SAMPLE_STRIDE["wkv4"]),
        "conv_gdn": np.arange(0, Cg, SAMPLE_STRIDE["conv_gdn"]),
        "gdn_keyheads": np.arange(Hk),  # every key head and its value heads
    }
    f64 = lambda t: t.detach().cpu().double().numpy()  # noqa: E731
    t_kernel, err = {}, {}

    def rel(got, ref):
        s = np.max(np.abs(ref)) if ref.size else 0.0
        return float(np.max(np.abs(got - ref)) / (s if s else 1.0)) if ref.size else 0.0

    # conv (Mamba, fp32) -- fresh state is zero
    c = torch.as_tensor(sel["conv_mamba"], device=W["xm"].device)
    x = f64(W["xm"][:, c]); wt = f64(W["wm"][c]); y = fresh["ym"]
    t0 = time.perf_counter(); e = 0.0
    for p in range(len(lens)):
        ry, _ = oracle.conv_rows(x[offs[p]:offs[p + 1]], np.zeros((3, len(c))), wt)
        e = max(e, rel(y[offs[p]:offs[p + 1]], ry) if lens[p] else 0.0)
    t_kernel["conv_mamba"] = (time.perf_counter() - t0) * Cm / len(c); err["conv_mamba"] = e
    # scan
    ci = torch.as_tensor(sel["scan"], device=W["a"].device)
    a = f64(W["a"].view(R, -1)[:, ci]); b = f64(W["b"].view(R, -1)[:, ci]); h = fresh["h"]
    t0 = time.perf_counter(); e = 0.0
    for p in range(len(lens)):
        rh, _ = oracle.scan(a[offs[p]:offs[p + 1]], b[offs[p]:offs[p + 1]], np.zeros(len(ci)))
        e = max(e, rel(h[offs[p]:offs[p + 1]], rh) if lens[p] else 0.0)
    t_kernel["scan"] = (time.perf_counter() - t0) * E / len(ci); err["scan"] = e
    del a, b
    # wkv
    ci = torch.as_tensor(sel["wkv4"], device=W["k"].device)
    k = f64(W["k"][:, ci]); v = f64(W["v"][:, ci]); w = f64(W["w"][ci]); u = f64(W["u"][ci]); o = fresh["wkv"]
    t0 = time.perf_counter(); e = 0.0
    for p in range(len(lens)):
        ro, *_ = oracle.wkv4(k[offs[p]:offs[p + 1]], v[offs[p]:offs[p + 1]], w, u, *oracle.empty_wkv_state(len(ci)))
        e = max(e, rel(o[offs[p]:offs[p + 1]], ro) if lens[p] else 0.0)
    t_kernel["wkv4"] = (time.perf_counter() - t0) * Cr / len(ci); err["wkv4"] = e
    # conv (DeltaNet, bf16)
    c = torch.as_tensor(sel["conv_gdn"], device=W["xg"].device)
    x = f64(W["xg"][:, c]); wt = f64(W["wg"][c]); y = fresh["yg"]
    t0 = time.perf_counter(); e = 0.0
    for p in range(len(lens)):
        ry, _ = oracle.conv_rows(x[offs[p]:offs[p + 1]], np.zeros((3, len(c))), wt)
        e = max(e, rel(y[offs[p]:offs[p + 1]], ry) if lens[p] else 0.0)
    t_kernel["conv_gdn"] = (time.perf_counter() - t0) * Cg / len(c); err["conv_gdn"] = e
    # gated deltanet: two key heads and their value heads
    kh = torch.as_tensor(sel["gdn_keyheads"], device=W["q"].device)
    grp = Hv // Hk
    vh = torch.as_tensor(np.concatenate([np.arange(grp * i, grp * (i + 1)) for i in sel["gdn_keyheads"]]),
                         device=W["q"].device)
    q = f64(W["q"][:, kh]); kk = f64(W["gk"][:, kh]); vv = f64(W["gv"][:, vh])
    be = f64(W["beta"][:, vh]); gg = f64(W["g"][:, vh]); o = fresh["o"]
    dk, dv = q.shape[2], vv.shape[2]
    t0 = time.perf_counter(); eo = 0.0
    for p in range(len(lens)):
        sl = slice(offs[p], offs[p + 1])
        ro, _ = oracle.gdn(q[sl], kk[sl], vv[sl], be[sl], gg[sl], np.zeros((len(vh), dk, dv)))
        eo = max(eo, rel(o[sl], ro) if lens[p] else 0.0)
    t_kernel["gdn"] = (time.perf_counter() - t0) * Hv / len(vh); err["gdn"] = eo
    total = sum(t_kernel.values())
    sample_s = sum(t_kernel[n] * frac for n, frac in [
        ("conv_mamba", len(sel["conv_mamba"]) / Cm), ("scan", len(sel["scan"]) / E),
        ("wkv4", len(sel["wkv4"]) / Cr), ("conv_gdn", len(sel["conv_gdn"]) / Cg), ("gdn", len(vh) / Hv)])
    return {
        "value": R / total, "unit": "rows/s", "cores": oracle.num_threads(), "kind": "oracle",
        "sample": (f"all {len(lens)} prompts ({R} rows); every Mamba conv channel, "
                   f"one in {SAMPLE_STRIDE['scan']} scan state elements, every RWKV channel, every DeltaNet conv "
                   f"channel, every DeltaNet head; {sample_s:.1f} s of oracle time, each kernel's time "
                   f"scaled by its sampled fraction"),
        "seconds_per_step_estimated": total,
        "per_kernel_s": {n: round(t, 3) for n, t in t_kernel.items()},
    }, err


def cpu_baseline_one_thread(W):
    """The oracle on ONE host thread over a smaller strided sample of the same step (every prompt; one
    in 16 conv and RWKV channels, one in 64 scan state elements, one key head of DeltaNet with its
    value heads), each kernel's time scaled by its sampled fraction: whole-step rows/s on one core."""
    import numpy as np
    import torch

    import oracle

    from linear_recurrence_chunked_amd import inputs

    sh = inputs.MIXED_SHAPES
    lens, R = W["lens"], W["R"]
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    f64 = lambda t: t.detach().cpu().double().numpy()  # noqa: E731
    Cm, Cg, Cr = sh["mamba_conv_c"], sh["gdn_conv_c"], sh["rwkv_c"]
    E = sh["mamba_d_inner"] * sh["mamba_d_state"]
    Hk, Hv = sh["gdn_hk"], sh["gdn_hv"]
    grp = Hv // Hk
    nthreads = oracle.num_threads()
    oracle.set_num_threads(1)
    t = {}
    try:
        for name, xs, ws, units, stride in [("conv_mamba", "xm", "wm", Cm, 16), ("conv_gdn", "xg", "wg", Cg, 16)]:
            c = torch.arange(0, units, stride, device=W[xs].device)
            x, wt = f64(W[xs][:, c]), f64(W[ws][c])
            t0 = time.perf_counter()
            for p in range(len(lens)):
                oracle.conv_rows(x[offs[p]:offs[p + 1]], np.zeros((3, len(c))), wt)
            t[name] = (time.perf_counter() - t0) * units / len(c)
        ci = torch.arange(0, E, 64, device=W["a"].device)
        a, b = f64(W["a"].view(R, -1)[:, ci]), f64(W["b"].view(R, -1)[:, ci])
        t0 = time.perf_counter()
        for p in range(len(lens)):
            oracle.scan(a[offs[p]:offs[p + 1]], b[offs[p]:offs[p + 1]], np.zeros(len(ci)))
        t["scan"] = (time.perf_counter() - t0) * E / len(ci)
        ci = torch.arange(0, Cr, 16, device=W["k"].device)
        k, v, w, u = f64(W["k"][:, ci]), f64(W["v"][:, ci]), f64(W["w"][ci]), f64(W["u"][ci])
        t0 = time.perf_counter()
        for p in range(len(lens)):
            oracle.wkv4(k[offs[p]:offs[p + 1]], v[offs[p]:offs[p + 1]], w, u, *oracle.empty_wkv_state(len(ci)))
        t["wkv4"] = (time.perf_counter() - t0) * Cr / len(ci)
        q, kk = f64(W["q"][:, :1]), f64(W["gk"][:, :1])
        vv, be, gg = f64(W["gv"][:, :grp]), f64(W["beta"][:, :grp]), f64(W["g"][:, :grp])
        dk, dv = q.shape[2], vv.shape[2]
        t0 = time.perf_counter()
        for p in range(len(lens)):
            sl = slice(offs[p], offs[p + 1])
            oracle.gdn(q[sl], kk[sl], vv[sl], be[sl], gg[sl], np.zeros((grp, dk, dv)))
        t["gdn"] = (time.perf_counter() - t0) * Hk
    finally:
        oracle.set_num_threads(nthreads)
    total = sum(t.values())
    return {"value": R / total, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"all {len(lens)} prompts; one in 16 conv and RWKV channels, one in 64 scan state elements, "
                      f"one DeltaNet key head with its {grp} value heads; each kernel's time scaled by its sampled "
                      f"fraction",
            "per_kernel_s": {n: round(x, 3) for n, x in t.items()}}


# ----------------------------------------------------------------------------- per-config measurement
def gdn_chunk_flops(lens, Hk, Hv, dk, dv):
    """Dense-contraction flops of the chunk form over prompts of the given lengths (see algorithmic_work)."""
    grp = Hv // Hk
    inv = 8 * 4 * 2 * 8 ** 3 + sum((64 // (2 * s)) * 2 * 2 * s ** 3 for s in (8, 16, 32))
    fl = 0
    for L in lens:
        for c0 in range(0, L, 64):
            r = min(64, L - c0)
            fl += ((2 * 2 * r * r * dk) / grp + 3 * 2 * r * dk * dv + 2 * 2 * r * r * dv + inv) * Hv
    return fl


def _time_ms(fn, stream, reps):
    import torch

    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _entry(ms, rows, bound, work, peak):
    """rows/s and the roofline fraction of one launch (work in bytes for hbm, flops for mfma)."""
    rate = work / (ms * 1e-3)
    d = {"ms": round(ms, 5), "rows_per_s": rows / (ms * 1e-3), "bound": bound}
    if bound == "hbm":
        d.update({"GBps": rate / 1e9, "peak_GBps": peak, "frac": rate / 1e9 / peak, "algorithmic_bytes": work})
    else:
        d.update({"TFLOPs": rate / 1e12, "peak_TFLOPs": peak, "frac": rate / 1e12 / peak, "algorithmic_flops": work})
    return d


CONFIG_NAMES = {
    "cfg1_mamba_tiny": "Mamba tiny: d_inner 64, d_state 16, one 75-row prompt (64 + 11), fp32; conv K=4 over 64 channels",
    "cfg2_rwkv4_169m": "RWKV-4 169M-like: 768 x 12 = 9216 channels, one 128-row prompt (2 x 64), fp32, from a 32-step warm state",
    "cfg3_gdn_small": "Gated DeltaNet small: 8 heads, dk = dv = 64, one 75-row prompt (64 + 11); fp32, bf16, and bf16 with 16 "
                      "nearly parallel keys and beta = 0.99",
    "cfg4_gdn_9b": "Gated DeltaNet 9B-like: 32 value heads on 16 key heads, dk = dv = 128, one 2048-row prompt (32 x 64), "
                   "bf16 q/k/v, fp32 state and decays, g from -1e-3 to -8 per row; conv K=4 over 8192 bf16 channels",
    "cfg5_mixed": "batched mixed prefill (the step): 16 prompts of U{1..4096} rows through every kernel",
}


def measure_configs(lrc, dev, stream):
    """GPU times of every kernel at the four single-prompt configs (HIP events on the launch stream).
    Returns the per-config entries and the inputs, for the oracle leg."""
    import torch

    from linear_recurrence_chunked_amd import inputs

    out, keep = {}, {}
    g = lambda t: t.to(dev).contiguous()  # noqa: E731
    # --- cfg1: Mamba tiny, conv + tiled scan
    d = inputs.mamba_tiny()
    R, C, K = d["conv_x"].shape[0], d["conv_x"].shape[1], d["conv_w"].shape[1]
    E = d["a"].shape[1]
    x, w, st0 = g(d["conv_x"]), g(d["conv_w"]), g(d["conv_state"])[None]
    y, st = torch.empty_like(x), st0.clone()
    a, b = g(d["a"]).view(R, 64, 16), g(d["b"]).view(R, 64, 16)
    h, hs0 = torch.empty_like(a), g(d["h0"]).view(1, 64, 16)
    hs = hs0.clone()
    ws = lrc.scan_workspace(1, 64, 16, dev)
    k1 = {
        "conv": _entry(_time_ms(lambda: lrc.conv_prefill(x, y, st, w, [R]), stream, 200), R, "hbm",
                       R * C * 8 + 2 * (K - 1) * C * 4 + C * K * 4, HBM_PEAK_GBS),
        "scan": _entry(_time_ms(lambda: lrc.scan_prefill_ws(a, b, h, hs, [R], ws), stream, 200), R, "hbm",
                       R * E * 12 + E * 8, HBM_PEAK_GBS),
    }
    out["cfg1_mamba_tiny"] = {"workload": CONFIG_NAMES["cfg1_mamba_tiny"], "rows": R, "kernels": k1}
    keep["cfg1"] = d
    # --- cfg2: RWKV-4 169M-like
    r = inputs.rwkv_169m()
    R, C = r["k"].shape
    k_, v_, w_, u_ = (g(r[n]) for n in ("k", "v", "w", "u"))
    o2 = torch.empty_like(k_)
    num, den = torch.zeros((1, C), device=dev), torch.zeros((1, C), device=dev)
    mx = torch.full((1, C), -1e38, device=dev)
    k2 = {"wkv4": _entry(_time_ms(lambda: lrc.wkv4_prefill(k_, v_, w_, u_, o2, num, den, mx, [R]), stream, 100),
                         R, "hbm", R * C * 12 + C * 24 + C * 8, HBM_PEAK_GBS)}
    out["cfg2_rwkv4_169m"] = {"workload": CONFIG_NAMES["cfg2_rwkv4_169m"], "rows": R, "kernels": k2}
    keep["cfg2"] = r
    # --- cfg3: Gated DeltaNet small (fused kernel; fp32 inputs, bf16, bf16 stress; chunk-parallel bf16)
    k3 = {}
    keep["cfg3"] = {}
    for name, dd in [("gdn_f32", inputs.gdn_small(dtype=torch.float32)),
                     ("gdn_bf16", inputs.gdn_small(dtype=torch.bfloat16)),
                     ("gdn_bf16_16_parallel_keys",
                      inputs.gdn_small(dtype=torch.bfloat16, parallel_keys=16, parallel_start=24, beta_const=0.99)),
                     ("gdn_bf16_chunk_parallel", inputs.gdn_small(dtype=torch.bfloat16))]:
        q, kk, vv, be, gg = (g(dd[n]) for n in ("q", "k", "v", "beta", "g"))
        S = g(dd["S0"])[None].clone()
        R, Hk, dk = q.shape
        Hv, dv = vv.shape[1], vv.shape[2]
        o = torch.empty((R, Hv, dv), device=dev)
        if name.endswith("chunk_parallel"):
            wsg = lrc.gdn_workspace(1, R, Hk, Hv, dk, dv, dev)
            fn = lambda: lrc.gdn_prefill_ws(q, kk, vv, be, gg, o, S, [R], wsg)  # noqa: E731
        else:
            fn = lambda: lrc.gdn_prefill(q, kk, vv, be, gg, o, S, [R])  # noqa: E731
        peak = MFMA_FP32_PEAK_TFS if q.dtype == torch.float32 else MFMA_BF16_PEAK_TFS
        k3[name] = _entry(_time_ms(fn, stream, 100), R, "mfma", gdn_chunk_flops([R], Hk, Hv, dk, dv), peak)
        keep["cfg3"][name] = dd
    out["cfg3_gdn_small"] = {"workload": CONFIG_NAMES["cfg3_gdn_small"], "rows": 75, "kernels": k3}
    # --- cfg4: Gated DeltaNet 9B-like: conv + chunk-parallel form (this config's path), fused and fp32 alongside
    d4 = inputs.gdn_9b()
    R, Hk, dk = d4["q"].shape
    Hv, dv = d4["v"].shape[1], d4["v"].shape[2]
    cx, cw = g(d4["conv_x"]), g(d4["conv_w"])
    C, K = cx.shape[1], cw.shape[1]
    cy, cst = torch.empty_like(cx), g(d4["conv_state"])[None].clone()
    k4 = {"conv_bf16": _entry(_time_ms(lambda: lrc.conv_prefill(cx, cy, cst, cw, [R]), stream, 50), R, "hbm",
                              R * C * 4 + 2 * (K - 1) * C * 2 + C * K * 4, HBM_PEAK_GBS)}
    q, kk, vv, be, gg = (g(d4[n]) for n in ("q", "k", "v", "beta", "g"))
    S = g(d4["S0"])[None].clone()
    o = torch.empty((R, Hv, dv), device=dev)
    wsg = lrc.gdn_workspace(1, R, Hk, Hv, dk, dv, dev)
    fl = gdn_chunk_flops([R], Hk, Hv, dk, dv)
    k4["gdn_bf16_chunk_parallel"] = _entry(
        _time_ms(lambda: lrc.gdn_prefill_ws(q, kk, vv, be, gg, o, S, [R], wsg), stream, 20), R, "mfma", fl,
        MFMA_BF16_PEAK_TFS)
    k4["gdn_bf16_fused"] = _entry(_time_ms(lambda: lrc.gdn_prefill(q, kk, vv, be, gg, o, S, [R]), stream, 20), R,
                                  "mfma", fl, MFMA_BF16_PEAK_TFS)
    q32, k32, v32 = q.float(), kk.float(), vv.float()
    k4["gdn_f32"] = _entry(_time_ms(lambda: lrc.gdn_prefill(q32, k32, v32, be, gg, o, S, [R]), stream, 10), R,
                           "mfma", fl, MFMA_FP32_PEAK_TFS)
    del q32, k32, v32, wsg
    out["cfg4_gdn_9b"] = {"workload": CONFIG_NAMES["cfg4_gdn_9b"], "rows": R, "kernels": k4,
                          "gdn_path": "gdn_bf16_chunk_parallel"}
    keep["cfg4"] = d4
    return out, keep


def config_errors(lrc, dev, keep, per_config):
    """Oracle leg of the per-config table: each config runs once more on the GPU from the same
    incoming state as the float64 oracle, and every output and state tensor gets its max rel err.
    Also times the oracle on each config, at the default thread count and on one thread."""
    import numpy as np
    import torch

    import oracle

    f64 = lambda t: t.detach().cpu().double().numpy()  # noqa: E731
    g = lambda t: t.to(dev).contiguous()  # noqa: E731

    def rel(got, ref):
        sc = float(np.max(np.abs(ref)))
        return float(np.max(np.abs(got - ref))) / (sc if sc else 1.0)

    nthreads = oracle.num_threads()

    def timed(fn):
        t0 = time.perf_counter(); res = fn(); t = time.perf_counter() - t0
        oracle.set_num_threads(1)
        t1 = time.perf_counter(); fn(); t1 = time.perf_counter() - t1
        oracle.set_num_threads(nthreads)
        return res, t, t1

    def put(cfg, kern, errs, tol):
        e = per_config[cfg]["kernels"][kern]
        e["max_rel_err"] = {n: v for n, v in errs.items()}
        e["tol"] = tol
        e["within_tol"] = bool(all(v <= tol for v in errs.values()) and all(np.isfinite(list(errs.values()))))

    orc = {}
    # cfg1
    d = keep["cfg1"]
    R = d["conv_x"].shape[0]
    (ry, rs), tc, tc1 = timed(lambda: oracle.conv_rows(f64(d["conv_x"]), f64(d["conv_state"]), f64(d["conv_w"])))
    x, w = g(d["conv_x"]), g(d["conv_w"])
    y, st = torch.empty_like(x), g(d["conv_state"])[None].clone()
    lrc.conv_prefill(x, y, st, w, [R])
    (rh, rhs), ts, ts1 = timed(lambda: oracle.scan(f64(d["a"]), f64(d["b"]), f64(d["h0"])))
    a, b = g(d["a"]).view(R, 64, 16), g(d["b"]).view(R, 64, 16)
    h, hs = torch.empty_like(a), g(d["h0"]).view(1, 64, 16).clone()
    lrc.scan_prefill_ws(a, b, h, hs, [R], lrc.scan_workspace(1, 64, 16, dev))
    torch.cuda.synchronize()
    put("cfg1_mamba_tiny", "conv", {"y": rel(f64(y), ry), "state": rel(f64(st[0]), rs)}, 1e-4)
    put("cfg1_mamba_tiny", "scan", {"h": rel(f64(h).reshape(R, -1), rh), "state": rel(f64(hs).reshape(-1), rhs)}, 1e-4)
    orc["cfg1_mamba_tiny"] = (R, tc + ts, tc1 + ts1)
    # cfg2: the incoming state is the oracle's, after 32 warm-up token steps from the empty state
    r = keep["cfg2"]
    R, C = r["k"].shape
    _, wn, wd, wm = oracle.wkv4(f64(r["warm_k"]), f64(r["warm_v"]), f64(r["w"]), f64(r["u"]), *oracle.empty_wkv_state(C))
    n32, d32, m32 = (torch.from_numpy(z).float() for z in (wn, wd, wm))
    (ro, rn, rd, rm), tw, tw1 = timed(lambda: oracle.wkv4(f64(r["k"]), f64(r["v"]), f64(r["w"]), f64(r["u"]),
                                                        f64(n32), f64(d32), f64(m32)))
    k_, v_, w_, u_ = (g(r[n]) for n in ("k", "v", "w", "u"))
    o2 = torch.empty_like(k_)
    num, den, mx = g(n32)[None].clone(), g(d32)[None].clone(), g(m32)[None].clone()
    lrc.wkv4_prefill(k_, v_, w_, u_, o2, num, den, mx, [R])
    torch.cuda.synchronize()
    gm = f64(mx[0])
    put("cfg2_rwkv4_169m", "wkv4", {"wkv": rel(f64(o2), ro), "num/den": rel(f64(num[0]) / f64(den[0]), rn / rd),
                                    "num*e^(max-M)": rel(f64(num[0]) * np.exp(gm - rm), rn),
                                    "den*e^(max-M)": rel(f64(den[0]) * np.exp(gm - rm), rd)}, 1e-4)
    orc["cfg2_rwkv4_169m"] = (R, tw, tw1)
    # cfg3 and cfg4 Gated DeltaNet
    def gdn_case(cfg, kern, dd, tol, chunk_parallel):
        q, kk, vv, be, gg = (g(dd[n]) for n in ("q", "k", "v", "beta", "g"))
        S = g(dd["S0"])[None].clone()
        R, Hk, dk = q.shape
        Hv, dv = vv.shape[1], vv.shape[2]
        o = torch.empty((R, Hv, dv), device=dev)
        if chunk_parallel:
            lrc.gdn_prefill_ws(q, kk, vv, be, gg, o, S, [R], lrc.gdn_workspace(1, R, Hk, Hv, dk, dv, dev))
        else:
            lrc.gdn_prefill(q, kk, vv, be, gg, o, S, [R])
        torch.cuda.synchronize()
        return o, S

    ttot = [0.0, 0.0]
    for kern, dd in keep["cfg3"].items():
        (ro, rs), t, t1 = timed(lambda: oracle.gdn(*(f64(dd[n]) for n in ("q", "k", "v", "beta", "g", "S0"))))
        ttot[0] += t; ttot[1] += t1
        o, S = gdn_case("cfg3_gdn_small", kern, dd, None, kern.endswith("chunk_parallel"))
        tol = 1e-4 if dd["q"].dtype == torch.float32 else 2e-2
        put("cfg3_gdn_small", kern, {"o": rel(f64(o), ro), "state": rel(f64(S[0]), rs)}, tol)
    orc["cfg3_gdn_small"] = (75, ttot[0] / len(keep["cfg3"]), ttot[1] / len(keep["cfg3"]))
    d4 = keep["cfg4"]
    args = [f64(d4[n]) for n in ("q", "k", "v", "beta", "g", "S0")]
    t0 = time.perf_counter(); ro, rs = oracle.gdn(*args); t4 = time.perf_counter() - t0
    # one thread on 4 of the 32 value heads (2 key heads), scaled to all heads
    oracle.set_num_threads(1)
    t0 = time.perf_counter(); oracle.gdn(args[0][:, :2], args[1][:, :2], args[2][:, :4], args[3][:, :4], args[4][:, :4],
                                         args[5][:4]); t41 = (time.perf_counter() - t0) * 8
    oracle.set_num_threads(nthreads)
    R = args[0].shape[0]
    for kern, cp in [("gdn_bf16_chunk_parallel", True), ("gdn_bf16_fused", False)]:
        o, S = gdn_case("cfg4_gdn_9b", kern, d4, None, cp)
        put("cfg4_gdn_9b", kern, {"o": rel(f64(o), ro), "state": rel(f64(S[0]), rs),
                                  "o_head31_g=-8": rel(f64(o[:, 31]), ro[:, 31]),
                                  "state_head31_g=-8": rel(f64(S[0, 31]), rs[31])}, 2e-2)
    d32 = dict(d4)
    for n in ("q", "k", "v"):
        d32[n] = d4[n].float()
    o, S = gdn_case("cfg4_gdn_9b", "gdn_f32", d32, None, False)
    put("cfg4_gdn_9b", "gdn_f32", {"o": rel(f64(o), ro), "state": rel(f64(S[0]), rs)}, 1e-4)
    cx, cw = d4["conv_x"], d4["conv_w"]
    (ry, rst), tcv, tcv1 = timed(lambda: oracle.conv_rows(f64(cx), f64(d4["conv_state"]), f64(cw)))
    x, w = g(cx), g(cw)
    y, st = torch.empty_like(x), g(d4["conv_state"])[None].clone()
    lrc.conv_prefill(x, y, st, w, [R])
    torch.cuda.synchronize()
    put("cfg4_gdn_9b", "conv_bf16", {"y": rel(f64(y), ry), "state": rel(f64(st[0]), rst)}, 2e-2)
    orc["cfg4_gdn_9b"] = (R, t4 + tcv, t41 + tcv1)
    for cfg, (rows, t, t1) in orc.items():
        per_config[cfg]["oracle"] = {"rows_per_s": rows / t, "cores": nthreads, "rows_per_s_1_thread": rows / t1}


# ALU peak for the fused mixer rows: 256 CUs x 4 SIMDs x 16 lanes at 2.4 GHz issue 39.3 T lane-slots/s;
# one (t, d, n) step costs 4 full-rate VALU slots (dt*A', dt x * B, the state FMA, the readout FMA) plus one
# exp at a quarter of that rate (4 slots), so 8 slots per step.
ALU_LANE_SLOTS = 256 * 4 * 16 * 2.4e9
MIXER_SLOTS_PER_STEP = 8


def time_launch(fn, stream, reps=10):
    """Average ms of fn() over reps launches on stream, after two untimed ones."""
    import torch

    for _ in range(2):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def measure_next_rows(lrc, dev, lens, reps=10):
    """Time the rows beyond the step's hot path -- the RWKV-4 time shift (three mixed inputs at
    the RWKV width), the fused Mamba mixer rows (Mamba width) and the WKV with a token-dependent
    decay (RWKV width) -- on the same prompt lengths, from fresh states, with HIP events on the
    launch stream."""
    import torch

    from linear_recurrence_chunked_amd import inputs

    sh = inputs.MIXED_SHAPES
    R, P = int(sum(lens)), len(lens)
    m = inputs.mixed_mamba_mixer(lens, dev)
    t = inputs.mixed_time_shift(lens, dev)
    td = inputs.mixed_wkv_tdecay(lens, dev)
    Dm, N = sh["mamba_d_inner"], sh["mamba_d_state"]
    C, M = t["x"].shape[1], t["mix"].shape[0]
    y = torch.empty_like(m["x"])
    out = torch.empty((M, R, C), device=dev)
    Ct = td["k"].shape[1]
    tdo = torch.empty_like(td["k"])
    runs = {
        "time_shift": (lambda: lrc.time_shift_prefill(t["x"], out, t["state"], t["mix"], lens),
                       R * C * 4 * (1 + M) + P * C * 8 + M * C * 4, None),
        "mamba_mixer": (lambda: lrc.mamba_mixer_prefill(m["x"], m["dt"], m["A"], m["B"], m["C"], m["D"], y,
                                                        m["h0"], lens),
                        R * Dm * 12 + R * N * 8 + P * Dm * N * 8 + Dm * N * 4 + Dm * 4, R * Dm * N),
        "wkv_tdecay": (lambda: lrc.wkv_tdecay_prefill(td["k"], td["v"], td["w"], td["u"], tdo, td["num"], td["den"],
                                                      td["max"], lens),
                       R * Ct * 16 + P * Ct * 24 + Ct * 4, None),
    }
    stream = torch.cuda.current_stream(dev)
    res = {}
    for name, (fn, nbytes, steps) in runs.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        d = {"ms": round(ms, 4), "rows_per_s": R / (ms * 1e-3), "GBps": nbytes / (ms * 1e-3) / 1e9,
             "algorithmic_bytes": nbytes}
        d["hbm_frac"] = d["GBps"] / HBM_PEAK_GBS
        if steps:
            rate = steps / (ms * 1e-3)
            peak = ALU_LANE_SLOTS / MIXER_SLOTS_PER_STEP
            d.update({"bound": "alu", "state_steps_per_s": rate, "alu_peak_steps_per_s": peak, "alu_frac": rate / peak})
        else:
            d["bound"] = "hbm"
        res[name] = d
    del m, t, y, out, td, tdo
    return res


def measure_skew(lrc, dev, stream, reps=10):
    """WKV (2560 channels) and the fused Mamba mixer rows (5120 x 16) on equal totals of rows with a few
    long prompts -- 8 x 3832 and 4 x 7664 rows -- beside the mixed lengths: the sequential chunk chain of
    the longest prompt and the number of (prompt, channel block) workgroups set these times."""
    import torch

    from linear_recurrence_chunked_amd import inputs

    sh = inputs.MIXED_SHAPES
    res = {}
    for name, lens in [("8x3832", [3832] * 8), ("4x7664", [7664] * 4)]:
        R, P = sum(lens), len(lens)
        r = inputs.mixed_rwkv(lens, dev)
        C = r["k"].shape[1]
        o = torch.empty_like(r["k"])
        ms = _time_ms(lambda: lrc.wkv4_prefill(r["k"], r["v"], r["w"], r["u"], o, r["num"], r["den"], r["max"], lens),
                      stream, reps)
        wkv = _entry(ms, R, "hbm", R * C * 12 + P * C * 24 + C * 8, HBM_PEAK_GBS)
        del r, o
        m = inputs.mixed_mamba_mixer(lens, dev)
        Dm, N = sh["mamba_d_inner"], sh["mamba_d_state"]
        y = torch.empty_like(m["x"])
        ms = _time_ms(lambda: lrc.mamba_mixer_prefill(m["x"], m["dt"], m["A"], m["B"], m["C"], m["D"], y, m["h0"], lens),
                      stream, reps)
        rate = R * Dm * N / (ms * 1e-3)
        peak = ALU_LANE_SLOTS / MIXER_SLOTS_PER_STEP
        mixer = {"ms": round(ms, 5), "rows_per_s": R / (ms * 1e-3), "bound": "alu", "state_steps_per_s": rate,
                 "frac": rate / peak}
        del m, y
        res[name] = {"rows": R, "wkv4": wkv, "mamba_mixer": mixer}
    return res


def fresh_outputs_sample(lrc, W):
    """Run one step from fresh states and keep host copies of the sampled outputs."""
    import numpy as np
    import torch

    from linear_recurrence_chunked_amd import inputs

    sh = inputs.MIXED_SHAPES
    E = sh["mamba_d_inner"] * sh["mamba_d_state"]
    for k in KERNELS:
        run_kernel(lrc, W, k)
    torch.cuda.synchronize()
    f64 = lambda t: t.detach().cpu().double().numpy()  # noqa: E731
    st = SAMPLE_STRIDE
    return {
        "ym": f64(W["ym"][:, ::st["conv_mamba"]]),
        "h": f64(W["h"].view(W["R"], E)[:, ::st["scan"]]),
        "wkv": f64(W["wkv"][:, ::st["wkv4"]]),
        "yg": f64(W["yg"][:, ::st["conv_gdn"]]),
        "o": f64(W["o"]),
    }


def reset_states(W):
    W["sm"].zero_(); W["hs"].zero_(); W["num"].zero_(); W["den"].zero_(); W["max"].fill_(-1e38)
    W["sg"].zero_(); W["S"].zero_()


def calibrate_copy():
    import torch

    n = 1 << 30  # 4 GiB of fp32
    src = torch.ones(n, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": 4 * n, "copy_bytes_written": 4 * n, "launches": 3}))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the kernels would shard over prompts, channels and heads with no communication).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        calibrate_copy()
        return
    from linear_recurrence_chunked_amd import lrc

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    W = make_workload(dev)
    torch.cuda.synchronize()
    kernels = [k for k in KERNELS if not args.only or k in args.only.split(",")]

    lrc.wait_timeouts(reset=True)  # bounded in-workgroup waits of the WKV kernels that ran out (expected 0)
    fresh = None if args.no_cpu_baseline else fresh_outputs_sample(lrc, W)
    reset_states(W)
    for _ in range(args.warmup):
        for k in kernels:
            run_kernel(lrc, W, k)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for s in range(args.steps):
        ev[s][0].record(stream)
        for i, k in enumerate(kernels):
            run_kernel(lrc, W, k)
            ev[s][i + 1].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    per_k = {k: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)) / args.steps
             for i, k in enumerate(kernels)}
    ms_per_step = total_ms / args.steps
    R = W["R"]
    work = algorithmic_work(W)

    kern = {}
    for k in kernels:
        ms = per_k[k]
        d = {"ms": round(ms, 4), "rows_per_s": R / (ms * 1e-3), "GBps": work[k]["bytes"] / (ms * 1e-3) / 1e9}
        d["hbm_frac"] = d["GBps"] / HBM_PEAK_GBS
        if "flops" in work[k]:
            d["TFLOPs"] = work[k]["flops"] / (ms * 1e-3) / 1e12
            d["mfma_bf16_frac"] = d["TFLOPs"] / MFMA_BF16_PEAK_TFS
        if k == "scan":  # carry hand-overs of the tiled driver that timed out over the whole run (expected 0)
            d["handover_timeouts"] = lrc.scan_workspace_timeouts(W["scan_ws"])
        if k == "wkv4":  # bounded waits between its waves that ran out over the whole run (expected 0)
            d["lds_wait_timeouts"] = lrc.wait_timeouts()
        kern[k] = d
    if "gdn" in kern and not args.no_extra_legs:  # the same launch with FP32 operands as hi + lo bf16 pairs (LRC_BF16_SPLIT), not in `value`
        ms = time_launch(lambda: lrc.gdn_prefill(W["q"], W["gk"], W["gv"], W["beta"], W["g"], W["o"], W["S"],
                                                 W["lens"], split=True), stream)
        tf = work["gdn"]["flops"] / (ms * 1e-3) / 1e12
        kern["gdn"]["split_form"] = {"ms": round(ms, 4), "TFLOPs": tf, "mfma_bf16_frac": tf / MFMA_BF16_PEAK_TFS}
        # the same rows with FP32 q, k, v (the FP32-input path, on the FP32 matrix cores), not in `value`
        q32, k32, v32 = (W[n].float() for n in ("q", "gk", "gv"))
        ms = time_launch(lambda: lrc.gdn_prefill(q32, k32, v32, W["beta"], W["g"], W["o"], W["S"], W["lens"]),
                         stream, reps=5)
        tf = work["gdn"]["flops"] / (ms * 1e-3) / 1e12
        kern["gdn"]["fp32_inputs"] = {"ms": round(ms, 4), "TFLOPs": tf,
                                      "mfma_fp32_frac": tf / MFMA_FP32_PEAK_TFS}
        del q32, k32, v32
    nxt = measure_next_rows(lrc, dev, W["lens"]) if not (args.only or args.no_extra_legs) else None
    if nxt:  # the token-dependent decay's waits, counted with those of the step's WKV
        nxt["wkv_tdecay"]["lds_wait_timeouts"] = lrc.wait_timeouts()
    if nxt:
        nxt["skewed_lengths"] = measure_skew(lrc, dev, stream)
    if nxt and "scan" in per_k:
        nxt["mamba_mixer"]["vs_scan_kernel_alone"] = per_k["scan"] / nxt["mamba_mixer"]["ms"]
    dom = max(kernels, key=lambda k: per_k[k])
    copy_gbps = measure_copy_gbps(dev)
    add_gbps = measure_add_gbps(dev)
    if dom == "gdn":
        roof = {"kernel": dom, "bound": "mfma", "achieved": kern[dom]["TFLOPs"], "peak": MFMA_BF16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": kern[dom]["mfma_bf16_frac"], "traffic": stored_traffic(dom),
                "algorithmic_per_launch": work[dom]["flops"]}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": kern[dom]["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": kern[dom]["hbm_frac"], "traffic": stored_traffic(dom),
                "algorithmic_per_launch": work[dom]["bytes"], "frac_of_measured_copy": kern[dom]["GBps"] / copy_gbps,
                "frac_of_measured_add": kern[dom]["GBps"] / add_gbps}
    roof["avg_launch_ms"] = per_k[dom]
    roof["measured_copy_GBps"] = copy_gbps
    roof["measured_add_GBps"] = add_gbps

    out = {
        "metric": "prefill rows/s per kernel at 1 GPU; % HBM or MFMA peak; max rel err vs oracle",
        "value": R / (ms_per_step * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": "batched mixed prefill: 16 prompts of U{1..4096} rows, 64-row chunks, through "
                               "Mamba conv (5120 fp32) + scan (5120x16 fp32), RWKV-4 WKV (2560 fp32), "
                               "DeltaNet conv (8192 bf16) + Gated DeltaNet (32x128x128, bf16 in, fp32 state)",
                   "prompts": len(W["lens"]), "rows": R, "lens": W["lens"], "kernels": kernels},
        "roofline": roof,
        "kernels": kern,
        # rows beyond the step (not in `value`): the RWKV-4 time shift and the fused Mamba mixer rows
        "next_rows": nxt,
    }
    per_config = None
    if not args.only and not args.no_configs:
        per_config, keep = measure_configs(lrc, dev, stream)
        per_config["cfg5_mixed"] = {"workload": CONFIG_NAMES["cfg5_mixed"], "rows": R, "kernels": {
            k: {"ms": kern[k]["ms"], "rows_per_s": kern[k]["rows_per_s"],
                **({"bound": "mfma", "TFLOPs": kern[k]["TFLOPs"], "peak_TFLOPs": MFMA_BF16_PEAK_TFS,
                    "frac": kern[k]["mfma_bf16_frac"]} if k == "gdn" else
                   {"bound": "hbm", "GBps": kern[k]["GBps"], "peak_GBps": HBM_PEAK_GBS, "frac": kern[k]["hbm_frac"]})}
            for k in kernels}}
    if not args.no_cpu_baseline and set(kernels) == set(KERNELS):
        cb, err = cpu_baseline(W, fresh, args.cpu_budget)
        cb["one_thread"] = cpu_baseline_one_thread(W)
        out["cpu_baseline"] = cb
        out["max_rel_err_sample"] = err
        if per_config:
            config_errors(lrc, dev, keep, per_config)
            for k, e in err.items():
                per_config["cfg5_mixed"]["kernels"][k]["max_rel_err_sampled"] = e
            per_config["cfg5_mixed"]["oracle"] = {"rows_per_s": cb["value"], "cores": cb["cores"],
                                                  "rows_per_s_1_thread": cb["one_thread"]["value"]}
    else:
        out["cpu_baseline"] = None
    out["per_config"] = per_config
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
