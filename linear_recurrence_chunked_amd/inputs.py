"""Seeded synthetic inputs for the five workloads.

This module only draws random numbers and shapes them; it performs none of
the recurrences.  The same arrays feed the HIP kernels and the float64
oracle, so an input is never rounded differently on the two sides: bf16
tensors are rounded once here (round-to-nearest-even, by torch) and the
oracle reads those bits upcast to float64.

Host workloads (Mamba tiny, RWKV 169M-like, Gated DeltaNet small and 9B-like)
use numpy's PCG64 ``default_rng(seed)`` in float64 and return torch CPU
tensors.  The batched mixed workload is too large for the host (the Mamba
a/b/h tensors alone are ~32 GB), so it is drawn on the target device with a
seeded ``torch.Generator``.

"N(0, s)" means a normal with standard deviation s.
"""
from __future__ import annotations

import math

import numpy as np
import torch

SEED_BASE = 20261202
MAX_ROWS = 64


def seed_for(cfg_index: int) -> int:
    return SEED_BASE + cfg_index


def _t(a: np.ndarray, dtype=torch.float32) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)).to(dtype)


def _l2_rows(x: np.ndarray) -> np.ndarray:
    """Normalise the last axis to unit length (the workload's q/k recipe)."""
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


# --------------------------------------------------------------------------
# Mamba tiny: batch 1, d_inner 64, d_state 16, 75 rows, fp32, conv K=4.
# --------------------------------------------------------------------------
def mamba_tiny(seed: int | None = None, rows: int = 75, d_inner: int = 64, d_state: int = 16,
               conv_k: int = 4, zero_conv_state: bool = False) -> dict:
    """a = exp(dt*A), dt ~ U(1e-3, 0.1) per (t, d), A = -U(1, 16) per (d, n);
    b = dt*B*x with B ~ N(0,1) per (t, n), x ~ N(0,1) per (t, d); h0 ~ N(0,1).
    Conv: x ~ N(0,1) [rows, d_inner], state ~ N(0,1) (or zeros), w ~ N(0, 0.5)."""
    rng = np.random.default_rng(seed_for(1) if seed is None else seed)
    dt = rng.uniform(1e-3, 0.1, size=(rows, d_inner))
    A = -rng.uniform(1.0, 16.0, size=(d_inner, d_state))
    B = rng.standard_normal((rows, d_state))
    x = rng.standard_normal((rows, d_inner))
    a = np.exp(dt[:, :, None] * A[None, :, :])
    b = dt[:, :, None] * B[:, None, :] * x[:, :, None]
    h0 = rng.standard_normal((d_inner, d_state))
    cx = rng.standard_normal((rows, d_inner))
    cstate = np.zeros((conv_k - 1, d_inner)) if zero_conv_state else rng.standard_normal((conv_k - 1, d_inner))
    cw = rng.normal(0.0, 0.5, size=(d_inner, conv_k))
    return {
        "a": _t(a.reshape(rows, d_inner * d_state)),
        "b": _t(b.reshape(rows, d_inner * d_state)),
        "h0": _t(h0.reshape(d_inner * d_state)),
        "conv_x": _t(cx),
        "conv_state": _t(cstate),
        "conv_w": _t(cw),
        "splits": [64, rows - 64] if rows > 64 else [rows],
    }


def mamba_mixer_tiny(seed: int | None = None, rows: int = 75, d_inner: int = 64, d_state: int = 16) -> dict:
    """Inputs of the fused mixer rows, in the Mamba-tiny recipe: dt ~ U(1e-3, 0.1) per (t, d),
    A = -U(1, 16) per (d, n), B, C ~ N(0,1) per (t, n), x ~ N(0,1) per (t, d), D ~ N(0,1) per d,
    h0 ~ N(0,1)."""
    rng = np.random.default_rng(seed_for(6) if seed is None else seed)
    return {
        "x": _t(rng.standard_normal((rows, d_inner))),
        "dt": _t(rng.uniform(1e-3, 0.1, size=(rows, d_inner))),
        "A": _t(-rng.uniform(1.0, 16.0, size=(d_inner, d_state))),
        "B": _t(rng.standard_normal((rows, d_state))),
        "C": _t(rng.standard_normal((rows, d_state))),
        "D": _t(rng.standard_normal(d_inner)),
        "h0": _t(rng.standard_normal((d_inner, d_state))),
    }


def rwkv_shift(seed: int | None = None, rows: int = 128, channels: int = 768 * 12, mixes: int = 3) -> dict:
    """Time-shift inputs at the 169M-like width: x ~ N(0,1) rows, incoming shift state ~ N(0,1),
    mixing vectors ~ U(0,1) (key, value, receptance)."""
    rng = np.random.default_rng(seed_for(7) if seed is None else seed)
    return {"x": _t(rng.standard_normal((rows, channels))), "state": _t(rng.standard_normal(channels)),
            "mix": _t(rng.uniform(0.0, 1.0, size=(mixes, channels)))}


# --------------------------------------------------------------------------
# RWKV-4 169M-like: hidden 768 x 12 layers as independent channels, 128 rows.
# --------------------------------------------------------------------------
def _rwkv_keys(rng, shape, spike_frac=0.01, spike=30.0):
    k = rng.normal(0.0, 3.0, size=shape)
    mask = rng.uniform(size=shape) < spike_frac
    sign = np.where(rng.uniform(size=shape) < 0.5, -1.0, 1.0)
    return np.where(mask, sign * spike, k)


def rwkv_169m(seed: int | None = None, rows: int = 128, channels: int = 768 * 12,
              warmup: int = 32) -> dict:
    """w = -exp(d), d ~ U(-6, 2); u ~ U(-2, 2); k ~ N(0, 3) with 1% of entries
    set to +-30; v ~ N(0, 1).  ``warm_k``/``warm_v`` are the 32 warm-up token
    rows from which the incoming (num, den, max) is built by running the
    recurrence from the empty state (the tests do that with the oracle)."""
    rng = np.random.default_rng(seed_for(2) if seed is None else seed)
    d = rng.uniform(-6.0, 2.0, size=channels)
    w = -np.exp(d)
    u = rng.uniform(-2.0, 2.0, size=channels)
    k = _rwkv_keys(rng, (rows, channels))
    v = rng.standard_normal((rows, channels))
    wk = _rwkv_keys(rng, (warmup, channels))
    wv = rng.standard_normal((warmup, channels))
    return {"k": _t(k), "v": _t(v), "w": _t(w), "u": _t(u), "warm_k": _t(wk), "warm_v": _t(wv),
            "splits": [MAX_ROWS] * (rows // MAX_ROWS) + ([rows % MAX_ROWS] if rows % MAX_ROWS else [])}


def rwkv_tdecay(seed: int | None = None, rows: int = 128, channels: int = 768 * 12, warmup: int = 32) -> dict:
    """The RWKV-4 recipe above with a decay per row and channel: w_t = -exp(d_t),
    d_t ~ U(-6, 2); the warm-up rows carry their own decays ``warm_w``."""
    rng = np.random.default_rng(seed_for(8) if seed is None else seed)
    u = rng.uniform(-2.0, 2.0, size=channels)
    k = _rwkv_keys(rng, (rows, channels))
    v = rng.standard_normal((rows, channels))
    w = -np.exp(rng.uniform(-6.0, 2.0, size=(rows, channels)))
    wk = _rwkv_keys(rng, (warmup, channels))
    wv = rng.standard_normal((warmup, channels))
    ww = -np.exp(rng.uniform(-6.0, 2.0, size=(warmup, channels)))
    return {"k": _t(k), "v": _t(v), "w": _t(w), "u": _t(u), "warm_k": _t(wk), "warm_v": _t(wv), "warm_w": _t(ww)}


# --------------------------------------------------------------------------
# Gated DeltaNet small: 8 heads, dk = dv = 64, 75 rows (64 + 11).
# --------------------------------------------------------------------------
def gdn_small(seed: int | None = None, rows: int = 75, heads: int = 8, dk: int = 64, dv: int = 64,
              dtype=torch.float32, parallel_keys: int = 0, parallel_start: int = 24,
              beta_const: float | None = None, key_heads: int | None = None) -> dict:
    """q, k rows N(0,1) then L2-normalised per head; v ~ N(0,1);
    beta = sigmoid(N(0,1)); g = -softplus(N(0,1)) * 0.5; S0 ~ N(0, 0.1).
    Stress: ``parallel_keys`` rows starting at ``parallel_start`` get keys
    normalise(kbar + 1e-3 n) (cosine > 0.999), and beta may be a constant."""
    rng = np.random.default_rng(seed_for(3) if seed is None else seed)
    hk = heads if key_heads is None else key_heads
    q = _l2_rows(rng.standard_normal((rows, hk, dk)))
    k = rng.standard_normal((rows, hk, dk))
    if parallel_keys:
        kbar = rng.standard_normal((1, hk, dk))
        n = rng.standard_normal((parallel_keys, hk, dk))
        k[parallel_start:parallel_start + parallel_keys] = kbar + 1e-3 * n
    k = _l2_rows(k)
    v = rng.standard_normal((rows, heads, dv))
    beta = _sigmoid(rng.standard_normal((rows, heads)))
    if beta_const is not None:
        beta = np.full((rows, heads), beta_const)
    g = -_softplus(rng.standard_normal((rows, heads))) * 0.5
    S0 = rng.normal(0.0, 0.1, size=(heads, dk, dv))
    return {"q": _t(q, dtype), "k": _t(k, dtype), "v": _t(v, dtype), "beta": _t(beta), "g": _t(g),
            "S0": _t(S0), "splits": [64, rows - 64] if rows > 64 else [rows]}


# --------------------------------------------------------------------------
# Gated DeltaNet 9B-like: 32 value heads on 16 key heads, 128 x 128, 2048 rows.
# --------------------------------------------------------------------------
def gdn_decays(rng, rows: int, heads: int) -> np.ndarray:
    """g = -exp(U(ln 1e-3, ln 8)) per (row, head); head 0 pinned to -1e-3 and
    the last head to -8 on every row so both ends of the range occur."""
    g = -np.exp(rng.uniform(math.log(1e-3), math.log(8.0), size=(rows, heads)))
    g[:, 0] = -1e-3
    g[:, heads - 1] = -8.0
    return g


def gdn_9b(seed: int | None = None, rows: int = 2048, hk: int = 16, hv: int = 32, dk: int = 128,
           dv: int = 128, conv_k: int = 4, dtype=torch.bfloat16) -> dict:
    rng = np.random.default_rng(seed_for(4) if seed is None else seed)
    q = _l2_rows(rng.standard_normal((rows, hk, dk)))
    k = _l2_rows(rng.standard_normal((rows, hk, dk)))
    v = rng.standard_normal((rows, hv, dv))
    beta = _sigmoid(rng.standard_normal((rows, hv)))
    g = gdn_decays(rng, rows, hv)
    S0 = rng.normal(0.0, 0.1, size=(hv, dk, dv))
    cc = 2 * hk * dk + hv * dv
    cx = rng.standard_normal((rows, cc))
    cstate = rng.standard_normal((conv_k - 1, cc))
    cw = rng.normal(0.0, 0.5, size=(cc, conv_k))
    return {"q": _t(q, dtype), "k": _t(k, dtype), "v": _t(v, dtype), "beta": _t(beta), "g": _t(g),
            "S0": _t(S0), "conv_x": _t(cx, dtype), "conv_state": _t(cstate, dtype), "conv_w": _t(cw),
            "splits": [MAX_ROWS] * (rows // MAX_ROWS)}


# --------------------------------------------------------------------------
# Batched mixed prefill: 16 prompts of U{1..4096} rows through every kernel.
# --------------------------------------------------------------------------
MIXED_SHAPES = {
    "mamba_d_inner": 5120, "mamba_d_state": 16, "mamba_conv_c": 5120,
    "rwkv_c": 2560,
    "gdn_hk": 16, "gdn_hv": 32, "gdn_dk": 128, "gdn_dv": 128, "gdn_conv_c": 2 * 16 * 128 + 32 * 128,
    "conv_k": 4,
}


def mixed_lengths(seed: int | None = None, prompts: int = 16, max_len: int = 4096) -> list[int]:
    rng = np.random.default_rng(seed_for(5) if seed is None else seed)
    return [int(x) for x in rng.integers(1, max_len + 1, size=prompts)]


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def mixed_mamba(lens, device, seed: int | None = None, d_inner=5120, d_state=16, conv_k=4,
                with_conv: bool = True) -> dict:
    """Packed rows [sum(lens), ...] of the Mamba-tiny recipe at model width."""
    gen = _gen(device, (seed_for(5) if seed is None else seed) * 8 + 1)
    R = int(sum(lens))
    P = len(lens)
    f = dict(device=device, dtype=torch.float32, generator=gen)
    dt = torch.rand((R, d_inner), **f) * (0.1 - 1e-3) + 1e-3
    A = -(torch.rand((d_inner, d_state), **f) * 15.0 + 1.0)
    B = torch.randn((R, d_state), **f)
    x = torch.randn((R, d_inner), **f)
    a = torch.exp(dt[:, :, None] * A[None])
    b = dt[:, :, None] * B[:, None, :]
    b.mul_(x[:, :, None])
    del dt, B
    out = {"a": a.reshape(R, d_inner * d_state), "b": b.reshape(R, d_inner * d_state),
           "h0": torch.zeros((P, d_inner * d_state), device=device, dtype=torch.float32)}
    if with_conv:
        out["conv_x"] = x
        out["conv_state"] = torch.zeros((P, conv_k - 1, d_inner), device=device, dtype=torch.float32)
        out["conv_w"] = torch.randn((d_inner, conv_k), **f) * 0.5
    return out


def mixed_rwkv(lens, device, seed: int | None = None, channels=2560) -> dict:
    gen = _gen(device, (seed_for(5) if seed is None else seed) * 8 + 2)
    R = int(sum(lens))
    P = len(lens)
    f = dict(device=device, dtype=torch.float32, generator=gen)
    w = -torch.exp(torch.rand((channels,), **f) * 8.0 - 6.0)
    u = torch.rand((channels,), **f) * 4.0 - 2.0
    k = torch.randn((R, channels), **f) * 3.0
    spike = torch.rand((R, channels), **f) < 0.01
    sign = torch.where(torch.rand((R, channels), **f) < 0.5, -1.0, 1.0)
    k = torch.where(spike, sign * 30.0, k)
    v = torch.randn((R, channels), **f)
    return {"k": k, "v": v, "w": w, "u": u,
            "num": torch.zeros((P, channels), device=device), "den": torch.zeros((P, channels), device=device),
            "max": torch.full((P, channels), -1e38, device=device)}


def mixed_gdn(lens, device, seed: int | None = None, hk=16, hv=32, dk=128, dv=128, conv_k=4,
              dtype=torch.bfloat16, with_conv: bool = True) -> dict:
    gen = _gen(device, (seed_for(5) if seed is None else seed) * 8 + 3)
    R = int(sum(lens))
    P = len(lens)
    f = dict(device=device, dtype=torch.float32, generator=gen)
    q = torch.randn((R, hk, dk), **f)
    q = q / q.norm(dim=-1, keepdim=True)
    k = torch.randn((R, hk, dk), **f)
    k = k / k.norm(dim=-1, keepdim=True)
    v = torch.randn((R, hv, dv), **f)
    beta = torch.sigmoid(torch.randn((R, hv), **f))
    lo, hi = math.log(1e-3), math.log(8.0)
    g = -torch.exp(torch.rand((R, hv), **f) * (hi - lo) + lo)
    g[:, 0] = -1e-3
    g[:, hv - 1] = -8.0
    out = {"q": q.to(dtype), "k": k.to(dtype), "v": v.to(dtype), "beta": beta, "g": g,
           "S0": torch.zeros((P, hv, dk, dv), device=device, dtype=torch.float32)}
    if with_conv:
        cc = 2 * hk * dk + hv * dv
        out["conv_x"] = torch.randn((R, cc), **f).to(dtype)
        out["conv_state"] = torch.zeros((P, conv_k - 1, cc), device=device, dtype=dtype)
        out["conv_w"] = torch.randn((cc, conv_k), **f) * 0.5
    return out


def mixed_mamba_mixer(lens, device, seed: int | None = None, d_inner=5120, d_state=16) -> dict:
    """Packed inputs of the fused mixer rows at model width (same recipe as mamba_mixer_tiny,
    fresh state)."""
    gen = _gen(device, (seed_for(5) if seed is None else seed) * 8 + 4)
    R = int(sum(lens))
    P = len(lens)
    f = dict(device=device, dtype=torch.float32, generator=gen)
    return {
        "x": torch.randn((R, d_inner), **f),
        "dt": torch.rand((R, d_inner), **f) * (0.1 - 1e-3) + 1e-3,
        "A": -(torch.rand((d_inner, d_state), **f) * 15.0 + 1.0),
        "B": torch.randn((R, d_state), **f),
        "C": torch.randn((R, d_state), **f),
        "D": torch.randn((d_inner,), **f),
        "h0": torch.zeros((P, d_inner, d_state), device=device, dtype=torch.float32),
    }


def mixed_wkv_tdecay(lens, device, seed: int | None = None, channels=2560) -> dict:
    """Packed rows of the token-dependent-decay WKV at the RWKV-4 width of the mixed workload:
    the mixed RWKV-4 recipe with w_t = -exp(d_t), d_t ~ U(-6, 2) per row and channel (fresh state)."""
    gen = _gen(device, (seed_for(5) if seed is None else seed) * 8 + 6)
    R = int(sum(lens))
    P = len(lens)
    f = dict(device=device, dtype=torch.float32, generator=gen)
    u = torch.rand((channels,), **f) * 4.0 - 2.0
    k = torch.randn((R, channels), **f) * 3.0
    spike = torch.rand((R, channels), **f) < 0.01
    sign = torch.where(torch.rand((R, channels), **f) < 0.5, -1.0, 1.0)
    k = torch.where(spike, sign * 30.0, k)
    v = torch.randn((R, channels), **f)
    w = -torch.exp(torch.rand((R, channels), **f) * 8.0 - 6.0)
    return {"k": k, "v": v, "w": w, "u": u,
            "num": torch.zeros((P, channels), device=device), "den": torch.zeros((P, channels), device=device),
            "max": torch.full((P, channels), -1e38, device=device)}


def mixed_time_shift(lens, device, seed: int | None = None, channels=2560, mixes=3) -> dict:
    """Packed time-shift inputs at the RWKV-4 width of the mixed workload (fresh state)."""
    gen = _gen(device, (seed_for(5) if seed is None else seed) * 8 + 5)
    R = int(sum(lens))
    P = len(lens)
    f = dict(device=device, dtype=torch.float32, generator=gen)
    return {"x": torch.randn((R, channels), **f), "mix": torch.rand((mixes, channels), **f),
            "state": torch.zeros((P, channels), device=device, dtype=torch.float32)}
