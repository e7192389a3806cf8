"""Float64 CPU oracle: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path
(``linear_recurrence_chunked_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, float64, one token at a time);
this module compiles it with gcc into ``liboracle.so`` and marshals numpy
arrays.  Every function takes arrays of any float dtype, upcasts them to
float64 once, and returns float64 arrays.  Citations to the pages are in the C
source next to each routine.

Parity of every routine is pinned by ``tests/test_oracle_*.py`` against
brute-force sums, closed forms, library routines and invariants, never against
the HIP path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_CFLAGS = ["-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no GPU code involved)."""
    global _lib
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
        _lib = None
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_conv_rows.argtypes = [P, P, P, P, I, I, I, P, P]
        lib.oracle_scan.argtypes = [P, P, P, I, ctypes.c_long, P, P]
        lib.oracle_wkv4.argtypes = [P, P, P, P, I, I, P, P, P, P]
        lib.oracle_wkv_tdecay.argtypes = [P, P, P, P, I, I, P, P, P, P]
        lib.oracle_gdn.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, P]
        lib.oracle_unit_lower_inverse.argtypes = [P, I, I, P]
        lib.oracle_time_shift.argtypes = [P, P, P, I, I, I, P, P]
        lib.oracle_mamba_mixer.argtypes = [P, P, P, P, P, P, P, I, I, I, P, P]
        lib.oracle_num_threads.restype = I
        lib.oracle_set_num_threads.argtypes = [I]
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def set_num_threads(n: int) -> None:
    _load().oracle_set_num_threads(int(n))


def conv_rows(x, state_in, w, bias=None):
    """Depthwise causal conv.  x [S, C], state_in [K-1, C], w [C, K], bias [C] or None.

    Returns (y [S, C], state_out [K-1, C]).
    """
    x, state_in, w = _f64(x), _f64(state_in), _f64(w)
    S, C = x.shape
    K = w.shape[1]
    assert w.shape == (C, K) and K >= 1 and state_in.shape == (K - 1, C)
    b = None if bias is None else _f64(bias)
    y = np.empty((S, C))
    st = np.empty((K - 1, C))
    _load().oracle_conv_rows(_p(x), _p(state_in), _p(w), None if b is None else _p(b), S, C, K, _p(y), _p(st))
    return y, st


def scan(a, b, h0):
    """Selective scan h_t = a_t h_{t-1} + b_t.  a, b [S, E], h0 [E].  Returns (h [S, E], hS [E])."""
    a, b, h0 = _f64(a), _f64(b), _f64(h0)
    S = a.shape[0]
    E = int(np.prod(a.shape[1:])) if a.ndim > 1 else 1
    assert b.shape == a.shape and h0.size == E
    h = np.empty(a.shape)
    hS = np.empty(h0.shape)
    _load().oracle_scan(_p(a), _p(b), _p(h0), S, E, _p(h), _p(hS))
    return h, hS


def empty_wkv_state(C: int):
    """(num, den, max) of an RWKV-4 channel that has seen no token."""
    return np.zeros(C), np.zeros(C), np.full(C, -1e38)


def wkv4(k, v, w, u, num, den, mx):
    """RWKV-4 WKV token loop.  k, v [S, C]; w, u, num, den, mx [C].

    Returns (wkv [S, C], num_S, den_S, max_S).
    """
    k, v, w, u = _f64(k), _f64(v), _f64(w), _f64(u)
    S, C = k.shape
    n, d, m = _f64(num).copy(), _f64(den).copy(), _f64(mx).copy()
    assert v.shape == (S, C) and w.shape == (C,) and u.shape == (C,) and n.shape == (C,)
    out = np.empty((S, C))
    _load().oracle_wkv4(_p(k), _p(v), _p(w), _p(u), S, C, _p(n), _p(d), _p(m), _p(out))
    return out, n, d, m


def wkv_tdecay(k, v, w, u, num, den, mx):
    """WKV token loop with a decay per row.  k, v, w [S, C]; u, num, den, mx [C].

    Returns (wkv [S, C], num_S, den_S, max_S).
    """
    k, v, w, u = _f64(k), _f64(v), _f64(w), _f64(u)
    S, C = k.shape
    n, d, m = _f64(num).copy(), _f64(den).copy(), _f64(mx).copy()
    assert v.shape == (S, C) and w.shape == (S, C) and u.shape == (C,) and n.shape == (C,)
    out = np.empty((S, C))
    _load().oracle_wkv_tdecay(_p(k), _p(v), _p(w), _p(u), S, C, _p(n), _p(d), _p(m), _p(out))
    return out, n, d, m


def gdn(q, k, v, beta, g, S0):
    """Gated DeltaNet token loop.  q, k [S, Hk, dk]; v [S, Hv, dv]; beta, g [S, Hv];
    S0 [Hv, dk, dv].  Returns (o [S, Hv, dv], S_S [Hv, dk, dv])."""
    q, k, v, beta, g, S0 = map(_f64, (q, k, v, beta, g, S0))
    S, Hk, dk = k.shape
    Hv, dv = v.shape[1], v.shape[2]
    assert q.shape == k.shape and v.shape[0] == S and beta.shape == (S, Hv) and g.shape == (S, Hv)
    assert S0.shape == (Hv, dk, dv) and Hv % Hk == 0 and dv <= 1024
    o = np.empty((S, Hv, dv))
    Sout = np.empty((Hv, dk, dv))
    _load().oracle_gdn(_p(q), _p(k), _p(v), _p(beta), _p(g), _p(S0), S, Hk, Hv, dk, dv, _p(o), _p(Sout))
    return o, Sout


def unit_lower_inverse(L):
    """Inverse of I + strictly_lower(L) by forward substitution.  L [..., n, n]."""
    L = _f64(L)
    n = L.shape[-1]
    batch = int(np.prod(L.shape[:-2])) if L.ndim > 2 else 1
    T = np.empty(L.shape)
    _load().oracle_unit_lower_inverse(_p(L), batch, n, _p(T))
    return T


def time_shift(x, state_in, mix):
    """RWKV-4 time shift.  x [S, C], state_in [C], mix [M, C].

    Returns (out [M, S, C], state_out [C]).
    """
    x, state_in, mix = _f64(x), _f64(state_in), _f64(mix)
    S, C = x.shape
    M = mix.shape[0]
    assert state_in.shape == (C,) and mix.shape == (M, C)
    out = np.empty((M, S, C))
    st = np.empty(C)
    _load().oracle_time_shift(_p(x), _p(state_in), _p(mix), S, C, M, _p(out), _p(st))
    return out, st


def mamba_mixer(x, dt, A, B, C, D, h0):
    """Mamba mixer rows: a = exp(dt A), b = dt B x, h_t = a h_{t-1} + b, y = C.h + D x.

    x, dt [S, Dm]; A [Dm, N]; B, C [S, N]; D [Dm]; h0 [Dm, N].  Returns (y [S, Dm], hS [Dm, N]).
    """
    x, dt, A, B, C, D, h0 = map(_f64, (x, dt, A, B, C, D, h0))
    S, Dm = x.shape
    N = A.shape[1]
    assert dt.shape == (S, Dm) and A.shape == (Dm, N) and B.shape == (S, N) and C.shape == (S, N)
    assert D.shape == (Dm,) and h0.shape == (Dm, N) and N <= 256
    y = np.empty((S, Dm))
    hS = np.empty((Dm, N))
    _load().oracle_mamba_mixer(_p(x), _p(dt), _p(A), _p(B), _p(C), _p(D), _p(h0), S, Dm, N, _p(y), _p(hS))
    return y, hS
