"""ctypes binding of liblrc.so (include/lrc.h), one Python function per C entry point.

Argument marshalling only: each function checks that the torch tensors it is
given are CUDA (HIP) tensors of the right dtype, contiguous and of matching
shapes, reads the sizes off them, and passes raw device pointers and the
current stream to the C ABI.  Outputs are caller-allocated tensors, written in
place.  Every step of the computation runs in the HIP kernels; there is no
fallback.  Importing this module raises if liblrc.so is missing.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblrc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m linear_recurrence_chunked_amd.build` "
        "(hipcc, gfx950). There is no CPU fallback.")

lib = ctypes.CDLL(LIB_PATH)

MAX_ROWS = 64
MAX_PROMPTS = 256
MAX_CONV_K = 8
MAX_MIX = 8
F32, BF16, BF16_SPLIT = 0, 1, 2  # lrc_dtype

STATUS = {0: "LRC_OK", 1: "LRC_ERR_NULL", 2: "LRC_ERR_ROWS", 3: "LRC_ERR_SHAPE", 4: "LRC_ERR_DTYPE",
          5: "LRC_ERR_ALIGN", 6: "LRC_ERR_LAUNCH", 7: "LRC_ERR_ALIAS"}

_P, _I, _S = ctypes.c_void_p, ctypes.c_int, ctypes.c_int
_IP = ctypes.POINTER(ctypes.c_int)

_SIGS = {
    "lrc_conv_rows": [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P],
    "lrc_conv_prefill": [_P, _P, _P, _P, _P, _IP, _I, _I, _I, _I, _P],
    "lrc_scan_rows": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P],
    "lrc_scan_prefill": [_P, _P, _P, _P, _IP, _I, _I, _I, _P],
    "lrc_scan_prefill_ws": [_P, _P, _P, _P, _IP, _I, _I, _I, _P, ctypes.c_size_t, _P],
    "lrc_scan_prefill_static": [_P, _P, _P, _P, _IP, _I, _I, _I, _P],
    "lrc_wkv4_rows": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P],
    "lrc_wkv4_prefill": [_P, _P, _P, _P, _P, _P, _P, _P, _IP, _I, _I, _P],
    "lrc_wkv_tdecay_rows": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _P],
    "lrc_wkv_tdecay_prefill": [_P, _P, _P, _P, _P, _P, _P, _P, _IP, _I, _I, _P],
    "lrc_gdn_chunk": [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P],
    "lrc_gdn_prefill": [_P, _P, _P, _P, _P, _P, _P, _IP, _I, _I, _I, _I, _I, _I, _P],
    "lrc_gdn_prefill_ws": [_P, _P, _P, _P, _P, _P, _P, _IP, _I, _I, _I, _I, _I, _I, _P, ctypes.c_size_t, _P],
    "lrc_unit_lower_inverse": [_P, _P, _I, _I, _P],
    "lrc_time_shift_rows": [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P],
    "lrc_time_shift_prefill": [_P, _P, _P, _P, _IP, _I, _I, _I, _P],
    "lrc_mamba_mixer_rows": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P],
    "lrc_mamba_mixer_prefill": [_P, _P, _P, _P, _P, _P, _P, _P, _IP, _I, _I, _I, _P],
}
for _name, _args in _SIGS.items():
    _fn = getattr(lib, _name)
    _fn.argtypes = _args
    _fn.restype = _S
lib.lrc_wait_timeouts.argtypes = [ctypes.POINTER(ctypes.c_uint), _I, _P]
lib.lrc_wait_timeouts.restype = _S
lib.lrc_gdn_workspace_bytes.argtypes = [_I, ctypes.c_long, _I, _I, _I, _I, _I]
lib.lrc_gdn_workspace_bytes.restype = ctypes.c_size_t
lib.lrc_scan_workspace_size.argtypes = [_I, _I, _I]
lib.lrc_scan_workspace_size.restype = ctypes.c_size_t
lib.lrc_status_string.argtypes = [_S]
lib.lrc_status_string.restype = ctypes.c_char_p
lib.lrc_last_error.argtypes = []
lib.lrc_last_error.restype = ctypes.c_char_p
lib.lrc_version.argtypes = []
lib.lrc_version.restype = ctypes.c_int


class LrcError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS.get(status, str(status))
        super().__init__(f"{self.name}: {detail}")


def _check(status: int) -> None:
    if status != 0:
        raise LrcError(status, lib.lrc_last_error().decode())


def version() -> tuple[int, int, int]:
    v = lib.lrc_version()
    return (v >> 16) & 0xff, (v >> 8) & 0xff, v & 0xff


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(*ts: torch.Tensor | None) -> None:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("liblrc takes device tensors only (no CPU path)")
        if not t.is_contiguous():
            raise ValueError("liblrc takes contiguous tensors only")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on one device")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _gdn_dtype_code(q: torch.Tensor, split: bool) -> int:
    code = _dtype_code(q)
    if not split:
        return code
    if code != BF16:
        raise ValueError("split applies to bf16 inputs only")
    return BF16_SPLIT


def _need(t: torch.Tensor, dtype, shape, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")


def _lens(lens):
    lens = [int(x) for x in lens]
    return (ctypes.c_int * len(lens))(*lens), len(lens), sum(max(x, 0) for x in lens)


# ------------------------------------------------------------------ K0 conv
def conv_rows(x, y, state_in, state_out, w, bias=None):
    """x, y [B, S, C]; state_in, state_out [B, K-1, C] (may be the same tensor); w [C, K] f32."""
    _dev(x, y, state_in, state_out, w, bias)
    B, S, C = x.shape
    K = w.shape[1]
    _need(y, x.dtype, x.shape, "y")
    _need(w, torch.float32, (C, K), "w")
    _need(state_in, x.dtype, (B, K - 1, C), "state_in")
    _need(state_out, x.dtype, (B, K - 1, C), "state_out")
    if bias is not None:
        _need(bias, torch.float32, (C,), "bias")
    _check(lib.lrc_conv_rows(_ptr(x), _ptr(y), _ptr(state_in), _ptr(state_out), _ptr(w), _ptr(bias),
                             B, S, C, K, _dtype_code(x), _stream(x)))


def conv_prefill(x, y, state, w, lens, bias=None):
    """x, y [R, C] packed rows of len(lens) prompts; state [P, K-1, C] updated in place."""
    _dev(x, y, state, w, bias)
    R, C = x.shape
    K = w.shape[1]
    arr, P, total = _lens(lens)
    if total != R:
        raise ValueError(f"sum(lens) = {total} but x has {R} rows")
    _need(y, x.dtype, x.shape, "y")
    _need(w, torch.float32, (C, K), "w")
    _need(state, x.dtype, (P, K - 1, C), "state")
    if bias is not None:
        _need(bias, torch.float32, (C,), "bias")
    _check(lib.lrc_conv_prefill(_ptr(x), _ptr(y), _ptr(state), _ptr(w), _ptr(bias), arr, P, C, K,
                                _dtype_code(x), _stream(x)))


# ------------------------------------------------------------------ K1 scan
def scan_rows(a, b, h, h0, hS):
    """a, b, h [B, S, D, N] f32; h0, hS [B, D, N] f32 (may be the same tensor)."""
    _dev(a, b, h, h0, hS)
    B, S, D, N = a.shape
    for t, n in ((b, "b"), (h, "h")):
        _need(t, torch.float32, a.shape, n)
    _need(a, torch.float32, a.shape, "a")
    _need(h0, torch.float32, (B, D, N), "h0")
    _need(hS, torch.float32, (B, D, N), "hS")
    _check(lib.lrc_scan_rows(_ptr(a), _ptr(b), _ptr(h), _ptr(h0), _ptr(hS), B, S, D, N, _stream(a)))


def scan_prefill(a, b, h, state, lens):
    """a, b, h [R, D, N] f32 packed rows; state [P, D, N] f32 updated in place."""
    _dev(a, b, h, state)
    R, D, N = a.shape
    arr, P, total = _lens(lens)
    if total != R:
        raise ValueError(f"sum(lens) = {total} but a has {R} rows")
    for t, n in ((a, "a"), (b, "b"), (h, "h")):
        _need(t, torch.float32, (R, D, N), n)
    _need(state, torch.float32, (P, D, N), "state")
    _check(lib.lrc_scan_prefill(_ptr(a), _ptr(b), _ptr(h), _ptr(state), arr, P, D, N, _stream(a)))


def scan_workspace_size(P: int, D: int, N: int) -> int:
    """Bytes of workspace scan_prefill_ws needs for P prompts of D x N state elements."""
    return int(lib.lrc_scan_workspace_size(P, D, N))


def scan_workspace(P: int, D: int, N: int, device) -> torch.Tensor:
    """A zero-filled workspace for scan_prefill_ws (uint8, reusable across calls that do not overlap)."""
    return torch.zeros(scan_workspace_size(P, D, N), dtype=torch.uint8, device=device)


def scan_workspace_timeouts(ws: torch.Tensor) -> int:
    """Hand-overs of scan_prefill_ws that timed out since the workspace was made (0 unless progress failed)."""
    return int(ws[:4].view(torch.int32).item())


def scan_prefill_ws(a, b, h, state, lens, ws):
    """scan_prefill in its tiled form; ws from scan_workspace(P, D, N, device)."""
    _dev(a, b, h, state, ws)
    R, D, N = a.shape
    arr, P, total = _lens(lens)
    if total != R:
        raise ValueError(f"sum(lens) = {total} but a has {R} rows")
    for t, n in ((a, "a"), (b, "b"), (h, "h")):
        _need(t, torch.float32, (R, D, N), n)
    _need(state, torch.float32, (P, D, N), "state")
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous 1-D uint8 tensor")
    _check(lib.lrc_scan_prefill_ws(_ptr(a), _ptr(b), _ptr(h), _ptr(state), arr, P, D, N, _ptr(ws), ws.numel(),
                                   _stream(a)))


def scan_prefill_static(a, b, h, state, lens):
    """scan_prefill_ws without a workspace: the library's fixed 2 MiB device scratch (one per GPU)
    holds the tiled driver's flags.  Calls that overlap on one GPU race."""
    _dev(a, b, h, state)
    R, D, N = a.shape
    arr, P, total = _lens(lens)
    if total != R:
        raise ValueError(f"sum(lens) = {total} but a has {R} rows")
    for t, n in ((a, "a"), (b, "b"), (h, "h")):
        _need(t, torch.float32, (R, D, N), n)
    _need(state, torch.float32, (P, D, N), "state")
    _check(lib.lrc_scan_prefill_static(_ptr(a), _ptr(b), _ptr(h), _ptr(state), arr, P, D, N, _stream(a)))


def wait_timeouts(reset: bool = False) -> int:
    """Bounded in-workgroup waits of the WKV kernels that gave up on the current GPU (0 unless a launch
    could not make progress).  Synchronizes the current stream; with reset, sets the count back to 0."""
    n = ctypes.c_uint(0)
    _check(lib.lrc_wait_timeouts(ctypes.byref(n), int(reset), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)))
    return int(n.value)


# ------------------------------------------------------------------ K2 wkv
def wkv4_rows(k, v, w, u, wkv, num, den, mx):
    """k, v, wkv [B, S, C] f32; w, u [C]; num, den, mx [B, C] updated in place."""
    _dev(k, v, w, u, wkv, num, den, mx)
    B, S, C = k.shape
    for t, n in ((k, "k"), (v, "v"), (wkv, "wkv")):
        _need(t, torch.float32, (B, S, C), n)
    for t, n in ((w, "w"), (u, "u")):
        _need(t, torch.float32, (C,), n)
    for t, n in ((num, "num"), (den, "den"), (mx, "max")):
        _need(t, torch.float32, (B, C), n)
    _check(lib.lrc_wkv4_rows(_ptr(k), _ptr(v), _ptr(w), _ptr(u), _ptr(wkv), _ptr(num), _ptr(den), _ptr(mx),
                             B, S, C, _stream(k)))


def wkv4_prefill(k, v, w, u, wkv, num, den, mx, lens):
    """k, v, wkv [R, C] packed rows; num, den, mx [P, C] updated in place."""
    _dev(k, v, w, u, wkv, num, den, mx)
    R, C = k.shape
    arr, P, total = _lens(lens)
    if total != R:
        raise ValueError(f"sum(lens) = {total} but k has {R} rows")
    for t, n in ((k, "k"), (v, "v"), (wkv, "wkv")):
        _need(t, torch.float32, (R, C), n)
    for t, n in ((w, "w"), (u, "u")):
        _need(t, torch.float32, (C,), n)
    for t, n in ((num, "num"), (den, "den"), (mx, "max")):
        _need(t, torch.float32, (P, C), n)
    _check(lib.lrc_wkv4_prefill(_ptr(k), _ptr(v), _ptr(w), _ptr(u), _ptr(wkv), _ptr(num), _ptr(den), _ptr(mx),
                                arr, P, C, _stream(k)))


# ------------------------------------------------------------------ WKV, token-dependent decay
def wkv_tdecay_rows(k, v, w, u, wkv, num, den, mx):
    """k, v, w, wkv [B, S, C] f32 (w: decay of each row); u [C]; num, den, mx [B, C] updated in place."""
    _dev(k, v, w, u, wkv, num, den, mx)
    B, S, C = k.shape
    for t, n in ((k, "k"), (v, "v"), (w, "w"), (wkv, "wkv")):
        _need(t, torch.float32, (B, S, C), n)
    _need(u, torch.float32, (C,), "u")
    for t, n in ((num, "num"), (den, "den"), (mx, "max")):
        _need(t, torch.float32, (B, C), n)
    _check(lib.lrc_wkv_tdecay_rows(_ptr(k), _ptr(v), _ptr(w), _ptr(u), _ptr(wkv), _ptr(num), _ptr(den), _ptr(mx),
                                   B, S, C, _stream(k)))


def wkv_tdecay_prefill(k, v, w, u, wkv, num, den, mx, lens):
    """k, v, w, wkv [R, C] packed rows; num, den, mx [P, C] updated in place."""
    _dev(k, v, w, u, wkv, num, den, mx)
    R, C = k.shape
    arr, P, total = _lens(lens)
    if total != R:
        raise ValueError(f"sum(lens) = {total} but k has {R} rows")
    for t, n in ((k, "k"), (v, "v"), (w, "w"), (wkv, "wkv")):
        _need(t, torch.float32, (R, C), n)
    _need(u, torch.float32, (C,), "u")
    for t, n in ((num, "num"), (den, "den"), (mx, "max")):
        _need(t, torch.float32, (P, C), n)
    _check(lib.lrc_wkv_tdecay_prefill(_ptr(k), _ptr(v), _ptr(w), _ptr(u), _ptr(wkv), _ptr(num), _ptr(den),
                                      _ptr(mx), arr, P, C, _stream(k)))


# ------------------------------------------------------------------ K3 gdn
def gdn_chunk(q, k, v, beta, g, o, S_in, S_out, split=False):
    """q, k [B, S, Hk, dk]; v [B, S, Hv, dv] (f32 or bf16); beta, g [B, S, Hv] f32;
    o [B, S, Hv, dv] f32; S_in, S_out [B, Hv, dk, dv] f32 (may be the same tensor).
    split (bf16 only): FP32 operands of the matrix products as hi + lo bf16 pairs."""
    _dev(q, k, v, beta, g, o, S_in, S_out)
    B, S, Hk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    _need(k, q.dtype, q.shape, "k")
    _need(v, q.dtype, (B, S, Hv, dv), "v")
    _need(beta, torch.float32, (B, S, Hv), "beta")
    _need(g, torch.float32, (B, S, Hv), "g")
    _need(o, torch.float32, (B, S, Hv, dv), "o")
    _need(S_in, torch.float32, (B, Hv, dk, dv), "S_in")
    _need(S_out, torch.float32, (B, Hv, dk, dv), "S_out")
    _check(lib.lrc_gdn_chunk(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(o), _ptr(S_in), _ptr(S_out),
                             B, S, Hk, Hv, dk, dv, _gdn_dtype_code(q, split), _stream(q)))


def gdn_prefill(q, k, v, beta, g, o, state, lens, split=False):
    """q, k [R, Hk, dk]; v [R, Hv, dv]; beta, g [R, Hv]; o [R, Hv, dv] packed rows;
    state [P, Hv, dk, dv] f32 updated in place.  split as in gdn_chunk."""
    _dev(q, k, v, beta, g, o, state)
    R, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    arr, P, total = _lens(lens)
    if total != R:
        raise ValueError(f"sum(lens) = {total} but q has {R} rows")
    _need(k, q.dtype, q.shape, "k")
    _need(v, q.dtype, (R, Hv, dv), "v")
    _need(beta, torch.float32, (R, Hv), "beta")
    _need(g, torch.float32, (R, Hv), "g")
    _need(o, torch.float32, (R, Hv, dv), "o")
    _need(state, torch.float32, (P, Hv, dk, dv), "state")
    _check(lib.lrc_gdn_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(o), _ptr(state), arr, P,
                               Hk, Hv, dk, dv, _gdn_dtype_code(q, split), _stream(q)))


def gdn_workspace_bytes(P: int, total_rows: int, Hk: int, Hv: int, dk: int, dv: int) -> int:
    """Bytes of workspace gdn_prefill_ws needs for P prompts of total_rows rows (bf16 inputs)."""
    return int(lib.lrc_gdn_workspace_bytes(P, total_rows, Hk, Hv, dk, dv, BF16))


def gdn_workspace(P: int, total_rows: int, Hk: int, Hv: int, dk: int, dv: int, device) -> torch.Tensor:
    """A workspace for gdn_prefill_ws (uint8; no initial contents needed)."""
    return torch.empty(gdn_workspace_bytes(P, total_rows, Hk, Hv, dk, dv), dtype=torch.uint8, device=device)


def gdn_prefill_ws(q, k, v, beta, g, o, state, lens, ws):
    """gdn_prefill in its chunk-parallel form (bf16 q, k, v): the state-free part of every chunk at
    once into ws, then the state products chunk by chunk.  ws from gdn_workspace."""
    _dev(q, k, v, beta, g, o, state, ws)
    R, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    arr, P, total = _lens(lens)
    if total != R:
        raise ValueError(f"sum(lens) = {total} but q has {R} rows")
    if q.dtype != torch.bfloat16:
        raise ValueError("gdn_prefill_ws takes bf16 q, k, v")
    _need(k, q.dtype, q.shape, "k")
    _need(v, q.dtype, (R, Hv, dv), "v")
    _need(beta, torch.float32, (R, Hv), "beta")
    _need(g, torch.float32, (R, Hv), "g")
    _need(o, torch.float32, (R, Hv, dv), "o")
    _need(state, torch.float32, (P, Hv, dk, dv), "state")
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous 1-D uint8 tensor")
    _check(lib.lrc_gdn_prefill_ws(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(o), _ptr(state), arr, P,
                                  Hk, Hv, dk, dv, BF16, _ptr(ws), ws.numel(), _stream(q)))


def unit_lower_inverse(A, T):
    """A, T [batch, n, n] f32: T = (I + strictly_lower(A))^-1, n <= 64."""
    _dev(A, T)
    batch, n, _ = A.shape
    _need(A, torch.float32, (batch, n, n), "A")
    _need(T, torch.float32, (batch, n, n), "T")
    _check(lib.lrc_unit_lower_inverse(_ptr(A), _ptr(T), batch, n, _stream(A)))


# ------------------------------------------------------------------ RWKV-4 time shift
def time_shift_rows(x, out, state_in, state_out, mix):
    """x [B, S, C] f32; out [M, B, S, C] f32; state_in, state_out [B, C] (may be the same tensor);
    mix [M, C] f32."""
    _dev(x, out, state_in, state_out, mix)
    B, S, C = x.shape
    M = mix.shape[0]
    _need(x, torch.float32, x.shape, "x")
    _need(out, torch.float32, (M, B, S, C), "out")
    _need(mix, torch.float32, (M, C), "mix")
    _need(state_in, torch.float32, (B, C), "state_in")
    _need(state_out, torch.float32, (B, C), "state_out")
    _check(lib.lrc_time_shift_rows(_ptr(x), _ptr(out), _ptr(state_in), _ptr(state_out), _ptr(mix), B, S, C, M,
                                   _stream(x)))


def time_shift_prefill(x, out, state, mix, lens):
    """x [R, C] packed rows; out [M, R, C]; state [P, C] updated in place; mix [M, C]."""
    _dev(x, out, state, mix)
    R, C = x.shape
    M = mix.shape[0]
    arr, P, total = _lens(lens)
    if total != R:
        raise ValueError(f"sum(lens) = {total} but x has {R} rows")
    _need(x, torch.float32, (R, C), "x")
    _need(out, torch.float32, (M, R, C), "out")
    _need(mix, torch.float32, (M, C), "mix")
    _need(state, torch.float32, (P, C), "state")
    _check(lib.lrc_time_shift_prefill(_ptr(x), _ptr(out), _ptr(state), _ptr(mix), arr, P, C, M, _stream(x)))


# ------------------------------------------------------------------ fused Mamba mixer rows
def mamba_mixer_rows(x, dt, A, Bm, Cm, Dp, y, h_in, h_out):
    """x, dt, y [B, S, D]; Bm, Cm [B, S, N]; A [D, N]; Dp [D]; h_in, h_out [B, D, N] (may be the
    same tensor); all f32."""
    _dev(x, dt, A, Bm, Cm, Dp, y, h_in, h_out)
    B, S, D = x.shape
    N = A.shape[1]
    for t, n in ((x, "x"), (dt, "dt"), (y, "y")):
        _need(t, torch.float32, (B, S, D), n)
    for t, n in ((Bm, "Bm"), (Cm, "Cm")):
        _need(t, torch.float32, (B, S, N), n)
    _need(A, torch.float32, (D, N), "A")
    _need(Dp, torch.float32, (D,), "Dp")
    _need(h_in, torch.float32, (B, D, N), "h_in")
    _need(h_out, torch.float32, (B, D, N), "h_out")
    _check(lib.lrc_mamba_mixer_rows(_ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dp), _ptr(y), _ptr(h_in),
                                    _ptr(h_out), B, S, D, N, _stream(x)))


def mamba_mixer_prefill(x, dt, A, Bm, Cm, Dp, y, state, lens):
    """x, dt, y [R, D]; Bm, Cm [R, N] packed rows; A [D, N]; Dp [D]; state [P, D, N] updated in place."""
    _dev(x, dt, A, Bm, Cm, Dp, y, state)
    R, D = x.shape
    N = A.shape[1]
    arr, P, total = _lens(lens)
    if total != R:
        raise ValueError(f"sum(lens) = {total} but x has {R} rows")
    for t, n in ((x, "x"), (dt, "dt"), (y, "y")):
        _need(t, torch.float32, (R, D), n)
    for t, n in ((Bm, "Bm"), (Cm, "Cm")):
        _need(t, torch.float32, (R, N), n)
    _need(A, torch.float32, (D, N), "A")
    _need(Dp, torch.float32, (D,), "Dp")
    _need(state, torch.float32, (P, D, N), "state")
    _check(lib.lrc_mamba_mixer_prefill(_ptr(x), _ptr(dt), _ptr(A), _ptr(Bm), _ptr(Cm), _ptr(Dp), _ptr(y),
                                       _ptr(state), arr, P, D, N, _stream(x)))
