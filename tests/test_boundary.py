"""The C ABI loads, exports every symbol include/lrc.h declares, and rejects bad
arguments on the host before any HIP call (these tests run without a GPU and
never pass validation, so nothing is launched).

Sources: the pages reject chunks of more than 64 rows ("perf(rwkv): ...",
"perf(mamba): ...", "perf(qwen3_5): ...", Tests) and validate before work is
queued; the argument rules themselves are this library's.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lrc.h")


@pytest.fixture(scope="module")
def L():
    from linear_recurrence_chunked_amd import lrc

    return lrc


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(lrc_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ["lrc_conv_rows", "lrc_conv_prefill", "lrc_scan_rows", "lrc_scan_prefill", "lrc_wkv4_rows",
              "lrc_wkv4_prefill", "lrc_gdn_chunk", "lrc_gdn_prefill", "lrc_unit_lower_inverse",
              "lrc_time_shift_rows", "lrc_time_shift_prefill", "lrc_mamba_mixer_rows", "lrc_mamba_mixer_prefill",
              "lrc_wkv_tdecay_rows", "lrc_wkv_tdecay_prefill", "lrc_scan_prefill_ws", "lrc_scan_workspace_size",
              "lrc_scan_prefill_static", "lrc_wait_timeouts", "lrc_gdn_prefill_ws", "lrc_gdn_workspace_bytes",
              "lrc_status_string", "lrc_last_error", "lrc_version"]:
        assert n in names


def test_library_exports_every_declared_symbol(L):
    missing = [n for n in _declared() if not hasattr(L.lib, n)]
    assert not missing, missing


def test_version_and_status_strings(L):
    assert L.version() >= (0, 1, 0)
    for code in range(8):
        s = L.lib.lrc_status_string(code).decode()
        assert s and s != "unknown status"


# Fake, 16-byte aligned, non-null "device" addresses, far apart so that they
# never overlap.  Validation rejects every call below before touching them.
A0, A1, A2, A3, A4, A5, A6, A7 = (0x10000000 * (i + 1) for i in range(8))
MIS = A0 + 4  # misaligned


def _st(L, code):
    return L.STATUS[code]


def test_scan_rejects_rows_above_64_and_negative(L):
    for S in (65, 1000, -1):
        assert _st(L, L.lib.lrc_scan_rows(A0, A1, A2, A3, A4, 1, S, 4, 16, None)) == "LRC_ERR_ROWS"
    assert "64" in L.lib.lrc_last_error().decode()


def test_scan_rejects_null_misaligned_alias(L):
    assert _st(L, L.lib.lrc_scan_rows(None, A1, A2, A3, A4, 1, 8, 4, 16, None)) == "LRC_ERR_NULL"
    assert _st(L, L.lib.lrc_scan_rows(MIS, A1, A2, A3, A4, 1, 8, 4, 16, None)) == "LRC_ERR_ALIGN"
    assert _st(L, L.lib.lrc_scan_rows(A0, A1, A0, A3, A4, 1, 8, 4, 16, None)) == "LRC_ERR_ALIAS"
    assert _st(L, L.lib.lrc_scan_rows(A0, A1, A2, A3, A4, 1, 8, 0, 16, None)) == "LRC_ERR_SHAPE"
    assert _st(L, L.lib.lrc_scan_rows(A0, A1, A2, A3, A4, -1, 8, 4, 16, None)) == "LRC_ERR_SHAPE"
    # partial overlap of the state buffers is rejected, exact aliasing is allowed (checked on GPU)
    assert _st(L, L.lib.lrc_scan_rows(A0, A1, A2, A3, A3 + 16, 1, 8, 4, 16, None)) == "LRC_ERR_ALIAS"


def test_prefill_rejects_bad_lengths(L):
    lens = (ctypes.c_int * 3)(5, -1, 7)
    assert _st(L, L.lib.lrc_scan_prefill(A0, A1, A2, A3, lens, 3, 4, 16, None)) == "LRC_ERR_ROWS"
    assert _st(L, L.lib.lrc_scan_prefill(A0, A1, A2, A3, None, 3, 4, 16, None)) == "LRC_ERR_NULL"
    lens = (ctypes.c_int * 1)(5)
    assert _st(L, L.lib.lrc_scan_prefill(A0, A1, A2, A3, lens, 0, 4, 16, None)) == "LRC_ERR_SHAPE"
    big = (ctypes.c_int * 300)(*([1] * 300))
    assert _st(L, L.lib.lrc_wkv4_prefill(A0, A1, A2, A3, A4, A5, A6, A7, big, 300, 8, None)) == "LRC_ERR_SHAPE"


def test_scan_tiled_workspace_size_and_rejects(L):
    # a control block, then one 8-byte flag per (prompt, block of 128 state elements)
    assert L.scan_workspace_size(16, 5120, 16) == 256 + 16 * 640 * 8
    assert L.scan_workspace_size(3, 5, 3) == 256 + 3 * 8
    assert L.scan_workspace_size(0, 4, 16) == 0
    f = L.lib.lrc_scan_prefill_ws
    lens = (ctypes.c_int * 3)(5, 1, 7)
    need = L.scan_workspace_size(3, 4, 16)
    assert _st(L, f(A0, A1, A2, A3, lens, 3, 4, 16, None, need, None)) == "LRC_ERR_NULL"
    assert _st(L, f(A0, A1, A2, A3, lens, 3, 4, 16, A4, need - 1, None)) == "LRC_ERR_SHAPE"
    assert _st(L, f(A0, A1, A2, A3, lens, 3, 4, 16, A4 + 4, need, None)) == "LRC_ERR_ALIGN"
    assert _st(L, f(A0, A1, A2, A3, lens, 3, 4, 16, A2 + 64, need, None)) == "LRC_ERR_ALIAS"  # inside h
    assert _st(L, f(A0, A1, A2, A3, lens, 3, 4, 16, A3, need, None)) == "LRC_ERR_ALIAS"  # on the state
    bad = (ctypes.c_int * 3)(5, -1, 7)
    assert _st(L, f(A0, A1, A2, A3, bad, 3, 4, 16, A4, need, None)) == "LRC_ERR_ROWS"


def test_scan_static_rejects_beyond_its_scratch(L):
    """The allocation-free tiled scan keeps its flags in a fixed 2 MiB array: a 256-byte control block
    and one 8-byte flag per (prompt, block of 128 state elements), so at most 262 112 such pairs."""
    f = L.lib.lrc_scan_prefill_static
    lens = (ctypes.c_int * 256)(*([3] * 256))
    far = [0x1000000000 * (i + 1) for i in range(4)]  # 64 GiB apart: the tensors below never overlap
    # 256 prompts x 1024 blocks (D * N = 131 072) need 256 + 8 * 262 144 bytes: one block too many per prompt
    assert _st(L, f(*far, lens, 256, 8192, 16, None)) == "LRC_ERR_SHAPE"
    assert "scratch" in L.lib.lrc_last_error().decode()
    bad = (ctypes.c_int * 3)(5, -1, 7)
    assert _st(L, f(A0, A1, A2, A3, bad, 3, 4, 16, None)) == "LRC_ERR_ROWS"
    lens3 = (ctypes.c_int * 3)(5, 1, 7)
    assert _st(L, f(None, A1, A2, A3, lens3, 3, 4, 16, None)) == "LRC_ERR_NULL"
    assert _st(L, f(A0, A1, A0, A3, lens3, 3, 4, 16, None)) == "LRC_ERR_ALIAS"
    assert _st(L, f(MIS, A1, A2, A3, lens3, 3, 4, 16, None)) == "LRC_ERR_ALIGN"


def test_gdn_chunk_parallel_workspace_and_rejects(L):
    """The chunk-parallel DeltaNet form: one workspace block per (64-row chunk, value head) of
    W, K^T, P (bf16), U' (FP32) and two per-row vectors, 72.5 KiB at dk = dv = 128; bf16 only."""
    blk = 256 * 128 + 64 * 64 * 2 + 256 * 128 + 512
    assert blk == 74240
    assert L.gdn_workspace_bytes(1, 2048, 16, 32, 128, 128) == (2048 // 64 + 1) * 32 * blk
    assert L.gdn_workspace_bytes(1, 64, 1, 1, 32, 32) == 2 * (256 * 32 + 8192 + 256 * 32 + 512)
    assert L.lib.lrc_gdn_workspace_bytes(1, 64, 1, 1, 32, 32, L.F32) == 0
    assert L.lib.lrc_gdn_workspace_bytes(1, 64, 2, 3, 32, 32, L.BF16) == 0
    f = L.lib.lrc_gdn_prefill_ws
    lens = (ctypes.c_int * 2)(70, 5)  # 3 chunks
    need = 3 * 4 * (256 * 64 + 8192 + 256 * 64 + 512)
    args = [A0, A1, A2, A3, A4, A5, A6, lens, 2, 2, 4, 64, 64]
    assert _st(L, f(*args, L.F32, A7, need, None)) == "LRC_ERR_DTYPE"
    assert _st(L, f(*args, L.BF16_SPLIT, A7, need, None)) == "LRC_ERR_DTYPE"
    assert _st(L, f(*args, L.BF16, A7, need - 1, None)) == "LRC_ERR_SHAPE"
    assert _st(L, f(*args, L.BF16, None, need, None)) == "LRC_ERR_NULL"
    assert _st(L, f(*args, L.BF16, A7 + 8, need, None)) == "LRC_ERR_ALIGN"
    assert _st(L, f(*args, L.BF16, A6 + 64, need, None)) == "LRC_ERR_ALIAS"  # inside the state
    bad = (ctypes.c_int * 2)(70, -5)
    assert _st(L, f(A0, A1, A2, A3, A4, A5, A6, bad, 2, 2, 4, 64, 64, L.BF16, A7, need, None)) == "LRC_ERR_ROWS"


def test_conv_rejects_bad_width_dtype_rows(L):
    f = L.lib.lrc_conv_rows
    assert _st(L, f(A0, A1, A2, A3, A4, None, 1, 8, 16, 0, 0, None)) == "LRC_ERR_SHAPE"
    assert _st(L, f(A0, A1, A2, A3, A4, None, 1, 8, 16, 9, 0, None)) == "LRC_ERR_SHAPE"
    assert _st(L, f(A0, A1, A2, A3, A4, None, 1, 8, 16, 4, 7, None)) == "LRC_ERR_DTYPE"
    assert _st(L, f(A0, A1, A2, A3, A4, None, 1, 8, 16, 4, L.BF16_SPLIT, None)) == "LRC_ERR_DTYPE"  # K3 only
    assert _st(L, f(A0, A1, A2, A3, A4, None, 1, 65, 16, 4, 0, None)) == "LRC_ERR_ROWS"
    assert _st(L, f(A0, A0, A2, A3, A4, None, 1, 8, 16, 4, 0, None)) == "LRC_ERR_ALIAS"
    assert _st(L, f(A0, A1, None, A3, A4, None, 1, 8, 16, 4, 0, None)) == "LRC_ERR_NULL"


def test_wkv_rejects(L):
    f = L.lib.lrc_wkv4_rows
    assert _st(L, f(A0, A1, A2, A3, A4, A5, A6, A7, 1, 65, 8, None)) == "LRC_ERR_ROWS"
    assert _st(L, f(A0, A1, A2, A3, A4, A5, A5, A7, 1, 8, 8, None)) == "LRC_ERR_ALIAS"
    assert _st(L, f(A0, A1, A2, A3, A4, A5, A6, None, 1, 8, 8, None)) == "LRC_ERR_NULL"
    assert _st(L, f(A0, A1, A2, A3, A4, A5, A6, A7, 1, 8, 0, None)) == "LRC_ERR_SHAPE"


def test_wkv_tdecay_rejects(L):
    f = L.lib.lrc_wkv_tdecay_rows
    assert _st(L, f(A0, A1, A2, A3, A4, A5, A6, A7, 1, 65, 8, None)) == "LRC_ERR_ROWS"
    assert _st(L, f(A0, A1, A2, A3, A2, A5, A6, A7, 1, 8, 8, None)) == "LRC_ERR_ALIAS"  # wkv over the decays
    assert _st(L, f(A0, A1, A2, A3, A4, A5, A6, A2, 1, 8, 8, None)) == "LRC_ERR_ALIAS"  # state over the decays
    assert _st(L, f(A0, A1, None, A3, A4, A5, A6, A7, 1, 8, 8, None)) == "LRC_ERR_NULL"
    assert _st(L, f(A0, A1, MIS, A3, A4, A5, A6, A7, 1, 8, 8, None)) == "LRC_ERR_ALIGN"
    assert _st(L, f(A0, A1, A2, A3, A4, A5, A6, A7, 1, 8, 0, None)) == "LRC_ERR_SHAPE"
    lens = (ctypes.c_int * 2)(8, -1)
    assert _st(L, L.lib.lrc_wkv_tdecay_prefill(A0, A1, A2, A3, A4, A5, A6, A7, lens, 2, 8, None)) == "LRC_ERR_ROWS"


def test_gdn_rejects(L):
    f = L.lib.lrc_gdn_chunk
    ok_args = [A0, A1, A2, A3, A4, A5, A6, A7]
    assert _st(L, f(*ok_args, 1, 65, 2, 4, 64, 64, 1, None)) == "LRC_ERR_ROWS"
    assert _st(L, f(*ok_args, 1, 8, 3, 4, 64, 64, 1, None)) == "LRC_ERR_SHAPE"   # Hv % Hk
    assert _st(L, f(*ok_args, 1, 8, 2, 4, 48, 64, 1, None)) == "LRC_ERR_SHAPE"   # dk
    assert _st(L, f(*ok_args, 1, 8, 2, 4, 64, 256, 1, None)) == "LRC_ERR_SHAPE"  # dv
    assert _st(L, f(*ok_args, 1, 8, 2, 4, 64, 64, 5, None)) == "LRC_ERR_DTYPE"
    assert _st(L, f(*ok_args, 1, 8, 2, 4, 64, 256, L.BF16_SPLIT, None)) == "LRC_ERR_SHAPE"  # split is a K3 dtype
    bad = list(ok_args)
    bad[5] = A0  # o aliases q
    assert _st(L, f(*bad, 1, 8, 2, 4, 64, 64, 1, None)) == "LRC_ERR_ALIAS"
    lens = (ctypes.c_int * 2)(70, -3)
    assert _st(L, L.lib.lrc_gdn_prefill(A0, A1, A2, A3, A4, A5, A6, lens, 2, 2, 4, 64, 64, 1, None)) == "LRC_ERR_ROWS"


def test_inverse_rejects(L):
    f = L.lib.lrc_unit_lower_inverse
    assert _st(L, f(A0, A1, 4, 65, None)) == "LRC_ERR_ROWS"
    assert _st(L, f(A0, A0, 4, 8, None)) == "LRC_ERR_ALIAS"
    assert _st(L, f(None, A1, 4, 8, None)) == "LRC_ERR_NULL"
    assert _st(L, f(A0, A1, -1, 8, None)) == "LRC_ERR_SHAPE"


def test_time_shift_rejects(L):
    f = L.lib.lrc_time_shift_rows
    assert _st(L, f(A0, A1, A2, A3, A4, 1, 65, 16, 3, None)) == "LRC_ERR_ROWS"
    assert _st(L, f(A0, A1, A2, A3, A4, 1, 8, 16, 0, None)) == "LRC_ERR_SHAPE"   # no mixed input
    assert _st(L, f(A0, A1, A2, A3, A4, 1, 8, 16, 9, None)) == "LRC_ERR_SHAPE"   # more than LRC_MAX_MIX
    assert _st(L, f(A0, A1, A2, A3, A4, 1, 8, 0, 3, None)) == "LRC_ERR_SHAPE"
    assert _st(L, f(A0, A0, A2, A3, A4, 1, 8, 16, 3, None)) == "LRC_ERR_ALIAS"   # out over x
    assert _st(L, f(A0, A1, A2, A2 + 16, A4, 1, 8, 16, 3, None)) == "LRC_ERR_ALIAS"
    assert _st(L, f(A0, A1, None, A3, A4, 1, 8, 16, 3, None)) == "LRC_ERR_NULL"
    assert _st(L, f(A0, MIS, A2, A3, A4, 1, 8, 16, 3, None)) == "LRC_ERR_ALIGN"
    lens = (ctypes.c_int * 2)(70, -1)
    assert _st(L, L.lib.lrc_time_shift_prefill(A0, A1, A2, A3, lens, 2, 16, 3, None)) == "LRC_ERR_ROWS"


def test_mamba_mixer_rejects(L):
    f = L.lib.lrc_mamba_mixer_rows
    ok_args = [A0, A1, A2, A3, A4, A5, A6, A7, A7 + 0x4000000]
    assert _st(L, f(*ok_args, 1, 65, 64, 16, None)) == "LRC_ERR_ROWS"
    assert _st(L, f(*ok_args, 1, 8, 64, 12, None)) == "LRC_ERR_SHAPE"   # d_state not a supported size
    assert _st(L, f(*ok_args, 1, 8, 64, 128, None)) == "LRC_ERR_SHAPE"
    assert _st(L, f(*ok_args, 1, 8, 0, 16, None)) == "LRC_ERR_SHAPE"
    bad = list(ok_args)
    bad[6] = A0  # y over x
    assert _st(L, f(*bad, 1, 8, 64, 16, None)) == "LRC_ERR_ALIAS"
    bad = list(ok_args)
    bad[8] = bad[7] + 16  # h_out partly over h_in
    assert _st(L, f(*bad, 1, 8, 64, 16, None)) == "LRC_ERR_ALIAS"
    bad = list(ok_args)
    bad[2] = None  # A
    assert _st(L, f(*bad, 1, 8, 64, 16, None)) == "LRC_ERR_NULL"
    lens = (ctypes.c_int * 1)(5)
    assert _st(L, L.lib.lrc_mamba_mixer_prefill(A0, A1, A2, A3, A4, A5, A6, A7, lens, 0, 64, 16, None)) \
        == "LRC_ERR_SHAPE"


def test_binding_refuses_cpu_tensors(L):
    import torch

    a = torch.zeros(1, 4, 2, 2)
    with pytest.raises(ValueError):
        L.scan_rows(a, a.clone(), a.clone(), torch.zeros(1, 2, 2), torch.zeros(1, 2, 2))


def test_package_import_does_not_load_the_library():
    import subprocess
    import sys

    code = ("import sys; import linear_recurrence_chunked_amd, linear_recurrence_chunked_amd.inputs;"
            "print('linear_recurrence_chunked_amd.lrc' in sys.modules)")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, check=True)
    assert out.stdout.strip() == "False"
