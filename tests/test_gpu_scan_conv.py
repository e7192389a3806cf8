"""GPU parity of K0 (short conv) and K1 (selective scan) against the float64 oracle.

Workloads: Mamba tiny (d_inner 64, d_state 16, one 75-row prompt as 64 + 11,
fp32, conv width 4) and the 9B-like DeltaNet short conv (8192 bf16 channels,
2048 rows), plus ragged batches, one-row chunks, empty chunks, chunks shorter
than the conv window and ragged channel counts.  Tolerance: max-abs error
relative to the tensor's max-abs value, 1e-4 for fp32 and 2e-2 for bf16.
"""
import numpy as np
import pytest
import torch

from gpu_util import chunks, f64, require_gpu, to_dev
from helpers import TOL_BF16, TOL_F32, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    require_gpu()
    from linear_recurrence_chunked_amd import lrc

    return lrc


@pytest.fixture(scope="module")
def tiny():
    from linear_recurrence_chunked_amd import inputs

    return inputs.mamba_tiny()


# ------------------------------------------------------------------ scan
def _scan_chunked(L, a, b, h0, D, N, splits):
    R = a.shape[0]
    h = torch.empty_like(a)
    st = h0.clone().view(1, D, N)
    for r, n in chunks(R, splits):
        out = torch.empty((1, n, D, N), device=a.device)
        L.scan_rows(a[r:r + n].reshape(1, n, D, N).contiguous(), b[r:r + n].reshape(1, n, D, N).contiguous(),
                    out, st, st)
        h[r:r + n] = out.view(n, D * N)
    torch.cuda.synchronize()
    return h, st.view(-1)


@pytest.mark.parametrize("splits", [[64, 11], [1] * 75, [32, 32, 11], [75 - 64, 64], [0, 64, 0, 11]])
def test_scan_mamba_tiny_chunked(L, orc, tiny, splits):
    a, b, h0 = to_dev(tiny["a"]), to_dev(tiny["b"]), to_dev(tiny["h0"])
    ref_h, ref_s = orc.scan(f64(tiny["a"]), f64(tiny["b"]), f64(tiny["h0"]))
    h, s = _scan_chunked(L, a, b, h0, 64, 16, splits)
    assert rel_err(f64(h), ref_h) < TOL_F32
    assert rel_err(f64(s), ref_s) < TOL_F32
    assert torch.isfinite(h).all()


def test_scan_mamba_tiny_prefill_and_determinism(L, orc, tiny):
    a, b, h0 = to_dev(tiny["a"]), to_dev(tiny["b"]), to_dev(tiny["h0"])
    ref_h, ref_s = orc.scan(f64(tiny["a"]), f64(tiny["b"]), f64(tiny["h0"]))
    outs = []
    for _ in range(2):
        h = torch.empty((75, 64, 16), device=a.device)
        st = h0.clone().view(1, 64, 16)
        L.scan_prefill(a.view(75, 64, 16), b.view(75, 64, 16), h, st, [75])
        torch.cuda.synchronize()
        outs.append((h.clone(), st.clone()))
    assert rel_err(f64(outs[0][0]).reshape(75, -1), ref_h) < TOL_F32
    assert rel_err(f64(outs[0][1]).reshape(-1), ref_s) < TOL_F32
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("D,N", [(5, 3), (7, 16), (64, 16), (2, 2)])
def test_scan_ragged_batch(L, orc, D, N):
    rng = np.random.default_rng(100 + D * N)
    lens = [1, 64, 65, 130, 0, 7, 200]
    R, E = sum(lens), D * N
    a = rng.uniform(0.2, 1.0, (R, E)).astype(np.float32)
    b = rng.standard_normal((R, E)).astype(np.float32)
    h0 = rng.standard_normal((len(lens), E)).astype(np.float32)
    ta, tb = to_dev(torch.from_numpy(a)), to_dev(torch.from_numpy(b))
    st = to_dev(torch.from_numpy(h0)).view(len(lens), D, N)
    h = torch.full((R, D, N), float("nan"), device=ta.device)
    L.scan_prefill(ta.view(R, D, N), tb.view(R, D, N), h, st, lens)
    torch.cuda.synchronize()
    r = 0
    for p, n in enumerate(lens):
        ref_h, ref_s = orc.scan(a[r:r + n].astype(np.float64), b[r:r + n].astype(np.float64), h0[p].astype(np.float64))
        if n:
            assert rel_err(f64(h[r:r + n]).reshape(n, E), ref_h) < TOL_F32
        assert rel_err(f64(st[p]).reshape(E), ref_s) < TOL_F32
        r += n


def test_scan_empty_chunk_copies_state(L):
    h0 = torch.randn(3, 4, 16, device="cuda")
    hS = torch.zeros_like(h0)
    a = torch.empty((3, 0, 4, 16), device="cuda")
    L.scan_rows(a, a.clone(), a.clone(), h0, hS)
    torch.cuda.synchronize()
    assert torch.equal(h0, hS)


def test_scan_rejects_65_rows_without_touching_state(L):
    a = torch.rand(1, 65, 4, 16, device="cuda")
    h0 = torch.randn(1, 4, 16, device="cuda")
    keep = h0.clone()
    with pytest.raises(L.LrcError) as ei:
        L.scan_rows(a, a.clone(), torch.empty_like(a), h0, h0)
    assert ei.value.name == "LRC_ERR_ROWS"
    torch.cuda.synchronize()
    assert torch.equal(h0, keep)


# ------------------------------------------------------------------ conv
def _conv_chunked(L, x, st0, w, splits, bias=None):
    R, C = x.shape
    y = torch.empty_like(x)
    st = st0.clone().unsqueeze(0)
    for r, n in chunks(R, splits):
        out = torch.empty((1, n, C), device=x.device, dtype=x.dtype)
        L.conv_rows(x[r:r + n].unsqueeze(0).contiguous(), out, st, st, w, bias)
        y[r:r + n] = out[0]
    torch.cuda.synchronize()
    return y, st[0]


@pytest.mark.parametrize("zero_state", [False, True])
@pytest.mark.parametrize("splits", [[64, 11], [1] * 75, [2, 1, 64, 8], [11, 64]])
def test_conv_mamba_tiny(L, orc, splits, zero_state):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.mamba_tiny(zero_conv_state=zero_state)
    x, st, w = to_dev(d["conv_x"]), to_dev(d["conv_state"]), to_dev(d["conv_w"])
    ref_y, ref_s = orc.conv_rows(f64(d["conv_x"]), f64(d["conv_state"]), f64(d["conv_w"]))
    y, s = _conv_chunked(L, x, st, w, splits)
    assert rel_err(f64(y), ref_y) < TOL_F32
    assert np.array_equal(f64(s), ref_s)  # the state is a copy of input rows
    yp = torch.empty_like(x)
    sp = st.clone()[None]
    L.conv_prefill(x, yp, sp, w, [x.shape[0]])
    torch.cuda.synchronize()
    assert torch.equal(yp, y) and torch.equal(sp[0], s)  # chunking changes no bit


def test_conv_bf16_deltanet_width(L, orc):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.gdn_9b()
    x, st, w = to_dev(d["conv_x"]), to_dev(d["conv_state"]), to_dev(d["conv_w"])
    R, C = x.shape
    y = torch.empty_like(x)
    s = st.clone().unsqueeze(0)
    L.conv_prefill(x, y, s, w, [R])
    torch.cuda.synchronize()
    ref_y, ref_s = orc.conv_rows(f64(d["conv_x"]), f64(d["conv_state"]), f64(d["conv_w"]))
    assert rel_err(f64(y), ref_y) < TOL_BF16
    assert np.array_equal(f64(s[0]), ref_s)
    # chunked at 64 gives the same bits as the whole prompt
    y2, s2 = _conv_chunked(L, x, st, w, [64] * (R // 64))
    assert torch.equal(y, y2) and torch.equal(s[0], s2)


@pytest.mark.parametrize("C,K,dtype", [(13, 4, torch.float32), (24, 1, torch.float32), (40, 8, torch.bfloat16),
                                       (16, 2, torch.bfloat16), (100, 3, torch.float32)])
def test_conv_ragged_prompts_short_chunks_and_bias(L, orc, C, K, dtype):
    rng = np.random.default_rng(200 + C + K)
    lens = [1, 2, 0, 64, 65, 33, 3]
    R, P = sum(lens), len(lens)
    x = torch.from_numpy(rng.standard_normal((R, C))).to(dtype)
    s0 = torch.from_numpy(rng.standard_normal((P, K - 1, C))).to(dtype)
    w = torch.from_numpy(rng.normal(0, 0.5, (C, K))).float()
    bias = torch.from_numpy(rng.standard_normal(C)).float()
    tx, ts, tw, tb = to_dev(x), to_dev(s0), to_dev(w), to_dev(bias)
    y = torch.empty_like(tx)
    L.conv_prefill(tx, y, ts, tw, lens, tb)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    r = 0
    for p, n in enumerate(lens):
        ref_y, ref_s = orc.conv_rows(f64(x[r:r + n]), f64(s0[p]), f64(w), f64(bias))
        if n:
            assert rel_err(f64(y[r:r + n]), ref_y) < tol
        assert np.array_equal(f64(ts[p]), ref_s)
        r += n


def test_conv_separate_state_buffers_and_empty_chunk(L):
    x = torch.randn(2, 0, 8, device="cuda")
    s_in = torch.randn(2, 3, 8, device="cuda")
    s_out = torch.zeros_like(s_in)
    w = torch.randn(8, 4, device="cuda")
    L.conv_rows(x, torch.empty_like(x), s_in, s_out, w)
    torch.cuda.synchronize()
    assert torch.equal(s_in, s_out)
