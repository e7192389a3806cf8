"""GPU parity of the next rows -- the RWKV-4 time shift and the fused Mamba
mixer rows -- against the float64 oracle.

Time shift: "perf(rwkv): prefill text prompts in multi-token chunks",
Implementation (each row mixed with the row before it, the first row with
the carried shift state).  Mixer rows: "perf(mamba): prefill text prompts in multi-token
chunks", Implementation (the scan between forming a, b and reading h out),
read as a = exp(dt A), b = dt B x, y = C.h + D x.

Cases: 169M-like widths chunked 64 + 64 and 11 + 64 + 53; ragged packed
prompts (including empty ones and a channel count that is not a multiple of
4 or of a workgroup); every supported d_state; a prefill followed by one-row
decode steps on the same state; the batched mixed workload at model width
(Mamba 5120 x 16, RWKV 2560 with three mixed inputs), sampled channels of
every prompt.  Tolerance: rel 1e-4 of each tensor's max-abs scale (FP32);
the time shift's new state is a copy and must match exactly.
"""
import numpy as np
import pytest
import torch

from gpu_util import chunks, f64, require_gpu, to_dev
from helpers import TOL_F32, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    require_gpu()
    from linear_recurrence_chunked_amd import lrc

    return lrc


# ----------------------------------------------------------------- time shift
@pytest.mark.parametrize("splits", [[64, 64], [11, 64, 53], [1] * 20 + [64, 44]])
def test_time_shift_169m_chunked(L, orc, splits):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.rwkv_shift()
    x, st0, mix = to_dev(d["x"]), to_dev(d["state"]), to_dev(d["mix"])
    R, C = x.shape
    M = mix.shape[0]
    out = torch.empty((M, R, C), device=x.device)
    st = st0.clone().unsqueeze(0)
    for r, n in chunks(R, splits):
        o = torch.empty((M, 1, n, C), device=x.device)
        L.time_shift_rows(x[r:r + n][None].contiguous(), o, st, st, mix)
        out[:, r:r + n] = o[:, 0]
    torch.cuda.synchronize()
    ro, rs = orc.time_shift(f64(d["x"]), f64(d["state"]), f64(d["mix"]))
    assert rel_err(f64(out), ro) < TOL_F32
    assert np.array_equal(f64(st[0]), rs)


@pytest.mark.parametrize("C", [300, 2560, 37])
def test_time_shift_prefill_ragged(L, orc, C):
    from linear_recurrence_chunked_amd import inputs

    lens = [128, 1, 0, 75, 64, 200]
    d = inputs.rwkv_shift(rows=sum(lens), channels=C, mixes=2, seed=11)
    x, mix = to_dev(d["x"]), to_dev(d["mix"])
    P = len(lens)
    state0 = torch.randn((P, C), generator=torch.Generator().manual_seed(3))
    st = to_dev(state0)
    out = torch.full((2, sum(lens), C), float("nan"), device=x.device)
    L.time_shift_prefill(x, out, st, mix, lens)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    for p in range(P):
        sl = slice(offs[p], offs[p + 1])
        ro, rs = orc.time_shift(f64(d["x"][sl]), f64(state0[p]), f64(d["mix"]))
        if lens[p]:
            assert rel_err(f64(out[:, sl]), ro) < TOL_F32
        assert np.array_equal(f64(st[p]), rs)


def test_time_shift_one_hot_mixes_exact(L):
    x = torch.randn(70, 64, device="cuda")
    st0 = torch.randn(1, 64, device="cuda")
    mix = torch.stack([torch.ones(64), torch.zeros(64)]).cuda()
    out = torch.empty(2, 70, 64, device="cuda")
    st = st0.clone()
    L.time_shift_prefill(x, out, st, mix, [70])
    torch.cuda.synchronize()
    assert torch.equal(out[0], x)
    assert torch.equal(out[1], torch.cat([st0, x[:-1]]))
    assert torch.equal(st[0], x[-1])


# ---------------------------------------------------------------- mixer rows
def _mixer_dev(d):
    return [to_dev(d[n]) for n in ("x", "dt", "A", "B", "C", "D", "h0")]


def _mixer_oracle(orc, d, h0=None):
    return orc.mamba_mixer(*(f64(d[n]) for n in ("x", "dt", "A", "B", "C", "D")),
                           f64(d["h0"]) if h0 is None else h0)


@pytest.mark.parametrize("splits", [[64, 11], [7, 4, 64], [1] * 11 + [64]])
def test_mixer_tiny_chunked(L, orc, splits):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.mamba_mixer_tiny()
    x, dt, A, B, C, D, h0 = _mixer_dev(d)
    R, Dm = x.shape
    y = torch.empty_like(x)
    h = h0.clone().unsqueeze(0)
    for r, n in chunks(R, splits):
        sl = slice(r, r + n)
        yc = torch.empty((1, n, Dm), device=x.device)
        L.mamba_mixer_rows(x[sl][None].contiguous(), dt[sl][None].contiguous(), A, B[sl][None].contiguous(),
                           C[sl][None].contiguous(), D, yc, h, h)
        y[sl] = yc[0]
    torch.cuda.synchronize()
    ry, rh = _mixer_oracle(orc, d)
    assert rel_err(f64(y), ry) < TOL_F32
    assert rel_err(f64(h[0]), rh) < TOL_F32


@pytest.mark.parametrize("N", [2, 4, 8, 16, 32, 64])
def test_mixer_prefill_ragged_every_state_size(L, orc, N):
    from linear_recurrence_chunked_amd import inputs

    lens = [130, 1, 0, 64, 75]
    d = inputs.mamba_mixer_tiny(rows=sum(lens), d_inner=200, d_state=N, seed=40 + N)
    x, dt, A, B, C, D, _ = _mixer_dev(d)
    P = len(lens)
    h0 = torch.randn((P, 200, N), generator=torch.Generator().manual_seed(N))
    st = to_dev(h0)
    y = torch.full_like(x, float("nan"))
    L.mamba_mixer_prefill(x, dt, A, B, C, D, y, st, lens)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    for p in range(P):
        sl = slice(offs[p], offs[p + 1])
        ry, rh = orc.mamba_mixer(f64(d["x"][sl]), f64(d["dt"][sl]), f64(d["A"]), f64(d["B"][sl]),
                                 f64(d["C"][sl]), f64(d["D"]), f64(h0[p]))
        if lens[p]:
            assert rel_err(f64(y[sl]), ry) < TOL_F32
        assert rel_err(f64(st[p]), rh) < TOL_F32


def test_mixer_prefill_then_decode(L, orc):
    from linear_recurrence_chunked_amd import inputs

    prompt, steps = 75, 3
    d = inputs.mamba_mixer_tiny(rows=prompt + steps)
    x, dt, A, B, C, D, h0 = _mixer_dev(d)
    R, Dm = x.shape
    y = torch.empty_like(x)
    h = h0.clone().unsqueeze(0)
    L.mamba_mixer_prefill(x[:prompt], dt[:prompt], A, B[:prompt], C[:prompt], D, y[:prompt], h, [prompt])
    for t in range(prompt, R):
        sl = slice(t, t + 1)
        yt = torch.empty((1, 1, Dm), device=x.device)
        L.mamba_mixer_rows(x[sl][None].contiguous(), dt[sl][None].contiguous(), A, B[sl][None].contiguous(),
                           C[sl][None].contiguous(), D, yt, h, h)
        y[t] = yt[0, 0]
    torch.cuda.synchronize()
    ry, rh = _mixer_oracle(orc, d)
    assert rel_err(f64(y), ry) < TOL_F32
    assert rel_err(f64(h[0]), rh) < TOL_F32


# ----------------------------------------------------- batched mixed, full size
def test_mixer_mixed_workload_sampled(L, orc):
    from linear_recurrence_chunked_amd import inputs

    lens = inputs.mixed_lengths()
    d = inputs.mixed_mamba_mixer(lens, torch.device("cuda:0"))
    y = torch.empty_like(d["x"])
    st = d["h0"].clone()
    L.mamba_mixer_prefill(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], y, st, lens)
    torch.cuda.synchronize()
    sel = torch.arange(3, d["x"].shape[1], 97, device="cuda")
    x, dt, yy = f64(d["x"][:, sel]), f64(d["dt"][:, sel]), f64(y[:, sel])
    A, Dv = f64(d["A"][sel]), f64(d["D"][sel])
    B, C = f64(d["B"]), f64(d["C"])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    for p in range(len(lens)):
        sl = slice(offs[p], offs[p + 1])
        ry, rh = orc.mamba_mixer(x[sl], dt[sl], A, B[sl], C[sl], Dv, np.zeros((len(sel), A.shape[1])))
        assert rel_err(yy[sl], ry) < TOL_F32
        assert rel_err(f64(st[p][sel]), rh) < TOL_F32


def test_time_shift_mixed_workload_sampled(L, orc):
    from linear_recurrence_chunked_amd import inputs

    lens = inputs.mixed_lengths()
    d = inputs.mixed_time_shift(lens, torch.device("cuda:0"))
    R, C = d["x"].shape
    M = d["mix"].shape[0]
    out = torch.empty((M, R, C), device="cuda")
    st = d["state"].clone()
    L.time_shift_prefill(d["x"], out, st, d["mix"], lens)
    torch.cuda.synchronize()
    sel = torch.arange(1, C, 13, device="cuda")
    x, mix, o = f64(d["x"][:, sel]), f64(d["mix"][:, sel]), f64(out[:, :, sel])
    offs = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    for p in range(len(lens)):
        sl = slice(offs[p], offs[p + 1])
        ro, rs = orc.time_shift(x[sl], np.zeros(len(sel)), mix)
        assert rel_err(o[:, sl], ro) < TOL_F32
        assert np.array_equal(f64(st[p][sel]), rs)
