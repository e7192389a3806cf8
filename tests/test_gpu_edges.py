"""GPU edge cases against the float64 oracle: the largest prefill-driver call
(256 prompts, lengths 0..130 with empty prompts among them) for every kernel,
a driver call whose prompts are all empty, chunk calls with a large uniform
batch, and the conv widths the other tests do not reach.

Sources: the pages' chunks are 1..64 rows with the state carried between
chunks ("perf(rwkv): ...", "perf(mamba): ...", "perf(qwen3_5): ...",
Implementation); the 256-prompt bound and the packed layout are this
library's (include/lrc.h).
"""
import numpy as np
import pytest
import torch

from gpu_util import f64, require_gpu, to_dev
from helpers import TOL_BF16, TOL_F32, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    require_gpu()
    from linear_recurrence_chunked_amd import lrc

    return lrc


@pytest.fixture(scope="module")
def lens():
    rng = np.random.default_rng(300)
    ls = rng.integers(0, 131, size=256)
    ls[[3, 100, 255]] = 0
    ls[7] = 64
    ls[8] = 65
    return [int(n) for n in ls]


def _offs(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(int)


def test_conv_256_prompts(L, orc, lens):
    rng = np.random.default_rng(301)
    R, P, C, K = sum(lens), len(lens), 24, 4
    x = torch.from_numpy(rng.standard_normal((R, C))).float()
    s0 = torch.from_numpy(rng.standard_normal((P, K - 1, C))).float()
    w = torch.from_numpy(rng.normal(0, 0.5, (C, K))).float()
    tx, ts = to_dev(x), to_dev(s0)
    y = torch.empty_like(tx)
    L.conv_prefill(tx, y, ts, to_dev(w), lens)
    torch.cuda.synchronize()
    o = _offs(lens)
    for p in range(P):
        ry, rs = orc.conv_rows(f64(x[o[p]:o[p + 1]]), f64(s0[p]), f64(w))
        if lens[p]:
            assert rel_err(f64(y[o[p]:o[p + 1]]), ry) < TOL_F32
        assert np.array_equal(f64(ts[p]), rs)


def test_scan_256_prompts(L, orc, lens):
    rng = np.random.default_rng(302)
    R, P, D, N = sum(lens), len(lens), 8, 4
    a = torch.from_numpy(np.exp(-rng.uniform(0.01, 1.0, (R, D, N)))).float()
    b = torch.from_numpy(rng.standard_normal((R, D, N))).float()
    h0 = torch.from_numpy(rng.standard_normal((P, D, N))).float()
    ta, tb, ts = to_dev(a), to_dev(b), to_dev(h0)
    h = torch.empty_like(ta)
    L.scan_prefill(ta, tb, h, ts, lens)
    torch.cuda.synchronize()
    o = _offs(lens)
    for p in range(P):
        sl = slice(o[p], o[p + 1])
        rh, rs = orc.scan(f64(a[sl]).reshape(lens[p], D * N), f64(b[sl]).reshape(lens[p], D * N),
                          f64(h0[p]).reshape(D * N))
        if lens[p]:
            assert rel_err(f64(h[sl]).reshape(lens[p], D * N), rh) < TOL_F32
        assert rel_err(f64(ts[p]).reshape(-1), rs) < TOL_F32


def test_wkv_256_prompts(L, orc, lens):
    from linear_recurrence_chunked_amd import inputs

    R, P, C = sum(lens), len(lens), 70
    d = inputs.rwkv_169m(rows=R, channels=C, seed=303)
    k, v, w, u = (to_dev(d[n]) for n in ("k", "v", "w", "u"))
    num, den = torch.zeros(P, C, device="cuda"), torch.zeros(P, C, device="cuda")
    mx = torch.full((P, C), -1e38, device="cuda")
    out = torch.empty_like(k)
    L.wkv4_prefill(k, v, w, u, out, num, den, mx, lens)
    torch.cuda.synchronize()
    o = _offs(lens)
    for p in range(P):
        sl = slice(o[p], o[p + 1])
        ro, rn, rd, rm = orc.wkv4(f64(d["k"][sl]), f64(d["v"][sl]), f64(d["w"]), f64(d["u"]), *orc.empty_wkv_state(C))
        if lens[p]:
            assert rel_err(f64(out[sl]), ro) < TOL_F32
            assert rel_err(f64(num[p] / den[p]), rn / rd) < TOL_F32
        else:
            assert torch.all(num[p] == 0) and torch.all(mx[p] == -1e38)


@pytest.mark.parametrize("dtype,tol", [(torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)])
def test_gated_deltanet_256_prompts(L, orc, lens, dtype, tol):
    from linear_recurrence_chunked_amd import inputs

    R, P = sum(lens), len(lens)
    d = inputs.gdn_small(rows=R, heads=2, key_heads=1, dk=32, dv=32, dtype=dtype, seed=304)
    q, k, v, beta, g = (to_dev(d[n]) for n in ("q", "k", "v", "beta", "g"))
    S0 = torch.from_numpy(np.random.default_rng(305).normal(0, 0.1, (P, 2, 32, 32))).float()
    st = to_dev(S0)
    o = torch.empty((R, 2, 32), device="cuda")
    L.gdn_prefill(q, k, v, beta, g, o, st, lens)
    torch.cuda.synchronize()
    off = _offs(lens)
    for p in range(P):
        sl = slice(off[p], off[p + 1])
        ro, rs = orc.gdn(*(f64(d[n][sl]) for n in ("q", "k", "v", "beta", "g")), f64(S0[p]))
        if lens[p]:
            assert rel_err(f64(o[sl]), ro) < tol
        assert rel_err(f64(st[p]), rs) < tol


def test_time_shift_and_mixer_256_prompts(L, orc, lens):
    from linear_recurrence_chunked_amd import inputs

    R, P = sum(lens), len(lens)
    t = inputs.rwkv_shift(rows=R, channels=20, mixes=3, seed=306)
    st0 = torch.from_numpy(np.random.default_rng(307).standard_normal((P, 20))).float()
    tst = to_dev(st0)
    tout = torch.empty((3, R, 20), device="cuda")
    L.time_shift_prefill(to_dev(t["x"]), tout, tst, to_dev(t["mix"]), lens)
    m = inputs.mamba_mixer_tiny(rows=R, d_inner=40, d_state=16, seed=308)
    h0 = torch.from_numpy(np.random.default_rng(309).standard_normal((P, 40, 16))).float()
    mh = to_dev(h0)
    my = torch.empty((R, 40), device="cuda")
    L.mamba_mixer_prefill(*(to_dev(m[n]) for n in ("x", "dt", "A", "B", "C", "D")), my, mh, lens)
    torch.cuda.synchronize()
    o = _offs(lens)
    for p in range(P):
        sl = slice(o[p], o[p + 1])
        ro, rs = orc.time_shift(f64(t["x"][sl]), f64(st0[p]), f64(t["mix"]))
        ry, rh = orc.mamba_mixer(f64(m["x"][sl]), f64(m["dt"][sl]), f64(m["A"]), f64(m["B"][sl]), f64(m["C"][sl]),
                                 f64(m["D"]), f64(h0[p]))
        if lens[p]:
            assert rel_err(f64(tout[:, sl]), ro) < TOL_F32
            assert rel_err(f64(my[sl]), ry) < TOL_F32
        assert np.array_equal(f64(tst[p]), rs)
        assert rel_err(f64(mh[p]), rh) < TOL_F32


def test_all_prompts_empty_leave_states(L):
    lens = [0] * 5
    st = torch.randn(5, 3, 16, device="cuda")
    before = st.clone()
    x = torch.empty(0, 16, device="cuda")
    L.conv_prefill(x, torch.empty_like(x), st, torch.randn(16, 4, device="cuda"), lens)
    S = torch.randn(5, 2, 32, 32, device="cuda")
    S_before = S.clone()
    q = torch.empty(0, 1, 32, device="cuda")
    L.gdn_prefill(q, q.clone(), torch.empty(0, 2, 32, device="cuda"), torch.empty(0, 2, device="cuda"),
                  torch.empty(0, 2, device="cuda"), torch.empty(0, 2, 32, device="cuda"), S, lens)
    torch.cuda.synchronize()
    assert torch.equal(st, before) and torch.equal(S, S_before)


def test_large_uniform_chunk_batch(L, orc):
    """A chunk call over 300 prompts of 64 rows each (the rows entry points take up to 65535)."""
    from linear_recurrence_chunked_amd import inputs

    B, S, C = 300, 64, 16
    d = inputs.rwkv_169m(rows=B * S, channels=C, seed=310)
    k, v = to_dev(d["k"]).view(B, S, C), to_dev(d["v"]).view(B, S, C)
    num, den = torch.zeros(B, C, device="cuda"), torch.zeros(B, C, device="cuda")
    mx = torch.full((B, C), -1e38, device="cuda")
    out = torch.empty_like(k)
    L.wkv4_rows(k, v, to_dev(d["w"]), to_dev(d["u"]), out, num, den, mx)
    torch.cuda.synchronize()
    for b in (0, 151, 299):
        sl = slice(b * S, (b + 1) * S)
        ro, *_ = orc.wkv4(f64(d["k"][sl]), f64(d["v"][sl]), f64(d["w"]), f64(d["u"]), *orc.empty_wkv_state(C))
        assert rel_err(f64(out[b]), ro) < TOL_F32


@pytest.mark.parametrize("K", [5, 6, 7])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_conv_remaining_widths(L, orc, K, dtype):
    rng = np.random.default_rng(320 + K)
    lens = [75, 2, 64]
    R, P, C = sum(lens), len(lens), 48
    x = torch.from_numpy(rng.standard_normal((R, C))).to(dtype)
    s0 = torch.from_numpy(rng.standard_normal((P, K - 1, C))).to(dtype)
    w = torch.from_numpy(rng.normal(0, 0.5, (C, K))).float()
    tx, ts = to_dev(x), to_dev(s0)
    y = torch.empty_like(tx)
    L.conv_prefill(tx, y, ts, to_dev(w), lens)
    torch.cuda.synchronize()
    tol = TOL_F32 if dtype == torch.float32 else TOL_BF16
    o = _offs(lens)
    for p in range(P):
        ry, rs = orc.conv_rows(f64(x[o[p]:o[p + 1]]), f64(s0[p]), f64(w))
        assert rel_err(f64(y[o[p]:o[p + 1]]), ry) < tol
        assert np.array_equal(f64(ts[p]), rs)
