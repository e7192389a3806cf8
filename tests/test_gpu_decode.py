"""Decode continuity on the GPU: a prompt prefilled through the chunk driver,
then one-row steps (S = 1) of the same kernels on the same state buffers,
checked against the float64 oracle's token loop over all rows.

Source: "perf(rwkv): prefill text prompts in multi-token chunks", Tests (a
prefill of 64 + 11 rows followed by three decode steps on the one-token path,
compared with token-by-token steps); "perf(qwen3_5): prefill text prompts in
multi-token chunks", Implementation (the prefill advances the same recurrent
state the decoder then reads).  Here the one-row step is the same entry point
called with one row, as a decoder would call it, with the state updated in
place.
"""
import numpy as np
import pytest
import torch

from gpu_util import f64, require_gpu, to_dev
from helpers import TOL_BF16, TOL_F32, rel_err

pytestmark = pytest.mark.gpu

PROMPT, STEPS = 75, 3


@pytest.fixture(scope="module")
def L():
    require_gpu()
    from linear_recurrence_chunked_amd import lrc

    return lrc


def test_conv_prefill_then_decode(L, orc):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.mamba_tiny(rows=PROMPT + STEPS)
    x, st0, w = to_dev(d["conv_x"]), to_dev(d["conv_state"]), to_dev(d["conv_w"])
    C = x.shape[1]
    y = torch.empty_like(x)
    st = st0.clone().unsqueeze(0)
    L.conv_prefill(x[:PROMPT], y[:PROMPT], st, w, [PROMPT])
    for t in range(PROMPT, PROMPT + STEPS):
        yt = torch.empty((1, 1, C), device=x.device)
        L.conv_rows(x[t:t + 1][None].contiguous(), yt, st, st, w)
        y[t] = yt[0, 0]
    torch.cuda.synchronize()
    ry, rs = orc.conv_rows(f64(d["conv_x"]), f64(d["conv_state"]), f64(d["conv_w"]))
    assert rel_err(f64(y), ry) < TOL_F32
    assert np.array_equal(f64(st[0]), rs)


def test_scan_prefill_then_decode(L, orc):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.mamba_tiny(rows=PROMPT + STEPS)
    a, b, h0 = to_dev(d["a"]), to_dev(d["b"]), to_dev(d["h0"])
    R, E = a.shape
    D, N = 64, E // 64
    h = torch.empty_like(a)
    st = h0.clone().view(1, D, N)
    L.scan_prefill(a[:PROMPT].view(PROMPT, D, N), b[:PROMPT].view(PROMPT, D, N), h[:PROMPT].view(PROMPT, D, N),
                   st, [PROMPT])
    for t in range(PROMPT, R):
        ht = torch.empty((1, 1, D, N), device=a.device)
        L.scan_rows(a[t].view(1, 1, D, N).contiguous(), b[t].view(1, 1, D, N).contiguous(), ht, st, st)
        h[t] = ht.view(E)
    torch.cuda.synchronize()
    rh, rs = orc.scan(f64(d["a"]), f64(d["b"]), f64(d["h0"]))
    assert rel_err(f64(h), rh) < TOL_F32
    assert rel_err(f64(st.reshape(E)), rs) < TOL_F32


def test_wkv_prefill_then_decode(L, orc):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.rwkv_169m(rows=PROMPT + STEPS, channels=1000)
    k, v, w, u = (to_dev(d[n]) for n in ("k", "v", "w", "u"))
    R, C = k.shape
    _, n0, d0, m0 = orc.wkv4(f64(d["warm_k"]), f64(d["warm_v"]), f64(d["w"]), f64(d["u"]), *orc.empty_wkv_state(C))
    num, den, mx = (torch.from_numpy(a).float().to("cuda").unsqueeze(0).contiguous() for a in (n0, d0, m0))
    out = torch.empty_like(k)
    L.wkv4_prefill(k[:PROMPT], v[:PROMPT], w, u, out[:PROMPT], num, den, mx, [PROMPT])
    for t in range(PROMPT, R):
        ot = torch.empty((1, 1, C), device=k.device)
        L.wkv4_rows(k[t:t + 1][None].contiguous(), v[t:t + 1][None].contiguous(), w, u, ot, num, den, mx)
        out[t] = ot[0, 0]
    torch.cuda.synchronize()
    ro, rn, rd, rm = orc.wkv4(f64(d["k"]), f64(d["v"]), f64(d["w"]), f64(d["u"]),
                              n0.astype(np.float32).astype(np.float64), d0.astype(np.float32).astype(np.float64),
                              m0.astype(np.float32).astype(np.float64))
    assert rel_err(f64(out), ro) < TOL_F32
    gn, gd, gm = f64(num[0]), f64(den[0]), f64(mx[0])
    f = np.exp(gm - rm)
    assert rel_err(gn / gd, rn / rd) < TOL_F32
    assert rel_err(gn * f, rn) < TOL_F32 and rel_err(gd * f, rd) < TOL_F32


@pytest.mark.parametrize("dtype,tol", [(torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)])
def test_gated_deltanet_prefill_then_decode(L, orc, dtype, tol):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.gdn_small(rows=PROMPT + STEPS, dtype=dtype)
    q, k, v, beta, g, S0 = (to_dev(d[n]) for n in ("q", "k", "v", "beta", "g", "S0"))
    R, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    o = torch.empty((R, Hv, dv), device=q.device)
    st = S0.clone().unsqueeze(0)
    L.gdn_prefill(q[:PROMPT], k[:PROMPT], v[:PROMPT], beta[:PROMPT], g[:PROMPT], o[:PROMPT], st, [PROMPT])
    for t in range(PROMPT, R):
        ot = torch.empty((1, 1, Hv, dv), device=q.device)
        sl = slice(t, t + 1)
        L.gdn_chunk(q[sl][None].contiguous(), k[sl][None].contiguous(), v[sl][None].contiguous(),
                    beta[sl][None].contiguous(), g[sl][None].contiguous(), ot, st, st)
        o[t] = ot[0, 0]
    torch.cuda.synchronize()
    ro, rs = orc.gdn(*(f64(d[n]) for n in ("q", "k", "v", "beta", "g", "S0")))
    assert rel_err(f64(o), ro) < tol
    assert rel_err(f64(st[0]), rs) < tol
