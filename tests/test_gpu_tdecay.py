"""GPU parity of the WKV with a token-dependent decay against the float64 oracle.

Reading ("perf(rwkv): prefill text prompts in multi-token chunks", Notes For
Future Readers: RWKV generations with a per-token decay call for a different
chunk form): the RWKV-4 recurrence with a decay w_t per row and channel.
Workloads: the 169M-like RWKV-4 recipe with w_t = -exp(U(-6, 2)) drawn per
row and channel, 128 rows from a 32-row warm-up state run by the oracle; the
mixed prefill lengths at the RWKV-4 width of 2560 channels from fresh states;
ragged prompts at a channel count that is not a multiple of 64; decode steps.

The state triple is compared scale-free, as for RWKV-4: num / den, and num,
den rescaled to the oracle's max.
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


@pytest.fixture(scope="module")
def cfg(orc):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.rwkv_tdecay()
    C = d["k"].shape[1]
    _, n, de, m = orc.wkv_tdecay(f64(d["warm_k"]), f64(d["warm_v"]), f64(d["warm_w"]), f64(d["u"]),
                                 *orc.empty_wkv_state(C))
    d["num0"], d["den0"], d["max0"] = (torch.from_numpy(x).float() for x in (n, de, m))
    return d


def _check_state(num, den, mx, rn, rd, rm):
    num, den, mx = f64(num), f64(den), f64(mx)
    assert np.all(np.isfinite(num)) and np.all(np.isfinite(den)) and np.all(np.isfinite(mx))
    assert rel_err(num / den, rn / rd) < TOL_F32
    f = np.exp(mx - rm)
    assert rel_err(num * f, rn) < TOL_F32
    assert rel_err(den * f, rd) < TOL_F32


@pytest.mark.parametrize("splits", [[64, 64], [64, 1, 63], [1] * 128, [11, 64, 53]])
def test_tdecay_chunked_from_warm_state(L, orc, cfg, splits):
    d = cfg
    k, v, w, u = (to_dev(d[n]) for n in ("k", "v", "w", "u"))
    R, C = k.shape
    num, den, mx = (to_dev(d[n]).unsqueeze(0).clone() for n in ("num0", "den0", "max0"))
    out = torch.empty_like(k)
    for r, n in chunks(R, splits):
        o = torch.empty((1, n, C), device=k.device)
        L.wkv_tdecay_rows(*(t[r:r + n].unsqueeze(0).contiguous() for t in (k, v, w)), u, o, num, den, mx)
        out[r:r + n] = o[0]
    torch.cuda.synchronize()
    ref, rn, rd, rm = orc.wkv_tdecay(f64(d["k"]), f64(d["v"]), f64(d["w"]), f64(d["u"]),
                                     f64(d["num0"]), f64(d["den0"]), f64(d["max0"]))
    assert torch.isfinite(out).all()
    assert rel_err(f64(out), ref) < TOL_F32
    _check_state(num[0], den[0], mx[0], rn, rd, rm)


def test_tdecay_prefill_ragged_and_determinism(L, orc):
    from linear_recurrence_chunked_amd import inputs

    lens = [130, 1, 0, 75, 64, 65, 200]
    d = inputs.rwkv_tdecay(rows=sum(lens), channels=70, seed=11)
    k, v, w, u = (to_dev(d[n]) for n in ("k", "v", "w", "u"))
    P, C = len(lens), k.shape[1]
    results = []
    for _ in range(2):
        num, den = torch.zeros(P, C, device="cuda"), torch.zeros(P, C, device="cuda")
        mx = torch.full((P, C), -1e38, device="cuda")
        out = torch.empty_like(k)
        L.wkv_tdecay_prefill(k, v, w, u, out, num, den, mx, lens)
        torch.cuda.synchronize()
        results.append((out.clone(), num.clone(), den.clone(), mx.clone()))
    for a, b in zip(*results):
        assert torch.equal(a, b)  # run-to-run bitwise
    out, num, den, mx = results[0]
    o = np.concatenate([[0], np.cumsum(lens)])
    for p in range(P):
        sl = slice(o[p], o[p + 1])
        ro, rn, rd, rm = orc.wkv_tdecay(f64(d["k"][sl]), f64(d["v"][sl]), f64(d["w"][sl]), f64(d["u"]),
                                        *orc.empty_wkv_state(C))
        if lens[p]:
            assert rel_err(f64(out[sl]), ro) < TOL_F32
            _check_state(num[p], den[p], mx[p], rn, rd, rm)
        else:
            assert torch.all(num[p] == 0) and torch.all(mx[p] == -1e38)


def test_tdecay_constant_decay_matches_rwkv4(L, orc):
    """A decay equal on every row is the RWKV-4 recurrence."""
    from linear_recurrence_chunked_amd import inputs

    d = inputs.rwkv_169m(rows=150, channels=192, seed=12)
    k, v, wc, u = (to_dev(d[n]) for n in ("k", "v", "w", "u"))
    w = wc.unsqueeze(0).expand_as(k).contiguous()
    num, den = torch.zeros(1, 192, device="cuda"), torch.zeros(1, 192, device="cuda")
    mx = torch.full((1, 192), -1e38, device="cuda")
    out = torch.empty_like(k)
    L.wkv_tdecay_prefill(k, v, w, u, out, num, den, mx, [150])
    torch.cuda.synchronize()
    ro, rn, rd, rm = orc.wkv4(f64(d["k"]), f64(d["v"]), f64(d["w"]), f64(d["u"]), *orc.empty_wkv_state(192))
    assert rel_err(f64(out), ro) < TOL_F32
    _check_state(num[0], den[0], mx[0], rn, rd, rm)


def test_tdecay_huge_decay_and_extreme_keys(L, orc):
    rng = np.random.default_rng(140)
    R, C = 300, 128
    k = rng.normal(0, 3, (R, C))
    k[rng.random((R, C)) < 0.05] = 30.0
    k[rng.random((R, C)) < 0.05] = -30.0
    v = rng.standard_normal((R, C))
    w = -np.exp(rng.uniform(-6, 2, (R, C)))
    w[:, 0], w[:, 1] = -np.exp(2.0), -np.exp(-6.0)
    w[77, :] = -1e4  # forgets everything before row 77
    u = rng.uniform(-2, 2, C)
    tk, tv, tw, tu = (to_dev(torch.from_numpy(x).float()) for x in (k, v, w, u))
    num, den = torch.zeros(1, C, device="cuda"), torch.zeros(1, C, device="cuda")
    mx = torch.full((1, C), -1e38, device="cuda")
    out = torch.empty_like(tk)
    L.wkv_tdecay_prefill(tk, tv, tw, tu, out, num, den, mx, [R])
    torch.cuda.synchronize()
    ro, rn, rd, rm = orc.wkv_tdecay(f64(tk), f64(tv), f64(tw), f64(tu), *orc.empty_wkv_state(C))
    assert torch.isfinite(out).all()
    assert rel_err(f64(out), ro) < TOL_F32
    _check_state(num[0], den[0], mx[0], rn, rd, rm)


def test_tdecay_prefill_then_decode(L, orc):
    """Prefill a prompt, then three one-row steps on the same state buffers."""
    from linear_recurrence_chunked_amd import inputs

    d = inputs.rwkv_tdecay(rows=78, channels=256, seed=13)
    k, v, w, u = (to_dev(d[n]) for n in ("k", "v", "w", "u"))
    C = 256
    num, den = torch.zeros(1, C, device="cuda"), torch.zeros(1, C, device="cuda")
    mx = torch.full((1, C), -1e38, device="cuda")
    out = torch.empty_like(k)
    L.wkv_tdecay_prefill(k[:75].contiguous(), v[:75].contiguous(), w[:75].contiguous(), u, out[:75], num, den, mx,
                         [75])
    for t in range(75, 78):
        o = torch.empty((1, 1, C), device="cuda")
        L.wkv_tdecay_rows(*(x[t:t + 1].unsqueeze(0).contiguous() for x in (k, v, w)), u, o, num, den, mx)
        out[t] = o[0, 0]
    torch.cuda.synchronize()
    ro, rn, rd, rm = orc.wkv_tdecay(f64(d["k"]), f64(d["v"]), f64(d["w"]), f64(d["u"]), *orc.empty_wkv_state(C))
    assert rel_err(f64(out), ro) < TOL_F32
    _check_state(num[0], den[0], mx[0], rn, rd, rm)


def test_tdecay_mixed_prefill_full_size(L, orc):
    """The 16 mixed prompt lengths at 2560 channels; every 11th channel checked."""
    from linear_recurrence_chunked_amd import inputs

    lens = inputs.mixed_lengths()
    W = inputs.mixed_wkv_tdecay(lens, torch.device("cuda"))
    out = torch.empty_like(W["k"])
    L.wkv_tdecay_prefill(W["k"], W["v"], W["w"], W["u"], out, W["num"], W["den"], W["max"], lens)
    torch.cuda.synchronize()
    sel = torch.arange(3, W["k"].shape[1], 11, device="cuda")
    k, v, w, o = (f64(t[:, sel]) for t in (W["k"], W["v"], W["w"], out))
    u = f64(W["u"][sel])
    offs = np.concatenate([[0], np.cumsum(lens)])
    for p in range(len(lens)):
        sl = slice(offs[p], offs[p + 1])
        ro, rn, rd, rm = orc.wkv_tdecay(k[sl], v[sl], w[sl], u, *orc.empty_wkv_state(len(sel)))
        assert rel_err(o[sl], ro) < TOL_F32
        _check_state(W["num"][p][sel], W["den"][p][sel], W["max"][p][sel], rn, rd, rm)
