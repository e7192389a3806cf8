"""GPU parity at full size: the batched mixed prefill workload (16 prompts of
U{1..4096} rows, 30 654 rows in all), built and launched exactly as bench.py
times it, checked against the float64 oracle on sampled channels, state
elements and heads -- every prompt, every row of the sample, outputs and final
states.
"""
import numpy as np
import pytest
import torch

from gpu_util import f64, require_gpu
from helpers import TOL_BF16, TOL_F32, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def run():
    require_gpu()
    import bench
    from linear_recurrence_chunked_amd import lrc

    W = bench.make_workload(torch.device("cuda:0"))
    # keep the fresh states the oracle starts from
    fresh = {n: W[n].clone() for n in ("sm", "hs", "num", "den", "max", "sg", "S")}
    for k in bench.KERNELS:
        bench.run_kernel(lrc, W, k)
    torch.cuda.synchronize()
    offs = np.concatenate([[0], np.cumsum(W["lens"])]).astype(int)
    yield W, fresh, offs
    del W


def _prompts(W):
    return range(len(W["lens"]))


def test_mixed_conv_mamba(run, orc):
    W, fresh, offs = run
    sel = torch.arange(3, W["xm"].shape[1], 97, device="cuda")
    x, y, w = f64(W["xm"][:, sel]), f64(W["ym"][:, sel]), f64(W["wm"][sel])
    for p in _prompts(W):
        sl = slice(offs[p], offs[p + 1])
        ry, rs = orc.conv_rows(x[sl], f64(fresh["sm"][p][:, sel]), w)
        if W["lens"][p]:
            assert rel_err(y[sl], ry) < TOL_F32
        assert np.array_equal(f64(W["sm"][p][:, sel]), rs)


def test_mixed_scan(run, orc):
    W, fresh, offs = run
    R = W["R"]
    sel = torch.arange(5, W["a"].shape[1] * W["a"].shape[2], 257, device="cuda")
    a = f64(W["a"].view(R, -1)[:, sel])
    b = f64(W["b"].view(R, -1)[:, sel])
    h = f64(W["h"].view(R, -1)[:, sel])
    for p in _prompts(W):
        sl = slice(offs[p], offs[p + 1])
        rh, rs = orc.scan(a[sl], b[sl], f64(fresh["hs"][p].reshape(-1)[sel]))
        assert rel_err(h[sl], rh) < TOL_F32
        assert rel_err(f64(W["hs"][p].reshape(-1)[sel]), rs) < TOL_F32


def test_mixed_wkv(run, orc):
    W, fresh, offs = run
    sel = torch.arange(1, W["k"].shape[1], 13, device="cuda")
    k, v, out = f64(W["k"][:, sel]), f64(W["v"][:, sel]), f64(W["wkv"][:, sel])
    w, u = f64(W["w"][sel]), f64(W["u"][sel])
    for p in _prompts(W):
        sl = slice(offs[p], offs[p + 1])
        st0 = [f64(fresh[n][p][sel]) for n in ("num", "den", "max")]
        ro, rn, rd, rm = orc.wkv4(k[sl], v[sl], w, u, *st0)
        assert rel_err(out[sl], ro) < TOL_F32
        num, den, mx = (f64(W[n][p][sel]) for n in ("num", "den", "max"))
        f = np.exp(mx - rm)
        assert rel_err(num / den, rn / rd) < TOL_F32
        assert rel_err(num * f, rn) < TOL_F32 and rel_err(den * f, rd) < TOL_F32


def test_mixed_conv_deltanet_bf16(run, orc):
    W, fresh, offs = run
    sel = torch.arange(7, W["xg"].shape[1], 61, device="cuda")
    x, y, w = f64(W["xg"][:, sel]), f64(W["yg"][:, sel]), f64(W["wg"][sel])
    for p in _prompts(W):
        sl = slice(offs[p], offs[p + 1])
        ry, rs = orc.conv_rows(x[sl], f64(fresh["sg"][p][:, sel]), w)
        if W["lens"][p]:
            assert rel_err(y[sl], ry) < TOL_BF16
        assert np.array_equal(f64(W["sg"][p][:, sel]), rs)


@pytest.mark.parametrize("key_head", [0, 7, 15])
def test_mixed_gated_deltanet(run, orc, key_head):
    W, fresh, offs = run
    Hv, Hk = W["gv"].shape[1], W["q"].shape[1]
    grp = Hv // Hk
    vh = list(range(key_head * grp, (key_head + 1) * grp))
    kh_t = torch.tensor([key_head], device="cuda")
    vh_t = torch.tensor(vh, device="cuda")
    q, k = f64(W["q"][:, kh_t]), f64(W["gk"][:, kh_t])
    v, be, g, o = f64(W["gv"][:, vh_t]), f64(W["beta"][:, vh_t]), f64(W["g"][:, vh_t]), f64(W["o"][:, vh_t])
    for p in _prompts(W):
        sl = slice(offs[p], offs[p + 1])
        ro, rs = orc.gdn(q[sl], k[sl], v[sl], be[sl], g[sl], f64(fresh["S"][p][vh_t]))
        assert np.all(np.isfinite(o[sl]))
        if W["lens"][p]:
            assert rel_err(o[sl], ro) < TOL_BF16
        assert rel_err(f64(W["S"][p][vh_t]), rs) < TOL_BF16
