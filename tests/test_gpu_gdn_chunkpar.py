"""GPU parity of the chunk-parallel Gated DeltaNet form (lrc_gdn_prefill_ws) against the float64
oracle, at the bf16 tolerance.

Reading ("perf(qwen3_5): prefill text prompts in multi-token chunks", Implementation): a chunk's
U = T (diag(beta) V - diag(beta Gamma) K S_0) is the same product as U' - W S_0 with
U' = T diag(beta) V and W = T diag(beta Gamma) K, which need no state, so every chunk's A, T, W, U'
and masked decayed Q K^T can be formed at once and only the state products run chunk by chunk.
Workloads: the small one (75 rows as one prompt), the nearly parallel keys with beta = 0.99 (16, 32
and 64 keys), the 9B-like shape (32 value heads on 16 key heads, 128 x 128, 2048 rows, decays -1e-3
to -8 per row, the g = -8 head on its own), one 59-chunk prompt at both decay extremes, ragged
batches over every (dk, dv), and empty and one-row prompts.
"""
import numpy as np
import pytest
import torch

from gpu_util import f64, require_gpu, to_dev
from helpers import TOL_BF16, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    require_gpu()
    from linear_recurrence_chunked_amd import lrc

    return lrc


def _run(L, t, lens):
    q, k, v, beta, g = (to_dev(t[n]) for n in ("q", "k", "v", "beta", "g"))
    S0 = to_dev(t["S0"])
    R, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    st = S0.clone() if S0.dim() == 4 else S0.clone().unsqueeze(0)
    o = torch.full((R, Hv, dv), float("nan"), device=q.device)
    ws = L.gdn_workspace(len(lens), R, Hk, Hv, dk, dv, q.device)
    L.gdn_prefill_ws(q, k, v, beta, g, o, st, lens, ws)
    torch.cuda.synchronize()
    return o, st


def _check_prompts(orc, t, lens, o, st, tol=TOL_BF16, heads=()):
    S0 = t["S0"] if t["S0"].dim() == 4 else t["S0"].unsqueeze(0)
    r = 0
    for p, n in enumerate(lens):
        sl = slice(r, r + n)
        ref_o, ref_s = orc.gdn(f64(t["q"][sl]), f64(t["k"][sl]), f64(t["v"][sl]), f64(t["beta"][sl]),
                               f64(t["g"][sl]), f64(S0[p]))
        if n:
            assert torch.isfinite(o[sl]).all()
            assert rel_err(f64(o[sl]), ref_o) < tol, p
            for h in heads:
                assert rel_err(f64(o[sl, h]), ref_o[:, h]) < tol, (p, h)
        assert torch.isfinite(st[p]).all()
        assert rel_err(f64(st[p]), ref_s) < tol, p
        for h in heads:
            assert rel_err(f64(st[p, h]), ref_s[h]) < tol, (p, h)
        r += n


def test_chunkpar_small_and_determinism(L, orc):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.gdn_small(dtype=torch.bfloat16)
    o1, s1 = _run(L, d, [75])
    o2, s2 = _run(L, d, [75])
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    _check_prompts(orc, d, [75], o1, s1)


@pytest.mark.parametrize("nkeys", [16, 32, 64])
def test_chunkpar_nearly_parallel_keys(L, orc, nkeys):
    from linear_recurrence_chunked_amd import inputs

    start = 24 if nkeys == 16 else 0
    d = inputs.gdn_small(dtype=torch.bfloat16, parallel_keys=nkeys, parallel_start=start, beta_const=0.99)
    o, s = _run(L, d, [75])
    _check_prompts(orc, d, [75], o, s)


def test_chunkpar_9b_shape_full(L, orc):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.gdn_9b()
    o, s = _run(L, d, [2048])
    _check_prompts(orc, d, [2048], o, s, heads=(0, 31))


def test_chunkpar_long_prompt_59_chunks(L, orc):
    rng = np.random.default_rng(941)
    R, Hk, Hv, dk, dv = 3742, 1, 2, 128, 128
    q = rng.standard_normal((R, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((R, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    t = {"q": torch.from_numpy(q).to(torch.bfloat16), "k": torch.from_numpy(k).to(torch.bfloat16),
         "v": torch.from_numpy(rng.standard_normal((R, Hv, dv))).to(torch.bfloat16),
         "beta": torch.from_numpy(1 / (1 + np.exp(-rng.standard_normal((R, Hv))))).float(),
         "g": torch.from_numpy(np.stack([np.full(R, -1e-3), np.full(R, -8.0)], axis=1)).float(),
         "S0": torch.from_numpy(rng.normal(0, 0.1, (Hv, dk, dv))).float()}
    o, s = _run(L, t, [R])
    _check_prompts(orc, t, [R], o, s, heads=(0, 1))


@pytest.mark.parametrize("dk,dv,Hk,Hv", [(32, 32, 2, 4), (32, 64, 1, 2), (32, 128, 2, 2), (64, 32, 1, 3),
                                         (64, 64, 2, 4), (64, 128, 1, 2), (128, 32, 2, 4), (128, 64, 4, 8),
                                         (128, 128, 2, 4)])
def test_chunkpar_ragged_batches(L, orc, dk, dv, Hk, Hv):
    rng = np.random.default_rng(950 + dk + dv + Hk + Hv)
    lens = [1, 64, 0, 65, 130, 7, 200]
    R, P = sum(lens), len(lens)
    q = rng.standard_normal((R, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((R, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    t = {"q": torch.from_numpy(q).to(torch.bfloat16), "k": torch.from_numpy(k).to(torch.bfloat16),
         "v": torch.from_numpy(rng.standard_normal((R, Hv, dv))).to(torch.bfloat16),
         "beta": torch.from_numpy(1 / (1 + np.exp(-rng.standard_normal((R, Hv))))).float(),
         "g": torch.from_numpy(-np.logaddexp(0, rng.standard_normal((R, Hv))) * 0.5).float(),
         "S0": torch.from_numpy(rng.normal(0, 0.1, (P, Hv, dk, dv))).float()}
    o, s = _run(L, t, lens)
    _check_prompts(orc, t, lens, o, s)


def test_chunkpar_all_empty_and_rejects(L):
    q = torch.zeros((0, 2, 32), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((0, 2, 32), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((0, 2), device="cuda")
    o = torch.zeros((0, 2, 32), device="cuda")
    st = torch.randn((3, 2, 32, 32), device="cuda")
    keep = st.clone()
    ws = L.gdn_workspace(3, 0, 2, 2, 32, 32, "cuda")
    L.gdn_prefill_ws(q, q, v, b, b, o, st, [0, 0, 0], ws)
    torch.cuda.synchronize()
    assert torch.equal(st, keep)
    # too small a workspace is rejected before anything runs
    q = torch.zeros((70, 2, 32), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((70, 2, 32), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((70, 2), device="cuda")
    o = torch.zeros((70, 2, 32), device="cuda")
    small = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.LrcError) as ei:
        L.gdn_prefill_ws(q, q, v, b, b, o, st[:1], [70], small)
    assert ei.value.name == "LRC_ERR_SHAPE"


def test_chunkpar_many_prompts_two_state_waves(L, orc):
    """16 ragged prompts at the 9B-like head shape: more (prompt, head, 16-column) slices than compute
    units, so the state kernel runs two state waves of 16 columns per workgroup."""
    from linear_recurrence_chunked_amd import inputs

    lens = [300, 0, 64, 65, 1, 257, 130, 190, 17, 128, 45, 99, 200, 33, 70, 150]
    R, P, Hk, Hv, dk, dv = sum(lens), len(lens), 16, 32, 128, 128
    assert P * Hv * (dv // 16) > torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(960)
    q = rng.standard_normal((R, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((R, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    t = {"q": torch.from_numpy(q).to(torch.bfloat16), "k": torch.from_numpy(k).to(torch.bfloat16),
         "v": torch.from_numpy(rng.standard_normal((R, Hv, dv))).to(torch.bfloat16),
         "beta": torch.from_numpy(1 / (1 + np.exp(-rng.standard_normal((R, Hv))))).float(),
         "g": torch.from_numpy(inputs.gdn_decays(rng, R, Hv)).float(),
         "S0": torch.from_numpy(rng.normal(0, 0.1, (P, Hv, dk, dv))).float()}
    o, s = _run(L, t, lens)
    _check_prompts(orc, t, lens, o, s, heads=(0, 31))
