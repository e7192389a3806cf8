"""GPU parity of K3 (Gated DeltaNet chunk) and of its triangular inverse
against the float64 oracle.

Workloads: small (8 heads, dk = dv = 64, 75 rows as 64 + 11) in fp32 (tol
1e-4) and bf16 (tol 2e-2; the split bf16 form, whose FP32 operands enter the
matrix cores as hi + lo pairs, to 1e-4); the stress case of nearly parallel keys
(cosine > 0.999) with beta = 0.99, for 16, 32 and 64 such keys; the 9B-like
shape (32 value heads on 16 key heads, 128 x 128, 2048 rows as 32 x 64 chunks,
bf16, decays from -1e-3 to -8 per row); ragged batches.  The inverse is
checked on its own at the precision the chunk uses (FP32), on full 64-row
matrices of nearly parallel keys, against forward substitution.
"""
import numpy as np
import pytest
import torch

from gpu_util import chunks, f64, require_gpu, to_dev
from helpers import TOL_BF16, TOL_F32, rel_err

pytestmark = pytest.mark.gpu

TOL_SPLIT = 1e-4  # hi + lo bf16 pairs carry about 16 mantissa bits


@pytest.fixture(scope="module")
def L():
    require_gpu()
    from linear_recurrence_chunked_amd import lrc

    return lrc


def _run_chunked(L, d, splits, split=False):
    q, k, v, beta, g, S0 = (to_dev(d[n]) for n in ("q", "k", "v", "beta", "g", "S0"))
    R, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    o = torch.empty((R, Hv, dv), device=q.device)
    st = S0.clone().unsqueeze(0)
    for r, n in chunks(R, splits):
        oc = torch.empty((1, n, Hv, dv), device=q.device)
        L.gdn_chunk(q[r:r + n][None].contiguous(), k[r:r + n][None].contiguous(), v[r:r + n][None].contiguous(),
                    beta[r:r + n][None].contiguous(), g[r:r + n][None].contiguous(), oc, st, st, split=split)
        o[r:r + n] = oc[0]
    torch.cuda.synchronize()
    return o, st[0]


def _run_prefill(L, d, split=False):
    q, k, v, beta, g, S0 = (to_dev(d[n]) for n in ("q", "k", "v", "beta", "g", "S0"))
    R = q.shape[0]
    Hv, dv = v.shape[1], v.shape[2]
    o = torch.empty((R, Hv, dv), device=q.device)
    st = S0.clone().unsqueeze(0)
    L.gdn_prefill(q, k, v, beta, g, o, st, [R], split=split)
    torch.cuda.synchronize()
    return o, st[0]


def _oracle(orc, d):
    return orc.gdn(*(f64(d[n]) for n in ("q", "k", "v", "beta", "g", "S0")))


@pytest.mark.parametrize("dtype,tol", [(torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)])
@pytest.mark.parametrize("splits", [[64, 11], [7, 4, 64], [1] * 11 + [64]])
def test_gdn_small_chunked(L, orc, dtype, tol, splits):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.gdn_small(dtype=dtype)
    ref_o, ref_s = _oracle(orc, d)
    o, s = _run_chunked(L, d, splits)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    assert rel_err(f64(o), ref_o) < tol
    assert rel_err(f64(s), ref_s) < tol


@pytest.mark.parametrize("dtype,tol", [(torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)])
def test_gdn_small_prefill_and_determinism(L, orc, dtype, tol):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.gdn_small(dtype=dtype)
    ref_o, ref_s = _oracle(orc, d)
    o1, s1 = _run_prefill(L, d)
    o2, s2 = _run_prefill(L, d)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    assert rel_err(f64(o1), ref_o) < tol
    assert rel_err(f64(s1), ref_s) < tol


@pytest.mark.parametrize("nkeys", [16, 32, 64])
@pytest.mark.parametrize("dtype,tol", [(torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)])
def test_gdn_nearly_parallel_keys_beta_near_one(L, orc, nkeys, dtype, tol):
    from linear_recurrence_chunked_amd import inputs

    start = 24 if nkeys == 16 else 0
    d = inputs.gdn_small(dtype=dtype, parallel_keys=nkeys, parallel_start=start, beta_const=0.99)
    kk = f64(d["k"])[start:start + nkeys, 0]
    cos = kk @ kk.T
    assert cos.min() > 0.999
    ref_o, ref_s = _oracle(orc, d)
    o, s = _run_prefill(L, d)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    assert rel_err(f64(o), ref_o) < tol
    assert rel_err(f64(s), ref_s) < tol


def test_gdn_9b_shape_full(L, orc):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.gdn_9b()
    ref_o, ref_s = _oracle(orc, d)
    o, s = _run_prefill(L, d)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    assert rel_err(f64(o), ref_o) < TOL_BF16
    assert rel_err(f64(s), ref_s) < TOL_BF16
    # the head with g = -8 per row: gamma reaches -512 inside a chunk
    assert rel_err(f64(o[:, 31]), ref_o[:, 31]) < TOL_BF16
    assert rel_err(f64(s[31]), ref_s[31]) < TOL_BF16


@pytest.mark.parametrize("dk,dv,Hk,Hv", [(32, 32, 2, 4), (64, 32, 1, 3), (128, 64, 2, 2), (32, 128, 1, 2)])
def test_gdn_ragged_batch(L, orc, dk, dv, Hk, Hv):
    rng = np.random.default_rng(300 + dk + dv + Hv)
    lens = [1, 64, 0, 65, 130, 7]
    R, P = sum(lens), len(lens)
    q = rng.standard_normal((R, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((R, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((R, Hv, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((R, Hv))))
    g = -np.logaddexp(0, rng.standard_normal((R, Hv))) * 0.5
    S0 = rng.normal(0, 0.1, (P, Hv, dk, dv))
    t = {n: torch.from_numpy(a).float() for n, a in dict(q=q, k=k, v=v, beta=beta, g=g, S0=S0).items()}
    dq, dk_, dv_, db, dg, dS = (to_dev(t[n]) for n in ("q", "k", "v", "beta", "g", "S0"))
    o = torch.full((R, Hv, dv), float("nan"), device="cuda")
    L.gdn_prefill(dq, dk_, dv_, db, dg, o, dS, lens)
    torch.cuda.synchronize()
    r = 0
    for p, n in enumerate(lens):
        sl = slice(r, r + n)
        ref_o, ref_s = orc.gdn(f64(t["q"][sl]), f64(t["k"][sl]), f64(t["v"][sl]), f64(t["beta"][sl]),
                               f64(t["g"][sl]), f64(t["S0"][p]))
        if n:
            assert rel_err(f64(o[sl]), ref_o) < TOL_F32
        assert rel_err(f64(dS[p]), ref_s) < TOL_F32
        r += n


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("dk,dv,Hk,Hv", [(32, 32, 8, 16), (64, 32, 16, 64), (32, 64, 12, 24), (32, 32, 4, 4),
                                         (64, 128, 2, 32), (32, 32, 8, 128), (32, 128, 1, 2), (64, 64, 2, 4),
                                         (128, 32, 2, 4), (128, 64, 4, 8)])
def test_gdn_bf16_head_layouts(L, orc, dk, dv, Hk, Hv, split):
    """The bf16 matrix-core path over ragged prompts with value-head groups of 1, 2, 4 and 16.
    Groups whose value heads fill whole multiples of 8 groups are placed so that siblings share
    an XCD; the others keep the plain order: both must give every head its own key head.  Every
    (dk, dv) build of the kernel runs in both forms (single rounding, and split at 1e-4)."""
    tol = TOL_SPLIT if split else TOL_BF16
    rng = np.random.default_rng(900 + dk + dv + Hk + Hv)
    lens = [1, 64, 0, 65, 130, 7]
    R, P = sum(lens), len(lens)
    q = rng.standard_normal((R, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((R, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((R, Hv, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((R, Hv))))
    g = -np.logaddexp(0, rng.standard_normal((R, Hv))) * 0.5
    S0 = rng.normal(0, 0.1, (P, Hv, dk, dv))
    t = {n: torch.from_numpy(a).float() for n, a in dict(beta=beta, g=g, S0=S0).items()}
    for n, a in dict(q=q, k=k, v=v).items():
        t[n] = torch.from_numpy(a).to(torch.bfloat16)
    dq, dk_, dv_, db, dg, dS = (to_dev(t[n]) for n in ("q", "k", "v", "beta", "g", "S0"))
    o = torch.full((R, Hv, dv), float("nan"), device="cuda")
    L.gdn_prefill(dq, dk_, dv_, db, dg, o, dS, lens, split=split)
    torch.cuda.synchronize()
    r = 0
    for p, n in enumerate(lens):
        sl = slice(r, r + n)
        ref_o, ref_s = orc.gdn(f64(t["q"][sl]), f64(t["k"][sl]), f64(t["v"][sl]), f64(t["beta"][sl]),
                               f64(t["g"][sl]), f64(t["S0"][p]))
        if n:
            assert rel_err(f64(o[sl]), ref_o) < tol
        assert rel_err(f64(dS[p]), ref_s) < tol
        r += n


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("dk,dv,Hk,Hv", [(32, 32, 16, 32), (128, 128, 16, 32), (32, 64, 12, 24), (64, 32, 4, 64)])
def test_gdn_bf16_lanes(L, orc, dk, dv, Hk, Hv, split):
    """Value heads over 16 ragged prompts with more workgroups than compute units, so the prompts
    run as lanes (256 CUs: 8 lanes of 32 heads, 10 of 24, 4 of 64), several per workgroup row, with
    chunks of different prompts back to back in one pipeline and the state swapped at each prompt
    boundary."""
    tol = TOL_SPLIT if split else TOL_BF16
    lens = [300, 0, 64, 65, 1, 257, 130, 190, 17, 128, 45, 99, 200, 33, 70, 150]
    R, P = sum(lens), len(lens)
    assert P * Hv > torch.cuda.get_device_properties(0).multi_processor_count
    rng = np.random.default_rng(910 + dk + dv + Hv)
    q = rng.standard_normal((R, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((R, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((R, Hv, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((R, Hv))))
    g = -np.logaddexp(0, rng.standard_normal((R, Hv))) * 0.5
    S0 = rng.normal(0, 0.1, (P, Hv, dk, dv))
    t = {n: torch.from_numpy(a).float() for n, a in dict(beta=beta, g=g, S0=S0).items()}
    for n, a in dict(q=q, k=k, v=v).items():
        t[n] = torch.from_numpy(a).to(torch.bfloat16)
    dq, dk_, dv_, db, dg, dS = (to_dev(t[n]) for n in ("q", "k", "v", "beta", "g", "S0"))
    o = torch.full((R, Hv, dv), float("nan"), device="cuda")
    L.gdn_prefill(dq, dk_, dv_, db, dg, o, dS, lens, split=split)
    torch.cuda.synchronize()
    first = (o.clone(), dS.clone())
    dS.copy_(to_dev(t["S0"]))
    L.gdn_prefill(dq, dk_, dv_, db, dg, o, dS, lens, split=split)  # same lengths again: the kept plan
    torch.cuda.synchronize()
    assert torch.equal(first[0], o) and torch.equal(first[1], dS)
    r = 0
    for p, n in enumerate(lens):
        sl = slice(r, r + n)
        ref_o, ref_s = orc.gdn(f64(t["q"][sl]), f64(t["k"][sl]), f64(t["v"][sl]), f64(t["beta"][sl]),
                               f64(t["g"][sl]), f64(t["S0"][p]))
        if n:
            assert rel_err(f64(o[sl]), ref_o) < tol
        assert rel_err(f64(dS[p]), ref_s) < tol
        r += n


def test_gdn_rejects_65_rows(L):
    q = torch.randn(1, 65, 1, 32, device="cuda")
    v = torch.randn(1, 65, 1, 32, device="cuda")
    b = torch.rand(1, 65, 1, device="cuda")
    S = torch.zeros(1, 1, 32, 32, device="cuda")
    with pytest.raises(L.LrcError) as ei:
        L.gdn_chunk(q, q.clone(), v, b, -b, torch.empty_like(v), S, S)
    assert ei.value.name == "LRC_ERR_ROWS"


def _near_parallel_A(rng, n, nkeys, beta=0.99, dk=64):
    k = rng.standard_normal((n, dk))
    k[:nkeys] = rng.standard_normal(dk) + 1e-3 * rng.standard_normal((nkeys, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    g = -np.logaddexp(0.0, rng.standard_normal(n)) * 0.01
    gam = np.cumsum(g)
    A = beta * np.exp(np.tril(gam[:, None] - gam[None, :], -1)) * (k @ k.T)
    return np.tril(A, -1)


@pytest.mark.parametrize("n,nkeys", [(64, 64), (64, 32), (64, 16), (37, 37), (8, 8), (1, 1)])
def test_inverse_full_chunk_production_precision(L, orc, n, nkeys):
    rng = np.random.default_rng(400 + n + nkeys)
    A = np.stack([_near_parallel_A(rng, n, nkeys) for _ in range(8)]).astype(np.float32)
    tA = to_dev(torch.from_numpy(A))
    T = torch.empty_like(tA)
    L.unit_lower_inverse(tA, T)
    torch.cuda.synchronize()
    ref = orc.unit_lower_inverse(A.astype(np.float64))
    got = f64(T)
    for b in range(8):
        assert rel_err(got[b], ref[b]) < TOL_F32
    assert np.all(np.triu(got, 1) == 0) and np.all(np.diagonal(got, axis1=1, axis2=2) == 1)


def test_gdn_bf16_random_lane_plans(L, orc):
    """Seeded random batches with more (prompt, head) workgroups than compute units, so each one runs
    a different lane plan: 9-40 prompts of 0-300 rows, 32 or 64 value heads over 16 key heads,
    dk = dv = 32.  Every prompt and head against the float64 oracle."""
    rng = np.random.default_rng(4242)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for case in range(6):
        Hk, Hv, dk, dv = 16, int(rng.choice([32, 64])), 32, 32
        P = int(rng.integers(cus // Hv + 1, 41))
        lens = [int(x) for x in rng.integers(0, 301, size=P)]
        lens[int(rng.integers(0, P))] = int(rng.choice([0, 64, 65]))
        if sum(lens) == 0:
            lens[0] = 7
        R = sum(lens)
        q = rng.standard_normal((R, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k = rng.standard_normal((R, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
        v = rng.standard_normal((R, Hv, dv))
        beta = 1 / (1 + np.exp(-rng.standard_normal((R, Hv))))
        g = -np.logaddexp(0, rng.standard_normal((R, Hv))) * 0.5
        S0 = rng.normal(0, 0.1, (P, Hv, dk, dv))
        t = {n: torch.from_numpy(a).float() for n, a in dict(beta=beta, g=g, S0=S0).items()}
        for n, a in dict(q=q, k=k, v=v).items():
            t[n] = torch.from_numpy(a).to(torch.bfloat16)
        dq, dk_, dv_, db, dg, dS = (to_dev(t[n]) for n in ("q", "k", "v", "beta", "g", "S0"))
        o = torch.full((R, Hv, dv), float("nan"), device="cuda")
        L.gdn_prefill(dq, dk_, dv_, db, dg, o, dS, lens)
        torch.cuda.synchronize()
        r = 0
        for p, n in enumerate(lens):
            sl = slice(r, r + n)
            ref_o, ref_s = orc.gdn(f64(t["q"][sl]), f64(t["k"][sl]), f64(t["v"][sl]), f64(t["beta"][sl]),
                                   f64(t["g"][sl]), f64(t["S0"][p]))
            if n:
                assert rel_err(f64(o[sl]), ref_o) < TOL_BF16, (case, p)
            assert rel_err(f64(dS[p]), ref_s) < TOL_BF16, (case, p)
            r += n



def _split_case(name):
    from linear_recurrence_chunked_amd import inputs

    if name == "small":
        return inputs.gdn_small(dtype=torch.bfloat16)
    if name == "parallel64":
        return inputs.gdn_small(dtype=torch.bfloat16, parallel_keys=64, parallel_start=0, beta_const=0.99)
    return inputs.gdn_9b()


@pytest.mark.parametrize("case", ["small", "parallel64", "9b"])
def test_gdn_bf16_split_precision(L, orc, case):
    """The split form against the oracle at 1e-4, and the default single
    rounding on the same inputs within the bf16 tolerance."""
    d = _split_case(case)
    ref_o, ref_s = _oracle(orc, d)
    o, s = _run_prefill(L, d, split=True)
    assert rel_err(f64(o), ref_o) < TOL_SPLIT
    assert rel_err(f64(s), ref_s) < TOL_SPLIT
    o1, s1 = _run_prefill(L, d)
    assert rel_err(f64(o1), ref_o) < TOL_BF16
    assert rel_err(f64(s1), ref_s) < TOL_BF16


def test_gdn_bf16_split_chunked_and_rejects_f32(L, orc):
    from linear_recurrence_chunked_amd import inputs

    d = inputs.gdn_small(dtype=torch.bfloat16)
    ref_o, ref_s = _oracle(orc, d)
    o, s = _run_chunked(L, d, [7, 4, 64], split=True)
    assert rel_err(f64(o), ref_o) < TOL_SPLIT
    assert rel_err(f64(s), ref_s) < TOL_SPLIT
    with pytest.raises(ValueError):
        _run_prefill(L, inputs.gdn_small(dtype=torch.float32), split=True)


# ---------------------------------------------------------------- FP32 inputs at the timed shape
def test_gdn_fp32_9b_shape_full(L, orc):
    """The FP32-input path at the 9B-like shape (32 value heads on 16 key heads, dk = dv = 128,
    2048 rows = 32 chunks of 64) against the oracle at 1e-4, every head, and the head whose decay is
    -8 on every row (gamma reaches -512 inside a chunk) on its own."""
    from linear_recurrence_chunked_amd import inputs

    d = inputs.gdn_9b(dtype=torch.float32)
    ref_o, ref_s = _oracle(orc, d)
    o, s = _run_prefill(L, d)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    assert rel_err(f64(o), ref_o) < TOL_F32
    assert rel_err(f64(s), ref_s) < TOL_F32
    for h in (0, 31):
        assert rel_err(f64(o[:, h]), ref_o[:, h]) < TOL_F32, h
        assert rel_err(f64(s[h]), ref_s[h]) < TOL_F32, h


def test_gdn_fp32_lane_lengths_128(L, orc):
    """The FP32-input path at dk = dv = 128 over the 16-prompt ragged length mix of the lane tests
    (32 value heads on 16 key heads, decays of the 9B-like recipe), every prompt against the oracle."""
    from linear_recurrence_chunked_amd import inputs

    lens = [300, 0, 64, 65, 1, 257, 130, 190, 17, 128, 45, 99, 200, 33, 70, 150]
    R, P, Hk, Hv, dk, dv = sum(lens), len(lens), 16, 32, 128, 128
    rng = np.random.default_rng(930)
    q = rng.standard_normal((R, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((R, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((R, Hv, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((R, Hv))))
    g = inputs.gdn_decays(rng, R, Hv)
    S0 = rng.normal(0, 0.1, (P, Hv, dk, dv))
    t = {n: torch.from_numpy(a).float() for n, a in dict(q=q, k=k, v=v, beta=beta, g=g, S0=S0).items()}
    dq, dk_, dv_, db, dg, dS = (to_dev(t[n]) for n in ("q", "k", "v", "beta", "g", "S0"))
    o = torch.full((R, Hv, dv), float("nan"), device="cuda")
    L.gdn_prefill(dq, dk_, dv_, db, dg, o, dS, lens)
    torch.cuda.synchronize()
    r = 0
    for p, n in enumerate(lens):
        sl = slice(r, r + n)
        ref_o, ref_s = orc.gdn(f64(t["q"][sl]), f64(t["k"][sl]), f64(t["v"][sl]), f64(t["beta"][sl]),
                               f64(t["g"][sl]), f64(t["S0"][p]))
        if n:
            assert rel_err(f64(o[sl]), ref_o) < TOL_F32, p
        assert rel_err(f64(dS[p]), ref_s) < TOL_F32, p
        r += n


@pytest.mark.parametrize("dtype,tol", [(torch.float32, TOL_F32), (torch.bfloat16, TOL_BF16)])
def test_gdn_long_prompt_59_chunks(L, orc, dtype, tol):
    """One prompt of 3 742 rows (59 chunks, the longest of the mixed prefill) at dk = dv = 128 on two
    value heads of one key head, one with the mildest (-1e-3) and one with the strongest (-8) decay of
    the range on every row: the error of the chunk chain over tens of chunks."""
    rng = np.random.default_rng(931)
    R, Hk, Hv, dk, dv = 3742, 1, 2, 128, 128
    q = rng.standard_normal((R, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((R, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((R, Hv, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((R, Hv))))
    g = np.stack([np.full(R, -1e-3), np.full(R, -8.0)], axis=1)
    S0 = rng.normal(0, 0.1, (Hv, dk, dv))
    t = {n: torch.from_numpy(a).float() for n, a in dict(beta=beta, g=g, S0=S0).items()}
    for n, a in dict(q=q, k=k, v=v).items():
        t[n] = torch.from_numpy(a).to(dtype)
    ref_o, ref_s = orc.gdn(*(f64(t[n]) for n in ("q", "k", "v", "beta", "g", "S0")))
    o, s = _run_prefill(L, t)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    for h in range(Hv):
        assert rel_err(f64(o[:, h]), ref_o[:, h]) < tol, h
        assert rel_err(f64(s[h]), ref_s[h]) < tol, h
