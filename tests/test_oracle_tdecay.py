"""Pins for the oracle's WKV with a token-dependent decay.

"perf(rwkv): prefill text prompts in multi-token chunks", Notes For Future
Readers: RWKV generations with a per-token decay call for a different chunk
form.  The pages print no formula for those versions; the oracle reads the
decay of the RWKV-4 step as a decay w_t of the row,
    A_t = e^{w_t} A_{t-1} + e^{k_t} v_t,   B_t = e^{w_t} B_{t-1} + e^{k_t},
    wkv_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t}).
Pins: a decay constant over rows is the (already pinned) RWKV-4 routine bit
for bit; brute-force sums of the unrolled recurrence on tiny inputs fix which
row's decay applies where; a zero decay gives a running mean in closed form;
a huge decay at one row forgets everything before that row; chunk splits
carry the state; extreme keys and decays stay finite.
"""
import numpy as np
import pytest

from helpers import rel_err


def _inputs(rng, S, C, sd=3.0):
    k = rng.normal(0, sd, (S, C))
    v = rng.standard_normal((S, C))
    w = -np.exp(rng.uniform(-6, 2, (S, C)))
    u = rng.uniform(-2, 2, C)
    return k, v, w, u


def test_tdecay_constant_decay_is_rwkv4(orc):
    rng = np.random.default_rng(130)
    k, v, w, u = _inputs(rng, 40, 9)
    wc = w[0]
    a = orc.wkv4(k, v, wc, u, *orc.empty_wkv_state(9))
    b = orc.wkv_tdecay(k, v, np.tile(wc, (40, 1)), u, *orc.empty_wkv_state(9))
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_tdecay_matches_brute_force_sums(orc):
    """The unrolled recurrence, summed term by term without any shift."""
    rng = np.random.default_rng(131)
    S, C = 6, 4
    k, v, w, u = _inputs(rng, S, C, sd=1.0)
    num0, den0, mx0 = rng.uniform(0.5, 2, C), rng.uniform(0.5, 2, C), rng.uniform(-1, 1, C)
    out, n, d, m = orc.wkv_tdecay(k, v, w, u, num0, den0, mx0)
    for c in range(C):
        for t in range(S + 1):
            # state after rows 0 .. t-1: the incoming state decayed by w_0 .. w_{t-1},
            # row i decayed by w_{i+1} .. w_{t-1}
            A = num0[c] * np.exp(mx0[c] + w[:t, c].sum())
            B = den0[c] * np.exp(mx0[c] + w[:t, c].sum())
            for i in range(t):
                f = np.exp(k[i, c] + w[i + 1:t, c].sum())
                A += f * v[i, c]
                B += f
            if t < S:
                eb = np.exp(u[c] + k[t, c])
                ref = (A + eb * v[t, c]) / (B + eb)
                assert abs(out[t, c] - ref) <= 1e-12 * max(1.0, abs(ref))
            else:
                assert abs(n[c] * np.exp(m[c]) - A) <= 1e-12 * abs(A)
                assert abs(d[c] * np.exp(m[c]) - B) <= 1e-12 * abs(B)


def test_tdecay_zero_decay_is_a_running_mean(orc):
    """w = 0 and k = 0: every row weighs 1, the bonus e^u, the incoming state den0 e^max0."""
    rng = np.random.default_rng(132)
    S, C = 30, 3
    v = rng.standard_normal((S, C))
    u = rng.uniform(-2, 2, C)
    num0, den0, mx0 = rng.uniform(0.5, 2, C), rng.uniform(0.5, 2, C), rng.uniform(-1, 1, C)
    out, *_ = orc.wkv_tdecay(np.zeros((S, C)), v, np.zeros((S, C)), u, num0, den0, mx0)
    A0, B0 = num0 * np.exp(mx0), den0 * np.exp(mx0)
    prefix = np.concatenate([np.zeros((1, C)), np.cumsum(v, axis=0)[:-1]])
    t = np.arange(S)[:, None]
    ref = (A0 + prefix + np.exp(u) * v) / (B0 + t + np.exp(u))
    assert rel_err(out, ref) < 1e-13


def test_tdecay_huge_decay_forgets_the_past(orc):
    """A decay of -1e4 at row r wipes the state: rows after r see only rows >= r."""
    rng = np.random.default_rng(133)
    S, C, r = 40, 6, 17
    k, v, w, u = _inputs(rng, S, C)
    num0, den0, mx0 = rng.uniform(0.5, 2, C), rng.uniform(0.5, 2, C), rng.uniform(-1, 1, C)
    w[r] = -1e4
    full, *_ = orc.wkv_tdecay(k, v, w, u, num0, den0, mx0)
    tail, *_ = orc.wkv_tdecay(k[r:], v[r:], w[r:], u, *orc.empty_wkv_state(C))
    assert rel_err(full[r + 1:], tail[1:]) < 1e-12


@pytest.mark.parametrize("splits", [[64, 11], [1] * 75, [7, 0, 68]])
def test_tdecay_chunk_split_invariance(orc, splits):
    rng = np.random.default_rng(134)
    k, v, w, u = _inputs(rng, 75, 5)
    ref = orc.wkv_tdecay(k, v, w, u, *orc.empty_wkv_state(5))
    st, parts, r = orc.empty_wkv_state(5), [], 0
    for n in splits:
        o, *st = orc.wkv_tdecay(k[r:r + n], v[r:r + n], w[r:r + n], u, *st)
        parts.append(o)
        r += n
    np.testing.assert_array_equal(np.concatenate(parts), ref[0])
    for a, b in zip(st, ref[1:]):
        np.testing.assert_array_equal(a, b)


def test_tdecay_finite_at_range_edges(orc):
    rng = np.random.default_rng(135)
    S, C = 300, 8
    k, v, w, u = _inputs(rng, S, C)
    k[rng.random((S, C)) < 0.05] = 30.0
    k[rng.random((S, C)) < 0.05] = -30.0
    w[:, 0], w[:, 1] = -np.exp(2.0), -np.exp(-6.0)
    out, n, d, m = orc.wkv_tdecay(k, v, w, u, *orc.empty_wkv_state(C))
    assert np.isfinite(out).all() and np.isfinite(n).all() and np.isfinite(d).all() and np.isfinite(m).all()
    assert (np.abs(out) <= np.abs(v).max() + 1e-12).all()  # a weighted mean of the v's
