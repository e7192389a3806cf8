"""Pins for the oracle's RWKV-4 WKV token loop.

Source: "perf(rwkv): prefill text prompts in multi-token chunks",
Implementation.  The oracle keeps A and B as (num, den, max) and subtracts
the largest exponent before each exp.  The pins:
  * the unscaled definition A_t = e^w A_{t-1} + e^{k_t} v_t (B likewise),
    wkv_t = (A_{t-1} + e^{u+k_t} v_t) / (B_{t-1} + e^{u+k_t}), evaluated with
    50-digit decimals, including keys of +-30;
  * the page's own chunk form (three exponent kinds per row, per-row max over
    an [S+1, S] tensor, row S is the outgoing state) evaluated in float64;
  * a fresh state gives wkv_0 = v_0; outputs are convex combinations;
  * finite results at the edges of the decay and key ranges.
"""
from decimal import Decimal, getcontext

import numpy as np
import pytest

from helpers import rel_err

getcontext().prec = 50


def _decimal_reference(k, v, w, u, num0, den0, mx0):
    """Unscaled recurrence in 50-digit decimals; returns wkv and final (A, B)."""
    S, C = k.shape
    wkv = np.zeros((S, C))
    A_out, B_out = [], []
    for c in range(C):
        if num0[c] == 0.0 and den0[c] == 0.0:
            A, B = Decimal(0), Decimal(0)
        else:
            scale = Decimal(float(mx0[c])).exp()
            A, B = Decimal(float(num0[c])) * scale, Decimal(float(den0[c])) * scale
        ew = Decimal(float(w[c])).exp()
        for t in range(S):
            kt, vt = Decimal(float(k[t, c])), Decimal(float(v[t, c]))
            eb = (Decimal(float(u[c])) + kt).exp()
            wkv[t, c] = float((A + eb * vt) / (B + eb))
            ek = kt.exp()
            A = ew * A + ek * vt
            B = ew * B + ek
        A_out.append(A)
        B_out.append(B)
    return wkv, A_out, B_out


def _row_form_chunk(k, v, w, u, num0, den0, mx0):
    """The page's chunk form: row t in [0, S] combines exponents max0 + t w
    (incoming state), k_i + (t-1-i) w for i < t, and u + k_t (t < S only), each
    row shifted by its own largest exponent.  Returns wkv rows and the state."""
    S, C = k.shape
    wkv = np.zeros((S, C))
    state = None
    for t in range(S + 1):
        ex = [mx0 + t * w]
        cn = [num0]
        cd = [den0]
        for i in range(t):
            ex.append(k[i] + (t - 1 - i) * w)
            cn.append(v[i])
            cd.append(np.ones(C))
        if t < S:
            ex.append(u + k[t])
            cn.append(v[t])
            cd.append(np.ones(C))
        ex = np.stack(ex)
        p = ex.max(axis=0)
        f = np.exp(ex - p)
        n = (f * np.stack(cn)).sum(axis=0)
        d = (f * np.stack(cd)).sum(axis=0)
        if t < S:
            wkv[t] = n / d
        else:
            state = (n, d, p)
    return wkv, state


def _inputs(rng, S, C, spikes=True):
    d = rng.uniform(-6.0, 2.0, C)
    w = -np.exp(d)
    u = rng.uniform(-2.0, 2.0, C)
    k = rng.normal(0.0, 3.0, (S, C))
    if spikes:
        m = rng.uniform(size=(S, C)) < 0.05
        k = np.where(m, np.where(rng.uniform(size=(S, C)) < 0.5, -30.0, 30.0), k)
    v = rng.standard_normal((S, C))
    return k, v, w, u


def _scaled(num, den, mx, M):
    f = np.exp(mx - M)
    return num * f, den * f


def test_wkv_matches_decimal_definition(orc):
    rng = np.random.default_rng(60)
    S, C = 24, 6
    k, v, w, u = _inputs(rng, S, C)
    n0, d0, m0 = orc.empty_wkv_state(C)
    out, n, d, m = orc.wkv4(k, v, w, u, n0, d0, m0)
    ref, A, B = _decimal_reference(k, v, w, u, n0, d0, m0)
    assert rel_err(out, ref) < 1e-13
    for c in range(C):
        got_A = Decimal(float(n[c])) * Decimal(float(m[c])).exp()
        got_B = Decimal(float(d[c])) * Decimal(float(m[c])).exp()
        assert abs(got_A - A[c]) <= Decimal("1e-12") * abs(B[c]) * Decimal(float(np.max(np.abs(v[:, c]))))
        assert abs(got_B / B[c] - 1) < Decimal("1e-12")


def test_wkv_matches_decimal_from_nonempty_state(orc):
    rng = np.random.default_rng(61)
    S, C = 16, 5
    k, v, w, u = _inputs(rng, S, C)
    n0 = rng.standard_normal(C)
    d0 = rng.uniform(0.5, 2.0, C)
    m0 = rng.uniform(-5.0, 30.0, C)
    out, n, d, m = orc.wkv4(k, v, w, u, n0, d0, m0)
    ref, A, B = _decimal_reference(k, v, w, u, n0, d0, m0)
    assert rel_err(out, ref) < 1e-13
    for c in range(C):
        got_B = Decimal(float(d[c])) * Decimal(float(m[c])).exp()
        assert abs(got_B / B[c] - 1) < Decimal("1e-12")


@pytest.mark.parametrize("splits", [[64, 11], [75], [7, 4, 64], [1] * 20])
def test_wkv_matches_page_row_form(orc, splits):
    rng = np.random.default_rng(62)
    S, C = sum(splits), 40
    k, v, w, u = _inputs(rng, S, C)
    n0, d0, m0 = orc.empty_wkv_state(C)
    out, n, d, m = orc.wkv4(k, v, w, u, n0, d0, m0)
    parts, st, r = [], (n0, d0, m0), 0
    for s in splits:
        y, st = _row_form_chunk(k[r:r + s], v[r:r + s], w, u, *st)
        parts.append(y)
        r += s
    assert rel_err(out, np.concatenate(parts)) < 1e-12
    # the state's max is the chunk's row-S max; the triple agrees up to rounding
    assert np.max(np.abs(m - st[2])) < 1e-9 * np.max(np.abs(m))
    on, od = _scaled(n, d, m, m)
    rn, rd = _scaled(*st, m)
    assert rel_err(on, rn) < 1e-12 and rel_err(od, rd) < 1e-12


def test_wkv_fresh_state_first_row_is_v(orc):
    rng = np.random.default_rng(63)
    C = 50
    k, v, w, u = _inputs(rng, 3, C)
    out, *_ = orc.wkv4(k, v, w, u, *orc.empty_wkv_state(C))
    np.testing.assert_array_equal(out[0], v[0])


def test_wkv_outputs_are_convex_combinations(orc):
    rng = np.random.default_rng(64)
    S, C = 64, 30
    k, v, w, u = _inputs(rng, S, C)
    n0 = rng.standard_normal(C)
    d0 = rng.uniform(0.5, 2.0, C)
    m0 = rng.uniform(-3.0, 3.0, C)
    out, *_ = orc.wkv4(k, v, w, u, n0, d0, m0)
    r0 = n0 / d0
    for t in range(S):
        lo = np.minimum(r0, v[: t + 1].min(axis=0))
        hi = np.maximum(r0, v[: t + 1].max(axis=0))
        assert np.all(out[t] >= lo - 1e-12) and np.all(out[t] <= hi + 1e-12)
    # constant v with the same incoming ratio gives a constant output
    vc = np.full((S, C), 0.75)
    out, *_ = orc.wkv4(k, vc, w, u, 0.75 * d0, d0, m0)
    assert np.max(np.abs(out - 0.75)) < 1e-14


def test_wkv_single_row_chunk_equals_one_step(orc):
    rng = np.random.default_rng(65)
    S, C = 9, 12
    k, v, w, u = _inputs(rng, S, C)
    st = orc.empty_wkv_state(C)
    full, *st_full = orc.wkv4(k, v, w, u, *st)
    rows = []
    for t in range(S):
        y, *st = orc.wkv4(k[t:t + 1], v[t:t + 1], w, u, *st)
        rows.append(y)
    np.testing.assert_array_equal(np.concatenate(rows), full)
    for a, b in zip(st, st_full):
        np.testing.assert_array_equal(a, b)


def test_wkv_finite_at_range_edges(orc):
    C = 8
    w = -np.exp(np.array([-6.0, 2.0, -6.0, 2.0, 0.0, -3.0, 1.0, -6.0]))
    u = np.array([-2.0, 2.0, 2.0, -2.0, 0.0, 1.0, -1.0, 2.0])
    S = 128
    k = np.where(np.arange(S)[:, None] % 2 == 0, 30.0, -30.0) * np.ones((S, C))
    v = np.cos(np.arange(S * C).reshape(S, C))
    out, n, d, m = orc.wkv4(k, v, w, u, *orc.empty_wkv_state(C))
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(n)) and np.all(np.isfinite(d)) and np.all(np.isfinite(m))
    assert np.all(d > 0)
