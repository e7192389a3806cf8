"""Pins for the oracle's selective scan h_t = a_t h_{t-1} + b_t.

Source: "perf(mamba): prefill text prompts in multi-token chunks",
Implementation (the scan over the chunk rows with the incoming state h_0,
every factor a decay in (0, 1]).  The pins: the unrolled closed form summed
by brute force, special cases that reduce to numpy/scipy routines (cumsum,
cumprod, a first-order IIR filter), the bound implied by decays in (0, 1],
and chunk-split invariance.
"""
import itertools

import numpy as np
import pytest
from scipy.signal import lfilter

from helpers import rel_err


def _closed_form(a, b, h0):
    """h_t = (prod_{j<=t} a_j) h0 + sum_{i<=t} (prod_{i<j<=t} a_j) b_i, by brute force."""
    S = a.shape[0]
    out = np.zeros_like(a)
    for t in range(S):
        acc = np.prod(a[: t + 1], axis=0) * h0
        for i in range(t + 1):
            acc = acc + np.prod(a[i + 1: t + 1], axis=0) * b[i]
        out[t] = acc
    return out


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8])
def test_scan_closed_form(orc, S):
    rng = np.random.default_rng(10 + S)
    E = 7
    a = rng.uniform(0.05, 1.0, (S, E))
    b = rng.standard_normal((S, E))
    h0 = rng.standard_normal(E)
    h, hS = orc.scan(a, b, h0)
    ref = _closed_form(a, b, h0)
    assert rel_err(h, ref) < 1e-14
    np.testing.assert_array_equal(hS, h[-1])


def test_scan_special_cases_reduce_to_library_routines(orc):
    rng = np.random.default_rng(20)
    S, E = 40, 6
    b = rng.standard_normal((S, E))
    a = rng.uniform(0.1, 1.0, (S, E))
    h0 = rng.standard_normal(E)
    h, _ = orc.scan(np.ones((S, E)), b, h0)                  # a = 1: prefix sum
    assert rel_err(h, h0 + np.cumsum(b, axis=0)) < 1e-14
    h, _ = orc.scan(a, np.zeros((S, E)), h0)                 # b = 0: prefix product
    assert rel_err(h, np.cumprod(a, axis=0) * h0) < 1e-14
    h, _ = orc.scan(np.zeros((S, E)), b, h0)                 # a = 0: memoryless
    np.testing.assert_array_equal(h, b)
    for e in range(E):                                       # constant a: IIR filter
        ac = float(a[0, e])
        ref = lfilter([1.0], [1.0, -ac], b[:, e], zi=[ac * h0[e]])[0]
        h, _ = orc.scan(np.full((S, 1), ac), b[:, e:e + 1], h0[e:e + 1])
        assert rel_err(h[:, 0], ref) < 1e-13


def test_scan_bound_for_decays_in_unit_interval(orc):
    rng = np.random.default_rng(30)
    S, E = 64, 50
    a = rng.uniform(1e-3, 1.0, (S, E))
    b = rng.standard_normal((S, E))
    h0 = rng.standard_normal(E)
    h, _ = orc.scan(a, b, h0)
    bound = np.abs(h0) + np.cumsum(np.abs(b), axis=0)
    assert np.all(np.abs(h) <= bound * (1 + 1e-12))


@pytest.mark.parametrize("splits", [[64, 11], [1] * 75, [32, 32, 11], [11, 64]])
def test_scan_chunk_split_invariance(orc, splits):
    rng = np.random.default_rng(40)
    S, E = 75, 33
    a = rng.uniform(0.2, 1.0, (S, E))
    b = rng.standard_normal((S, E))
    h0 = rng.standard_normal(E)
    h_ref, hS_ref = orc.scan(a, b, h0)
    parts, cur, r = [], h0, 0
    for n in splits:
        h, cur = orc.scan(a[r:r + n], b[r:r + n], cur)
        parts.append(h)
        r += n
    np.testing.assert_array_equal(np.concatenate(parts), h_ref)
    np.testing.assert_array_equal(cur, hS_ref)


def test_scan_superposition(orc):
    rng = np.random.default_rng(50)
    S, E = 30, 4
    a = rng.uniform(0.2, 1.0, (S, E))
    b1, b2 = rng.standard_normal((S, E)), rng.standard_normal((S, E))
    z1, z2 = rng.standard_normal(E), rng.standard_normal(E)
    h1, _ = orc.scan(a, b1, z1)
    h2, _ = orc.scan(a, b2, z2)
    h12, _ = orc.scan(a, b1 + 3 * b2, z1 + 3 * z2)
    assert rel_err(h12, h1 + 3 * h2) < 1e-13
    for S_small, E_small in itertools.product([1, 4], [1, 3]):
        hh, hs = orc.scan(np.ones((S_small, E_small)), np.zeros((S_small, E_small)), np.arange(E_small) + 1.0)
        np.testing.assert_array_equal(hs, np.arange(E_small) + 1.0)
