"""Pins for the oracle's depthwise causal short conv.

Source: "perf(mamba): prefill text prompts in multi-token chunks",
Implementation (a causal depthwise window that reaches back into K-1 stored
state rows; the next state keeps the final K-1 rows).  The pins: numpy's
library correlation on the concatenated window, one-hot taps that expose the
tap order, the state rule for chunks shorter than the window, and chunk-split
invariance.
"""
import numpy as np
import pytest

from helpers import rel_err


def _rand(rng, S, C, K):
    return rng.standard_normal((S, C)), rng.standard_normal((K - 1, C)), rng.normal(0, 0.5, (C, K))


@pytest.mark.parametrize("S,C,K", [(75, 64, 4), (1, 5, 4), (3, 7, 2), (10, 3, 1), (9, 4, 6)])
def test_conv_matches_numpy_correlate(orc, S, C, K):
    rng = np.random.default_rng(1)
    x, st, w = _rand(rng, S, C, K)
    y, st_out = orc.conv_rows(x, st, w)
    full = np.concatenate([st, x], axis=0)
    for c in range(C):
        ref = np.correlate(full[:, c], w[c], mode="valid")
        assert rel_err(y[:, c], ref) < 1e-14
    np.testing.assert_array_equal(st_out, full[S:])


def test_conv_one_hot_taps_expose_tap_order(orc):
    rng = np.random.default_rng(2)
    S, C, K = 12, 6, 4
    x, st, _ = _rand(rng, S, C, K)
    last = np.zeros((C, K)); last[:, K - 1] = 1.0
    y, _ = orc.conv_rows(x, st, last)
    np.testing.assert_array_equal(y, x)                       # tap K-1 is the current row
    first = np.zeros((C, K)); first[:, 0] = 1.0
    y, _ = orc.conv_rows(x, st, first)
    np.testing.assert_array_equal(y[:K - 1], st)              # tap 0 reaches into the state
    np.testing.assert_array_equal(y[K - 1:], x[:S - (K - 1)])


def test_conv_bias_and_linearity(orc):
    rng = np.random.default_rng(3)
    S, C, K = 20, 5, 4
    x1, s1, w = _rand(rng, S, C, K)
    x2, s2, _ = _rand(rng, S, C, K)
    bias = rng.standard_normal(C)
    y1, _ = orc.conv_rows(x1, s1, w)
    y2, _ = orc.conv_rows(x2, s2, w)
    y12, _ = orc.conv_rows(2.0 * x1 - x2, 2.0 * s1 - s2, w)
    assert rel_err(y12, 2.0 * y1 - y2) < 1e-13
    yb, _ = orc.conv_rows(x1, s1, w, bias)
    assert rel_err(yb, y1 + bias[None, :]) < 1e-14


@pytest.mark.parametrize("S", [0, 1, 2])
def test_conv_short_chunk_keeps_old_state_rows(orc, S):
    rng = np.random.default_rng(4)
    C, K = 3, 4
    x, st, w = _rand(rng, S, C, K)
    _, st_out = orc.conv_rows(x, st, w)
    np.testing.assert_array_equal(st_out, np.concatenate([st, x], axis=0)[S:S + K - 1])


@pytest.mark.parametrize("splits", [[64, 11], [1] * 75, [32, 32, 11], [2, 1, 72]])
def test_conv_chunk_split_invariance(orc, splits):
    rng = np.random.default_rng(5)
    S, C, K = 75, 16, 4
    x, st, w = _rand(rng, S, C, K)
    y_ref, st_ref = orc.conv_rows(x, st, w)
    ys, cur, r = [], st, 0
    for n in splits:
        y, cur = orc.conv_rows(x[r:r + n], cur, w)
        ys.append(y)
        r += n
    np.testing.assert_array_equal(np.concatenate(ys), y_ref)
    np.testing.assert_array_equal(cur, st_ref)
