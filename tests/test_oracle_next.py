"""Pins for the oracle's RWKV-4 time shift and its fused Mamba mixer rows.

Time shift -- "perf(rwkv): prefill text prompts in multi-token chunks",
Implementation: each row is mixed with the row before it, the first row with
the carried shift state; the next state is the last row.  Pins: the two one-hot mixes reproduce
the rows and the shifted rows exactly, a mix is the same affine combination
of those two, chunk splits carry the state exactly, an empty chunk keeps it.

Mamba mixer rows -- "perf(mamba): prefill text prompts in multi-token
chunks", Implementation (the scan h_t = a_t h_{t-1} + b_t between forming a,
b and reading h out), read as the selective state-space step a = exp(dt A),
b = dt B x, y = C.h + D x.  Pins: A = 0 reduces the scan to a cumulative sum;
a decay constant over rows gives the geometric closed form; brute force in
the product form on tiny inputs; the already pinned scan routine fed with a, b
formed from the definition; B = 0 isolates the skip term and the decayed
incoming state; chunk-split invariance; linearity in x from a zero state.
"""
import numpy as np
import pytest

from helpers import rel_err


# ----------------------------------------------------------------- time shift
def _ts_inputs(rng, S=20, C=7, M=3):
    return rng.standard_normal((S, C)), rng.standard_normal(C), rng.uniform(0, 1, (M, C))


def test_time_shift_one_hot_mixes_are_rows_and_shifted_rows(orc):
    rng = np.random.default_rng(90)
    x, st, _ = _ts_inputs(rng)
    C = x.shape[1]
    mix = np.stack([np.ones(C), np.zeros(C)])
    out, st_out = orc.time_shift(x, st, mix)
    np.testing.assert_array_equal(out[0], x)
    np.testing.assert_array_equal(out[1], np.concatenate([st[None], x[:-1]]))
    np.testing.assert_array_equal(st_out, x[-1])


def test_time_shift_mix_is_affine_between_the_one_hot_cases(orc):
    rng = np.random.default_rng(91)
    x, st, mix = _ts_inputs(rng)
    out, _ = orc.time_shift(x, st, mix)
    C = x.shape[1]
    ends, _ = orc.time_shift(x, st, np.stack([np.ones(C), np.zeros(C)]))
    for j in range(mix.shape[0]):
        ref = mix[j][None] * ends[0] + (1 - mix[j][None]) * ends[1]
        assert rel_err(out[j], ref) < 1e-15


@pytest.mark.parametrize("splits", [[64, 11], [1] * 75, [7, 0, 68]])
def test_time_shift_chunk_split_invariance(orc, splits):
    rng = np.random.default_rng(92)
    x, st, mix = _ts_inputs(rng, S=75, C=5)
    ref, ref_st = orc.time_shift(x, st, mix)
    parts, cur, r = [], st, 0
    for n in splits:
        o, cur = orc.time_shift(x[r:r + n], cur, mix)
        parts.append(o)
        r += n
    np.testing.assert_array_equal(np.concatenate(parts, axis=1), ref)
    np.testing.assert_array_equal(cur, ref_st)


def test_time_shift_empty_chunk_keeps_state(orc):
    rng = np.random.default_rng(93)
    _, st, mix = _ts_inputs(rng)
    out, st_out = orc.time_shift(np.zeros((0, st.size)), st, mix)
    assert out.shape == (mix.shape[0], 0, st.size)
    np.testing.assert_array_equal(st_out, st)


# ---------------------------------------------------------------- mamba mixer
def _mx_inputs(rng, S=30, Dm=6, N=4):
    x = rng.standard_normal((S, Dm))
    dt = rng.uniform(1e-3, 0.1, (S, Dm))
    A = -rng.uniform(1.0, 16.0, (Dm, N))
    B = rng.standard_normal((S, N))
    C = rng.standard_normal((S, N))
    D = rng.standard_normal(Dm)
    h0 = rng.standard_normal((Dm, N))
    return x, dt, A, B, C, D, h0


def test_mixer_without_decay_is_a_cumulative_sum(orc):
    rng = np.random.default_rng(94)
    x, dt, A, B, C, D, h0 = _mx_inputs(rng)
    A = np.zeros_like(A)
    y, hS = orc.mamba_mixer(x, dt, A, B, C, D, h0)
    b = dt[:, :, None] * B[:, None, :] * x[:, :, None]        # [S, Dm, N]
    h = h0[None] + np.cumsum(b, axis=0)
    ref = np.einsum("tn,tdn->td", C, h) + D[None] * x
    assert rel_err(y, ref) < 1e-12
    assert rel_err(hS, h[-1]) < 1e-12


def test_mixer_constant_decay_geometric_closed_form(orc):
    rng = np.random.default_rng(95)
    S = 25
    x, _, A, B, C, D, h0 = _mx_inputs(rng, S=S)
    dt = np.full_like(x, 0.07)
    y, hS = orc.mamba_mixer(x, dt, A, B, C, D, h0)
    a = np.exp(0.07 * A)                                        # [Dm, N], the same every row
    b = dt[:, :, None] * B[:, None, :] * x[:, :, None]
    for t in (0, 1, 9, S - 1):
        h = a ** (t + 1) * h0 + sum(a ** (t - i) * b[i] for i in range(t + 1))
        assert rel_err(y[t], np.einsum("n,dn->d", C[t], h) + D * x[t]) < 1e-12
    h = a ** S * h0 + sum(a ** (S - 1 - i) * b[i] for i in range(S))
    assert rel_err(hS, h) < 1e-12


def test_mixer_brute_force_product_form(orc):
    rng = np.random.default_rng(96)
    x, dt, A, B, C, D, h0 = _mx_inputs(rng, S=6, Dm=3, N=2)
    y, hS = orc.mamba_mixer(x, dt, A, B, C, D, h0)
    S, Dm, N = 6, 3, 2
    for t in range(S):
        for d in range(Dm):
            acc = D[d] * x[t, d]
            for n in range(N):
                decay = [np.exp(dt[i, d] * A[d, n]) for i in range(S)]
                h = np.prod(decay[:t + 1]) * h0[d, n]
                for i in range(t + 1):
                    h += np.prod(decay[i + 1:t + 1]) * dt[i, d] * B[i, n] * x[i, d]
                acc += C[t, n] * h
            assert abs(y[t, d] - acc) < 1e-12 * max(1.0, abs(acc))


def test_mixer_agrees_with_the_pinned_scan(orc):
    rng = np.random.default_rng(97)
    x, dt, A, B, C, D, h0 = _mx_inputs(rng, S=40, Dm=5, N=8)
    y, hS = orc.mamba_mixer(x, dt, A, B, C, D, h0)
    a = np.exp(dt[:, :, None] * A[None])
    b = dt[:, :, None] * B[:, None, :] * x[:, :, None]
    h, hs = orc.scan(a.reshape(40, -1), b.reshape(40, -1), h0.reshape(-1))
    ref = np.einsum("tn,tdn->td", C, h.reshape(40, 5, 8)) + D[None] * x
    assert rel_err(y, ref) < 1e-13
    assert rel_err(hS, hs.reshape(5, 8)) < 1e-13


def test_mixer_zero_input_weight_leaves_skip_and_decayed_state(orc):
    rng = np.random.default_rng(98)
    x, dt, A, B, C, D, h0 = _mx_inputs(rng)
    y, hS = orc.mamba_mixer(x, dt, A, np.zeros_like(B), C, D, h0)
    cum = np.cumsum(dt, axis=0)                                 # sum of dt over rows 0..t, per d
    h = np.exp(cum[:, :, None] * A[None]) * h0[None]
    ref = np.einsum("tn,tdn->td", C, h) + D[None] * x
    assert rel_err(y, ref) < 1e-12


@pytest.mark.parametrize("splits", [[64, 11], [7, 4, 64], [1] * 75])
def test_mixer_chunk_split_invariance(orc, splits):
    rng = np.random.default_rng(99)
    x, dt, A, B, C, D, h0 = _mx_inputs(rng, S=75, Dm=4, N=3)
    ref, ref_h = orc.mamba_mixer(x, dt, A, B, C, D, h0)
    parts, h, r = [], h0, 0
    for n in splits:
        y, h = orc.mamba_mixer(x[r:r + n], dt[r:r + n], A, B[r:r + n], C[r:r + n], D, h)
        parts.append(y)
        r += n
    np.testing.assert_array_equal(np.concatenate(parts), ref)
    np.testing.assert_array_equal(h, ref_h)


def test_mixer_linear_in_x_from_zero_state(orc):
    rng = np.random.default_rng(100)
    x1, dt, A, B, C, D, _ = _mx_inputs(rng)
    x2 = rng.standard_normal(x1.shape)
    z = np.zeros((x1.shape[1], A.shape[1]))
    y1, _ = orc.mamba_mixer(x1, dt, A, B, C, D, z)
    y2, _ = orc.mamba_mixer(x2, dt, A, B, C, D, z)
    y12, _ = orc.mamba_mixer(2 * x1 - 3 * x2, dt, A, B, C, D, z)
    assert rel_err(y12, 2 * y1 - 3 * y2) < 1e-13
