"""Pins for the oracle's Gated DeltaNet token loop and its triangular inverse.

Source: "perf(qwen3_5): prefill text prompts in multi-token chunks",
Implementation.  The page states the chunk form
  (I + A) U = beta V - diag(beta Gamma) K S_0,  A_ij = beta_i e^{gamma_i - gamma_j} k_i.k_j (j < i)
  O   = diag(Gamma) Q S_0 + (e^{gamma_t - gamma_i} q_t.k_i)_{i <= t} U
  S_S = e^{gamma_S} S_0 + (K * e^{gamma_S - gamma})^T U
with gamma the inclusive cumulative sum of g and Gamma = e^gamma.  The oracle
walks one token at a time (the form's one-row case); these tests pin it
  * to the chunk form evaluated in float64 with numpy's dense solver, for
    several chunk splits (64 + 11, 7 + 4, one chunk);
  * to the delta rule's exact-recall property with orthonormal keys;
  * to the beta = 0 and single-row special cases;
  * to the value-head -> key-head map (consecutive value heads share a key head);
and pin the forward-substitution inverse to numpy's dense inverse on nearly
parallel keys and beta close to 1, the case the page itself checks its solve on.
"""
import numpy as np
import pytest

from helpers import rel_err


def _inputs(rng, S, Hk, Hv, dk, dv, g_scale=0.5):
    q = rng.standard_normal((S, Hk, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((S, Hk, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((S, Hv, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((S, Hv))))
    g = -np.logaddexp(0.0, rng.standard_normal((S, Hv))) * g_scale
    S0 = rng.normal(0.0, 0.1, (Hv, dk, dv))
    return q, k, v, beta, g, S0


def chunk_form(q, k, v, beta, g, S0):
    """The page's chunk form in float64 (numpy dense solve for I + A)."""
    S, Hk, dk = k.shape
    Hv, dv = v.shape[1], v.shape[2]
    grp = Hv // Hk
    o = np.zeros((S, Hv, dv))
    SS = np.zeros((Hv, dk, dv))
    lower = np.tril(np.ones((S, S), dtype=bool), -1)
    causal = np.tril(np.ones((S, S), dtype=bool))
    for h in range(Hv):
        K, Q, V, b = k[:, h // grp], q[:, h // grp], v[:, h], beta[:, h]
        gam = np.cumsum(g[:, h])
        Gam = np.exp(gam)
        diff = gam[:, None] - gam[None, :]
        A = np.where(lower, b[:, None] * np.exp(np.where(lower, diff, 0.0)) * (K @ K.T), 0.0)
        rhs = b[:, None] * V - (b * Gam)[:, None] * (K @ S0[h])
        U = np.linalg.solve(np.eye(S) + A, rhs)
        P = np.where(causal, np.exp(np.where(causal, diff, 0.0)) * (Q @ K.T), 0.0)
        o[:, h] = Gam[:, None] * (Q @ S0[h]) + P @ U
        dec = np.exp(np.minimum(gam[-1] - gam, 0.0))
        SS[h] = np.exp(gam[-1]) * S0[h] + (K * dec[:, None]).T @ U
    return o, SS


@pytest.mark.parametrize("splits", [[64, 11], [7, 4], [75], [11, 64], [1, 1, 1, 8]])
def test_gdn_token_loop_equals_page_chunk_form(orc, splits):
    rng = np.random.default_rng(70)
    S = sum(splits)
    q, k, v, beta, g, S0 = _inputs(rng, S, 2, 4, 16, 12)
    o_ref, S_ref = orc.gdn(q, k, v, beta, g, S0)
    parts, st, r = [], S0, 0
    for n in splits:
        o, st = chunk_form(q[r:r + n], k[r:r + n], v[r:r + n], beta[r:r + n], g[r:r + n], st)
        parts.append(o)
        r += n
    assert rel_err(np.concatenate(parts), o_ref) < 1e-12
    assert rel_err(st, S_ref) < 1e-12


def test_gdn_exact_recall_with_orthonormal_keys(orc):
    rng = np.random.default_rng(71)
    S, dk, dv = 16, 32, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:S].reshape(S, 1, dk)
    v = rng.standard_normal((S, 1, dv))
    S0 = rng.standard_normal((1, dk, dv))
    _, SS = orc.gdn(keys, keys, v, np.ones((S, 1)), np.zeros((S, 1)), S0)
    recall = np.einsum("sd,dv->sv", keys[:, 0], SS[0])
    assert np.max(np.abs(recall - v[:, 0])) < 1e-12
    # unwritten directions keep what S0 held
    free = Qm[S:]
    assert np.max(np.abs(free @ SS[0] - free @ S0[0])) < 1e-12


def test_gdn_repeated_key_overwrites(orc):
    rng = np.random.default_rng(72)
    S, dk, dv = 10, 8, 5
    key = rng.standard_normal(dk); key /= np.linalg.norm(key)
    k = np.tile(key, (S, 1, 1))
    v = rng.standard_normal((S, 1, dv))
    o, SS = orc.gdn(k, k, v, np.ones((S, 1)), np.zeros((S, 1)), rng.standard_normal((1, dk, dv)))
    assert np.max(np.abs(o[:, 0] - v[:, 0])) < 1e-12          # q = k reads back the last value
    assert np.max(np.abs(key @ SS[0] - v[-1, 0])) < 1e-12


def test_gdn_zero_beta_only_decays(orc):
    rng = np.random.default_rng(73)
    q, k, v, _, g, S0 = _inputs(rng, 20, 2, 2, 8, 6)
    beta = np.zeros((20, 2))
    o, SS = orc.gdn(q, k, v, beta, g, S0)
    gam = np.cumsum(g, axis=0)
    for h in range(2):
        ref = np.exp(gam[:, h])[:, None] * (q[:, h] @ S0[h])
        assert rel_err(o[:, h], ref) < 1e-13
        assert rel_err(SS[h], np.exp(gam[-1, h]) * S0[h]) < 1e-13


def test_gdn_single_row_householder_form(orc):
    rng = np.random.default_rng(74)
    q, k, v, beta, g, S0 = _inputs(rng, 1, 1, 1, 8, 6)
    o, SS = orc.gdn(q, k, v, beta, g, S0)
    kk = k[0, 0]
    ref = np.exp(g[0, 0]) * (np.eye(8) - beta[0, 0] * np.outer(kk, kk)) @ S0[0] + beta[0, 0] * np.outer(kk, v[0, 0])
    assert rel_err(SS[0], ref) < 1e-14
    assert rel_err(o[0, 0], q[0, 0] @ ref) < 1e-14


def test_gdn_value_heads_share_consecutive_key_heads(orc):
    rng = np.random.default_rng(75)
    q, k, v, beta, g, S0 = _inputs(rng, 12, 2, 6, 8, 4)
    o, SS = orc.gdn(q, k, v, beta, g, S0)
    rep = np.repeat(np.arange(2), 3)                             # value head h -> key head h // 3
    o2, SS2 = orc.gdn(q[:, rep], k[:, rep], v, beta, g, S0)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(SS, SS2)


def test_gdn_finite_under_extreme_decay(orc):
    rng = np.random.default_rng(76)
    S = 300
    q, k, v, beta, _, S0 = _inputs(rng, S, 1, 2, 8, 8)
    g = np.stack([np.full(S, -8.0), np.full(S, -1e-3)], axis=1)
    o, SS = orc.gdn(q, k, v, beta, g, S0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(SS))
    # with g = -8 per row the incoming state is gone after one row
    o_fresh, _ = orc.gdn(q, k, v, beta, g, np.zeros_like(S0))
    assert rel_err(o[5:, 0], o_fresh[5:, 0]) < 1e-12


def _near_parallel_A(rng, n, dk=64, beta=0.99, par=(0, 64)):
    k = rng.standard_normal((n, dk))
    kbar = rng.standard_normal(dk)
    lo, hi = par
    k[lo:hi] = kbar + 1e-3 * rng.standard_normal((hi - lo, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    g = -np.logaddexp(0.0, rng.standard_normal(n)) * 0.01
    gam = np.cumsum(g)
    A = beta * np.exp(np.tril(gam[:, None] - gam[None, :], -1)) * (k @ k.T)
    return np.tril(A, -1)


@pytest.mark.parametrize("n,par", [(64, (0, 64)), (64, (24, 40)), (40, (0, 32)), (8, (0, 8)), (1, (0, 1))])
def test_unit_lower_inverse_matches_numpy(orc, n, par):
    rng = np.random.default_rng(77 + n)
    A = _near_parallel_A(rng, n, par=par)
    T = orc.unit_lower_inverse(A)
    ref = np.linalg.inv(np.eye(n) + A)
    assert rel_err(T, ref) < 1e-9
    assert np.max(np.abs(T @ (np.eye(n) + A) - np.eye(n))) < 1e-9 * max(1.0, np.max(np.abs(T)))
    assert np.all(np.triu(T, 1) == 0.0) and np.all(np.diag(T) == 1.0)


def test_unit_lower_inverse_ignores_upper_part_and_batches(orc):
    rng = np.random.default_rng(78)
    A = rng.standard_normal((3, 10, 10)) * 0.3
    T = orc.unit_lower_inverse(A)
    for b in range(3):
        ref = np.linalg.inv(np.eye(10) + np.tril(A[b], -1))
        assert rel_err(T[b], ref) < 1e-12
