"""GPU parity of the tiled selective-scan driver (lrc_scan_prefill_ws).

Reading ("perf(mamba): prefill text prompts in multi-token chunks",
Implementation): every 64-row chunk is the doubling scan with the carried state
applied last.  The tiled driver runs each (chunk, block of 128 state elements)
in its own workgroup and takes the carry from the previous chunk's last h row;
its chunk arithmetic and carry values are those of the long-lived driver
(lrc_scan_prefill), so the two must agree bit for bit, and both must be within
the FP32 tolerance of the float64 oracle.  Inputs: decays a in [0.5, 1] with
1% exactly 1, b ~ N(0, 1), random incoming states.
"""
import numpy as np
import pytest
import torch

from gpu_util import f64, require_gpu, to_dev
from helpers import TOL_F32, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    require_gpu()
    from linear_recurrence_chunked_amd import lrc

    return lrc


def _case(seed, lens, D, N):
    rng = np.random.default_rng(seed)
    R, P = sum(lens), len(lens)
    a = rng.uniform(0.5, 1.0, (R, D, N))
    a[rng.random((R, D, N)) < 0.01] = 1.0
    b = rng.standard_normal((R, D, N))
    h0 = rng.standard_normal((P, D, N))
    return a, b, h0


def _edge_lens():
    rng = np.random.default_rng(300)
    ls = rng.integers(0, 131, size=256)
    ls[[3, 100, 255]] = 0
    return [int(n) for n in ls]


@pytest.mark.parametrize("lens,D,N", [
    ([130, 1, 0, 75, 64, 65, 200, 3], 64, 16),   # ragged, 4 blocks of 256
    ([300, 129, 64], 20, 16),                    # 320 elements: a partial block
    ([77], 5, 3),                                # D*N not a multiple of 4: the long-lived kernel
    ([0, 0, 5], 8, 4),                           # prompts without rows
    (_edge_lens(), 64, 16),                      # 256 prompts
])
def test_tiled_equals_long_lived_and_oracle(L, orc, lens, D, N):
    a, b, h0 = _case(700 + D + N + len(lens), lens, D, N)
    P = len(lens)
    ta, tb = (to_dev(torch.from_numpy(x).float()) for x in (a, b))
    th0 = to_dev(torch.from_numpy(h0).float())
    h1, st1 = torch.empty_like(ta), th0.clone()
    L.scan_prefill(ta, tb, h1, st1, lens)
    ws = torch.zeros(L.scan_workspace_size(P, D, N) + 1000, dtype=torch.uint8, device="cuda")  # larger is fine
    h2 = torch.empty_like(ta)
    for _ in range(3):  # one workspace, a new generation every call
        st2 = th0.clone()
        h2.fill_(float("nan"))
        L.scan_prefill_ws(ta, tb, h2, st2, lens, ws)
        torch.cuda.synchronize()
        assert torch.equal(h1, h2) and torch.equal(st1, st2)
    assert L.scan_workspace_timeouts(ws) == 0
    off = np.concatenate([[0], np.cumsum(lens)]).astype(int)
    for p in range(P):
        sl = slice(off[p], off[p + 1])
        if not lens[p]:
            assert torch.equal(st2[p], th0[p])
            continue
        E = D * N
        rh, rs = orc.scan(a[sl].reshape(lens[p], E), b[sl].reshape(lens[p], E), h0[p].reshape(E))
        assert rel_err(f64(h2[sl]).reshape(lens[p], E), rh) < TOL_F32
        assert rel_err(f64(st2[p]).reshape(E), rs) < TOL_F32


def test_tiled_mixed_prefill_full_size_equals_long_lived(L):
    """The 16 mixed prompt lengths at 5120 x 16 state elements (320 blocks): bit for bit."""
    from linear_recurrence_chunked_amd import inputs

    lens = inputs.mixed_lengths()
    m = inputs.mixed_mamba(lens, torch.device("cuda"), with_conv=False)
    a, b = m["a"].view(-1, 5120, 16), m["b"].view(-1, 5120, 16)
    P = len(lens)
    st0 = torch.randn((P, 5120, 16), device="cuda", generator=torch.Generator("cuda").manual_seed(5))
    h1, st1 = torch.empty_like(a), st0.clone()
    L.scan_prefill(a, b, h1, st1, lens)
    ws = L.scan_workspace(P, 5120, 16, "cuda")
    h2, st2 = torch.empty_like(a), st0.clone()
    L.scan_prefill_ws(a, b, h2, st2, lens, ws)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2) and torch.equal(st1, st2)
    assert L.scan_workspace_timeouts(ws) == 0


def test_tiled_two_streams_at_once(L):
    """Two tiled scans with their own workspaces on two streams at the same time: each chain's
    hand-overs stay within its own call, and both equal the long-lived driver bit for bit."""
    lens_a, lens_b = [700, 3, 129, 64, 0, 1000], [1, 517, 256, 2000]
    D, N = 256, 16
    outs = []
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    cases = []
    for seed, lens in ((41, lens_a), (42, lens_b)):
        a, b, h0 = _case(seed, lens, D, N)
        ta, tb = (to_dev(torch.from_numpy(x).float()) for x in (a, b))
        th0 = to_dev(torch.from_numpy(h0).float())
        ref_h, ref_s = torch.empty_like(ta), th0.clone()
        L.scan_prefill(ta, tb, ref_h, ref_s, lens)
        cases.append((lens, ta, tb, th0, ref_h, ref_s, L.scan_workspace(len(lens), D, N, "cuda")))
    torch.cuda.synchronize()
    for _ in range(3):
        for (lens, ta, tb, th0, ref_h, ref_s, ws), st in zip(cases, (s1, s2)):
            st.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(st):
                h, s = torch.empty_like(ta), th0.clone()
                L.scan_prefill_ws(ta, tb, h, s, lens, ws)
            outs.append((h, s, ref_h, ref_s, ws))
        torch.cuda.synchronize()
    for h, s, ref_h, ref_s, ws in outs:
        assert torch.equal(h, ref_h) and torch.equal(s, ref_s)
        assert L.scan_workspace_timeouts(ws) == 0


def test_tiled_random_shapes_equal_long_lived(L):
    """Seeded random batches (1-64 prompts of 0-700 rows, some exactly on chunk boundaries; 4-2048 state
    elements, multiples of 4, so the tiled form runs): bit for bit the long-lived driver, no timeouts."""
    rng = np.random.default_rng(2024)
    for case in range(24):
        P = int(rng.integers(1, 65))
        lens = [int(x) for x in rng.integers(0, 701, size=P)]
        for i in rng.choice(P, size=min(P, 3), replace=False):
            lens[i] = int(rng.choice([0, 1, 63, 64, 65, 128]))
        E = 4 * int(rng.integers(1, 513))
        D = E // 4 if E % 16 else E // 16
        N = E // D
        a, b, h0 = _case(3000 + case, lens, D, N)
        ta, tb = (to_dev(torch.from_numpy(x).float()) for x in (a, b))
        th0 = to_dev(torch.from_numpy(h0).float())
        h1, s1 = torch.empty_like(ta), th0.clone()
        L.scan_prefill(ta, tb, h1, s1, lens)
        ws = L.scan_workspace(P, D, N, "cuda")
        h2, s2 = torch.empty_like(ta), th0.clone()
        L.scan_prefill_ws(ta, tb, h2, s2, lens, ws)
        torch.cuda.synchronize()
        assert torch.equal(h1, h2) and torch.equal(s1, s2), (case, P, E)
        assert L.scan_workspace_timeouts(ws) == 0, (case, P, E)
