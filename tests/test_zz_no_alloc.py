"""GPU check of the allocation-free tiled scan (lrc_scan_prefill_static) against the tiled scan with a
caller's workspace (lrc_scan_prefill_ws), through the C ABI.

Both run the same tiles with the same arithmetic, so their outputs and final states must agree bit
for bit; both are also held to the FP32 tolerance of the float64 oracle on sampled state elements.
Two calls in a row, the second on a smaller batch, check that the fixed scratch is reused correctly
(the second call sees the first call's flags, from an older generation).  Inputs: decays a in
[0.5, 1] with 1% exactly 1, b ~ N(0, 1), random incoming states.
"""
import numpy as np
import pytest
import torch

from gpu_util import f64, require_gpu
from helpers import TOL_F32, rel_err

pytestmark = pytest.mark.gpu


def _inputs(seed, lens, D, N):
    g = torch.Generator(device="cuda").manual_seed(seed)
    R, P = sum(lens), len(lens)
    a = torch.rand((R, D, N), device="cuda", generator=g) * 0.5 + 0.5
    a[torch.rand((R, D, N), device="cuda", generator=g) < 0.01] = 1.0
    b = torch.randn((R, D, N), device="cuda", generator=g)
    s0 = torch.randn((P, D, N), device="cuda", generator=g)
    return a, b, s0


@pytest.mark.parametrize("lens,D,N", [([1413, 3587, 33, 64, 65, 0, 1], 512, 16), ([200, 7], 64, 16)])
def test_scan_static_matches_workspace_form(orc, lens, D, N):
    require_gpu()
    from linear_recurrence_chunked_amd import lrc

    for call in range(2):  # twice in a row on the same fixed scratch
        a, b, s0 = _inputs(77 + call + D, lens, D, N)
        h_ws, s_ws = torch.empty_like(a), s0.clone()
        ws = lrc.scan_workspace(len(lens), D, N, a.device)
        lrc.scan_prefill_ws(a, b, h_ws, s_ws, lens, ws)
        h_st, s_st = torch.full_like(a, float("nan")), s0.clone()
        lrc.scan_prefill_static(a, b, h_st, s_st, lens)
        torch.cuda.synchronize()
        assert lrc.scan_workspace_timeouts(ws) == 0
        assert torch.equal(h_ws, h_st), call
        assert torch.equal(s_ws, s_st), call
        # sampled state elements against the oracle, every prompt
        cols = np.arange(0, D * N, max(1, D * N // 96))
        ci = torch.as_tensor(cols, device=a.device)
        A, B, H, S0, S = (f64(t.view(t.shape[0], -1)[:, ci]) for t in (a, b, h_st, s0, s_st))
        r = 0
        for p, n in enumerate(lens):
            ref_h, ref_s = orc.scan(A[r:r + n], B[r:r + n], S0[p])
            if n:
                assert rel_err(H[r:r + n], ref_h) < TOL_F32, (call, p)
            assert rel_err(S[p], ref_s) < TOL_F32, (call, p)
            r += n
