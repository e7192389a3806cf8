"""Shared test helpers: tolerance metric and chunk splitting (no method arithmetic)."""
import numpy as np

TOL_F32 = 1e-4   # fp32 paths: max-abs error relative to the tensor's max-abs value
TOL_BF16 = 2e-2  # bf16-input Gated DeltaNet and bf16 conv, fp32 accumulation


def rel_err(got, ref):
    """max |got - ref| / max |ref|; the absolute max |got - ref| when ref is all zero."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 0.0
    scale = float(np.max(np.abs(ref)))
    diff = float(np.max(np.abs(got - ref)))
    return diff if scale == 0.0 else diff / scale


def split_offsets(splits):
    off = [0]
    for s in splits:
        off.append(off[-1] + s)
    return off
