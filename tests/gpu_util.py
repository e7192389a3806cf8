"""Helpers for the GPU parity tests (marshalling and comparison only)."""
import numpy as np
import torch

DEV = "cuda:0"


def to_dev(t: torch.Tensor) -> torch.Tensor:
    return t.to(DEV).contiguous()


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact upcast of the tensor's values (fp32 or bf16) to float64 on the host."""
    return t.detach().to("cpu").to(torch.float64).numpy()


def chunks(total: int, splits):
    r = 0
    for n in splits:
        yield r, n
        r += n
    assert r == total


def require_gpu():
    import pytest

    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
