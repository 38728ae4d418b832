"""Helpers shared by the GPU parity tests (conversions and the tolerance rule)."""
import numpy as np
import pytest
import torch

ON_GPU = torch.cuda.is_available()


def need_gpu():
    if not ON_GPU:
        pytest.skip("needs a GPU")


def u64(t: torch.Tensor) -> np.ndarray:
    """Device uint64 tensor -> numpy uint64 (through an int64 view)."""
    return t.view(torch.int64).cpu().numpy().view(np.uint64)


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def rel_err(x, ref) -> float:
    """max |x - ref| / max |ref| over one tensor (the parity tolerance rule)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(x - ref)) / (den if den > 0 else 1.0))


def rel_err_rows(x, ref, row: int) -> float:
    """The tolerance rule per row of `row` trailing elements (one (node, head) output row):
    max over rows of max |x - ref| / max |ref| within the row.  A tensor-wide denominator
    would let a row of small outputs (e.g. a long prefix's average) hide behind a row of
    large ones (a lone node's own value); all-zero reference rows must be matched exactly
    up to 1e-30."""
    x = np.asarray(x, dtype=np.float64).reshape(-1, row)
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, row)
    den = np.max(np.abs(ref), axis=1)
    num = np.max(np.abs(x - ref), axis=1)
    zero = den == 0
    assert np.all(num[zero] <= 1e-30), "rows the reference leaves at zero are not zero"
    if np.all(zero):
        return 0.0
    return float(np.max(num[~zero] / den[~zero]))


def lse_err(x, ref) -> float:
    """|x - ref| / max(1, |ref|), -inf must match -inf."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(x), ninf), "-inf pattern differs"
    if np.all(ninf):
        return 0.0
    return float(np.max(np.abs(x[~ninf] - ref[~ninf]) / np.maximum(1.0, np.abs(ref[~ninf]))))


TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
