"""Shared test helpers (error measures); no layer arithmetic lives here."""
import numpy as np


def normwise_err(got, ref) -> float:
    """max |got - ref| / max |ref| over all elements (normwise, infinity norm)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.max(np.abs(ref))
    num = np.max(np.abs(got - ref))
    if den == 0.0:
        return float(num)
    return float(num / den)
