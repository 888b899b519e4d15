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


# Diagnostic bars: the device against the oracle's bf16-rounded intermediates
# (oracle.mlp_rank_bf16h and oracle.bf16_round), where only fp32 accumulation
# and the rounding decisions it flips remain.
# normwise, fp32 results computed from bf16 intermediates.  Observed: 1e-7
# where no H element flips (the few-token kernel at one token), up to 3.5e-4
# where an H element of the largest magnitudes lands one bf16 step from the
# oracle's rounding (the step, 2^-8 of that element, times its W_down row).
# Dropping two K terms of a row moves it by about 1e-2.
DIAG_TOL = 1e-3
DIAG_BF16_FLIPS = 0.02   # largest fraction of bf16 outputs one rounding step off
BF16_STEP = 2.0 ** -8    # one bf16 step at the top of the range, normwise


def bf16_flips(got, ref_bf16) -> float:
    """Fraction of elements of a bf16 result that differ from the oracle's
    bf16-rounded value (an fp32 sum that lands on the other side of a
    rounding boundary flips one element by one step)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref_bf16, dtype=np.float64)
    assert got.shape == ref.shape
    return float(np.count_nonzero(got != ref)) / max(1, got.size)
