"""GPU parity of tp_residual_rmsnorm (residual update after a row-parallel
block's reduce, then the replicated RMSNorm) against the fp64 oracle.
Bars: normwise 1e-5 where every stored value is fp32, 2e-2 once bf16 is
involved (h or x stored in bf16)."""
import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from megatron_tensor_layer_amd import datagen
from tests.common import normwise_err
from tests.gpu_util import empty, to_dev, to_host, torch

pytestmark = pytest.mark.gpu

# (t, I, D, h dtype, x dtype or None, eps, with residual)
CASES = [
    (0, 5, 256, "f32", "f32", 1e-5, True),        # the norm alone (first block of a layer)
    (2, 4, 1536, "bf16", "bf16", 1e-6, True),     # Qwen2.5-1.5B TP=2 decode
    (8, 32, 8192, "bf16", "bf16", 1e-5, True),    # Llama-70B TP=8 decode 32
    (8, 512, 8192, "f32", "bf16", 1e-5, True),    # Llama-70B TP=8 prefill 512
    (3, 7, 264, "f32", "f32", 0.5, False),        # no residual, D/4 not a multiple of 64
    (1, 2, 32768, "bf16", "f32", 1e-5, True),     # largest D
    (5, 9, 8192, "f32", None, 0.0, True),         # residual update only
]


def _inputs(t, I, D, h_dt, x_dt, seed):
    P = datagen.gaussian("P", (t, I, D), 1.0, "f32", seed) if t else None
    R = datagen.gaussian("h", (I, D), 1.0, h_dt, seed)
    g = datagen.rmsnorm_gamma(D, seed, x_dt or "f32")
    return P, R, g


@pytest.mark.parametrize("t,I,D,h_dt,x_dt,eps,with_res", CASES)
def test_residual_rmsnorm(orc, t, I, D, h_dt, x_dt, eps, with_res):
    P, R, g = _inputs(t, I, D, h_dt, x_dt, 100 + t + I)
    if not with_res:
        R = None
    T = torch()
    h = empty((I, D), h_dt)
    x = empty((I, D), x_dt) if x_dt else None
    gd = to_dev(g, x_dt) if x_dt else None
    tp.residual_rmsnorm(to_dev(P, "f32") if P is not None else None,
                        to_dev(R, h_dt) if R is not None else None, h, gd, x, eps)
    T.cuda.synchronize()
    h_ref, x_ref = orc.residual_rmsnorm(P, R, g if x_dt else None, eps)
    tol_h = 1e-5 if h_dt == "f32" else 2e-2
    assert normwise_err(to_host(h), h_ref) <= tol_h
    if x_dt:
        tol_x = 1e-5 if (h_dt == "f32" and x_dt == "f32") else 2e-2
        assert normwise_err(to_host(x), x_ref) <= tol_x


def test_residual_rmsnorm_in_place_and_deterministic(orc):
    """h may be the residual buffer itself; repeated calls give the same bits."""
    t, I, D = 8, 32, 8192
    P, R, g = _inputs(t, I, D, "bf16", "bf16", 7)
    T = torch()
    Pd, gd = to_dev(P, "f32"), to_dev(g, "bf16")
    outs = []
    for _ in range(2):
        hd = to_dev(R, "bf16")
        x = empty((I, D), "bf16")
        tp.residual_rmsnorm(Pd, hd, hd, gd, x, 1e-5)
        outs.append((hd, x))
    T.cuda.synchronize()
    assert T.equal(outs[0][0], outs[1][0]) and T.equal(outs[0][1], outs[1][1])
    h_ref, x_ref = orc.residual_rmsnorm(P, R, g, 1e-5)
    assert normwise_err(to_host(outs[0][0]), h_ref) <= 2e-2
    assert normwise_err(to_host(outs[0][1]), x_ref) <= 2e-2


def test_residual_rmsnorm_errors_touch_nothing():
    T = torch()
    h = empty((4, 64), "f32")
    before = to_host(h).copy()
    with pytest.raises(tp.TPError, match="INVALID"):
        tp.residual_rmsnorm(None, to_dev(np.ones((4, 64), np.float32), "f32"), h,
                            to_dev(np.ones(64, np.float32), "f32"), h, 1e-5)  # x == h
    T.cuda.synchronize()
    assert np.array_equal(to_host(h), before, equal_nan=True)


@pytest.mark.parametrize("t,I,D,h_dt", [(8, 512, 8192, "bf16"), (2, 64, 1536, "f32"),
                                        (4, 4, 264, "bf16")])
def test_sequence_parallel_reduce_scatter_norm_allgather(orc, t, I, D, h_dt):
    """Each rank's reduce-scatter + norm on its I/t rows, x written into its
    rows of one [I, D] buffer (the all-gather): the same bits as the
    all-reduce form, and the oracle's values."""
    P, R, g = _inputs(t, I, D, h_dt, "bf16", 900 + t)
    T = torch()
    Pd, gd = to_dev(P, "f32"), to_dev(g, "bf16")
    Is = I // t
    h_sp = to_dev(R, h_dt)
    x_sp = empty((I, D), "bf16")
    for r in range(t):
        tp.reduce_scatter_rmsnorm(Pd, r, h_sp[r * Is:(r + 1) * Is], h_sp[r * Is:(r + 1) * Is],
                                  gd, x_sp[r * Is:(r + 1) * Is], 1e-5)
    h_ar = to_dev(R, h_dt)
    x_ar = empty((I, D), "bf16")
    tp.residual_rmsnorm(Pd, h_ar, h_ar, gd, x_ar, 1e-5)
    T.cuda.synchronize()
    assert T.equal(h_sp, h_ar) and T.equal(x_sp, x_ar)
    h_ref, x_ref = orc.residual_rmsnorm(P, R, g, 1e-5)
    assert normwise_err(to_host(h_sp), h_ref) <= (1e-5 if h_dt == "f32" else 2e-2)
    assert normwise_err(to_host(x_sp), x_ref) <= 2e-2

