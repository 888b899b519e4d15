"""GPU parity of tp_partial_reduce: the fp64 oracle sum within fp32
rounding, and the documented rank-order fp32 summation bit for bit."""
import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from megatron_tensor_layer_amd import datagen
from tests.common import normwise_err
from tests.gpu_util import empty, to_dev, to_host, torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("t,n", [(1, 8), (2, 4104), (8, 32 * 8192), (8, 512 * 8192), (3, 1000)])
def test_reduce(orc, t, n):
    P = datagen.gaussian("A", (t, n), 1.0, "f32", t * 1000 + n % 997)
    Pd = to_dev(P, "f32")
    Y = empty((n,), "f32")
    Yb = empty((n,), "bf16")
    tp.partial_reduce(Pd, Y)
    tp.partial_reduce(Pd, Yb)
    torch().cuda.synchronize()
    ref = orc.reduce(P)
    y = to_host(Y)
    assert normwise_err(y, ref) <= 1e-6
    # rank order 0..t-1 in fp32, bit for bit
    s = P[0].copy()
    for r in range(1, t):
        s += P[r]
    assert np.array_equal(y.astype(np.float32), s)
    # bf16 output: the fp32 sum rounded to nearest-even
    u = s.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32) << 16
    assert np.array_equal(to_host(Yb).astype(np.float32).view(np.uint32), rne.astype(np.uint32))
    assert normwise_err(to_host(Yb), ref) <= 2.0 ** -8
