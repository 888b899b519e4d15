"""tp_shard_mlp_noalloc: the MLP rank share with the library's static
scratch array instead of a caller workspace, called through the C ABI.  Its
outputs must equal tp_shard_mlp's (same kernels, so bit for bit) and the
fp64 oracle's within the bf16 bar, on calls in a row whose scratch needs
shrink, so leftovers of a larger call are in the array when a smaller one
runs."""
import ctypes

import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from megatron_tensor_layer_amd import datagen
from tests.common import normwise_err
from tests.gpu_util import empty, to_dev, to_host, torch

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _p(t):
    return ctypes.c_void_p(t.data_ptr())


def noalloc(X, Wg, Wu, Wd, H, P):
    I, D = X.shape
    F_local = Wg.shape[0]
    return tp.lib().tp_shard_mlp_noalloc(I, D, F_local, tp.TP_BF16, _p(X), _p(Wg), _p(Wu),
                                         _p(Wd), _p(H), _p(P), None)


@pytest.fixture(scope="module")
def shards():
    """Rank 3 of the Llama-3.1-70B-shaped MLP at TP=8 (D=8192, F_local=3584)."""
    D, F, t, r = 8192, 28672, 8, 3
    Wg, Wu, Wd = datagen.mlp_weights(D, F, "bf16", 21)
    host = datagen.mlp_rank_shards(Wg, Wu, Wd, t, r)
    yield dict(D=D, F_local=F // t, W=(Wg, Wu, Wd), t=t, r=r,
               dev=tuple(to_dev(a, "bf16") for a in host))
    torch().cuda.empty_cache()


def test_noalloc_matches_workspace_entry_point(orc, shards):
    """Calls in a row: 64 tokens (split-K gate/up and down, 14 MiB of
    scratch), then 32 (split-K gate/up, 5.4 MiB), then 9 (1.5 MiB), then 4
    (no scratch): each equal, bit for bit, to tp_shard_mlp with its own
    workspace, and to the oracle within 2e-2."""
    S = shards
    T = torch()
    assert tp.lib().tp_shard_mlp_noalloc_max_workspace() == 32 << 20
    for I in (64, 32, 9, 4):
        need = tp.mlp_workspace_bytes(I, S["D"], S["F_local"])
        assert need <= 32 << 20
        X = datagen.gaussian("X", (I, S["D"]), 1.0, "bf16", 300 + I)
        Xd = to_dev(X, "bf16")
        H0, P0 = empty((I, S["F_local"]), "bf16"), empty((I, S["D"]), "f32")
        tp.shard_mlp(Xd, *S["dev"], H0, P0)
        H1, P1 = empty((I, S["F_local"]), "bf16"), empty((I, S["D"]), "f32")
        print(f"noalloc call I={I} scratch={need}", flush=True)
        assert noalloc(Xd, *S["dev"], H1, P1) == 0
        T.cuda.synchronize()
        assert T.equal(H0, H1) and T.equal(P0, P1), I
        Href, Pref = orc.mlp_rank(X, *S["W"], S["t"], S["r"])
        assert normwise_err(to_host(H1), Href) <= TOL
        assert normwise_err(to_host(P1), Pref) <= TOL


def test_noalloc_rejects_sizes_beyond_its_array():
    """A call needing more scratch than the array holds (the unsharded
    Llama-shaped MLP at 512 tokens needs 32 MiB of partials and 8 KiB of
    counters) returns TP_ERR_WORKSPACE and
    launches nothing: the NaN canaries of H and P survive."""
    T = torch()
    I, D, F = 512, 8192, 28672
    assert tp.mlp_workspace_bytes(I, D, F) > 32 << 20
    X = T.zeros((I, D), dtype=T.bfloat16, device="cuda")
    Wg = T.zeros((F, D), dtype=T.bfloat16, device="cuda")
    Wd = T.zeros((D, F), dtype=T.bfloat16, device="cuda")
    H, P = empty((I, F), "bf16"), empty((I, D), "f32")
    assert noalloc(X, Wg, Wg, Wd, H, P) == 5  # TP_ERR_WORKSPACE
    with pytest.raises(tp.TPError, match="WORKSPACE"):
        tp.shard_mlp_noalloc(X, Wg, Wg, Wd, H, P)
    T.cuda.synchronize()
    assert T.isnan(H).all() and T.isnan(P).all()
