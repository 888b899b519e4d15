"""GPU parity of tp_shard_mlp against the fp64 oracle.

Tolerance (normwise, max|gpu - ref| / max|ref|): 2e-2 for bf16 inputs with
fp32 accumulation, 1e-5 for fp32.  The oracle takes the FULL weights and the
rank index; the GPU gets the rank's contiguous shard buffers."""
import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from megatron_tensor_layer_amd import datagen
from tests.common import normwise_err
from tests.gpu_util import empty, to_dev, to_host, torch

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-5}


def gpu_mlp(X, Wg_r, Wu_r, Wd_r, dtype):
    I, D = X.shape
    F_local = Wg_r.shape[0]
    Xd, Gd, Ud, Dd = (to_dev(a, dtype) for a in (X, Wg_r, Wu_r, Wd_r))
    H = empty((I, F_local), dtype)
    P = empty((I, D), "f32")
    tp.shard_mlp(Xd, Gd, Ud, Dd, H, P)
    torch().cuda.synchronize()
    return H, P


# (I, D, F_local, t, r, dtype): few-token kernel (I <= 8), MFMA kernels (I > 8),
# weight-streaming MFMA kernel (9..64 tokens), ragged K tiles and steps
# (D = 264, 520, 1000), ragged F tiles (F_local = 200, 328, 136, 24, 1000),
# long K (lanes holding 4 and 8 chunks), the fp32 path in 8- and 4-token launches
SMALL = [
    (1, 264, 200, 2, 1, "bf16"), (2, 264, 200, 2, 0, "bf16"), (3, 136, 72, 1, 0, "bf16"),
    (5, 520, 136, 4, 3, "bf16"), (8, 264, 200, 2, 1, "bf16"), (4, 16384, 64, 1, 0, "bf16"),
    (1, 24576, 32, 1, 0, "bf16"), (6, 24576, 32, 1, 0, "bf16"),
    (9, 264, 200, 2, 1, "bf16"), (17, 520, 328, 1, 0, "bf16"), (40, 264, 200, 2, 0, "bf16"),
    (64, 136, 72, 2, 1, "bf16"), (65, 264, 200, 1, 0, "bf16"), (130, 520, 136, 2, 1, "bf16"),
    (257, 264, 200, 2, 1, "bf16"), (33, 72, 24, 2, 1, "bf16"), (48, 1000, 1000, 1, 0, "bf16"),
    (16, 2048, 4096, 1, 0, "bf16"),
    # one M block with K a multiple of 2048: the GEMM starts each W tile's K
    # range at a different stage (and wraps), split K on both
    (80, 2048, 200, 2, 1, "bf16"), (100, 4096, 136, 1, 0, "bf16"),
    # one gate/up tile split 16 ways: the finishing workgroup sums its items
    # over four rounds of 4 splits
    (70, 8192, 64, 1, 0, "bf16"),
    # whole-K row blocks (9..32 tokens, 128..256 workgroups): gate/up with a
    # ragged last K slice, down with a ragged last row block, a full grid
    (20, 1040, 2064, 1, 0, "bf16"), (9, 4104, 1032, 1, 0, "bf16"), (32, 1024, 4096, 1, 0, "bf16"),
    (4, 256, 512, 2, 0, "f32"), (11, 264, 200, 2, 1, "f32"), (3, 9216, 64, 1, 0, "f32"),
]


@pytest.mark.parametrize("I,D,F_local,t,r,dtype", SMALL,
                         ids=[f"I{c[0]}-D{c[1]}-F{c[2]}-t{c[3]}r{c[4]}-{c[5]}" for c in SMALL])
def test_mlp_small_shapes(orc, I, D, F_local, t, r, dtype):
    pool = I * 7 + D + F_local
    X = datagen.gaussian("X", (I, D), 1.0, dtype, pool)
    Wg, Wu, Wd = datagen.mlp_weights(D, F_local * t, dtype, pool)
    H, P = gpu_mlp(X, *datagen.mlp_rank_shards(Wg, Wu, Wd, t, r), dtype)
    Href, Pref = orc.mlp_rank(X, Wg, Wu, Wd, t, r)
    assert normwise_err(to_host(H), Href) <= TOL[dtype]
    assert normwise_err(to_host(P), Pref) <= TOL[dtype]


def test_tiny_f32_tp2_sum_of_partials(orc):
    """Tiny Megatron SwiGLU MLP, TP=2 on one GPU: D=256, F=1024, 4 tokens, fp32.
    The reduced rank partials equal the unsharded layer (oracle) and the GPU's
    own t=1 run."""
    D, F, t, I = 256, 1024, 2, 4
    X = datagen.gaussian("X", (I, D), 1.0, "f32")
    Wg, Wu, Wd = datagen.mlp_weights(D, F, "f32")
    T = torch()
    parts = T.empty((t, I, D), dtype=T.float32, device="cuda")
    for r in range(t):
        _, P = gpu_mlp(X, *datagen.mlp_rank_shards(Wg, Wu, Wd, t, r), "f32")
        parts[r].copy_(P)
    Y = empty((I, D), "f32")
    tp.partial_reduce(parts, Y)
    _, Y1 = gpu_mlp(X, Wg, Wu, Wd, "f32")
    T.cuda.synchronize()
    _, Yref = orc.mlp_full(X, Wg, Wu, Wd)
    assert normwise_err(to_host(Y), Yref) <= 1e-5
    assert normwise_err(to_host(Y1), Yref) <= 1e-5
    assert normwise_err(to_host(Y), to_host(Y1)) <= 1e-5


@pytest.mark.parametrize("I", [1, 8, 64])
def test_qwen_mlp_tp2(orc, I):
    """Qwen2.5-1.5B-shaped MLP at TP=2 (D=1536, F=8960): both ranks, reduce."""
    D, F, t = 1536, 8960, 2
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 100 + I)
    Wg, Wu, Wd = datagen.mlp_weights(D, F, "bf16", 100)
    T = torch()
    parts = T.empty((t, I, D), dtype=T.float32, device="cuda")
    for r in range(t):
        H, P = gpu_mlp(X, *datagen.mlp_rank_shards(Wg, Wu, Wd, t, r), "bf16")
        parts[r].copy_(P)
        if r == 1:
            Href, Pref = orc.mlp_rank(X, Wg, Wu, Wd, t, r)
            assert normwise_err(to_host(H), Href) <= TOL["bf16"]
            assert normwise_err(to_host(P), Pref) <= TOL["bf16"]
    Y = empty((I, D), "f32")
    tp.partial_reduce(parts, Y)
    T.cuda.synchronize()
    _, Yref = orc.mlp_full(X, Wg, Wu, Wd)
    assert normwise_err(to_host(Y), Yref) <= TOL["bf16"]


# ---------------------------------------------------------------- Llama-70B
@pytest.fixture(scope="module")
def llama_mlp():
    """Full Llama-3.1-70B-shaped MLP weights (D=8192, F=28672), host fp32 and
    fp64 copies, and the 8 TP rank shards resident on the GPU."""
    D, F, t = 8192, 28672, 8
    Wg, Wu, Wd = datagen.mlp_weights(D, F, "bf16", 7)
    shards = [tuple(to_dev(a, "bf16") for a in datagen.mlp_rank_shards(Wg, Wu, Wd, t, r))
              for r in range(t)]
    W64 = tuple(a.astype(np.float64) for a in (Wg, Wu, Wd))
    yield dict(D=D, F=F, t=t, W=(Wg, Wu, Wd), W64=W64, shards=shards)
    del shards
    torch().cuda.empty_cache()


def sample_rows(I):
    return sorted({0, I // 2, I - 1})


@pytest.mark.parametrize("I", [1, 6, 16, 32, 64, 256])
def test_llama_mlp_decode_tp8(orc, llama_mlp, I):
    """Llama-3.1-70B-shaped MLP, all 8 TP=8 rank shares on one GPU, decode I tokens;
    sampled token rows against the oracle (every row depends only on its own
    input row)."""
    L = llama_mlp
    D, F_local, t = L["D"], L["F"] // L["t"], L["t"]
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 200 + I)
    Xd = to_dev(X, "bf16")
    T = torch()
    parts = T.empty((t, I, D), dtype=T.float32, device="cuda")
    Hs = []
    for r in range(t):
        H = empty((I, F_local), "bf16")
        tp.shard_mlp(Xd, *L["shards"][r], H, parts[r])
        Hs.append(H)
    Y = empty((I, D), "f32")
    tp.partial_reduce(parts, Y)
    T.cuda.synchronize()
    rows = sample_rows(I)
    _, Yref = orc.mlp_full(X, *L["W64"], rows=rows)
    assert normwise_err(to_host(Y)[rows], Yref) <= TOL["bf16"]
    for r in (0, t - 1):
        Href, Pref = orc.mlp_rank(X, *L["W64"], t, r, rows=rows)
        assert normwise_err(to_host(Hs[r])[rows], Href) <= TOL["bf16"]
        assert normwise_err(to_host(parts[r])[rows], Pref) <= TOL["bf16"]
    # no canary survives anywhere in the outputs
    assert not T.isnan(Y).any() and all(not T.isnan(h).any() for h in Hs)


def test_llama_mlp_prefill(orc, llama_mlp):
    """512-token prefill: TP=8 rank shares (sampled rows vs oracle; their sum
    vs the GPU's own TP=1 run, all elements) and the TP=1 unsharded MLP."""
    L = llama_mlp
    D, F, t, I = L["D"], L["F"], L["t"], 512
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 512)
    Xd = to_dev(X, "bf16")
    T = torch()
    parts = T.empty((t, I, D), dtype=T.float32, device="cuda")
    H0 = None
    for r in range(t):
        H = empty((I, F // t), "bf16")
        tp.shard_mlp(Xd, *L["shards"][r], H, parts[r])
        if r == 0:
            H0 = H
    Y = empty((I, D), "f32")
    tp.partial_reduce(parts, Y)
    rows = [0, 1, 255, 256, 511]
    Href, Pref = orc.mlp_rank(X, *L["W64"], t, 0, rows=rows)
    T.cuda.synchronize()
    assert normwise_err(to_host(H0)[rows], Href) <= TOL["bf16"]
    assert normwise_err(to_host(parts[0])[rows], Pref) <= TOL["bf16"]
    # TP=1: the whole 8192 x 28672 MLP as one rank
    full = tuple(to_dev(a, "bf16") for a in L["W"])
    H1 = empty((I, F), "bf16")
    Y1 = empty((I, D), "f32")
    tp.shard_mlp(Xd, *full, H1, Y1)
    T.cuda.synchronize()
    _, Yref = orc.mlp_full(X, *L["W64"], rows=rows)
    assert normwise_err(to_host(Y1)[rows], Yref) <= TOL["bf16"]
    assert normwise_err(to_host(Y)[rows], Yref) <= TOL["bf16"]
    assert normwise_err(to_host(Y), to_host(Y1)) <= TOL["bf16"]
    del full, H1


def test_mlp_deterministic(llama_mlp):
    """Same inputs, same bits: no atomics, fixed summation orders."""
    L = llama_mlp
    T = torch()
    for I in (1, 32, 64, 512):
        X = to_dev(datagen.gaussian("X", (I, L["D"]), 1.0, "bf16", 9), "bf16")
        outs = []
        for _ in range(2):
            H = empty((I, L["F"] // L["t"]), "bf16")
            P = empty((I, L["D"]), "f32")
            tp.shard_mlp(X, *L["shards"][3], H, P)
            outs.append((H, P))
        T.cuda.synchronize()
        assert T.equal(outs[0][0], outs[1][0]) and T.equal(outs[0][1], outs[1][1]), I


def test_mlp_empty_and_errors_touch_nothing():
    """I = 0 is a no-op; a rejected call launches nothing (canaries survive)."""
    T = torch()
    X = to_dev(np.zeros((4, 64), np.float32), "bf16")
    W = to_dev(np.zeros((32, 64), np.float32), "bf16")
    Wd = to_dev(np.zeros((64, 32), np.float32), "bf16")
    H = empty((4, 32), "bf16")
    P = empty((4, 64), "f32")
    tp.shard_mlp(X[:0], W, W, Wd, H[:0], P[:0])
    L = tp.lib()
    # H aliasing the input X
    assert L.tp_shard_mlp(4, 64, 32, tp.TP_BF16, X.data_ptr(), W.data_ptr(), W.data_ptr(),
                          Wd.data_ptr(), X.data_ptr(), P.data_ptr(), None, 0, None) == 1
    # P not 16-byte aligned
    assert L.tp_shard_mlp(4, 64, 32, tp.TP_BF16, X.data_ptr(), W.data_ptr(), W.data_ptr(),
                          Wd.data_ptr(), H.data_ptr(), P.data_ptr() + 4, None, 0, None) == 2
    # the binding raises on an error status (n = 12 is not a multiple of 8)
    parts = empty((2, 4, 3), "f32")
    Y = empty((4, 3), "f32")
    with pytest.raises(tp.TPError, match="MISALIGNED"):
        tp.partial_reduce(parts, Y)
    T.cuda.synchronize()
    assert T.isnan(H).all() and T.isnan(P).all() and T.isnan(Y).all()


COUNTER_BYTES = 8192  # leading arrival-counter area of a split-K workspace


def test_explicit_workspace_scratch_contents_do_not_matter(llama_mlp):
    """Split-K calls (9..64 tokens on the streaming kernel, 65..256 on the
    tiled one) keep arrival counters and fp32 partials in the workspace: a
    caller buffer whose counter area is zero and whose partial area is NaN
    gives the same bits as the binding's own, twice in a row, and leaves the
    counter area zero."""
    L = llama_mlp
    T = torch()
    for I in (9, 32, 64, 128, 256):
        X = to_dev(datagen.gaussian("X", (I, L["D"]), 1.0, "bf16", 77), "bf16")
        need = tp.mlp_workspace_bytes(I, L["D"], L["F"] // L["t"])
        assert need > COUNTER_BYTES, I
        ws = T.full((need // 4 + 4,), float("nan"), dtype=T.float32, device="cuda")
        ws[:COUNTER_BYTES // 4].view(T.int32).zero_()
        outs = []
        for w in (None, ws, ws):
            H = empty((I, L["F"] // L["t"]), "bf16")
            P = empty((I, L["D"]), "f32")
            tp.shard_mlp(X, *L["shards"][5], H, P, workspace=w)
            outs.append((H, P))
        T.cuda.synchronize()
        for o in outs[1:]:
            assert T.equal(outs[0][0], o[0]) and T.equal(outs[0][1], o[1]), I
        assert int(ws[:COUNTER_BYTES // 4].view(T.int32).abs().sum()) == 0, I
        with pytest.raises(tp.TPError, match="WORKSPACE"):
            tp.shard_mlp(X, *L["shards"][5], outs[0][0], outs[0][1], workspace=ws[:8])
