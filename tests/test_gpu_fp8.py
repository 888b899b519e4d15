"""GPU parity of tp_shard_mlp_fp8 (weight-only FP8 storage, OCP E4M3 with a
fp32 scale per output row; bf16 activations) against the fp64 oracle on the
dequantized weights: the few-token kernel (1..8 tokens), the split-K MFMA
kernel (9..64) and the one-byte GEMM (more tokens).  Bar: normwise 2e-2
(bf16 inputs and H, fp32 sums)."""
import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from megatron_tensor_layer_amd import datagen
from tests.common import normwise_err
from tests.gpu_util import empty, to_dev, to_host, torch

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _dev_fp8(pair):
    T = torch()
    codes, scales = pair
    return (T.from_numpy(np.ascontiguousarray(codes)).cuda(),
            T.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)).cuda())


def _run(X, shards):
    I, D = X.shape
    F_local = shards[0][0].shape[0]
    H = empty((I, F_local), "bf16")
    P = empty((I, D), "f32")
    tp.shard_mlp_fp8(to_dev(X, "bf16"), *(_dev_fp8(s) for s in shards), H, P)
    torch().cuda.synchronize()
    return to_host(H), to_host(P)


def _reference(orc, X, shards, rows=None):
    (cg, sg), (cu, su), (cd, sd) = shards
    return orc.mlp_full(X, orc.dequant_fp8(cg, sg), orc.dequant_fp8(cu, su),
                        orc.dequant_fp8(cd, sd), rows=rows)


def _shards(D, Fl, pool):
    return (datagen.fp8_weights("W_gate8", (Fl, D), D ** -0.5, pool),
            datagen.fp8_weights("W_up8", (Fl, D), D ** -0.5, pool),
            datagen.fp8_weights("W_down8", (D, Fl), D ** -0.5, pool))


@pytest.fixture(scope="module")
def llama_fp8():
    return _shards(8192, 3584, 60)


@pytest.mark.parametrize("I", [1, 2, 4, 8])
def test_llama_rank_share_decode(orc, llama_fp8, I):
    """One Llama-3.1-70B TP=8 MLP rank share (D = 8192, F_local = 3584)."""
    D = 8192
    shards = llama_fp8
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 600 + I)
    H, P = _run(X, shards)
    H_ref, P_ref = _reference(orc, X, shards)
    assert normwise_err(H, H_ref) <= TOL
    assert normwise_err(P, P_ref) <= TOL


@pytest.mark.parametrize("I", [16, 32, 64])
def test_llama_rank_share_split_k(orc, llama_fp8, I):
    """9..64 tokens: the split-K MFMA kernel on the same rank share; every
    row against the oracle."""
    D = 8192
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 640 + I)
    H, P = _run(X, llama_fp8)
    H_ref, P_ref = _reference(orc, X, llama_fp8)
    assert normwise_err(H, H_ref) <= TOL
    assert normwise_err(P, P_ref) <= TOL


@pytest.mark.parametrize("I", [65, 128, 512])
def test_llama_rank_share_gemm(orc, llama_fp8, I):
    """More than 64 tokens: the one-byte GEMM (gate/up split K at 65 and 128
    tokens, unsplit at 512); every row against the oracle."""
    D = 8192
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 660 + I)
    H, P = _run(X, llama_fp8)
    H_ref, P_ref = _reference(orc, X, llama_fp8)
    assert normwise_err(H, H_ref) <= TOL
    assert normwise_err(P, P_ref) <= TOL


@pytest.mark.parametrize("I,D,Fl", [(65, 16, 16), (70, 1040, 272), (130, 272, 1040),
                                    (300, 528, 400), (100, 4112, 272), (520, 1536, 4480)])
def test_gemm_ragged_shapes(orc, I, D, Fl):
    """The one-byte GEMM on a K of one 16-code chunk, ragged K stages (1040 =
    8 x 128 + 16), ragged weight tiles (272 = 4 x 64 + 16 gate/up columns),
    a ragged last M tile (130, 300, 520 tokens), a long K over few tiles
    (split K with a ragged last range) and the Qwen2.5-1.5B TP=2 share at 520
    tokens."""
    shards = _shards(D, Fl, 64)
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 650 + I)
    H, P = _run(X, shards)
    H_ref, P_ref = _reference(orc, X, shards)
    assert normwise_err(H, H_ref) <= TOL
    assert normwise_err(P, P_ref) <= TOL


@pytest.mark.parametrize("I", [1, 8, 24])
def test_qwen_tp2_partials_sum_to_layer(orc, I):
    """Qwen2.5-1.5B MLP (D = 1536, F = 8960) at TP=2: each rank's FP8 share
    against the oracle, and the two partials sum to the unsharded layer."""
    D, F, t = 1536, 8960, 2
    full = datagen.fp8_mlp_weights(D, F, 61)
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 610 + I)
    Ps = []
    for r in range(t):
        shards = datagen.fp8_mlp_rank_shards(full, t, r)
        H, P = _run(X, shards)
        H_ref, P_ref = _reference(orc, X, shards)
        assert normwise_err(H, H_ref) <= TOL
        assert normwise_err(P, P_ref) <= TOL
        Ps.append(P)
    _, Y_ref = _reference(orc, X, full)
    assert normwise_err(Ps[0] + Ps[1], Y_ref) <= TOL


@pytest.mark.parametrize("I,D,Fl", [(3, 16, 16), (5, 48, 80), (8, 1040, 272), (1, 16384, 16),
                                    (9, 48, 80), (17, 1040, 272), (40, 272, 1040),
                                    (64, 1536, 4480), (2, 32768, 64),
                                    # down on the whole-K row-streaming kernel: a ragged
                                    # last row tile (9 rows per tile), a full grid
                                    (20, 4112, 1040), (9, 4096, 2064), (6, 4112, 1040)])
def test_small_and_ragged_shapes(orc, I, D, Fl):
    """K of one 16-byte chunk, chunks not filling a wave, two chunks per lane;
    split K with ragged K ranges and row tiles; K past the few-token limit."""
    shards = _shards(D, Fl, 62)
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 620 + I)
    H, P = _run(X, shards)
    H_ref, P_ref = _reference(orc, X, shards)
    assert normwise_err(H, H_ref) <= TOL
    assert normwise_err(P, P_ref) <= TOL


def test_deterministic(orc):
    """Bitwise the same twice: the few-token kernel, split K (fixed summation
    order) and the one-byte GEMM with split K."""
    D, Fl = 1536, 4480
    shards = _shards(D, Fl, 63)
    for I, seed in ((8, 630), (33, 632), (65, 631)):
        X = datagen.gaussian("X", (I, D), 1.0, "bf16", seed)
        a, b = _run(X, shards), _run(X, shards)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), I
