"""GPU parity of tp_shard_mlp_int8 (weight-only int8 storage: a signed code
and a fp32 scale per output row; bf16 activations) against the fp64 oracle on
the dequantized weights, through every kernel the call uses: the few-token
kernel (1..4 tokens), split-K gate/up with whole-K or split-K down (5..64),
the one-byte GEMM (more tokens).
Bar: normwise 2e-2 (bf16 inputs and H, fp32 sums)."""
import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from megatron_tensor_layer_amd import datagen
from tests.common import normwise_err
from tests.gpu_util import empty, to_dev, to_host, torch

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _dev_i8(pair):
    T = torch()
    codes, scales = pair
    return (T.from_numpy(np.ascontiguousarray(codes, dtype=np.int8)).cuda(),
            T.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)).cuda())


def _run(X, shards):
    I, D = X.shape
    F_local = shards[0][0].shape[0]
    H = empty((I, F_local), "bf16")
    P = empty((I, D), "f32")
    tp.shard_mlp_int8(to_dev(X, "bf16"), *(_dev_i8(s) for s in shards), H, P)
    torch().cuda.synchronize()
    return to_host(H), to_host(P)


def _reference(orc, X, shards):
    (cg, sg), (cu, su), (cd, sd) = shards
    return orc.mlp_full(X, orc.dequant_int8(cg, sg), orc.dequant_int8(cu, su),
                        orc.dequant_int8(cd, sd))


def _shards(D, Fl, pool):
    return (datagen.int8_weights("W_gate8", (Fl, D), D ** -0.5, pool),
            datagen.int8_weights("W_up8", (Fl, D), D ** -0.5, pool),
            datagen.int8_weights("W_down8", (D, Fl), D ** -0.5, pool))


def test_int8_codes_use_the_signed_range():
    """The synthetic storage: codes in [-127, 127] with both signs, the row
    absmax at +-127, scales positive."""
    codes, scales = datagen.int8_weights("W_gate8", (64, 256), 256 ** -0.5, 3)
    assert codes.dtype == np.int8 and codes.min() < 0 < codes.max()
    assert np.all(np.abs(codes.astype(np.int32)).max(axis=1) == 127)
    assert np.all(scales > 0)


@pytest.fixture(scope="module")
def llama_i8():
    return _shards(8192, 3584, 70)


@pytest.mark.parametrize("I", [1, 2, 4, 5, 8, 16, 32, 64, 65, 256, 512])
def test_llama_rank_share(orc, llama_i8, I):
    """One Llama-3.1-70B TP=8 MLP rank share (D = 8192, F_local = 3584),
    every row against the oracle."""
    X = datagen.gaussian("X", (I, 8192), 1.0, "bf16", 700 + I)
    H, P = _run(X, llama_i8)
    H_ref, P_ref = _reference(orc, X, llama_i8)
    assert normwise_err(H, H_ref) <= TOL
    assert normwise_err(P, P_ref) <= TOL


@pytest.mark.parametrize("I,D,Fl", [(3, 528, 272), (12, 1040, 400), (40, 2064, 528),
                                    (70, 1040, 272), (130, 272, 1040), (300, 528, 400)])
def test_ragged_shapes(orc, I, D, Fl):
    """Contraction lengths and row counts that are not multiples of the
    kernels' tiles (multiples of 16 only)."""
    shards = _shards(D, Fl, D + Fl)
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 710 + I)
    H, P = _run(X, shards)
    H_ref, P_ref = _reference(orc, X, shards)
    assert normwise_err(H, H_ref) <= TOL
    assert normwise_err(P, P_ref) <= TOL


@pytest.mark.parametrize("I", [1, 8, 24])
def test_qwen_tp2_partials_sum_to_layer(orc, I):
    """Qwen2.5-1.5B MLP (D = 1536, F = 8960) at TP=2: the two ranks' int8
    partials sum on the GPU to the unsharded layer of the dequantized
    weights (lecture §4.3)."""
    D, F, t = 1536, 8960, 2
    full = _shards(D, F, 71)
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 720 + I)
    T = torch()
    parts = T.full((t, I, D), float("nan"), dtype=T.float32, device="cuda")
    Xd = to_dev(X, "bf16")
    for r in range(t):
        sh = datagen.fp8_mlp_rank_shards(full, t, r)  # contiguous F block, codes of any dtype
        H = empty((I, F // t), "bf16")
        tp.shard_mlp_int8(Xd, *(_dev_i8(s) for s in sh), H, parts[r])
    Y = empty((I, D), "f32")
    tp.partial_reduce(parts, Y)
    T.cuda.synchronize()
    _, Y_ref = _reference(orc, X, full)
    assert normwise_err(to_host(Y), Y_ref) <= TOL


def test_int8_matches_the_same_weights_as_bf16():
    """The int8 decode is exact: int8 weights given to the bf16 entry point as
    bf16 values (code * 1.0, scale 1) give the same H as the int8 entry point
    with unit scales, up to fp32 summation order."""
    D, Fl, I = 1024, 512, 8
    rng = np.random.default_rng(9)
    codes = [rng.integers(-128, 128, size=shp, dtype=np.int8)
             for shp in ((Fl, D), (Fl, D), (D, Fl))]
    ones = [np.ones(c.shape[0], np.float32) for c in codes]
    X = datagen.gaussian("X", (I, D), 0.05, "bf16", 730)
    H8, P8 = _run(X, list(zip(codes, ones)))
    Hb = empty((I, Fl), "bf16")
    Pb = empty((I, D), "f32")
    tp.shard_mlp(to_dev(X, "bf16"), *(to_dev(c.astype(np.float32), "bf16") for c in codes), Hb, Pb)
    torch().cuda.synchronize()
    assert normwise_err(H8, to_host(Hb)) <= 2.0 ** -8
    assert normwise_err(P8, to_host(Pb)) <= 1e-3
