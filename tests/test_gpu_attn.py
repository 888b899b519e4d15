"""GPU parity of tp_shard_attn_proj (head-split QKV, row-split o_proj) and of
the per-rank attention core against the fp64 oracle (normwise 2e-2, bf16)."""
import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from megatron_tensor_layer_amd import datagen
from tests.common import normwise_err
from tests.gpu_util import empty, to_dev, to_host, torch

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.mark.parametrize("I", [1, 8, 64])
def test_qwen_attn_projections_tp2(orc, I):
    """Qwen2.5-1.5B-shaped attention projections at TP=2: 6 of 12 query heads
    and 1 of 2 KV groups per rank at head_dim 128 (N_qkv = 1024, K_o = 768)."""
    D, n_q, n_kv, hd, t = 1536, 12, 2, 128, 2
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 300 + I)
    Wq, Wk, Wv, Wo = datagen.attn_weights(D, n_q, n_kv, hd, "bf16", 300)
    A = datagen.gaussian("A", (I, n_q * hd), 1.0, "bf16", 300 + I)
    T = torch()
    Xd = to_dev(X, "bf16")
    parts = T.empty((t, I, D), dtype=T.float32, device="cuda")
    nql, nkl = n_q // t, n_kv // t
    for r in range(t):
        Wr = to_dev(datagen.qkv_rank_shard(Wq, Wk, Wv, n_q, n_kv, hd, t, r), "bf16")
        out = empty((I, (nql + 2 * nkl) * hd), "bf16")
        tp.shard_attn_proj(tp.TP_ATTN_QKV, Xd, Wr, out, nql, nkl, hd)
        Ar = to_dev(np.ascontiguousarray(A[:, r * nql * hd:(r + 1) * nql * hd]), "bf16")
        Wor = to_dev(datagen.oproj_rank_shard(Wo, n_q, hd, t, r), "bf16")
        tp.shard_attn_proj(tp.TP_ATTN_O, Ar, Wor, parts[r], nql, nkl, hd)
        T.cuda.synchronize()
        ref = orc.qkv_rank(X, Wq, Wk, Wv, n_q, n_kv, hd, t, r)
        assert normwise_err(to_host(out), ref) <= TOL
        Pref = orc.oproj_rank(A[:, r * nql * hd:(r + 1) * nql * hd], Wo, n_q, hd, t, r)
        assert normwise_err(to_host(parts[r]), Pref) <= TOL
    Y = empty((I, D), "f32")
    tp.partial_reduce(parts, Y)
    T.cuda.synchronize()
    assert normwise_err(to_host(Y), orc.oproj_rank(A, Wo, n_q, hd)) <= TOL


def test_qkv_split_tail(orc):
    """A QKV projection of 320 GEMM tiles (130 tokens, N_qkv = 160 heads x
    128): 256 tiles in one launch, the last 64 with K split in a second."""
    I, D, n_q, n_kv, hd = 130, 1040, 144, 8, 128
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 310)
    Wq, Wk, Wv, _ = datagen.attn_weights(D, n_q, n_kv, hd, "bf16", 310)
    W = datagen.qkv_rank_shard(Wq, Wk, Wv, n_q, n_kv, hd, 1, 0)
    out = empty((I, W.shape[0]), "bf16")
    tp.shard_attn_proj(tp.TP_ATTN_QKV, to_dev(X, "bf16"), to_dev(W, "bf16"), out, n_q, n_kv, hd)
    torch().cuda.synchronize()
    assert normwise_err(to_host(out), orc.qkv_rank(X, Wq, Wk, Wv, n_q, n_kv, hd, 1, 0)) <= TOL


# (I, S, n_q_local, n_kv_local, head_dim): several sequences, GQA groups,
# head_dim below one wavefront, and above two (lanes holding 3 elements)
CORE = [(12, 4, 4, 2, 64), (7, 7, 2, 1, 136), (16, 16, 8, 1, 128), (5, 1, 4, 4, 32),
        (40, 20, 6, 2, 256),
        # sequences straddling the 32-row query blocks, head_dim of 3 column tiles
        (96, 48, 4, 2, 64), (70, 35, 3, 1, 72),
        # one causal sequence of 512 tokens at the Llama-70B TP=8 head layout
        (512, 512, 8, 1, 128),
        # blocks wholly below the diagonal (no mask) between sequence starts
        # aligned to the key blocks, and a 1024-token sequence
        (384, 128, 4, 2, 64), (1024, 1024, 8, 1, 128)]


@pytest.mark.parametrize("I,S,nq,nkv,hd", CORE)
def test_attn_core(orc, I, S, nq, nkv, hd):
    qkv = datagen.gaussian("A", (I, (nq + 2 * nkv) * hd), 1.0, "bf16", I * S + hd)
    A = empty((I, nq * hd), "bf16")
    tp.attn_core(to_dev(qkv, "bf16"), A, S, nq, nkv, hd)
    torch().cuda.synchronize()
    assert normwise_err(to_host(A), orc.attn_core(qkv, S, nq, nkv, hd)) <= TOL


def test_attn_core_single_token_is_value():
    """One token per sequence: the output is the value of the head's group, bit
    for bit (softmax over one score is exactly 1)."""
    I, nq, nkv, hd = 6, 4, 2, 128
    qkv = datagen.gaussian("A", (I, (nq + 2 * nkv) * hd), 1.0, "bf16", 5)
    A = empty((I, nq * hd), "bf16")
    tp.attn_core(to_dev(qkv, "bf16"), A, 1, nq, nkv, hd)
    torch().cuda.synchronize()
    got = to_host(A)
    for j in range(nq):
        g = j * nkv // nq
        assert np.array_equal(got[:, j * hd:(j + 1) * hd],
                              qkv[:, (nq + nkv + g) * hd:(nq + nkv + g + 1) * hd])
