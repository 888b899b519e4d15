"""The full Llama-3.1-70B-shaped layer with all 8 TP ranks emulated in turn on
one GPU: QKV (column, by heads) -> attention core -> o_proj (row) -> reduce
-> MLP (column gate/up, SwiGLU, row down) -> reduce, against the unsharded
fp64 oracle layer (normwise 2e-2).  The GPU carries the attention block's
output to the MLP in bf16; the oracle does not round it."""
import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from megatron_tensor_layer_amd import datagen
from tests.common import normwise_err
from tests.gpu_util import empty, to_dev, to_host, torch

pytestmark = pytest.mark.gpu
TOL = 2e-2
D, F, NQ, NKV, HD, T_ = 8192, 28672, 64, 8, 128, 8


def shard_set(Wq, Wk, Wv, Wo, Wg, Wu, Wd, t, r):
    return dict(
        qkv=to_dev(datagen.qkv_rank_shard(Wq, Wk, Wv, NQ, NKV, HD, t, r), "bf16"),
        o=to_dev(datagen.oproj_rank_shard(Wo, NQ, HD, t, r), "bf16"),
        mlp=tuple(to_dev(a, "bf16") for a in datagen.mlp_rank_shards(Wg, Wu, Wd, t, r)))


@pytest.fixture(scope="module")
def layer():
    """The layer's weights on the host, its 8 TP rank shares on the GPU, and
    the unsharded layer on the GPU (the TP=1 run)."""
    Wq, Wk, Wv, Wo = datagen.attn_weights(D, NQ, NKV, HD, "bf16", 11)
    Wg, Wu, Wd = datagen.mlp_weights(D, F, "bf16", 11)
    W = (Wq, Wk, Wv, Wo, Wg, Wu, Wd)
    ranks = [shard_set(*W, T_, r) for r in range(T_)]
    full = [shard_set(*W, 1, 0)]
    yield dict(attn=(Wq, Wk, Wv, Wo), mlp=(Wg, Wu, Wd), ranks=ranks, full=full)
    del ranks, full
    torch().cuda.empty_cache()


def gpu_layer(L, X, S, t=T_):
    """t rank shares of the layer in turn (t = 8: L["ranks"], t = 1:
    L["full"]).  Returns (QKV of rank 0, A of rank 0, o-partial of rank 0,
    attention block output y1 in bf16, layer output y).  Partial buffers are
    pre-filled with NaN, so a row no kernel writes shows."""
    T = torch()
    I = X.shape[0]
    nql, nkl = NQ // t, NKV // t
    Xd = to_dev(X, "bf16")
    po = T.full((t, I, D), float("nan"), dtype=T.float32, device="cuda")
    keep = {}
    for r, R in enumerate(L["ranks"] if t == T_ else L["full"]):
        qkv = empty((I, (nql + 2 * nkl) * HD), "bf16")
        tp.shard_attn_proj(tp.TP_ATTN_QKV, Xd, R["qkv"], qkv, nql, nkl, HD)
        A = empty((I, nql * HD), "bf16")
        tp.attn_core(qkv, A, S, nql, nkl, HD)
        tp.shard_attn_proj(tp.TP_ATTN_O, A, R["o"], po[r], nql, nkl, HD)
        if r == 0:
            keep = dict(qkv=qkv, A=A)
    y1 = empty((I, D), "bf16")
    tp.partial_reduce(po, y1)
    pm = T.full((t, I, D), float("nan"), dtype=T.float32, device="cuda")
    for r, R in enumerate(L["ranks"] if t == T_ else L["full"]):
        H = empty((I, F // t), "bf16")
        tp.shard_mlp(y1, *R["mlp"], H, pm[r])
    y = empty((I, D), "f32")
    tp.partial_reduce(pm, y)
    T.cuda.synchronize()
    return keep["qkv"], keep["A"], po[0], y1, y


def test_layer_decode32(orc, layer):
    """Decode batch 32: 32 independent sequences of one token each.  Rank 0's
    stages, the attention block output y1 (all rows) and the layer output y
    (all rows) against the unsharded oracle; the 8-rank result against the
    GPU's own TP=1 run of the same layer, every element."""
    I, S = 32, 1
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 32)
    qkv0, A0, po0, y1, y = gpu_layer(layer, X, S)
    _, _, _, y1_t1, y_t1 = gpu_layer(layer, X, S, t=1)
    Wq, Wk, Wv, Wo = layer["attn"]
    # rank 0 stages
    q_ref, A_ref, po_ref = orc.attn_block_rank(X, Wq, Wk, Wv, Wo, NQ, NKV, HD, S, T_, 0)
    assert normwise_err(to_host(qkv0), q_ref) <= TOL
    assert normwise_err(to_host(A0), A_ref) <= TOL
    assert normwise_err(to_host(po0), po_ref) <= TOL
    # unsharded attention block, then the unsharded MLP
    _, _, y1_ref = orc.attn_block_rank(X, Wq, Wk, Wv, Wo, NQ, NKV, HD, S)
    assert normwise_err(to_host(y1), y1_ref) <= TOL
    _, y_ref = orc.mlp_full(y1_ref, *layer["mlp"])
    yh = to_host(y)
    assert normwise_err(yh, y_ref) <= TOL
    # sum of the 8 ranks' partials against the GPU's TP=1 layer
    assert normwise_err(to_host(y1), to_host(y1_t1)) <= TOL
    assert normwise_err(yh, to_host(y_t1)) <= TOL


def test_layer_prefill512(orc, layer):
    """Prefill of one causal sequence of 512 tokens.  Rank 0's QKV (all rows),
    attention output and o_proj partial (a seeded 32-row sample) against the
    oracle; the attention block output y1 against the unsharded oracle block
    on every row; the layer output y against the unsharded oracle MLP (of the
    oracle's y1) on a seeded 32-row sample holding rows 0 and 511; and the
    8-rank result against the GPU's own TP=1 run, every element."""
    I, S = 512, 512
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 512)
    qkv0, A0, po0, y1, y = gpu_layer(layer, X, S)
    _, _, _, y1_t1, y_t1 = gpu_layer(layer, X, S, t=1)
    Wq, Wk, Wv, Wo = layer["attn"]
    q_ref, A_ref, po_ref = orc.attn_block_rank(X, Wq, Wk, Wv, Wo, NQ, NKV, HD, S, T_, 0)
    rows = sample_rows(I)
    assert normwise_err(to_host(qkv0), q_ref) <= TOL
    assert normwise_err(to_host(A0)[rows], A_ref[rows]) <= TOL
    assert normwise_err(to_host(po0)[rows], po_ref[rows]) <= TOL
    _, _, y1_ref = orc.attn_block_rank(X, Wq, Wk, Wv, Wo, NQ, NKV, HD, S)
    y1h = to_host(y1)
    assert normwise_err(y1h, y1_ref) <= TOL
    _, y_ref = orc.mlp_full(y1_ref, *layer["mlp"], rows=rows)
    yh = to_host(y)
    assert normwise_err(yh[rows], y_ref) <= TOL
    assert normwise_err(y1h, to_host(y1_t1)) <= TOL
    assert normwise_err(yh, to_host(y_t1)) <= TOL


def sample_rows(I, n=32, seed=0):
    """Seeded sample of n token rows that always holds rows 0 and I - 1."""
    if I <= n:
        return list(range(I))
    rng = np.random.default_rng(seed + I)
    mid = rng.choice(np.arange(1, I - 1), size=n - 2, replace=False)
    return sorted({0, I - 1, *map(int, mid)})


def test_prenorm_block_decode32(orc, layer):
    """The layer as a pre-norm block on the residual stream h (bf16), decode
    32: x = RMSNorm(h); 8 ranks' attention blocks; h += sum of the o_proj
    partials, x = RMSNorm(h); 8 ranks' MLPs; h += sum of the MLP partials,
    x = RMSNorm(h).  Against the unsharded fp64 oracle (MLP on sampled rows)."""
    T = torch()
    I, S, eps = 32, 1, 1e-5
    nql, nkl = NQ // T_, NKV // T_
    h0 = datagen.gaussian("h", (I, D), 1.0, "bf16", 77)
    gs = [datagen.rmsnorm_gamma(D, 40 + k, "bf16") for k in range(3)]
    gd = [to_dev(g, "bf16") for g in gs]
    h = to_dev(h0, "bf16")
    x = empty((I, D), "bf16")
    tp.residual_rmsnorm(None, h, h, gd[0], x, eps)
    x1 = to_host(x).copy()
    po = T.empty((T_, I, D), dtype=T.float32, device="cuda")
    for r, R in enumerate(layer["ranks"]):
        qkv = empty((I, (nql + 2 * nkl) * HD), "bf16")
        tp.shard_attn_proj(tp.TP_ATTN_QKV, x, R["qkv"], qkv, nql, nkl, HD)
        A = empty((I, nql * HD), "bf16")
        tp.attn_core(qkv, A, S, nql, nkl, HD)
        tp.shard_attn_proj(tp.TP_ATTN_O, A, R["o"], po[r], nql, nkl, HD)
    tp.residual_rmsnorm(po, h, h, gd[1], x, eps)
    T.cuda.synchronize()
    h1, x2 = to_host(h).copy(), to_host(x).copy()
    pm = T.empty((T_, I, D), dtype=T.float32, device="cuda")
    for r, R in enumerate(layer["ranks"]):
        H = empty((I, F // T_), "bf16")
        tp.shard_mlp(x, *R["mlp"], H, pm[r])
    tp.residual_rmsnorm(pm, h, h, gd[2], x, eps)
    T.cuda.synchronize()
    h2, x3 = to_host(h), to_host(x)

    Wq, Wk, Wv, Wo = layer["attn"]
    _, x1_ref = orc.residual_rmsnorm(None, h0, gs[0], eps)
    assert normwise_err(x1, x1_ref) <= TOL
    _, _, a_ref = orc.attn_block_rank(x1_ref, Wq, Wk, Wv, Wo, NQ, NKV, HD, S)
    h1_ref, x2_ref = orc.residual_rmsnorm(a_ref[None], h0, gs[1], eps)
    assert normwise_err(h1, h1_ref) <= TOL
    assert normwise_err(x2, x2_ref) <= TOL
    rows = [0, 17, 31]
    _, y_ref = orc.mlp_full(x2_ref, *layer["mlp"], rows=rows)
    h2_ref, x3_ref = orc.residual_rmsnorm(y_ref[None], h1_ref[rows], gs[2], eps)
    assert normwise_err(h2[rows], h2_ref) <= TOL
    assert normwise_err(x3[rows], x3_ref) <= TOL
