"""GPU parity of tp_attn_decode (decode attention over a rank's head-sharded
KV cache) against the fp64 oracle, normwise 2e-2; the cache slot of the new
token must receive its k and v bit for bit.  The oracle takes both caches as
[B, groups, L_max, head_dim]; the device V cache is its transpose
[B, groups, head_dim, L_max]."""
import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from megatron_tensor_layer_amd import datagen
from tests.common import normwise_err
from tests.gpu_util import empty, to_dev, to_host, torch

pytestmark = pytest.mark.gpu
TOL = 2e-2


def _case(B, nq, nkv, hd, Lmax, lens, seed):
    """bf16 qkv of the new tokens and caches holding lens[b]-1 earlier tokens
    (the rest of each cache is NaN bits: never read)."""
    qkv = datagen.gaussian("A", (B, (nq + 2 * nkv) * hd), 1.0, "bf16", seed)
    Kc = np.full((B, nkv, Lmax, hd), np.nan, dtype=np.float32)
    Vc = np.full((B, nkv, Lmax, hd), np.nan, dtype=np.float32)
    k = datagen.gaussian("h", (B, nkv, Lmax, hd), 1.0, "bf16", seed)
    v = datagen.gaussian("P", (B, nkv, Lmax, hd), 1.0, "bf16", seed)
    for b, L in enumerate(lens):
        Kc[b, :, :L - 1] = k[b, :, :L - 1]
        Vc[b, :, :L - 1] = v[b, :, :L - 1]
    return qkv, Kc, Vc


def _nan_bf16_dev(a):
    """Cache to the device as bf16 bits; NaN entries become a bf16 NaN."""
    T = torch()
    bits = np.where(np.isnan(a), np.uint32(0x7FC00000), a.view(np.uint32))
    return T.from_numpy((bits >> 16).astype(np.uint16).view(np.int16)).view(T.bfloat16).cuda()


def _run(qkv, Kc, Vc, lens, nq, nkv, hd, workspace=None):
    T = torch()
    B = qkv.shape[0]
    qd, Kd = to_dev(qkv, "bf16"), _nan_bf16_dev(Kc)
    Vd = _nan_bf16_dev(np.ascontiguousarray(Vc.transpose(0, 1, 3, 2)))
    ld = T.tensor(np.asarray(lens, dtype=np.int32)).cuda()
    A = empty((B, nq * hd), "bf16")
    tp.attn_decode(ld, qd, Kd, Vd, A, nq, nkv, hd, workspace=workspace)
    T.cuda.synchronize()
    return to_host(A), Kd, Vd, qd


@pytest.mark.parametrize("B,nq,nkv,hd,Lmax,seed", [
    (32, 8, 1, 128, 2048, 1),    # Llama-3.1-70B TP=8 rank: 8 heads, 1 KV group
    (8, 6, 1, 128, 296, 2),      # Qwen2.5-1.5B TP=2 rank, cache length not a multiple of 32
    (3, 8, 2, 64, 104, 3),       # two groups of 4 heads
    (5, 4, 4, 32, 72, 4),        # one head per group
    (7, 4, 1, 40, 8, 5),         # head_dim not a multiple of 32, a cache of 8 positions
    (4, 8, 1, 128, 192, 6),      # chunks of 96 positions: a round with one wave idle
    (2, 8, 1, 128, 1000, 7),     # the last chunk's round partly past the cache
    (32, 8, 1, 128, 2144, 8),    # three rounds per chunk, the last one a single block
    (16, 8, 2, 64, 1600, 9),     # two groups, rounds of 128 and 96 positions
    (4, 32, 1, 128, 200, 10),    # 32 heads in one group and head_dim 128: the largest
])
def test_attn_decode(orc, B, nq, nkv, hd, Lmax, seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, Lmax + 1, B)
    lens[0], lens[-1] = 1, Lmax
    qkv, Kc, Vc = _case(B, nq, nkv, hd, Lmax, lens, seed)
    A, Kd, Vd, qd = _run(qkv, Kc, Vc, lens, nq, nkv, hd)
    ref = orc.attn_decode(qkv, Kc, Vc, lens, nq, nkv, hd)
    assert normwise_err(A, ref) <= TOL
    Kh, Vh = to_host(Kd), to_host(Vd).transpose(0, 1, 3, 2)
    for b, L in enumerate(lens):
        for g in range(nkv):
            assert np.array_equal(Kh[b, g, L - 1], qkv[b, (nq + g) * hd:(nq + g + 1) * hd])
            assert np.array_equal(Vh[b, g, L - 1],
                                  qkv[b, (nq + nkv + g) * hd:(nq + nkv + g + 1) * hd])


def test_single_position_is_value():
    B, nq, nkv, hd = 6, 4, 2, 64
    lens = [1] * B
    qkv, Kc, Vc = _case(B, nq, nkv, hd, 40, lens, 9)
    A, *_ = _run(qkv, Kc, Vc, lens, nq, nkv, hd)
    for j in range(nq):
        g = j * nkv // nq
        assert np.array_equal(A[:, j * hd:(j + 1) * hd],
                              qkv[:, (nq + nkv + g) * hd:(nq + nkv + g + 1) * hd])


def test_ranks_with_replicated_kv_groups(orc):
    """More ranks than KV groups (t = 4, 2 groups): each rank stores the one
    group its 2 query heads use, so groups are replicated; the ranks' heads,
    side by side, are the full model's decode attention."""
    B, nq, nkv, hd, Lmax, t = 4, 8, 2, 64, 96, 4
    rng = np.random.default_rng(12)
    lens = rng.integers(1, Lmax + 1, B)
    qkv, Kc, Vc = _case(B, nq, nkv, hd, Lmax, lens, 12)
    full = orc.attn_decode(qkv, Kc, Vc, lens, nq, nkv, hd)
    nql = nq // t
    for r in range(t):
        g = (r * nql) * nkv // nq  # the group of this rank's heads
        qkv_r = np.concatenate([qkv[:, r * nql * hd:(r + 1) * nql * hd],
                                qkv[:, (nq + g) * hd:(nq + g + 1) * hd],
                                qkv[:, (nq + nkv + g) * hd:(nq + nkv + g + 1) * hd]], axis=1)
        A, *_ = _run(np.ascontiguousarray(qkv_r), np.ascontiguousarray(Kc[:, g:g + 1]),
                     np.ascontiguousarray(Vc[:, g:g + 1]), lens, nql, 1, hd)
        assert normwise_err(A, full[:, r * nql * hd:(r + 1) * nql * hd]) <= TOL


def test_explicit_workspace_deterministic(orc):
    T = torch()
    B, nq, nkv, hd, Lmax = 4, 8, 1, 128, 1024
    lens = [1024, 700, 33, 512]
    qkv, Kc, Vc = _case(B, nq, nkv, hd, Lmax, lens, 14)
    need = tp.lib().tp_attn_decode_workspace_size(B, nq, nkv, hd, Lmax)
    assert need > 8192
    ws = T.zeros((need,), dtype=T.uint8, device="cuda")
    a1, *_ = _run(qkv, Kc, Vc, lens, nq, nkv, hd, workspace=ws)
    a2, *_ = _run(qkv, Kc, Vc, lens, nq, nkv, hd, workspace=ws)
    a3, *_ = _run(qkv, Kc, Vc, lens, nq, nkv, hd)
    assert np.array_equal(a1, a2) and np.array_equal(a1, a3)
    assert int(ws[:8192].view(T.int32).abs().sum()) == 0
    assert normwise_err(a1, orc.attn_decode(qkv, Kc, Vc, lens, nq, nkv, hd)) <= TOL
