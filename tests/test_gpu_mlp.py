"""GPU parity of tp_shard_mlp against the fp64 oracle.

Tolerance (normwise, max|gpu - ref| / max|ref|): 2e-2 for bf16 inputs with
fp32 accumulation, 1e-5 for fp32.  The oracle takes the FULL weights and the
rank index; the GPU gets the rank's contiguous shard buffers."""
import numpy as np
import pytest

import megatron_tensor_layer_amd as tp
from megatron_tensor_layer_amd import datagen
from tests.common import BF16_STEP, DIAG_BF16_FLIPS, DIAG_TOL, bf16_flips, normwise_err
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
    # the few-token kernel's longest K: 32768 (bf16) and 16384 (fp32)
    (2, 32768, 16, 1, 0, "bf16"), (3, 16384, 16, 1, 0, "f32"),
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
    # 256 x 128 GEMM tiles (384 tokens and more): gate/up in one K range and
    # split 3 ways with a ragged last M tile (390 = 256 + 134), down in one K
    # range (K = 520, ragged last stage) and split 5 ways
    (384, 1040, 6152, 1, 0, "bf16"), (390, 3080, 2064, 1, 0, "bf16"),
    (390, 8200, 520, 1, 0, "bf16"), (390, 3080, 8200, 1, 0, "bf16"),
    # more than one round of GEMM tiles with a partial last round: whole
    # rounds in one launch, the last round's tiles split over K in a second
    # (gate/up: 300 128 x 128 tiles, then 532 256 x 128 tiles)
    (130, 1040, 9600, 1, 0, "bf16"), (390, 1040, 17000, 1, 0, "bf16"),
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
    """Qwen2.5-1.5B-shaped MLP at TP=2 (D=1536, F=8960): both ranks (H and P
    of each against the oracle), the reduce against the unsharded oracle, and
    the GPU's sum of partials against its own TP=1 run, every element."""
    D, F, t = 1536, 8960, 2
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", 100 + I)
    Wg, Wu, Wd = datagen.mlp_weights(D, F, "bf16", 100)
    T = torch()
    parts = T.full((t, I, D), float("nan"), dtype=T.float32, device="cuda")
    for r in range(t):
        H, P = gpu_mlp(X, *datagen.mlp_rank_shards(Wg, Wu, Wd, t, r), "bf16")
        parts[r].copy_(P)
        Href, Pref = orc.mlp_rank(X, Wg, Wu, Wd, t, r)
        assert normwise_err(to_host(H), Href) <= TOL["bf16"], r
        assert normwise_err(to_host(P), Pref) <= TOL["bf16"], r
    Y = empty((I, D), "f32")
    tp.partial_reduce(parts, Y)
    _, Y1 = gpu_mlp(X, Wg, Wu, Wd, "bf16")
    T.cuda.synchronize()
    _, Yref = orc.mlp_full(X, Wg, Wu, Wd)
    assert normwise_err(to_host(Y), Yref) <= TOL["bf16"]
    assert normwise_err(to_host(Y1), Yref) <= TOL["bf16"]
    assert normwise_err(to_host(Y), to_host(Y1)) <= TOL["bf16"]


# ---------------------------------------------------------------- Llama-70B
@pytest.fixture(scope="module")
def llama_mlp():
    """Full Llama-3.1-70B-shaped MLP weights (D=8192, F=28672), host fp32 and
    fp64 copies, the 8 TP rank shards resident on the GPU, and the unsharded
    weights on the GPU (the TP=1 run)."""
    D, F, t = 8192, 28672, 8
    Wg, Wu, Wd = datagen.mlp_weights(D, F, "bf16", 7)
    shards = [tuple(to_dev(a, "bf16") for a in datagen.mlp_rank_shards(Wg, Wu, Wd, t, r))
              for r in range(t)]
    full = tuple(to_dev(a, "bf16") for a in (Wg, Wu, Wd))
    W64 = tuple(a.astype(np.float64) for a in (Wg, Wu, Wd))
    yield dict(D=D, F=F, t=t, W=(Wg, Wu, Wd), W64=W64, shards=shards, full=full)
    del shards, full
    torch().cuda.empty_cache()


def sample_rows(I, n=32, seed=0):
    """Seeded sample of n token rows that always holds rows 0 and I - 1."""
    if I <= n:
        return list(range(I))
    rng = np.random.default_rng(seed + I)
    mid = rng.choice(np.arange(1, I - 1), size=n - 2, replace=False)
    return sorted({0, I - 1, *map(int, mid)})


def sharded_mlp(L, Xd, I, keep_h=True):
    """All t rank shares on the GPU (partials pre-filled with NaN, so a row
    a kernel never writes shows), then the on-device reduce; plus the GPU's
    own TP=1 run of the unsharded weights."""
    T = torch()
    D, F, t = L["D"], L["F"], L["t"]
    parts = T.full((t, I, D), float("nan"), dtype=T.float32, device="cuda")
    Hs = []
    for r in range(t):
        H = empty((I, F // t), "bf16")
        tp.shard_mlp(Xd, *L["shards"][r], H, parts[r])
        Hs.append(H if keep_h else None)
    Y = empty((I, D), "f32")
    tp.partial_reduce(parts, Y)
    H1 = empty((I, F), "bf16")
    Y1 = empty((I, D), "f32")
    tp.shard_mlp(Xd, *L["full"], H1, Y1)
    T.cuda.synchronize()
    del H1
    return Hs, parts, Y, Y1


@pytest.mark.parametrize("I", [1, 6, 16, 32, 64, 256])
def test_llama_mlp_decode_tp8(orc, llama_mlp, I):
    """Llama-3.1-70B-shaped MLP, all 8 TP=8 rank shares on one GPU, decode I
    tokens.  Every row of every rank's H and P and of the reduced Y against
    the oracle; Y against the unsharded oracle layer on a seeded row sample
    (lecture §4.3: the sharded output equals the single-device output); the
    GPU's sum of partials against the GPU's own TP=1 run, every element."""
    L = llama_mlp
    t = L["t"]
    X = datagen.gaussian("X", (I, L["D"]), 1.0, "bf16", 200 + I)
    Hs, parts, Y, Y1 = sharded_mlp(L, to_dev(X, "bf16"), I)
    Prefs, Pbs = [], []
    for r in range(t):
        Href, Pref, Hb, Pb = orc.mlp_rank_bf16h(X, *L["W64"], t, r)
        Hg, Pg = to_host(Hs[r]), to_host(parts[r])
        assert normwise_err(Hg, Href) <= TOL["bf16"], r
        assert normwise_err(Pg, Pref) <= TOL["bf16"], r
        # diagnostic: against the oracle with H rounded to bf16 as stored
        print(f"diagnostic I={I} rank {r}: H flips {bf16_flips(Hg, Hb):.2e}, "
              f"H {normwise_err(Hg, Hb):.2e}, P {normwise_err(Pg, Pb):.2e}")
        assert bf16_flips(Hg, Hb) <= DIAG_BF16_FLIPS, r
        assert normwise_err(Hg, Hb) <= BF16_STEP, r
        assert normwise_err(Pg, Pb) <= DIAG_TOL, r
        Prefs.append(Pref)
        Pbs.append(Pb)
    Yref = orc.reduce(np.stack(Prefs))
    Yh = to_host(Y)
    assert normwise_err(Yh, Yref) <= TOL["bf16"]
    assert normwise_err(Yh, orc.reduce(np.stack(Pbs))) <= DIAG_TOL
    rows = sample_rows(I)
    _, Yfull = orc.mlp_full(X, *L["W64"], rows=rows)
    assert normwise_err(Yh[rows], Yfull) <= TOL["bf16"]
    assert normwise_err(Yh, to_host(Y1)) <= TOL["bf16"]


def test_llama_mlp_prefill(orc, llama_mlp):
    """512-token prefill.  TP=8: every row of every rank's H and P and of the
    reduced Y against the oracle.  TP=1 (the unsharded 8192 x 28672 MLP): a
    seeded 32-row sample holding rows 0 and 511 against the unsharded oracle.
    The GPU's sum of partials against its TP=1 run, every element."""
    L = llama_mlp
    t, I = L["t"], 512
    X = datagen.gaussian("X", (I, L["D"]), 1.0, "bf16", 512)
    Hs, parts, Y, Y1 = sharded_mlp(L, to_dev(X, "bf16"), I)
    Prefs, Pbs = [], []
    for r in range(t):
        Href, Pref, Hb, Pb = orc.mlp_rank_bf16h(X, *L["W64"], t, r)
        Hg, Pg = to_host(Hs[r]), to_host(parts[r])
        assert normwise_err(Hg, Href) <= TOL["bf16"], r
        assert normwise_err(Pg, Pref) <= TOL["bf16"], r
        print(f"diagnostic prefill rank {r}: H flips {bf16_flips(Hg, Hb):.2e}, "
              f"H {normwise_err(Hg, Hb):.2e}, P {normwise_err(Pg, Pb):.2e}")
        assert bf16_flips(Hg, Hb) <= DIAG_BF16_FLIPS, r
        assert normwise_err(Hg, Hb) <= BF16_STEP, r
        assert normwise_err(Pg, Pb) <= DIAG_TOL, r
        Prefs.append(Pref)
        Pbs.append(Pb)
    Yh, Y1h = to_host(Y), to_host(Y1)
    assert normwise_err(Yh, orc.reduce(np.stack(Prefs))) <= TOL["bf16"]
    assert normwise_err(Yh, orc.reduce(np.stack(Pbs))) <= DIAG_TOL
    rows = sample_rows(I)
    _, Yfull, _, Yfull_b = orc.mlp_rank_bf16h(X, *L["W64"], rows=rows)
    assert normwise_err(Y1h[rows], Yfull) <= TOL["bf16"]
    assert normwise_err(Y1h[rows], Yfull_b) <= DIAG_TOL
    assert normwise_err(Yh[rows], Yfull) <= TOL["bf16"]
    assert normwise_err(Yh, Y1h) <= TOL["bf16"]


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


def test_split_tail_deterministic():
    """The GEMM plan whose last partial round of tiles runs as a second,
    split-K launch (130 tokens: 300 gate/up tiles) gives the same bits on
    every call, with the binding's workspace and with a fresh one."""
    T = torch()
    I, D, F = 130, 1040, 9600
    X = to_dev(datagen.gaussian("X", (I, D), 1.0, "bf16", 21), "bf16")
    Wg, Wu, Wd = (to_dev(w, "bf16") for w in datagen.mlp_weights(D, F, "bf16", 21))
    need = tp.mlp_workspace_bytes(I, D, F)
    assert need > COUNTER_BYTES
    fresh = T.zeros((need // 4 + 4,), dtype=T.int32, device="cuda")
    outs = []
    for ws in (None, None, fresh):
        H = empty((I, F), "bf16")
        P = empty((I, D), "f32")
        tp.shard_mlp(X, Wg, Wu, Wd, H, P, workspace=ws)
        outs.append((H, P))
    T.cuda.synchronize()
    for o in outs[1:]:
        assert T.equal(outs[0][0], o[0]) and T.equal(outs[0][1], o[1])
    assert int(fresh[:COUNTER_BYTES // 4].abs().sum()) == 0


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
    tiled one) keep arrival counters and fp32 partials in the workspace.  A
    caller buffer filled with arbitrary bits -- counter area included -- and
    then prepared with tp_workspace_reset gives the same bits as the
    binding's own workspace, twice in a row, and is left with a zero counter
    area."""
    L = llama_mlp
    T = torch()
    gen = T.Generator(device="cuda")
    gen.manual_seed(1234)
    for I in (9, 32, 64, 128, 256):
        X = to_dev(datagen.gaussian("X", (I, L["D"]), 1.0, "bf16", 77), "bf16")
        need = tp.mlp_workspace_bytes(I, L["D"], L["F"] // L["t"])
        assert need > COUNTER_BYTES, I
        ws = T.randint(-2**31, 2**31 - 1, (need // 4 + 4,), dtype=T.int32, device="cuda",
                       generator=gen)
        assert int((ws[:COUNTER_BYTES // 4] != 0).sum()) > 0
        tp.workspace_reset(ws)
        outs = []
        for w in (None, ws, ws):
            H = empty((I, L["F"] // L["t"]), "bf16")
            P = empty((I, L["D"]), "f32")
            tp.shard_mlp(X, *L["shards"][5], H, P, workspace=w)
            outs.append((H, P))
        T.cuda.synchronize()
        for o in outs[1:]:
            assert T.equal(outs[0][0], o[0]) and T.equal(outs[0][1], o[1]), I
        assert int(ws[:COUNTER_BYTES // 4].abs().sum()) == 0, I
        with pytest.raises(tp.TPError, match="WORKSPACE"):
            tp.shard_mlp(X, *L["shards"][5], outs[0][0], outs[0][1], workspace=ws[:8])


def test_binding_workspace_per_stream(llama_mlp):
    """The binding keeps one workspace per (device, stream): calls on two
    streams, each waiting only for its own inputs, give the bits of the
    same calls on the default stream."""
    L = llama_mlp
    T = torch()
    I = 32
    X = to_dev(datagen.gaussian("X", (I, L["D"]), 1.0, "bf16", 78), "bf16")
    ref = []
    for r in (2, 6):
        H = empty((I, L["F"] // L["t"]), "bf16")
        P = empty((I, L["D"]), "f32")
        tp.shard_mlp(X, *L["shards"][r], H, P)
        ref.append((H, P))
    T.cuda.synchronize()
    streams = [T.cuda.Stream(), T.cuda.Stream()]
    got = []
    for s, r in zip(streams, (2, 6)):
        H = empty((I, L["F"] // L["t"]), "bf16")
        P = empty((I, L["D"]), "f32")
        s.wait_stream(T.cuda.current_stream())
        with T.cuda.stream(s):
            for _ in range(3):
                tp.shard_mlp(X, *L["shards"][r], H, P)
        got.append((H, P))
    T.cuda.synchronize()
    for (h0, p0), (h1, p1) in zip(ref, got):
        assert T.equal(h0, h1) and T.equal(p0, p1)
