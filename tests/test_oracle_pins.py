"""Pins of the fp64 CPU oracle against what the pages and mathematics fix.

Page 5 is "Lecture 4 - Distributed Serving" (cs349e notes).  The pages print no
numeric output of a sharded layer, so the oracle is pinned by:

* brute force in exact rational arithmetic on tiny shapes (P4),
* a textbook library routine, numpy float64 matmul (P5),
* the sharding invariants the lecture states: column shards concatenate to
  the full output (§3.2 case 1, §4.1), row-shard partials sum to it (§3.2
  case 3, §4.1, §4.3), attention heads are independent (§4.2) (P1-P3),
* closed forms: zero and one-hot inputs, SiLU identities, attention with one
  key or with zero queries (P6),
* sizes printed in the lecture's exercises (P7, in test_pages_pins.py).

Each pin is a plain function taking an oracle object, so test_oracle_mutants
can run the same pins against copies of the oracle with planted mistakes.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from megatron_tensor_layer_amd import datagen
from tests.common import normwise_err


# ---------------------------------------------------------------- inputs
def tiny_mlp(I=3, D=16, F=32, dtype="bf16", pool=0):
    X = datagen.gaussian("X", (I, D), 1.0, dtype, pool)
    Wg, Wu, Wd = datagen.mlp_weights(D, F, dtype, pool)
    return X, Wg, Wu, Wd


def tiny_attn(I=6, D=32, n_q=8, n_kv=4, hd=8, pool=0):
    X = datagen.gaussian("X", (I, D), 1.0, "bf16", pool)
    Wq, Wk, Wv, Wo = datagen.attn_weights(D, n_q, n_kv, hd, "bf16", pool)
    return X, Wq, Wk, Wv, Wo


def _silu_ref(z: float) -> float:
    # written out independently of the oracle: z * sigmoid(z)
    return z * (1.0 / (1.0 + math.exp(-z)))


# ---------------------------------------------------------------- pins
def pin_silu_closed_forms(orc):
    assert orc.silu(0.0) == 0.0
    for z in (0.25, 1.0, 2.5, 7.0, 19.0):
        # silu(-z) = silu(z) - z, because sigmoid(-z) = 1 - sigmoid(z)
        assert abs(orc.silu(-z) - (orc.silu(z) - z)) <= 1e-13 * max(1.0, z)
        assert abs(orc.silu(z) - _silu_ref(z)) <= 1e-15 * z
    assert abs(orc.silu(40.0) - 40.0) < 1e-12           # sigmoid -> 1
    assert abs(orc.silu(-40.0)) < 1e-15                  # sigmoid -> 0
    assert orc.silu(1.0) == pytest.approx(1.0 / (1.0 + math.e ** -1), rel=1e-15)


def pin_mlp_bruteforce_exact(orc):
    """P4: gate/up/down contractions in exact rationals, SiLU via math.exp."""
    for (I, D, F, t, pool) in ((3, 16, 32, 1, 0), (2, 16, 32, 2, 1), (3, 8, 16, 4, 2),
                               (1, 12, 24, 2, 3)):
        X, Wg, Wu, Wd = tiny_mlp(I, D, F, pool=pool)
        Xf = [[Fraction(float(v)) for v in row] for row in X]
        Wgf = [[Fraction(float(v)) for v in row] for row in Wg]
        Wuf = [[Fraction(float(v)) for v in row] for row in Wu]
        Wdf = [[Fraction(float(v)) for v in row] for row in Wd]
        Fl = F // t
        for r in range(t):
            H, P = orc.mlp_rank(X, Wg, Wu, Wd, t, r)
            Hx = np.zeros((I, Fl))
            Px = np.zeros((I, D))
            for i in range(I):
                hrow = []
                for fl in range(Fl):
                    f = r * Fl + fl          # rank r owns the r-th block of F
                    g = sum(Xf[i][d] * Wgf[f][d] for d in range(D))   # W_gate[d, f]
                    u = sum(Xf[i][d] * Wuf[f][d] for d in range(D))   # W_up[d, f]
                    h = Fraction(_silu_ref(float(g))) * u
                    hrow.append(h)
                    Hx[i, fl] = float(h)
                for n in range(D):
                    # W_down[f, n] is stored at Wd[n][f]
                    Px[i, n] = float(sum(hrow[fl] * Wdf[n][r * Fl + fl] for fl in range(Fl)))
            assert normwise_err(H, Hx) <= 1e-13, (I, D, F, t, r)
            assert normwise_err(P, Px) <= 1e-13, (I, D, F, t, r)


def pin_mlp_numpy_reference(orc):
    """P5: numpy float64 matmul of the plain definition, full layer."""
    for (I, D, F, dtype) in ((4, 256, 1024, "f32"), (8, 384, 1152, "bf16")):
        X, Wg, Wu, Wd = tiny_mlp(I, D, F, dtype)
        X64, Wg64, Wu64, Wd64 = (a.astype(np.float64) for a in (X, Wg, Wu, Wd))
        G = X64 @ Wg64.T
        U = X64 @ Wu64.T
        Href = G / (1.0 + np.exp(-G)) * U
        Yref = Href @ Wd64.T
        H, Y = orc.mlp_full(X, Wg, Wu, Wd)
        assert normwise_err(H, Href) <= 1e-12
        assert normwise_err(Y, Yref) <= 1e-12


def pin_column_shards_concatenate(orc):
    """P1: column-parallel gate/up (case 1): rank H blocks are the full H's
    columns, bit for bit (identical per-element loops)."""
    X, Wg, Wu, Wd = tiny_mlp(5, 64, 256, pool=7)
    H, _ = orc.mlp_full(X, Wg, Wu, Wd)
    for t in (2, 4, 8):
        Hs = [orc.mlp_rank(X, Wg, Wu, Wd, t, r)[0] for r in range(t)]
        assert np.array_equal(np.concatenate(Hs, axis=1), H), t


def pin_row_partials_sum(orc):
    """P2: row-parallel down (case 3): the t partials sum to the full output
    up to summation order; the reduce sums them in rank order."""
    X, Wg, Wu, Wd = tiny_mlp(5, 64, 256, pool=8)
    _, Y = orc.mlp_full(X, Wg, Wu, Wd)
    for t in (1, 2, 4, 8):
        Ps = np.stack([orc.mlp_rank(X, Wg, Wu, Wd, t, r)[1] for r in range(t)])
        Ysum = orc.reduce(Ps)
        assert normwise_err(Ysum, Y) <= 1e-12, t
        # the reduce itself: rank-order sum, checked against numpy's sum
        assert normwise_err(Ysum, Ps.sum(axis=0)) <= 1e-15, t
    # rank partials are genuinely partial (not each the whole output)
    P0 = orc.mlp_rank(X, Wg, Wu, Wd, 4, 0)[1]
    assert normwise_err(P0, Y) > 0.1


def pin_reduce_exact_small(orc):
    """The reduce on values whose sums are exact in binary fp."""
    P = np.array([[1.0, 2.0, -3.5], [0.25, -2.0, 3.5], [4.0, 0.0, 1.0]])
    assert np.array_equal(orc.reduce(P), np.array([5.25, 0.0, 1.0]))
    P4 = np.arange(24, dtype=np.float64).reshape(4, 2, 3)
    assert np.array_equal(orc.reduce(P4), P4.sum(axis=0))


def pin_mlp_closed_forms(orc):
    """P6: X = 0 gives H = 0 and P = 0; a one-hot X = e_k picks row k of the
    logical W_gate[D, F] (column k of the stored [F, D] array)."""
    _, Wg, Wu, Wd = tiny_mlp(1, 32, 64, pool=9)
    Z = np.zeros((2, 32))
    H, P = orc.mlp_full(Z, Wg, Wu, Wd)
    assert not H.any() and not P.any()
    for k in (0, 5, 31):
        X = np.zeros((1, 32))
        X[0, k] = 1.0
        H, P = orc.mlp_full(X, Wg, Wu, Wd)
        g = Wg[:, k].astype(np.float64)
        u = Wu[:, k].astype(np.float64)
        h = np.array([_silu_ref(v) for v in g]) * u
        assert normwise_err(H[0], h) <= 1e-15
        p = np.array([sum(h[f] * float(Wd[n, f]) for f in range(64)) for n in range(32)])
        assert normwise_err(P[0], p) <= 1e-13
        # scaling X by 2 is not linear through SiLU: the oracle must see that
        H2, _ = orc.mlp_full(2 * X, Wg, Wu, Wd)
        assert normwise_err(H2[0], 2 * h) > 1e-3


def pin_row_subset(orc):
    """Computing selected token rows equals those rows of the full call."""
    X, Wg, Wu, Wd = tiny_mlp(7, 32, 64, pool=10)
    H, P = orc.mlp_rank(X, Wg, Wu, Wd, 2, 1)
    rows = [6, 0, 3]
    Hs, Ps = orc.mlp_rank(X, Wg, Wu, Wd, 2, 1, rows=rows)
    assert np.array_equal(Hs, H[rows]) and np.array_equal(Ps, P[rows])


def _attn_bruteforce(qkv, S, nq, nkv, hd):
    """Causal grouped-query softmax attention, pure Python with math.exp."""
    I = qkv.shape[0]
    A = np.zeros((I, nq * hd))
    for i in range(I):
        s0 = (i // S) * S
        for j in range(nq):
            g = (j * nkv) // nq
            q = qkv[i, j * hd:(j + 1) * hd]
            scores = []
            for p in range(s0, i + 1):
                k = qkv[p, (nq + g) * hd:(nq + g + 1) * hd]
                scores.append(sum(float(a) * float(b) for a, b in zip(q, k)) / math.sqrt(hd))
            m = max(scores)
            e = [math.exp(s - m) for s in scores]
            z = sum(e)
            for c in range(hd):
                A[i, j * hd + c] = sum(e[p - s0] / z * float(qkv[p, (nq + nkv + g) * hd + c])
                                       for p in range(s0, i + 1))
    return A


def pin_attention(orc):
    nq, nkv, hd = 4, 2, 8
    rng = np.random.default_rng(5)
    qkv = rng.standard_normal((6, (nq + 2 * nkv) * hd))
    # brute force, two sequences of 3
    assert normwise_err(orc.attn_core(qkv, 3, nq, nkv, hd),
                        _attn_bruteforce(qkv, 3, nq, nkv, hd)) <= 1e-13
    # one token per sequence: A is the value of the head's group, exactly
    A1 = orc.attn_core(qkv, 1, nq, nkv, hd)
    for j in range(nq):
        g = (j * nkv) // nq
        assert np.array_equal(A1[:, j * hd:(j + 1) * hd],
                              qkv[:, (nq + nkv + g) * hd:(nq + nkv + g + 1) * hd])
    # zero queries: uniform weights, A_i = mean of values up to i
    q0 = qkv.copy()
    q0[:, :nq * hd] = 0.0
    A0 = orc.attn_core(q0, 6, nq, nkv, hd)
    for j in range(nq):
        g = (j * nkv) // nq
        V = q0[:, (nq + nkv + g) * hd:(nq + nkv + g + 1) * hd]
        means = np.cumsum(V, axis=0) / np.arange(1, 7)[:, None]
        assert normwise_err(A0[:, j * hd:(j + 1) * hd], means) <= 1e-14
    # causality: changing the last token's keys/values leaves earlier rows alone
    q2 = qkv.copy()
    q2[5, nq * hd:] += 3.0
    A2 = orc.attn_core(q2, 6, nq, nkv, hd)
    Af = orc.attn_core(qkv, 6, nq, nkv, hd)
    assert np.array_equal(A2[:5], Af[:5]) and not np.array_equal(A2[5], Af[5])


def pin_qkv_column_shards(orc):
    """QKV split by heads (lecture §4.2): rank blocks are the full projection's
    head columns, bit for bit; full = X @ [Wq; Wk; Wv]^T."""
    n_q, n_kv, hd = 8, 4, 8
    X, Wq, Wk, Wv, _ = tiny_attn(5, 32, n_q, n_kv, hd, pool=11)
    full = orc.qkv_rank(X, Wq, Wk, Wv, n_q, n_kv, hd)
    X64 = X.astype(np.float64)
    ref = X64 @ np.concatenate([Wq, Wk, Wv]).astype(np.float64).T
    assert normwise_err(full, ref) <= 1e-13
    Q, K, V = full[:, :n_q * hd], full[:, n_q * hd:(n_q + n_kv) * hd], full[:, (n_q + n_kv) * hd:]
    for t in (2, 4):
        parts = [orc.qkv_rank(X, Wq, Wk, Wv, n_q, n_kv, hd, t, r) for r in range(t)]
        nql, nkl = n_q // t * hd, n_kv // t * hd
        assert np.array_equal(np.concatenate([p[:, :nql] for p in parts], 1), Q)
        assert np.array_equal(np.concatenate([p[:, nql:nql + nkl] for p in parts], 1), K)
        assert np.array_equal(np.concatenate([p[:, nql + nkl:] for p in parts], 1), V)


def pin_oproj_row_partials(orc):
    """o_proj split by rows: partials of each rank's heads sum to A @ Wo^T."""
    n_q, hd, D = 8, 8, 32
    rng = np.random.default_rng(12)
    A = rng.standard_normal((5, n_q * hd))
    Wo = datagen.gaussian("W_o", (D, n_q * hd), D ** -0.5, "bf16", 12)
    full = orc.oproj_rank(A, Wo, n_q, hd)
    assert normwise_err(full, A @ Wo.astype(np.float64).T) <= 1e-13
    for t in (2, 4, 8):
        parts = np.stack([orc.oproj_rank(A[:, r * (n_q // t) * hd:(r + 1) * (n_q // t) * hd],
                                         Wo, n_q, hd, t, r) for r in range(t)])
        assert normwise_err(orc.reduce(parts), full) <= 1e-12


def pin_attention_block_sharded_equals_full(orc):
    """Lecture §4.2/§4.3: with heads split over t ranks, the reduced partials
    of QKV -> attention -> o_proj equal the single-device block."""
    n_q, n_kv, hd, D = 8, 4, 8, 32
    X, Wq, Wk, Wv, Wo = tiny_attn(6, D, n_q, n_kv, hd, pool=13)
    _, _, full = orc.attn_block_rank(X, Wq, Wk, Wv, Wo, n_q, n_kv, hd, S=6)
    for t in (2, 4):
        parts = np.stack([orc.attn_block_rank(X, Wq, Wk, Wv, Wo, n_q, n_kv, hd, 6, t, r)[2]
                          for r in range(t)])
        assert normwise_err(orc.reduce(parts), full) <= 1e-12, t


def _residual_rmsnorm_decimal(P, R, g, eps):
    """Independent brute force in 40-digit decimal arithmetic."""
    from decimal import Decimal, getcontext
    getcontext().prec = 40
    t, I, D = P.shape
    h = [[Decimal(float(R[i, j])) + sum(Decimal(float(P[r, i, j])) for r in range(t))
          for j in range(D)] for i in range(I)]
    x = []
    for i in range(I):
        ms = sum(v * v for v in h[i]) / D
        inv = 1 / (ms + Decimal(eps)).sqrt()
        x.append([h[i][j] * inv * Decimal(float(g[j])) for j in range(D)])
    return (np.array([[float(v) for v in row] for row in h]),
            np.array([[float(v) for v in row] for row in x]))


def pin_residual_rmsnorm_bruteforce(orc):
    """Residual add + RMSNorm (standard definition: the pages name RMSNorm,
    replicated on every rank, without spelling it out) against a 40-digit
    decimal evaluation of the same definition."""
    rng = np.random.default_rng(11)
    for t, I, D, eps in ((3, 2, 7, 1e-5), (1, 3, 16, 0.5), (2, 1, 5, 1e-6)):
        P = rng.standard_normal((t, I, D))
        R = rng.standard_normal((I, D))
        g = rng.uniform(0.5, 1.5, D)
        h, x = orc.residual_rmsnorm(P, R, g, eps)
        hb, xb = _residual_rmsnorm_decimal(P, R, g, eps)
        assert np.allclose(h, hb, rtol=1e-14, atol=1e-14)
        assert np.allclose(x, xb, rtol=1e-13, atol=1e-14)


def pin_rmsnorm_closed_forms(orc):
    """A constant row c gives x_j = c g_j / sqrt(c^2 + eps); with eps = 0 the
    result is invariant to scaling the row; mean_j (x_j / g_j)^2 equals
    ms / (ms + eps); no partials leave the residual, no residual leaves the
    rank-order sum (exact small values)."""
    D = 16
    g = np.linspace(0.5, 2.0, D)
    for c, eps in ((3.0, 0.25), (-2.0, 1e-5), (0.5, 0.0)):
        _, x = orc.residual_rmsnorm(None, np.full((1, D), c), g, eps)
        assert np.allclose(x[0], c * g / math.sqrt(c * c + eps), rtol=1e-15)
    rng = np.random.default_rng(3)
    R = rng.standard_normal((4, D))
    _, x1 = orc.residual_rmsnorm(None, R, g, 0.0)
    _, x3 = orc.residual_rmsnorm(None, 3.0 * R, g, 0.0)
    assert np.allclose(x1, x3, rtol=1e-14)
    eps = 0.3
    _, x = orc.residual_rmsnorm(None, R, g, eps)
    ms = (R ** 2).mean(axis=1)
    assert np.allclose(((x / g) ** 2).mean(axis=1), ms / (ms + eps), rtol=1e-14)
    h, xn = orc.residual_rmsnorm(None, R, None)
    assert np.array_equal(h, R) and xn is None
    P = np.arange(2 * 3 * 4, dtype=np.float64).reshape(2, 3, 4) - 7.0
    Rs = np.full((3, 4), 0.5)
    h, _ = orc.residual_rmsnorm(P, None)
    assert np.array_equal(h, P.sum(axis=0))
    h, _ = orc.residual_rmsnorm(P, Rs)
    assert np.array_equal(h, P.sum(axis=0) + 0.5)


def _e4m3_fraction(code: int):
    """The E4M3 "fn" value of a byte as an exact Fraction (None for NaN),
    written from the format's definition."""
    sign = -1 if code & 0x80 else 1
    exp, man = (code >> 3) & 0xF, code & 0x7
    if exp == 0xF and man == 0x7:
        return None
    if exp == 0:
        return sign * Fraction(man, 8) * Fraction(1, 2 ** 6)
    return sign * (1 + Fraction(man, 8)) * (Fraction(2) ** (exp - 7))


def pin_fp8_decode(orc):
    """All 256 codes against the exact definition; closed forms (1, 2, 448 the
    largest, 2^-9 the smallest subnormal, 2^-6 the smallest normal, -0, NaN);
    positive codes increase monotonically."""
    for c in range(256):
        ref = _e4m3_fraction(c)
        v = orc.e4m3(c)
        if ref is None:
            assert math.isnan(v), c
        else:
            assert Fraction(v) == ref, (c, v, ref)
    assert orc.e4m3(0x38) == 1.0 and orc.e4m3(0x40) == 2.0 and orc.e4m3(0x7E) == 448.0
    assert orc.e4m3(0x01) == 2.0 ** -9 and orc.e4m3(0x08) == 2.0 ** -6
    assert orc.e4m3(0x80) == 0.0 and math.copysign(1.0, orc.e4m3(0x80)) == -1.0
    assert math.isnan(orc.e4m3(0x7F)) and math.isnan(orc.e4m3(0xFF))
    pos = [orc.e4m3(c) for c in range(0x7F)]
    assert all(a < b for a, b in zip(pos, pos[1:]))


def pin_fp8_dequant_rows(orc):
    """Each row scales its decoded codes by its own scale."""
    codes = np.array([[0x38, 0x40, 0xB8, 0x00], [0x7E, 0x01, 0x08, 0x30]], dtype=np.uint8)
    W = orc.dequant_fp8(codes, [0.5, -2.0])
    ref = np.array([[0.5, 1.0, -0.5, 0.0], [-896.0, -2.0 ** -8, -2.0 ** -5, -1.0]])
    assert np.array_equal(W, ref)


def pin_int8_dequant_rows(orc):
    """int8 weight-only storage: each row scales its signed codes by its own
    scale, over the whole code range (two's complement bytes)."""
    codes = np.array([[-128, -1, 0, 1], [127, 64, -64, 5]], dtype=np.int8)
    W = orc.dequant_int8(codes, [0.5, -2.0])
    ref = np.array([[-64.0, -0.5, 0.0, 0.5], [-254.0, -128.0, 128.0, -10.0]])
    assert np.array_equal(W, ref)
    allc = np.arange(-128, 128, dtype=np.int8).reshape(2, 128)
    W = orc.dequant_int8(allc, [1.0, 3.0])
    assert np.array_equal(W[0], np.arange(-128, 0, dtype=np.float64))
    assert np.array_equal(W[1], 3.0 * np.arange(0, 128, dtype=np.float64))


def pin_sequence_shards_concatenate(orc):
    """Sequence parallelism (reduce-scatter, norm on each rank's rows,
    all-gather) gives the all-reduce layout's values: the residual update and
    RMSNorm act row by row, so rank blocks of rows concatenate bit for bit."""
    rng = np.random.default_rng(5)
    t, I, D = 4, 8, 12
    P = rng.standard_normal((t, I, D))
    R = rng.standard_normal((I, D))
    g = rng.uniform(0.5, 1.5, D)
    h, x = orc.residual_rmsnorm(P, R, g, 1e-5)
    hs, xs = [], []
    for r in range(t):
        rows = slice(r * I // t, (r + 1) * I // t)
        a, b = orc.residual_rmsnorm(P[:, rows], R[rows], g, 1e-5)
        hs.append(a)
        xs.append(b)
    assert np.array_equal(np.concatenate(hs), h) and np.array_equal(np.concatenate(xs), x)


def _decode_case(rng, B, nq, nkv, hd, Lmax, lens):
    """qkv of the new tokens and caches whose entries past each sequence's
    previous tokens hold NaN (they must never be read)."""
    N = (nq + 2 * nkv) * hd
    qkv = rng.standard_normal((B, N))
    Kc = np.full((B, nkv, Lmax, hd), np.nan)
    Vc = np.full((B, nkv, Lmax, hd), np.nan)
    for b, L in enumerate(lens):
        Kc[b, :, :L - 1] = rng.standard_normal((nkv, L - 1, hd))
        Vc[b, :, :L - 1] = rng.standard_normal((nkv, L - 1, hd))
    return qkv, Kc, Vc


def pin_attn_decode(orc):
    """Decode attention over the KV cache: one position gives the new token's
    v; equal keys give the mean of v; entries past lens[b] are never read;
    a cache filled with a causal sequence's first tokens reproduces the
    causal attention core's last row (itself pinned by brute force)."""
    rng = np.random.default_rng(21)
    nq, nkv, hd = 4, 2, 8
    qkv, Kc, Vc = _decode_case(rng, 3, nq, nkv, hd, 6, [1, 1, 1])
    A = orc.attn_decode(qkv, Kc, Vc, [1, 1, 1], nq, nkv, hd)
    for j in range(nq):
        g = j * nkv // nq
        assert np.array_equal(A[:, j * hd:(j + 1) * hd],
                              qkv[:, (nq + nkv + g) * hd:(nq + nkv + g + 1) * hd])
    qkv, Kc, Vc = _decode_case(rng, 2, nq, nkv, hd, 7, [5, 7])
    for b, L in enumerate([5, 7]):
        Kc[b, :, :L - 1] = qkv[b, nq * hd:(nq + nkv) * hd].reshape(nkv, 1, hd)
    A = orc.attn_decode(qkv, Kc, Vc, [5, 7], nq, nkv, hd)
    for b, L in enumerate([5, 7]):
        for j in range(nq):
            g = j * nkv // nq
            vs = np.concatenate([Vc[b, g, :L - 1],
                                 qkv[b, (nq + nkv + g) * hd:(nq + nkv + g + 1) * hd][None]])
            assert np.allclose(A[b, j * hd:(j + 1) * hd], vs.mean(axis=0), rtol=1e-13, atol=1e-14)
    S = 9
    seq = rng.standard_normal((S, (nq + 2 * nkv) * hd))
    Kc = np.full((1, nkv, 12, hd), np.nan)
    Vc = np.full((1, nkv, 12, hd), np.nan)
    for g in range(nkv):
        Kc[0, g, :S - 1] = seq[:S - 1, (nq + g) * hd:(nq + g + 1) * hd]
        Vc[0, g, :S - 1] = seq[:S - 1, (nq + nkv + g) * hd:(nq + nkv + g + 1) * hd]
    A = orc.attn_decode(seq[S - 1:], Kc, Vc, [S], nq, nkv, hd)
    ref = orc.attn_core(seq, S, nq, nkv, hd)[S - 1]
    assert np.allclose(A[0], ref, rtol=1e-12, atol=1e-13)


def _bf16_round_ref(x: float) -> float:
    """Nearest bfloat16 value by enumeration, written out independently of the
    oracle: bfloat16 values are the float32 values whose low 16 bits are
    zero; take the candidates around x, keep the nearest in exact rationals,
    ties to the candidate whose last kept bit (bit 16) is 0."""
    import struct
    if x == 0.0 or math.isnan(x) or math.isinf(x):
        return x
    sign = -1.0 if x < 0 else 1.0
    ax = abs(x)
    b32 = struct.unpack("<I", struct.pack("<f", ax))[0] & 0xFFFF0000
    cands = []
    for d in (-2, -1, 0, 1, 2):
        bits = b32 + d * 0x10000
        if 0 <= bits < 0x7F800000:
            cands.append((struct.unpack("<f", struct.pack("<I", bits))[0], bits))
    xf = Fraction(ax)
    best = min(cands, key=lambda c: (abs(Fraction(c[0]) - xf), (c[1] >> 16) & 1))
    return sign * best[0]


def pin_bf16_round(orc):
    """The rounding of bf16 intermediates: the enumeration above on values
    across the range (normal, below the smallest normal, exact ties), and
    hand-worked cases."""
    rng = np.random.default_rng(5)
    xs = list(rng.standard_normal(400) * np.exp(rng.uniform(-30, 30, 400)))
    xs += [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 3.0 * 2.0 ** -134,
           2.0 ** -126 * (1 + 2.0 ** -8), 1e-40, 65504.0, 1.0 / 3.0]
    for x in xs:
        assert orc.bf16_round(float(x)) == _bf16_round_ref(float(x)), x
    assert orc.bf16_round(1.0 + 2.0 ** -8) == 1.0                  # tie to even (down)
    assert orc.bf16_round(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6   # tie to even (up)
    assert orc.bf16_round(1.0 + 2.0 ** -8 + 2.0 ** -30) == 1.0 + 2.0 ** -7
    assert orc.bf16_round(-2.0) == -2.0 and orc.bf16_round(0.0) == 0.0
    a = np.array(xs[:50])
    assert np.array_equal(orc.bf16_round(a), [orc.bf16_round(float(v)) for v in a])


def pin_mlp_bf16h(orc):
    """The diagnostic form of the MLP share: H and P equal mlp_rank's bit for
    bit, Hb is H rounded to bf16 (enumeration reference), and Pb is the
    down projection of Hb in exact rationals."""
    for (I, D, F, t, r, pool) in ((3, 16, 32, 2, 1, 4), (2, 8, 16, 1, 0, 5), (1, 16, 64, 4, 3, 6)):
        X, Wg, Wu, Wd = tiny_mlp(I, D, F, pool=pool)
        H0, P0 = orc.mlp_rank(X, Wg, Wu, Wd, t, r)
        H, P, Hb, Pb = orc.mlp_rank_bf16h(X, Wg, Wu, Wd, t, r)
        assert np.array_equal(H, H0) and np.array_equal(P, P0)
        for i in range(I):
            for f in range(F // t):
                assert Hb[i, f] == _bf16_round_ref(float(H[i, f]))
        Fl = F // t
        for i in range(I):
            for n in range(D):
                exact = sum(Fraction(float(Hb[i, fl])) * Fraction(float(Wd[n, r * Fl + fl]))
                            for fl in range(Fl))
                assert abs(Pb[i, n] - float(exact)) <= 1e-14 * max(1.0, abs(float(exact)))
        rows = [I - 1, 0]
        _, _, Hs, Ps = orc.mlp_rank_bf16h(X, Wg, Wu, Wd, t, r, rows=rows)
        assert np.array_equal(Hs, Hb[rows]) and np.array_equal(Ps, Pb[rows])


ALL_PINS = [
    pin_silu_closed_forms,
    pin_mlp_bruteforce_exact,
    pin_mlp_numpy_reference,
    pin_column_shards_concatenate,
    pin_row_partials_sum,
    pin_reduce_exact_small,
    pin_mlp_closed_forms,
    pin_row_subset,
    pin_attention,
    pin_qkv_column_shards,
    pin_oproj_row_partials,
    pin_attention_block_sharded_equals_full,
    pin_residual_rmsnorm_bruteforce,
    pin_rmsnorm_closed_forms,
    pin_fp8_decode,
    pin_fp8_dequant_rows,
    pin_int8_dequant_rows,
    pin_sequence_shards_concatenate,
    pin_attn_decode,
    pin_bf16_round,
    pin_mlp_bf16h,
]


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)
