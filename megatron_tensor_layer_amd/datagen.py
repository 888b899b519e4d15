"""Seeded synthetic inputs for one tensor-parallel rank's layer share.

This module draws the inputs that both the HIP path and the CPU oracle
consume.  It holds none of the layer's arithmetic: it only draws Gaussians,
rounds them to the storage type and cuts rank shards out of full tensors.

Recipe (the same for every consumer):

* Tensor ``name`` of workload pool ``pool`` is drawn in chunks of 2**24
  consecutive elements (row-major order); chunk k comes from numpy's PCG64
  generator seeded with ``SeedSequence([42, TENSOR_IDS[name], pool, k])``, so
  chunks can be drawn in parallel and the result does not depend on the
  thread count.  The base 42 echoes the shared default sampling seed of the
  Pico-vLLM TP post (koas-w blog, "Engine" section).
* Activations are N(0, 1); every weight matrix is N(0, 1/D) (variance 1/D,
  sigma = D**-0.5, D the model width), drawn in float32 with numpy's ziggurat
  normal sampler, scaled in float32.
* bf16 tensors are rounded from float32 to the nearest bf16, ties to even,
  and returned as float32 arrays whose values are exactly bf16-representable
  (``bf16_bits`` gives the 16-bit patterns for upload).  fp32 tensors are
  returned as drawn.
* Full tensors are drawn first and rank shards are contiguous slices of them,
  so the union of the shards is exactly the unsharded weight.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BASE_SEED = 42

TENSOR_IDS = {
    "X": 0,        # layer input [I, D]
    "W_gate": 1,   # [F, D]  output-major logical W_gate[D, F]
    "W_up": 2,     # [F, D]
    "W_down": 3,   # [D, F]  output-major logical W_down[F, D]
    "W_q": 4,      # [n_q*hd, D]
    "W_k": 5,      # [n_kv*hd, D]
    "W_v": 6,      # [n_kv*hd, D]
    "W_o": 7,      # [D, n_q*hd]
    "A": 8,        # stand-alone attention output [I, n_q*hd] (o_proj-only cases)
    "P": 9,        # stand-alone row-parallel partials [t, I, D] (reduce / norm cases)
    "h": 10,       # residual stream [I, D]
    "gamma": 11,   # RMSNorm scale [D]: 1 + N(0, sigma^2), near 1 like trained scales
    "W_gate8": 12, "W_up8": 13, "W_down8": 14,  # FP8 weight-only MLP shards
}

_CHUNK = 1 << 24  # elements per draw, bounds the temporaries of the rounding


def _round_to_bf16_inplace(a: np.ndarray) -> None:
    """float32 -> nearest bf16 (ties to even), kept in a float32 container."""
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    u += np.uint32(0x7FFF) + lsb
    u &= np.uint32(0xFFFF0000)


def gaussian(name: str, shape, sigma: float = 1.0, dtype: str = "bf16",
             pool: int = 0) -> np.ndarray:
    """Seeded N(0, sigma^2) tensor, rounded to ``dtype`` ("bf16" or "f32").

    Returned as a C-contiguous float32 array."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"unsupported dtype {dtype!r}")
    shape = tuple(int(s) for s in shape)
    n = int(np.prod(shape)) if shape else 1
    out = np.empty(n, dtype=np.float32)
    s = np.float32(sigma)

    def draw(k: int) -> None:
        lo, hi = k * _CHUNK, min(n, (k + 1) * _CHUNK)
        rng = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence([BASE_SEED, TENSOR_IDS[name], int(pool), k])))
        blk = out[lo:hi]
        rng.standard_normal(out=blk, dtype=np.float32)
        if s != np.float32(1.0):
            blk *= s
        if dtype == "bf16":
            _round_to_bf16_inplace(blk)

    nchunks = (n + _CHUNK - 1) // _CHUNK
    if nchunks <= 1:
        for k in range(nchunks):
            draw(k)
    else:
        workers = min(nchunks, len(os.sched_getaffinity(0)), 16)
        with ThreadPoolExecutor(workers) as ex:
            list(ex.map(draw, range(nchunks)))
    return out.reshape(shape)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """16-bit patterns of a float32 array whose values are bf16-representable."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    if np.any(u & np.uint32(0xFFFF)):
        raise ValueError("array holds values that are not bf16-representable")
    return (u >> 16).astype(np.uint16)


def rank_block(n: int, t: int, r: int) -> slice:
    """Contiguous block of rank r when a dimension of size n is split t ways."""
    if n % t:
        raise ValueError(f"{n} is not divisible by t={t}")
    step = n // t
    return slice(r * step, (r + 1) * step)


def mlp_weights(D: int, F: int, dtype: str = "bf16", pool: int = 0):
    """Full W_gate [F, D], W_up [F, D], W_down [D, F], all N(0, 1/D)."""
    sig = D ** -0.5
    return (gaussian("W_gate", (F, D), sig, dtype, pool),
            gaussian("W_up", (F, D), sig, dtype, pool),
            gaussian("W_down", (D, F), sig, dtype, pool))


def mlp_rank_shards(Wg, Wu, Wd, t: int, r: int):
    """Rank r's contiguous shards: gate/up rows F_r, down columns F_r."""
    F = Wg.shape[0]
    b = rank_block(F, t, r)
    return (np.ascontiguousarray(Wg[b]), np.ascontiguousarray(Wu[b]),
            np.ascontiguousarray(Wd[:, b]))


def attn_weights(D: int, n_q: int, n_kv: int, hd: int, dtype: str = "bf16",
                 pool: int = 0):
    """Full W_q [n_q*hd, D], W_k, W_v [n_kv*hd, D], W_o [D, n_q*hd]; N(0, 1/D)."""
    sig = D ** -0.5
    return (gaussian("W_q", (n_q * hd, D), sig, dtype, pool),
            gaussian("W_k", (n_kv * hd, D), sig, dtype, pool),
            gaussian("W_v", (n_kv * hd, D), sig, dtype, pool),
            gaussian("W_o", (D, n_q * hd), sig, dtype, pool))


def qkv_rank_shard(Wq, Wk, Wv, n_q: int, n_kv: int, hd: int, t: int, r: int):
    """Rank r's packed [q heads | k heads | v heads] weight, [N_qkv, D]."""
    bq = rank_block(n_q, t, r)
    bk = rank_block(n_kv, t, r)
    rows_q = slice(bq.start * hd, bq.stop * hd)
    rows_k = slice(bk.start * hd, bk.stop * hd)
    return np.ascontiguousarray(np.concatenate([Wq[rows_q], Wk[rows_k], Wv[rows_k]], axis=0))


def oproj_rank_shard(Wo, n_q: int, hd: int, t: int, r: int):
    """Rank r's W_o block: columns of its own heads, [D, (n_q/t)*hd]."""
    bq = rank_block(n_q, t, r)
    return np.ascontiguousarray(Wo[:, bq.start * hd:bq.stop * hd])


def rmsnorm_gamma(D: int, pool: int, dtype: str = "f32", sigma: float = 0.1) -> np.ndarray:
    """RMSNorm scale: 1 + N(0, sigma^2) per hidden unit, float32, rounded to
    bf16 (nearest-even) when dtype == 'bf16'."""
    g = (1.0 + gaussian("gamma", (D,), sigma, "f32", pool)).astype(np.float32)
    if dtype == "bf16":
        _round_to_bf16_inplace(g)
    return g


# Non-negative finite OCP E4M3 ("fn") values, in code order 0x00..0x7E (code
# order is value order); used only to encode synthetic weights.
_E4M3_POS = np.array([(m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
                      for e in range(16) for m in range(8)][:0x7F])


def fp8_weights(name: str, shape, sigma: float, pool: int):
    """Synthetic FP8 weight-only storage of an [N, K] matrix: N(0, sigma^2)
    weights, one fp32 scale per row (row absmax / 448, the largest E4M3
    value) and each weight / scale encoded as the nearest E4M3 code (ties to
    the even code).  Returns (codes uint8 [N, K], scales float32 [N])."""
    w = gaussian(name, shape, sigma, "f32", pool).astype(np.float64)
    amax = np.abs(w).max(axis=1)
    scales = (np.where(amax > 0, amax, 1.0) / 448.0).astype(np.float32)
    q = np.abs(w) / scales.astype(np.float64)[:, None]
    hi = np.clip(np.searchsorted(_E4M3_POS, q), 1, 0x7E)
    lo = hi - 1
    dlo, dhi = q - _E4M3_POS[lo], _E4M3_POS[hi] - q
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    codes = np.where(pick_hi, hi, lo).astype(np.uint8)
    codes |= np.where(w < 0, 0x80, 0).astype(np.uint8)
    return codes, scales


def fp8_mlp_weights(D: int, F: int, pool: int):
    """FP8 storage of a full MLP: (gate, up [F, D], down [D, F]) as
    (codes, scales) pairs, weights N(0, 1/D)."""
    sigma = D ** -0.5
    return (fp8_weights("W_gate8", (F, D), sigma, pool),
            fp8_weights("W_up8", (F, D), sigma, pool),
            fp8_weights("W_down8", (D, F), sigma, pool))


def int8_weights(name: str, shape, sigma: float, pool: int):
    """Synthetic int8 weight-only storage of an [N, K] matrix: N(0, sigma^2)
    weights, one fp32 scale per row (row absmax / 127) and each weight /
    scale rounded to the nearest integer (ties to even), which lies in
    [-127, 127].  Returns (codes int8 [N, K], scales float32 [N])."""
    w = gaussian(name, shape, sigma, "f32", pool).astype(np.float64)
    amax = np.abs(w).max(axis=1)
    scales = (np.where(amax > 0, amax, 1.0) / 127.0).astype(np.float32)
    q = np.rint(w / scales.astype(np.float64)[:, None])
    return np.clip(q, -127, 127).astype(np.int8), scales


def int8_mlp_weights(D: int, F: int, pool: int):
    """int8 storage of a full MLP: (gate, up [F, D], down [D, F]) as
    (codes, scales) pairs, weights N(0, 1/D)."""
    sigma = D ** -0.5
    return (int8_weights("W_gate8", (F, D), sigma, pool),
            int8_weights("W_up8", (F, D), sigma, pool),
            int8_weights("W_down8", (D, F), sigma, pool))


def fp8_mlp_rank_shards(fp8_full, t: int, r: int):
    """Rank r's contiguous F block of FP8 MLP storage: gate/up rows and down
    columns (the down scales are per output row, so they are shared)."""
    (cg, sg), (cu, su), (cd, sd) = fp8_full
    blk = rank_block(cg.shape[0], t, r)
    return ((np.ascontiguousarray(cg[blk]), sg[blk].copy()),
            (np.ascontiguousarray(cu[blk]), su[blk].copy()),
            (np.ascontiguousarray(cd[:, blk]), sd.copy()))
