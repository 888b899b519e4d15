"""Plain fp64 CPU oracle for one tensor-parallel rank's layer share.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the CPU-baseline
leg of the benchmark are the only users.  The product path never imports it.

``oracle.c`` holds the arithmetic (fp64, increasing-index sums, OpenMP over
independent outputs); this module only marshals numpy arrays to float64 and
calls it through ctypes.  Functions take the FULL (unsharded) weights plus the
rank (t, r) and cut the rank's block themselves, so their slicing is
independent of the harness that prepares per-rank GPU buffers.
"""
from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess

import numpy as np

HERE = pathlib.Path(__file__).resolve().parent
SRC = HERE / "oracle.c"
LIB = HERE / "liboracle.so"

CFLAGS = ["-O2", "-fopenmp", "-fno-fast-math", "-ffp-contract=off", "-fPIC",
          "-shared", "-std=c11", "-Wall"]

_i64 = ctypes.c_int64
_pd = ctypes.POINTER(ctypes.c_double)
_pi64 = ctypes.POINTER(ctypes.c_int64)


def build(src: pathlib.Path = SRC, out: pathlib.Path = LIB) -> pathlib.Path:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = out.with_suffix(".so.tmp")
    subprocess.run(["gcc", *CFLAGS, str(src), "-o", str(tmp), "-lm"], check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: pathlib.Path | str = LIB):
        path = pathlib.Path(path)
        if not path.exists():
            build(out=path)
        self.lib = lib = ctypes.CDLL(str(path))
        lib.orc_silu.restype = ctypes.c_double
        lib.orc_silu.argtypes = [ctypes.c_double]
        lib.orc_shard_range.restype = None
        lib.orc_shard_range.argtypes = [_i64, _i64, _i64, _pi64, _pi64]
        lib.orc_mlp_rank.restype = None
        lib.orc_mlp_rank.argtypes = [_i64] * 5 + [_pd] * 6 + [_pi64, _i64]
        lib.orc_bf16_round.restype = ctypes.c_double
        lib.orc_bf16_round.argtypes = [ctypes.c_double]
        lib.orc_bf16_round_array.restype = None
        lib.orc_bf16_round_array.argtypes = [_i64, _pd, _pd]
        lib.orc_mlp_rank_bf16h.restype = None
        lib.orc_mlp_rank_bf16h.argtypes = [_i64] * 5 + [_pd] * 8 + [_pi64, _i64]
        lib.orc_reduce.restype = None
        lib.orc_reduce.argtypes = [_i64, _i64, _pd, _pd]
        lib.orc_qkv_rank.restype = None
        lib.orc_qkv_rank.argtypes = [_i64] * 7 + [_pd] * 5
        lib.orc_attn_core.restype = None
        lib.orc_attn_core.argtypes = [_i64] * 5 + [_pd] * 2
        lib.orc_oproj_rank.restype = None
        lib.orc_oproj_rank.argtypes = [_i64] * 6 + [_pd] * 3
        lib.orc_attn_decode.restype = None
        lib.orc_attn_decode.argtypes = [_i64] * 5 + [ctypes.POINTER(ctypes.c_int)] + [_pd] * 4
        lib.orc_e4m3.restype = ctypes.c_double
        lib.orc_e4m3.argtypes = [ctypes.c_ubyte]
        lib.orc_dequant_fp8.restype = None
        lib.orc_dequant_fp8.argtypes = [_i64, _i64, ctypes.POINTER(ctypes.c_ubyte), _pd, _pd]
        lib.orc_dequant_int8.restype = None
        lib.orc_dequant_int8.argtypes = [_i64, _i64, ctypes.POINTER(ctypes.c_byte), _pd, _pd]
        lib.orc_residual_rmsnorm.restype = None
        lib.orc_residual_rmsnorm.argtypes = [_i64] * 3 + [_pd] * 3 + [ctypes.c_double, _pd, _pd]

    # ------------------------------------------------------------ helpers
    @staticmethod
    def _f64(a) -> np.ndarray:
        return np.ascontiguousarray(a, dtype=np.float64)

    @staticmethod
    def _p(a: np.ndarray):
        return a.ctypes.data_as(_pd)

    # ------------------------------------------------------------ API
    def silu(self, z: float) -> float:
        return self.lib.orc_silu(float(z))

    def shard_range(self, n: int, t: int, r: int):
        lo, hi = ctypes.c_int64(), ctypes.c_int64()
        self.lib.orc_shard_range(n, t, r, ctypes.byref(lo), ctypes.byref(hi))
        return lo.value, hi.value

    def mlp_rank(self, X, Wg, Wu, Wd, t: int = 1, r: int = 0, rows=None):
        """Rank r's (H_r [I', F/t], P_r [I', D]) from full weights; rows selects
        a subset of token rows (I' = len(rows)), None = all."""
        X, Wg, Wu, Wd = (self._f64(a) for a in (X, Wg, Wu, Wd))
        I, D = X.shape
        F = Wg.shape[0]
        assert Wg.shape == (F, D) and Wu.shape == (F, D) and Wd.shape == (D, F)
        assert F % t == 0 and 0 <= r < t
        if rows is None:
            n_out, rp = I, None
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            assert rows.min() >= 0 and rows.max() < I
            n_out, rp = len(rows), rows.ctypes.data_as(_pi64)
        H = np.empty((n_out, F // t))
        P = np.empty((n_out, D))
        self.lib.orc_mlp_rank(I, D, F, t, r, self._p(X), self._p(Wg), self._p(Wu),
                              self._p(Wd), self._p(H), self._p(P), rp, n_out)
        return H, P

    def mlp_rank_bf16h(self, X, Wg, Wu, Wd, t: int = 1, r: int = 0, rows=None):
        """(H, P, Hb, Pb): mlp_rank's H and P, plus H rounded to bf16 as the
        device stores it and the partial computed from that rounded H."""
        X, Wg, Wu, Wd = (self._f64(a) for a in (X, Wg, Wu, Wd))
        I, D = X.shape
        F = Wg.shape[0]
        assert Wg.shape == (F, D) and Wu.shape == (F, D) and Wd.shape == (D, F)
        assert F % t == 0 and 0 <= r < t
        if rows is None:
            n_out, rp = I, None
        else:
            rows = np.ascontiguousarray(rows, dtype=np.int64)
            assert rows.min() >= 0 and rows.max() < I
            n_out, rp = len(rows), rows.ctypes.data_as(_pi64)
        H, Hb = np.empty((n_out, F // t)), np.empty((n_out, F // t))
        P, Pb = np.empty((n_out, D)), np.empty((n_out, D))
        self.lib.orc_mlp_rank_bf16h(I, D, F, t, r, self._p(X), self._p(Wg), self._p(Wu),
                                    self._p(Wd), self._p(H), self._p(P), self._p(Hb),
                                    self._p(Pb), rp, n_out)
        return H, P, Hb, Pb

    def bf16_round(self, a):
        """Nearest bfloat16 value of each element (ties to even), as float64."""
        if np.isscalar(a):
            return self.lib.orc_bf16_round(float(a))
        a = self._f64(a)
        out = np.empty_like(a)
        self.lib.orc_bf16_round_array(a.size, self._p(a), self._p(out))
        return out

    def mlp_full(self, X, Wg, Wu, Wd, rows=None):
        return self.mlp_rank(X, Wg, Wu, Wd, 1, 0, rows)

    def reduce(self, partials) -> np.ndarray:
        P = self._f64(partials)
        t = P.shape[0]
        n = P[0].size
        Y = np.empty(P.shape[1:])
        self.lib.orc_reduce(t, n, self._p(P), self._p(Y))
        return Y

    def qkv_rank(self, X, Wq, Wk, Wv, n_q: int, n_kv: int, hd: int, t: int = 1,
                 r: int = 0) -> np.ndarray:
        X, Wq, Wk, Wv = (self._f64(a) for a in (X, Wq, Wk, Wv))
        I, D = X.shape
        assert Wq.shape == (n_q * hd, D) and Wk.shape == (n_kv * hd, D)
        assert Wv.shape == (n_kv * hd, D)
        assert n_q % t == 0 and n_kv % t == 0
        N = (n_q // t + 2 * (n_kv // t)) * hd
        out = np.empty((I, N))
        self.lib.orc_qkv_rank(I, D, n_q, n_kv, hd, t, r, self._p(X), self._p(Wq),
                              self._p(Wk), self._p(Wv), self._p(out))
        return out

    def attn_core(self, qkv, S: int, nq_l: int, nkv_l: int, hd: int) -> np.ndarray:
        qkv = self._f64(qkv)
        I = qkv.shape[0]
        assert qkv.shape[1] == (nq_l + 2 * nkv_l) * hd and I % S == 0
        A = np.empty((I, nq_l * hd))
        self.lib.orc_attn_core(I, S, nq_l, nkv_l, hd, self._p(qkv), self._p(A))
        return A

    def oproj_rank(self, A_r, Wo, n_q: int, hd: int, t: int = 1, r: int = 0):
        A_r, Wo = self._f64(A_r), self._f64(Wo)
        I = A_r.shape[0]
        D = Wo.shape[0]
        assert Wo.shape == (D, n_q * hd) and A_r.shape[1] == (n_q // t) * hd
        P = np.empty((I, D))
        self.lib.orc_oproj_rank(I, D, n_q, hd, t, r, self._p(A_r), self._p(Wo),
                                self._p(P))
        return P

    def attn_decode(self, qkv, Kc, Vc, lens, nq_l: int, nkv_l: int, hd: int) -> np.ndarray:
        """Decode attention over the KV cache: positions < lens[b]-1 from Kc/Vc
        [B, nkv_l, Lmax, hd], position lens[b]-1 from the new token's k, v in qkv."""
        Q, K, V = self._f64(qkv), self._f64(Kc), self._f64(Vc)
        B, _, Lmax, _ = K.shape
        ln = np.ascontiguousarray(lens, dtype=np.int32)
        assert ln.min() >= 1 and ln.max() <= Lmax
        A = np.empty((B, nq_l * hd))
        self.lib.orc_attn_decode(B, nq_l, nkv_l, hd, Lmax,
                                 ln.ctypes.data_as(ctypes.POINTER(ctypes.c_int)), self._p(Q),
                                 self._p(K), self._p(V), self._p(A))
        return A

    # ------------------------------------------------------------ chains
    def attn_block_rank(self, X, Wq, Wk, Wv, Wo, n_q, n_kv, hd, S, t=1, r=0):
        """QKV (column) -> attention core -> o_proj (row): rank r's partial."""
        qkv = self.qkv_rank(X, Wq, Wk, Wv, n_q, n_kv, hd, t, r)
        A = self.attn_core(qkv, S, n_q // t, n_kv // t, hd)
        return qkv, A, self.oproj_rank(A, Wo, n_q, hd, t, r)

    # ------------------------------------------------------------ FP8 weights
    def e4m3(self, code: int) -> float:
        return self.lib.orc_e4m3(code)

    def dequant_fp8(self, codes, scales) -> np.ndarray:
        """W[n, k] = scales[n] * e4m3(codes[n, k]) (fp64)."""
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        sc = self._f64(scales)
        N, K = c.shape
        W = np.empty((N, K))
        self.lib.orc_dequant_fp8(N, K, c.ctypes.data_as(ctypes.POINTER(ctypes.c_ubyte)),
                                 self._p(sc), self._p(W))
        return W

    def dequant_int8(self, codes, scales) -> np.ndarray:
        """W[n, k] = scales[n] * codes[n, k] for int8 codes (fp64)."""
        c = np.ascontiguousarray(codes, dtype=np.int8)
        sc = self._f64(scales)
        N, K = c.shape
        W = np.empty((N, K))
        self.lib.orc_dequant_int8(N, K, c.ctypes.data_as(ctypes.POINTER(ctypes.c_byte)),
                                  self._p(sc), self._p(W))
        return W

    # ------------------------------------------------------------ around the block
    def residual_rmsnorm(self, partials, residual, gamma=None, eps: float = 1e-5):
        """h = residual + sum_r partials[r] and x = RMSNorm(h) * gamma.
        partials [t, I, D] or None (t = 0); residual [I, D] or None (zero);
        gamma None: returns (h, None)."""
        if partials is None and residual is None:
            raise ValueError("need partials or a residual")
        if partials is not None:
            P = self._f64(partials)
            t, I, D = P.shape
        else:
            P, t = None, 0
            I, D = np.asarray(residual).shape
        R = self._f64(residual) if residual is not None else None
        G = self._f64(gamma) if gamma is not None else None
        h = np.zeros((I, D))
        x = np.zeros((I, D)) if G is not None else None
        self.lib.orc_residual_rmsnorm(t, I, D, self._p(P) if P is not None else None,
                                      self._p(R) if R is not None else None,
                                      self._p(G) if G is not None else None, float(eps),
                                      self._p(h), self._p(x) if x is not None else None)
        return h, x


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``oracle.c`` in this directory."""
    global _default
    if _default is None:
        _default = Oracle(LIB)
    return _default


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all CPUs it may run on)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env:
        return int(env)
    return len(os.sched_getaffinity(0))
