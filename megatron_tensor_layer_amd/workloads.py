"""Per-rank shapes of the benchmarked layers and their algorithmic work.

Work accounting (what the method must move or compute, not what a kernel
happens to move):

* FLOPs of one projection [I, K] x [K, N] are 2*I*K*N.  For the sharded MLP
  this is the per-device 2*B*D*F/n of "Lecture 4 - Distributed Serving",
  §3.4, per matrix.
* Compulsory HBM bytes of one call are the weights read once, the input read
  once and the output written once.  Decode is bound by that weight read:
  each of n devices reads 1/n of the weights per step (lecture §1.1 and
  §3.4).  The bf16 intermediate H of the MLP never has to leave the chip in
  principle, so its round trip is not credited.
"""
from __future__ import annotations

from dataclasses import dataclass

BF16 = 2
F32 = 4


@dataclass(frozen=True)
class MlpShape:
    I: int
    D: int
    F_local: int
    esize: int = BF16          # bytes per input element

    def flops(self) -> int:
        # gate, up and down: three [I, K] x [K, N] products
        return 2 * self.I * self.D * self.F_local * 3

    def weight_bytes(self) -> int:
        return 3 * self.D * self.F_local * self.esize

    def bytes(self) -> int:
        # weights + X in + fp32 partial out
        return self.weight_bytes() + self.I * self.D * self.esize + self.I * self.D * F32


@dataclass(frozen=True)
class QkvShape:
    I: int
    D: int
    n_q_local: int
    n_kv_local: int
    head_dim: int
    esize: int = BF16

    @property
    def N(self) -> int:
        return (self.n_q_local + 2 * self.n_kv_local) * self.head_dim

    def flops(self) -> int:
        return 2 * self.I * self.D * self.N

    def bytes(self) -> int:
        return (self.N * self.D + self.I * self.D + self.I * self.N) * self.esize


@dataclass(frozen=True)
class OprojShape:
    I: int
    D: int
    n_q_local: int
    head_dim: int
    esize: int = BF16

    @property
    def K(self) -> int:
        return self.n_q_local * self.head_dim

    def flops(self) -> int:
        return 2 * self.I * self.K * self.D

    def bytes(self) -> int:
        return (self.D * self.K + self.I * self.K) * self.esize + self.I * self.D * F32


@dataclass(frozen=True)
class ReduceShape:
    t: int
    n: int
    out_esize: int = F32

    def bytes(self) -> int:
        return self.t * self.n * F32 + self.n * self.out_esize


@dataclass(frozen=True)
class ResidualNormShape:
    """Residual update + RMSNorm after a block's reduce: reads t fp32
    partials, the residual and gamma, writes h and x (each once)."""
    t: int
    I: int
    D: int
    h_esize: int = BF16
    x_esize: int = BF16
    residual: bool = True
    norm: bool = True

    def bytes(self) -> int:
        n = self.I * self.D
        b = self.t * n * F32 + n * self.h_esize
        if self.residual:
            b += n * self.h_esize
        if self.norm:
            b += n * self.x_esize + self.D * self.x_esize
        return b


def allreduce_message_bytes(B: int, D: int, esize: int = BF16) -> int:
    """Size of one layer all-reduce message [B, D] (lecture §4.5, exercise 3)."""
    return B * D * esize


def ring_allreduce_bytes_sent(n: int, V: int) -> float:
    """Bytes one device sends in a ring all-reduce of V bytes: 2 (n-1)/n V
    (lecture §3.3)."""
    return 2.0 * (n - 1) / n * V


def shard_bytes(rows: int, cols: int, t: int, esize: int = BF16) -> int:
    """Bytes per device of a [rows_X, cols] tensor split t ways on rows."""
    return (rows // t) * cols * esize


# ---------------------------------------------------------------- configs
# The five workloads: a tiny fp32 parity case, a Qwen2.5-1.5B-shaped layer at
# TP=2, and Llama-3.1-70B-shaped MLP / full layer at TP=8 (prefill also TP=1).

TINY = dict(name="tiny-f32-tp2", D=256, F=1024, t=2, I=(4,), dtype="f32")
QWEN = dict(name="qwen2.5-1.5b-tp2", D=1536, F=8960, t=2, n_q=12, n_kv=2,
            head_dim=128, I=(1, 8, 64), dtype="bf16")
LLAMA_MLP_DECODE = dict(name="llama3.1-70b-mlp-tp8-decode", D=8192, F=28672,
                        t=8, I=(1, 16, 64, 256), dtype="bf16")
LLAMA_MLP_PREFILL = dict(name="llama3.1-70b-mlp-prefill", D=8192, F=28672,
                         t=(8, 1), I=(512,), dtype="bf16")
LLAMA_LAYER = dict(name="llama3.1-70b-layer-tp8", D=8192, F=28672, t=8,
                   n_q=64, n_kv=8, head_dim=128, I=(32, 512), dtype="bf16")

# Peaks of one MI355X (AMD public specification).
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
