"""One tensor-parallel rank's share of a Megatron-style layer on MI355X.

Thin Python binding of the C ABI in include/tpshard.h (libtpshard.so, built
from csrc/ for gfx950).  It only checks and marshals arguments: every step of
the computation runs in the library's HIP kernels.  torch supplies device
memory and the stream.  There is no fallback: if the library is missing the
calls raise.

    shard_mlp(X, W_gate, W_up, W_down, H, P)         column gate/up, SwiGLU, row down
    shard_attn_proj(QKV|O, X_or_A, W, out, ...)      head-split QKV / row-split o_proj
    partial_reduce(partials, Y)                      sum of the t rank partials
    attn_core(qkv, A, S, n_q_local, n_kv_local, hd)  per-rank attention (test support)
"""
from __future__ import annotations

import ctypes
import pathlib

LIB_PATH = pathlib.Path(__file__).resolve().parent / "libtpshard.so"
HEADER = pathlib.Path(__file__).resolve().parent.parent / "include" / "tpshard.h"

TP_F32, TP_BF16 = 0, 1
TP_ATTN_QKV, TP_ATTN_O = 0, 1
STATUS = {0: "TP_OK", 1: "TP_ERR_INVALID", 2: "TP_ERR_MISALIGNED", 3: "TP_ERR_UNSUPPORTED",
          4: "TP_ERR_LAUNCH", 5: "TP_ERR_WORKSPACE"}

_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/tpshard.h
SIGNATURES = {
    "tp_abi_version": (ctypes.c_int, []),
    "tp_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "tp_shard_mlp_workspace_size": (_sz, [_i64, _i64, _i64, ctypes.c_int]),
    "tp_shard_mlp": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _sz, _vp]),
    "tp_shard_attn_proj_workspace_size": (_sz, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                                ctypes.c_int]),
    "tp_shard_attn_proj": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                          ctypes.c_int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "tp_partial_reduce": (ctypes.c_int, [_i32, _i64, _vp, ctypes.c_int, _vp, _vp]),
    "tp_attn_core": (ctypes.c_int, [_i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp]),
    "tp_reduce_scatter_rmsnorm": (ctypes.c_int, [_i32, _i32, _i64, _i64, _vp, _vp, ctypes.c_int,
                                                 _vp, _vp, ctypes.c_int, _vp, ctypes.c_float,
                                                 _vp]),
    "tp_attn_decode_workspace_size": (_sz, [_i64] * 5),
    "tp_attn_decode": (ctypes.c_int, [_i64] * 5 + [_vp] * 6 + [_sz, _vp]),
    "tp_shard_mlp_fp8_workspace_size": (_sz, [_i64] * 3),
    "tp_shard_mlp_fp8": (ctypes.c_int, [_i64, _i64, _i64] + [_vp] * 10 + [_sz, _vp]),
    "tp_shard_mlp_int8_workspace_size": (_sz, [_i64] * 3),
    "tp_shard_mlp_int8": (ctypes.c_int, [_i64, _i64, _i64] + [_vp] * 10 + [_sz, _vp]),
    "tp_residual_rmsnorm": (ctypes.c_int, [_i32, _i64, _i64, _vp, _vp, ctypes.c_int, _vp, _vp,
                                           ctypes.c_int, _vp, ctypes.c_float, _vp]),
    "tp_workspace_reset": (ctypes.c_int, [_vp, _sz, _vp]),
    "tp_shard_mlp_noalloc_max_workspace": (_sz, []),
    "tp_shard_mlp_noalloc": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int] + [_vp] * 7),
    "tp_stream_read_sink_words": (_sz, []),
    "tp_stream_read": (ctypes.c_int, [_vp, _sz, _vp, _sz, _vp]),
}


class TPError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m megatron_tensor_layer_amd.build`")
        L = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(fn: str, code: int) -> None:
    if code != 0:
        raise TPError(fn, code)


# ------------------------------------------------------------------ torch glue
def _torch():
    import torch
    return torch


def _dt(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return TP_BF16
    if t.dtype == torch.float32:
        return TP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    dev = ts[0].device
    for t in ts:
        if t.device.type != "cuda" or t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return dev


def _stream(stream, dev):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def mlp_workspace_bytes(I: int, D: int, F_local: int, dtype: int = TP_BF16) -> int:
    return lib().tp_shard_mlp_workspace_size(I, D, F_local, dtype)


def attn_workspace_bytes(phase: int, I: int, D: int, n_q_local: int, n_kv_local: int,
                         head_dim: int, dtype: int = TP_BF16) -> int:
    return lib().tp_shard_attn_proj_workspace_size(phase, I, D, n_q_local, n_kv_local,
                                                   head_dim, dtype)


# One scratch buffer per (device, stream), grown on demand, used when a caller
# passes no workspace.  A new buffer's leading counter area is zeroed with
# tp_workspace_reset on the call's stream before its first use; every
# completed call leaves it zero.  Keying by stream keeps calls that run
# concurrently on different streams off each other's counters.  A buffer
# that is outgrown is kept alive (not freed), since a call still in flight on
# its stream may be using it.
_ws_cache: dict = {}
_ws_retired: list = []


def _workspace(dev, nbytes: int, stream=None):
    if nbytes <= 0:
        return None, 0
    torch = _torch()
    s = _stream(stream, dev)
    key = (dev, s.value)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        if buf is not None:
            _ws_retired.append(buf)
        buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _check("tp_workspace_reset", lib().tp_workspace_reset(_ptr(buf), buf.numel(), s))
        _ws_cache[key] = buf
    return _ptr(buf), buf.numel()


def workspace_reset(workspace, stream=None) -> None:
    """Zero the counter area of a caller-owned workspace (once after
    allocating it, or after a call that did not complete)."""
    dev = _dev(workspace)
    _check("tp_workspace_reset",
           lib().tp_workspace_reset(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                    _stream(stream, dev)))


def _user_workspace(workspace):
    _dev(workspace)
    return _ptr(workspace), workspace.numel() * workspace.element_size()


def shard_mlp(X, W_gate, W_up, W_down, H, P, workspace=None, stream=None) -> None:
    """P[I,D]{U_X} = (silu(X W_gate[D,F_X]) * (X W_up[D,F_X])) W_down[F_X,D]; H gets
    the SwiGLU activations.  Weights output-major: W_gate/W_up [F_local, D],
    W_down [D, F_local]."""
    torch = _torch()
    dev = _dev(X, W_gate, W_up, W_down, H, P)
    I, D = X.shape
    F_local = W_gate.shape[0]
    dt = _dt(X)
    for t in (W_gate, W_up, W_down, H):
        if _dt(t) != dt:
            raise TypeError("X, weights and H must share one dtype")
    if P.dtype != torch.float32:
        raise TypeError("P must be float32")
    if (W_gate.shape != (F_local, D) or W_up.shape != (F_local, D)
            or W_down.shape != (D, F_local) or H.shape != (I, F_local) or P.shape != (I, D)):
        raise ValueError("shape mismatch")
    if workspace is not None:
        ws_ptr, ws_bytes = _user_workspace(workspace)
    else:
        ws_ptr, ws_bytes = _workspace(dev, mlp_workspace_bytes(I, D, F_local, dt), stream)
    _check("tp_shard_mlp", lib().tp_shard_mlp(I, D, F_local, dt, _ptr(X), _ptr(W_gate),
                                              _ptr(W_up), _ptr(W_down), _ptr(H), _ptr(P),
                                              ws_ptr, ws_bytes, _stream(stream, dev)))


def shard_mlp_noalloc(X, W_gate, W_up, W_down, H, P, stream=None) -> None:
    """shard_mlp without a workspace: the library's own static scratch array
    (calls that overlap on one GPU race on it; see tp_shard_mlp_noalloc)."""
    torch = _torch()
    dev = _dev(X, W_gate, W_up, W_down, H, P)
    I, D = X.shape
    F_local = W_gate.shape[0]
    dt = _dt(X)
    for t in (W_gate, W_up, W_down, H):
        if _dt(t) != dt:
            raise TypeError("X, weights and H must share one dtype")
    if P.dtype != torch.float32:
        raise TypeError("P must be float32")
    if (W_gate.shape != (F_local, D) or W_up.shape != (F_local, D)
            or W_down.shape != (D, F_local) or H.shape != (I, F_local) or P.shape != (I, D)):
        raise ValueError("shape mismatch")
    _check("tp_shard_mlp_noalloc",
           lib().tp_shard_mlp_noalloc(I, D, F_local, dt, _ptr(X), _ptr(W_gate), _ptr(W_up),
                                      _ptr(W_down), _ptr(H), _ptr(P), _stream(stream, dev)))


def shard_attn_proj(phase: int, inp, W, out, n_q_local: int, n_kv_local: int, head_dim: int,
                    workspace=None, stream=None) -> None:
    """phase TP_ATTN_QKV: out[I, N_qkv] = X W_qkv (W [N_qkv, D], rows q|k|v heads);
    phase TP_ATTN_O: out(fp32)[I, D] = A W_o (W [D, n_q_local*head_dim])."""
    torch = _torch()
    dev = _dev(inp, W, out)
    dt = _dt(inp)
    if _dt(W) != dt:
        raise TypeError("input and weight must share one dtype")
    I = inp.shape[0]
    if phase == TP_ATTN_QKV:
        D = inp.shape[1]
        N = (n_q_local + 2 * n_kv_local) * head_dim
        if W.shape != (N, D) or out.shape != (I, N) or _dt(out) != dt:
            raise ValueError("shape/dtype mismatch (QKV)")
    elif phase == TP_ATTN_O:
        D = W.shape[0]
        K = n_q_local * head_dim
        if inp.shape != (I, K) or W.shape != (D, K) or out.shape != (I, D) \
                or out.dtype != torch.float32:
            raise ValueError("shape/dtype mismatch (O)")
    else:
        raise ValueError("bad phase")
    if workspace is not None:
        ws_ptr, ws_bytes = _user_workspace(workspace)
    else:
        ws_ptr, ws_bytes = _workspace(dev, attn_workspace_bytes(phase, I, D, n_q_local,
                                                                n_kv_local, head_dim, dt), stream)
    _check("tp_shard_attn_proj",
           lib().tp_shard_attn_proj(phase, I, D, n_q_local, n_kv_local, head_dim, dt, _ptr(inp),
                                    _ptr(W), _ptr(out), ws_ptr, ws_bytes, _stream(stream, dev)))


def partial_reduce(partials, Y, stream=None) -> None:
    """Y = sum over r of partials[r] (rank order, fp32); Y float32 or bfloat16."""
    torch = _torch()
    dev = _dev(partials, Y)
    if partials.dtype != torch.float32:
        raise TypeError("partials must be float32")
    t = partials.shape[0]
    n = partials[0].numel()
    if Y.numel() != n:
        raise ValueError("Y must hold one partial's elements")
    _check("tp_partial_reduce", lib().tp_partial_reduce(t, n, _ptr(partials), _dt(Y), _ptr(Y),
                                                        _stream(stream, dev)))


def stream_read(buf, sink=None, stream=None):
    """Measurement aid: read the device tensor `buf` (its byte size a multiple
    of 1024, at most 2 GiB) once with the decode kernels' access pattern.
    Returns the int32 sink; the XOR of its words equals the XOR, over the
    buffer's 16-byte chunks, of each chunk's first and last 32-bit words."""
    torch = _torch()
    dev = _dev(buf)
    L = lib()
    words = L.tp_stream_read_sink_words()
    if sink is None:
        sink = torch.empty(words, dtype=torch.int32, device=buf.device)
    elif sink.dtype != torch.int32 or sink.numel() < words or not sink.is_contiguous():
        raise ValueError(f"sink must be a contiguous int32 tensor of at least {words} words")
    nbytes = buf.numel() * buf.element_size()
    _check("tp_stream_read", L.tp_stream_read(_ptr(buf), nbytes, _ptr(sink), sink.numel(),
                                              _stream(stream, dev)))
    return sink


def _shard_mlp_bytew(kind, X, gate, up, down, H, P, workspace, stream) -> None:
    torch = _torch()
    code_dtype = torch.uint8 if kind == "fp8" else torch.int8
    (Wg, sg), (Wu, su), (Wd, sd) = gate, up, down
    dev = _dev(X, Wg, sg, Wu, su, Wd, sd, H, P)
    I, D = X.shape
    F_local = Wg.shape[0]
    if X.dtype != torch.bfloat16 or H.dtype != torch.bfloat16 or P.dtype != torch.float32:
        raise TypeError("X and H bfloat16, P float32")
    for W, s_, shape in ((Wg, sg, (F_local, D)), (Wu, su, (F_local, D)), (Wd, sd, (D, F_local))):
        if W.dtype != code_dtype or tuple(W.shape) != shape:
            raise ValueError(f"{kind} codes must be {code_dtype} {shape}")
        if s_.dtype != torch.float32 or s_.numel() != shape[0]:
            raise ValueError("scales must be float32, one per output row")
    if tuple(H.shape) != (I, F_local) or tuple(P.shape) != (I, D):
        raise ValueError("H [I, F_local], P [I, D]")
    L = lib()
    size_fn = getattr(L, f"tp_shard_mlp_{kind}_workspace_size")
    if workspace is not None:
        ws_ptr, ws_bytes = _user_workspace(workspace)
    else:
        ws_ptr, ws_bytes = _workspace(dev, size_fn(I, D, F_local), stream)
    name = f"tp_shard_mlp_{kind}"
    _check(name, getattr(L, name)(
        I, D, F_local, _ptr(X), _ptr(Wg), _ptr(sg), _ptr(Wu), _ptr(su), _ptr(Wd), _ptr(sd),
        _ptr(H), _ptr(P), ws_ptr, ws_bytes, _stream(stream, dev)))


def shard_mlp_fp8(X, gate, up, down, H, P, workspace=None, stream=None) -> None:
    """Weight-only FP8 MLP rank share for decode (1..64 tokens): gate, up, down
    are (codes uint8, scales float32) pairs -- gate/up codes [F_local, D] with
    scales [F_local], down codes [D, F_local] with scales [D]; X and H bf16,
    P float32.  Past 4 tokens the call needs a workspace (the binding keeps
    one per device and stream unless one is passed)."""
    _shard_mlp_bytew("fp8", X, gate, up, down, H, P, workspace, stream)


def shard_mlp_int8(X, gate, up, down, H, P, workspace=None, stream=None) -> None:
    """Weight-only int8 MLP rank share for decode (1..64 tokens): as
    shard_mlp_fp8 with int8 codes, W[n, k] = scale[n] * code[n, k]."""
    _shard_mlp_bytew("int8", X, gate, up, down, H, P, workspace, stream)


def residual_rmsnorm(partials, residual, h, gamma=None, x=None, eps: float = 1e-5,
                     stream=None) -> None:
    """h = residual + sum over r of partials[r] (rank order, fp32), then
    x = h / sqrt(mean(h^2) + eps) * gamma from h as stored.  partials [t, I, D]
    float32 or None; residual [I, D] (h's dtype) or None; h may be residual
    itself; gamma [D] and x [I, D] (same dtype) both None for h only."""
    torch = _torch()
    tensors = [a for a in (partials, residual, h, gamma, x) if a is not None]
    dev = _dev(*tensors)
    I, D = h.shape
    t = 0
    if partials is not None:
        if partials.dtype != torch.float32 or partials.dim() != 3 or \
                tuple(partials.shape[1:]) != (I, D):
            raise ValueError("partials must be float32 [t, I, D]")
        t = partials.shape[0]
    if residual is not None and (residual.dtype != h.dtype or tuple(residual.shape) != (I, D)):
        raise ValueError("residual must match h's dtype and shape")
    if (gamma is None) != (x is None):
        raise ValueError("gamma and x go together")
    x_dt = TP_F32
    if x is not None:
        if x.dtype != gamma.dtype or tuple(x.shape) != (I, D) or gamma.numel() != D:
            raise ValueError("x [I, D] and gamma [D] must share a dtype")
        x_dt = _dt(x)
    _check("tp_residual_rmsnorm", lib().tp_residual_rmsnorm(
        t, I, D, _ptr(partials) if partials is not None else None,
        _ptr(residual) if residual is not None else None, _dt(h), _ptr(h),
        _ptr(gamma) if gamma is not None else None, x_dt,
        _ptr(x) if x is not None else None, float(eps), _stream(stream, dev)))


def reduce_scatter_rmsnorm(partials, rank: int, residual, h, gamma=None, x=None,
                           eps: float = 1e-5, stream=None) -> None:
    """Sequence-parallel rank `rank`: rows [rank*I/t, (rank+1)*I/t) of
    h = residual + sum_r partials[r], then x = RMSNorm(h) * gamma.  partials
    [t, I, D] float32; residual, h, x [I/t, D] (x may be a row slice of a full
    [I, D] buffer: over all ranks it then holds the all-gathered x)."""
    torch = _torch()
    tensors = [a for a in (partials, residual, h, gamma, x) if a is not None]
    dev = _dev(*tensors)
    if partials.dtype != torch.float32 or partials.dim() != 3:
        raise ValueError("partials must be float32 [t, I, D]")
    t, I, D = partials.shape
    if tuple(h.shape) != (I // t, D):
        raise ValueError("h must be [I/t, D]")
    if residual is not None and (residual.dtype != h.dtype or residual.shape != h.shape):
        raise ValueError("residual must match h")
    if (gamma is None) != (x is None):
        raise ValueError("gamma and x go together")
    x_dt = TP_F32
    if x is not None:
        if x.dtype != gamma.dtype or x.shape != h.shape or gamma.numel() != D:
            raise ValueError("x [I/t, D] and gamma [D] must share a dtype")
        x_dt = _dt(x)
    _check("tp_reduce_scatter_rmsnorm", lib().tp_reduce_scatter_rmsnorm(
        t, rank, I, D, _ptr(partials), _ptr(residual) if residual is not None else None,
        _dt(h), _ptr(h), _ptr(gamma) if gamma is not None else None, x_dt,
        _ptr(x) if x is not None else None, float(eps), _stream(stream, dev)))


def attn_decode(lens, qkv, K_cache, V_cache, A, n_q_local: int, n_kv_local: int,
                head_dim: int, workspace=None, stream=None) -> None:
    """Decode attention over the rank's KV cache: lens [B] int32, qkv [B, N_qkv]
    bf16 (the new tokens), K_cache [B, n_kv_local, L_max, head_dim] and the
    transposed V_cache [B, n_kv_local, head_dim, L_max] bf16 (position
    lens[b]-1 is written with the new k, v), A [B, n_q_local * head_dim] bf16."""
    torch = _torch()
    dev = _dev(lens, qkv, K_cache, V_cache, A)
    if lens.dtype != torch.int32:
        raise TypeError("lens must be int32")
    for a in (qkv, K_cache, V_cache, A):
        if a.dtype != torch.bfloat16:
            raise TypeError("qkv, caches and A are bfloat16")
    B, nkv, L_max, hd = K_cache.shape
    if nkv != n_kv_local or hd != head_dim or tuple(V_cache.shape) != (B, nkv, hd, L_max):
        raise ValueError("K_cache [B, n_kv_local, L_max, head_dim], "
                         "V_cache [B, n_kv_local, head_dim, L_max]")
    if lens.numel() != B or qkv.shape[0] != B or tuple(A.shape) != (B, n_q_local * head_dim):
        raise ValueError("lens [B], qkv [B, N_qkv], A [B, n_q_local * head_dim]")
    if workspace is not None:
        ws_ptr, ws_bytes = _user_workspace(workspace)
    else:
        ws_ptr, ws_bytes = _workspace(dev, lib().tp_attn_decode_workspace_size(
            B, n_q_local, n_kv_local, head_dim, L_max), stream)
    _check("tp_attn_decode", lib().tp_attn_decode(
        B, n_q_local, n_kv_local, head_dim, L_max, _ptr(lens), _ptr(qkv), _ptr(K_cache),
        _ptr(V_cache), _ptr(A), ws_ptr, ws_bytes, _stream(stream, dev)))


def attn_core(qkv, A, S: int, n_q_local: int, n_kv_local: int, head_dim: int,
              stream=None) -> None:
    """Per-rank causal GQA attention over sequences of S tokens (bf16)."""
    torch = _torch()
    dev = _dev(qkv, A)
    if qkv.dtype != torch.bfloat16 or A.dtype != torch.bfloat16:
        raise TypeError("attn_core is bf16 only")
    I = qkv.shape[0]
    _check("tp_attn_core", lib().tp_attn_core(I, S, n_q_local, n_kv_local, head_dim, _ptr(qkv),
                                              _ptr(A), _stream(stream, dev)))
