"""The C ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments before touching the GPU.

Every call here fails validation (or is a host-only query), so no HIP
runtime call and no kernel launch happens: pointers are fake addresses that
are never dereferenced."""
import ctypes
import re

import pytest

import megatron_tensor_layer_amd as tp

OK, INVALID, MISALIGNED, UNSUPPORTED, LAUNCH, WORKSPACE = range(6)
FAKE = 0x10000000          # 16-byte aligned, never dereferenced
STEP = 1 << 32             # distinct fake buffers 4 GB apart


@pytest.fixture(scope="module")
def lib():
    if not tp.LIB_PATH.exists():
        from megatron_tensor_layer_amd import build
        build.build()
    return tp.lib()


def header_functions():
    src = tp.HEADER.read_text()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_0-9]+)\s*\(", src)))


def fake(k):
    return ctypes.c_void_p(FAKE + k * STEP)


def test_exports_every_header_function(lib):
    names = header_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/tpshard.h but not exported"
    # the binding declares exactly the header's functions
    assert sorted(tp.SIGNATURES) == names


def test_version_and_status_strings(lib):
    assert lib.tp_abi_version() == 1
    for code, name in tp.STATUS.items():
        assert lib.tp_status_string(code).decode() == name
    assert lib.tp_status_string(99).decode() == "TP_ERR_UNKNOWN"


def mlp(lib, I=4, D=256, F=512, dt=tp.TP_BF16, ptrs=None, ws=None, wsb=0):
    p = ptrs or [fake(k) for k in range(6)]
    return lib.tp_shard_mlp(I, D, F, dt, *p, ws, wsb, None)


def test_mlp_validation(lib):
    assert mlp(lib, dt=7) == INVALID
    assert mlp(lib, I=-1) == INVALID
    assert mlp(lib, D=0) == INVALID
    assert mlp(lib, F=0) == INVALID
    assert mlp(lib, D=1 << 40) == INVALID
    # I == 0 is a no-op even with null pointers
    assert mlp(lib, I=0, ptrs=[None] * 6) == OK
    for k in range(6):
        p = [fake(j) for j in range(6)]
        p[k] = None
        assert mlp(lib, ptrs=p) == INVALID, k
    assert mlp(lib, D=260) == MISALIGNED
    assert mlp(lib, F=508) == MISALIGNED
    for k in range(6):
        p = [fake(j) for j in range(6)]
        p[k] = ctypes.c_void_p(p[k].value + 8)
        assert mlp(lib, ptrs=p) == MISALIGNED, k
    # output overlapping an input, outputs overlapping each other
    p = [fake(j) for j in range(6)]
    p[4] = fake(0)
    assert mlp(lib, ptrs=p) == INVALID
    p = [fake(j) for j in range(6)]
    p[5] = ctypes.c_void_p(p[4].value + 64)
    assert mlp(lib, ptrs=p) == INVALID
    # fp32 beyond the few-token kernel's K range
    assert mlp(lib, D=32768, dt=tp.TP_F32) == UNSUPPORTED
    # a GEMM-size call (300 tokens) whose down K is past the GEMM's 32-bit
    # operand offsets (2^22); the same K at 4 tokens streams on VALU
    assert mlp(lib, I=300, D=64, F=(1 << 22) + 8) == UNSUPPORTED
    assert mlp(lib, I=300, D=64, F=1 << 22, ws=None) == WORKSPACE


def test_attn_validation(lib):
    f = lambda *a, **k: lib.tp_shard_attn_proj(*a, None, 0, None)
    P = [fake(k) for k in range(3)]
    assert f(5, 4, 256, 2, 1, 128, tp.TP_BF16, *P) == INVALID
    assert f(tp.TP_ATTN_QKV, 4, 256, 0, 1, 128, tp.TP_BF16, *P) == INVALID
    assert f(tp.TP_ATTN_QKV, 4, 256, 2, 0, 128, tp.TP_BF16, *P) == INVALID
    assert f(tp.TP_ATTN_O, 0, 256, 2, 0, 128, tp.TP_BF16, None, None, None) == OK
    assert f(tp.TP_ATTN_QKV, 4, 256, 2, 1, 12, tp.TP_BF16, *P) == MISALIGNED
    assert f(tp.TP_ATTN_QKV, 4, 256, 2, 1, 128, tp.TP_BF16, P[0], None, P[2]) == INVALID
    assert f(tp.TP_ATTN_O, 4, 256, 2, 1, 128, tp.TP_BF16, P[0], P[1],
             ctypes.c_void_p(P[2].value + 4)) == MISALIGNED
    assert f(tp.TP_ATTN_O, 4, 256, 2, 1, 128, tp.TP_BF16, P[0], P[1], P[0]) == INVALID
    # o_proj at 300 tokens with K = n_q_local * head_dim past the GEMM's 2^22
    assert f(tp.TP_ATTN_O, 300, 8, (1 << 15) + 1, 1, 128, tp.TP_BF16, *P) == UNSUPPORTED


def test_reduce_validation(lib):
    r = lib.tp_partial_reduce
    assert r(0, 64, fake(0), tp.TP_F32, fake(1), None) == INVALID
    assert r(2, -1, fake(0), tp.TP_F32, fake(1), None) == INVALID
    assert r(2, 64, fake(0), 3, fake(1), None) == INVALID
    assert r(2, 0, None, tp.TP_F32, None, None) == OK
    assert r(2, 60, fake(0), tp.TP_F32, fake(1), None) == MISALIGNED
    assert r(2, 64, ctypes.c_void_p(FAKE + 4), tp.TP_F32, fake(1), None) == MISALIGNED
    assert r(2, 64, fake(0), tp.TP_F32, ctypes.c_void_p(FAKE + 128), None) == INVALID


def test_attn_core_validation(lib):
    c = lib.tp_attn_core
    assert c(8, 3, 4, 2, 64, fake(0), fake(1), None) == INVALID      # S does not divide I
    assert c(8, 4, 2, 4, 64, fake(0), fake(1), None) == INVALID      # more KV groups than heads
    assert c(8, 4, 4, 2, 512, fake(0), fake(1), None) == UNSUPPORTED
    assert c(8, 4, 4, 2, 60, fake(0), fake(1), None) == MISALIGNED
    assert c(0, 1, 4, 2, 64, None, None, None) == OK
    assert c(1 << 20, 1, 8, 1, 128, fake(0), fake(1), None) == UNSUPPORTED  # qkv over 2 GiB


def test_residual_rmsnorm_validation(lib):
    n = lib.tp_residual_rmsnorm
    F, B = tp.TP_F32, tp.TP_BF16
    eps = ctypes.c_float(1e-5)
    P, R, H, G, X = (fake(k) for k in range(5))
    assert n(0, 0, 64, None, None, F, None, None, F, None, eps, None) == OK          # empty
    assert n(-1, 2, 64, P, R, F, H, G, B, X, eps, None) == INVALID
    assert n(2, 2, 0, P, R, F, H, G, B, X, eps, None) == INVALID
    assert n(2, 2, 64, P, R, 7, H, G, B, X, eps, None) == INVALID                   # bad dtype
    for bad in (-1.0, float("nan"), float("inf")):
        assert n(2, 2, 64, P, R, F, H, G, B, X, ctypes.c_float(bad), None) == INVALID
    assert n(2, 2, 64, P, R, F, None, G, B, X, eps, None) == INVALID                # no h
    assert n(2, 2, 64, None, R, F, H, G, B, X, eps, None) == INVALID                # t > 0, no partials
    assert n(0, 2, 64, None, None, F, H, G, B, X, eps, None) == INVALID             # nothing to add
    assert n(2, 2, 64, P, R, F, H, G, B, None, eps, None) == INVALID                # gamma without x
    assert n(2, 2, 60, P, R, F, H, G, B, X, eps, None) == MISALIGNED
    assert n(2, 2, 40000, P, R, F, H, G, B, X, eps, None) == UNSUPPORTED
    assert n(2, 2, 64, P, ctypes.c_void_p(FAKE + STEP + 8), F, H, G, B, X, eps, None) == MISALIGNED
    near_h = ctypes.c_void_p(FAKE + 2 * STEP + 256)
    assert n(2, 2, 64, P, near_h, F, H, G, B, X, eps, None) == INVALID             # h overlaps residual
    assert n(2, 2, 64, P, R, F, H, G, B, near_h, eps, None) == INVALID             # x overlaps h
    assert n(2, 2, 64, P, R, F, ctypes.c_void_p(FAKE + 128), G, B, X, eps, None) == INVALID  # h in partials


def test_reduce_scatter_rmsnorm_validation(lib):
    n = lib.tp_reduce_scatter_rmsnorm
    F = tp.TP_F32
    eps = ctypes.c_float(1e-5)
    P, R, H, G, X = (fake(k) for k in range(5))
    assert n(4, 0, 0, 64, P, R, F, H, G, F, X, eps, None) == OK
    assert n(4, 4, 8, 64, P, R, F, H, G, F, X, eps, None) == INVALID   # rank out of range
    assert n(0, 0, 8, 64, P, R, F, H, G, F, X, eps, None) == INVALID   # no ranks
    assert n(3, 0, 8, 64, P, R, F, H, G, F, X, eps, None) == INVALID   # t does not divide I
    assert n(4, 1, 8, 64, None, R, F, H, G, F, X, eps, None) == INVALID
    assert n(4, 1, 8, 60, P, R, F, H, G, F, X, eps, None) == MISALIGNED


def test_attn_decode_validation(lib):
    d = lib.tp_attn_decode
    L, Q, K, V, A = (fake(k) for k in range(5))
    ws_need = lib.tp_attn_decode_workspace_size(4, 8, 1, 128, 2048)
    assert ws_need > 0 and lib.tp_attn_decode_workspace_size(4, 8, 3, 128, 2048) == 0
    W = fake(6)
    assert d(0, 8, 1, 128, 2048, None, None, None, None, None, None, 0, None) == OK
    assert d(4, 8, 3, 128, 2048, L, Q, K, V, A, W, ws_need, None) == INVALID   # groups uneven
    assert d(4, 8, 1, 136, 2048, L, Q, K, V, A, W, ws_need, None) == UNSUPPORTED
    assert d(4, 8, 1, 60, 2048, L, Q, K, V, A, W, ws_need, None) == MISALIGNED
    assert d(4, 8, 1, 128, 2044, L, Q, K, V, A, W, ws_need, None) == MISALIGNED  # L_max % 8
    assert d(4, 64, 1, 128, 2048, L, Q, K, V, A, W, ws_need, None) == UNSUPPORTED  # 64 heads/group
    assert d(64, 8, 1, 128, 1 << 17, L, Q, K, V, A, W, ws_need, None) == UNSUPPORTED  # cache > 2 GiB
    assert d(4, 8, 1, 128, 2048, L, Q, K, V, A, None, 0, None) == WORKSPACE
    assert d(4, 8, 1, 128, 2048, None, Q, K, V, A, W, ws_need, None) == INVALID
    assert d(4, 8, 1, 128, 2048, L, Q, K, ctypes.c_void_p(FAKE + 2 * STEP + 4096), A, W,
             ws_need, None) == INVALID                                         # V inside K


def test_mlp_fp8_validation(lib):
    m = lib.tp_shard_mlp_fp8
    # X, Wg, sg, Wu, su, Wd, sd, H, P, workspace, workspace_bytes, stream
    args = [fake(k) for k in range(9)] + [None, 0, None]
    assert m(0, 64, 128, *args) == OK
    assert m(-1, 64, 128, *args) == INVALID
    assert m(65, 64, (1 << 22) + 16, *args) == UNSUPPORTED           # GEMM K past 2^22
    assert m(9, 64, 128, *args) == WORKSPACE                         # split K: needs one
    assert m(1, 24, 128, *args) == MISALIGNED                        # D not a multiple of 16
    assert m(1, 32768, 128, *args) == WORKSPACE                      # K above 16384: split K
    assert lib.tp_shard_mlp_fp8_workspace_size(4, 8192, 3584) == 0     # VALU kernel
    assert lib.tp_shard_mlp_fp8_workspace_size(5, 8192, 3584) > 0      # split K from 5
    need = lib.tp_shard_mlp_fp8_workspace_size(32, 8192, 3584)
    assert need > 8192
    # more than 64 tokens: the one-byte GEMM; at 65 tokens its 56 gate/up
    # tiles split K 4 ways (224 workgroups)
    assert lib.tp_shard_mlp_fp8_workspace_size(65, 8192, 3584) == 8192 + 4 * 56 * 128 * 128 * 4
    assert lib.tp_shard_mlp_int8_workspace_size(65, 8192, 3584) == 8192 + 4 * 56 * 128 * 128 * 4
    small = lib.tp_shard_mlp_fp8_workspace_size(32, 64, 128)
    ws = list(args)
    ws[9], ws[10] = ctypes.c_void_p(FAKE + 9 * STEP + 8), small
    assert m(32, 64, 128, *ws) == MISALIGNED                         # workspace not aligned
    ws[9] = fake(7)
    assert m(32, 64, 128, *ws) == INVALID                            # workspace is H
    ws[9], ws[10] = fake(9), small - 1
    assert m(32, 64, 128, *ws) == WORKSPACE                          # too small
    bad = list(args)
    bad[2] = None
    assert m(1, 64, 128, *bad) == INVALID                            # missing scale
    bad[2] = ctypes.c_void_p(FAKE + 2 * STEP + 2)
    assert m(1, 64, 128, *bad) == MISALIGNED                         # scale not 4-byte aligned
    bad = list(args)
    bad[7] = ctypes.c_void_p(FAKE + 16)                              # H inside X
    assert m(1, 64, 128, *bad) == INVALID


def test_workspace_queries_are_host_only(lib):
    # calls that split K (9..64 tokens on the streaming kernel, up to 256 on
    # the tiled one, and the 512-token TP=8 gate/up on 256 x 128 tiles) need
    # counters + fp32 partials; few-token calls need none; invalid sizes
    # report 0
    ws = lib.tp_shard_mlp_workspace_size
    assert ws(32, 8192, 3584, tp.TP_BF16) > 0
    assert ws(256, 8192, 3584, tp.TP_BF16) > 0
    assert ws(64, 8192, 3584, tp.TP_BF16) >= ws(32, 8192, 3584, tp.TP_BF16) // 4
    assert ws(1, 8192, 3584, tp.TP_BF16) == 0
    # 8 KiB of counters + 2 K splits x 112 tiles of 256 x 128 fp32
    assert ws(512, 8192, 3584, tp.TP_BF16) == 8192 + 2 * 112 * 256 * 128 * 4
    assert ws(32, 8192, 3584, tp.TP_F32) == 0
    assert ws(0, 8192, 3584, tp.TP_BF16) == 0 and ws(32, 0, 3584, tp.TP_BF16) == 0
    wa = lib.tp_shard_attn_proj_workspace_size
    assert wa(tp.TP_ATTN_QKV, 32, 8192, 8, 1, 128, tp.TP_BF16) > 0
    assert wa(tp.TP_ATTN_O, 32, 8192, 8, 1, 128, tp.TP_BF16) == 0   # whole-K row blocks
    assert wa(tp.TP_ATTN_O, 32, 1536, 6, 1, 128, tp.TP_BF16) > 0    # split K (Qwen o_proj)
    assert wa(tp.TP_ATTN_QKV, 1, 8192, 8, 1, 128, tp.TP_BF16) == 0
    assert wa(7, 32, 8192, 8, 1, 128, tp.TP_BF16) == 0


def test_workspace_required_and_checked(lib):
    need = lib.tp_shard_mlp_workspace_size(32, 256, 512, tp.TP_BF16)
    assert need > 0
    assert mlp(lib, I=32, D=256, F=512) == WORKSPACE                       # none given
    assert mlp(lib, I=32, D=256, F=512, ws=fake(6), wsb=need - 1) == WORKSPACE
    assert mlp(lib, I=32, D=256, F=512, ws=ctypes.c_void_p(fake(6).value + 8),
               wsb=need) == MISALIGNED
    assert mlp(lib, I=32, D=256, F=512, ws=fake(1), wsb=need) == INVALID   # overlaps W_gate
    f = lambda *a: lib.tp_shard_attn_proj(*a, None)
    P = [fake(k) for k in range(3)]
    assert f(tp.TP_ATTN_QKV, 32, 256, 2, 1, 64, tp.TP_BF16, *P, None, 0) == WORKSPACE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(tp, "_lib", None)
    monkeypatch.setattr(tp, "LIB_PATH", tmp_path / "missing.so")
    with pytest.raises(RuntimeError, match="missing"):
        tp.lib()


def test_stream_read_validation(lib):
    """The read-ceiling probe rejects a null buffer, a size that is not a
    multiple of 1 KB, and sizes past 2 GiB, before any device query."""
    sink_words = 1 << 20
    assert lib.tp_stream_read(None, 1024, fake(1), sink_words, None) == INVALID
    assert lib.tp_stream_read(fake(0), 1024, None, sink_words, None) == INVALID
    assert lib.tp_stream_read(fake(0), 0, fake(1), sink_words, None) == INVALID
    assert lib.tp_stream_read(fake(0), (1 << 31) + 1024, fake(1), sink_words, None) == INVALID
    assert lib.tp_stream_read(fake(0), 1000, fake(1), sink_words, None) == MISALIGNED
    assert lib.tp_stream_read(ctypes.c_void_p(FAKE + 8), 1024, fake(1), sink_words,
                              None) == MISALIGNED


def test_workspace_reset_validation(lib):
    """tp_workspace_reset rejects a null or empty workspace and a misaligned
    pointer before launching anything."""
    assert lib.tp_workspace_reset(None, 8192, None) == INVALID
    assert lib.tp_workspace_reset(fake(0), 0, None) == INVALID
    assert lib.tp_workspace_reset(ctypes.c_void_p(FAKE + 4), 8192, None) == MISALIGNED
