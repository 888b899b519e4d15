"""bench.py's measurement contract, checked without a GPU: the algorithmic
byte and FLOP counts its figures divide by, and the one-GPU guard."""
import importlib.util
import os
import pathlib
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parents[1]


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", ROOT / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_mlp_call_bytes_and_flops():
    """One rank's MLP call at 32 tokens (D = 8192, F_local = 28672 / 8):
    the three weight matrices once in bf16, X in (bf16) and the fp32 partial
    out; 2 I K N FLOPs per projection."""
    b = _bench()
    m = b.wl.MlpShape(32, 8192, 3584)
    assert m.bytes() == 3 * 8192 * 3584 * 2 + 32 * 8192 * 2 + 32 * 8192 * 4 == 177_733_632
    assert m.flops() == 2 * 32 * 8192 * 3584 * 3


def test_layer_step_bytes():
    """The decode-32 step of the 8 emulated ranks: per rank QKV (10 heads of
    128 rows x 8192), o_proj (8192 x 1024), the MLP and the attention core's
    q/k/v in and A out; then the two reduces of 8 partials."""
    b = _bench()
    I, D, hd = 32, 8192, 128
    nq, nkv, t = 64 // 8, 8 // 8, 8
    n_qkv = (nq + 2 * nkv) * hd
    qkv = (n_qkv * D + I * D + I * n_qkv) * 2
    o = (D * nq * hd + I * nq * hd) * 2 + I * D * 4
    mlp = 3 * D * 3584 * 2 + I * D * 2 + I * D * 4
    attn = (I * n_qkv + I * nq * hd) * 2
    red = (t * I * D * 4 + I * D * 2) + (t * I * D * 4 + I * D * 4)
    assert b.step_bytes(I, 1) == t * (qkv + o + mlp + attn) + red == 1_757_151_232


def test_more_than_one_gpu_is_refused():
    env = dict(os.environ, WORLD_SIZE="1")
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_prefill_roofline_flops():
    """The prefill side of the line: one TP=8 rank's 512-token MLP call,
    2 * 512 * 8192 * 3584 FLOPs per matrix, three matrices; per matrix this is
    the lecture's per-device 2 B D F / n at B = 512, D = 8192, F = 28672, n = 8."""
    b = _bench()
    m = b.wl.MlpShape(b.PREFILL_I, 8192, 3584)
    assert m.flops() == 90_194_313_216
    assert m.flops() // 3 == 2 * 512 * 8192 * 28672 // 8
