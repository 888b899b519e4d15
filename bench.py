"""Benchmark of one tensor-parallel rank's layer share on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-detail] [--no-cpu]

A step is one pass of the whole hot path over one batch: the Llama-3.1-70B-
shaped layer (D=8192, F=28672, 64 query heads, 8 KV groups, head_dim 128) at
TP=8 with all 8 rank shares computed in turn on the one GPU, decode batch 32
(32 sequences of one token):

    per rank: QKV (column, by heads) -> attention core -> o_proj (row partial)
    reduce of the 8 o_proj partials (bf16 out)
    per rank: gate/up (column) + SwiGLU -> down (row partial)
    reduce of the 8 MLP partials (fp32 out)

value = the step's compulsory HBM bytes (weights, inputs and outputs of every
call, each once) / the step's time, in GB/s.  The 8 ranks' weights (1.71 GB)
exceed the 256 MB Infinity Cache, so every step streams them from HBM.

The printed JSON line also carries
  roofline:     the dominant call (one rank's tp_shard_mlp at I=32) timed with
                HIP events on its stream inside the timed region (one event
                pair per step around the 8 ranks' back-to-back calls, divided
                by 8), against the 8 TB/s HBM peak;
  roofline_prefill: the prefill side of the metric, one rank's tp_shard_mlp
                at 512 tokens (TP=8 shapes), event-timed on its stream in
                groups of 8 back-to-back calls (one per rank share), against
                the dense bf16 MFMA peak;
  clocks:       SCLK and MCLK sampled with amd-smi while those prefill calls
                run back to back;
  read_ceiling: the achievable read rate, tp_stream_read over 2 GiB with the
                decode kernels' access pattern; roofline and config also give
                their fraction of it;
  cpu_baseline: the fp64 oracle on the host cores running one whole step
                (about 55 GFLOP in fp64, a second or so on 16 cores);
  detail:       per-config figures (MLP shard decode I=1/16/64/256 GB/s,
                prefill 512 TFLOP/s at TP=8 and TP=1, Qwen2.5-1.5B TP=2 calls,
                the layer at prefill 512, the partial reduce, the residual
                update + RMSNorm after a block, the layer as a pre-norm block
                with those at decode 32, the MLP with weight-only FP8
                storage at 1, 8, 32, 128 and 512 tokens, the same with int8
                storage,
                and decode attention over a
                rank's KV cache); calls rotating over weight sets are timed
                in groups of back-to-back calls, one per set, with one event
                pair per group, queued behind a spin kernel.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import pathlib
import statistics
import sys
import time

import numpy as np

ROOT = pathlib.Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

from megatron_tensor_layer_amd import datagen, workloads as wl  # noqa: E402

D, F, NQ, NKV, HD, TP = 8192, 28672, 64, 8, 128, 8
PEAK_HBM = wl.PEAK_HBM_GBS
PEAK_BF16 = wl.PEAK_BF16_TFLOPS


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=32, help="decode tokens of the timed step")
    ap.add_argument("--no-detail", action="store_true", help="skip the per-config breakdown")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--calls", type=int, default=200, help="timed calls per detail config")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="for rocprofv3 --pmc: one calibration copy of COPY_MIB MiB, then one "
                         "tp_shard_mlp call per rank at the bench batch; no timing")
    ap.add_argument("--prefill-profile", action="store_true",
                    help="for rocprofv3: each 512-token prefill projection of a TP=8 rank "
                         "(MLP, QKV, o_proj) and the TP=1 MLP in phases of its own, no timing")
    ap.add_argument("--decode-profile", action="store_true",
                    help="for rocprofv3: the TP=8 rank's MLP at 1, 8, 32, 128 and 512 tokens "
                         "with bf16, FP8 and int8 weights, each in a phase of its own, no timing")
    ap.add_argument("--attn-profile", action="store_true",
                    help="for rocprofv3: one calibration copy of COPY_MIB MiB, then decode "
                         "attention of a TP=8 rank (B = 32) at 2048 and 8192 positions, "
                         "each in a phase of its own, no timing")
    ap.add_argument("--ingest-prefill-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the FETCH_SIZE and WRITE_SIZE passes over --prefill-profile "
                         "into the 512-token MLP entry of profiles/traffic.json")
    ap.add_argument("--ingest-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn the counter_collection.csv files of the FETCH_SIZE and "
                         "WRITE_SIZE passes over --traffic-probe into profiles/traffic.json")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers
def to_dev(torch, a, dtype="bf16"):
    if dtype == "bf16":
        return torch.from_numpy(datagen.bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


_SPIN_US_PER_MCYCLE = None


def _spin_cycles(torch, us):
    """Cycles of torch's spin kernel that keep the GPU busy for about `us`
    microseconds (calibrated once)."""
    global _SPIN_US_PER_MCYCLE
    if not hasattr(torch.cuda, "_sleep"):
        return 0
    if _SPIN_US_PER_MCYCLE is None:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1_000_000)
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        torch.cuda.synchronize()
        _SPIN_US_PER_MCYCLE = max(a.elapsed_time(b) * 1e3, 1.0)
    return int(us / _SPIN_US_PER_MCYCLE * 1e6)


def time_calls(torch, fns, n, warm=10):
    """Event-time about n calls, cycling through fns (one per weight set) in
    groups of len(fns) back-to-back calls with one event pair per group (an
    event pair around every call adds about 3 us to a decode call).  A spin
    kernel ahead of each group keeps the GPU busy while the host queues the
    group, so calls shorter than the binding's host overhead (about 10 us)
    are timed on the device, not on the host.  Returns per-call
    microseconds, one figure per group."""
    for i in range(warm):
        fns[i % len(fns)]()
    groups = max(1, n // len(fns))
    spin = _spin_cycles(torch, 15.0 * len(fns) + 50.0)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(groups)]
    s = torch.cuda.current_stream()
    for g in range(groups):
        if spin:
            torch.cuda._sleep(spin)
        ev[g][0].record(s)
        for f in fns:
            f()
        ev[g][1].record(s)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 / len(fns) for a, b in ev]


def log(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


PREFILL_I = 512


def prefill_mlp_fns(torch, tp, layer, I=PREFILL_I):
    """One TP=8 rank's 512-token MLP call per rank share (rotating the 8
    shares keeps the 176 MB per call coming from HBM)."""
    X = to_dev(torch, datagen.gaussian("X", (I, D), 1.0, "bf16", 3000 + I))
    H = torch.empty((I, F // TP), dtype=torch.bfloat16, device="cuda")
    P = torch.empty((I, D), dtype=torch.float32, device="cuda")
    return [(lambda R=R: tp.shard_mlp(X, *R["mlp"], H, P)) for R in layer.ranks]


def prefill_roofline(torch, tp, layer, calls):
    """The prefill side of the metric: one TP=8 rank's tp_shard_mlp at 512
    tokens (gate/up + SwiGLU GEMM, then the down GEMM), timed with HIP events
    on its launch stream, one event pair per group of 8 back-to-back calls
    (one per rank share), against the dense bf16 MFMA peak."""
    fns = prefill_mlp_fns(torch, tp, layer)
    us = time_calls(torch, fns, calls)
    avg = statistics.mean(us)
    m = wl.MlpShape(PREFILL_I, D, F // TP)
    tf = m.flops() / (avg * 1e-6) / 1e12
    return dict(bound="mfma", achieved=round(tf, 1), peak=PEAK_BF16, unit="TFLOP/s",
                frac=round(tf / PEAK_BF16, 4), traffic=None,
                kernel=f"tp_shard_mlp I={PREFILL_I} D={D} F_local={F // TP} "
                       "(gate/up + SwiGLU on gemm_wide_kernel, 256 x 128 tiles with K split "
                       "2 ways, then down on gemm_kernel, 128 x 128 tiles)",
                avg_call_us=round(avg, 2), median_call_us=stats(us)["median_us"],
                algorithmic_flops_per_call=m.flops())


def sample_clocks(torch, fns, samples=3):
    """SCLK (per XCD) and MCLK while the GPU runs `fns` back to back: each
    sample is one `amd-smi metric -c --json` child process, queried while
    the calls keep the GPU busy.  None when amd-smi is unavailable."""
    import shutil
    import subprocess
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe):
        return None
    sclk, mclk = [], []
    t0 = time.perf_counter()  # bring the clocks up from idle before the first sample
    while time.perf_counter() - t0 < 0.5:
        for _ in range(8):
            for f in fns:
                f()
        torch.cuda.synchronize()
    for k in range(samples):
        if k:  # the clock readings refresh about once a second: space the samples
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < 1.0:
                for _ in range(8):
                    for f in fns:
                        f()
                torch.cuda.synchronize()
        proc = subprocess.Popen([exe, "metric", "-c", "--json"], stdout=subprocess.PIPE,
                                stderr=subprocess.DEVNULL, text=True)
        t0 = time.perf_counter()
        inflight = []
        while proc.poll() is None and time.perf_counter() - t0 < 20.0:
            # keep two bursts queued so the GPU never idles while polling
            for _ in range(8):
                for f in fns:
                    f()
            ev = torch.cuda.Event()
            ev.record()
            inflight.append(ev)
            if len(inflight) > 2:
                inflight.pop(0).synchronize()
        torch.cuda.synchronize()
        try:
            out, _ = proc.communicate(timeout=10)
            clk = json.loads(out)["gpu_data"][0]["clock"]
        except Exception:  # noqa: BLE001 - a missing field only loses the sample
            continue
        g = [v["clk"]["value"] for k, v in clk.items()
             if k.startswith("gfx_") and isinstance(v.get("clk"), dict)]
        if g:
            sclk.append(g)
        m = clk.get("mem_0", {}).get("clk")
        if isinstance(m, dict):
            mclk.append(m["value"])
    if not sclk:
        return None
    return dict(sclk_mhz_per_xcd=sclk, mclk_mhz=mclk, sclk_spec_mhz=2400,
                how="amd-smi metric -c --json (each sample: the 8 XCDs' current GFX "
                    "clocks; samples at least 1 s apart) while the 512-token TP=8 MLP calls "
                    "run back to back")


def prefill_profile(torch, tp, layer, reps=20):
    """For rocprofv3 --kernel-trace: every 512-token prefill projection of a
    TP=8 rank in a phase of its own (reps calls each, rotating the rank
    shares), then the TP=1 MLP, so each kernel's dispatches can be told
    apart by grid and order."""
    T = torch
    I = PREFILL_I
    fns = prefill_mlp_fns(T, tp, layer)
    log("profile phase 1: TP=8 MLP 512 (gate/up + SwiGLU, down)")
    for k in range(reps):
        fns[k % TP]()
    T.cuda.synchronize()
    X = to_dev(T, datagen.gaussian("X", (I, D), 1.0, "bf16", 3600))
    nql, nkl = NQ // TP, NKV // TP
    qkv = T.empty((I, (nql + 2 * nkl) * HD), dtype=T.bfloat16, device="cuda")
    log("profile phase 2: TP=8 QKV 512")
    for k in range(reps):
        tp.shard_attn_proj(tp.TP_ATTN_QKV, X, layer.ranks[k % TP]["qkv"], qkv, nql, nkl, HD)
    T.cuda.synchronize()
    A = to_dev(T, datagen.gaussian("A", (I, nql * HD), 1.0, "bf16", 3601))
    Po = T.empty((I, D), dtype=T.float32, device="cuda")
    log("profile phase 3: TP=8 o_proj 512")
    for k in range(reps):
        tp.shard_attn_proj(tp.TP_ATTN_O, A, layer.ranks[k % TP]["o"], Po, nql, nkl, HD)
    T.cuda.synchronize()
    log("profile phase 4: TP=1 MLP 512")
    full = tuple(to_dev(T, a) for a in layer.host["mlp"])
    H1 = T.empty((I, F), dtype=T.bfloat16, device="cuda")
    Y1 = T.empty((I, D), dtype=T.float32, device="cuda")
    for _ in range(max(2, reps // 4)):
        tp.shard_mlp(X, *full, H1, Y1)
    T.cuda.synchronize()
    log("profile phases done")


def onebyte_ranks(T, kind):
    """8 seeded TP=8 Llama MLP rank shares stored one byte per weight with one
    fp32 scale per row: finite E4M3 codes with random signs (no 0x7F / 0xFF)
    for "fp8", signed int8 codes for "int8"."""
    Fl = F // TP
    gen = T.Generator(device="cuda")
    gen.manual_seed(8 if kind == "fp8" else 9)

    def codes(n, k):
        if kind == "int8":
            return T.randint(-128, 128, (n, k), generator=gen, device="cuda",
                             dtype=T.int32).to(T.int8)
        c = T.randint(0, 0x7F, (n, k), generator=gen, device="cuda", dtype=T.int32)
        c |= T.randint(0, 2, (n, k), generator=gen, device="cuda", dtype=T.int32) << 7
        return c.to(T.uint8)

    def scales(n):
        return T.rand((n,), generator=gen, device="cuda") * 1e-3 + 1e-4

    return [tuple((codes(n, k), scales(n)) for n, k in ((Fl, D), (Fl, D), (D, Fl)))
            for _ in range(TP)]


DECODE_PROFILE_I = (1, 8, 32, 128, 512)


def decode_profile(torch, tp, layer, reps=16):
    """For rocprofv3: the TP=8 rank's MLP at 1, 8, 32, 128 and 512 tokens
    with bf16, FP8 and int8 weights, each in a phase of its own (reps calls
    rotating the 8 rank shares), so each kernel's dispatches can be told
    apart by order."""
    T = torch
    Fl = F // TP
    phases = [("bf16", tp.shard_mlp, [R["mlp"] for R in layer.ranks])]
    phases += [(kind, call, onebyte_ranks(T, kind))
               for kind, call in (("fp8", tp.shard_mlp_fp8), ("int8", tp.shard_mlp_int8))]
    for kind, call, ranks in phases:
        for I in DECODE_PROFILE_I:
            X = to_dev(T, datagen.gaussian("X", (I, D), 1.0, "bf16", 1300 + I))
            H = T.empty((I, Fl), dtype=T.bfloat16, device="cuda")
            P = T.empty((I, D), dtype=T.float32, device="cuda")
            log(f"profile phase: {kind} MLP I={I}")
            for k in range(reps):
                call(X, *ranks[k % TP], H, P)
            T.cuda.synchronize()
    log("profile phases done")


ATTN_PROFILE_L = (2048, 8192)


def attn_profile(torch, tp, reps=8):
    """For rocprofv3: a plain copy of known size (the FETCH_SIZE / WRITE_SIZE
    calibration), then tp_attn_decode of a TP=8 rank (32 sequences, 8 query
    heads, 1 KV group, head_dim 128) at full cache length, reps calls per
    length rotating over cache copies larger than the Infinity Cache."""
    T = torch
    n = COPY_MIB * 2**20 // 4
    src = T.ones(n, dtype=T.float32, device="cuda")
    dst = T.empty_like(src)
    T.cuda.synchronize()
    T.mul(src, 1.0, out=dst)
    T.cuda.synchronize()
    del src, dst
    B, nql, nkl = 32, NQ // TP, NKV // TP
    qkv = to_dev(T, datagen.gaussian("A", (B, (nql + 2 * nkl) * HD), 1.0, "bf16", 4700))
    A = T.empty((B, nql * HD), dtype=T.bfloat16, device="cuda")
    for L in ATTN_PROFILE_L:
        cache_b = B * nkl * L * HD * 2
        copies = max(2, -(-300_000_000 // (2 * cache_b)))
        caches = [(T.randn((B, nkl, L, HD), device="cuda").to(T.bfloat16),
                   T.randn((B, nkl, HD, L), device="cuda").to(T.bfloat16)) for _ in range(copies)]
        lens = T.full((B,), L, dtype=T.int32, device="cuda")
        T.cuda.synchronize()
        log(f"profile phase: decode attention B=32 L={L}")
        for k in range(reps):
            kv = caches[k % copies]
            tp.attn_decode(lens, qkv, kv[0], kv[1], A, nql, nkl, HD)
        T.cuda.synchronize()
        del caches
    log("profile phases done")


def stats(us):
    us = sorted(us)
    q = lambda p: us[min(len(us) - 1, int(p * len(us)))]
    return dict(median_us=round(statistics.median(us), 2), p10_us=round(q(0.1), 2),
                p90_us=round(q(0.9), 2))


# Sources of everything a decode-size tp_shard_mlp call runs: the dispatch, the
# split-K gate/up kernel, the whole-K row-stream down kernel and their headers.
MLP_DECODE_SOURCES = tuple(f"megatron_tensor_layer_amd/csrc/{f}" for f in (
    "tpshard_api.cpp", "kernels.h", "common.h", "splitk.hip", "rowstream.hip"))


MLP_PREFILL_SOURCES = tuple(f"megatron_tensor_layer_amd/csrc/{f}" for f in (
    "tpshard_api.cpp", "kernels.h", "common.h", "gemm.hip"))


def src_hash(files=MLP_DECODE_SOURCES):
    """Hash of the sources the counted kernels are built from: stored counter
    figures are used only while those kernels are unchanged."""
    h = hashlib.sha256()
    for f in files:
        h.update((ROOT / f).read_bytes())
    return h.hexdigest()[:16]


COPY_MIB = 512  # calibration copy: reads and writes COPY_MIB MiB of fp32


def traffic_probe(torch, tp, layer, I):
    """Launch sequence read back by --ingest-traffic: a plain copy of known
    size (torch's elementwise multiply by 1), then tp_shard_mlp once per rank."""
    n = COPY_MIB * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    X = to_dev(torch, datagen.gaussian("X", (I, D), 1.0, "bf16", 42))
    B = layer.buffers(I)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    for R in layer.ranks:
        tp.shard_mlp(X, *R["mlp"], B["H"], B["pm"][0])
    torch.cuda.synchronize()
    log(f"traffic probe: copy of {COPY_MIB} MiB, then {len(layer.ranks)} tp_shard_mlp calls at I={I}")


def ingest_prefill_traffic(fetch_csv, write_csv):
    """FETCH_SIZE / WRITE_SIZE of one TP=8 rank's 512-token tp_shard_mlp call
    from the --prefill-profile counter runs: the first phase's gate/up and
    down GEMM dispatches, scaled by the copy calibration stored with the
    decode figures (the same counters on the same chip)."""
    import csv
    tf = ROOT / "profiles" / "traffic.json"
    tr = json.loads(tf.read_text())
    cal = tr[next(k for k in tr if k.startswith("mlp_I"))]["copy_calibration"]

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter
                and "tpk::" in r["Kernel_Name"] and "zero_words_kernel" not in r["Kernel_Name"]]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        phase = []
        for r in rows:  # phase 1 ends at the first QKV GEMM (bf16 epilogue)
            if "gemm_kernel<1>" in r["Kernel_Name"]:
                break
            phase.append(float(r["Counter_Value"]))
        if len(phase) % 2:
            raise SystemExit(f"{path}: odd number of MLP GEMM dispatches in phase 1")
        return phase

    fetch = read(fetch_csv, "FETCH_SIZE")
    write = read(write_csv, "WRITE_SIZE")
    calls = len(fetch) // 2
    fb = sum(fetch) * 1024 * cal["fetch_factor"] / calls
    wb = sum(write) * 1024 * cal["write_factor"] / calls
    tr["mlp_prefill_I512"] = dict(
        bytes_per_call=round(fb + wb), fetch_bytes_per_call=round(fb),
        write_bytes_per_call=round(wb), calls=calls, src_hash=src_hash(MLP_PREFILL_SOURCES),
        command="rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- "
                "python3 bench.py --prefill-profile")
    tf.write_text(json.dumps(tr, indent=1) + "\n")
    log(f"mlp_prefill_I512: {fb / 1e6:.1f} MB fetched + {wb / 1e6:.1f} MB written per call")


def ingest_traffic(fetch_csv, write_csv, I):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of one tp_shard_mlp call,
    each scaled by what the counter reads for the calibration copy."""
    import csv

    def read(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copy = [r for r in rows if "MulFunctor" in r["Kernel_Name"]]
        if len(copy) != 1:
            raise SystemExit(f"{path}: expected one calibration copy dispatch, found {len(copy)}")
        # the MLP call's kernels; the binding's one-off workspace reset is not part of a call
        after = [r for r in rows if int(r["Dispatch_Id"]) > int(copy[0]["Dispatch_Id"])
                 and "tpk::" in r["Kernel_Name"] and "zero_words_kernel" not in r["Kernel_Name"]]
        per_kernel = {}
        for r in after:
            per_kernel.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return float(copy[0]["Counter_Value"]), per_kernel

    true_bytes = COPY_MIB * 2**20
    cf, kf = read(fetch_csv, "FETCH_SIZE")
    cw, kw = read(write_csv, "WRITE_SIZE")
    f_fetch, f_write = true_bytes / (cf * 1024), true_bytes / (cw * 1024)
    calls = max(len(v) for v in kf.values())
    fetch = sum(sum(v) for v in kf.values()) * 1024 * f_fetch / calls
    write = sum(sum(v) for v in kw.values()) * 1024 * f_write / calls
    key = f"mlp_I{I}"
    tf = ROOT / "profiles" / "traffic.json"
    tr = json.loads(tf.read_text()) if tf.exists() else {}
    tr[key] = dict(
        bytes_per_call=round(fetch + write), fetch_bytes_per_call=round(fetch),
        write_bytes_per_call=round(write), calls=calls,
        copy_calibration=dict(bytes_read=true_bytes, bytes_written=true_bytes,
                              fetch_size_kib=cf, write_size_kib=cw,
                              fetch_factor=round(f_fetch, 4), write_factor=round(f_write, 4)),
        kernels_kib_per_dispatch={k: dict(fetch=round(sum(kf[k]) / len(kf[k]), 1),
                                          write=round(sum(kw.get(k, [0])) / max(1, len(kw.get(k, [0]))), 1))
                                  for k in kf},
        src_hash=src_hash(),
        command="rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --output-format csv -- "
                f"python3 bench.py --traffic-probe --batch {I}")
    tf.write_text(json.dumps(tr, indent=1) + "\n")
    log(f"{key}: {fetch / 1e6:.1f} MB fetched + {write / 1e6:.1f} MB written per call "
        f"(copy factors {f_fetch:.3f} / {f_write:.3f})")


# ------------------------------------------------------------------ the layer
class Layer:
    """All 8 TP rank shares of the Llama-3.1-70B-shaped layer, resident in HBM."""

    def __init__(self, torch, tp, pool=11):
        self.torch, self.tp = torch, tp
        Wq, Wk, Wv, Wo = datagen.attn_weights(D, NQ, NKV, HD, "bf16", pool)
        Wg, Wu, Wd = datagen.mlp_weights(D, F, "bf16", pool)
        self.host = dict(attn=(Wq, Wk, Wv, Wo), mlp=(Wg, Wu, Wd))
        self.ranks = []
        for r in range(TP):
            self.ranks.append(dict(
                qkv=to_dev(torch, datagen.qkv_rank_shard(Wq, Wk, Wv, NQ, NKV, HD, TP, r)),
                o=to_dev(torch, datagen.oproj_rank_shard(Wo, NQ, HD, TP, r)),
                mlp=tuple(to_dev(torch, a) for a in datagen.mlp_rank_shards(Wg, Wu, Wd, TP, r))))
        self.nql, self.nkl = NQ // TP, NKV // TP
        # replicated RMSNorm scales in front of attention and MLP (and of the next layer)
        self.gammas = [to_dev(torch, datagen.rmsnorm_gamma(D, pool + k, "bf16"))
                       for k in range(3)]

    def buffers(self, I):
        T = self.torch
        bf, f32 = T.bfloat16, T.float32
        return dict(I=I, qkv=T.empty((I, (self.nql + 2 * self.nkl) * HD), dtype=bf, device="cuda"),
                    A=T.empty((I, self.nql * HD), dtype=bf, device="cuda"),
                    po=T.empty((TP, I, D), dtype=f32, device="cuda"),
                    y1=T.empty((I, D), dtype=bf, device="cuda"),
                    H=T.empty((I, F // TP), dtype=bf, device="cuda"),
                    pm=T.empty((TP, I, D), dtype=f32, device="cuda"),
                    y=T.empty((I, D), dtype=f32, device="cuda"),
                    x=T.empty((I, D), dtype=bf, device="cuda"))

    def step(self, X, B, S, mlp_events=None):
        tp = self.tp
        for r, R in enumerate(self.ranks):
            tp.shard_attn_proj(tp.TP_ATTN_QKV, X, R["qkv"], B["qkv"], self.nql, self.nkl, HD)
            tp.attn_core(B["qkv"], B["A"], S, self.nql, self.nkl, HD)
            tp.shard_attn_proj(tp.TP_ATTN_O, B["A"], R["o"], B["po"][r], self.nql, self.nkl, HD)
        tp.partial_reduce(B["po"], B["y1"])
        s = self.torch.cuda.current_stream()
        if mlp_events is not None:  # one event pair around the 8 back-to-back calls
            e0, e1 = (self.torch.cuda.Event(enable_timing=True) for _ in range(2))
            e0.record(s)
        for r, R in enumerate(self.ranks):
            tp.shard_mlp(B["y1"], *R["mlp"], B["H"], B["pm"][r])
        if mlp_events is not None:
            e1.record(s)
            mlp_events.append((e0, e1))
        tp.partial_reduce(B["pm"], B["y"])


    def prenorm_step(self, h, B, S):
        """The layer as a pre-norm block on the residual stream h [I, D] bf16
        (updated in place): x = RMSNorm(h); per rank QKV -> attention core ->
        o_proj; h += sum of the partials, x = RMSNorm(h); per rank MLP;
        h += sum of the partials, x = RMSNorm(h) (the next layer's input).
        The RMSNorm every rank repeats is computed once here: same result."""
        tp, g = self.tp, self.gammas
        tp.residual_rmsnorm(None, h, h, g[0], B["x"])
        for r, R in enumerate(self.ranks):
            tp.shard_attn_proj(tp.TP_ATTN_QKV, B["x"], R["qkv"], B["qkv"], self.nql, self.nkl, HD)
            tp.attn_core(B["qkv"], B["A"], S, self.nql, self.nkl, HD)
            tp.shard_attn_proj(tp.TP_ATTN_O, B["A"], R["o"], B["po"][r], self.nql, self.nkl, HD)
        tp.residual_rmsnorm(B["po"], h, h, g[1], B["x"])
        for r, R in enumerate(self.ranks):
            tp.shard_mlp(B["x"], *R["mlp"], B["H"], B["pm"][r])
        tp.residual_rmsnorm(B["pm"], h, h, g[2], B["x"])


def step_bytes(I, S):
    """Compulsory HBM bytes of one step (all 8 ranks, both reduces)."""
    q = wl.QkvShape(I, D, NQ // TP, NKV // TP, HD)
    o = wl.OprojShape(I, D, NQ // TP, HD)
    m = wl.MlpShape(I, D, F // TP)
    attn_core = (I * q.N + I * o.K) * wl.BF16 if S == 1 else None
    per_rank = q.bytes() + o.bytes() + m.bytes() + (attn_core or 0)
    red = wl.ReduceShape(TP, I * D, wl.BF16).bytes() + wl.ReduceShape(TP, I * D, wl.F32).bytes()
    return TP * per_rank + red


def prenorm_step_bytes(I, S):
    """Compulsory bytes of the pre-norm block: the projections and attention
    as in step_bytes, plus the first RMSNorm and the two residual updates
    with RMSNorm in place of the two reduces."""
    red = wl.ReduceShape(TP, I * D, wl.BF16).bytes() + wl.ReduceShape(TP, I * D, wl.F32).bytes()
    norms = (wl.ResidualNormShape(0, I, D).bytes() +
             2 * wl.ResidualNormShape(TP, I, D).bytes())
    return step_bytes(I, S) - red + norms


def step_flops(I):
    q = wl.QkvShape(I, D, NQ // TP, NKV // TP, HD)
    o = wl.OprojShape(I, D, NQ // TP, HD)
    m = wl.MlpShape(I, D, F // TP)
    return TP * (q.flops() + o.flops() + m.flops())


# ------------------------------------------------------------------ detail
def detail(torch, tp, layer, calls):
    out = {}
    T = torch
    # Llama-3.1-70B MLP rank share, TP=8: rotate through the 8 real rank shards
    for I in (1, 8, 16, 32, 64, 256):
        X = to_dev(T, datagen.gaussian("X", (I, D), 1.0, "bf16", 1000 + I))
        H = T.empty((I, F // TP), dtype=T.bfloat16, device="cuda")
        P = T.empty((I, D), dtype=T.float32, device="cuda")
        fns = [(lambda R=R: tp.shard_mlp(X, *R["mlp"], H, P)) for R in layer.ranks]
        st = stats(time_calls(T, fns, calls))
        m = wl.MlpShape(I, D, F // TP)
        gbs = m.bytes() / (st["median_us"] * 1e-6) / 1e9
        log(f"MLP TP=8 decode I={I}: {st['median_us']} us")
        out[f"llama70b_mlp_tp8_decode_I{I}"] = dict(
            **st, GBps=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM, 3),
            TFLOPs=round(m.flops() / (st["median_us"] * 1e-6) / 1e12, 1),
            tokens_per_s=round(I / (st["median_us"] * 1e-6)))
    # the same rank shares with weight-only FP8 storage (E4M3 codes + one fp32
    # scale per row), then with int8 storage (signed codes + one fp32 scale per
    # row): 8 seeded random shares each, one byte per weight
    Fl = F // TP
    for kind, call, seed in (("fp8", tp.shard_mlp_fp8, 1100), ("int8", tp.shard_mlp_int8, 1200)):
        ranks = onebyte_ranks(T, kind)
        for I in (1, 8, 32, 128, 512):
            X = to_dev(T, datagen.gaussian("X", (I, D), 1.0, "bf16", seed + I))
            H = T.empty((I, Fl), dtype=T.bfloat16, device="cuda")
            P = T.empty((I, D), dtype=T.float32, device="cuda")
            fns = [(lambda w=w: call(X, *w, H, P)) for w in ranks]
            st = stats(time_calls(T, fns, calls))
            nbytes = 3 * D * Fl + 4 * (2 * Fl + D) + 2 * I * D + 4 * I * D
            gbs = nbytes / (st["median_us"] * 1e-6) / 1e9
            log(f"{'FP8' if kind == 'fp8' else 'int8'} MLP TP=8 decode I={I}: {st['median_us']} us")
            m = wl.MlpShape(I, D, Fl)
            tf = m.flops() / (st["median_us"] * 1e-6) / 1e12
            out[f"llama70b_mlp_{kind}_tp8_{'decode' if I <= 256 else 'prefill'}_I{I}"] = dict(
                **st, bytes_per_call=nbytes, GBps=round(gbs, 1),
                frac_hbm=round(gbs / PEAK_HBM, 3), TFLOPs=round(tf, 1),
                frac_mfma=round(tf / PEAK_BF16, 3), tokens_per_s=round(I / (st["median_us"] * 1e-6)))
        del ranks
    # the attention projections of the layer's rank shares at decode 32
    I = 32
    nql, nkl = NQ // TP, NKV // TP
    X = to_dev(T, datagen.gaussian("X", (I, D), 1.0, "bf16", 1032))
    A = to_dev(T, datagen.gaussian("A", (I, nql * HD), 1.0, "bf16", 1032))
    Q = T.empty((I, (nql + 2 * nkl) * HD), dtype=T.bfloat16, device="cuda")
    P = T.empty((I, D), dtype=T.float32, device="cuda")
    for name, fns, nbytes in (
            ("qkv", [(lambda R=R: tp.shard_attn_proj(tp.TP_ATTN_QKV, X, R["qkv"], Q, nql, nkl, HD))
                     for R in layer.ranks], wl.QkvShape(I, D, nql, nkl, HD).bytes()),
            ("o_proj", [(lambda R=R: tp.shard_attn_proj(tp.TP_ATTN_O, A, R["o"], P, nql, nkl, HD))
                        for R in layer.ranks], wl.OprojShape(I, D, nql, HD).bytes())):
        st = stats(time_calls(T, fns, calls))
        gbs = nbytes / (st["median_us"] * 1e-6) / 1e9
        out[f"llama70b_{name}_tp8_decode_I32"] = dict(**st, GBps=round(gbs, 1),
                                                      frac_hbm=round(gbs / PEAK_HBM, 3))
    # prefill 512, TP=8 shards and the TP=1 unsharded MLP
    I = 512
    X = to_dev(T, datagen.gaussian("X", (I, D), 1.0, "bf16", 1512))
    H = T.empty((I, F // TP), dtype=T.bfloat16, device="cuda")
    P = T.empty((I, D), dtype=T.float32, device="cuda")
    fns = [(lambda R=R: tp.shard_mlp(X, *R["mlp"], H, P)) for R in layer.ranks]
    st = stats(time_calls(T, fns, calls // 2))
    m = wl.MlpShape(I, D, F // TP)
    tf = m.flops() / (st["median_us"] * 1e-6) / 1e12
    out["llama70b_mlp_tp8_prefill_I512"] = dict(**st, TFLOPs=round(tf, 1),
                                                frac_mfma=round(tf / PEAK_BF16, 3),
                                                tokens_per_s=round(I / (st["median_us"] * 1e-6)))
    # the attention projections of the rank shares at prefill 512
    A = to_dev(T, datagen.gaussian("A", (I, nql * HD), 1.0, "bf16", 1512))
    Q = T.empty((I, (nql + 2 * nkl) * HD), dtype=T.bfloat16, device="cuda")
    for name, fns, shape in (
            ("qkv", [(lambda R=R: tp.shard_attn_proj(tp.TP_ATTN_QKV, X, R["qkv"], Q, nql, nkl, HD))
                     for R in layer.ranks], wl.QkvShape(I, D, nql, nkl, HD)),
            ("o_proj", [(lambda R=R: tp.shard_attn_proj(tp.TP_ATTN_O, A, R["o"], P, nql, nkl, HD))
                        for R in layer.ranks], wl.OprojShape(I, D, nql, HD))):
        st = stats(time_calls(T, fns, calls // 2))
        tf = shape.flops() / (st["median_us"] * 1e-6) / 1e12
        out[f"llama70b_{name}_tp8_prefill_I512"] = dict(**st, TFLOPs=round(tf, 1),
                                                        frac_mfma=round(tf / PEAK_BF16, 3))
    full = tuple(to_dev(T, a) for a in layer.host["mlp"])
    H1 = T.empty((I, F), dtype=T.bfloat16, device="cuda")
    st = stats(time_calls(T, [lambda: tp.shard_mlp(X, *full, H1, P)], max(10, calls // 10), 3))
    m = wl.MlpShape(I, D, F)
    tf = m.flops() / (st["median_us"] * 1e-6) / 1e12
    out["llama70b_mlp_tp1_prefill_I512"] = dict(**st, TFLOPs=round(tf, 1),
                                                frac_mfma=round(tf / PEAK_BF16, 3))
    del full, H1
    # layer prefill 512 (one causal sequence), 8 ranks + reduces
    B = layer.buffers(512)
    X = to_dev(T, datagen.gaussian("X", (512, D), 1.0, "bf16", 2512))
    st = stats(time_calls(T, [lambda: layer.step(X, B, 512)], 10, 2))
    tf = step_flops(512) / (st["median_us"] * 1e-6) / 1e12
    out["llama70b_layer_tp8x8_prefill_I512"] = dict(
        **st, TFLOPs_projections=round(tf, 1), frac_mfma=round(tf / PEAK_BF16, 3),
        tokens_per_s_excl_comm=round(512 / (st["median_us"] * 1e-6)))
    del B
    # partial reduce of 8 fp32 partials
    for I in (32, 512):
        Pp = T.randn((TP, I, D), device="cuda")
        Y = T.empty((I, D), dtype=T.float32, device="cuda")
        st = stats(time_calls(T, [lambda: tp.partial_reduce(Pp, Y)], calls))
        gbs = wl.ReduceShape(TP, I * D).bytes() / (st["median_us"] * 1e-6) / 1e9
        out[f"reduce_t8_I{I}"] = dict(**st, GBps=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM, 3))
    # residual update + RMSNorm after a block's reduce of 8 partials (bf16 h, x)
    for I in (32, 512):
        Pp = T.randn((TP, I, D), device="cuda")
        h = to_dev(T, datagen.gaussian("h", (I, D), 1.0, "bf16", 4000 + I))
        x = T.empty((I, D), dtype=T.bfloat16, device="cuda")
        g = layer.gammas[1]
        st = stats(time_calls(T, [lambda: tp.residual_rmsnorm(Pp, h, h, g, x)], calls))
        gbs = wl.ResidualNormShape(TP, I, D).bytes() / (st["median_us"] * 1e-6) / 1e9
        out[f"residual_rmsnorm_t8_I{I}"] = dict(**st, GBps=round(gbs, 1),
                                                frac_hbm=round(gbs / PEAK_HBM, 3))
    # decode attention of a TP=8 rank over its KV cache (8 query heads, 1 KV
    # group, head_dim 128), 32 sequences at full cache length; cache copies
    # rotate so the reads come from HBM, not the Infinity Cache
    B, nql, nkl = 32, NQ // TP, NKV // TP
    qkv = to_dev(T, datagen.gaussian("A", (B, (nql + 2 * nkl) * HD), 1.0, "bf16", 4700))
    A = T.empty((B, nql * HD), dtype=T.bfloat16, device="cuda")
    for L in (2048, 8192):
        cache_b = B * nkl * L * HD * 2
        copies = max(2, -(-300_000_000 // (2 * cache_b)))
        caches = [(T.randn((B, nkl, L, HD), device="cuda").to(T.bfloat16),
                   T.randn((B, nkl, HD, L), device="cuda").to(T.bfloat16)) for _ in range(copies)]
        lens = T.full((B,), L, dtype=T.int32, device="cuda")
        fns = [(lambda kv=kv: tp.attn_decode(lens, qkv, kv[0], kv[1], A, nql, nkl, HD))
               for kv in caches]
        st = stats(time_calls(T, fns, calls // 2))
        nbytes = 2 * cache_b + qkv.numel() * 2 + A.numel() * 2
        gbs = nbytes / (st["median_us"] * 1e-6) / 1e9
        out[f"llama70b_attn_decode_tp8_B32_L{L}"] = dict(**st, bytes_per_call=nbytes,
                                                        GBps=round(gbs, 1),
                                                        frac_hbm=round(gbs / PEAK_HBM, 3))
        log(f"decode attention B=32 L={L}: {st['median_us']} us")
        del caches
    # the sequence-parallel form at prefill 512: 8 ranks' reduce-scatter + norm
    # on their 64 rows each, x gathered in place into one [512, D] buffer
    I = 512
    Pp = T.randn((TP, I, D), device="cuda")
    h = to_dev(T, datagen.gaussian("h", (I, D), 1.0, "bf16", 4512))
    x = T.empty((I, D), dtype=T.bfloat16, device="cuda")
    g = layer.gammas[1]
    Is = I // TP

    def sp_all():
        for r in range(TP):
            sl = slice(r * Is, (r + 1) * Is)
            tp.reduce_scatter_rmsnorm(Pp, r, h[sl], h[sl], g, x[sl])

    st = stats(time_calls(T, [sp_all], calls // 2))
    gbs = wl.ResidualNormShape(TP, I, D).bytes() / (st["median_us"] * 1e-6) / 1e9
    out["sequence_parallel_norm_t8_I512_all_ranks"] = dict(**st, GBps=round(gbs, 1),
                                                           frac_hbm=round(gbs / PEAK_HBM, 3))
    # the layer as a pre-norm block (RMSNorm, attention block, residual + RMSNorm,
    # MLP, residual + RMSNorm), decode 32
    I = 32
    B = layer.buffers(I)
    h = to_dev(T, datagen.gaussian("h", (I, D), 1.0, "bf16", 4032))
    st = stats(time_calls(T, [lambda: layer.prenorm_step(h, B, 1)], 20, 3))
    nb = prenorm_step_bytes(I, 1)
    gbs = nb / (st["median_us"] * 1e-6) / 1e9
    out["llama70b_prenorm_layer_tp8x8_decode_I32"] = dict(
        **st, bytes_per_step=nb, GBps=round(gbs, 1), frac_hbm=round(gbs / PEAK_HBM, 3),
        tokens_per_s_excl_comm=round(I / (st["median_us"] * 1e-6)))
    log(f"pre-norm layer decode 32: {st['median_us']} us")
    del B
    # Qwen2.5-1.5B-shaped rank share at TP=2: 24 independently seeded rank
    # shares rotate so the calls stream from HBM, not the Infinity Cache
    Dq, Fq, nq, nkv, t = 1536, 8960, 12, 2, 2
    pools = []
    for p in range(24):
        Wg = datagen.gaussian("W_gate", (Fq // t, Dq), Dq ** -0.5, "bf16", 5000 + p)
        Wu = datagen.gaussian("W_up", (Fq // t, Dq), Dq ** -0.5, "bf16", 5000 + p)
        Wd = datagen.gaussian("W_down", (Dq, Fq // t), Dq ** -0.5, "bf16", 5000 + p)
        Wqkv = datagen.gaussian("W_q", ((nq // t + 2 * nkv // t) * 128, Dq), Dq ** -0.5, "bf16",
                                5000 + p)
        Wo = datagen.gaussian("W_o", (Dq, nq // t * 128), Dq ** -0.5, "bf16", 5000 + p)
        pools.append(tuple(to_dev(T, a) for a in (Wg, Wu, Wd, Wqkv, Wo)))
    for I in (1, 8, 64):
        X = to_dev(T, datagen.gaussian("X", (I, Dq), 1.0, "bf16", 3000 + I))
        A = to_dev(T, datagen.gaussian("A", (I, nq // t * 128), 1.0, "bf16", 3000 + I))
        H = T.empty((I, Fq // t), dtype=T.bfloat16, device="cuda")
        P = T.empty((I, Dq), dtype=T.float32, device="cuda")
        Q = T.empty((I, (nq // t + 2 * nkv // t) * 128), dtype=T.bfloat16, device="cuda")
        row = {}
        for name, fns, nbytes in (
                ("mlp", [(lambda w=w: tp.shard_mlp(X, w[0], w[1], w[2], H, P)) for w in pools],
                 wl.MlpShape(I, Dq, Fq // t).bytes()),
                ("qkv", [(lambda w=w: tp.shard_attn_proj(tp.TP_ATTN_QKV, X, w[3], Q, nq // t,
                                                         nkv // t, 128)) for w in pools],
                 wl.QkvShape(I, Dq, nq // t, nkv // t, 128).bytes()),
                ("o_proj", [(lambda w=w: tp.shard_attn_proj(tp.TP_ATTN_O, A, w[4], P, nq // t,
                                                            nkv // t, 128)) for w in pools],
                 wl.OprojShape(I, Dq, nq // t, 128).bytes())):
            st = stats(time_calls(T, fns, calls))
            row[name] = dict(**st, GBps=round(nbytes / (st["median_us"] * 1e-6) / 1e9, 1))
        out[f"qwen2.5_1.5b_tp2_decode_I{I}"] = row
    del pools
    return out


# ------------------------------------------------------------------ CPU baseline
CPU_SAMPLE_S = 10.0  # oracle work timed for the baseline


def cpu_baseline(layer, X, I, S, bytes_per_step):
    """The fp64 oracle, untuned, on whole steps (all 8 ranks' QKV, attention
    core, o_proj and MLP for all I tokens, plus both reduces), repeated until
    about CPU_SAMPLE_S seconds of work; the rate is the mean over the steps."""
    import oracle
    orc = oracle.get()
    # fp64 copies made before the clock starts: the oracle's own work is timed
    Wq, Wk, Wv, Wo = (a.astype(np.float64) for a in layer.host["attn"])
    Wg, Wu, Wd = (a.astype(np.float64) for a in layer.host["mlp"])
    X = X.astype(np.float64)
    steps = 0
    t0 = time.perf_counter()
    while True:
        po = np.stack([orc.attn_block_rank(X, Wq, Wk, Wv, Wo, NQ, NKV, HD, S, TP, r)[2]
                       for r in range(TP)])
        y1 = orc.reduce(po)
        pm = np.stack([orc.mlp_rank(y1, Wg, Wu, Wd, TP, r)[1] for r in range(TP)])
        orc.reduce(pm)
        steps += 1
        total_s = time.perf_counter() - t0
        if total_s >= CPU_SAMPLE_S:
            break
    step_s = total_s / steps
    return dict(value=round(bytes_per_step / step_s / 1e9, 3), unit="GB/s",
                cores=oracle.num_threads(), cpu=cpu_model(), kind="oracle",
                sample=f"{steps} whole steps: 8 ranks x (QKV, attention core, o_proj, MLP) for "
                       f"all {I} tokens plus both reduces, {total_s:.1f} s in all")


def read_ceiling(torch, tp, calls=20):
    """The achievable read rate: tp_stream_read over 2 GiB (8x the Infinity
    Cache), the decode kernels' access pattern, median of `calls` reads."""
    nbytes = 1 << 31
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    sink = tp.stream_read(buf)
    for _ in range(3):
        tp.stream_read(buf, sink)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(calls)]
    for a, b in ev:
        a.record()
        tp.stream_read(buf, sink)
        b.record()
    torch.cuda.synchronize()
    us = statistics.median(a.elapsed_time(b) * 1e3 for a, b in ev)
    del buf, sink
    torch.cuda.empty_cache()
    return dict(GBps=round(nbytes / (us * 1e-6) / 1e9, 1), bytes=nbytes, calls=calls,
                median_us=round(us, 2), frac_of_peak=round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM, 4),
                kernel="tp_stream_read: one 16-wave workgroup per CU, 1 KB per wave load, "
                       "3 loads in flight per wave")


def cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ main
def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for {max(args.gpus, world)}): the TP "
              "ranks are emulated in turn on a single device and no collective is used.",
              file=sys.stderr)
        sys.exit(2)

    I, S = args.batch, 1
    if args.ingest_traffic:
        ingest_traffic(*args.ingest_traffic, I)
        return
    if args.ingest_prefill_traffic:
        ingest_prefill_traffic(*args.ingest_prefill_traffic)
        return

    import torch
    import megatron_tensor_layer_amd as tp

    torch.cuda.set_device(0)
    tp.lib()
    layer = Layer(torch, tp)
    log("8 rank shares of the layer resident in HBM")
    if args.traffic_probe:
        traffic_probe(torch, tp, layer, I)
        return
    if args.prefill_profile:
        prefill_profile(torch, tp, layer)
        return
    if args.decode_profile:
        decode_profile(torch, tp, layer)
        return
    if args.attn_profile:
        attn_profile(torch, tp)
        return
    Xh = datagen.gaussian("X", (I, D), 1.0, "bf16", 42)
    X = to_dev(torch, Xh)
    B = layer.buffers(I)

    for _ in range(args.warmup):
        layer.step(X, B, S)
    torch.cuda.synchronize()
    mlp_ev = []
    t0 = time.perf_counter()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(args.steps):
        layer.step(X, B, S, mlp_events=mlp_ev)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = e0.elapsed_time(e1) / args.steps
    nbytes = step_bytes(I, S)
    value = nbytes / (ms * 1e-3) / 1e9

    log(f"timed {args.steps} steps: {ms:.3f} ms/step")
    mlp_us = statistics.mean(a.elapsed_time(b) * 1e3 for a, b in mlp_ev) / TP  # per call
    mlp_bytes = wl.MlpShape(I, D, F // TP).bytes()
    achieved = mlp_bytes / (mlp_us * 1e-6) / 1e9
    roof = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM, unit="GB/s",
                frac=round(achieved / PEAK_HBM, 4), traffic=None,
                kernel=f"tp_shard_mlp I={I} D={D} F_local={F // TP} "
                       "(gate/up+SwiGLU kernel, then down kernel)",
                avg_call_us=round(mlp_us, 2), algorithmic_bytes_per_call=mlp_bytes)
    ceiling = read_ceiling(torch, tp)
    log(f"read ceiling: {ceiling['GBps']} GB/s over 2 GiB")
    roof["frac_of_read_ceiling"] = round(achieved / ceiling["GBps"], 4)
    roof_pf = prefill_roofline(torch, tp, layer, max(args.calls, 8))
    log(f"prefill roofline: TP=8 MLP 512 {roof_pf['avg_call_us']} us, "
        f"{roof_pf['achieved']} TFLOP/s")
    clocks = sample_clocks(torch, prefill_mlp_fns(torch, tp, layer))
    log(f"clocks under load: {clocks}")
    tf = ROOT / "profiles" / "traffic.json"
    if tf.exists():
        tr = json.loads(tf.read_text())
        key = f"mlp_I{I}"
        if key in tr and tr[key].get("src_hash") == src_hash():
            roof["traffic"] = tr[key]["bytes_per_call"]
        pk = "mlp_prefill_I512"
        if pk in tr and tr[pk].get("src_hash") == src_hash(MLP_PREFILL_SOURCES):
            roof_pf["traffic"] = tr[pk]["bytes_per_call"]

    line = dict(
        metric="TP-rank MLP shard: decode HBM GB/s, prefill MFMA TFLOP/s, % roofline",
        value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms, 4), wall_ms_per_step=round(wall_ms, 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload=f"llama3.1-70b-shaped layer, TP=8 ranks emulated in turn on one "
                             f"GPU, decode batch {I} (32 sequences x 1 token): QKV, attention "
                             "core, o_proj, reduce, SwiGLU MLP, reduce",
                    D=D, F=F, n_q=NQ, n_kv=NKV, head_dim=HD, tp=TP, tokens=I,
                    bytes_per_step=nbytes, flops_per_step=step_flops(I),
                    tokens_per_s_excl_comm=round(I / (ms * 1e-3), 1),
                    frac_hbm=round(value / PEAK_HBM, 4),
                    frac_read_ceiling=round(value / ceiling["GBps"], 4)),
        roofline=roof, roofline_prefill=roof_pf, clocks=clocks, read_ceiling=ceiling)

    if not args.no_detail:
        line["detail"] = detail(torch, tp, layer, args.calls)
        log("per-config detail done")
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(layer, Xh, I, S, nbytes)
        log("cpu baseline done")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
