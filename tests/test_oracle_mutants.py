"""The oracle's pins must catch plausible mistakes.

Each case copies oracle.c, plants one mistake by a text substitution (on the
CPU, in a temporary directory), compiles the copy and runs every pin of
test_oracle_pins against it: at least one pin has to fail.  The committed
oracle itself is never modified."""
import pathlib
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = {
    "gate_up_swapped": ("orc_silu(g) * u", "orc_silu(u) * g"),
    "silu_sign": ("1.0 + exp(-z)", "1.0 + exp(z)"),
    "dropped_last_k": ("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k + 1 < K; ++k)"),
    "down_shard_offset": ("Wd[n * F + f]", "Wd[n * F + (f - f0)]"),
    "down_transposed": ("Wd[n * F + f]", "Wd[f * D + n]"),
    "reduce_drops_rank": ("for (int64_t r = 0; r < t; ++r)", "for (int64_t r = 0; r + 1 < t; ++r)"),
    "shard_start": ("*lo = r * (n / t);", "*lo = r * (n / t) + (r > 0);"),
    "attn_no_scale": ("1.0 / sqrt((double)hd)", "1.0"),
    "attn_not_causal_per_seq": ("const int64_t s0 = (i / S) * S;", "const int64_t s0 = 0;"),
    "gqa_map": ("const int64_t g = (j * nkl) / nql;", "const int64_t g = j % nkl;"),
    "qkv_k_from_v": ("w = Wk + (g0 * hd + (c - Nq)) * D;", "w = Wv + (g0 * hd + (c - Nq)) * D;"),
    "oproj_offset": ("Wo[n * K + c0 + c]", "Wo[n * K + c]"),
    "rms_no_eps": ("sqrt(ss / (double)D + eps)", "sqrt(ss / (double)D)"),
    "rms_sum_not_mean": ("ss / (double)D + eps", "ss + eps"),
    "rms_no_gamma": ("* inv * gamma[j]", "* inv"),
    "rms_no_sqrt": ("1.0 / sqrt(ss / (double)D + eps)", "1.0 / (ss / (double)D + eps)"),
    "residual_dropped": ("double v = residual ? residual[i * D + j] : 0.0;", "double v = 0.0;"),
    "e4m3_bias": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "e4m3_no_subnormal": ("ldexp(m / 8.0, -6)", "ldexp(1.0 + m / 8.0, -7)"),
    "e4m3_mantissa": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 16.0, e - 7)"),
    "decode_drops_new_token": ("for (int64_t p = 0; p < L; ++p) {\n        const double *k", "for (int64_t p = 0; p + 1 < L; ++p) {\n        const double *k"),
    "decode_new_k_from_cache": ("const double *k = (p == L - 1) ? qkv + b * N + (nq + g) * hd", "const double *k = (p == L) ? qkv + b * N + (nq + g) * hd"),
    "decode_gqa_map": ("const int64_t g = (j * nkv) / nq, L = lens[b];", "const int64_t g = j % nkv, L = lens[b];"),
    "decode_cache_batch": (": Kc + ((b * nkv + g) * Lmax + p) * hd;", ": Kc + (g * Lmax + p) * hd;"),
    "decode_v_new_token": ("const double *v = (p == L - 1) ? qkv + b * N + (nq + nkv + g) * hd", "const double *v = (p == L - 1) ? qkv + b * N + (nq + g) * hd"),
    "bf16_round_toward_zero": ("ldexp(nearbyint(ldexp(x, -q)), q)", "ldexp(trunc(ldexp(x, -q)), q)"),
    "bf16_round_extra_bit": ("int q = e - 8;", "int q = e - 9;"),
    "bf16_round_no_subnormal_floor": ("if (q < -133) q = -133;", "if (q < -140) q = -140;"),
    "bf16h_down_from_unrounded": ("sb += Hb[q * Fl + (f - f0)] * Wd[n * F + f];", "sb += H[q * Fl + (f - f0)] * Wd[n * F + f];"),
    "int8_unsigned": ("scales[n] * (double)codes[n * K + k]", "scales[n] * (double)(unsigned char)codes[n * K + k]"),
    "int8_row_scale": ("W[n * K + k] = scales[n] * (double)codes", "W[n * K + k] = scales[k % N] * (double)codes"),
    "fp8_row_scale": ("scales[n] * orc_e4m3(codes[n * K + k])", "scales[k % N] * orc_e4m3(codes[n * K + k])"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path: pathlib.Path):
    old, new = MUTANTS[name]
    src = oracle.SRC.read_text()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = tmp_path / "oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", *oracle.CFLAGS, str(mutated), "-o", str(lib), "-lm"], check=True)
    mut = oracle.Oracle(lib)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(mut)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin caught the planted mistake {name}"
