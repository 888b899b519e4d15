/*
 * oracle.c -- plain, slow, fp64 CPU oracle for one tensor-parallel rank's
 * share of a Megatron-style transformer layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or helper with the
 * HIP library.
 *
 * Every value is read as the exact fp64 of its (bf16 or fp32) input and every
 * sum runs in increasing index order in fp64.  There is no blocking, fusion or
 * reordering: each output element is one plain loop.  OpenMP only spreads
 * independent output elements over threads; it never splits a sum.
 *
 * Notation follows "Lecture 4 - Distributed Serving" (cs349e notes), §3.1:
 * A[I_X, J] means dimension I of A is split over mesh axis X.  Weights are
 * stored output-major, one contiguous K-vector per output channel, the way the
 * vLLM ColumnParallelLinear keeps its [output_size_per_partition, input_size]
 * parameter (intelliparadigm vLLM article, §2.1).  So a logical W[D, F] is the
 * array Ws[F][D] with W[d, f] == Ws[f][d].
 *
 * Shards are contiguous blocks in rank order (the plainest reading of the
 * "I/|X| rows per device" statement of §3.1): rank r of t owns
 * [r*N/t, (r+1)*N/t) of a split dimension of size N.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* SiLU, the gate nonlinearity of the SwiGLU MLP (lecture §4.1 names SwiGLU
 * but not its form; the Llama form silu(gate) * up is taken):
 * silu(z) = z * sigmoid(z) = z / (1 + exp(-z)). */
double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* Contiguous rank block [lo, hi) of a dimension of size n split t ways. */
void orc_shard_range(int64_t n, int64_t t, int64_t r, int64_t *lo, int64_t *hi) {
  *lo = r * (n / t);
  *hi = (r + 1) * (n / t);
}

/* Dot product of two K-vectors, increasing k, fp64. */
static double dot(const double *a, const double *b, int64_t K) {
  double s = 0.0;
  for (int64_t k = 0; k < K; ++k) s += a[k] * b[k];
  return s;
}

/*
 * One rank's MLP share, lecture §4.1 ("MLP: column then row").
 *   gate/up are column-parallel (case 1 of §3.2): rank r owns output columns
 *   F_r of W_gate[D, F_X] and W_up[D, F_X], needs the replicated input, and
 *   computes h[i, f] = silu(g) * u locally for f in F_r.
 *   down is row-parallel (case 3 of §3.2): rank r owns rows F_r of
 *   W_down[F_X, D] and produces the unreduced partial p_r[I, D]{U_X}.
 *
 * Full (unsharded) weights are passed; the rank indexes its block itself.
 *   X   [I, D]
 *   Wg  [F, D]   (stores logical W_gate[D, F])
 *   Wu  [F, D]   (stores logical W_up[D, F])
 *   Wd  [D, F]   (stores logical W_down[F, D])
 *   H   [I, F/t] out: silu(x.Wg[:,f]) * (x.Wu[:,f]) for f in F_r
 *   P   [I, D]   out: sum over f in F_r of H[i,f] * W_down[f, n]
 * rows: optional list of nrows token rows to compute (NULL = all I rows);
 * H and P are then [nrows, ...], in list order.
 * With t = 1, r = 0 this is the unsharded layer.
 */
void orc_mlp_rank(int64_t I, int64_t D, int64_t F, int64_t t, int64_t r,
                  const double *X, const double *Wg, const double *Wu,
                  const double *Wd, double *H, double *P,
                  const int64_t *rows, int64_t nrows) {
  int64_t f0, f1;
  orc_shard_range(F, t, r, &f0, &f1);
  const int64_t Fl = f1 - f0;
  const int64_t n_out = rows ? nrows : I;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t q = 0; q < n_out; ++q)
    for (int64_t f = f0; f < f1; ++f) {
      const int64_t i = rows ? rows[q] : q;
      const double g = dot(X + i * D, Wg + f * D, D);
      const double u = dot(X + i * D, Wu + f * D, D);
      H[q * Fl + (f - f0)] = orc_silu(g) * u;
    }
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t q = 0; q < n_out; ++q)
    for (int64_t n = 0; n < D; ++n) {
      double s = 0.0;
      for (int64_t f = f0; f < f1; ++f) s += H[q * Fl + (f - f0)] * Wd[n * F + f];
      P[q * D + n] = s;
    }
}

/*
 * Nearest bfloat16 value of x, ties to even (the storage rounding of every
 * bf16 intermediate on the device: H, the QKV output, the attention output,
 * a bf16 reduce output).  bfloat16 keeps 8 significant bits (1 implicit +
 * 7 stored) and the float32 exponent range, so near x, with x = m 2^e and
 * 1/2 <= |m| < 1, the representable values are the multiples of 2^(e-8);
 * below the smallest normal (2^-126) the spacing stays at 2^-133.  nearbyint
 * in the default rounding mode rounds half to even.  Zero, infinities and NaN
 * pass through.  Results past the largest bf16 (about 3.39e38) are not
 * clamped to infinity: no value of this layer comes near it.
 */
double orc_bf16_round(double x) {
  if (x == 0.0 || isnan(x) || isinf(x)) return x;
  int e;
  frexp(x, &e);
  int q = e - 8;
  if (q < -133) q = -133;
  return ldexp(nearbyint(ldexp(x, -q)), q);
}

void orc_bf16_round_array(int64_t n, const double *in, double *out) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) out[j] = orc_bf16_round(in[j]);
}

/*
 * orc_mlp_rank with the device's storage of H made explicit (the diagnostic
 * reading of the oracle): the same H and P as orc_mlp_rank, and also
 *   Hb[i, f] = bf16(H[i, f])                       (H as the bf16 path stores it)
 *   Pb[i, n] = sum over f in F_r of Hb[i, f] W_down[f, n]
 * so that a bf16 device result can be compared with what its arithmetic
 * would give with exact fp64 sums: Pb differs from a correct device P by
 * fp32 accumulation error only.  The plain P is accumulated exactly as in
 * orc_mlp_rank.  Arguments as orc_mlp_rank; Hb and Pb have the shapes of H
 * and P.
 */
void orc_mlp_rank_bf16h(int64_t I, int64_t D, int64_t F, int64_t t, int64_t r,
                        const double *X, const double *Wg, const double *Wu,
                        const double *Wd, double *H, double *P, double *Hb, double *Pb,
                        const int64_t *rows, int64_t nrows) {
  int64_t f0, f1;
  orc_shard_range(F, t, r, &f0, &f1);
  const int64_t Fl = f1 - f0;
  const int64_t n_out = rows ? nrows : I;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t q = 0; q < n_out; ++q)
    for (int64_t f = f0; f < f1; ++f) {
      const int64_t i = rows ? rows[q] : q;
      const double g = dot(X + i * D, Wg + f * D, D);
      const double u = dot(X + i * D, Wu + f * D, D);
      H[q * Fl + (f - f0)] = orc_silu(g) * u;
      Hb[q * Fl + (f - f0)] = orc_bf16_round(H[q * Fl + (f - f0)]);
    }
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t q = 0; q < n_out; ++q)
    for (int64_t n = 0; n < D; ++n) {
      double s = 0.0, sb = 0.0;
      for (int64_t f = f0; f < f1; ++f) {
        s += H[q * Fl + (f - f0)] * Wd[n * F + f];
        sb += Hb[q * Fl + (f - f0)] * Wd[n * F + f];
      }
      P[q * D + n] = s;
      Pb[q * D + n] = sb;
    }
}

/*
 * Sum of the t rank partials in rank order 0..t-1: what the all-reduce after
 * a row-parallel block delivers (lecture §3.3: all-reduce sums the partials;
 * §4.3: the sharded result equals the single-device one up to the order of
 * that sum).  partials [t, n] -> Y [n].
 */
void orc_reduce(int64_t t, int64_t n, const double *partials, double *Y) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < n; ++j) {
    double s = 0.0;
    for (int64_t r = 0; r < t; ++r) s += partials[r * n + j];
    Y[j] = s;
  }
}

/*
 * Column-parallel QKV projection split by heads, lecture §4.2: rank r owns
 * query heads [r*nq/t, (r+1)*nq/t) and KV groups [r*nkv/t, (r+1)*nkv/t)
 * (lecture §4.4: KV follows the heads while t <= number of groups).
 *   X   [I, D]
 *   Wq  [nq*hd, D], Wk [nkv*hd, D], Wv [nkv*hd, D]   (output-major)
 *   out [I, (nq/t + 2*nkv/t)*hd], columns laid out [q heads | k heads | v heads]
 */
void orc_qkv_rank(int64_t I, int64_t D, int64_t nq, int64_t nkv, int64_t hd,
                  int64_t t, int64_t r, const double *X, const double *Wq,
                  const double *Wk, const double *Wv, double *out) {
  int64_t q0, q1, g0, g1;
  orc_shard_range(nq, t, r, &q0, &q1);
  orc_shard_range(nkv, t, r, &g0, &g1);
  const int64_t nql = q1 - q0, nkl = g1 - g0;
  const int64_t Nq = nql * hd, Nk = nkl * hd, N = Nq + 2 * Nk;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < I; ++i)
    for (int64_t c = 0; c < N; ++c) {
      const double *w;
      if (c < Nq)
        w = Wq + (q0 * hd + c) * D;
      else if (c < Nq + Nk)
        w = Wk + (g0 * hd + (c - Nq)) * D;
      else
        w = Wv + (g0 * hd + (c - Nq - Nk)) * D;
      out[i * N + c] = dot(X + i * D, w, D);
    }
}

/*
 * Attention core of one rank (lecture §4.2: each device computes its own
 * heads' attention completely).  Not on the projection hot path; it joins
 * QKV to o_proj.  The pages do not fix its details; taken here: scaled dot
 * product with scale 1/sqrt(hd), causal mask inside each sequence, no
 * rotary embedding, grouped-query map: local head j reads local KV group
 * floor(j * nkv_l / nq_l).  Tokens form I/S sequences of S consecutive rows.
 *   qkv [I, (nq_l + 2*nkv_l)*hd] as produced by orc_qkv_rank
 *   A   [I, nq_l*hd]
 */
void orc_attn_core(int64_t I, int64_t S, int64_t nql, int64_t nkl, int64_t hd,
                   const double *qkv, double *A) {
  const int64_t N = (nql + 2 * nkl) * hd;
  const double scale = 1.0 / sqrt((double)hd);
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < I; ++i)
    for (int64_t j = 0; j < nql; ++j) {
      const int64_t g = (j * nkl) / nql;
      const int64_t s0 = (i / S) * S; /* first token of i's sequence */
      const double *q = qkv + i * N + j * hd;
      /* scores over the causal window s0..i, softmax with the max taken
       * out first, then the probability-weighted sum of the values */
      const int64_t L = i - s0 + 1;
      double *w = (double *)malloc((size_t)L * sizeof(double));
      double m = -INFINITY;
      for (int64_t p = s0; p <= i; ++p) {
        w[p - s0] = dot(q, qkv + p * N + nql * hd + g * hd, hd) * scale;
        if (w[p - s0] > m) m = w[p - s0];
      }
      double den = 0.0;
      for (int64_t p = 0; p < L; ++p) {
        w[p] = exp(w[p] - m);
        den += w[p];
      }
      for (int64_t c = 0; c < hd; ++c) {
        double acc = 0.0;
        for (int64_t p = s0; p <= i; ++p)
          acc += (w[p - s0] / den) * qkv[p * N + (nql + nkl) * hd + g * hd + c];
        A[i * (nql * hd) + j * hd + c] = acc;
      }
      free(w);
    }
}

/*
 * Row-parallel output projection, lecture §4.2: W_o is split by rows (its
 * input dimension, the concatenated heads), so rank r multiplies its own
 * heads' attention output by its row block of W_o and gets a partial
 * p_r[I, D]{U_X}.
 *   A_r [I, (nq/t)*hd]  this rank's attention output
 *   Wo  [D, nq*hd]      output-major full weight (stores logical W_o[nq*hd, D])
 *   P   [I, D]
 */
void orc_oproj_rank(int64_t I, int64_t D, int64_t nq, int64_t hd, int64_t t,
                    int64_t r, const double *A_r, const double *Wo, double *P) {
  int64_t q0, q1;
  orc_shard_range(nq, t, r, &q0, &q1);
  const int64_t Kl = (q1 - q0) * hd, K = nq * hd, c0 = q0 * hd;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < I; ++i)
    for (int64_t n = 0; n < D; ++n) {
      double s = 0.0;
      for (int64_t c = 0; c < Kl; ++c) s += A_r[i * Kl + c] * Wo[n * K + c0 + c];
      P[i * D + n] = s;
    }
}

/*
 * Residual add and RMSNorm around a row-parallel block.  The lecture (§4.2)
 * has the RMSNorm scale replicated on every rank, each rank normalising the
 * full hidden row itself; after the block's all-reduce the residual stream
 * is updated.  The pages name RMSNorm without defining it; the standard
 * definition (root mean square over the hidden dimension, plus eps, scaled
 * elementwise by gamma) is used:
 *   h[i, j] = residual[i, j] + sum_{r<t} partials[r, i, j]   (r in order)
 *   x[i, j] = h[i, j] / sqrt(mean_k h[i, k]^2 + eps) * gamma[j]
 *   partials [t, I, D] (t may be 0), residual [I, D] or NULL (zero),
 *   gamma [D] and x [I, D] both NULL: h only.
 */
void orc_residual_rmsnorm(int64_t t, int64_t I, int64_t D, const double *partials,
                          const double *residual, const double *gamma, double eps,
                          double *h, double *x) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < I; ++i) {
    double ss = 0.0;
    for (int64_t j = 0; j < D; ++j) {
      double v = residual ? residual[i * D + j] : 0.0;
      for (int64_t r = 0; r < t; ++r) v += partials[(r * I + i) * D + j];
      h[i * D + j] = v;
      ss += v * v;
    }
    if (!gamma || !x) continue;
    const double inv = 1.0 / sqrt(ss / (double)D + eps);
    for (int64_t j = 0; j < D; ++j) x[i * D + j] = h[i * D + j] * inv * gamma[j];
  }
}

/*
 * Weight-only FP8 storage for decode (the pages' cost frontier points are
 * FP8; they give no storage convention, so the reading here is): each
 * weight is one byte in the OCP E4M3 "fn" encoding -- sign bit, 4 exponent
 * bits with bias 7, 3 mantissa bits; exponent 0 holds subnormals m/8 * 2^-6;
 * all-ones exponent and mantissa is NaN; no infinities -- and every output
 * row n carries one scale s[n]: W[n, k] = s[n] * e4m3(code[n, k]).
 */
double orc_e4m3(unsigned char code) {
  const int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -v : v;
}

/* W[n, k] = scales[n] * e4m3(codes[n, k]) for n < N rows of K bytes. */
void orc_dequant_fp8(int64_t N, int64_t K, const unsigned char *codes, const double *scales,
                     double *W) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) W[n * K + k] = scales[n] * orc_e4m3(codes[n * K + k]);
}

/*
 * Weight-only int8 storage for decode (the PaLM int8-weight figures of
 * lecture §5.5; the pages give no convention, the reading here is): each
 * weight is one signed byte and every output row n carries one scale s[n]:
 * W[n, k] = s[n] * code[n, k], codes in [-128, 127].
 */
void orc_dequant_int8(int64_t N, int64_t K, const signed char *codes, const double *scales,
                      double *W) {
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) W[n * K + k] = scales[n] * (double)codes[n * K + k];
}

/*
 * Decode attention of one rank over its KV cache, lecture §4.4: the cache is
 * split with the heads, each rank storing and reading only the KV groups of
 * its own query heads (a group is stored on every rank that needs it once
 * the ranks outnumber the groups).  Sequence b has lens[b] positions: 0 ..
 * lens[b]-2 are in the cache, lens[b]-1 is the new token, whose k and v come
 * from the QKV projection's output.  Local head j reads local group
 * floor(j nkv / nq); scores are scaled by 1/sqrt(hd), softmax over all
 * lens[b] positions (no mask: every position is in the past).
 *   qkv  [B, (nq + 2 nkv) hd]   columns [q heads | k heads | v heads]
 *   Kc   [B, nkv, Lmax, hd], Vc [B, nkv, Lmax, hd]
 *   A    [B, nq hd]
 */
void orc_attn_decode(int64_t B, int64_t nq, int64_t nkv, int64_t hd, int64_t Lmax,
                     const int *lens, const double *qkv, const double *Kc, const double *Vc,
                     double *A) {
  const int64_t N = (nq + 2 * nkv) * hd;
  const double scale = 1.0 / sqrt((double)hd);
#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t j = 0; j < nq; ++j) {
      const int64_t g = (j * nkv) / nq, L = lens[b];
      const double *q = qkv + b * N + j * hd;
      double *w = malloc(sizeof(double) * (size_t)L);
      double m = -INFINITY;
      for (int64_t p = 0; p < L; ++p) {
        const double *k = (p == L - 1) ? qkv + b * N + (nq + g) * hd
                                       : Kc + ((b * nkv + g) * Lmax + p) * hd;
        w[p] = dot(q, k, hd) * scale;
        if (w[p] > m) m = w[p];
      }
      double den = 0.0;
      for (int64_t p = 0; p < L; ++p) {
        w[p] = exp(w[p] - m);
        den += w[p];
      }
      for (int64_t c = 0; c < hd; ++c) {
        double acc = 0.0;
        for (int64_t p = 0; p < L; ++p) {
          const double *v = (p == L - 1) ? qkv + b * N + (nq + nkv + g) * hd
                                         : Vc + ((b * nkv + g) * Lmax + p) * hd;
          acc += (w[p] / den) * v[c];
        }
        A[b * (nq * hd) + j * hd + c] = acc;
      }
      free(w);
    }
}
