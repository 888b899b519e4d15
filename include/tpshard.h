/*
 * tpshard.h -- C ABI of one tensor-parallel rank's share of a Megatron-style
 * transformer layer, for AMD Instinct MI355X (gfx950).
 *
 * Sources of the method (the pages this library follows):
 *   [L4]  "Lecture 4 - Distributed Serving" (semidirectx.com, cs349e notes):
 *         §3.1 sharding notation A[I_X, J]; §3.2 the four sharded-matmul
 *         cases, case 1 (contracting dim unsplit: local, no communication)
 *         and case 3 (contracting dim split the same way on both operands:
 *         local partial sum C[I, K]{U_X}, then all-reduce); §4.1 the MLP
 *         split column-then-row; §4.2 attention split by heads, W_o by rows.
 *   [V]   "vLLM model parallelism" article (intelliparadigm.com), §2.1: a
 *         column-parallel layer keeps its weight as
 *         [output_size_per_partition, input_size].
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers unless said otherwise; every buffer is
 *     owned by the caller (e.g. torch tensors).  The library allocates no
 *     device memory and keeps no state: calls are reentrant.
 *   - Every call enqueues its kernels on `stream` (a hipStream_t; NULL is
 *     the null stream) and returns without synchronising.  A device fault
 *     surfaces at the caller's next synchronisation.
 *   - Row-major layouts.  Weights are output-major: each output channel's
 *     K-vector is contiguous ([V] §2.1), so a logical W[K, N] is stored as
 *     Ws[N][K].
 *   - dt selects the element type of X, weights, H and bf16/f32 outputs:
 *     TP_BF16 (inputs bf16, fp32 accumulation, bf16 outputs rounded to
 *     nearest-even) or TP_F32 (fp32 throughout).  Partials P are always fp32.
 *   - Alignment: every pointer 16-byte aligned; every contraction length and
 *     every row length a multiple of 8 elements.
 *   - I == 0 is a no-op returning TP_OK.  Every other size must be >= 1.
 *   - On any error status nothing is launched and no output is touched.
 *   - Outputs must not overlap inputs or each other.
 */
#ifndef TPSHARD_H
#define TPSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { TP_F32 = 0, TP_BF16 = 1 } tp_dtype_t;

typedef enum {
  TP_OK = 0,
  TP_ERR_INVALID = 1,     /* null pointer, size < 1, t does not divide, bad enum, overlap */
  TP_ERR_MISALIGNED = 2,  /* pointer not 16-byte aligned, or a length not a multiple of 8 */
  TP_ERR_UNSUPPORTED = 3, /* valid request outside the sizes this build handles */
  TP_ERR_LAUNCH = 4,      /* the HIP runtime reported an error when enqueuing */
  TP_ERR_WORKSPACE = 5    /* workspace smaller than the *_workspace_size query */
} tp_status_t;

typedef enum { TP_ATTN_QKV = 0, TP_ATTN_O = 1 } tp_attn_phase_t;

/* Version of this ABI (bumped on any signature change). */
int tp_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* tp_status_string(tp_status_t s);

/*
 * Device workspace, in bytes, that tp_shard_mlp needs for these sizes
 * (0 if none: calls that do not split K over workgroups need none).  Host-only; never
 * touches the GPU.  Returns 0 for invalid sizes (the call itself then reports
 * the error).
 */
size_t tp_shard_mlp_workspace_size(int64_t I, int64_t D, int64_t F_local, tp_dtype_t dt);

/*
 * One rank's share of the SwiGLU MLP, [L4] §4.1, with F split t ways
 * (F_local = F / t):
 *
 *   H[I, F_X]     = silu(X . W_gate[D, F_X]) * (X . W_up[D, F_X])
 *                   column-parallel: case 1 of [L4] §3.2, no communication;
 *                   silu(z) = z / (1 + exp(-z)), the product elementwise.
 *   P[I, D]{U_X}  = H[I, F_X] . W_down[F_X, D]
 *                   row-parallel: case 3 of [L4] §3.2, an UNREDUCED partial;
 *                   the t ranks' P summed (the all-reduce) give the layer's
 *                   MLP output.
 *
 *   X       [I, D]        dt, the replicated layer input
 *   W_gate  [F_local, D]  dt, stores logical W_gate[D, F_X] (K = D contiguous)
 *   W_up    [F_local, D]  dt
 *   W_down  [D, F_local]  dt, stores logical W_down[F_X, D] (K = F_local contiguous)
 *   H       [I, F_local]  dt, written: the SwiGLU activations (bf16 rounded
 *                         to nearest-even on the bf16 path)
 *   P       [I, D]        fp32, overwritten (never accumulated into)
 *   workspace, workspace_bytes: device scratch of at least
 *           tp_shard_mlp_workspace_size(...) bytes, 16-byte aligned, not
 *           overlapping any other argument (may be NULL when the size is 0).
 *           bf16 calls that split K over workgroups (from 5 tokens, by
 *           shape: wherever the tiles alone leave CUs idle, prefill shapes
 *           included) keep arrival counters and fp32 partial sums there.
 *           The first 8 KiB (the counters) must be zero before the workspace's
 *           first use (tp_workspace_reset, once after allocating it); every
 *           completed call leaves them zero again, so one workspace serves
 *           any sequence of calls on one stream.  Counters left non-zero (a
 *           workspace never reset, or a call that did not complete) make
 *           later calls produce wrong output without an error: reset then.
 *           The rest is scratch: contents on entry ignored, on return
 *           undefined.  Two calls in flight at once (other streams) need
 *           separate workspaces.
 * Errors: TP_ERR_INVALID, TP_ERR_MISALIGNED (D or F_local not a multiple of 8,
 * a pointer not 16-byte aligned), TP_ERR_UNSUPPORTED (fp32 with D or F_local
 * above the few-token kernel's K range; a projection that falls on the MFMA
 * GEMM with a contraction length above 2^22), TP_ERR_WORKSPACE,
 * TP_ERR_LAUNCH.
 */
tp_status_t tp_shard_mlp(int64_t I, int64_t D, int64_t F_local, tp_dtype_t dt,
                         const void* X, const void* W_gate, const void* W_up,
                         const void* W_down, void* H, float* P,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * tp_shard_mlp with weight-only FP8 storage, for any token count.  The
 * pages' cost frontier is FP8 throughout but they give no storage convention;
 * the one used here: every weight is one byte in the OCP E4M3 ("fn") encoding
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, 0x7F and
 * 0xFF NaN, no infinities) and every output row n of a matrix carries one
 * fp32 scale, W[n, k] = s[n] * e4m3(code[n, k]).  Activations stay bf16:
 *
 *   H[I, F_X]    = silu(X . W_gate[D, F_X]) * (X . W_up[D, F_X])   (bf16)
 *   P[I, D]{U_X} = H[I, F_X] . W_down[F_X, D]                      (fp32)
 *
 *   X       [I, D]        bf16
 *   W_gate  [F_local, D]  E4M3 codes, s_gate [F_local] fp32
 *   W_up    [F_local, D]  E4M3 codes, s_up   [F_local] fp32
 *   W_down  [D, F_local]  E4M3 codes, s_down [D] fp32 (scales per output row)
 *   H       [I, F_local]  bf16 written; P [I, D] fp32 overwritten
 *   workspace as tp_shard_mlp: tp_shard_mlp_fp8_workspace_size bytes (0 for
 *           up to 4 tokens, and where the GEMM does not split K), counter
 *           area zero before first use, left zero
 * D and F_local multiples of 16.  Up to 4 tokens (D, F_local at most 16384)
 * the weights stream through VALU dot products; 5..64 tokens (or larger K)
 * through the split-K MFMA kernel; more tokens through the one-byte MFMA
 * GEMM (TP_ERR_UNSUPPORTED there for D or F_local above 2^22).  Scales
 * 4-byte aligned, every other pointer 16-byte aligned.
 * Errors: TP_ERR_INVALID, TP_ERR_MISALIGNED, TP_ERR_UNSUPPORTED,
 * TP_ERR_WORKSPACE, TP_ERR_LAUNCH.
 */
size_t tp_shard_mlp_fp8_workspace_size(int64_t I, int64_t D, int64_t F_local);
tp_status_t tp_shard_mlp_fp8(int64_t I, int64_t D, int64_t F_local, const void* X,
                             const void* W_gate, const float* s_gate, const void* W_up,
                             const float* s_up, const void* W_down, const float* s_down,
                             void* H, float* P, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * tp_shard_mlp for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and kernels, with the split-K scratch taken from an array
 * the library holds in device memory instead of a caller workspace.  The
 * array, tp_shard_mlp_noalloc_max_workspace() bytes (32 MiB), is part of the
 * library's code object, so each GPU the library runs on holds its own copy
 * until the process ends; the call allocates nothing.  Every call clears the
 * array's counter area (a small fill kernel on `stream`) before its kernels.
 * All calls on one GPU share that GPU's array: calls that may overlap on one
 * GPU (other streams, other threads) race and give wrong results -- keep
 * them on one stream, or use tp_shard_mlp with a workspace each.
 * Arguments and results as tp_shard_mlp, without the workspace.
 * Errors as tp_shard_mlp; TP_ERR_WORKSPACE when the call needs more scratch
 * than the array holds (tp_shard_mlp_workspace_size(...) above the maximum),
 * TP_ERR_LAUNCH also when the array's device address cannot be looked up.
 */
size_t tp_shard_mlp_noalloc_max_workspace(void);
tp_status_t tp_shard_mlp_noalloc(int64_t I, int64_t D, int64_t F_local, tp_dtype_t dt,
                                 const void* X, const void* W_gate, const void* W_up,
                                 const void* W_down, void* H, float* P, void* stream);

/* Workspace bytes tp_shard_attn_proj needs (0 if none); host-only. */
size_t tp_shard_attn_proj_workspace_size(tp_attn_phase_t phase, int64_t I, int64_t D,
                                         int64_t n_q_local, int64_t n_kv_local,
                                         int64_t head_dim, tp_dtype_t dt);

/*
 * Attention projections of one rank, split by heads, [L4] §4.2.  The rank
 * holds n_q_local query heads and n_kv_local KV groups of head_dim each.
 *
 * phase TP_ATTN_QKV (column-parallel, [L4] §3.2 case 1):
 *   out[I, N_qkv] = X[I, D] . W_qkv[D, N_qkv],  N_qkv = (n_q_local + 2 n_kv_local) head_dim
 *   in   X      [I, D]      dt
 *   W           [N_qkv, D]  dt; rows are this rank's q heads, then its k
 *                           heads, then its v heads (each head head_dim rows)
 *   out         [I, N_qkv]  dt, same column order
 * phase TP_ATTN_O (row-parallel, [L4] §3.2 case 3):
 *   out[I, D]{U_X} = A[I, K_o] . W_o[K_o, D],  K_o = n_q_local head_dim
 *   in   A      [I, K_o]    dt, this rank's attention output (its heads)
 *   W           [D, K_o]    dt, stores the rank's row block of logical W_o
 *   out         [I, D]      fp32 partial, overwritten
 * n_kv_local is ignored for TP_ATTN_O (pass any value >= 1).
 * Errors as tp_shard_mlp; head_dim must be a multiple of 8.
 */
tp_status_t tp_shard_attn_proj(tp_attn_phase_t phase, int64_t I, int64_t D,
                               int64_t n_q_local, int64_t n_kv_local, int64_t head_dim,
                               tp_dtype_t dt, const void* in, const void* W, void* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sum of t rank partials in rank order 0..t-1, in fp32: the value the
 * all-reduce after a row-parallel block delivers ([L4] §3.3; §4.3 notes the
 * sharded layer equals the single-device one up to this summation order).
 * It stands in for the collective when all t ranks run on one device.
 *   partials [t, n] fp32 (rank r's partial at partials + r*n)
 *   Y        [n]    out_dt: fp32, or bf16 rounded to nearest-even
 * n counts elements (I*D for a layer output) and must be a multiple of 8.
 */
tp_status_t tp_partial_reduce(int32_t t, int64_t n, const float* partials,
                              tp_dtype_t out_dt, void* Y, void* stream);

/*
 * tp_shard_mlp_fp8 with int8 codes: weight-only int8 storage for decode, the
 * variant behind the pages' PaLM int8-weight figures ([L4] §5.5).  Every
 * weight is one signed byte c in [-128, 127] and every output row n of a
 * matrix carries one fp32 scale, W[n, k] = s[n] * c[n, k].  Activations, H
 * and P keep the dtypes of the bf16 path; the int8 values are exact in bf16,
 * so the products are those of the dequantized weights.  Arguments, shapes,
 * alignment, workspace, supported sizes and errors as tp_shard_mlp_fp8,
 * with W_gate, W_up, W_down holding int8 codes.
 */
size_t tp_shard_mlp_int8_workspace_size(int64_t I, int64_t D, int64_t F_local);
tp_status_t tp_shard_mlp_int8(int64_t I, int64_t D, int64_t F_local, const void* X,
                              const void* W_gate, const float* s_gate, const void* W_up,
                              const float* s_up, const void* W_down, const float* s_down,
                              void* H, float* P, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * The step after a row-parallel block's all-reduce, fused into one pass over
 * each hidden row: the residual update and the replicated RMSNorm in front of
 * the next column-parallel projection ([L4] §4.2: the RMSNorm scale is
 * replicated and every rank normalises the full row itself).  The pages name
 * RMSNorm without defining it; the standard definition is used:
 *   h[i, :] = residual[i, :] + sum_{r<t} partials[r, i, :]    fp32, r in order
 *   x[i, :] = h[i, :] / sqrt(mean_j h[i, j]^2 + eps) * gamma  from h as stored
 *   partials [t, I, D] fp32, t >= 0 (may be NULL when t == 0)
 *   residual [I, D] h_dt, or NULL (zero; then t >= 1)
 *   h        [I, D] h_dt out (fp32, or bf16 rounded to nearest-even); may be
 *            the residual pointer itself (in-place update), no other overlap
 *   gamma    [D] x_dt and x [I, D] x_dt out: both NULL to compute h only
 *   eps      >= 0, finite
 * D a multiple of 8 and at most 32768.  With t partials of the o_proj (or
 * MLP) block this is what every rank does right after the block's all-reduce.
 * Errors: TP_ERR_INVALID, TP_ERR_MISALIGNED, TP_ERR_UNSUPPORTED, TP_ERR_LAUNCH.
 */
tp_status_t tp_residual_rmsnorm(int32_t t, int64_t I, int64_t D, const float* partials,
                                const void* residual, tp_dtype_t h_dt, void* h,
                                const void* gamma, tp_dtype_t x_dt, void* x, float eps,
                                void* stream);

/*
 * The sequence-parallel form of tp_residual_rmsnorm ([L4] §4.5): the
 * all-reduce after a row-parallel block becomes a reduce-scatter -- rank
 * `rank` of t receives the sum of the t partials for its own I/t token rows
 * -- followed by the residual update and RMSNorm on those rows only, and an
 * all-gather of x before the next column-parallel projection.  This call is
 * rank `rank`'s reduce-scatter plus norm, with the t partials all on this
 * device:
 *   rows     i in [rank*I/t, (rank+1)*I/t)  (t must divide I)
 *   partials [t, I, D] fp32, the full partials of every rank
 *   residual [I/t, D] h_dt, this rank's rows of the residual stream, or NULL
 *   h        [I/t, D] h_dt out; may be the residual pointer itself
 *   gamma    [D] x_dt, x [I/t, D] x_dt out (both NULL: h only); point x at
 *            row rank*I/t of a full [I, D] buffer and, over all ranks, the
 *            buffer holds the all-gathered x
 * Same values as tp_residual_rmsnorm on those rows.  D a multiple of 8, at
 * most 32768.  Errors as tp_residual_rmsnorm.
 */
tp_status_t tp_reduce_scatter_rmsnorm(int32_t t, int32_t rank, int64_t I, int64_t D,
                                      const float* partials, const void* residual,
                                      tp_dtype_t h_dt, void* h, const void* gamma,
                                      tp_dtype_t x_dt, void* x, float eps, void* stream);

/*
 * Decode attention of one rank over its KV cache ([L4] §4.4: the cache is
 * split with the heads -- a rank stores and reads only the KV groups of its
 * own query heads; once the ranks outnumber the groups, a group is stored on
 * every rank whose heads use it).  For each of B sequences the new token
 * attends to lens[b] positions: 0 .. lens[b]-2 from the cache, lens[b]-1 the
 * new token itself, whose k and v are taken from qkv.  The call also stores
 * that k and v into cache slot lens[b]-1, ready for the next step.  Local
 * head j uses local group floor(j n_kv_local / n_q_local); scale
 * 1/sqrt(head_dim); softmax over all lens[b] positions.
 *   lens      [B] int32 device array, each in [1, L_max] (clamped to it)
 *   qkv       [B, (n_q_local + 2 n_kv_local) head_dim] bf16, as TP_ATTN_QKV
 *             writes it for the new tokens
 *   K_cache   [B, n_kv_local, L_max, head_dim] bf16: row p holds position
 *             p's k; read, and row lens[b]-1 written
 *   V_cache   [B, n_kv_local, head_dim, L_max] bf16, transposed: column p
 *             holds position p's v; read, and column lens[b]-1 written
 *   A         [B, n_q_local head_dim] bf16 out
 *   workspace as tp_shard_mlp (tp_attn_decode_workspace_size bytes, counter
 *             area zero before first use, left zero)
 * head_dim and L_max multiples of 8 (TP_ERR_MISALIGNED otherwise), head_dim
 * at most 128; n_kv_local divides n_q_local, at most 32 heads per group; each
 * cache below 2 GiB.
 * Errors: TP_ERR_INVALID, TP_ERR_MISALIGNED, TP_ERR_UNSUPPORTED,
 * TP_ERR_WORKSPACE, TP_ERR_LAUNCH.
 */
size_t tp_attn_decode_workspace_size(int64_t B, int64_t n_q_local, int64_t n_kv_local,
                                     int64_t head_dim, int64_t L_max);
tp_status_t tp_attn_decode(int64_t B, int64_t n_q_local, int64_t n_kv_local, int64_t head_dim,
                           int64_t L_max, const int32_t* lens, const void* qkv, void* K_cache,
                           void* V_cache, void* A, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Attention core of one rank (test support, not a projection): each rank
 * computes its own heads' attention completely ([L4] §4.2).  Scaled dot
 * product (scale 1/sqrt(head_dim)), causal inside each sequence, no rotary
 * embedding; local head j reads local KV group floor(j n_kv_local / n_q_local).
 * Tokens form I/S sequences of S consecutive rows.
 *   qkv [I, (n_q_local + 2 n_kv_local) head_dim] bf16, as TP_ATTN_QKV writes it
 *   A   [I, n_q_local head_dim] bf16 out
 * bf16 only; head_dim a multiple of 8 and at most 256; S must divide I;
 * qkv at most 2 GiB (TP_ERR_UNSUPPORTED beyond).
 */
tp_status_t tp_attn_core(int64_t I, int64_t S, int64_t n_q_local, int64_t n_kv_local,
                         int64_t head_dim, const void* qkv, void* A, void* stream);

/*
 * Prepare a workspace for the calls above that take one: enqueue on `stream`
 * a fill kernel that zeroes its leading counter area (the first
 * min(workspace_bytes, 8 KiB) bytes; the rest is scratch and left alone).
 * Split sums keep one 32-bit arrival counter per output block there; every
 * completed call leaves them zero again, so one reset after allocating a
 * workspace serves any sequence of calls on one stream.  Reset again after a
 * call that did not run to completion, or when handing a workspace that was
 * used for anything else to these calls.  It is a kernel, not a memset, so it
 * may be recorded into a HIP graph.
 * Errors: TP_ERR_INVALID (NULL, zero bytes), TP_ERR_MISALIGNED (not 16-byte
 * aligned), TP_ERR_LAUNCH.
 */
tp_status_t tp_workspace_reset(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Measurement aid (not a step of the layer): the achievable read rate.
 * Decode is bound by reading the rank's weights once ([L4] §1.1, §3.4);
 * this reads `bytes` of device memory once with the same access pattern as
 * the decode kernels' weight streams (1 KB contiguous per wave load, three
 * loads in flight per wave, one 16-wave workgroup per CU), so bytes / time
 * is the ceiling those kernels are compared with.
 *   buf   device buffer of `bytes` bytes (a multiple of 1024, at most 2 GiB)
 *   sink  tp_stream_read_sink_words() uint32 words out: word i is the XOR,
 *         over the 16-byte chunks thread i read, of each chunk's first and
 *         last 32-bit words (so the XOR of all of sink is that of the buffer)
 * Errors: TP_ERR_INVALID (null pointer, bytes 0 or over 2 GiB, sink too
 * small, no device), TP_ERR_MISALIGNED (bytes not a multiple of 1024, or a
 * pointer not 16-byte aligned), TP_ERR_LAUNCH.
 */
size_t tp_stream_read_sink_words(void);
tp_status_t tp_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                           void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TPSHARD_H */
