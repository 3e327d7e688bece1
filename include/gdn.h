/*
 * gdn.h -- C ABI of libgdn: the chunk-wise Gated DeltaNet intra-chunk solve on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages the operations follow (cited by title):
 *   [GEO]  "When Good Enough Is Optimal: Multiplication-Only Matrix Inversion
 *           Approximation for Quantized Gated DeltaNet" (technical summary):
 *           problem statement (per-chunk T = (I - A)^-1 with A strictly lower),
 *           Methodologie SS1 (truncated low-order Neumann sum, Lemma 3.1),
 *           SS2 (structural diagonal mask), SS3 (parallel residual correction),
 *           "Adaptation a la Quantification" (low-bit ranges, N = 3).
 *   [PSDA] "A Persistent-State Dataflow Accelerator for Memory-Bound Linear
 *           Attention Decode on FPGA" (technical summary), section 2.B (the state
 *           read / delta correction / state write split of one recurrence step).
 *
 * Notation for one block (one chunk of one (batch, head)), positions r = 0..C-1:
 *   K [C][d_k], V [C][d_v], Q [C][d_k]; beta[C]; gamma[C] per-token log-gates (<= 0);
 *   G = cumulative sum of gamma restarted at every chunk start;
 *   A_ij = -beta_i (k_i . k_j) exp(G_i - G_j) for i > j, 0 otherwise   (strictly lower)
 *   T    = (I - A)^-1 (exact), or its truncated / masked approximation.
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers, row-major and contiguous, 16-byte
 *     aligned (else GDN_ERR_BAD_ALIGNMENT).  The caller allocates and frees them.
 *     Inputs are read-only; outputs are fully overwritten, never accumulated into.
 *     Inputs and outputs must not overlap.
 *   - Descriptor structs (gdn_blocks, gdn_inverse_cfg) are HOST pointers, read
 *     during the call only.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Work is
 *     enqueued on it and the call returns without synchronising.  Argument errors
 *     and launch errors are returned synchronously; device faults surface at the
 *     caller's next synchronisation.  No C++ exception crosses the ABI.
 *   - The library allocates nothing, keeps no per-call state and is reentrant.  Where
 *     a call needs device scratch memory (gdn_chunk_fwd for most inverse variants),
 *     the caller passes it in and a query states its size.
 *   - n_blocks == 0 (or B*H == 0, T == 0) is valid and enqueues nothing.
 *   - Supported chunk sizes C: 16, 32, 64 (all entry points); 128 and 256 for the
 *     inverse entry points and gdn_wy with bf16 keys and bf16 products (compute =
 *     GDN_BF16), d_k and d_v in {64, 128}.  d_k and d_v otherwise: multiples of 32,
 *     at most 256, as each entry point states.  Anything else: GDN_ERR_UNSUPPORTED.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 2

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL_POINTER = 1,  /* a required pointer is NULL                          */
  GDN_ERR_BAD_SHAPE = 2,     /* negative size, T % C != 0, N out of range, ...      */
  GDN_ERR_BAD_DTYPE = 3,     /* dtype code not accepted for that argument           */
  GDN_ERR_BAD_ALIGNMENT = 4, /* a tensor pointer is not 16-byte aligned             */
  GDN_ERR_UNSUPPORTED = 5,   /* valid request this build does not implement         */
  GDN_ERR_WORKSPACE = 6,     /* workspace missing or smaller than the query returned */
  GDN_ERR_HIP = 7            /* the HIP runtime reported an error at launch         */
} gdn_status;

/* element types (int32 codes in every signature) */
typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1, GDN_FP8_E4M3 = 2, GDN_INT8 = 3, GDN_INT16 = 4 } gdn_dtype;

/* inverse variants */
typedef enum gdn_inv_mode {
  GDN_INV_NEUMANN = 0, /* truncated sum_{n<=N} A^n ([GEO] Methodologie SS1), optional
                          band mask i - j <= N ([GEO] Methodologie SS2)                */
  GDN_INV_EXACT = 1,   /* prod_{i<m} (I + A^(2^i)), m = ceil(log2 C): exact because
                          A^C = 0 (Lemma 3.1 of [GEO])                                */
  GDN_INV_NEUMANN_PRODUCTS = 2 /* gdn_chunk_fwd only: the GDN_INV_NEUMANN sum, always
                          formed by its Horner products on MFMA (in the pre-pass), also
                          where the masked band with N <= 3 would otherwise be formed
                          element by element from A's sub-diagonals (identical in exact
                          arithmetic; the products round their operands to bf16)      */
} gdn_inv_mode;

/* How T is formed.  `compute` is the MFMA operand type of the power chain:
 *   GDN_F32  fp32 operands (16x16x4 f32 MFMA)
 *   GDN_BF16 bf16 operands, fp32 accumulation (16x16x32 bf16 MFMA)
 *   GDN_FP8_E4M3 OCP e4m3 operands with one absmax/448 scale per block and tensor,
 *            fp32 accumulation (16x16x32 fp8 MFMA); Neumann mode only.
 *   GDN_INT8 int8 codes with one power-of-two scale per block and operand (the
 *            smallest 2^e with max|x| <= 127 2^e), int32 accumulation (16x16x64 i8
 *            MFMA), Horner on X = H - I ([GEO] "Adaptation a la Quantification");
 *            gdn_tri_inverse_neumann only, C <= 64.
 *   GDN_INT16 the same chain on 16-bit codes, |code| <= 32639 = 127 * 257, the range
 *            whose balanced base-256 digits (code = 256 hi + lo, lo in [-128, 127]) both
 *            fit int8: each product is four 16x16x64 i8 MFMAs (hi hi, hi lo, lo hi, lo
 *            lo) recombined exactly in fp64, and each sum A' + P 2^e is formed in fp64
 *            and rounded to fp32; gdn_tri_inverse_neumann only, C <= 64.
 * N is ignored for GDN_INV_EXACT. */
typedef struct gdn_inverse_cfg {
  int32_t mode;    /* gdn_inv_mode                  */
  int32_t N;       /* truncation order, 1 <= N < C  */
  int32_t mask;    /* 0 / 1: apply M^(N)            */
  int32_t compute; /* gdn_dtype                     */
} gdn_inverse_cfg;

/* A batch of independent C x C blocks.  Either A is given (then K, beta, g are not
 * read), or A is built on the fly from K, beta and g.
 *   A     [n_blocks][C][C] fp32; only the strictly lower triangle is read.
 *   K     [n_blocks][C][d_k], k_dtype GDN_BF16 or GDN_F32 (for a [B][H][T][d_k]
 *         tensor with T % C == 0 this is the same memory with n_blocks = B*H*T/C).
 *   beta  [n_blocks][C] fp32.
 *   g     [n_blocks][C] fp32 per-token log-gates; if g_cumulative != 0 they are
 *         already the in-chunk cumulative sums G. */
typedef struct gdn_blocks {
  const float* A;
  const void* K;
  int32_t k_dtype;
  int32_t g_cumulative;
  const float* beta;
  const float* g;
  int64_t n_blocks;
  int32_t C;
  int32_t d_k;
} gdn_blocks;

/* fp8 diagnostics of the e4m3 power chain ([GEO] "Adaptation a la Quantification"),
 * a DEVICE struct accumulated by the fp8 paths.  The chain runs on X = H - I:
 * A' = s_A q(A), X_1 = A', X_{k+1} = A' + s_A s_X (q(A) q(X_k)), T = I + s_T q(X_N),
 * q() the e4m3 codes under the tensor's own absmax/448 scale.  Counted over every
 * quantised tensor of every block, once per block: A, the right operands X_1..X_{N-1}
 * and X_N (N >= 2).  x counts as
 *   nonfinite    not finite;
 *   sat_dynamic  |x| / s_Y >= 464 under its own scale s_Y (it would round beyond 448;
 *                0 by construction of an absmax scale, kept as a check);
 *   sat_static   |x| / s_A >= 464 under A's scale: had A's range been fixed for its
 *                powers and T, this value would overflow (the regime the mask is for);
 *   underflow    x != 0 and |x| / s_Y <= 2^-10 (rounds to the code 0).            */
typedef struct gdn_fp8_stats {
  unsigned long long nonfinite, sat_dynamic, sat_static, underflow;
} gdn_fp8_stats;
#define GDN_FP8_STATS_COUNT 4

int gdn_abi_version(void);
const char* gdn_status_string(int32_t status);

/* A = -tril(diag(beta) (K K^T .* exp(G_i - G_j)), -1) per block ([GEO] problem
 * statement: A strictly lower).  in->A must be NULL.  A_out [n_blocks][C][C] fp32,
 * upper triangle and diagonal written as exact zeros. */
gdn_status gdn_build_A(const gdn_blocks* in, float* A_out, void* stream);

/* T = M^(N) .* sum_{n=0}^{N} A^n (mask != 0) or the plain truncated sum (mask == 0),
 * evaluated as N-1 Horner products H <- I + A H ([GEO] Methodologie SS1-2).
 * compute: GDN_F32, GDN_BF16, GDN_FP8_E4M3, GDN_INT8 or GDN_INT16 (C <= 64).  With
 * GDN_INT8 or GDN_INT16 and a given fp32 A the result is exactly determined: every scaling is by a power of two,
 * integer products are exact and each intermediate sum is rounded once to fp32.
 * T_out [n_blocks][C][C], t_dtype GDN_F32
 * or GDN_BF16.  stats: device gdn_fp8_stats (see above) or NULL; when given it is
 * zeroed on `stream` and then accumulated (fp8 compute only; other computes write
 * zeros). */
gdn_status gdn_tri_inverse_neumann(const gdn_blocks* in, int32_t N, int32_t mask,
                                   int32_t compute, void* T_out, int32_t t_dtype,
                                   gdn_fp8_stats* stats, void* stream);

/* T = prod_{i=0}^{m-1} (I + A^(2^i)), m = ceil(log2 C): the exact inverse by
 * multiplications only.  compute GDN_F32 or GDN_BF16. */
gdn_status gdn_tri_inverse_exact(const gdn_blocks* in, int32_t compute, void* T_out,
                                 int32_t t_dtype, void* stream);

/* The truncated sum T(0) as in gdn_tri_inverse_neumann (N, mask) refined by the
 * parallel residual correction of [GEO] Methodologie SS3: E = I - (I - A) T(0), then
 * T = T(0) sum_{s=0}^{S} E^s, the sum of powers in Horner form (S products).  With the
 * mask, E vanishes on subdiagonals 0..N, so T is exact on subdiagonals below
 * (S+1)(N+1).  0 <= S <= 64 (GDN_ERR_BAD_SHAPE otherwise).  compute must be GDN_F32:
 * E is a small difference of O(1) terms, which bf16 operands would not resolve
 * (GDN_ERR_UNSUPPORTED otherwise).  C in {16, 32, 64}.  T_out as above. */
gdn_status gdn_tri_inverse_residual(const gdn_blocks* in, int32_t N, int32_t mask, int32_t S,
                                    int32_t compute, void* T_out, int32_t t_dtype, void* stream);

/* T = (I - A)^-1 by forward substitution, T = I + A T row by row ([GEO] problem
 * statement: the sequential baseline the multiplication-only inverses replace), in
 * fp32 with C (C-1)/2 dependent-row multiply-adds per block.  C in {16, 32, 64}, and
 * C = 128 with A given or bf16 keys (d_k 64 or 128); other C: GDN_ERR_UNSUPPORTED.
 * T_out [n_blocks][C][C], t_dtype GDN_F32 or GDN_BF16. */
gdn_status gdn_tri_inverse_fs(const gdn_blocks* in, void* T_out, int32_t t_dtype, void* stream);

/* WY products per block: W = T diag(s) K, U = T diag(beta) V with s = beta
 * (gate_k == 0) or s = beta .* exp(G) (gate_k != 0, the form the gated chunk
 * recurrence consumes).  T: if non-NULL, [n_blocks][C][C] of t_dtype (GDN_F32 or
 * GDN_BF16), used as given; if NULL, T is formed on the fly from in (K, beta, g;
 * in->A must be NULL) with `inv`.  V [n_blocks][C][d_v] bf16.  W_out
 * [n_blocks][C][d_k], U_out [n_blocks][C][d_v], out_dtype GDN_F32 or GDN_BF16. */
gdn_status gdn_wy(const gdn_blocks* in, const void* T, int32_t t_dtype,
                  const gdn_inverse_cfg* inv, const void* V, int32_t d_v, int32_t gate_k,
                  void* W_out, void* U_out, int32_t out_dtype, void* stream);

/* Device workspace, in bytes, that gdn_chunk_fwd needs for these arguments.  The
 * band-masked truncated sum with N <= 3 on bf16 operands forms T inside the scan and
 * needs none (0).  The same sum on fp8 operands (GDN_INV_NEUMANN) forms the band of
 * T - I of all B*H*T/C chunks in a pre-pass: 512 bytes per chunk at C = 64.  Every other
 * inverse variant (GDN_INV_NEUMANN_PRODUCTS included) forms T - I of all chunks in a
 * batched pre-pass of MFMA products: 6144 bytes per chunk at C = 64.  Returns 0 as well
 * for arguments gdn_chunk_fwd rejects (it then reports why).  No HIP call is made. */
size_t gdn_chunk_fwd_workspace_bytes(int32_t B, int32_t H, int64_t T, int32_t d_k, int32_t d_v,
                                     int32_t C, const gdn_inverse_cfg* inv);

/* Chunk-wise gated delta rule forward over whole sequences ([GEO] problem statement:
 * the chunk-wise form inverts I - A per chunk and carries a fixed-size state; [PSDA]
 * section 2.A: the state stays on chip).  Per (b, h), chunks in order, state S
 * [d_k][d_v] fp32 starting at S0 (zeros if NULL):
 *   T from A (inv); U' = T diag(beta) (V - diag(exp(G)) K S)   (= U - W S, W gated)
 *   O  = scale (diag(exp(G)) Q S + (Q K^T .* exp(G_i - G_j) .* [i >= j]) U')
 *   S <- exp(G_C) S + K^T diag(exp(G_C - G)) U'
 * Q, K [B][H][T][d_k] and V [B][H][T][d_v] in qkv_dtype (GDN_BF16); beta, g
 * [B][H][T] fp32 (g per-token log-gates); S0, S_out [B][H][d_k][d_v] fp32;
 * O [B][H][T][d_v] in o_dtype (GDN_BF16 or GDN_F32).  T % C == 0; C = 64.
 * workspace: device memory of at least gdn_chunk_fwd_workspace_bytes(...) bytes,
 * 16-byte aligned (GDN_ERR_WORKSPACE if it is needed and NULL or smaller; may be NULL
 * when none is needed).  Its contents are scratch: overwritten by the call and read
 * back by it on `stream`, so one workspace must not serve two calls in flight at
 * once.  stats as for gdn_tri_inverse_neumann (fp8 compute, each chunk counted once). */
gdn_status gdn_chunk_fwd(const void* Q, const void* K, const void* V, int32_t qkv_dtype,
                         const float* beta, const float* g, const float* S0, void* O,
                         int32_t o_dtype, float* S_out, int32_t B, int32_t H, int64_t T,
                         int32_t d_k, int32_t d_v, int32_t C, float scale,
                         const gdn_inverse_cfg* inv, void* workspace, size_t workspace_bytes,
                         gdn_fp8_stats* stats, void* stream);

/* gdn_chunk_fwd without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The workspace the variant needs (gdn_chunk_fwd_workspace_bytes) comes
 * from a fixed device array inside the library, GDN_NOALLOC_SCRATCH_BYTES per GPU,
 * held from library load until the process ends; a call needing more returns
 * GDN_ERR_WORKSPACE before enqueuing anything (64 MiB covers 10922 chunks of 64 for
 * the MFMA pre-pass, e.g. B*H = 64 heads of 8192 tokens, and 131072 chunks for the fp8
 * band pre-pass).  The call allocates nothing.  Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (concurrent streams or
 * threads) race on it and must be serialised by the caller.  Arguments, results and
 * errors otherwise as gdn_chunk_fwd (GDN_ERR_HIP if the array's device address
 * cannot be obtained). */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_chunk_fwd_noalloc(const void* Q, const void* K, const void* V, int32_t qkv_dtype,
                                 const float* beta, const float* g, const float* S0, void* O,
                                 int32_t o_dtype, float* S_out, int32_t B, int32_t H, int64_t T,
                                 int32_t d_k, int32_t d_v, int32_t C, float scale,
                                 const gdn_inverse_cfg* inv, gdn_fp8_stats* stats, void* stream);

/* The gated delta rule one token at a time (decode).  Per (b, h), tokens t = 0..n-1 in
 * order, a = exp(g_t), state S [d_k][d_v] fp32 entering as S_in (zeros if NULL):
 *   r = S^T k_t, p = S^T q_t;  u = beta_t (v_t - a r);  S <- a S + k_t u^T;
 *   o_t = scale (a p + (k_t . q_t) u)
 * (the state read / delta correction / state write split of one step, [PSDA] section
 * 2.B).  The state stays on chip for all n tokens of the call and is read and written
 * once ([PSDA] section 2.A's persistent state); n = 1 is one decode step.
 * Q, K [B][H][n][d_k] and V [B][H][n][d_v] in qkv_dtype (GDN_BF16 or GDN_F32); beta, g
 * [B][H][n] fp32; S_in, S_out [B][H][d_k][d_v] fp32, and here S_out MAY equal S_in (the
 * update in place; any other overlap is invalid); O [B][H][n][d_v] in o_dtype (GDN_BF16
 * or GDN_F32).  d_k in {64, 128}; d_v a multiple of 32, at most 256
 * (GDN_ERR_UNSUPPORTED otherwise).  n == 0 writes S_out = S_in (or zeros). */
gdn_status gdn_decode(const void* Q, const void* K, const void* V, int32_t qkv_dtype,
                      const float* beta, const float* g, const float* S_in, float* S_out,
                      void* O, int32_t o_dtype, int32_t B, int32_t H, int32_t n,
                      int32_t d_k, int32_t d_v, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
