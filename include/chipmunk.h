/*
 * chipmunk.h -- C ABI of the column-sparse cross-step delta library (MI355X, gfx950).
 *
 * Method: "Chipmunk: Training-Free Acceleration of Diffusion Transformers with
 * Dynamic Column-Sparse Deltas" (Silveria, Govande, Fu; Together AI research post,
 * 2025), called "the Chipmunk post" here.  Section "Activation Deltas Across
 * Diffusion Steps are Very Sparse" writes attention as softmax(Q K^T) V and the
 * MLP as gelu(x W1) W2, reads both as sums of value vectors weighted by
 * coefficients from a non-linearity (rows of V; rows of W2 plus a static bias),
 * caches those vectors and coefficients, and turns each step into a delta: only
 * a chosen subset of vectors (single hidden units, single keys) is recomputed,
 * the others are kept from the earlier step.  Its section "Motivation" asks for
 * dense on-chip tiles packed from non-contiguous columns in global memory.
 *
 * Operational shape used here: tokens are grouped in row blocks of 128
 * (CHIPMUNK_ROW_BLOCK); each block recomputes its own top-k columns (MLP hidden
 * units) or keys (attention); GELU is the tanh form; the attention cache holds
 * the refresh-step row max, numerator and denominator.
 *
 * Conventions (all entry points)
 *  - Every tensor is a caller-owned HIP DEVICE pointer on the current device,
 *    16-byte aligned except idx, score, b1, b2, m and den (4-byte aligned).
 *    bf16 tensors are passed as their raw 16-bit patterns (uint16_t).  The
 *    library allocates no device memory; scratch space is caller-provided and
 *    sized by chipmunk_workspace_bytes().
 *  - Every compute call only ENQUEUES work on `stream` (a hipStream_t passed as
 *    void*; NULL = the null stream) and returns without synchronising.
 *    CHIPMUNK_OK means "validated and enqueued"; a fault during execution shows
 *    up at the caller's next synchronisation.
 *  - Every argument is validated before any HIP call, so a rejected call has
 *    touched nothing.  On a non-zero return, chipmunk_last_error() gives a
 *    thread-local message.  No C++ exception crosses this boundary.
 *  - Row blocks: nb = ceil(n / 128); the last block may be partial.  Rows past
 *    n inside it are padding: they are never read from inputs, never written to
 *    outputs, and are kept at zero in the activation cache.
 *  - Index sets (`idx`): int32 [rows][k], each row ascending and unique, every
 *    value in [0, cols).  Kernels clamp out-of-range values into range (so a
 *    bad index cannot fault) but the result is then meaningless;
 *    chipmunk_check_index_sets() checks sets a caller built itself.
 *  - Offsets are 64-bit, except the gathered K/V rows of the attention
 *    kernels, addressed by 32-bit byte offsets from each head's base: the
 *    attention calls require n < 2^24.  Calls are re-entrant; the only shared
 *    mutable state is the optional kernel timer (chipmunk_timing_*), which
 *    takes a lock.
 *  - Two calls that write the same buffers must be ordered by the caller
 *    (same stream, or events).
 */
#ifndef CHIPMUNK_H
#define CHIPMUNK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CHIPMUNK_ABI_VERSION 8
#define CHIPMUNK_ROW_BLOCK 128
#define CHIPMUNK_HEAD_DIM 128

/* Return codes. */
enum chipmunk_status {
  CHIPMUNK_OK = 0,
  CHIPMUNK_E_NULLPTR = 1,     /* a required pointer is NULL */
  CHIPMUNK_E_SHAPE = 2,       /* a size is out of range or misaligned to the tiling */
  CHIPMUNK_E_UNSUPPORTED = 3, /* valid request this build does not implement (head_dim != 128) */
  CHIPMUNK_E_ALIGN = 4,       /* a pointer is not 16-byte aligned */
  CHIPMUNK_E_WORKSPACE = 5,   /* workspace missing or smaller than chipmunk_workspace_bytes() */
  CHIPMUNK_E_HIP = 6,         /* a HIP runtime call (launch, event) failed */
  CHIPMUNK_E_INTERNAL = 7     /* unexpected internal failure */
};

enum chipmunk_kind { CHIPMUNK_MLP = 0, CHIPMUNK_ATTN = 1 };
enum chipmunk_attn_mode { CHIPMUNK_ATTN_SPARSE = 0, CHIPMUNK_ATTN_REFRESH = 1 };
enum chipmunk_op {
  CHIPMUNK_OP_DENSE_MLP = 0,
  CHIPMUNK_OP_SPARSE_MLP = 1,
  CHIPMUNK_OP_TOPK = 2,
  CHIPMUNK_OP_DENSE_ATTN = 3,
  CHIPMUNK_OP_SPARSE_ATTN = 4,
  CHIPMUNK_OP_DENSE_MLP_FP8 = 5, /* the dense MLP step of a CHIPMUNK_MLP_FP8 layer */
  CHIPMUNK_OP_SPARSE_MLP_FP8 = 6 /* the sparse MLP delta of a CHIPMUNK_MLP_FP8 layer */
};

/* One MLP layer: y = gelu(x W1 + b1) W2 + b2, plus its caches.
 *   n      tokens (>= 1)
 *   d      model width, a multiple of 128
 *   h      hidden width, a multiple of 64
 *   w1t    [h][d] bf16, row j = hidden unit j's input weights (an nn.Linear
 *          fc1.weight as stored); column j of W1 is row j here, so a gathered
 *          hidden unit is one contiguous row
 *   b1     [h] fp32 or NULL (= zero)
 *   w2     [h][d] bf16, row j = hidden unit j's output vector (fc2.weight
 *          transposed once), again one contiguous row per hidden unit
 *   b2     [d] fp32 or NULL (= zero); only the dense step adds it -- a static
 *          vector cancels from every delta
 *   a_cache [nb][h][128] bf16 activation cache, block-column-major: hidden unit
 *          j of block b is 128 contiguous values (256 bytes), one per row
 *   score  [nb][h] fp32 per-block column scores written by the dense step
 *          (and, with CHIPMUNK_MLP_RESCORE, by every sparse step for its S)
 *   flags  0, or CHIPMUNK_MLP_RESCORE: the sparse delta also sets score[b][j]
 *          for each recomputed unit j of S_b to this step's column L1 over the
 *          block's rows, sum_i |a_S[i,j] - a_cache[i,j]| (the dense step's
 *          score formula, applied to the units the step recomputed), so the
 *          next identification can choose a different S (the Chipmunk post
 *          chooses which vectors to recompute dynamically, in each step;
 *          Activation Deltas section).  Units outside S_b keep their scores.
 *          Requires score.  0 keeps S fixed until the next dense step.
 *          CHIPMUNK_MLP_FP8 (may be combined with RESCORE): the first product
 *          (dense and sparse) runs on fp8 operands -- the Chipmunk post
 *          sparsifies an FP8 FLUX model (Results section).  Each call
 *          quantizes x into its workspace row by row (chipmunk_quantize_fp8's
 *          encoding) and reads W1^T from w1t_f8 / w1t_scale, which the caller
 *          fills once with chipmunk_quantize_fp8(w1t).  The matrix cores take
 *          the e4m3 codes with the row scales as E8M0 scale operands and
 *          accumulate in fp32; everything after the product (b1, GELU, bf16
 *          cache, D, the second product) is unchanged.  w1t may then be NULL.
 *          CHIPMUNK_MLP_FP8_W2 (may be combined with the others): the
 *          second product of the sparse delta runs on fp8 operands too.  The
 *          first product's epilogue rounds D to bf16 (as always) and then to
 *          e4m3 codes with one E8M0 scale per (row, 32 consecutive units of
 *          S_b), chipmunk_quantize_fp8's rule applied to each such block; W2
 *          comes from w2_f8 / w2_scale, which the caller fills once with
 *          chipmunk_quantize_fp8_cols(w2) (one scale per output column).  The
 *          dense step's second product stays bf16 (it reads w2).  The
 *          workspace is the same as without the flag.
 *   w1t_f8    [h][d] e4m3 codes of W1^T (FP8 layers only; 16-byte aligned)
 *   w1t_scale [h] E8M0 scale bytes of those rows (FP8 layers only)
 *   w2_f8     [h][d] e4m3 codes of W2 (FP8_W2 layers only; 16-byte aligned)
 *   w2_scale  [d] E8M0 scale bytes of W2's columns (FP8_W2 layers only)
 */
typedef struct chipmunk_mlp {
  int64_t n;
  int32_t d;
  int32_t h;
  const uint16_t* w1t;
  const float* b1;
  const uint16_t* w2;
  const float* b2;
  uint16_t* a_cache;
  float* score;
  uint32_t flags;
  const uint8_t* w1t_f8;
  const uint8_t* w1t_scale;
  const uint8_t* w2_f8;
  const uint8_t* w2_scale;
} chipmunk_mlp;

#define CHIPMUNK_MLP_RESCORE 1u
#define CHIPMUNK_MLP_FP8 2u
#define CHIPMUNK_MLP_FP8_W2 4u

/* One attention layer's cache (all heads).
 *   n        tokens (queries = keys, 1 <= n < 2^24)
 *   heads    number of heads (>= 1)
 *   head_dim must be 128
 *   scale    softmax scale (usually 1/sqrt(head_dim))
 *   m        [heads][n] fp32 row max of scale*q.k at the latest refresh
 *   num      [heads][n][128] fp32 softmax numerator sum_j exp(s_ij - m_i) v_j;
 *            after a REFRESH call only the part over keys outside S
 *   den      [heads][n] fp32 denominator sum_j exp(s_ij - m_i); after REFRESH
 *            only the part outside S
 *   score    [heads][nb][n] fp32 key-mass scores of the latest refresh
 */
typedef struct chipmunk_attn {
  int64_t n;
  int32_t heads;
  int32_t head_dim;
  float scale;
  float* m;
  float* num;
  float* den;
  float* score;
} chipmunk_attn;

/* Dense refresh step (the ordinary full forward pass that also fills the
 * caches; Chipmunk post, Activation Deltas section).
 *
 * kind = CHIPMUNK_MLP: layer is a const chipmunk_mlp*; x_or_q = x [n][d] bf16;
 *   k and v must be NULL; out = the output cache y [n][d] fp32.  Computes
 *   z = x W1 + b1, a = bf16(gelu_tanh(z)) (fp32 math, round to nearest even),
 *   score[b][j] = sum over block b's real rows of |a - a_cache_old| (fp32),
 *   then a_cache <- a and y = a W2 + b2 (fp32 accumulate).  ws may be NULL,
 *   except for a CHIPMUNK_MLP_FP8 layer: chipmunk_workspace_bytes(
 *   CHIPMUNK_OP_DENSE_MLP_FP8, n, d, h, 0) bytes, 16-byte aligned.
 * kind = CHIPMUNK_ATTN: layer is a const chipmunk_attn*; x_or_q, k, v =
 *   q, k, v [heads][n][128] bf16; out = o [heads][n][128] fp32.  Per head, with
 *   s = scale q k^T: m = rowmax(s), den = sum_j exp(s - m), num = exp(s - m) v,
 *   o = num / den, score[h][b][j] = sum over block b's rows of exp(s_ij - m_i)
 *   / den_i.  Follow it with chipmunk_identify_topk on the scores and
 *   chipmunk_sparse_attn_delta(mode = CHIPMUNK_ATTN_REFRESH) to leave only the
 *   part outside S in num/den.  ws may be NULL.
 */
int chipmunk_dense_step(int kind, const void* layer, const uint16_t* x_or_q, const uint16_t* k,
                        const uint16_t* v, float* out, void* ws, size_t ws_bytes, void* stream);

/* Sparsity identification: for each of `rows` score rows of length `cols`
 * (row-major fp32, row stride = cols), the k columns with the largest score,
 * written ascending to idx [rows][k].  Order: larger score first, equal scores
 * to the lower column index, -0 equal to +0, NaN below everything, +inf above
 * every finite value.  Integer work on monotone 32-bit keys, so the result is
 * exact and deterministic.  0 <= k <= cols; k = 0 or rows = 0 enqueues nothing.
 * ws may be NULL. */
int chipmunk_identify_topk(const float* score, int64_t rows, int64_t cols, int32_t k, int32_t* idx,
                           void* ws, size_t ws_bytes, void* stream);

/* Checks index sets against the contract above, on the device: for each of
 * `rows` rows of idx [rows][k] (row stride k), whether every value is in
 * [0, cols) and the row is strictly ascending (so its values are unique).
 * Writes result[0] = the number of rows that break the contract and
 * result[1] = the smallest such row (`rows` if none), as int64 in device
 * memory the caller owns (8-byte aligned); the call allocates nothing.  For
 * callers that build index sets themselves (the kernels clamp bad values,
 * which hides the mistake).  0 <= k <= cols; rows = 0 or k = 0 writes
 * {0, rows}.  Enqueues two small kernels on `stream`. */
int chipmunk_check_index_sets(const int32_t* idx, int64_t rows, int32_t k, int64_t cols, int64_t* result,
                              void* stream);

/* Sparse MLP delta step (Chipmunk post, Activation Deltas section): per block b
 * with S = idx[b] (k hidden units), gather the rows W1^T[S], W2[S] and the cache
 * columns a_cache[b][S] into on-chip tiles and compute
 *   a_S = bf16(gelu_tanh(x_b W1[:,S] + b1[S]))
 *   D   = a_S - a_cache[b][:,S]       (exact in fp32, then bf16 as the matrix operand)
 *   y_b = y_b + D W2[S,:]             (fp32 accumulate, in place)
 * and write a_S back: into a_cache[b][S] when a_new_packed is NULL (fused
 * writeback), else into a_new_packed [nb][k][128] bf16 (same block-column-major
 * order, for chipmunk_cache_writeback) leaving the cache unchanged.
 * x [n][d] bf16, idx [nb][k] int32, y [n][d] fp32.  0 <= k <= h; k = 0 leaves
 * every buffer bit-unchanged.  ws must hold chipmunk_workspace_bytes(
 * CHIPMUNK_OP_SPARSE_MLP, n, d, h, k) bytes: the D tiles, [nb][kp/32][128][32]
 * bf16 (per block, 32-unit chunks of the kept units in idx order, each chunk
 * token row by token row; kp = k rounded up to 64, units past k are written as
 * zero); for a
 * CHIPMUNK_MLP_FP8 layer, chipmunk_workspace_bytes(CHIPMUNK_OP_SPARSE_MLP_FP8,
 * n, d, h, k) bytes: the D tiles, then the fp8 copy of x. */
int chipmunk_sparse_mlp_delta(const chipmunk_mlp* layer, const uint16_t* x, const int32_t* idx,
                              int32_t k, float* y, uint16_t* a_new_packed, void* ws, size_t ws_bytes,
                              void* stream);

/* chipmunk_sparse_mlp_delta for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments and results as chipmunk_sparse_mlp_delta (bit
 * for bit: the same kernels), without ws: the workspace is a scratch array
 * inside the library, CHIPMUNK_NOALLOC_SCRATCH_BYTES (64 MiB) of device
 * memory that every GPU the library runs on holds from module load until the
 * process ends.  Calls whose workspace (chipmunk_workspace_bytes of
 * CHIPMUNK_OP_SPARSE_MLP, or of CHIPMUNK_OP_SPARSE_MLP_FP8 for an FP8 layer)
 * exceeds it fail with CHIPMUNK_E_WORKSPACE before anything is enqueued (the
 * FLUX.1-dev 1280x768 shape, 4352 tokens at k = 3686, needs 32.3 MB).  The
 * call allocates nothing.  Every call on one GPU shares that GPU's array:
 * calls that may overlap in time on one GPU (other streams, other threads)
 * race on it and must be ordered by the caller.  Nothing in the array needs
 * to start at zero (each call writes every byte it later reads). */
#define CHIPMUNK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int chipmunk_sparse_mlp_delta_noalloc(const chipmunk_mlp* layer, const uint16_t* x, const int32_t* idx, int32_t k,
                                      float* y, uint16_t* a_new_packed, void* stream);

/* Sparse attention delta (Chipmunk post, Activation Deltas section): per head h
 * and query block b with S = idx[h*nb + b] (kk keys), gather K[S], V[S] into
 * on-chip tiles, p = exp(scale q_b K[S]^T - m) with the refresh row max m,
 * num_S = p V[S], den_S = sum p, then
 *   mode SPARSE : o = (num + num_S) / (den + den_S)   (num, den hold the part
 *                 outside S, as left by REFRESH; they are not modified)
 *   mode REFRESH: num <- num - num_S, den <- den - den_S (o may be NULL; called
 *                 once after the dense step, on the dense step's q, k, v)
 * q, k, v [heads][n][128] bf16; idx [heads][nb][kk] int32; o [heads][n][128]
 * fp32.  0 <= kk <= n; kk = 0 in SPARSE mode writes o = num / den. */
int chipmunk_sparse_attn_delta(const chipmunk_attn* layer, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* idx, int32_t kk, int mode, float* o,
                               void* stream);

/* Sparse attention step with per-step re-identification (Chipmunk post,
 * Activation Deltas section: the vectors to recompute are chosen anew in each
 * step, and a step swaps the earlier step's chosen vectors for its own).  Here
 * num and den hold TOTALS over all keys, as chipmunk_dense_step(CHIPMUNK_ATTN)
 * leaves them (no REFRESH call), and S = idx[h*nb + b] may change from step to
 * step (typically chipmunk_identify_topk on the layer's scores, run before each
 * step).  Per head h and query block b, with the refresh row max m:
 *   p_old = exp(scale q_prev_b K_prev[S]^T - m)   (the previous step's share)
 *   p_new = exp(scale q_b K[S]^T - m)             (this step's share)
 *   num <- num - p_old V_prev[S] + p_new V[S],  den <- den - sum p_old + sum p_new
 *   o    = num / den
 *   score[h][b][j] <- sum over the block's rows of p_new / den_before, j in S
 *                     (den_before: den when the call starts); other scores kept.
 * The bf16 products use p rounded to bf16 (p_old negated exactly); den sums
 * the fp32 p; the scores are fp32 sums of fp16 p times fp16 2^14 / den_before
 * (den_before must lie in [2^-2, 2^28], which holds while the row max is
 * close to the refresh's).  q_prev, k_prev, v_prev are the previous step's
 * inputs (the dense step's for the first sparse step); they may be the same
 * buffers as q, k, v.  layer->score is required.  No buffer the call writes
 * (o, num, den, score) may overlap another buffer of the call:
 * CHIPMUNK_E_SHAPE.  kk = 0 writes o = num / den and leaves num, den and score
 * as they are.  Shapes, alignment and kk as for chipmunk_sparse_attn_delta. */
int chipmunk_sparse_attn_reident(const chipmunk_attn* layer, const uint16_t* q_prev, const uint16_t* k_prev,
                                 const uint16_t* v_prev, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                 const int32_t* idx, int32_t kk, float* o, void* stream);

/* Both sparse deltas of one step in two launches: chipmunk_sparse_mlp_delta on
 * `mlp` and chipmunk_sparse_attn_delta(mode = CHIPMUNK_ATTN_SPARSE) on `attn`,
 * with the arguments of those two calls and the same results, bit for bit.
 * The MLP's sparse phase 1 runs first; one kernel then holds the MLP's phase-2
 * tiles and the attention units side by side (the method computes each delta
 * separately, see the two calls above; sharing one grid is a scheduling choice
 * that keeps the chip full at the tails of both).  For deltas that do not
 * depend on each other, e.g. a block that applies attention and MLP to the
 * same input: no buffer written by one delta (y, a_cache, a_new_packed, ws;
 * o) may overlap a buffer that the other reads or writes, and the call fails
 * with CHIPMUNK_E_SHAPE when the ranges it can see overlap.  k = 0 skips the
 * MLP part; kk = 0 writes o = num / den. */
int chipmunk_sparse_step(const chipmunk_mlp* mlp, const uint16_t* x, const int32_t* mlp_idx, int32_t k,
                         float* y, uint16_t* a_new_packed, void* ws, size_t ws_bytes,
                         const chipmunk_attn* attn, const uint16_t* q, const uint16_t* kx, const uint16_t* v,
                         const int32_t* attn_idx, int32_t kk, float* o, void* stream);

/* chipmunk_sparse_step with the re-identifying attention step: the MLP delta
 * of chipmunk_sparse_mlp_delta and chipmunk_sparse_attn_reident on `attn`,
 * with the arguments of those two calls and the same results, bit for bit,
 * in two launches (the MLP's phase 1, then one grid with the MLP's phase-2
 * tiles and the attention units).  The same independence rule as
 * chipmunk_sparse_step: no buffer either delta writes (y, a_cache,
 * a_new_packed, ws, the MLP score when rescoring; o, num, den, the attention
 * score) may overlap a buffer the other reads or writes (CHIPMUNK_E_SHAPE). */
int chipmunk_sparse_step_reident(const chipmunk_mlp* mlp, const uint16_t* x, const int32_t* mlp_idx, int32_t k,
                                 float* y, uint16_t* a_new_packed, void* ws, size_t ws_bytes,
                                 const chipmunk_attn* attn, const uint16_t* q_prev, const uint16_t* k_prev,
                                 const uint16_t* v_prev, const uint16_t* q, const uint16_t* kx, const uint16_t* v,
                                 const int32_t* attn_idx, int32_t kk, float* o, void* stream);

/* Cache writeback (the separate form of the fused writeback above): copy the
 * packed new activations a_new_packed [nb][k][128] into a_cache[b][idx[b][p]]
 * for every block b and position p.  Contiguous 256-byte segments. */
int chipmunk_cache_writeback(const chipmunk_mlp* layer, const uint16_t* a_new_packed, const int32_t* idx,
                             int32_t k, void* stream);

/* Row-wise fp8 quantization (the operand encoding of CHIPMUNK_MLP_FP8): for
 * each row of src [rows][cols] bf16, e = the smallest integer >= -126 with
 * max|row| * 2^-e <= 448 (e = 0 for an all-zero row); dst[r][c] = the OCP e4m3
 * code of src[r][c] * 2^-e rounded to nearest even (the scaling is exact and
 * the result never exceeds 448); scale[r] = 127 + e, the E8M0 byte of 2^e.
 * Inputs must be finite.  cols a positive multiple of 8; src and dst 16-byte
 * aligned, scale any alignment; dst and scale must not overlap src.  rows = 0
 * enqueues nothing.  Bit-exact (integer work after an exact scaling). */
int chipmunk_quantize_fp8(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* dst, uint8_t* scale,
                          void* stream);

/* Column-wise form (the encoding of w2_f8 / w2_scale): the same rule with one
 * scale per column, scale[c] = 127 + e_c for e_c from max over rows of
 * |src[r][c]|.  Same arguments and conditions as chipmunk_quantize_fp8
 * (scale has cols bytes). */
int chipmunk_quantize_fp8_cols(const uint16_t* src, int64_t rows, int32_t cols, uint8_t* dst, uint8_t* scale,
                               void* stream);

/* Scratch bytes an op needs for these sizes (0 when none).  op: chipmunk_op.
 * CHIPMUNK_OP_SPARSE_MLP: nb*kp*128*2 with kp = k rounded up to 64 (the D
 * tiles); CHIPMUNK_OP_SPARSE_MLP_FP8: that plus the fp8 copy of x, n*d codes
 * and n scale bytes rounded up to 16; CHIPMUNK_OP_DENSE_MLP_FP8: the fp8 copy
 * of x alone; the others: 0. */
size_t chipmunk_workspace_bytes(int op, int64_t n, int32_t d, int32_t h, int32_t k);

/* Thread-local text of the last failure on this thread ("" if none). */
const char* chipmunk_last_error(void);

/* CHIPMUNK_ABI_VERSION of the loaded library. */
int chipmunk_abi_version(void);

/* Digest of the sources the library was built from: the first 16 hex digits
 * of SHA-256 over every file of the library's source and include folders, as
 * the package's build step computes it ("unknown" for a build that did not
 * pass one).  The Python binding refuses a library whose digest differs from
 * the sources beside it.  Static string, never freed. */
const char* chipmunk_source_digest(void);

/* Optional per-kernel timer.  While enabled, every kernel the library launches
 * is bracketed by a pair of HIP events on its own stream.  chipmunk_timing_read
 * waits for the recorded events and returns, for kernel id `kid` (0 <=
 * kid < chipmunk_kernel_count()), the summed duration in milliseconds and the
 * launch count since the last enable.  Names: chipmunk_kernel_name(kid).
 * Enabling clears earlier records.  Guarded by a process-wide lock. */
int chipmunk_timing_enable(int on);
int chipmunk_timing_read(int kid, double* total_ms, int64_t* launches);
int chipmunk_kernel_count(void);
const char* chipmunk_kernel_name(int kid);

#ifdef __cplusplus
}
#endif

#endif /* CHIPMUNK_H */
