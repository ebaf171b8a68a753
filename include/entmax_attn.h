/*
 * entmax_attn.h -- C ABI of the fused alpha-entmax attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For every batch b, head h and query row i:
 *   s_ij  = q_i . k_j / sqrt(d)                       (j visible: all j, or j <= i when causal)
 *   x_ij  = (alpha - 1) s_ij
 *   tau_i : the unique root of  sum_j [x_ij - tau_i]_+^(1/(alpha-1)) = 1
 *   p_ij  = [x_ij - tau_i]_+^(1/(alpha-1))
 *   o_i   = sum_j p_ij v_j
 * alpha = 2 is sparsemax, alpha -> 1 tends to softmax ("AdaSplash: Adaptive
 * Sparse Flash Attention", ICML 2025 talk summary, section "Background").
 * tau is found per row by Halley steps guarded by a bisection bracket (same
 * page, "Accelerated Alpha-Entmax Transformation"), optionally started from a
 * coarse per-row score histogram kept on chip ("AdaSplash-2: The Transformer
 * Revolution We Didn't See Coming", section "Sparse Attention Makes Waves").
 * S and P are never written to memory: Q tiles stay on chip and K/V tiles are
 * streamed ("AdaSplash ...", section "AdaSplash: Fused GPU Kernel for
 * Attention"), and key tiles whose probabilities are all zero are skipped in
 * the output pass and in the backward (same page, "Exploiting Sparsity").
 *
 * Backward: with t = [x - tau]_+ and u = t^(1/(alpha-1) - 1) (= p^(2-alpha))
 * on the support, dS = u * (dP - delta_i), delta_i = sum_j u_ij dP_ij / sum_j u_ij,
 * dP = dO V^T, dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d), dV = P^T dO.
 *
 * Conventions shared by every entry point:
 *  - Tensors are dense, row-major [B, H, N, d] (d fastest), device memory,
 *    16-byte aligned.  tau is float32 [B, H, N] in the x-domain above.
 *  - in_dtype (q, k, v, dout) and out_dtype (out, dq, dk, dv) are EA_F32 or
 *    EA_BF16.  d must be 64 or 128.  N >= 0 is arbitrary (ragged tails are
 *    masked, N <= 2^20); B, H >= 1.  1 < alpha <= 2.
 *  - The caller owns every buffer, including the workspace.  The library
 *    allocates no device memory, keeps no mutable global state, and enqueues
 *    all work asynchronously on `stream` (a hipStream_t; NULL = default
 *    stream).  Calls on distinct buffers may run concurrently.
 *  - Errors: every argument check happens before any work is enqueued, so a
 *    call that returns an error has written nothing.  A failed launch returns
 *    EA_ERR_LAUNCH.  No C++ exception crosses this interface.
 */
#ifndef ENTMAX_ATTN_H
#define ENTMAX_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (0 = success). */
#define EA_OK               0
#define EA_ERR_NULL        -1   /* a required pointer is NULL */
#define EA_ERR_SHAPE       -2   /* B, H < 1, N < 0, d not in {64, 128}, or a key length outside [0, N] */
#define EA_ERR_DTYPE       -3   /* unknown in_dtype / out_dtype */
#define EA_ERR_ALPHA       -4   /* alpha outside (1, 2] or not finite */
#define EA_ERR_ALIGN       -5   /* a tensor pointer is not 16-byte aligned */
#define EA_ERR_WORKSPACE   -6   /* ws_bytes smaller than entmax_attn_workspace_bytes() */
#define EA_ERR_LAUNCH      -7   /* the HIP runtime rejected a kernel launch */
#define EA_ERR_UNSUPPORTED -8   /* unknown tau_mode, negative max_iters, bad tol or flags */

/* Element types. */
#define EA_F32  0
#define EA_BF16 1

/* tau initialisation / refinement modes. */
#define EA_TAU_HIST_HALLEY   0  /* histogram-initialised Halley-bisection (default) */
#define EA_TAU_HALLEY_BISECT 1  /* Halley-bisection started at the bracket's lower end */
#define EA_TAU_BISECT        2  /* plain bisection of the bracket */

/* Flags. */
#define EA_FLAG_FORCE_DENSE  1  /* mark every visible tile active: no tile skipping */

/* Tile shape of block_mask: one byte per (32 queries) x (64 keys). */
#define EA_MASK_BM 32
#define EA_MASK_BN 64

typedef struct {
  int32_t B, H, N, d;   /* batch, heads, sequence length, head dim (64 or 128) */
  int32_t in_dtype;     /* EA_F32 | EA_BF16: q, k, v, dout */
  int32_t out_dtype;    /* EA_F32 | EA_BF16: out, dq, dk, dv */
  int32_t tau_mode;     /* EA_TAU_* */
  int32_t max_iters;    /* refinement sweeps per row; 0 = default (12, or 40 for BISECT) */
  float   tol;          /* stop when |f(tau)| <= tol; 0 = default 1e-6 */
  int32_t flags;        /* EA_FLAG_* */
  /* Optional timing hook: NULL, or 2 * EA_NUM_STAGES caller-created hipEvent_t
   * handles.  Stage s (EA_STAGE_*) is bracketed by events[2s] and
   * events[2s+1], recorded on `stream`; stages a call does not run are not
   * recorded.  The library never creates or destroys events. */
  void* const* events;
  /* Variable-length batches (key padding), "AdaSplash: Adaptive Sparse Flash
   * Attention", "Downstream Task Performance" (encoder models): NULL, or a
   * host array of B lengths 0 <= L_b <= N, read during the call.  Batch b
   * then attends over its first L_b keys only, and its query rows past L_b
   * see no key: their output rows are 0, tau = +inf (every p is 0), their
   * sweep count 0; dQ rows and dK / dV rows past L_b are 0, and block-mask
   * entries outside the batch's first ceil(L_b/32) x ceil(L_b/64) tiles are 0.
   * The stage events are not recorded for such calls. */
  const int32_t* key_lens;
} ea_desc;

/* Stages, for the timing hook. */
#define EA_STAGE_FWD_PREP  0   /* forward: V^T copy (fp32 inputs only) */
#define EA_STAGE_ROWMAX    1   /* forward: the full score sweep (row maxima and block codes) */
#define EA_STAGE_TAU       2   /* forward: histogram and Halley sweeps over candidate tiles, block mask;
                                  for bf16 inputs also O = P V (one kernel) */
#define EA_STAGE_PV        3   /* forward: O = P V over active tiles (fp32 inputs; empty for bf16) */
#define EA_STAGE_BWD_PREP  4   /* backward: K^T, Q^T, dO^T copies (fp32 inputs only) */
#define EA_STAGE_DQ        5   /* backward: delta, then dQ, over active tiles */
#define EA_STAGE_DKDV      6   /* backward: dK, dV over active tiles */
#define EA_NUM_STAGES      7

/* Bytes of device workspace both entry points need for `desc`: one float per
 * row; (forward) one byte per (32-query block, 64-key tile), rows padded to 64
 * tiles -- the size of the block mask, B*H*ceil(N/32)*ceil(N/64) bytes, never
 * a score matrix (the fused kernel's memory grows like its inputs and its
 * block mask: "AdaSplash: Adaptive Sparse Flash Attention", "AdaSplash: Fused
 * GPU Kernel for Attention"); 256 bytes of work-queue counters (forward;
 * the call sets them itself); (backward) the block mask transposed; and for
 * fp32 inputs transposed copies of V (forward) or of K, Q, dO (backward).
 * Returns 0 for an invalid desc. */
size_t entmax_attn_workspace_bytes(const ea_desc* desc);

/* Shape of block_mask: [B, H, n_qt, n_kt] bytes with n_qt = ceil(N/bm),
 * n_kt = ceil(N/bn), bm = 32 queries, bn = 64 keys: the tiles whose all-zero
 * probabilities the output pass and the backward skip ("AdaSplash: Adaptive
 * Sparse Flash Attention", "Exploiting Sparsity").  Any output pointer may be
 * NULL.  Returns a status. */
int entmax_attn_mask_dims(const ea_desc* desc, int* n_qt, int* n_kt, int* bm, int* bn);

/* Forward pass: tau, the block mask and o = P V, with S and P never written
 * to memory ("AdaSplash: Adaptive Sparse Flash Attention", "AdaSplash: Fused
 * GPU Kernel for Attention"; tau by Halley-bisection, "Accelerated
 * Alpha-Entmax Transformation", started from a per-row histogram in
 * EA_TAU_HIST_HALLEY mode, "AdaSplash-2: The Transformer Revolution We Didn't
 * See Coming", "Sparse Attention Makes Waves").
 *  q, k, v     [B,H,N,d] in_dtype                     (read)
 *  out         [B,H,N,d] out_dtype                    (written)
 *  tau         float32 [B,H,N]                        (written)
 *  block_mask  uint8 [B,H,n_qt,n_kt] (mask_dims)      (written): nonzero where
 *              the tile holds a visible entry with x > tau, 0 otherwise (a
 *              tile marked nonzero may still be all-zero only within float32
 *              rounding).  Bit 0 marks the tile; bits 1 and 2 mark the 32x32
 *              micro-tiles (keys 0-31, 32-63 of the tile) that hold such an
 *              entry, which P V and the backward skip on their own ("AdaSplash:
 *              Adaptive Sparse Flash Attention", "Exploiting Sparsity": zero
 *              blocks skipped at micro-tile granularity).  With
 *              EA_FLAG_FORCE_DENSE every visible tile reads 7.
 *  tau_iters   uint8 [B,H,N] or NULL                  (written if non-NULL):
 *              refinement sweeps that evaluated f(tau) for the row (the
 *              row-max and histogram sweeps are not counted).
 *  alpha       1 < alpha <= 2;  causal: 0 or 1.
 *  ws          device workspace of ws_bytes >= entmax_attn_workspace_bytes(desc).
 */
int entmax_attn_fwd(const void* q, const void* k, const void* v, float alpha, int causal,
                    void* out, float* tau, uint8_t* block_mask, uint8_t* tau_iters,
                    const ea_desc* desc, void* ws, size_t ws_bytes, void* stream);

/* Forward pass without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and errors as
 * entmax_attn_fwd, minus ws / ws_bytes: the workspace is a fixed 32 MiB
 * device array inside the library, one per GPU for the life of the process,
 * and this call allocates nothing.  A desc whose forward workspace exceeds
 * 32 MiB returns EA_ERR_WORKSPACE before anything is enqueued (about
 * B*H*(4 N + N^2/2048) bytes for bf16 inputs: e.g. 16 heads at N = 32768 fit).
 * All calls on one GPU share the array: calls that overlap on one GPU (other
 * streams, other host threads) race.  entmax_attn_bwd still takes a caller
 * workspace. */
int entmax_attn_fwd_static(const void* q, const void* k, const void* v, float alpha, int causal,
                           void* out, float* tau, uint8_t* block_mask, uint8_t* tau_iters,
                           const ea_desc* desc, void* stream);

/* Backward pass over the tiles the forward found nonzero ("AdaSplash:
 * Adaptive Sparse Flash Attention", "Backward Pass": skipping all-zero tiles
 * makes the backward sub-quadratic; the gradient formula above is derived
 * from the definition of tau).  tau and block_mask must come from entmax_attn_fwd on the
 * same q, k, v, alpha, causal and desc (they are the only forward state the
 * backward needs; delta_i = sum_j u_ij dP_ij / sum_j u_ij is recomputed, so
 * no other forward-to-backward buffer exists).  Skips the tiles and 32x32
 * micro-tiles block_mask marks empty.
 *  dout        [B,H,N,d] in_dtype                     (read)
 *  dq, dk, dv  [B,H,N,d] out_dtype                    (written)
 */
int entmax_attn_bwd(const void* q, const void* k, const void* v, float alpha, int causal,
                    const void* dout, const float* tau, const uint8_t* block_mask,
                    void* dq, void* dk, void* dv,
                    const ea_desc* desc, void* ws, size_t ws_bytes, void* stream);

/* Row-wise alpha-entmax of materialised score rows, without attention
 * ("AdaSplash: Adaptive Sparse Flash Attention", "Accelerated Alpha-Entmax
 * Transformation": the entmax transform whose threshold Halley-bisection
 * finds in far fewer iterations than bisection; "AdaSplash-2: The Transformer
 * Revolution We Didn't See Coming", "Sparse Attention Makes Waves": the
 * histogram start).  For each row r:
 *   x_j = (alpha - 1) s_rj,  tau_r: sum_j [x_j - tau_r]_+^(1/(alpha-1)) = 1,
 *   p_rj = [x_j - tau_r]_+^(1/(alpha-1)).
 * -inf scores are masked entries (p = 0, not counted); a row with no finite
 * score gets tau = +inf and p = 0.  tau_mode selects the start and the steps
 * exactly as for the attention forward; tau_iters counts the sweeps that
 * evaluated f (the row-max and histogram passes are not counted).
 *  s          [rows, n] in_dtype, dense row-major        (read)
 *  p          [rows, n] out_dtype                        (written)
 *  tau        float32 [rows]                             (written)
 *  tau_iters  uint8 [rows] or NULL                       (written if non-NULL)
 * Device pointers; s, p and tau 16-byte aligned.  1 <= n <= 2^20, rows >= 0.
 * Errors: EA_ERR_NULL, EA_ERR_SHAPE, EA_ERR_DTYPE, EA_ERR_ALPHA, EA_ERR_ALIGN,
 * EA_ERR_UNSUPPORTED (tau_mode, max_iters, tol) before anything is enqueued;
 * EA_ERR_LAUNCH if the launch fails.  Asynchronous on `stream`; allocates
 * nothing. */
typedef struct {
  int64_t rows;         /* number of rows */
  int32_t n;            /* scores per row */
  int32_t in_dtype;     /* EA_F32 | EA_BF16: s */
  int32_t out_dtype;    /* EA_F32 | EA_BF16: p */
  int32_t tau_mode;     /* EA_TAU_* */
  int32_t max_iters;    /* 0 = default (12, or 40 for BISECT) */
  float   tol;          /* stop when |f(tau)| <= tol; 0 = default 1e-6 */
} ea_rows_desc;

int entmax_rows(const void* s, float alpha, void* p, float* tau, uint8_t* tau_iters,
                const ea_rows_desc* desc, void* stream);

/* Static, human-readable text for a status code. */
const char* entmax_attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* ENTMAX_ATTN_H */
