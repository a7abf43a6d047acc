/*
 * fa.h -- C ABI of the exact tiled attention library (libfa.so) for gfx950.
 *
 * The library computes exact attention O = softmax(scale * Q K^T) V and its
 * gradients without ever forming the N x N score matrix:
 *
 *   fa_fwd             forward: Q in row tiles, K/V streamed in column tiles
 *                      through an online softmax; saves only O and the
 *                      per-row logsumexp L = m + ln(l).
 *   fa_bwd_preprocess  D_i = sum_k dO_ik * O_ik, computed once before the
 *                      backward proper.
 *   fa_bwd_dkdv        dK, dV: outer loop over key/value tiles, P recomputed
 *                      on chip as exp(S - L).
 *   fa_bwd_dq          dQ: outer loop over query tiles, P recomputed again.
 *   fa_fwd_rect, fa_bwd_dkdv_rect, fa_bwd_dq_rect
 *                      the same with nq queries attending to nk keys
 *                      (causal masking aligned to the end of the keys), for
 *                      a chunk of new queries against a longer key/value
 *                      cache, and an optional causal sliding window;
 *                      fa_bwd_preprocess serves both forms.
 *   fa_bwd_fused       the single-kernel backward that the two-kernel form
 *                      is weighed against: dK, dV and dQ from one pass over
 *                      the key/value tiles, dQ gathered with atomic adds.
 *   fa_bwd_fused_noalloc
 *                      the same without a workspace argument, for callers
 *                      that cannot allocate device memory.
 *
 * Source of the method (cited by page and section):
 *   "Assignment2: FlashAttention & Distributed Data Parallel notes"
 *   (CS336), Part 1: section 1.2 (FA-2 forward: running max m, running sum l,
 *   unnormalised accumulator, final O / l, saved L = m + log l), section 1.3
 *   (one program per (batch, query tile); key tiles wholly above the
 *   diagonal are skipped in causal mode), section 1.4 (Eq 13-19 and the
 *   two-kernel backward that needs no atomics).
 *   "CS349E lecture 11, 03_flash_backward.py" demo1_gradcheck (D from one row
 *   of O and dO, computed before the backward), demo4_causal (only tiles
 *   crossing the diagonal need an in-tile mask; in decode one new token
 *   sees every cached key).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Tensors.  q, k, v, o, dO, dq, dk, dv are contiguous row-major device
 *   buffers of shape [bh][n][d] (bh = batch * heads; the head dimension d is
 *   the fastest-moving index) holding elements of `dtype`.  lse (L) and
 *   delta (D) are contiguous float32 device buffers of shape [bh][n].  Every
 *   pointer must be 16-byte aligned.
 * Math.  S = scale * Q K^T.  With causal != 0, key j is visible to query i
 *   iff j <= i (top-left aligned, queries and keys both of length n); key
 *   tiles with no visible key are skipped and only tiles crossing the
 *   diagonal are masked.  L is the natural-log logsumexp of the scaled,
 *   masked scores of each row.  Accumulation is float32; with FA_BF16 the
 *   probabilities P and dS are rounded to bf16 (round to nearest even)
 *   before they enter a bf16 matrix product, and outputs are rounded to
 *   bf16 once at the end.  With FA_F32 every product is float32.
 * n.  Any n >= 1 is accepted; a last tile shorter than the tile size is
 *   masked (rows past n are neither read nor written).
 * Tiles.  block_m (query rows per tile) and block_n (key columns per tile)
 *   select the tiling; 0, 0 picks the library default.  FA_F32 accepts
 *   block_m in {16, 32, 64, 128} and block_n in 4..128 (multiple of 4),
 *   subject to the 160 KiB LDS budget.  FA_BF16 accepts only its tuned
 *   tilings (0, 0 or the values fa_default_tiles reports).  The result does
 *   not depend on the tiling beyond float rounding.
 * Ownership.  The caller allocates and owns every buffer.  The library never
 *   allocates, frees or synchronises and is safe to call from several host
 *   threads.  The only state it keeps is the fixed device scratch array of
 *   fa_bwd_fused_noalloc (part of the library's device code, one copy per
 *   GPU) and the cached address of that array on each device.  Outputs are
 *   fully overwritten (never accumulated into) and must not alias any input.
 * Streams.  `stream` is a hipStream_t (NULL = the default stream).  Every call
 *   only enqueues work on it and returns.  The caller orders
 *   fa_bwd_preprocess before fa_bwd_dkdv and fa_bwd_dq (which are
 *   independent of each other) or before fa_bwd_fused.  Calls whose
 *   outputs or workspace overlap must not run concurrently.
 * Empty input.  bh == 0 or n == 0 is a no-op that returns FA_OK (pointers
 *   are not touched and may be NULL).
 * Queries and keys of different lengths (the *_rect calls).  q, o, dO, dq
 *   are [bh][nq][d], lse and delta [bh][nq]; k, v, dk, dv are [bh][nk][d].
 *   With causal != 0 the queries are the last nq positions of the key
 *   sequence: key j is visible to query i iff j <= i + (nk - nq), so every
 *   row sees at least one key; causal with nq > nk would leave rows with no
 *   key and returns FA_ERR_UNSUPPORTED.  bh == 0 or nq == nk == 0 is a
 *   no-op; exactly one of nq, nk zero is FA_ERR_INVALID_ARG.  The square
 *   calls are the case nq = nk = n.
 * Errors.  Arguments are validated on the host before any HIP call; an
 *   invalid call launches nothing and returns a non-zero status.  A launch
 *   failure reported by the HIP runtime returns FA_ERR_HIP.  Faults during
 *   execution surface at the caller's next synchronisation.  Nothing throws
 *   or exits across this boundary.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_ABI_VERSION 5

typedef enum { FA_F32 = 0, FA_BF16 = 1 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,   /* null pointer, negative size, bad dtype/scale, aliasing */
  FA_ERR_UNSUPPORTED = 2,   /* head dim, tiling or size not provided */
  FA_ERR_MISALIGNED = 3,    /* a pointer is not 16-byte aligned */
  FA_ERR_HIP = 4,           /* the HIP runtime rejected a launch */
  FA_ERR_TOO_LARGE = 5      /* the problem exceeds a fixed capacity (fa_bwd_fused_noalloc) */
} fa_status;

/* Bytes of the fixed device scratch array behind fa_bwd_fused_noalloc (one
 * copy on each GPU the library runs on). */
#define FA_NOALLOC_SCRATCH_BYTES ((size_t)1 << 27)

/* Forward (CS336 notes 1.2-1.3).  Reads q, k, v; writes o [bh][n][d] and
 * lse [bh][n] (float32, natural log). */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int bh, int n, int d, fa_dtype dtype, float scale, int causal,
                 int block_m, int block_n, void* stream);

/* Backward step 1 (CS336 notes 1.4 Eq 17, D = rowsum(O * dO)).  Reads o and
 * dO; writes delta [bh][n] float32. */
fa_status fa_bwd_preprocess(const void* o, const void* dO, float* delta,
                            int bh, int n, int d, fa_dtype dtype, void* stream);

/* Backward step 2 (CS336 notes 1.4 Eq 13-17, 15 and 19; the key/value-outer
 * kernel).  Reads q, k, v, dO, lse (from fa_fwd with the same q, k, v, scale
 * and causal) and delta (from fa_bwd_preprocess); writes dk and dv. */
fa_status fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO,
                      const float* lse, const float* delta, void* dk, void* dv,
                      int bh, int n, int d, fa_dtype dtype, float scale, int causal,
                      int block_m, int block_n, void* stream);

/* Backward step 3 (CS336 notes 1.4 Eq 13-18; the query-outer kernel).
 * Same inputs as fa_bwd_dkdv; writes dq. */
fa_status fa_bwd_dq(const void* q, const void* k, const void* v, const void* dO,
                    const float* lse, const float* delta, void* dq,
                    int bh, int n, int d, fa_dtype dtype, float scale, int causal,
                    int block_m, int block_n, void* stream);

/* The three calls above for nq queries against nk keys (see "Queries and
 * keys of different lengths").  fa_bwd_preprocess(o, dO, delta, bh, nq, d,
 * ...) provides delta.  window > 0 (only with causal != 0) is a sliding
 * window ("CS324 lecture 8, 03_online_softmax_and_flash.py",
 * window_attention_torch): key j is also hidden from query i when
 * j <= i + (nk - nq) - window, so each query sees its `window` most recent
 * keys; key tiles wholly outside the band are skipped and only tiles that
 * cross one of its edges are masked.  window == 0 means no window;
 * window < 0, or window > 0 without causal, is FA_ERR_INVALID_ARG.  With a
 * window (narrower than nk) and block_m = block_n = 0, the bf16 forward at
 * d = 128 uses the (128, 64) tiling instead of fa_default_tiles' (256, 64),
 * and fa_bwd_dq_rect at d = 128 the (128, 32) tiling instead of (256, 32). */
fa_status fa_fwd_rect(const void* q, const void* k, const void* v, void* o, float* lse,
                      int bh, int nq, int nk, int d, fa_dtype dtype, float scale, int causal,
                      int window, int block_m, int block_n, void* stream);
fa_status fa_bwd_dkdv_rect(const void* q, const void* k, const void* v, const void* dO,
                           const float* lse, const float* delta, void* dk, void* dv,
                           int bh, int nq, int nk, int d, fa_dtype dtype, float scale,
                           int causal, int window, int block_m, int block_n, void* stream);
fa_status fa_bwd_dq_rect(const void* q, const void* k, const void* v, const void* dO,
                         const float* lse, const float* delta, void* dq,
                         int bh, int nq, int nk, int d, fa_dtype dtype, float scale,
                         int causal, int window, int block_m, int block_n, void* stream);

/* Single-kernel backward (the alternative to steps 2 and 3 that CS336 notes
 * 1.4 sets aside: one kernel with dQ accumulated by atomic adds).  One pass
 * over the key/value tiles writes dk and dv exactly as fa_bwd_dkdv_rect
 * does and adds each (key tile, query tile) pair's dS K into dQ with float32
 * atomic adds, so dQ depends on the order in which the adds land (not
 * bitwise reproducible) and P is rebuilt once instead of twice.  Arguments
 * as fa_bwd_dkdv_rect plus dq ([bh][nq][d], `dtype`) and `workspace`:
 * FA_BF16 accumulates dQ in float32 in `workspace`
 * (fa_bwd_fused_workspace_bytes bytes of device memory, 16-byte aligned,
 * distinct from every other buffer; its contents on entry are ignored and
 * on return unspecified) and rounds scale * dQ to bf16 into dq at the end;
 * FA_F32 accumulates in dq itself and ignores `workspace` (may be NULL).
 * Tilings: kernel id 3 of fa_default_tiles (bf16: block_m = 64 query rows
 * per step, block_n = 128 keys per workgroup; float32: as fa_bwd_dkdv within
 * the LDS budget).  Needs delta from fa_bwd_preprocess like steps 2 and 3. */
fa_status fa_bwd_fused(const void* q, const void* k, const void* v, const void* dO,
                       const float* lse, const float* delta, void* dq, void* dk, void* dv,
                       float* workspace, int bh, int nq, int nk, int d, fa_dtype dtype,
                       float scale, int causal, int window, int block_m, int block_n,
                       void* stream);
/* Bytes of `workspace` fa_bwd_fused needs: bh * nq * d * 4 for FA_BF16, 0 for
 * FA_F32 (and 0 for non-positive sizes).  Pure host function. */
size_t fa_bwd_fused_workspace_bytes(int bh, int nq, int d, fa_dtype dtype);

/* Allocation-free single-kernel backward, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of fa_bwd_fused without `workspace`.  FA_BF16 accumulates dQ in float32 in
 * a fixed device array of the library (FA_NOALLOC_SCRATCH_BYTES bytes, one
 * copy on each GPU the library runs on, held until the process ends) instead
 * of a caller workspace; FA_F32 accumulates in dq as fa_bwd_fused does.  The
 * call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine); its first call on a device looks up that device's copy of the
 * array (the device of `stream`).  With FA_BF16, bh * nq * d * 4 >
 * FA_NOALLOC_SCRATCH_BYTES returns FA_ERR_TOO_LARGE before any HIP call.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (each call clears it before use): calls that overlap on one GPU
 * (on concurrent streams or from several host threads) race on it and must
 * be serialised by the caller. */
fa_status fa_bwd_fused_noalloc(const void* q, const void* k, const void* v, const void* dO,
                               const float* lse, const float* delta, void* dq, void* dk, void* dv,
                               int bh, int nq, int nk, int d, fa_dtype dtype, float scale,
                               int causal, int window, int block_m, int block_n, void* stream);

/* The tiling (block_m, block_n) that block_m = block_n = 0 selects for a
 * kernel (0 = fwd, 1 = dkdv, 2 = dq, 3 = fused backward) at this dtype and
 * head dim.  Returns
 * FA_ERR_UNSUPPORTED for a head dim or dtype the library does not provide.  Pure
 * host function. */
fa_status fa_default_tiles(fa_dtype dtype, int d, int kernel, int* block_m, int* block_n);

/* Static string for a status code (never NULL). */
const char* fa_status_str(fa_status s);

/* FA_ABI_VERSION of the built library. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
