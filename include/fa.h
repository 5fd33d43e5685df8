/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * The operation.  For every (batch b, head h), with Q, K, V the N x D
 * slices q[b][h], k[b][h], v[b][h]:
 *
 *     S = scale * Q K^T                       (N x N, never stored)
 *     P = row-wise softmax of S               (causal: S[i][j] = -inf for j > i)
 *     O = P V                                 (N x D)
 *     L[i] = m_i + ln(l_i)                    (natural-log log-sum-exp of row i)
 *
 * where m_i is the row max of S and l_i = sum_j exp(S[i][j] - m_i).  This is
 * the exact-attention definition of the "Flash Attention" page (opening
 * definition) and of "Learning Metal with FlashAttention" (section
 * FlashAttention); L is the statistic the forward kernel of the
 * metal-flash-attention README saves for the backward ("Quantifying
 * performance", forward pseudocode).  Causal masking is top-left aligned:
 * query i sees keys 0..i.
 *
 * The backward entry points compute the gradients of O with respect to Q, K
 * and V given dO, split the way the metal-flash-attention README's backward
 * pseudocode splits them ("Quantifying performance": a backward-query kernel
 * and a backward-key-value kernel, no floating-point atomics):
 *
 *     delta[i] = sum_d dO[i][d] * O[i][d]
 *     P = exp(S - L)            (S the scaled scores, L from the forward)
 *     dP = dO V^T,  dS = P * (dP - delta)    (elementwise)
 *     dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dO
 *
 * Conventions for every entry point
 * ---------------------------------
 * Layout.   Q, K, V, O, dO, dQ, dK, dV are contiguous [B][H][N][D] (BHND,
 *           D fastest).  L and delta are contiguous float32 [B][H][N].
 * Pointers. All tensor pointers are DEVICE pointers.  The caller allocates
 *           and owns every buffer; the library never allocates, frees,
 *           copies between host and device or synchronises.  Outputs must
 *           not alias inputs.
 * Stream.   `stream` is a hipStream_t passed as void*; NULL is the default
 *           stream.  Each call enqueues its kernels and returns; results are
 *           ready when the stream reaches that point.
 * Errors.   0 on success, else a negative FA_ERR_* code; nothing is thrown
 *           or aborted across the ABI.  Argument checks happen before any
 *           HIP call, so a rejected call touches no device state.
 * Threads.  No global mutable state: calls from several host threads on
 *           different streams are safe.
 * Sizes.    B, H, N >= 1; B*H*N*D must fit in 2^31 - 1 elements per tensor.
 *           Head dims: D in {32, 64, 96, 128, 160, 256} for the bf16
 *           forward entry points, {32, 64, 96, 128, 256} for the backward,
 *           {64, 128, 256} for fa_fwd_f32; each entry point below states its
 *           own.
 *           scale must be finite and > 0 (the scores use scale = 1/sqrt(D)
 *           in every workload here; any positive scale is accepted).
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_OK 0
#define FA_ERR_INVALID_ARG (-1) /* null pointer, B/H/N/D <= 0, bad scale, size overflow */
#define FA_ERR_UNSUPPORTED (-2) /* valid but not supported: head dim or sequence length */
#define FA_ERR_LAUNCH (-3)      /* the kernel launch failed (hipGetLastError) */

/*
 * Forward, bfloat16 in and out, float32 accumulation.
 *   q, k, v : bf16 [B][H][N][D]        (read)
 *   o       : bf16 [B][H][N][D]        (written; O rounded to nearest-even)
 *   lse     : f32  [B][H][N]           (written; L = m + ln l, natural log)
 * D in {32, 64, 96, 128, 160, 256}.  Any N >= 1.  causal: 0 or 1.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D,
           float scale, int causal, void* stream);

/*
 * Forward with query and key lengths apart, keys optionally split over
 * several workgroups per query block (bf16 in and out, float32
 * accumulation).
 *   q       : bf16 [B][H][Nq][D]       (read)
 *   k, v    : bf16 [B][H][Nk][D]       (read)
 *   o       : bf16 [B][H][Nq][D]       (written)
 *   lse     : f32  [B][H][Nq]          (written; natural log)
 * Query row i sees every key without causal masking.  With causal = 1 the
 * query rows are the last Nq positions of the key sequence: row i sees keys
 * 0 .. i + (Nk - Nq), so Nq = Nk is fa_fwd's mask and Nq = 1 (decoding one
 * row) sees every key.  The pages fix no alignment for Nq != Nk; this is
 * the reading taken.  causal = 1 requires Nq <= Nk.
 *
 * The "Flash Attention" page (section on the technique's boundaries) sets
 * decoding apart: a few query rows cannot fill a matrix tile, so the
 * (query block, batch, head) grid is too small to occupy the GPU.  Here the
 * keys a query block sees are divided into num_splits contiguous ranges,
 * one workgroup each; every range writes the attention of its keys (O
 * normalised by its own row sum, float32) and its L_s into the workspace,
 * and a second kernel merges them exactly:
 * L = ln sum_s e^{L_s}, O = sum_s e^{L_s - L} O_s.
 * Nq <= 4 runs a vector kernel (the pages' "separate vector kernel" for
 * decoding; P kept in float32), larger Nq the matrix-core forward kernel
 * (P rounded to bf16 for the P V product, as in fa_fwd).
 *
 *   num_splits      : 0 = the library's choice (fa_fwd_kv_splits), else
 *                     1..256.  1 runs without workspace or merge.
 *   workspace       : device memory of at least
 *                     fa_fwd_kv_workspace_bytes(B, H, Nq, D, splits) bytes,
 *                     16-byte aligned, owned by the caller (may be NULL when
 *                     that size is 0).  Its contents on entry do not
 *                     matter; it is overwritten.  Two calls in flight at
 *                     once must not share it.
 * D in {32, 64, 96, 128, 160, 256} (the vector kernel for Nq <= 4 serves 64,
 * 128 and 256; the others run on the matrix-core kernel); any Nq, Nk >= 1.
 * Errors: FA_ERR_INVALID_ARG also
 * for causal with Nq > Nk, num_splits outside 0..256, a missing, short or
 * misaligned workspace, or more than 2^31 - 1 workgroups (query blocks x
 * key ranges x B x H).
 */
int fa_fwd_kv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk, int D,
              float scale, int causal, int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * fa_fwd_kv for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, semantics, kernels and results as fa_fwd_kv, except that
 * the key-range partials go to a scratch array of
 * FA_FWD_KV_NOALLOC_MAX_BYTES the library holds on each device (set up on
 * the first call on that device, kept until the process ends) instead of
 * a caller workspace.  The call allocates nothing.
 *   Errors: FA_ERR_INVALID_ARG as fa_fwd_kv, and also when the partials
 *   need more than FA_FWD_KV_NOALLOC_MAX_BYTES, i.e. when
 *   fa_fwd_kv_workspace_bytes(B, H, Nq, D, splits) exceeds it for the
 *   range count used (pass a smaller num_splits, or use fa_fwd_kv);
 *   FA_ERR_LAUNCH if the scratch array's device address cannot be read.
 * Every call on one device shares that device's scratch array: calls
 * that overlap on one device (other streams, other host threads) race and
 * must be ordered by the caller.  A call with one key range uses no scratch.
 */
#define FA_FWD_KV_NOALLOC_MAX_BYTES ((size_t)64 << 20)
int fa_fwd_kv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Nq, int Nk,
                      int D, float scale, int causal, int num_splits, void* stream);

/*
 * The key-range count fa_fwd_kv uses for num_splits = 0, at most 256.  For
 * Nq > 4 (matrix-core kernel): enough workgroups to occupy every CU of the
 * current device, at least two key tiles of 64 per range.  For Nq <= 4
 * (vector decode kernel): about one workgroup per CU (two for Nq > 2), at
 * least two ranges, each over at least 256 keys.  Returns a count >= 1, or a negative
 * FA_ERR_* code for invalid sizes.  Queries the current device's CU count
 * (no device state is changed).
 */
int fa_fwd_kv_splits(int B, int H, int Nq, int Nk, int D, int causal);

/*
 * Workspace bytes fa_fwd_kv needs for num_splits ranges:
 * num_splits * B * H * Nq * (D + 1) * 4 when num_splits > 1, else 0
 * (also 0 for non-positive arguments).
 */
size_t fa_fwd_kv_workspace_bytes(int B, int H, int Nq, int D, int num_splits);

/*
 * Block-sparse forward (bf16 in and out, float32 accumulation): fa_fwd
 * restricted to the (query block, key block) pairs a block mask keeps.
 *   q, k, v, o, lse : as fa_fwd ([B][H][N][D] bf16, lse f32 [B][H][N])
 *   block_mask      : DEVICE pointer, uint8 [mask_heads][nb][nb] with
 *                     nb = ceil(N / 64); entry (a, c) != 0 lets query rows
 *                     64a .. 64a+63 see key rows 64c .. 64c+63 (read only).
 *   mask_heads      : 1 (one mask for every batch and head) or B*H (mask
 *                     of head h of batch b at index b*H + h).
 * With causal = 1 a key must also satisfy j <= i.  Key tiles no row of a
 * workgroup may see are never loaded or multiplied: this is the causal
 * tile skip of the "Flash Attention" page's kernel anatomy generalised to
 * any block pattern, the extension the metal-flash-attention README names.
 * A row that sees no key at all gets O = 0 and L = -inf (the pages do not
 * define it; -inf gives such a row weight 0 in any log-sum-exp merge).
 * D in {32, 64, 96, 128, 160, 256}; 1 <= N <= 4096 * 64 (FA_ERR_UNSUPPORTED
 * above); FA_ERR_INVALID_ARG for a null mask or another mask_heads.
 */
int fa_fwd_sparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int D,
                  float scale, int causal, const unsigned char* block_mask, int mask_heads, void* stream);

/*
 * Forward, float32 in and out, float32 arithmetic throughout.  Same
 * arguments and semantics as fa_fwd.  D in {64, 128, 256}; any N >= 1.
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int H, int N, int D,
               float scale, int causal, void* stream);

/*
 * Backward, query side (metal-flash-attention README, "Quantifying
 * performance", backward-query pseudocode).  Computes
 *   delta : f32  [B][H][N]   delta[i] = sum_d dO[i][d] O[i][d]   (written)
 *   dq    : bf16 [B][H][N][D]                                     (written)
 * from q, k, v, o (the forward output), dO (bf16) and lse (the forward's
 * L).  Each workgroup owns a block of query rows and loops over key blocks,
 * so no two workgroups write the same element: no atomics, no workspace.
 * D in {32, 64, 96, 128, 160, 256}; any N >= 1.
 */
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
              float* delta, void* dq, int B, int H, int N, int D, float scale, int causal, void* stream);

/*
 * Backward, key/value side (metal-flash-attention README, "Quantifying
 * performance", backward-key-value pseudocode).  Computes
 *   dk, dv : bf16 [B][H][N][D]   (written)
 * from q, k, v, dO, lse and delta.  delta must be the one fa_bwd_dq wrote:
 * enqueue this call after fa_bwd_dq on the same stream (or otherwise order
 * it after).  Each workgroup owns a block of key rows and loops over query
 * blocks: no atomics, no workspace.  D in {32, 64, 96, 128, 160, 256}; any N >= 1.
 */
int fa_bwd_dkdv(const void* q, const void* k, const void* v, const void* dO, const float* lse, const float* delta,
                void* dk, void* dv, int B, int H, int N, int D, float scale, int causal, void* stream);

/* A static, human-readable string for an FA_* code (never NULL). */
const char* fa_strerror(int code);

/* Library ABI version: (major << 16) | minor. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
