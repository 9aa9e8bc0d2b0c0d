/*
 * fa.h -- C ABI of the exact IO-aware attention library for MI355X (gfx950).
 *
 * The operation is exact scaled-dot-product attention,
 *     O = softmax(scale * Q K^T [+ causal mask]) V,
 * the formula displayed in the problem section of the page "FlashAttention
 * (EL)".  It is computed tile by tile with an online softmax (running maximum
 * and running sum of exponentials: same page, section on online softmax;
 * "Flash Attention: Ako transformery zvladaju miliony tokenov", section 2), so
 * the N x N score matrix never reaches device memory.  The backward pass
 * recomputes the scores from a saved per-row log-sum-exp instead of storing
 * them ("Flash Attention uitgelegd", section "Recomputation").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or synchronises, and keeps no per-call
 *    state; it enqueues kernels on `stream` and returns at once.  `stream` is
 *    a hipStream_t passed as void* (so that this header needs no HIP
 *    include); NULL is the default stream.
 *  - Tensors are dense, row-major, [B, H, N, d] (d fastest).  LSE tensors
 *    are [B, H, N] float32 and hold the natural-log log-sum-exp of the
 *    scaled, masked scores of each query row.
 *  - Grouped-query attention: every entry point takes Hkv, the number of K/V
 *    heads, after H.  Hkv must divide H (FA_ERR_ARG otherwise); query head h
 *    uses K/V head h / (H/Hkv).  Hkv = H is ordinary multi-head attention,
 *    Hkv = 1 multi-query attention.
 *  - `scale` multiplies Q K^T; the pages' value is 1/sqrt(d).  It must be
 *    finite and > 0 (FA_ERR_ARG otherwise).
 *  - Causal masking (the decoder-only variant: Slovak page, section 5, and
 *    its is_causal usage example in section 6): key j is visible to query i
 *    iff j <= i (top-left aligned).
 *  - Head dimension: d in {64, 128} for every entry point; d = 256 also for
 *    the bf16 fa_fwd, fa_bwd, fa_decode, fa_decode_noalloc and fa_decode_paged
 *    (not for fp32 inputs or fa_fwd_fp8).  Other values return
 *    FA_ERR_UNSUPPORTED.
 *  - Any N >= 1 (ragged tails are masked inside the kernels); all offsets
 *    are 64-bit.
 *  - Every pointer must be 16-byte aligned.
 *  - Errors: arguments are validated before anything is enqueued; on error
 *    nothing is launched and the status says why.  A failed launch returns
 *    FA_ERR_HIP.  Kernel faults surface at the caller's next synchronisation,
 *    as for any asynchronous HIP call.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_NULL = 1,        /* a required pointer is NULL                      */
    FA_ERR_ARG = 2,         /* a size is < 1, Hkv does not divide H, or scale
                               is not finite and positive                      */
    FA_ERR_UNSUPPORTED = 3, /* a dtype / head-dim combination not built, or a
                               bf16 head too large (N*d*2 >= 2^32 bytes)       */
    FA_ERR_ALIGN = 4,       /* a pointer is not 16-byte aligned                */
    FA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required      */
    FA_ERR_HIP = 6,         /* the HIP runtime reported an error at launch     */
    FA_ERR_SCRATCH_LIMIT = 7 /* fa_decode_noalloc: the call needs more scratch
                               than FA_NOALLOC_SCRATCH_BYTES                   */
} fa_status_t;

/* Size of the static device scratch array behind fa_decode_noalloc (16 MiB
 * per GPU the library runs on, held until the process ends). */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

typedef enum {
    FA_FP32 = 0,            /* IEEE binary32                                   */
    FA_BF16 = 1             /* bfloat16 (rounded to nearest even on output)    */
} fa_dtype_t;

/*
 * fa_fwd -- forward pass: O and the per-row LSE.
 *
 * Computes O = softmax(scale Q K^T [causal]) V and LSE_i = ln sum_j
 * exp(scale q_i.k_j) over visible j ("FlashAttention (EL)", displayed formula
 * of the problem section; all operations fused in one kernel as its section
 * on fusing operations describes).  Uses no workspace: memory beyond the
 * outputs is O(1) in N.
 *
 *   q         [B,H,N,d] of in_dtype (FA_BF16: bf16 MFMA with fp32
 *             accumulation; FA_FP32: fp32 MFMA).
 *   k, v      [B,Hkv,N,d] of in_dtype.  Hkv divides H; query head h attends
 *             with K/V head h / (H/Hkv) -- grouped-query attention, which the
 *             Slovak page (section 5) and the Greek page (FlashAttention-2
 *             section, multi-query) name; Hkv = 1 is multi-query and Hkv = H
 *             ordinary multi-head attention.
 *   o         [B,H,N,d] of o_dtype.  in_dtype FA_BF16 allows o_dtype FA_BF16
 *             or FA_FP32; in_dtype FA_FP32 requires o_dtype FA_FP32.
 *   lse       [B,H,N] float32, natural log; never NULL (backward needs it).
 *
 * With in_dtype FA_BF16 one head's K (and V) must span fewer than 2^32 bytes
 * (N*d*2 < 2^32, i.e. N < 2^24 at d = 128): the kernels address a head
 * with 32-bit offsets.  Larger heads return FA_ERR_UNSUPPORTED.
 */
fa_status_t fa_fwd(const void* q, const void* k, const void* v,
                   void* o, fa_dtype_t o_dtype, float* lse,
                   int B, int H, int Hkv, int N, int d, fa_dtype_t in_dtype,
                   int causal, float scale, void* stream);

/*
 * fa_fwd_fp8 -- forward pass on fp8 inputs (the FP8 variant of FlashAttention
 * named on "Flash Attention uitgelegd", FA3 section; gfx950's e4m3 matrix
 * products run at twice the bf16 rate).  Computes the same O and LSE as
 * fa_fwd for the real-valued inputs Q = q_scale * q, K = k_scale * k,
 * V = v_scale * v.
 *
 *   q         [B,H,N,d] e4m3 (OCP FP8 E4M3: 1 sign, 4 exponent, 3 mantissa
 *             bits, bias 7, largest finite 448, no infinities; one byte each).
 *   k         [B,Hkv,N,d] e4m3, grouped as for fa_fwd.
 *   vt        V transposed: [B,Hkv,d,N] e4m3 (for each head, d rows of N keys).
 *   q_scale, k_scale, v_scale   per-tensor dequantisation factors, finite and
 *             > 0 (else FA_ERR_ARG).
 *   o         [B,H,N,d], o_dtype FA_BF16 or FA_FP32.
 *   lse       [B,H,N] float32, natural log.
 *
 * Arithmetic: S accumulates exact e4m3 products in fp32.  The probabilities
 * are taken against a reference max that is the running row max rounded up
 * to an integer in base-2 units (so each is at most 1), multiplied by 2^8 and
 * rounded to e4m3 (nearest even) for the second product; that rounding (3
 * mantissa bits, relative error at most 2^-4) is the only approximation
 * beyond fp32 accumulation.  The row sum and the LSE use the unrounded
 * values.  Uses no workspace.
 *
 * d must be 64 or 128 (else FA_ERR_UNSUPPORTED); any N >= 1, the ragged tail
 * masked as in fa_fwd.  The inputs must be finite (no e4m3 NaN codes): keys
 * past N of a ragged last tile may read the next row of vt, which is then
 * weighted by exactly zero.  All pointers 16-byte aligned.
 */
fa_status_t fa_fwd_fp8(const void* q, const void* k, const void* vt,
                       float q_scale, float k_scale, float v_scale,
                       void* o, fa_dtype_t o_dtype, float* lse,
                       int B, int H, int Hkv, int N, int d,
                       int causal, float scale, void* stream);

/*
 * fa_bwd_workspace_bytes -- bytes of workspace fa_bwd needs for this shape:
 * the fp32 row statistic D = rowsum(dO * O), [B,H,N], and the LSE in base-2
 * units (LSE log2 e), [B,H,N] fp32, each padded to 256 bytes.
 * With grouped heads (Hkv < H) and fewer than 512 (K/V head, 128-key tile)
 * pairs, fa_bwd splits the G = H/Hkv query heads of a K/V head into groups of
 * s, each with dK/dV workgroups of its own: s is the largest divisor of G
 * below G that gives at least 512 workgroups (1 if none does).  The workspace
 * then also holds their fp32 partial dK and dV, [B*H/s, N, d] each, summed
 * over the groups by a second kernel.  Returns 0 if a size is < 1, Hkv does
 * not divide H or the total overflows.
 */
size_t fa_bwd_workspace_bytes(int B, int H, int Hkv, int N, int d);

/*
 * fa_bwd -- backward pass with recomputation ("Flash Attention uitgelegd",
 * section "Recomputation"; Slovak page, section 2): the scores and
 * probabilities are recomputed tile by tile from Q, K and the saved LSE; the
 * gradients are the chain rule through the forward definition:
 *     dV = P^T dO,  dP = dO V^T,  D_i = sum_k dO_ik O_ik,
 *     dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *
 *   q, dout        [B,H,N,d] bf16 (in_dtype must be FA_BF16).
 *   k, v           [B,Hkv,N,d] bf16, grouped as for fa_fwd.
 *   o              [B,H,N,d] of o_dtype (FA_BF16 or FA_FP32), from fa_fwd.
 *   lse            [B,H,N] float32, from fa_fwd with the same causal/scale.
 *   dq             [B,H,N,d] bf16 output.
 *   dk, dv         [B,Hkv,N,d] bf16 outputs; a shared K/V head receives the
 *                  sum over the H/Hkv query heads that use it.  fp32
 *                  accumulation inside; no atomics, so the results are
 *                  bitwise reproducible.
 *   workspace      device memory of at least fa_bwd_workspace_bytes(B, H,
 *                  Hkv, N, d), 16-byte aligned; its contents on entry do not
 *                  matter and are clobbered.
 *
 * As for fa_fwd, N*d*2 must be below 2^32 bytes (else FA_ERR_UNSUPPORTED).
 */
fa_status_t fa_bwd(const void* q, const void* k, const void* v,
                   const void* o, fa_dtype_t o_dtype, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes,
                   int B, int H, int Hkv, int N, int d, fa_dtype_t in_dtype,
                   int causal, float scale, void* stream);

/*
 * fa_decode_num_splits -- the split count fa_decode uses when called with
 * num_splits = 0 for this shape (always >= 1 and <= L); fa_decode_paged
 * makes the same choice for L = max_pages_per_seq * page_size.
 */
int fa_decode_num_splits(int B, int H, int Hkv, int L, int d);

/*
 * fa_decode_workspace_bytes -- workspace of fa_decode and fa_decode_paged:
 * fp32 partial outputs [B,H,S,d] and partial LSEs [B,H,S] for S splits
 * (num_splits = 0: room for the library's own choice, which is the same for
 * both calls).  Returns 0 if a size is < 1.
 */
size_t fa_decode_workspace_bytes(int B, int H, int Hkv, int L, int d, int num_splits);

/*
 * fa_decode -- one generation step against a KV cache (the cache the
 * attention-backend page describes): one query token per (b, h) attends to
 * all L cached keys, no mask.  The cache is cut into S contiguous chunks;
 * each chunk's (o_s, lse_s) is computed with the online softmax and the
 * chunks are merged with the same max-and-rescale rule applied to whole
 * chunks:  M = max_s lse_s,  lse = M + ln sum_s exp(lse_s - M),
 *          O = sum_s exp(lse_s - lse) o_s.
 *
 *   q                 [B,H,1,d] bf16 (dtype must be FA_BF16).
 *   k_cache, v_cache  [B,Hkv,L,d] bf16, contiguous; query head h reads cache
 *                     head h / (H/Hkv) (grouped-query attention, as for fa_fwd).
 *   o                 [B,H,1,d] bf16 output.
 *   lse               [B,H] float32 output, or NULL if not wanted.
 *   workspace         at least fa_decode_workspace_bytes(B,H,Hkv,L,d,num_splits).
 *   num_splits        0 = library's choice, else 1..L.
 */
fa_status_t fa_decode(const void* q, const void* k_cache, const void* v_cache,
                      void* o, float* lse,
                      void* workspace, size_t workspace_bytes,
                      int B, int H, int Hkv, int L, int d, fa_dtype_t dtype,
                      int num_splits, float scale, void* stream);

/*
 * fa_decode_noalloc -- fa_decode without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  It computes exactly what fa_decode
 * computes with the same num_splits, and allocates nothing: the per-chunk
 * partials (o_s, lse_s) go to a static device array of
 * FA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on.
 *
 *   q, k_cache, v_cache, o, lse, B, H, Hkv, L, d, dtype, num_splits, scale,
 *   stream            as for fa_decode.  The pointers and the stream must
 *                     belong to the device current on the calling thread.
 *
 * Limit: the call's partials, 4*B*H*S*(d+1) bytes for S splits (plus padding
 * to 256 bytes), must fit FA_NOALLOC_SCRATCH_BYTES; every call with
 * fa_decode_workspace_bytes(B, H, Hkv, L, d, num_splits) <= that size does.
 * Larger calls return FA_ERR_SCRATCH_LIMIT and launch nothing (a smaller
 * num_splits shrinks the need).  Other errors as for fa_decode; FA_ERR_HIP if
 * the scratch array's device address cannot be looked up.
 *
 * The array is shared by every call on one GPU and keeps the last call's
 * contents (every partial is written before it is read, so nothing needs
 * clearing).  Calls that overlap in time on one GPU race on it: issue them on
 * one stream, or order them.
 */
fa_status_t fa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              void* o, float* lse,
                              int B, int H, int Hkv, int L, int d, fa_dtype_t dtype,
                              int num_splits, float scale, void* stream);

/*
 * fa_decode_paged -- fa_decode against a paged KV cache.  The attention-backend
 * page (sections "Wat is het precies?" and "Voorbeelden uit de praktijk")
 * describes PagedAttention: the cache is cut into small blocks allocated from a
 * pool rather than one contiguous reservation, with the same result.  Here a
 * page holds page_size consecutive tokens of every K/V head, and sequence b
 * lists its pages in token order in row b of a block table.  The result is
 * fa_decode over the first seq_lens[b] tokens of that page sequence; a length
 * of 0 gives O = 0 and LSE = -inf.
 *
 *   q                 [B,H,1,d] bf16.
 *   k_pool, v_pool    [num_pages, Hkv, page_size, d] bf16 (page p of head h is
 *                     the contiguous block k_pool[p][h]).
 *   block_table       [B, max_pages_per_seq] int32, device memory: page indices
 *                     in [0, num_pages).  Entries past a sequence's last page
 *                     are not read.  Keys on a page index outside the pool are
 *                     skipped (treated as absent) rather than read.
 *   seq_lens          [B] int32, device memory; values are clamped to
 *                     [0, max_pages_per_seq * page_size].
 *   o, lse            as for fa_decode (lse may be NULL).
 *   workspace         at least fa_decode_workspace_bytes(B, H, Hkv,
 *                     max_pages_per_seq * page_size, d, num_splits).
 *   page_size         a power of two, 32 .. 65536.
 *   num_splits        0 = library's choice for that maximal length, else
 *                     1 .. max_pages_per_seq * page_size.
 *
 * Errors: FA_ERR_NULL for a missing pointer (lse excepted); FA_ERR_ARG for
 * sizes < 1, a page size that is not a power of two in range, Hkv not
 * dividing H, a bad scale or split count; FA_ERR_ALIGN for q, pools, o, lse or
 * workspace not 16-byte aligned or the int32 arrays not 4-byte aligned.
 */
fa_status_t fa_decode_paged(const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens,
                            void* o, float* lse,
                            void* workspace, size_t workspace_bytes,
                            int B, int H, int Hkv, int num_pages, int page_size,
                            int max_pages_per_seq, int d, fa_dtype_t dtype,
                            int num_splits, float scale, void* stream);

/* fa_status_string -- a static, human-readable name for a status code. */
const char* fa_status_string(fa_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
