/*
 * parallax.h -- C ABI of the MI355X (gfx950) Parallax attention library.
 *
 * Parallax ("Parallax: Parameterized Local Linear Attention for Language
 * Modeling"; PyPI README, "Quickstart"; neuraltrendhub summary, "What the
 * paper found"; original abstract) keeps the softmax readout of attention
 * and adds a learned probe r, one per query head, whose scores s = r . k
 * read out the key-value covariance. For one query row with visible keys J:
 *
 *   z_j  = qk_scale * <q, k_j>,   w = softmax(z) over J
 *   s_j  = rk_scale * <r, k_j>,   sbar = sum_j w_j s_j
 *   o    = sum_j w_j v_j + sum_j w_j (s_j - sbar) v_j
 *
 * r = 0 gives softmax attention exactly (encorp.ai article, FAQ). The pages
 * print no equation; this is the local-linear intercept of the cere-bro
 * blog's diagram with the solver's output replaced by the probe, and the
 * plus sign is that intercept's. The pages leave the scale of s open:
 * rk_scale = 1 is the plain reading, and the argument keeps the other one
 * expressible.
 *
 * Conventions shared by every entry point:
 *  - Every tensor pointer is a DEVICE pointer; buffers are dense row-major
 *    in the layouts stated below. The caller owns every buffer, including
 *    the decode workspace; the library never allocates or frees memory
 *    (the scratch of parallax_decode_noalloc is a static device array that
 *    comes with the loaded library).
 *  - dtype: PLX_F32 (float) or PLX_BF16 (bfloat16 bits). q, r, k, v and o
 *    share it. Arithmetic is fp32 (bf16 inputs are contracted on matrix
 *    cores with fp32 accumulation); bf16 outputs are rounded to nearest-even.
 *  - Query head h reads KV head h / (Hq / Hkv) (consecutive groups, as
 *    torch's repeat_interleave). The pages show only Hq == Hkv.
 *  - Argument checks are synchronous, host-only, and happen before any
 *    launch: a failing check returns a status and touches no memory.
 *    Launch failures return PLX_ERR_HIP. Work is enqueued on `stream`
 *    (a hipStream_t; NULL is the default stream); nothing synchronises.
 *  - Results do not depend on timing: a fixed split plan and no atomic
 *    accumulation of values (the work-queue counters of packed prefill and
 *    backward batches decide which workgroup computes an item, never how;
 *    masked decode counts visible blocks with integer adds), so repeated
 *    calls return bit-identical outputs.
 *  - Non-finite inputs propagate; they are not checked.
 *  - qk_scale must be finite and > 0, rk_scale finite (else INVALID_ARG).
 *  - window (sliding-window attention; the PyPI README's overview calls it
 *    structurally compatible with Parallax and defines none): 0 = none; W > 0
 *    lets a prefill query i see keys max(0, i - W + 1) .. i, and a decode
 *    query see the last min(n, W) of its sequence's n cached keys. < 0 is
 *    INVALID_ARG.
 *  - block_mask (block-sparse attention; the same overview calls block
 *    sparsity structurally compatible and defines none): NULL = none, else
 *    a DEVICE array of bytes (nonzero = visible) over blocks of
 *    PLX_MASK_BLOCK positions counted from the start of each sequence, one
 *    mask per (sequence, KV head), shared by that KV head's query heads:
 *      decode  [B, Hkv, ceil(kv_len / PLX_MASK_BLOCK)]: byte kb shows key
 *              positions kb*128 .. kb*128 + 127 to the sequence's query;
 *      prefill [B, Hkv, nb, nb], nb = ceil(L / PLX_MASK_BLOCK) (L = max_len
 *              for packed calls): byte [qb][kb] shows key block kb to query
 *              block qb; only kb < qb is read.
 *    It applies on top of causality and the window. A query always sees its
 *    own block (prefill: the diagonal block; decode: the block holding the
 *    sequence's last key), so every row keeps at least one key. Hidden
 *    blocks are neither read nor computed on the matrix-core paths. The
 *    mask is read on the device only and not validated; a backward call must
 *    get the mask its forward call got.
 */
#ifndef PARALLAX_H
#define PARALLAX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PARALLAX_ABI_VERSION 5

/* Block size of block_mask, in positions (keys and prefill queries). */
#define PLX_MASK_BLOCK 128

typedef enum {
    PLX_OK = 0,
    PLX_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, Hq % Hkv != 0 */
    PLX_ERR_UNSUPPORTED = 2, /* valid but not implemented (head_dim, dtype) */
    PLX_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
    PLX_ERR_HIP = 4          /* the HIP runtime reported an error */
} plx_status;

typedef enum {
    PLX_F32 = 0,
    PLX_BF16 = 1,
    /* Not element types: these two make every 32-bit int a value of
     * plx_dtype, so that any code a caller passes is a valid argument and an
     * unknown one is rejected with PLX_ERR_UNSUPPORTED. */
    PLX_DTYPE_RANGE_MIN_ = -0x7fffffff - 1,
    PLX_DTYPE_RANGE_MAX_ = 0x7fffffff
} plx_dtype;

/* PARALLAX_ABI_VERSION of the built library. */
int parallax_abi_version(void);

/* Static, never-NULL description of a status code (any int: values that are
 * no plx_status give "unknown status"). */
const char *parallax_status_string(int status);

/* ------------------------------------------------------------------------
 * Decode: one new query token per sequence against its KV cache (PyPI
 * README, "Decoding (CuTeDSL)": q, r (B, 1, H, D); k, v (B, kv_len, H, D);
 * qk_scale = 1/sqrt(D)). Every cached key of a sequence is visible.
 *
 *   q, r, o : [B, Hq, D]                  (the (B, 1, Hq, D) of the pages)
 *   k, v    : [B, kv_len, Hkv, D]         when cu_seqlens_k == NULL
 *             [cu_seqlens_k[B], Hkv, D]   packed, when cu_seqlens_k != NULL
 *   cu_seqlens_k : NULL, or DEVICE int32 [B + 1], non-decreasing from 0;
 *             sequence b owns tokens cu[b] .. cu[b+1]-1 and its length
 *             must not exceed kv_len (kv_len is the maximum length). A
 *             zero-length sequence yields o = 0. The offsets are not read
 *             on the host, so they are not validated.
 *   B, Hq, Hkv, D, kv_len : sizes, all >= 1; Hq % Hkv == 0; D in {64, 128}.
 *   qk_scale : softmax logit scale (pass 1/sqrt(D) for the pages' default).
 *   rk_scale : probe score scale (1 is the plain reading).
 *   num_splits : 0 lets the library choose how many key ranges (splits)
 *             each sequence is cut into; >= 1 forces that many. With more
 *             than one split the per-split streaming states are written
 *             to the workspace and merged by a second kernel. A packed
 *             cache (cu_seqlens_k != NULL) with num_splits == 0, no window
 *             and the matrix-core path (bf16, D == 128, Hq / Hkv in
 *             1 to 8) is instead cut into equal token ranges per KV
 *             head across all sequences (one range per workgroup), which
 *             balances a mix of lengths.
 *   workspace, workspace_bytes : device scratch of at least
 *             parallax_decode_workspace_bytes(...) bytes for the same
 *             arguments (may be NULL when that size is 0). The size covers
 *             either plan, dense or packed.
 * Returns PLX_OK or an error status.
 * ---------------------------------------------------------------------- */
size_t parallax_decode_workspace_bytes(int B, int Hq, int Hkv, int D, int kv_len, int window,
                                       plx_dtype dtype, int num_splits);

plx_status parallax_decode(const void *q, const void *r, const void *k, const void *v, void *o,
                    const int32_t *cu_seqlens_k, int B, int Hq, int Hkv, int D, int kv_len,
                    int window, const uint8_t *block_mask, float qk_scale, float rk_scale,
                    plx_dtype dtype, int num_splits, void *workspace, size_t workspace_bytes,
                    void *stream);

/* Plain softmax-attention decode on the same kernels and loader with the
 * probe path compiled out: o = sum_j w_j v_j. The baseline against which the
 * cost of the Parallax correction is measured; same layouts and rules as
 * parallax_decode without r and rk_scale. Uses the same workspace size. */
plx_status softmax_decode(const void *q, const void *k, const void *v, void *o,
                   const int32_t *cu_seqlens_k, int B, int Hq, int Hkv, int D, int kv_len,
                   int window, const uint8_t *block_mask, float qk_scale, plx_dtype dtype,
                   int num_splits, void *workspace, size_t workspace_bytes, void *stream);

/* Size of the device workspace that the library itself holds for
 * parallax_decode_noalloc (one copy per device that runs it). */
#define PLX_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)

/* parallax_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, kernels and split plan, with the split records kept
 * in a file-scope device array of PLX_NOALLOC_SCRATCH_BYTES owned by the
 * library instead of a caller workspace. The call allocates nothing; the
 * caller still passes q, r, k, v, o (and cu_seqlens_k, block_mask) as for
 * parallax_decode. The array's device address is looked up on the first call
 * on each device (with that device current); HIP errors of that lookup
 * return PLX_ERR_HIP.
 * Returns PLX_ERR_WORKSPACE, before touching the device, when the records of
 * the plan the call runs need more than PLX_NOALLOC_SCRATCH_BYTES: B * Hq *
 * splits * (2 D + 4) * 4 bytes for the per-sequence split plan (none with one
 * split), Hq * (ranges + B - 1) * (2 D + 4) * 4 bytes for a packed cache's
 * stream-K plan (parallax_decode_workspace_bytes(...) bounds both); other
 * errors as parallax_decode. Every call on one device shares that device's
 * array and keeps the last call's records there, so calls that overlap in
 * time on one device (other streams, other host threads) race and must be
 * serialised by the caller. */
plx_status parallax_decode_noalloc(const void *q, const void *r, const void *k, const void *v, void *o,
                            const int32_t *cu_seqlens_k, int B, int Hq, int Hkv, int D,
                            int kv_len, int window, const uint8_t *block_mask, float qk_scale,
                            float rk_scale, plx_dtype dtype, int num_splits, void *stream);

/* The split count parallax_decode / softmax_decode use for these
 * arguments (num_splits resolved when it is 0), or 0 when they are invalid. */
int parallax_decode_num_splits(int B, int Hq, int Hkv, int D, int kv_len, int window, plx_dtype dtype,
                               int num_splits);

/* ------------------------------------------------------------------------
 * Decode in two halves: the streaming kernel that writes one record per
 * (sequence, query head, split), and the merge of records into o. For the
 * per-sequence split plan parallax_decode is exactly partial + merge (or one
 * fused kernel when the plan has a single split); these two calls always use
 * that plan, also for packed caches. Exposed so that records can be produced where
 * the keys live and merged elsewhere -- e.g. a long sequence whose key
 * range is cut across devices: each device streams its range, the records
 * are gathered, one merge produces o -- and so that each half can be timed.
 *
 * Record layout: records[B][Hq][num_records], each 2*D + 4 floats:
 *   A[D] = sum_j e_j v_j,  B[D] = sum_j e_j (s_j - pi) v_j,
 *   m    = max_j z_j * log2(e)   (z_j = qk_scale q.k_j; -inf: empty record),
 *   l    = sum_j e_j,  S = sum_j e_j (s_j - pi),  pi,
 * with e_j = 2^(z_j log2(e) - m) and pi the pivot the record's probe terms
 * are taken against (the streaming kernel keeps it near the running weighted
 * mean of s, which keeps the bf16 rounding of the probe terms small; any
 * value is valid). Merging re-bases every record onto one pivot (exact in
 * real arithmetic), so records from different calls combine.
 * ---------------------------------------------------------------------- */

/* Bytes of a records array for (B, Hq, D, num_records); 0 if invalid. */
size_t parallax_decode_record_bytes(int B, int Hq, int D, int num_records);

/* Streaming half of parallax_decode: same arguments and layouts, but writes
 * parallax_decode_num_splits(...) records per (b, h) into `records`
 * (DEVICE, at least parallax_decode_record_bytes(B, Hq, D, that count)
 * bytes) instead of o. r == NULL selects the softmax baseline (the probe
 * terms of the records are then zero). Returns PLX_ERR_WORKSPACE when
 * `records` is NULL or too small. */
plx_status parallax_decode_partial(const void *q, const void *r, const void *k, const void *v,
                            const int32_t *cu_seqlens_k, int B, int Hq, int Hkv, int D, int kv_len,
                            int window, const uint8_t *block_mask, float qk_scale,
                            float rk_scale, plx_dtype dtype, int num_splits, void *records,
                            size_t records_bytes, void *stream);

/* Merge records[B][Hq][num_records] (DEVICE) into o [B, Hq, D] (DEVICE,
 * dtype): o = (A + B - (S / l) A) / l over the combined state, or A / l
 * when with_probe == 0. Empty records are skipped; a row with none gets
 * o = 0. D in {64, 128}. */
plx_status parallax_decode_merge(const void *records, void *o, int B, int Hq, int D, int num_records,
                          plx_dtype dtype, int with_probe, void *stream);

/* ------------------------------------------------------------------------
 * Causal prefill / training forward (PyPI README, "Training (Triton)":
 * parallax_func(q, r, k, v) on (B, H, L, D) tensors, causal, returns
 * (B, H, L, D)). Query row i sees keys 0 .. i.
 *
 *   q, r, o : [B, Hq, L, D]
 *   k, v    : [B, Hkv, L, D]
 *   lse     : NULL or DEVICE float [B, Hq, L]: m + ln(sum_j exp(z_j - m))
 *   sbar    : NULL or DEVICE float [B, Hq, L]: sum_j w_j s_j
 *   vbar    : NULL or DEVICE [B, Hq, L, D] in dtype: the softmax readout
 *             sum_j w_j v_j (o without the correction)
 *             (statistics for a backward pass; not on the pages. With vbar
 *             the backward skips one of its two sweeps over the keys, at the
 *             cost of one more o-sized activation)
 *   D == 128 and dtype == PLX_BF16 run on bf16 MFMA with fp32 accumulation;
 *   other D in {64, 128} and PLX_F32 run on a plain fp32 kernel. L <= 2^22.
 * ---------------------------------------------------------------------- */
plx_status parallax_prefill(const void *q, const void *r, const void *k, const void *v, void *o,
                     float *lse, float *sbar, void *vbar, int B, int Hq, int Hkv, int L, int D,
                     int window, const uint8_t *block_mask, float qk_scale, float rk_scale,
                     plx_dtype dtype, void *stream);

/* ------------------------------------------------------------------------
 * Backward of the causal prefill (PyPI README, "Training (Triton)": the
 * output of parallax_func is differentiated with autograd; its "Helion"
 * section holds the four gradients to the same tolerance as the output).
 * Given d_o = dLoss/do, writes dq, dr, dk, dv for the forward
 *   o_i = sum_{j<=i} w_ij (1 + s_ij - sbar_i) v_j,
 *   w_i = softmax_j(qk_scale q_i.k_j), s_ij = rk_scale r_i.k_j.
 * The attention weights are recomputed from the forward's lse; nothing of
 * size L x L is stored.
 *
 *   q, r, o, d_o, dq, dr : [B, Hq, L, D]
 *   k, v, dk, dv         : [B, Hkv, L, D]     (dk, dv sum over the Hq / Hkv
 *                                              query heads of each KV head)
 *   lse, sbar : DEVICE float [B, Hq, L], as written by parallax_prefill for
 *               the same q, r, k, v, window, scales and dtype; o likewise.
 *   vbar      : NULL, or the vbar that forward call wrote.
 *   workspace, workspace_bytes : DEVICE scratch of at least
 *               parallax_prefill_backward_workspace_bytes(B, Hq, L) bytes
 *               (16 bytes per query row).
 *   Sizes, dtype and kernel choice as parallax_prefill (bf16 with D == 128
 *   on MFMA); L <= 2^22. Gradients are written in dtype, computed in fp32.
 * ---------------------------------------------------------------------- */
size_t parallax_prefill_backward_workspace_bytes(int B, int Hq, int L);

plx_status parallax_prefill_backward(const void *q, const void *r, const void *k, const void *v,
                              const void *o, const void *d_o, const float *lse,
                              const float *sbar, const void *vbar, void *dq, void *dr, void *dk,
                              void *dv, int B, int Hq, int Hkv, int L, int D, int window,
                              const uint8_t *block_mask, float qk_scale, float rk_scale,
                              plx_dtype dtype, void *workspace, size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Packed-sequence (varlen) prefill and its backward (the pages name
 * parallax_varlen_func next to parallax_func in the PyPI README's API
 * listing): a batch of B sequences of different lengths stored back to back,
 * each an independent causal prefill (with the optional window).
 *
 *   q, r, o, d_o, dq, dr : [total_tokens, Hq, D]
 *   k, v, dk, dv         : [total_tokens, Hkv, D]
 *   lse, sbar            : NULL (forward only) or DEVICE float [total_tokens, Hq]
 *   vbar                 : NULL or DEVICE [total_tokens, Hq, D], as in the dense calls
 *   cu_seqlens : DEVICE int32 [B + 1], non-decreasing from 0 to total_tokens;
 *                sequence b owns tokens cu[b] .. cu[b+1] - 1. Read on the device
 *                only, so not validated: lengths must not exceed max_len.
 *   max_len    : the longest sequence (sizes the launch grid), >= 1.
 *   workspace, workspace_bytes : DEVICE scratch of at least
 *                parallax_prefill_varlen_workspace_bytes(Hq, total_tokens, 0)
 *                bytes for the forward, (..., 1) for the backward: the work
 *                queue counters of the persistent launch (cleared by the call
 *                itself) and, for the backward, 16 bytes per query row.
 *                Calls that share a workspace must not overlap in time.
 * Other arguments, rules and errors as the dense calls; total_tokens == 0
 * (every sequence empty) returns PLX_OK without a launch. max_len times
 * max(Hq, Hkv) * D * element size must stay below 2^31 bytes.
 * ---------------------------------------------------------------------- */
size_t parallax_prefill_varlen_workspace_bytes(int Hq, int total_tokens, int backward);

plx_status parallax_prefill_varlen(const void *q, const void *r, const void *k, const void *v, void *o,
                            float *lse, float *sbar, void *vbar, const int32_t *cu_seqlens, int B,
                            int Hq, int Hkv, int max_len, int total_tokens, int D, int window,
                            const uint8_t *block_mask, float qk_scale, float rk_scale, plx_dtype dtype,
                            void *workspace, size_t workspace_bytes, void *stream);

plx_status parallax_prefill_varlen_backward(const void *q, const void *r, const void *k, const void *v,
                                     const void *o, const void *d_o, const float *lse,
                                     const float *sbar, const void *vbar,
                                     const int32_t *cu_seqlens, void *dq, void *dr, void *dk,
                                     void *dv, int B, int Hq, int Hkv,
                                     int max_len, int total_tokens, int D, int window,
                                     const uint8_t *block_mask, float qk_scale, float rk_scale,
                                     plx_dtype dtype, void *workspace, size_t workspace_bytes,
                                     void *stream);

#ifdef __cplusplus
}
#endif

#endif /* PARALLAX_H */
