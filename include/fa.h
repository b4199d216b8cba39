/*
 * fa.h - exact tiled attention on AMD Instinct MI355X (gfx950), C ABI.
 *
 * What is computed.  For every batch b and query head hq, with the key/value
 * head kv = hq / (Hq / Hkv):
 *
 *     S   = scale * Q[b,hq] K[b,kv]^T                  (never stored)
 *     P   = softmax(S) row by row, over visible keys
 *     O   = P V[b,kv]
 *     lse = natural log of sum_j exp(S[i,j]) over visible keys j
 *
 * This is the attention of "Fast Inference and Training at Scale", section
 * 6.21 FlashAttention, computed the way that section and "Week 13. GPUs and
 * FlashAttention", Step 2, describe: Q is split into row blocks, K and V into
 * column blocks staged through on-chip memory, and a running maximum and
 * running sum per row (the online softmax of "Hardware Co-Design") stitch the
 * blocks together, so the S x S score matrix never reaches HBM.  Grouped
 * query heads follow section 6.2 (contiguous groups), the paged cache follows
 * section 6.3, and the single-token decode step follows section 6.1.
 *
 * Causal masking is bottom-right aligned: key j is visible to query i iff
 * j <= i + (Sk - Sq).  A query row with no visible key gets O = 0 and
 * lse = -inf (never NaN).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates, frees and synchronises nothing; work is enqueued on
 *     `stream` (a hipStream_t passed as void*; NULL is the default stream)
 *     and the call returns without waiting for it.
 *   - Tensors are contiguous, row-major, last dimension innermost, and
 *     16-byte aligned.
 *   - Arguments are validated on the host before anything is launched; a
 *     non-zero status means nothing was enqueued (except FA_ERR_HIP, which
 *     reports a launch failure).  No C++ exception crosses this boundary.
 *   - The library keeps no global mutable state; calls are re-entrant and
 *     calls on different streams may overlap.
 */
#ifndef EXACT_TILED_ATTENTION_FA_H
#define EXACT_TILED_ATTENTION_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1,   /* null pointer, bad size, misalignment, scale not finite and > 0 */
    FA_ERR_UNSUPPORTED = -2,   /* valid request outside the built kernel set (head dim, dtype, page size) */
    FA_ERR_WORKSPACE = -3,     /* workspace missing, misaligned or smaller than the matching *_workspace_size() */
    FA_ERR_HIP = -4            /* the HIP runtime reported an error at launch */
} fa_status;

typedef enum {
    FA_BF16 = 0,               /* q, k, v, o are bfloat16; arithmetic accumulates in fp32 */
    FA_F32 = 1                 /* q, k, v, o are fp32 */
} fa_dtype;

/*
 * fa_fwd - prefill / full-sequence attention forward.
 *
 * Passage: "Fast Inference and Training at Scale", section 6.21 (definition,
 * tiling, online softmax); "Week 13. GPUs and FlashAttention", Step 2
 * (per-row m and running sum, logsumexp stored per row, causal blocks above
 * the diagonal skipped); "FlashAttention scaling, multi-GPU training and
 * weight quantization", section 1 (division by the running sum postponed to
 * the end; outer loop over Q blocks, parallel over the sequence).
 *
 *   q    [B, Hq,  Sq, d]   dtype        (read)
 *   k    [B, Hkv, Sk, d]   dtype        (read)
 *   v    [B, Hkv, Sk, d]   dtype        (read)
 *   o    [B, Hq,  Sq, d]   dtype        (written)
 *   lse  [B, Hq,  Sq]      fp32         (written; may be NULL to skip)
 *   B, Hq, Hkv, Sq, Sk >= 1, Hq % Hkv == 0; causal is 0 or 1; scale finite
 *   and > 0 (the usual choice is 1/sqrt(d)).
 *   Supported head dims: d in {64, 128} for FA_BF16, d in {32, 64, 128} for
 *   FA_F32; anything else returns FA_ERR_UNSUPPORTED.
 *   Index arithmetic is 64-bit; every tensor may exceed 2^31 elements.
 *
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale,
           int dtype, void* stream);

/*
 * fa_bwd_workspace_size - bytes of scratch that fa_bwd needs: one fp32 per
 * query row (the row sums D = rowsum(dO * O)), rounded up to 256 bytes.
 * Returns 0 for sizes fa_bwd would reject.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Sq);

/*
 * fa_bwd - attention backward: gradients of sum(dout * o) with respect to
 * q, k and v, where o = softmax(scale q k^T) v as computed by fa_fwd.
 *
 * Passage: "Fast Inference and Training at Scale", section 6.21, Idea 2
 * (the backward pass recomputes the probabilities block by block instead of
 * loading them); "Week 13. GPUs and FlashAttention", Step 2 (only O and the
 * per-row logsumexp are kept from the forward).  The probabilities are
 * P = exp(scale q k^T - lse) from the stored lse, and
 * dv = P^T dout, dS = P * (dout v^T - rowsum(dout * o)),
 * dq = scale dS k, dk = scale dS^T q; under grouped-query attention dk and
 * dv of a K/V head sum over its Hq/Hkv query heads.
 *
 *   q, o, dout  [B, Hq,  Sq, d]   bf16   (read)
 *   k, v        [B, Hkv, Sk, d]   bf16   (read)
 *   lse         [B, Hq,  Sq]      fp32   (read; natural log, as fa_fwd writes it;
 *                                        -inf marks a row with no visible key)
 *   dq          [B, Hq,  Sq, d]   bf16   (written)
 *   dk, dv      [B, Hkv, Sk, d]   bf16   (written)
 *   workspace   caller-owned device scratch of at least
 *               fa_bwd_workspace_size(B, Hq, Sq) bytes, 256-byte aligned
 *
 *   Sizes, causal and scale as for fa_fwd (bottom-right causal alignment).
 *   Supported: d == 128; anything else returns FA_ERR_UNSUPPORTED.  All
 *   tensor pointers 16-byte aligned, lse 4-byte aligned.  dq, dk, dv must
 *   not overlap the inputs.  Deterministic: no atomics.
 *
 * Returns FA_OK or a negative fa_status.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq,
           int Sk, int d, int causal, float scale, void* workspace, size_t workspace_bytes,
           void* stream);

/*
 * fa_decode_workspace_size - bytes of scratch that fa_decode needs.
 *
 * The decode step splits every sequence's cache into ranges, attends to each
 * range on its own, and merges the per-range results with their log-sum-exp
 * (the online-softmax update of "Hardware Co-Design" applied to whole
 * ranges).  The scratch holds the per-range partial outputs and lse values.
 * Returns 0 for arguments fa_decode would reject.
 */
size_t fa_decode_workspace_size(int nseq, int Hq, int Hkv, int d, int block_size,
                                int max_blocks_per_seq);

/*
 * fa_decode - one new query token per sequence attending to a paged KV cache.
 *
 * Passage: "Fast Inference and Training at Scale", section 6.1 (the new
 * token's query attends over the whole cache, which already holds its own
 * K and V), section 6.2 (Hq/Hkv query heads share one K/V head), section 6.3
 * (fixed-size blocks, non-contiguous, found through a page table).
 *
 *   q            [nseq, Hq, d]                        bf16   (read)
 *   kcache       [num_blocks, Hkv, block_size, d]     bf16   (read)
 *   vcache       [num_blocks, Hkv, block_size, d]     bf16   (read)
 *   block_table  [nseq, max_blocks_per_seq]           int32  (read) physical
 *                block of each logical block; entries past a sequence's
 *                last block are never read
 *   seqlens      [nseq]                               int32  (read) cached
 *                tokens per sequence, all of them visible
 *   o            [nseq, Hq, d]                        bf16   (written)
 *   lse          [nseq, Hq]                           fp32   (written; may be NULL)
 *   workspace    caller-owned device scratch of at least
 *                fa_decode_workspace_size(...) bytes, 256-byte aligned
 *
 *   num_blocks   physical blocks in each cache (>= 1); scale finite and > 0.
 *   Supported: d == 128, block_size == 16, Hq / Hkv in {1, 2, 4, 8},
 *   nseq and Hkv <= 65535.
 *   Device-side values are made safe by the kernels rather than trusted:
 *   a sequence length is clamped to [0, max_blocks_per_seq * block_size]; a
 *   block id outside [0, num_blocks) contributes no key (its tokens are
 *   treated as masked).  Slots of a last, partly filled block past the
 *   sequence length are never used, even when they hold NaN.  A sequence of
 *   length 0 gets o = 0 and lse = -inf.
 *
 * Returns FA_OK or a negative fa_status.
 */
int fa_decode(const void* q, const void* kcache, const void* vcache,
              const int32_t* block_table, const int32_t* seqlens, void* o, float* lse,
              int nseq, int Hq, int Hkv, int d, int block_size, int max_blocks_per_seq,
              int num_blocks, float scale, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * fa_time_next_call - kernel-boundary timing of the next call on this thread.
 *
 * Measurement hook, not part of any attention computation.  start_event and
 * stop_event are hipEvent_t handles (created by the caller with timing
 * enabled; the library does not own them), both non-NULL, or both NULL to
 * clear.  The next fa_fwd, fa_bwd or fa_decode call made on the same host
 * thread launches its kernels with these events attached
 * (hipExtLaunchKernel): start_event records when the call's first kernel
 * begins executing and stop_event when its last kernel ends, so the elapsed
 * time between them is the call's GPU time without the stream markers that a
 * separate hipEventRecord pair adds.  That call clears the setting when it
 * returns, whatever its status; a call that fails validation records neither
 * event.
 *
 * Returns FA_OK, or FA_ERR_INVALID_ARG when exactly one handle is NULL.
 */
int fa_time_next_call(void* start_event, void* stop_event);

/* fa_status_string - a static, human-readable name for a status code. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_TILED_ATTENTION_FA_H */
