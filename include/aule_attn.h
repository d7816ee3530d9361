/*
 * aule_attn — tiled scaled-dot-product attention forward for AMD Instinct MI355X (gfx950).
 *
 * Computes  O = softmax(scale * Q K^T + causal mask) V  without materialising the
 * [seqlen_q x seqlen_k] score matrix: K/V are streamed tile by tile and the softmax is kept
 * online as a running row max and row sum. This is the FlashAttention forward described in
 * the xxqk.cn article "Attention算子实战：从CUDA优化到昇腾/CANN部署" (section 2.2: Q split
 * into BLOCK_M tiles, K/V into BLOCK_N tiles, stable softmax with max subtraction kept in
 * registers, partial results multiplied into V and accumulated, only O written back) and in
 * the online-softmax practice of the FlashAttention-T commentary (ai-stack.site,
 * "FlashAttention-T：张量化注意力机制优化方案", best practices 4 and 5: running max_score and
 * sum_exp, fp32 reductions, fp16/bf16 matrix products).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, owned by the caller. The library allocates
 *     nothing, keeps no state between calls and is reentrant. O must not overlap an input.
 *   - Every call is asynchronous on `stream` (0 = the null stream). The library never
 *     synchronises and never reads device memory on the host (cu_seqlens included).
 *   - On any error a status other than AULE_OK is returned synchronously and no kernel is
 *     launched; aule_last_error() then describes the failure for the calling thread.
 *   - Tensor data pointers must be 16-byte aligned (the kernels use 128-bit accesses).
 *   - dtype selects the element type of Q, K, V and O alike: fp32, fp16 or bf16. Products
 *     and softmax statistics are accumulated in fp32; O is rounded to dtype
 *     round-to-nearest-even.
 */
#ifndef AULE_ATTN_H
#define AULE_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    AULE_DTYPE_F32 = 0,
    AULE_DTYPE_F16 = 1,
    AULE_DTYPE_BF16 = 2
} aule_dtype_t;

typedef enum {
    AULE_OK = 0,
    AULE_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, misaligned or overlapping buffer, non-finite scale */
    AULE_ERR_UNSUPPORTED = 2,      /* head_dim > 128 or not a multiple of 8, causal with seqlen_q != seqlen_k, unknown dtype,
                                      a 16-bit (sequence, head) slice of 1 GiB or more */
    AULE_ERR_HIP = 3               /* the HIP runtime reported an error at launch */
} aule_status_t;

/*
 * Dense / grouped-query attention forward.
 *
 * Operation: the [batch, heads, seq_len, head_dim] attention of the Aule-Attention API
 * (jeff.news article "AMD GPU에서도 동작하는 FlashAttention 구현체, Aule-Attention", API
 * bullets): fp16/bf16/fp32, head_dim up to 128, heads_q a multiple of heads_kv. Query head
 * hq reads key/value head hq / (heads_q / heads_kv) — K/V repeated in place, as in the GQA
 * (32 query / 8 kv heads) and MQA (one kv head) examples of the jdon.com Aule-Attention
 * article.
 *
 *   q : [batch, heads_q,  seqlen_q, head_dim]  contiguous, dtype
 *   k : [batch, heads_kv, seqlen_k, head_dim]  contiguous, dtype
 *   v : [batch, heads_kv, seqlen_k, head_dim]  contiguous, dtype
 *   o : [batch, heads_q,  seqlen_q, head_dim]  contiguous, dtype (written)
 *   causal : nonzero masks key j for query i when j > i (needs seqlen_q == seqlen_k)
 *   scale  : multiplies Q K^T before the softmax; any finite value (1/sqrt(head_dim) is
 *            the usual choice, 0 gives the mean of the visible V rows)
 *
 * batch == 0 or seqlen_q == 0 is an empty problem: AULE_OK, nothing launched, pointers not
 * inspected. Otherwise heads_q, heads_kv, seqlen_k >= 1 and heads_q % heads_kv == 0
 * (AULE_ERR_INVALID_ARGUMENT); 8 <= head_dim <= 128 with head_dim % 8 == 0
 * (AULE_ERR_UNSUPPORTED below or above that). fp16/bf16 problems run on the matrix cores,
 * whose kernels address one (batch, head) slice with 32-bit offsets: a slice of 1 GiB or
 * more (about seqlen * head_dim * 2 bytes) is AULE_ERR_UNSUPPORTED. fp32 has no such bound.
 */
aule_status_t aule_attn_fwd(const void* q, const void* k, const void* v, void* o,
                            int32_t batch, int32_t heads_q, int32_t heads_kv,
                            int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                            int32_t causal, float scale, aule_dtype_t dtype,
                            hipStream_t stream);

/*
 * Variable-length attention forward over packed QKV.
 *
 * Operation: flash_attn_varlen_qkvpacked_func as documented in the ewbang.com article on a
 * PyTorch FlashAttention for Turing (docstring of the varlen function): packed
 * qkv [total_tokens, 3, heads, head_dim]; cu_seqlens [num_seqs + 1] cumulative lengths
 * ([0, 5, 12] = two sequences, qkv[0:5] and qkv[5:12]); each sequence attends only within
 * itself; causal positions count from the sequence start; output [total_tokens, heads,
 * head_dim].
 *
 *   qkv        : [total_tokens, 3, heads, head_dim] contiguous, dtype
 *   cu_seqlens : [num_seqs + 1] int32, DEVICE memory, cu[0] = 0, non-decreasing,
 *                cu[num_seqs] = total_tokens. Not read on the host; a violating array is
 *                undefined behaviour of the caller, but the kernels clamp every index to
 *                [0, total_tokens) so it cannot make them read or write out of bounds.
 *   o          : [total_tokens, heads, head_dim] contiguous, dtype (written)
 *   max_seqlen : the longest sequence length (as the varlen docstring defines it, the
 *                batch's maximum); >= 1 when total_tokens > 0. Tokens of a sequence past
 *                max_seqlen are neither read as keys nor written (their rows of o keep
 *                their contents), so a bound below the true maximum truncates sequences.
 *
 * total_tokens == 0 is an empty problem: AULE_OK, nothing launched. Otherwise num_seqs >= 1,
 * heads >= 1, max_seqlen >= 1, and the head_dim / dtype / scale rules of aule_attn_fwd apply,
 * including the fp16/bf16 slice bound (here: max_seqlen * 3 * heads * head_dim * 2 bytes).
 */
aule_status_t aule_attn_fwd_varlen(const void* qkv, const int32_t* cu_seqlens, void* o,
                                   int32_t num_seqs, int32_t total_tokens,
                                   int32_t max_seqlen, int32_t heads, int32_t head_dim,
                                   int32_t causal, float scale, aule_dtype_t dtype,
                                   hipStream_t stream);

/*
 * Varlen attention with score modifiers: the three parameters the varlen signature of the
 * ewbang.com article lists beside the scale and causal flag (sliding window (left, right),
 * soft-capping value, ALiBi slopes of shape [heads] or [batch, heads]), fused into the
 * score step.
 *
 * Arguments as aule_attn_fwd_varlen, plus
 *   window_left, window_right : key j is visible to query i only if j >= i - window_left
 *                  (when window_left >= 0) and j <= i + window_right (when >= 0), positions
 *                  counted from the sequence start; -1 = unbounded. With causal,
 *                  window_right must be -1 or 0 (the causal mask already hides j > i).
 *   softcap      : > 0 replaces each scaled score x = scale * q_i . k_j by
 *                  softcap * tanh(x / softcap); 0 = off. Must be finite and >= 0.
 *   alibi_slopes : NULL = off, else fp32 DEVICE slopes, 4-byte aligned, read only:
 *                  slope = alibi_slopes[seq * alibi_batch_stride + head], and
 *                  slope * |i - j| is subtracted from the (capped) score.
 *   alibi_batch_stride : 0 for [heads] slopes, heads for [batch, heads]; else invalid.
 * Order: scaled score, soft cap, ALiBi, masks, softmax. With every modifier off this is
 * aule_attn_fwd_varlen. Errors: INVALID_ARGUMENT for a window size below -1, a positive
 * window_right with causal, a negative or non-finite softcap, misaligned slopes, a bad
 * alibi_batch_stride or slopes overlapping o; otherwise as aule_attn_fwd_varlen.
 */
aule_status_t aule_attn_fwd_varlen_mods(const void* qkv, const int32_t* cu_seqlens, void* o,
                                        int32_t num_seqs, int32_t total_tokens,
                                        int32_t max_seqlen, int32_t heads, int32_t head_dim,
                                        int32_t causal, float scale, int32_t window_left,
                                        int32_t window_right, float softcap,
                                        const float* alibi_slopes, int32_t alibi_batch_stride,
                                        aule_dtype_t dtype, hipStream_t stream);

/*
 * Attention of a few new queries against a key/value cache (decoding), split over the key
 * range.
 *
 * Operation: the same attention as aule_attn_fwd (same layouts, GQA head mapping, dtype and
 * scale rules) for seqlen_q new queries per sequence against seqlen_k cached keys, with the
 * KV cache processed in blocks as the FlashAttention-T commentary (ai-stack.site, FAQ 4,
 * inference bullet) describes for inference. Under `causal` the new queries are the last
 * seqlen_q positions of the sequence: query i sees keys j <= i + seqlen_k - seqlen_q
 * (bottom-right alignment; equal to aule_attn_fwd's mask when seqlen_q == seqlen_k).
 *
 * The key range is cut into splits, each reduced to a partial row max, row sum and
 * unnormalised output in fp32 in `workspace`, then merged into o. The workspace is DEVICE
 * memory owned by the caller, at least aule_attn_splitkv_workspace_size(...) bytes for the
 * same arguments, 16-byte aligned, not overlapping any tensor; its contents on entry do not
 * matter and are overwritten. Calls that overlap in time must not share a workspace.
 *
 *   q, o : [batch, heads_q, seqlen_q, head_dim] contiguous, dtype
 *   k, v : [batch, heads_kv, seqlen_k, head_dim] contiguous, dtype
 *   num_splits : key-range splits; 0 chooses about C / (batch * heads_kv) (at least 1), with
 *                C the device's compute-unit count for fp16/bf16 problems of at most 32
 *                query rows per kv head (head_dim <= 128: the matrix-core kernel, one
 *                workgroup per CU) and C = 1024 otherwise; any value is clamped to
 *                [1, ceil(seqlen_k / tile)] with tile = 128 keys for those matrix-core
 *                problems, else 64 (32 for fp32), and splits that would be empty are dropped
 *
 * batch == 0 or seqlen_q == 0 is an empty problem (AULE_OK, nothing launched). Besides the
 * rules of aule_attn_fwd: (heads_q / heads_kv) * seqlen_q <= 64 query rows per kv head
 * (AULE_ERR_UNSUPPORTED above that: use aule_attn_fwd), seqlen_q <= seqlen_k under causal
 * (AULE_ERR_UNSUPPORTED), num_splits >= 0 and a large enough, aligned workspace
 * (AULE_ERR_INVALID_ARGUMENT).
 */
aule_status_t aule_attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o,
                                    int32_t batch, int32_t heads_q, int32_t heads_kv,
                                    int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                    int32_t causal, float scale, aule_dtype_t dtype,
                                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/*
 * Workspace bytes aule_attn_fwd_splitkv needs for these arguments (a pure host computation;
 * nothing is launched). Returns 0 for an empty problem and for arguments the call would
 * reject (aule_last_error() then says why).
 */
size_t aule_attn_splitkv_workspace_size(int32_t batch, int32_t heads_q, int32_t heads_kv,
                                        int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                        aule_dtype_t dtype, int32_t num_splits);

/*
 * aule_attn_fwd_splitkv without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. The split partials go to a fixed 32 MiB array inside the library, one per
 * GPU, held from the library's first use on that GPU until the process ends; this call
 * allocates nothing (no hipMalloc / hipFree, no allocating library routine).
 *
 * Arguments, operation, results and errors as aule_attn_fwd_splitkv (same split plan, same
 * kernels: the outputs are identical), without workspace / workspace_bytes. A problem whose
 * partials need more than 32 MiB (aule_attn_splitkv_workspace_size(...) > 33554432) is
 * AULE_ERR_UNSUPPORTED, nothing launched. Every call on a GPU shares that GPU's array, which
 * keeps the last call's contents: calls that overlap in time on one GPU (other streams, other
 * threads) race and must be serialised by the caller.
 */
aule_status_t aule_attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                            int32_t batch, int32_t heads_q, int32_t heads_kv,
                                            int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                            int32_t causal, float scale, aule_dtype_t dtype,
                                            int32_t num_splits, hipStream_t stream);

/*
 * Attention forward that also writes the per-row log-sum-exp needed by the backward.
 *
 * Same operation, arguments and rules as aule_attn_fwd, plus
 *   lse : [batch, heads_q, seqlen_q] fp32, DEVICE, written: the natural-log log-sum-exp of
 *         the scaled, masked scores of each query row, log(sum_j exp(scale * q_i . k_j)).
 * The forward keeps no score matrix; the backward recomputes it from Q, K and lse
 * (FlashAttention-T commentary, ai-stack.site, FAQ 4, training bullet). For fp16/bf16 the
 * row sum is taken over the probabilities as rounded to dtype (those that multiply V), so lse
 * is within about the dtype's unit roundoff (2^-11 fp16, 2^-8 bf16) of the exact value; fp32
 * is exact up to fp32 rounding. lse must be 4-byte aligned and must not overlap any tensor.
 */
aule_status_t aule_attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t batch, int32_t heads_q, int32_t heads_kv,
                                int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                int32_t causal, float scale, aule_dtype_t dtype,
                                hipStream_t stream);

/*
 * Attention backward: gradients of O = attention(q, k, v) for the output gradient do.
 *
 *   q, o, do, dq : [batch, heads_q, seqlen_q, head_dim] contiguous, dtype (dq written)
 *   k, v, dk, dv : [batch, heads_kv, seqlen_k, head_dim] contiguous, dtype (dk, dv written)
 *   lse          : [batch, heads_q, seqlen_q] fp32, as written by aule_attn_fwd_lse for the
 *                  same q, k, v, causal and scale
 *
 * With P = exp(scale * q k^T - lse) (masked entries 0), dV = P^T dO, dS = P * (dO v^T - D)
 * with D_i = do_i . o_i, dQ = scale * dS k and dK = scale * dS^T q; a key/value head shared
 * by several query heads (GQA) receives the sum of their gradients. fp32 arithmetic for all
 * dtypes; gradients rounded to dtype (RNE). Needs no workspace (the row terms D are kept
 * in dq until dq itself is written, in the same call); deterministic (no atomics).
 * Arguments and rules as aule_attn_fwd; the gradient buffers must not overlap any input or
 * each other. With seqlen_q == 0 and seqlen_k > 0 (non-causal) only dk and dv are read
 * (written as zeros); with batch == 0 nothing is read or launched.
 */
aule_status_t aule_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            int32_t batch, int32_t heads_q, int32_t heads_kv,
                            int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                            int32_t causal, float scale, aule_dtype_t dtype,
                            hipStream_t stream);

/* Static, NUL-terminated name of a status code. Never NULL. */
const char* aule_status_string(aule_status_t status);

/* Text describing the most recent failing call made by the calling thread ("" if none).
 * Valid until the next call into the library from this thread. */
const char* aule_last_error(void);

#ifdef __cplusplus
} /* extern "C" */
#endif

#endif /* AULE_ATTN_H */
