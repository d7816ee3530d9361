// Internal description of one attention-forward launch, shared by the C-ABI front end and
// the kernel launchers. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace aule {

enum class Dtype : int { F32 = 0, F16 = 1, BF16 = 2 };

// One attention problem, dense or varlen, in element strides.
//
// Dense:  tensors are [batch, heads, seq, head_dim]; a (b, h) slice starts at
//         b * bstride + h * hstride and consecutive tokens are rstride apart.
// Varlen: packed qkv [total_tokens, 3, heads, head_dim]; sequence s covers tokens
//         cu_seqlens[s] .. cu_seqlens[s+1]; a (s, h) slice starts at
//         cu_seqlens[s] * rstride + h * hstride (bstride is unused).
struct AttnProblem {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int64_t q_bstride, q_hstride, q_rstride;
    int64_t k_bstride, k_hstride, k_rstride;
    int64_t v_bstride, v_hstride, v_rstride;
    int64_t o_bstride, o_hstride, o_rstride;
    int32_t batch;        // dense: batch size; varlen: number of sequences
    int32_t heads_q;
    int32_t heads_kv;
    int32_t group;        // heads_q / heads_kv
    int32_t seqlen_q;     // dense only
    int32_t seqlen_k;     // dense only
    int32_t head_dim;
    int32_t causal;
    float scale_log2;     // softmax scale * log2(e): scores are exponentiated with exp2
    const int32_t* cu_seqlens;  // varlen only, else nullptr
    int32_t total_tokens;       // varlen only
    int32_t max_seqlen;         // varlen hint
    float* lse;                 // dense only, optional: per-row log-sum-exp [batch, heads_q, seqlen_q]
    // Score modifiers (varlen only; read only when `mods` is nonzero). With x the scaled
    // score in natural units: x <- softcap * tanh(x / softcap) when softcap > 0, then
    // x <- x - slope * |i - j| with slope = alibi[seq * alibi_sstride + head] when alibi is
    // set; key j is masked when j < i - win_left (win_left >= 0) or j > i + win_right
    // (win_right >= 0).
    int32_t mods;
    int32_t win_left, win_right;
    float softcap;
    const float* alibi;
    int32_t alibi_sstride;
};

// Launchers. Each returns hipSuccess or the launch error; none synchronises.
hipError_t launch_attn_fwd_valu(const AttnProblem& p, Dtype dt, hipStream_t stream);
// fp32 on the matrix cores (full-precision fp32 products); score modifiers and slices past
// the kernel's 32-bit offsets stay on the vector-ALU kernel
hipError_t launch_attn_fwd_f32_mfma(const AttnProblem& p, Dtype dt, hipStream_t stream);
bool f32_mfma_supports(const AttnProblem& p, Dtype dt);
hipError_t launch_attn_fwd_mfma(const AttnProblem& p, Dtype dt, hipStream_t stream);
// True when the MFMA path handles this problem (fp16/bf16 and a supported head_dim).
bool mfma_supports(const AttnProblem& p, Dtype dt);
// Short sequences (dense fp16/bf16, at most 128 keys, at most 16 (query head, 32-row block)
// items per kv head): the whole K/V slice in LDS, one workgroup per (batch, kv head).
hipError_t launch_attn_fwd_short(const AttnProblem& p, Dtype dt, hipStream_t stream);
bool short_supports(const AttnProblem& p, Dtype dt);

}  // namespace aule
