// Internal description of one attention backward launch, shared by the C-ABI front end and
// the backward kernels. Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"

namespace aule {

// All tensors dense and contiguous: q, o, do_, dq: [batch, heads_q, seqlen_q, head_dim];
// k, v, dk, dv: [batch, heads_kv, seqlen_k, head_dim]; lse: [batch, heads_q, seqlen_q] fp32
// natural log-sum-exp of the scaled, masked scores (what the forward writes).
struct BwdProblem {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* do_;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    int32_t batch;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t group;      // heads_q / heads_kv
    int32_t seqlen_q;
    int32_t seqlen_k;
    int32_t head_dim;
    int32_t causal;     // top-left: key j is visible to query i iff j <= i
    float scale;
};

// Launches the dK/dV and dQ kernels on `stream`; does not synchronise. The vector-ALU
// kernels take every dtype; the matrix-core kernels take fp16 and bf16.
hipError_t launch_attn_bwd(const BwdProblem& p, Dtype dt, hipStream_t stream);
hipError_t launch_attn_bwd_mfma(const BwdProblem& p, Dtype dt, hipStream_t stream);
// fp32 on the matrix cores (full-precision fp32 products); slices past its 32-bit buffer
// offsets stay on the vector-ALU kernels. Writes D_i = do_i . o_i into dq before dq itself.
hipError_t launch_attn_bwd_f32_mfma(const BwdProblem& p, hipStream_t stream);
bool bwd_f32_mfma_supports(const BwdProblem& p);

}  // namespace aule
