// Internal description of one split-KV decoding launch (new queries against a key/value
// cache), shared by the C-ABI front end and the decode kernels. Not part of the public
// interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_device.h"

namespace aule {

// q, o: [batch, heads_q, seqlen_q, head_dim]; k, v: [batch, heads_kv, seqlen_k, head_dim];
// all contiguous. The workspace holds, per split and output row (batch, head, query), the
// partial max (log2 units) and sum, and the unnormalised partial O, all fp32.
struct DecodeProblem {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int32_t batch;
    int32_t heads_q;
    int32_t heads_kv;
    int32_t group;          // heads_q / heads_kv
    int32_t seqlen_q;       // new queries per sequence
    int32_t seqlen_k;       // cached keys per sequence
    int32_t head_dim;
    int32_t causal;         // bottom-right aligned: query i sees keys j <= i + seqlen_k - seqlen_q
    float scale;
    int32_t num_splits;     // key-range splits (grid x)
    int32_t keys_per_split; // a multiple of the kernel's key tile
    float* ws_ml;           // [num_splits][rows][2]: m, l
    float* ws_o;            // [num_splits][rows][head_dim]
};

// Keys per tile of the partial kernel for this element type (splits are multiples of it).
int decode_keys_per_tile(Dtype dt);
// Launches the partial kernel and the merge kernel on `stream`; does not synchronise.
hipError_t launch_attn_decode(const DecodeProblem& p, Dtype dt, hipStream_t stream);
// The matrix-core partial kernel (fp16/bf16, at most 32 query rows per kv head, head_dim up
// to 128): whether it covers a problem, and its launch (same workspace layout).
bool decode_mfma_supports(const DecodeProblem& p, Dtype dt);
// Whether a problem shape takes the matrix-core kernel (decided before the split plan), and
// the key granule its splits should be a multiple of (every wave gets whole tiles).
bool decode_mfma_eligible(Dtype dt, int rows_per_kv_head, int head_dim);
int decode_mfma_keys_granule();
hipError_t launch_attn_decode_mfma_partial(const DecodeProblem& p, Dtype dt, hipStream_t stream);
// The fixed device workspace of the no-allocation entry point: its size, and its address on
// the current device (looked up once per device).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);

}  // namespace aule
