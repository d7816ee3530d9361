// Device helpers shared by the attention kernels: element conversion and the mapping from a
// workgroup to the query tile it owns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_problem.h"

namespace aule {

typedef __bf16 bf16_t;
typedef _Float16 f16_t;

template <typename T> __device__ __forceinline__ float to_f32(T x) { return static_cast<float>(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x) { return static_cast<T>(x); }

// cap * tanh(x / cap) for cap > 0, through tanh(y) = 1 - 2 / (exp(2y) + 1): exp2 overflows
// to +inf for large y (tanh -> 1) and underflows to 0 for very negative y (tanh -> -1).
__device__ __forceinline__ float soft_cap(float x, float cap, float two_log2e_over_cap) {
    const float e = __builtin_amdgcn_exp2f(x * two_log2e_over_cap);
    return cap * (1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f));
}

// Where a query tile lives.
struct TileSlot {
    int valid;       // 0: this workgroup has no work (varlen padding of the grid)
    int seq;         // dense: batch index; varlen: sequence index
    int64_t tok0;    // varlen: first token of the sequence; dense: 0
    int len_q;       // query rows of this (batch|sequence)
    int len_k;       // keys of this (batch|sequence)
    int tile;        // query tile index within the sequence
};

__device__ __forceinline__ int clamp_tok(int x, int total) {
    return x < 0 ? 0 : (x > total ? total : x);
}

// Varlen grid mapping. Sequence s owns the virtual tile ids
//   [first(s), first(s) + ceil(L_s / BM))   with   first(s) = floor(cu[s] / BM) + s,
// which never overlap and all lie below floor(T / BM) + num_seqs, the grid size. A
// workgroup finds its sequence by binary search over first(.) and exits if its id falls in
// the gap after the sequence's last tile. Every cu value is clamped to [0, T], so even a
// malformed cu_seqlens cannot move a tile outside the packed tensor, and a sequence's length
// is clamped to max_len (the caller's max_seqlen): tokens past it are neither read as keys
// nor written, and the kernels' per-sequence 32-bit offsets stay within the bound the host
// checked. When `reverse` is set the tiles of a sequence are handed out last-tile-first (the
// longest causal tiles start earliest).
__device__ __forceinline__ TileSlot locate_varlen_tile(const int32_t* __restrict__ cu, int nseq,
                                                       int total, int max_len, int BM, int x,
                                                       bool reverse) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        int first = clamp_tok(cu[mid], total) / BM + mid;
        if (first <= x) lo = mid; else hi = mid - 1;
    }
    TileSlot t;
    int start = clamp_tok(cu[lo], total);
    int end = clamp_tok(cu[lo + 1], total);
    int len = end > start ? end - start : 0;
    len = len < max_len ? len : max_len;
    int local = x - (start / BM + lo);
    int ntiles = (len + BM - 1) / BM;
    t.valid = local < ntiles;
    t.seq = lo;
    t.tok0 = start;
    t.len_q = len;
    t.len_k = len;
    t.tile = reverse ? (ntiles - 1 - local) : local;
    return t;
}

__host__ __device__ __forceinline__ int varlen_grid_tiles(int total, int nseq, int BM) {
    return total / BM + nseq;
}

}  // namespace aule
