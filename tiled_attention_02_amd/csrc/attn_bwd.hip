// Attention backward (dQ, dK, dV) on the vector ALUs, fp32 arithmetic throughout.
//
// The forward keeps no score matrix; the backward recomputes it tile by tile from Q, K and
// the per-row log-sum-exp the forward wrote (FlashAttention-T commentary, ai-stack.site,
// FAQ 4, training bullet). Per (query i, key j) pair of a tile:
//   P  = exp(scale * q_i.k_j - LSE_i)            (0 where masked)
//   dP = do_i . v_j
//   dS = P * (dP - D_i),   D_i = do_i . o_i      (the row term of the softmax Jacobian)
// and the gradients accumulate as dV_j += P dO_i, dK_j += scale dS q_i, dQ_i += scale dS k_j.
//
// Two kernels, neither with atomics (results are deterministic):
//   * dK/dV: one workgroup per (batch, kv head, 32-key tile) walks every query head of its
//     group and every 32-row query tile (causal: from the tile holding its first key), with
//     the K/V tile and its gradient accumulators kept on chip;
//   * dQ: one workgroup per (batch, query head, 32-row tile) walks the key tiles.
// Both compute D_i themselves from the O and dO tiles they load.
// Workgroup: 256 threads. Score-like work: thread t takes row/key t / 8 and the 4 partners
// t % 8 + 8u; gradient accumulation: thread t owns one row (key) and columns t % 8 + 8u.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_bwd.h"

namespace aule {
namespace {

constexpr int kT = 32;         // rows per query tile = keys per key tile
constexpr int kThreads = 256;
constexpr int kTPR = 8;        // threads per row
constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
__device__ __forceinline__ float ld(const T* base, int64_t idx) { return to_f32(base[idx]); }

// Loads rows [r0, r0 + kT) of a [rows, d] slice into an fp32 LDS tile (zero outside).
template <typename T, int DMAX>
__device__ __forceinline__ void load_tile(float (*dst)[DMAX + 1], const T* src, int r0, int rows, int d) {
    for (int idx = threadIdx.x; idx < kT * DMAX; idx += kThreads) {
        const int rr = idx / DMAX, cc = idx % DMAX;
        const int r = r0 + rr;
        dst[rr][cc] = (r < rows && cc < d) ? ld(src, (int64_t)r * d + cc) : 0.f;
    }
}

// P and dS of one (query tile, key tile) pair into LDS: rows of sQ/sdO against keys of
// sK/sV. lse2 = LSE * log2(e) and delta = D per row; causal is top-left.
template <int DMAX>
__device__ __forceinline__ void p_and_ds(const float (*sQ)[DMAX + 1], const float (*sdO)[DMAX + 1],
                                         const float (*sK)[DMAX + 1], const float (*sV)[DMAX + 1],
                                         const float* lse2, const float* delta, float (*sP)[kT + 1],
                                         float (*sdS)[kT + 1], int i0, int j0, int Nq, int Nk,
                                         bool causal, float c2) {
    const int t = threadIdx.x;
    const int il = t / kTPR;
    const int i = i0 + il;
#pragma unroll
    for (int u = 0; u < kT / kTPR; ++u) {
        const int jl = t % kTPR + kTPR * u;
        const int j = j0 + jl;
        float s = 0.f, dp = 0.f;
#pragma unroll 8
        for (int cc = 0; cc < DMAX; ++cc) {
            s = fmaf(sQ[il][cc], sK[jl][cc], s);
            dp = fmaf(sdO[il][cc], sV[jl][cc], dp);
        }
        const bool visible = i < Nq && j < Nk && (!causal || j <= i);
        const float pij = visible ? __builtin_amdgcn_exp2f(s * c2 - lse2[il]) : 0.f;
        sP[il][jl] = pij;
        sdS[il][jl] = pij * (dp - delta[il]);
    }
}

// D_i = do_i . o_i for the kT rows of a query tile (8 threads per row + lane shuffles).
template <int DMAX>
__device__ __forceinline__ void row_delta(const float (*sdO)[DMAX + 1], const float (*sO)[DMAX + 1], float* delta) {
    const int t = threadIdx.x;
    const int il = t / kTPR, cl = t % kTPR;
    float x = 0.f;
    for (int cc = cl; cc < DMAX; cc += kTPR) x = fmaf(sdO[il][cc], sO[il][cc], x);
#pragma unroll
    for (int off = 1; off < kTPR; off <<= 1) x += __shfl_xor(x, off);
    if (cl == 0) delta[il] = x;
}

template <typename T, int DMAX>
__global__ __launch_bounds__(kThreads) void attn_bwd_dkdv_kernel(BwdProblem p) {
    __shared__ float sK[kT][DMAX + 1], sV[kT][DMAX + 1];
    __shared__ float sQ[kT][DMAX + 1], sdO[kT][DMAX + 1], sO[kT][DMAX + 1];
    __shared__ float sP[kT][kT + 1], sdS[kT][kT + 1];
    __shared__ float lse2[kT], delta[kT];

    const int j0 = blockIdx.x * kT, hk = blockIdx.y, b = blockIdx.z;
    const int Nq = p.seqlen_q, Nk = p.seqlen_k, d = p.head_dim, G = p.group;
    const float c2 = p.scale * kLog2e;
    const int64_t kv_off = ((int64_t)b * p.heads_kv + hk) * Nk * d;
    if (Nq > 0) {                     // with no query rows only the zero gradients are written
        load_tile<T, DMAX>(sK, static_cast<const T*>(p.k) + kv_off, j0, Nk, d);
        load_tile<T, DMAX>(sV, static_cast<const T*>(p.v) + kv_off, j0, Nk, d);
    }

    const int t = threadIdx.x;
    const int jl = t / kTPR, cl = t % kTPR;     // accumulation: key jl, columns cl + 8u
    constexpr int CPT = DMAX / kTPR;
    float dk[CPT], dv[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) { dk[u] = 0.f; dv[u] = 0.f; }

    // causal: query rows before j0 see none of these keys
    const int i_start = p.causal ? (j0 / kT) * kT : 0;
    for (int g = 0; g < G; ++g) {
        const int hq = hk * G + g;
        const int64_t q_off = ((int64_t)b * p.heads_q + hq) * Nq * d;
        const float* lse_row = p.lse + ((int64_t)b * p.heads_q + hq) * Nq;
        for (int i0 = i_start; i0 < Nq; i0 += kT) {
            __syncthreads();                              // previous tile consumed
            load_tile<T, DMAX>(sQ, static_cast<const T*>(p.q) + q_off, i0, Nq, d);
            load_tile<T, DMAX>(sdO, static_cast<const T*>(p.do_) + q_off, i0, Nq, d);
            load_tile<T, DMAX>(sO, static_cast<const T*>(p.o) + q_off, i0, Nq, d);
            if (t < kT) lse2[t] = i0 + t < Nq ? lse_row[i0 + t] * kLog2e : 0.f;
            __syncthreads();
            row_delta<DMAX>(sdO, sO, delta);
            __syncthreads();
            p_and_ds<DMAX>(sQ, sdO, sK, sV, lse2, delta, sP, sdS, i0, j0, Nq, Nk, p.causal != 0, c2);
            __syncthreads();
            for (int il = 0; il < kT; ++il) {
                const float pij = sP[il][jl], dsij = sdS[il][jl];
#pragma unroll
                for (int u = 0; u < CPT; ++u) {
                    const int cc = cl + kTPR * u;
                    dv[u] = fmaf(pij, sdO[il][cc], dv[u]);
                    dk[u] = fmaf(dsij, sQ[il][cc], dk[u]);
                }
            }
        }
    }
    const int j = j0 + jl;
    if (j < Nk) {
        T* dkr = static_cast<T*>(p.dk) + kv_off + (int64_t)j * d;
        T* dvr = static_cast<T*>(p.dv) + kv_off + (int64_t)j * d;
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int cc = cl + kTPR * u;
            if (cc < d) {
                dkr[cc] = from_f32<T>(dk[u] * p.scale);
                dvr[cc] = from_f32<T>(dv[u]);
            }
        }
    }
}

template <typename T, int DMAX>
__global__ __launch_bounds__(kThreads) void attn_bwd_dq_kernel(BwdProblem p) {
    __shared__ float sQ[kT][DMAX + 1], sdO[kT][DMAX + 1], sO[kT][DMAX + 1];
    __shared__ float sK[kT][DMAX + 1], sV[kT][DMAX + 1];
    __shared__ float sP[kT][kT + 1], sdS[kT][kT + 1];
    __shared__ float lse2[kT], delta[kT];

    const int i0 = blockIdx.x * kT, hq = blockIdx.y, b = blockIdx.z;
    const int Nq = p.seqlen_q, Nk = p.seqlen_k, d = p.head_dim;
    const int hk = hq / p.group;
    const float c2 = p.scale * kLog2e;
    const int64_t q_off = ((int64_t)b * p.heads_q + hq) * Nq * d;
    const int64_t kv_off = ((int64_t)b * p.heads_kv + hk) * Nk * d;
    load_tile<T, DMAX>(sQ, static_cast<const T*>(p.q) + q_off, i0, Nq, d);
    load_tile<T, DMAX>(sdO, static_cast<const T*>(p.do_) + q_off, i0, Nq, d);
    load_tile<T, DMAX>(sO, static_cast<const T*>(p.o) + q_off, i0, Nq, d);
    const float* lse_row = p.lse + ((int64_t)b * p.heads_q + hq) * Nq;
    const int t = threadIdx.x;
    if (t < kT) lse2[t] = i0 + t < Nq ? lse_row[i0 + t] * kLog2e : 0.f;
    __syncthreads();
    row_delta<DMAX>(sdO, sO, delta);

    const int il = t / kTPR, cl = t % kTPR;     // accumulation: row il, columns cl + 8u
    constexpr int CPT = DMAX / kTPR;
    float dq[CPT];
#pragma unroll
    for (int u = 0; u < CPT; ++u) dq[u] = 0.f;

    const int j_end = p.causal ? min(Nk, i0 + kT) : Nk;
    for (int j0 = 0; j0 < j_end; j0 += kT) {
        __syncthreads();                                  // previous tile consumed
        load_tile<T, DMAX>(sK, static_cast<const T*>(p.k) + kv_off, j0, Nk, d);
        load_tile<T, DMAX>(sV, static_cast<const T*>(p.v) + kv_off, j0, Nk, d);
        __syncthreads();
        p_and_ds<DMAX>(sQ, sdO, sK, sV, lse2, delta, sP, sdS, i0, j0, Nq, Nk, p.causal != 0, c2);
        __syncthreads();
        for (int jl = 0; jl < kT; ++jl) {
            const float dsij = sdS[il][jl];
#pragma unroll
            for (int u = 0; u < CPT; ++u) dq[u] = fmaf(dsij, sK[jl][cl + kTPR * u], dq[u]);
        }
    }
    const int i = i0 + il;
    if (i < Nq) {
        T* dqr = static_cast<T*>(p.dq) + q_off + (int64_t)i * d;
#pragma unroll
        for (int u = 0; u < CPT; ++u) {
            const int cc = cl + kTPR * u;
            if (cc < d) dqr[cc] = from_f32<T>(dq[u] * p.scale);
        }
    }
}

template <typename T, int DMAX>
hipError_t launch_typed(const BwdProblem& p, hipStream_t stream) {
    dim3 gk((p.seqlen_k + kT - 1) / kT, p.heads_kv, p.batch);
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, DMAX>), gk, dim3(kThreads), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.seqlen_q == 0) return hipSuccess;     // dK = dV = 0 written above, no dQ rows
    dim3 gq((p.seqlen_q + kT - 1) / kT, p.heads_q, p.batch);
    hipLaunchKernelGGL((attn_bwd_dq_kernel<T, DMAX>), gq, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dim(const BwdProblem& p, hipStream_t stream) {
    if (p.head_dim <= 64) return launch_typed<T, 64>(p, stream);
    return launch_typed<T, 128>(p, stream);
}

}  // namespace

hipError_t launch_attn_bwd(const BwdProblem& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::F32) return launch_dim<float>(p, stream);   // fp32 only
    return hipErrorInvalidValue;
}

}  // namespace aule
