// Tiled attention forward on the vector ALUs, fp32 arithmetic throughout.
//
// This is the fp32 path (no reduced-precision matrix instruction touches fp32 inputs). It
// follows the
// FlashAttention block loop of the xxqk.cn article "Attention算子实战：从CUDA优化到昇腾/CANN部署"
// (section 2.2): a Q tile stays on chip, K/V tiles stream through LDS, each tile updates a
// running row max m and row sum l (online softmax, FlashAttention-T commentary on
// ai-stack.site, best practice 4) and rescales the output accumulator, and only O is
// written back.
//
// Workgroup: 128 threads = 16 query rows x 8 threads per row. Tile: BM = 16 query rows,
// BN = 32 keys. Thread (r, c) computes the scores of keys c, c+8, c+16, c+24 of row r and
// owns output columns c, c+8, ... of row r. Row max / row sum use lane shuffles inside
// the 8-lane group of a row.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_device.h"

namespace aule {
namespace {

constexpr int kBM = 16;
constexpr int kBN = 32;
constexpr int kTPR = 8;  // threads per query row
constexpr int kThreads = kBM * kTPR;
constexpr float kLog2eF = 1.4426950408889634f;

template <typename T, int DMAX, bool VARLEN, bool MODS>
__global__ __launch_bounds__(kThreads) void attn_fwd_valu_kernel(AttnProblem p) {
    __shared__ float sQ[kBM][DMAX + 1];
    __shared__ float sK[kBN][DMAX + 1];
    __shared__ float sV[kBN][DMAX];
    __shared__ float sP[kBM][kBN + 1];

    const int tid = threadIdx.x;
    const int r = tid / kTPR;
    const int c = tid % kTPR;
    const int hq = blockIdx.y;
    const int hk = hq / p.group;
    const int d = p.head_dim;

    TileSlot slot;
    if constexpr (VARLEN) {
        slot = locate_varlen_tile(p.cu_seqlens, p.batch, p.total_tokens, p.max_seqlen, kBM, blockIdx.x, false);
        if (!slot.valid) return;
    } else {
        slot.valid = 1;
        slot.seq = blockIdx.z;
        slot.tok0 = 0;
        slot.len_q = p.seqlen_q;
        slot.len_k = p.seqlen_k;
        slot.tile = blockIdx.x;
    }

    const T* qb = static_cast<const T*>(p.q) + (VARLEN ? slot.tok0 * p.q_rstride : slot.seq * p.q_bstride) + hq * p.q_hstride;
    const T* kb = static_cast<const T*>(p.k) + (VARLEN ? slot.tok0 * p.k_rstride : slot.seq * p.k_bstride) + hk * p.k_hstride;
    const T* vb = static_cast<const T*>(p.v) + (VARLEN ? slot.tok0 * p.v_rstride : slot.seq * p.v_bstride) + hk * p.v_hstride;
    T* ob = static_cast<T*>(p.o) + (VARLEN ? slot.tok0 * p.o_rstride : slot.seq * p.o_bstride) + hq * p.o_hstride;

    const int row0 = slot.tile * kBM;
    const int Lq = slot.len_q, Lk = slot.len_k;

    // Q tile -> LDS (zero rows past the end and columns past head_dim)
    for (int idx = tid; idx < kBM * DMAX; idx += kThreads) {
        int rr = idx / DMAX, dd = idx % DMAX;
        int i = row0 + rr;
        sQ[rr][dd] = (i < Lq && dd < d) ? to_f32(qb[(int64_t)i * p.q_rstride + dd]) : 0.f;
    }

    const int i = row0 + r;  // this thread's query row
    float m = -INFINITY, l = 0.f;
    float acc[DMAX / kTPR];
#pragma unroll
    for (int u = 0; u < DMAX / kTPR; ++u) acc[u] = 0.f;

    int kend = Lk;
    const int last_row = min(row0 + kBM, Lq) - 1;
    if (p.causal) kend = min(Lk, last_row + 1);
    int kbeg = 0;
    float slope = 0.f, cap = 0.f, cap_k = 0.f;
    const float scale_nat = p.scale_log2 * 0.69314718055994531f;
    if constexpr (MODS) {
        // key tiles entirely outside every row's window are skipped
        if (p.win_left >= 0) kbeg = max(0, row0 - p.win_left) / kBN * kBN;
        if (!p.causal && p.win_right >= 0) kend = min(Lk, last_row + 1 + p.win_right);
        if (p.alibi) slope = p.alibi[(int64_t)slot.seq * p.alibi_sstride + hq];
        cap = p.softcap;
        cap_k = cap > 0.f ? 2.f * kLog2eF / cap : 0.f;
    }

    for (int j0 = kbeg; j0 < kend; j0 += kBN) {
        __syncthreads();  // previous tile fully consumed (and Q written, first time)
        for (int idx = tid; idx < kBN * DMAX; idx += kThreads) {
            int jj = idx / DMAX, dd = idx % DMAX;
            int j = j0 + jj;
            bool ok = (j < Lk && dd < d);
            sK[jj][dd] = ok ? to_f32(kb[(int64_t)j * p.k_rstride + dd]) : 0.f;
            sV[jj][dd] = ok ? to_f32(vb[(int64_t)j * p.v_rstride + dd]) : 0.f;
        }
        __syncthreads();

        float s[kBN / kTPR];
        float tmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < kBN / kTPR; ++u) {
            int jj = c + kTPR * u;
            // eight partial sums over interleaved columns, combined pairwise: about an eighth
            // of the rounding error of one serial chain over head_dim terms
            float part[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) part[e] = 0.f;
#pragma unroll
            for (int dd = 0; dd < DMAX; dd += 8)
#pragma unroll
                for (int e = 0; e < 8; ++e) part[e] = fmaf(sQ[r][dd + e], sK[jj][dd + e], part[e]);
            const float dot = ((part[0] + part[1]) + (part[2] + part[3])) + ((part[4] + part[5]) + (part[6] + part[7]));
            int j = j0 + jj;
            bool masked = (j >= Lk) || (p.causal && j > i);
            if constexpr (MODS) {
                masked = masked || (p.win_left >= 0 && j < i - p.win_left) ||
                         (p.win_right >= 0 && j > i + p.win_right);
                float x = dot * scale_nat;
                if (cap > 0.f) x = soft_cap(x, cap, cap_k);
                x = fmaf(-slope, fabsf((float)(i - j)), x);
                s[u] = masked ? -INFINITY : x * kLog2eF;
            } else {
                s[u] = masked ? -INFINITY : dot * p.scale_log2;
            }
            tmax = fmaxf(tmax, s[u]);
        }
#pragma unroll
        for (int off = 1; off < kTPR; off <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, off));

        float m_new = fmaxf(m, tmax);
        float m_use = (m_new == -INFINITY) ? 0.f : m_new;   // fully masked so far: keep 0s
        float alpha = __builtin_amdgcn_exp2f(m - m_use);     // m = -inf -> 0
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < kBN / kTPR; ++u) {
            float pv = __builtin_amdgcn_exp2f(s[u] - m_use);
            psum += pv;
            sP[r][c + kTPR * u] = pv;
        }
#pragma unroll
        for (int off = 1; off < kTPR; off <<= 1) psum += __shfl_xor(psum, off);
        l = l * alpha + psum;
        m = m_new;
        __syncthreads();

#pragma unroll
        for (int u = 0; u < DMAX / kTPR; ++u) {
            int dd = c + kTPR * u;
            float a0 = 0.f, a1 = 0.f;   // the tile's contribution in two chains
#pragma unroll 8
            for (int jj = 0; jj < kBN; jj += 2) {
                a0 = fmaf(sP[r][jj], sV[jj][dd], a0);
                a1 = fmaf(sP[r][jj + 1], sV[jj + 1][dd], a1);
            }
            acc[u] = fmaf(acc[u], alpha, a0 + a1);
        }
    }

    if (!VARLEN && p.lse && c == 0 && i < Lq)   // natural log-sum-exp of the scaled scores
        p.lse[((int64_t)slot.seq * p.heads_q + hq) * p.seqlen_q + i] = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
    if (i < Lq) {
        float inv = 1.f / l;
#pragma unroll
        for (int u = 0; u < DMAX / kTPR; ++u) {
            int dd = c + kTPR * u;
            if (dd < d) ob[(int64_t)i * p.o_rstride + dd] = from_f32<T>(acc[u] * inv);
        }
    }
}

template <typename T, int DMAX>
hipError_t launch_typed(const AttnProblem& p, hipStream_t stream) {
    dim3 block(kThreads);
    if (p.cu_seqlens) {
        dim3 grid(varlen_grid_tiles(p.total_tokens, p.batch, kBM), p.heads_q, 1);
        if (p.mods)
            hipLaunchKernelGGL((attn_fwd_valu_kernel<T, DMAX, true, true>), grid, block, 0, stream, p);
        else
            hipLaunchKernelGGL((attn_fwd_valu_kernel<T, DMAX, true, false>), grid, block, 0, stream, p);
    } else {
        dim3 grid((p.seqlen_q + kBM - 1) / kBM, p.heads_q, p.batch);
        hipLaunchKernelGGL((attn_fwd_valu_kernel<T, DMAX, false, false>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dim(const AttnProblem& p, hipStream_t stream) {
    if (p.head_dim <= 64) return launch_typed<T, 64>(p, stream);
    return launch_typed<T, 128>(p, stream);
}

}  // namespace

hipError_t launch_attn_fwd_valu(const AttnProblem& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::F32) return launch_dim<float>(p, stream);   // fp32 only
    return hipErrorInvalidValue;
}

}  // namespace aule
