// fp32 attention forward on the matrix cores: v_mfma_f32_32x32x2_f32 takes fp32 operands and
// accumulates in fp32 (a full-precision product, no rounding of the inputs), at the same
// 157 TFLOP/s as the vector ALUs' fp32 FMA on MI355X. In fp32 the products dominate by far:
// a 32-query x 32-key step is 128 products of 64 cycles per wave against ~100 vector
// instructions of softmax, so the kernel is built around feeding the matrix core.
//
// The FlashAttention block loop of the xxqk.cn article "Attention算子实战：从CUDA优化到昇腾/CANN部署"
// (section 2.2: Q block on chip, K/V tiles streamed, online softmax, only O written) with the
// running max / sum of the FlashAttention-T commentary (ai-stack.site, best practice 4),
// everything in fp32.
//
// Work split: workgroup = 4 waves, wave = 32 query rows of one query head; GH query heads that
// share one kv head sit in one workgroup (GQA) and the other 4/GH waves take further 32-row
// blocks. K/V tiles of 32 keys, double-buffered in LDS, copied global -> LDS with
// buffer_load_dwordx4 ... lds; the descriptor's range check zeroes rows past the end, and
// chunks past head_dim are sent out of range.
//
// Products (v_mfma_f32_32x32x2_f32: A 32 x 2, lane l holds A[l % 32][l / 32]; B 2 x 32, lane l
// holds B[l / 32][l % 32]; C 32 x 32 as for the 16-bit 32x32 products):
//   S^T = K Q^T   the contraction over head_dim is split by lane half: at step ks, half h
//                 supplies dimension h D/2 + ks, so a lane reads 4 consecutive dimensions of
//                 its key with one 16-byte LDS read and holds its query's D/2 dimensions of
//                 Q in registers. Register r of lane l then holds key 8(r/4) + 4(l/32) + r%4
//                 of the tile and query l % 32.
//   O^T += V^T P^T  the contraction over the tile's keys takes, at step kk, key
//                 8(kk/4) + 4h + kk%4 for half h: exactly the key in register kk of the S^T
//                 accumulator, so P enters as a B operand with no data movement; the A
//                 operand is one 4-byte LDS read of V per lane (32 lanes read 128 contiguous
//                 bytes of one key row).
// LDS swizzles (16-byte chunk c of row r stored at chunk c ^ swz(r)): K rows c ^ (r % 16), so
// each 16-lane pass of the S^T reads hits 16 distinct chunk slots; V rows c ^ 8 for rows
// with bit 2 set, so the two lane halves of a P V read (keys 4 apart) fall 128 bytes apart
// in the bank space.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_device.h"
#include "attn_mfma.h"
#include "attn_problem.h"

namespace aule {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kF32Waves = 4;
constexpr int kF32Threads = kF32Waves * 64;
constexpr int kF32Keys = 32;   // keys per K/V tile

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ int kswz_f32(int row) { return row & 15; }
__device__ __forceinline__ int vswz_f32(int row) { return ((row >> 2) & 1) << 3; }
#endif

template <int D, int GH, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kF32Threads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_f32_mfma_kernel(AttnProblem p, int n_qtiles) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int RB = kF32Waves / GH;            // 32-row blocks per workgroup
    constexpr int BM = 32 * RB;                   // query rows per workgroup (per head)
    constexpr int KC = D / 4;                     // 16-byte chunks per K / V row
    constexpr int HALF = D / 2;                   // contraction steps of S^T
    constexpr int DB = D / 32;                    // 32-row d-blocks of O^T
    constexpr int NACC = 4;                       // product chains of S^T
    constexpr int TILE_CHUNKS = kF32Keys * KC;
    constexpr int NI = TILE_CHUNKS / kF32Threads; // copy instructions per wave per tile (K or V)
    static_assert(KC >= 16 && NI >= 1 && NI * kF32Threads == TILE_CHUNKS, "head_dim 64 or 128");

    __shared__ f32x4 sK[2][TILE_CHUNKS];
    __shared__ f32x4 sV[2][TILE_CHUNKS];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, ln = lane & 31;
    const int hd = p.head_dim;

    // ---------------------------------------------------------------- work item
    int bidx, hq0, tile, Lq, Lk;
    int64_t tok0 = 0;
    if constexpr (VARLEN) {
        const TileSlot s = locate_varlen_tile(p.cu_seqlens, p.batch, p.total_tokens, p.max_seqlen, BM, blockIdx.x, CAUSAL);
        if (!s.valid) return;
        bidx = s.seq; tok0 = s.tok0; tile = s.tile; Lq = s.len_q; Lk = s.len_k;
        hq0 = blockIdx.y * GH;
    } else {
        // (q-tile rank, group) with the group fastest; causal: the longest tiles first
        const int ngroups = p.heads_q / GH;
        const int NG = p.batch * ngroups;
        const int t = blockIdx.x / NG, g = blockIdx.x - t * NG;
        tile = CAUSAL ? n_qtiles - 1 - t : t;
        bidx = g / ngroups;
        hq0 = (g - bidx * ngroups) * GH;
        Lq = p.seqlen_q; Lk = p.seqlen_k;
    }
    const int hq = hq0 + wave % GH;
    const int hk = hq0 / p.group;
    const int qr0 = tile * BM + 32 * (wave / GH);   // this wave's first query row
    const float* qb = static_cast<const float*>(p.q) + (VARLEN ? tok0 * p.q_rstride : bidx * p.q_bstride) + hq * p.q_hstride;
    const float* kb = static_cast<const float*>(p.k) + (VARLEN ? tok0 * p.k_rstride : bidx * p.k_bstride) + hk * p.k_hstride;
    const float* vb = static_cast<const float*>(p.v) + (VARLEN ? tok0 * p.v_rstride : bidx * p.v_bstride) + hk * p.v_hstride;
    float* ob = static_cast<float*>(p.o) + (VARLEN ? tok0 * p.o_rstride : bidx * p.o_bstride) + hq * p.o_hstride;
    const uint32_t q_rs = (uint32_t)(p.q_rstride * 4), k_rs = (uint32_t)(p.k_rstride * 4);
    const uint32_t v_rs = (uint32_t)(p.v_rstride * 4), o_rs = (uint32_t)(p.o_rstride * 4);

    // keys walked by the workgroup (causal: up to its last row)
    const int wg_rows_end = min(tile * BM + BM, Lq);
    const int keys = CAUSAL ? min(Lk, wg_rows_end) : Lk;
    const int n_kt = keys > 0 ? (keys + kF32Keys - 1) / kF32Keys : 0;

    // ---------------------------------------------------------------- K/V copies
    // K/V descriptors cover exactly the Lk valid rows; each lane fetches the global chunk
    // that belongs at its LDS slot (slot = (wave NI + i) 64 + lane of the tile).
    const i32x4 rk = buffer_desc(kb, Lk > 0 ? (int)((int64_t)(Lk - 1) * k_rs + hd * 4) : 0);
    const i32x4 rv = buffer_desc(vb, Lk > 0 ? (int)((int64_t)(Lk - 1) * v_rs + hd * 4) : 0);
    uint32_t koff[NI], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int slot = (wave * NI + i) * 64 + lane;
        const int row = slot / KC, pc = slot % KC;
        const int kc = pc ^ kswz_f32(row), vc = pc ^ vswz_f32(row);
        koff[i] = kc * 4 < hd ? row * k_rs + kc * 16 : kOobOffset;
        voff[i] = vc * 4 < hd ? row * v_rs + vc * 16 : kOobOffset;
    }
    auto lds_off = [](const f32x4* q) { return (uint32_t)(uintptr_t)(lds_void*)q; };
    auto issue_tile = [&](int t, int buf) {
        const uint32_t gk = (uint32_t)(t * kF32Keys) * k_rs, gv = (uint32_t)(t * kF32Keys) * v_rs;
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const uint32_t slot = (uint32_t)(wave * NI + i) * 64u * 16u;
            lds_copy16(rk, koff[i] + gk, __builtin_amdgcn_readfirstlane(lds_off(sK[buf]) + slot));
            lds_copy16(rv, voff[i] + gv, __builtin_amdgcn_readfirstlane(lds_off(sV[buf]) + slot));
        }
    };
    if (n_kt > 0) issue_tile(0, 0);

    // ---------------------------------------------------------------- Q -> registers
    // lane (query ln, half h): dimensions [h D/2, h D/2 + D/2) of its query row; rows past Lq
    // and columns past head_dim read as zero
    float qf[HALF];
    {
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(qb), (short)0, Lq > 0 ? (int)((int64_t)Lq * q_rs) : 0, (int)kBufferFlags);
        const uint32_t row_off = (uint32_t)(qr0 + ln) * q_rs;
#pragma unroll
        for (int j = 0; j < HALF / 4; ++j) {
            const int col = h * HALF + 4 * j;
            const uint32_t off = col < hd ? row_off + (uint32_t)col * 4u : kOobOffset;
            const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)off, 0, 0));
            qf[4 * j] = x[0]; qf[4 * j + 1] = x[1]; qf[4 * j + 2] = x[2]; qf[4 * j + 3] = x[3];
        }
    }

    // ---------------------------------------------------------------- main loop
    const float c = p.scale_log2;
    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    float m = -INFINITY, l_part = 0.f;
    const int q_row = qr0 + ln;

    auto body = [&](int t, int buf) {
        // all waves finished tile t-1 (its buffer is free) and every copy of tile t landed
        __builtin_amdgcn_s_waitcnt(0x70);   // vmcnt(0) lgkmcnt(0)
        asm volatile("s_barrier" ::: "memory");
        if (t + 1 < n_kt) issue_tile(t + 1, buf ^ 1);
        // S^T = K Q^T in NACC independent product chains (step ks feeds chain ks % NACC),
        // summed pairwise: one chain over all D/2 steps measured 1.5e-5 off the exact result at
        // scale 2, head_dim 64 (the rounding of a long running sum), against the 1e-5 bar
        f32x16 sa[NACC];
#pragma unroll
        for (int a = 0; a < NACC; ++a) sa[a] = f32x16{};
        const f32x4* kt = sK[buf] + ln * KC;
#pragma unroll
        for (int j = 0; j < HALF / 4; ++j) {
            const f32x4 kq = kt[(h * (HALF / 4) + j) ^ kswz_f32(ln)];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ks = 4 * j + e;
                sa[ks % NACC] = __builtin_amdgcn_mfma_f32_32x32x2f32(kq[e], qf[ks], sa[ks % NACC], 0, 0, 0);
            }
        }
#pragma unroll
        for (int w = 1; w < NACC; w *= 2)
#pragma unroll
            for (int a = 0; a + w < NACC; a += 2 * w) sa[a] += sa[a + w];
        f32x16 s = sa[0];
        // scale, mask (tiles that reach past the end or the diagonal), online softmax
        const int k0 = t * kF32Keys;
        const bool edge = (k0 + kF32Keys > Lk) || (CAUSAL && k0 + kF32Keys - 1 > qr0);
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float x = s[r] * c;
            if (edge) {
                const int key = k0 + 8 * (r >> 2) + 4 * h + (r & 3);
                const bool masked = key >= Lk || (CAUSAL && key > q_row);
                x = masked ? -INFINITY : x;
            }
            s[r] = x;
            mx = fmaxf(mx, x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m, mx);
        // a row with no visible key yet keeps m = -inf: its P and factor are then 0
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m - m_use);
        float psum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            s[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
            psum += s[r];
        }
        l_part = l_part * alpha + psum;
        m = m_new;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] *= alpha;
        // O^T += V^T P^T
        const float* vt = reinterpret_cast<const float*>(sV[buf]);
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int key = 8 * (kk >> 2) + 4 * h + (kk & 3);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int chunk = (8 * db + (ln >> 2)) ^ vswz_f32(key);
                const float va = vt[(key * KC + chunk) * 4 + (ln & 3)];
                o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, s[kk], o[db], 0, 0, 0);
            }
        }
    };
    for (int t = 0; t < n_kt; t += 2) {
        body(t, 0);
        if (t + 1 < n_kt) body(t + 1, 1);
    }

    // ---------------------------------------------------------------- epilogue
    // O = O^T / l: register r of block db holds dimension 32db + 8(r/4) + 4h + r%4 of query
    // ln; four consecutive dimensions per 16-byte store, rows past Lq dropped by the
    // descriptor, chunks past head_dim sent out of range
    const float l = l_part + __shfl_xor(l_part, 32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        ob, (short)0, Lq > 0 ? (int)((int64_t)Lq * o_rs) : 0, (int)kBufferFlags);
    const uint32_t row_off = (uint32_t)q_row * o_rs;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int col = 32 * db + 8 * g + 4 * h;
            const f32x4 w = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
            const uint32_t off = col < hd ? row_off + (uint32_t)col * 4u : kOobOffset;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, w), ro, (int)off, 0, 0);
        }
    if (!VARLEN && p.lse && h == 0 && q_row < Lq)
        p.lse[((int64_t)bidx * p.heads_q + hq) * p.seqlen_q + q_row] =
            l > 0.f ? (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : -INFINITY;
#endif  // __HIP_DEVICE_COMPILE__
}

template <int D, int GH, bool CAUSAL, bool VARLEN>
hipError_t launch_cfg(const AttnProblem& p, hipStream_t stream) {
    constexpr int BM = 32 * (kF32Waves / GH);
    const dim3 block(kF32Threads);
    if constexpr (VARLEN) {
        const int64_t nt = varlen_grid_tiles(p.total_tokens, p.batch, BM);
        if (nt > INT32_MAX || p.heads_q > 65535) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((attn_fwd_f32_mfma_kernel<D, GH, CAUSAL, true>), dim3((unsigned)nt, (unsigned)(p.heads_q / GH)),
                           block, 0, stream, p, 0);
    } else {
        const int n_qtiles = (p.seqlen_q + BM - 1) / BM;
        const int64_t nb = (int64_t)n_qtiles * p.batch * (p.heads_q / GH);
        if (nb == 0) return hipSuccess;
        if (nb > INT32_MAX) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((attn_fwd_f32_mfma_kernel<D, GH, CAUSAL, false>), dim3((unsigned)nb), block, 0, stream, p,
                           n_qtiles);
    }
    return hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
hipError_t launch_gh(const AttnProblem& p, hipStream_t stream) {
    const int gh = VARLEN ? 1 : (p.group % 4 == 0 ? 4 : p.group % 2 == 0 ? 2 : 1);
    if (gh == 4) return launch_cfg<D, 4, CAUSAL, VARLEN>(p, stream);
    if (gh == 2) return launch_cfg<D, 2, CAUSAL, VARLEN>(p, stream);
    return launch_cfg<D, 1, CAUSAL, VARLEN>(p, stream);
}

template <int D>
hipError_t launch_d(const AttnProblem& p, hipStream_t stream) {
    const bool varlen = p.cu_seqlens != nullptr;
    if (p.causal) return varlen ? launch_gh<D, true, true>(p, stream) : launch_gh<D, true, false>(p, stream);
    return varlen ? launch_gh<D, false, true>(p, stream) : launch_gh<D, false, false>(p, stream);
}

}  // namespace

bool f32_mfma_supports(const AttnProblem& p, Dtype dt) {
    if (dt != Dtype::F32 || p.mods || p.head_dim > 128 || p.head_dim % 8 != 0) return false;
    // 32-bit buffer offsets from a (sequence, head) slice's first row: the slice plus one tile
    // of headroom below 2^30 bytes
    const int64_t rows_k = p.cu_seqlens ? p.max_seqlen : p.seqlen_k;
    const int64_t rows_q = p.cu_seqlens ? p.max_seqlen : p.seqlen_q;
    const int64_t stride_k = p.k_rstride > p.v_rstride ? p.k_rstride : p.v_rstride;
    const int64_t stride_q = p.q_rstride > p.o_rstride ? p.q_rstride : p.o_rstride;
    const int64_t limit = int64_t(1) << 30;
    return (rows_k + 64) * stride_k * 4 < limit && (rows_q + 256) * stride_q * 4 < limit;
}

hipError_t launch_attn_fwd_f32_mfma(const AttnProblem& p, Dtype dt, hipStream_t stream) {
    if (dt != Dtype::F32) return hipErrorInvalidValue;
    if (p.head_dim <= 64) return launch_d<64>(p, stream);
    return launch_d<128>(p, stream);
}

}  // namespace aule
