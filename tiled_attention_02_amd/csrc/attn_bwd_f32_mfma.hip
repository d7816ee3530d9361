// fp32 attention backward on the matrix cores (v_mfma_f32_32x32x2_f32: fp32 operands, fp32
// accumulation). The score matrix is recomputed tile by tile from Q, K and the forward's
// per-row log-sum-exp (FlashAttention-T commentary, ai-stack.site, FAQ 4, training bullet).
// Per (query i, key j): P = exp2(scale log2(e) q_i.k_j - LSE_i log2(e)) (0 where masked),
// dP = do_i.v_j, dS = P (dP - D_i) with D_i = do_i.o_i; dV_j += P dO_i, dK_j += scale dS q_i,
// dQ_i += scale dS k_j. Deterministic: no atomics.
//
// Four launches:
//   * D: D_i = do_i.o_i for every query row, written into the first element of that row of
//     dQ (dQ is written in full by the last launch, so it serves as the scratch row store).
//   * dV pass and dK pass (one kernel, two instantiations): wave w owns 32 keys of the
//     workgroup's 128, with its keys' K (and, for dK, V) held as B operands in registers and
//     one transposed accumulator (dV^T or dK^T, head_dim x 32 keys). The workgroup walks
//     every query head of its GQA group and every 32-row query tile (causal: from its first
//     key on, the last tile first); Q and dO tiles are copied global -> LDS
//     (buffer_load_dwordx4 ... lds), double-buffered. S = Q K^T and dP = dO V^T leave P and
//     dS in the accumulator layout, whose register kk of lane l holds query row
//     8(kk/4) + 4(l/32) + kk%4: exactly the contraction index that the B operand of the
//     next product takes at step kk, so dV^T += dO^T P and dK^T += Q^T dS read P / dS
//     straight from registers and their A operands (dO^T, Q^T) as 4-byte column reads of
//     the staged tiles.
//   * dQ: wave w owns 32 query rows (Q and dO as B operands in registers, LSE_i and D_i per
//     lane) and walks the key tiles (causal: up to its last row): S^T = K Q^T,
//     dP^T = V dO^T, dQ^T += K^T dS^T with K^T as column reads of the K tile.
// Products: lane l holds A[l % 32][l / 32] and B[l / 32][l % 32]; C as for every 32x32
// product (register r: row 8(r/4) + 4(l/32) + r%4, column l % 32). The head_dim contraction
// of S, dP, S^T, dP^T is split by lane half (half h supplies dimension h D/2 + ks at step ks),
// so the row reads of a tile are 16-byte reads of 4 consecutive dimensions.
// Tiles are 32 rows of head_dim floats, 16-byte chunk c of row r stored at c ^ swz(r), swz
// swapping bits 2 and 3 of r % 16: a bijection on 16 rows (each 16-lane pass of the row reads
// hits 16 distinct chunk slots) that puts rows 4 apart — the two lane halves of a column read
// — 8 chunks apart, in the other half of the banks.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_bwd.h"
#include "attn_mfma.h"

namespace aule {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBW = 4;               // waves per workgroup
constexpr int kBT = kBW * 64;        // threads per workgroup
constexpr float kLog2e = 1.4426950408889634f;

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ int swz_b(int row) {
    const int r = row & 15;
    return (r & 3) | ((r & 4) << 1) | ((r >> 1) & 4);
}

// Per-lane source offsets of the copy of a 32-row tile (NI instructions per wave, slot
// (wave NI + i) 64 + lane): the global chunk that belongs at the lane's LDS slot, or an
// out-of-range offset for chunks past head_dim.
template <int KC, int NI>
__device__ __forceinline__ void tile_offsets(uint32_t (&off)[NI], int wave, int lane, uint32_t rs, int hd) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int slot = (wave * NI + i) * 64 + lane;
        const int row = slot / KC, c = (slot % KC) ^ swz_b(row);
        off[i] = c * 4 < hd ? row * rs + c * 16 : kOobOffset;
    }
}
template <int NI>
__device__ __forceinline__ void copy_tile(i32x4 rsrc, const uint32_t (&off)[NI], uint32_t base, const f32x4* dst, int wave) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const uint32_t slot = (uint32_t)(wave * NI + i) * 64u * 16u;
        lds_copy16(rsrc, off[i] + base,
                   __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void*)dst + slot));
    }
}
// all waves past their reads of the previous tile, and this wave's copies landed
__device__ __forceinline__ void tile_barrier() {
    __builtin_amdgcn_s_waitcnt(0x70);   // vmcnt(0) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}
#endif

// D_i = do_i . o_i into dq[row * head_dim]: 16 lanes per row, 8 dimensions each.
__global__ __launch_bounds__(256) void attn_bwd_f32_delta_kernel(BwdProblem p, int64_t rows) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15, d = p.head_dim;
    float x = 0.f;
    if (row < rows && sub * 8 < d) {
        const f32x4* a = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.do_) + row * d + sub * 8);
        const f32x4* b = reinterpret_cast<const f32x4*>(static_cast<const float*>(p.o) + row * d + sub * 8);
        const f32x4 a0 = a[0], a1 = a[1], b0 = b[0], b1 = b[1];
        x = (a0[0] * b0[0] + a0[1] * b0[1]) + (a0[2] * b0[2] + a0[3] * b0[3]) +
            ((a1[0] * b1[0] + a1[1] * b1[1]) + (a1[2] * b1[2] + a1[3] * b1[3]));
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    if (row < rows && sub == 0) static_cast<float*>(p.dq)[row * d] = x;
#endif
}

// Waves per SIMD: the dK pass and the dQ kernel at head_dim 128 hold 192 registers of
// operands and accumulators for the whole walk plus two 16-register score tiles, past the
// 256 of two waves per SIMD (spilling ~100), so they run one wave per SIMD with the whole
// register file; each of their products takes 64 cycles against little vector work.
template <int D, int PASS> constexpr int kv_waves_per_simd() { return D == 128 && PASS == 1 ? 1 : 2; }

// PASS 0: dV^T += dO^T P; PASS 1: dK^T += Q^T dS.
template <int D, int PASS>
__global__ __launch_bounds__(kBT) __attribute__((amdgpu_waves_per_eu(kv_waves_per_simd<D, PASS>())))
void attn_bwd_f32_kv_kernel(BwdProblem p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int KC = D / 4, HALF = D / 2, DB = D / 32, TC = 32 * KC, NI = TC / kBT;
    static_assert(NI >= 1 && NI * kBT == TC, "head_dim 64 or 128");
    __shared__ f32x4 sQ[2][TC];
    __shared__ f32x4 sdO[2][TC];
    __shared__ __attribute__((aligned(16))) float sL[2][32];
    __shared__ __attribute__((aligned(16))) float sD[2][32];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, ln = lane & 31;
    const int Nq = p.seqlen_q, Nk = p.seqlen_k, d = p.head_dim, G = p.group;
    const uint32_t rs = (uint32_t)(d * 4);
    // flat grid, key blocks slowest (causal: block 0 walks every query tile, so the longest
    // workgroups start first); the key blocks of one (batch, kv head) are batch * heads_kv
    // apart, which keeps them on one XCD when that count is a multiple of 8
    const int per_kb = p.heads_kv * p.batch;
    const int kb = blockIdx.x / per_kb, rem = blockIdx.x - kb * per_kb;
    const int hk = rem % p.heads_kv, b = rem / p.heads_kv;
    const int j0 = kb * 32 * kBW;
    const int key = j0 + 32 * wave + ln;   // this lane's key (column of S, dP)
    const int64_t kv_off = ((int64_t)b * p.heads_kv + hk) * Nk * d;
    const int i_start = p.causal ? j0 : 0;
    const int ntile = Nq > i_start ? (Nq - i_start + 31) / 32 : 0;
    const int nit = G * ntile;

    // this lane's key: half h of its dimensions, as B operands
    float kreg[HALF], vreg[PASS == 1 ? HALF : 1];
    if (nit > 0) {
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(static_cast<const float*>(p.k) + kv_off), (short)0, Nk * d * 4, (int)kBufferFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(static_cast<const float*>(p.v) + kv_off), (short)0, Nk * d * 4, (int)kBufferFlags);
#pragma unroll
        for (int j = 0; j < HALF / 4; ++j) {
            const int col = h * HALF + 4 * j;
            const uint32_t off = col < d && key < Nk ? (uint32_t)key * rs + col * 4 : kOobOffset;
            const f32x4 x = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, (int)off, 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) kreg[4 * j + e] = x[e];
            if constexpr (PASS == 1) {
                const f32x4 y = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, (int)off, 0, 0));
#pragma unroll
                for (int e = 0; e < 4; ++e) vreg[4 * j + e] = y[e];
            }
        }
    }
    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    const float c2 = p.scale * kLog2e;

    uint32_t toff[NI];
    tile_offsets<KC, NI>(toff, wave, lane, rs, d);
    // iteration it: query tile (counted from the last) it / G, head g = it % G
    auto tile_of = [&](int it, int& i0, int64_t& bh) {
        const int tr = it / G, g = it - tr * G;
        i0 = i_start + 32 * (ntile - 1 - tr);
        bh = (int64_t)b * p.heads_q + (int64_t)hk * G + g;
    };
    float lnext = 0.f, dnext = 0.f;   // threads < 32: LSE log2(e) and D of the next tile's rows
    auto fetch = [&](int it, int buf) {
        int i0;
        int64_t bh;
        tile_of(it, i0, bh);
        const int64_t q_off = bh * Nq * d;
        const i32x4 rq = buffer_desc(static_cast<const float*>(p.q) + q_off, Nq * d * 4);
        const i32x4 rdo = buffer_desc(static_cast<const float*>(p.do_) + q_off, Nq * d * 4);
        copy_tile<NI>(rq, toff, (uint32_t)i0 * rs, sQ[buf], wave);
        copy_tile<NI>(rdo, toff, (uint32_t)i0 * rs, sdO[buf], wave);
        const int t = (int)threadIdx.x;
        if (t < 32) {
            const int i = i0 + t;
            lnext = i < Nq ? p.lse[bh * Nq + i] * kLog2e : 0.f;
            if constexpr (PASS == 1) dnext = i < Nq ? static_cast<const float*>(p.dq)[(bh * Nq + i) * d] : 0.f;
        }
    };
    auto commit_small = [&](int buf) {
        const int t = (int)threadIdx.x;
        if (t < 32) {
            sL[buf][t] = lnext;
            if constexpr (PASS == 1) sD[buf][t] = dnext;
        }
    };

    auto body = [&](int it, int buf) {
        tile_barrier();   // tile it (copies and row terms) visible; tile it-1's buffer free
        if (it + 1 < nit) fetch(it + 1, buf ^ 1);
        int i0;
        int64_t bh;
        tile_of(it, i0, bh);
        // S = Q K^T (and dP = dO V^T): register r of lane (ln, h) holds query
        // i0 + 8(r/4) + 4h + r%4 and key `key`
        f32x16 s = f32x16{}, dp = f32x16{};
        const f32x4* qt = sQ[buf] + ln * KC;
        const f32x4* dt = sdO[buf] + ln * KC;
#pragma unroll
        for (int j = 0; j < HALF / 4; ++j) {
            const int c = (h * (HALF / 4) + j) ^ swz_b(ln);
            const f32x4 qv = qt[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_32x32x2f32(qv[e], kreg[4 * j + e], s, 0, 0, 0);
            if constexpr (PASS == 1) {
                const f32x4 dv = dt[c];
#pragma unroll
                for (int e = 0; e < 4; ++e) dp = __builtin_amdgcn_mfma_f32_32x32x2f32(dv[e], vreg[4 * j + e], dp, 0, 0, 0);
            }
            // a few reads in flight at a time: hoisting all of them (the scheduler's choice)
            // needs more registers than the operands and accumulators leave
            if (j % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
        // P (and dS); row terms of 4 consecutive rows as one 16-byte read
        const bool inner = i0 + 32 <= Nq && j0 + 32 * kBW <= Nk && (!p.causal || j0 + 32 * kBW - 1 <= i0);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            const int q0 = 8 * g4 + 4 * h;
            const f32x4 lq = *reinterpret_cast<const f32x4*>(&sL[buf][q0]);
            f32x4 dq4 = {};
            if constexpr (PASS == 1) dq4 = *reinterpret_cast<const f32x4*>(&sD[buf][q0]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e;
                float pv = __builtin_amdgcn_exp2f(s[r] * c2 - lq[e]);
                if (!inner) {
                    const int qi = i0 + q0 + e;
                    const bool vis = qi < Nq && key < Nk && (!p.causal || key <= qi);
                    pv = vis ? pv : 0.f;
                }
                s[r] = PASS == 1 ? pv * (dp[r] - dq4[e]) : pv;
            }
        }
        // dV^T += dO^T P or dK^T += Q^T dS: at step kk the contraction takes tile row
        // 8(kk/4) + 4h + kk%4; the A operand is column 32db + ln of that row
        const float* src = reinterpret_cast<const float*>(PASS == 1 ? sQ[buf] : sdO[buf]);
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int row = 8 * (kk >> 2) + 4 * h + (kk & 3);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int chunk = (8 * db + (ln >> 2)) ^ swz_b(row);
                const float a = src[(row * KC + chunk) * 4 + (ln & 3)];
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kk], acc[db], 0, 0, 0);
            }
            if (kk % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
        if (it + 1 < nit) commit_small(buf ^ 1);
    };
    if (nit > 0) {
        fetch(0, 0);
        commit_small(0);
    }
    for (int it = 0; it < nit; it += 2) {
        body(it, 0);
        if (it + 1 < nit) body(it + 1, 1);
    }
    // dV[key] = dV^T column, dK[key] = scale dK^T column: four consecutive dimensions per
    // 16-byte store
    if (key < Nk) {
        float* dst = static_cast<float*>(PASS == 1 ? p.dk : p.dv) + kv_off + (int64_t)key * d;
        const float mul = PASS == 1 ? p.scale : 1.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * db + 8 * g + 4 * h;
                if (col < d)
                    *reinterpret_cast<f32x4*>(dst + col) = f32x4{acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul,
                                                                 acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul};
            }
    }
#endif
}

template <int D>
__global__ __launch_bounds__(kBT) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2)))
void attn_bwd_f32_dq_kernel(BwdProblem p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int KC = D / 4, HALF = D / 2, DB = D / 32, TC = 32 * KC, NI = TC / kBT;
    __shared__ f32x4 sK[2][TC];
    __shared__ f32x4 sV[2][TC];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, ln = lane & 31;
    const int Nq = p.seqlen_q, Nk = p.seqlen_k, d = p.head_dim;
    const uint32_t rs = (uint32_t)(d * 4);
    // flat grid, query blocks slowest, causal: the last (longest) block first; the G query
    // heads of one (batch, kv head) are batch * heads_kv apart (one XCD when a multiple of 8)
    const int per_qb = p.heads_q * p.batch;
    const int t_ = blockIdx.x / per_qb, rem = blockIdx.x - t_ * per_qb;
    const int nqb = (Nq + 32 * kBW - 1) / (32 * kBW);
    const int qblk = p.causal ? nqb - 1 - t_ : t_;
    const int nkvu = p.batch * p.heads_kv;
    const int gi = rem / nkvu, u = rem - gi * nkvu;
    const int b = u / p.heads_kv, hq = (u - b * p.heads_kv) * p.group + gi;
    const int hk = hq / p.group;
    const int i0 = qblk * 32 * kBW;
    const int qi = i0 + 32 * wave + ln;   // this lane's query
    const int64_t bh = (int64_t)b * p.heads_q + hq;
    const int64_t q_off = bh * Nq * d;
    const int64_t kv_off = ((int64_t)b * p.heads_kv + hk) * Nk * d;

    // Q and dO of this lane's query (half h of the dimensions) as B operands; D from O
    float qreg[HALF], doreg[HALF];
    float delta;
    {
        const int nb = Nq * d * 4;
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(static_cast<const float*>(p.q) + q_off), (short)0, nb, (int)kBufferFlags);
        const __amdgpu_buffer_rsrc_t rdo = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(static_cast<const float*>(p.do_) + q_off), (short)0, nb, (int)kBufferFlags);
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(static_cast<const float*>(p.o) + q_off), (short)0, nb, (int)kBufferFlags);
        float x = 0.f;
#pragma unroll
        for (int j = 0; j < HALF / 4; ++j) {
            const int col = h * HALF + 4 * j;
            const uint32_t off = col < d && qi < Nq ? (uint32_t)qi * rs + col * 4 : kOobOffset;
            const f32x4 a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)off, 0, 0));
            const f32x4 c = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rdo, (int)off, 0, 0));
            const f32x4 o = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(ro, (int)off, 0, 0));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qreg[4 * j + e] = a[e];
                doreg[4 * j + e] = c[e];
            }
            x += (c[0] * o[0] + c[1] * o[1]) + (c[2] * o[2] + c[3] * o[3]);
        }
        delta = x + __shfl_xor(x, 32);   // the other half of the row
    }
    const float lse2 = qi < Nq ? p.lse[bh * Nq + qi] * kLog2e : 0.f;
    const float c2 = p.scale * kLog2e;

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};

    const int j_end = p.causal ? min(Nk, i0 + 32 * kBW) : Nk;
    const int nkt = (j_end + 31) / 32;
    const i32x4 rk = buffer_desc(static_cast<const float*>(p.k) + kv_off, Nk * d * 4);
    const i32x4 rv = buffer_desc(static_cast<const float*>(p.v) + kv_off, Nk * d * 4);
    uint32_t toff[NI];
    tile_offsets<KC, NI>(toff, wave, lane, rs, d);
    auto fetch = [&](int t, int buf) {
        copy_tile<NI>(rk, toff, (uint32_t)(32 * t) * rs, sK[buf], wave);
        copy_tile<NI>(rv, toff, (uint32_t)(32 * t) * rs, sV[buf], wave);
    };
    const int qw0 = i0 + 32 * wave;   // this wave's first query row
    auto body = [&](int t, int buf) {
        tile_barrier();
        if (t + 1 < nkt) fetch(t + 1, buf ^ 1);
        // S^T = K Q^T, dP^T = V dO^T: register r holds key 32t + 8(r/4) + 4h + r%4, query qi
        f32x16 s = f32x16{}, dp = f32x16{};
        const f32x4* kt = sK[buf] + ln * KC;
        const f32x4* vt = sV[buf] + ln * KC;
#pragma unroll
        for (int j = 0; j < HALF / 4; ++j) {
            const int c = (h * (HALF / 4) + j) ^ swz_b(ln);
            const f32x4 kv = kt[c], vv = vt[c];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qreg[4 * j + e], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[e], doreg[4 * j + e], dp, 0, 0, 0);
            }
            if (j % 2 == 1) __builtin_amdgcn_sched_barrier(0);   // a few reads in flight at a time
        }
        const bool inner = qw0 + 32 <= Nq && 32 * t + 32 <= Nk && (!p.causal || 32 * t + 31 <= qw0);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float pv = __builtin_amdgcn_exp2f(s[r] * c2 - lse2);
            if (!inner) {
                const int kj = 32 * t + 8 * (r >> 2) + 4 * h + (r & 3);
                const bool vis = qi < Nq && kj < Nk && (!p.causal || kj <= qi);
                pv = vis ? pv : 0.f;
            }
            s[r] = pv * (dp[r] - delta);
        }
        // dQ^T += K^T dS^T: at step kk the contraction takes key 8(kk/4) + 4h + kk%4 of the
        // tile; the A operand is column 32db + ln of that K row
        const float* ksrc = reinterpret_cast<const float*>(sK[buf]);
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) {
            const int row = 8 * (kk >> 2) + 4 * h + (kk & 3);
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int chunk = (8 * db + (ln >> 2)) ^ swz_b(row);
                const float a = ksrc[(row * KC + chunk) * 4 + (ln & 3)];
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kk], acc[db], 0, 0, 0);
            }
            if (kk % 2 == 1) __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (nkt > 0) fetch(0, 0);
    for (int t = 0; t < nkt; t += 2) {
        body(t, 0);
        if (t + 1 < nkt) body(t + 1, 1);
    }
    if (qi < Nq) {
        float* dst = static_cast<float*>(p.dq) + q_off + (int64_t)qi * d;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = 32 * db + 8 * g + 4 * h;
                if (col < d)
                    *reinterpret_cast<f32x4*>(dst + col) = f32x4{acc[db][4 * g] * p.scale, acc[db][4 * g + 1] * p.scale,
                                                                 acc[db][4 * g + 2] * p.scale, acc[db][4 * g + 3] * p.scale};
            }
    }
#endif
}

template <int D>
hipError_t launch_d(const BwdProblem& p, hipStream_t stream) {
    const int R = 32 * kBW;
    const int64_t nk = (int64_t)((p.seqlen_k + R - 1) / R) * p.heads_kv * p.batch;
    const int64_t nq = (int64_t)((p.seqlen_q + R - 1) / R) * p.heads_q * p.batch;
    const int64_t rows = (int64_t)p.batch * p.heads_q * p.seqlen_q;
    if (nk > INT32_MAX || nq > INT32_MAX || (rows + 15) / 16 > INT32_MAX) return hipErrorInvalidConfiguration;
    hipError_t e;
    if (rows > 0) {   // D into the rows of dQ, before the dK pass reads it
        hipLaunchKernelGGL(attn_bwd_f32_delta_kernel, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, p, rows);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (nk > 0) {
        hipLaunchKernelGGL((attn_bwd_f32_kv_kernel<D, 0>), dim3((unsigned)nk), dim3(kBT), 0, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL((attn_bwd_f32_kv_kernel<D, 1>), dim3((unsigned)nk), dim3(kBT), 0, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if (nq > 0) {
        hipLaunchKernelGGL((attn_bwd_f32_dq_kernel<D>), dim3((unsigned)nq), dim3(kBT), 0, stream, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace

bool bwd_f32_mfma_supports(const BwdProblem& p) {
    // one (batch, head) slice addressed with 32-bit buffer offsets, plus a tile of headroom
    const int64_t rows = (p.seqlen_q > p.seqlen_k ? p.seqlen_q : p.seqlen_k) + 32;
    return p.head_dim <= 128 && p.head_dim % 8 == 0 && rows * p.head_dim * 4 < (int64_t(1) << 30);
}

hipError_t launch_attn_bwd_f32_mfma(const BwdProblem& p, hipStream_t stream) {
    if (p.head_dim <= 64) return launch_d<64>(p, stream);
    return launch_d<128>(p, stream);
}

}  // namespace aule
