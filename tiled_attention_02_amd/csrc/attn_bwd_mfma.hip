// Attention backward (dQ, dK, dV) on the matrix cores, fp16/bf16 inputs, fp32 accumulation.
//
// The score matrix is recomputed tile by tile from Q, K and the forward's per-row
// log-sum-exp (FlashAttention-T commentary, ai-stack.site, FAQ 4, training bullet). Per
// (query i, key j) pair: P = exp2(scale log2(e) q_i.k_j - LSE_i log2(e)) (0 where masked),
// dP = do_i.v_j, dS = P (dP - D_i) with D_i = do_i.o_i; dV_j += P dO_i,
// dK_j += scale dS q_i, dQ_i += scale dS k_j.
//
// Four launches, no atomics (deterministic), 32-row / 32-key steps:
//   * D pre-pass: D_i = do_i . o_i (fp32) into the first 4 bytes of row i of dq, which holds
//     it until the dQ kernel, launched last, writes dq in full.
//   * dV pass and dK pass (one kernel, two instantiations) and dQ, each with WV = 8 waves per
//     workgroup at head_dim 128, 4 at 64.
//   * dV / dK pass: wave w owns 32 keys (its K rows and, for dK, its V rows held as B operands
//     in registers) and one transposed accumulator (dV^T or dK^T, d x 32 keys). The workgroup
//     walks every query head of its GQA group and every query tile (causal: from its first
//     key on). Per 32-row half: S = Q K^T (and dP = dO V^T) with Q / dO rows fed in sigma
//     order, so P and dS leave the accumulators already in the B-operand layout of
//     dV^T += dO^T P and dK^T += Q^T dS, whose A operands (dO^T, Q^T) are transposing LDS
//     reads (ds_read_b64_tr_b16).
//   * dQ: wave w owns 32 query rows (Q and dO rows in registers, LSE_i and D_i per lane); the
//     workgroup walks the key tiles (causal: up to its last row). Per 32-key half:
//     S^T = K Q^T, dP^T = V dO^T with K / V rows in sigma order, then dQ^T += K^T dS^T with
//     K^T read transposed from LDS.
// Every staged tile (Q and dO, or K and V) is copied global -> LDS by the buffer unit, in the
// XOR-swizzled layout of the read that uses it (twice when it is read both ways), two 32-row
// halves per barrier, double-buffered: the next tile's copies are issued right after the
// barrier that starts a tile.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn_bwd.h"
#include "attn_mfma.h"

namespace aule {
namespace {

// 32-row query tiles (dV, dK) or 32-key tiles (dQ) per barrier, and LDS buffers, measured on
// the bf16 causal GQA backward (B4 Hq32 Hkv8 N4096, head_dim 128, and the same at 64): two
// tiles, double-buffered, in all three (four tiles, triple buffering or one tile per barrier
// were 1-5% slower at head_dim 128; the triple-buffered dK pass 7% slower at 64).
constexpr int kTiles = 2, kBufs = 2;
constexpr float kLog2eF = 1.4426950408889634f;

template <int D>
struct Tile {
    static constexpr int RS = D * 2;                      // bytes per LDS row
    static constexpr int CPR = D / 8;                     // 16-byte chunks per row
    static constexpr int BYTES = 32 * RS;                 // one 32-row tile
    static constexpr int KS = D / 16;                     // k-steps over head_dim
    static constexpr int DB = D / 32;                     // 32-row blocks of head_dim
};

// Two LDS layouts of a 32-row tile, one per read pattern, with the XOR swizzles of the
// forward kernel's K and V tiles (chunk c of row r stored at chunk c ^ swz(r)):
//   ROWS: rd_rows reads one chunk of rows sigma(0..31) per instruction -> kswz;
//   COLS: rd_cols reads 4 consecutive rows x 2 neighbouring chunks per 16 lanes -> vswz.
// A tile read both ways is stored twice.
enum Layout { ROWS = 0, COLS = 1 };
template <int D, int L>
__device__ __forceinline__ int swz(int row) {
    if constexpr (L == ROWS) return kswz<D / 8>(row);
    else return vswz<D / 8>(row);
}

// A operand with rows in sigma order from a ROWS tile: lane l supplies row sigma(l % 32),
// k-chunk 2ks + h (stored at chunk (2ks + h) ^ kswz(sigma(l % 32)) = (2ks + h) ^ kx_lane(l % 32)).
template <int D>
__device__ __forceinline__ u32x4 rd_rows(const char* tile, int ks, int lane) {
    const int l32 = lane & 31;
    const int x = kx_lane<Tile<D>::CPR>(l32);
    return *reinterpret_cast<const u32x4*>(tile + sigma(l32) * Tile<D>::RS + (((2 * ks + (lane >> 5)) ^ x) * 16));
}
// A operand of a transposed COLS tile: A[m = column 32db + l % 32][k = row 16kk + 8h .. + 7],
// two transposing 8-byte reads (each 16-lane group reads 4 rows x 16 columns); vswz depends
// on the row modulo 4 only, the same for both reads.
template <int D>
__device__ __forceinline__ u32x4 rd_cols(const char* tile, int db, int kk, int lane) {
    const int tg = lane >> 4, tc = lane & 15;
    const int row0 = 16 * kk + 8 * (tg >> 1) + (tc >> 2);
    const int x = vswz<D / 8>(row0);
    const int coff = ((4 * db + 2 * (tg & 1) + ((tc & 3) >> 1)) ^ x) * 16 + (tc & 1) * 8;
    u32x4 out;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const char* addr = tile + (row0 + 4 * t) * Tile<D>::RS + coff;
        const i16x4_t part = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<char*>(addr)));
        const u32x2 w = __builtin_bit_cast(u32x2, part);
        out[2 * t] = w[0];
        out[2 * t + 1] = w[1];
    }
    return out;
}

// One row (this lane's) of a [rows, d] slice as B-operand chunks: chunk 2ks + h of row r.
template <typename T, int D>
__device__ __forceinline__ void fetch_operand(u32x4 (&f)[Tile<D>::KS], const T* base, int r, int rows, int d, int h) {
#pragma unroll
    for (int ks = 0; ks < Tile<D>::KS; ++ks) {
        const int col = (2 * ks + h) * 8;
        f[ks] = (r < rows && col < d) ? *reinterpret_cast<const u32x4*>(base + (int64_t)r * d + col)
                                      : u32x4{0u, 0u, 0u, 0u};
    }
}

// Transposed accumulators (register r of block db: column 32db + 8(r/4) + 4h + r%4 of this
// lane's row) scaled and rounded to T, four consecutive columns per 8-byte store.
template <typename T, int D>
__device__ __forceinline__ void store_rowT(T* row, const f32x16 (&acc)[Tile<D>::DB], float mul, int d, int h) {
#pragma unroll
    for (int db = 0; db < Tile<D>::DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int c0 = 32 * db + 8 * q4 + 4 * h;
            if (c0 < d) {
                const u32x2 w = {Mfma<T>::pack2(acc[db][4 * q4] * mul, acc[db][4 * q4 + 1] * mul),
                                 Mfma<T>::pack2(acc[db][4 * q4 + 2] * mul, acc[db][4 * q4 + 3] * mul)};
                *reinterpret_cast<u32x2*>(row + c0) = w;
            }
        }
}

#if defined(__HIP_DEVICE_COMPILE__)
// One 4-byte global -> LDS copy per lane: LDS[m0 + 4 * lane] = buffer[voffset] (zero past the
// descriptor's size); inline asm for the same reason as lds_copy16, M0 saved and restored.
__device__ __forceinline__ void lds_copy4(i32x4 rsrc, uint32_t voffset, uint32_t lds_addr) {
    uint32_t saved_m0;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dword %1, %2, 0 offen lds\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved_m0)
        : "v"(voffset), "s"(rsrc), "s"(lds_addr));
}
#endif

// D_i = do_i . o_i (fp32) into the first 4 bytes of row i of dq, which the dQ kernel writes in
// full afterwards: 16 lanes per row, 8 dimensions each.
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(BwdProblem p, int64_t rows) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int sub = threadIdx.x & 15, d = p.head_dim;
    float x = 0.f;
    if (row < rows && sub * 8 < d) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(static_cast<const T*>(p.do_) + row * d + sub * 8);
        const u32x4 b = *reinterpret_cast<const u32x4*>(static_cast<const T*>(p.o) + row * d + sub * 8);
#pragma unroll
        for (int w = 0; w < 4; ++w) x = Mfma<T>::dot2(a[w], b[w], x);
    }
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m);
    if (row < rows && sub == 0) *reinterpret_cast<float*>(static_cast<T*>(p.dq) + row * d) = x;
#endif
}

// The dV pass (PASS 0: S and dV^T += dO^T P) and the dK pass (PASS 1: S, dP and
// dK^T += Q^T dS). One gradient per pass halves the accumulators, so each pass fits two waves
// per SIMD, whose matrix products then overlap the other wave's exponentials; the price is S
// computed twice. WV waves own 32 keys each (K rows, and V rows for dK, held as B operands in
// registers): the Q / dO rows of the group are read once per 32 * WV keys.
//
// The query tiles are copied global -> LDS by the buffer unit (buffer_load ... lds), no
// register staging: per 32-row half, Q in the ROWS layout, dO in the COLS layout (dV) or Q in
// the COLS and dO in the ROWS layout (dK), one 16-byte chunk per lane each, and the rows'
// LSE (and D, from the pre-pass, in dq) as 4-byte copies. QH halves are staged per barrier;
// NBUF buffers, the copies of tile it + NBUF - 1 issued right after the barrier that starts
// tile it. Every wave issues the same number of copies per tile, so one explicit vmcnt per
// tile orders them.
template <typename T, int D, int PASS, int WV, int QH, int NBUF>
__global__ __launch_bounds__(WV * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bwd_kv_mfma_kernel(BwdProblem p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int NT = WV * 64;
    using TL = Tile<D>;
    static_assert(32 * TL::CPR == NT, "one 16-byte chunk per thread per tile");
    static_assert(NBUF == 2 || NBUF == 3, "at most one later tile in flight at a barrier");
    constexpr int QR = 32 * QH;              // query rows per tile
    constexpr int NL = (QR + 63) / 64;       // 4-byte copies per row term (64 rows each)
    constexpr int NCOPY = QH * (PASS == 1 ? 3 : 2) + NL * (PASS == 1 ? 2 : 1);   // per wave and tile
    static_assert(NCOPY * (NBUF - 2) < 64, "vmcnt range");
    __shared__ __attribute__((aligned(16))) char sQ[NBUF][QH][TL::BYTES];    // ROWS
    __shared__ __attribute__((aligned(16))) char sdO[NBUF][QH][TL::BYTES];   // COLS (dV), ROWS (dK)
    __shared__ __attribute__((aligned(16))) char sQc[PASS == 1 ? NBUF : 1][QH][PASS == 1 ? TL::BYTES : 16];
    __shared__ __attribute__((aligned(16))) float sL[NBUF][64 * NL];                  // LSE
    __shared__ __attribute__((aligned(16))) float sD[PASS == 1 ? NBUF : 1][64 * NL];  // D

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5;
    const int Nq = p.seqlen_q, Nk = p.seqlen_k, d = p.head_dim, G = p.group;
    const uint32_t rs = (uint32_t)(d * (int)sizeof(T));
    // (key block, group) of this workgroup; group = (batch, kv head). Workgroups go to the 8
    // XCDs round-robin (blockIdx % 8). At head_dim 128 (one workgroup per CU) with S groups'
    // key blocks filling an XCD's 32 CUs exactly, each XCD takes whole groups, S at a time,
    // their key blocks interleaved and longest first (under causal masking block 0 walks
    // every query tile, later blocks fewer). The first set's blocks start together and walk
    // the query tiles from the last one down, all on the same tile; the next set's blocks
    // start one by one as the short blocks free their CUs, longest first, so every CU ends at
    // about the same time, and walk upwards from their first key, which puts them too on one
    // common tile at any moment (block k starts when the front reaches its first tile). Each
    // Q / dO tile is then read from HBM about once per set. Otherwise key blocks slowest,
    // groups fastest, every walk downwards.
    const int ng = p.heads_kv * p.batch, nkb = (int)(gridDim.x / (unsigned)ng);
    const int S = D == 128 && nkb <= 32 ? 32 / nkb : 0;
    int kb, grp;
    bool up = false;
    if (ng % 8 == 0 && S > 0 && S * nkb == 32 && (ng / 8) % S == 0) {
        const int x = blockIdx.x % 8, idx = blockIdx.x / 8;
        const int set = idx / 32, r = idx - set * 32;
        kb = r / S;
        grp = x + 8 * (set * S + (r - kb * S));
        up = (set & 1) != 0;
    } else {
        kb = blockIdx.x / ng;
        grp = blockIdx.x - kb * ng;
    }
    const int hk = grp % p.heads_kv, b = grp / p.heads_kv;
    const int j0 = kb * 32 * WV;
    const int key = j0 + 32 * wave + (lane & 31);   // this lane's key (B-operand column)
    const int64_t kv_off = ((int64_t)b * p.heads_kv + hk) * Nk * d;
    // work: (QR-row query tile, query head g of the group), causal from the first key on,
    // the group's heads inner, the tiles in the direction chosen above, so that the
    // workgroups of one (batch, kv head), which run on one XCD, read the same Q / dO tile at
    // about the same time and share it through that XCD's L2. With no query rows (nit == 0)
    // only the zero gradients are written: q, k, v, o, do and lse may then be null and are
    // not read.
    const int i_start = p.causal ? j0 : 0;
    const int ntile = Nq > i_start ? (Nq - i_start + QR - 1) / QR : 0;
    const int nit = G * ntile;

    u32x4 kf[TL::KS], vf[PASS == 1 ? TL::KS : 1];
    if (nit > 0) {
        fetch_operand<T, D>(kf, static_cast<const T*>(p.k) + kv_off, key, Nk, d, h);
        if constexpr (PASS == 1) fetch_operand<T, D>(vf, static_cast<const T*>(p.v) + kv_off, key, Nk, d, h);
    }
    f32x16 acc[TL::DB];   // dV^T (PASS 0) or dK^T (PASS 1)
#pragma unroll
    for (int db = 0; db < TL::DB; ++db) acc[db] = f32x16{};
    const float c2 = p.scale * kLog2eF;

    // this lane's chunk of a tile in each layout: slot wave * 64 + lane of the LDS image
    // holds chunk slot % CPR of row slot / CPR, which is global chunk (slot % CPR) ^ swz(row)
    uint32_t off_rows, off_cols;
    {
        const int slot = wave * 64 + lane;
        const int row = slot / TL::CPR, pc = slot % TL::CPR;
        const int cr = pc ^ swz<D, ROWS>(row), cc = pc ^ swz<D, COLS>(row);
        off_rows = cr * 8 < d ? row * rs + cr * 16 : kOobOffset;
        off_cols = cc * 8 < d ? row * rs + cc * 16 : kOobOffset;
    }
    const uint32_t off_q = off_rows, off_do = PASS == 0 ? off_cols : off_rows;
    auto lds_addr = [](const void* q) { return (uint32_t)(uintptr_t)(lds_void*)q; };
    auto tile_of = [&](int it, int& i0, int64_t& bh) {
        const int tr = it / G, g = it - tr * G;
        i0 = i_start + QR * (up ? tr : ntile - 1 - tr);
        bh = (int64_t)b * p.heads_q + (int64_t)hk * G + g;
    };
    auto issue = [&](int it, int buf) {
        int i0;
        int64_t bh;
        tile_of(it, i0, bh);
        const int64_t q_off = bh * Nq * d;
        const int nb = Nq * (int)rs;
        const i32x4 rq = buffer_desc(static_cast<const T*>(p.q) + q_off, nb);
        const i32x4 rdo = buffer_desc(static_cast<const T*>(p.do_) + q_off, nb);
        const uint32_t slot = (uint32_t)wave * 1024u;
#pragma unroll
        for (int hf = 0; hf < QH; ++hf) {
            const uint32_t base = (uint32_t)(i0 + 32 * hf) * rs;
            lds_copy16(rq, off_q + base, __builtin_amdgcn_readfirstlane(lds_addr(sQ[buf][hf]) + slot));
            if constexpr (PASS == 1)
                lds_copy16(rq, off_cols + base, __builtin_amdgcn_readfirstlane(lds_addr(sQc[buf][hf]) + slot));
            lds_copy16(rdo, off_do + base, __builtin_amdgcn_readfirstlane(lds_addr(sdO[buf][hf]) + slot));
        }
        // every wave copies the same row terms (identical bytes), which keeps the copy count
        // uniform across waves; rows past the tile or the sequence read as zero
        const i32x4 rl = buffer_desc(p.lse + bh * Nq, Nq * 4);
#pragma unroll
        for (int c = 0; c < NL; ++c) {
            const int r = 64 * c + lane;
            lds_copy4(rl, r < QR ? (uint32_t)(i0 + r) * 4u : kOobOffset,
                      __builtin_amdgcn_readfirstlane(lds_addr(&sL[buf][64 * c])));
        }
        if constexpr (PASS == 1) {
            const i32x4 rd = buffer_desc(static_cast<const T*>(p.dq) + q_off, nb);
#pragma unroll
            for (int c = 0; c < NL; ++c) {
                const int r = 64 * c + lane;
                lds_copy4(rd, r < QR ? (uint32_t)(i0 + r) * rs : kOobOffset,
                          __builtin_amdgcn_readfirstlane(lds_addr(&sD[buf][64 * c])));
            }
        }
    };

    const int kw0 = j0 + 32 * wave;   // this wave's first key
    auto body = [&](int it, int buf) {
        // tile it landed everywhere (the copies of the NBUF - 2 later tiles may still be in
        // flight) and every wave is past tile it - 1, whose buffer takes tile it + NBUF - 1
        if (NBUF > 2 && it + 1 < nit) {
            constexpr int n = NCOPY * (NBUF - 2);
            __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));   // vmcnt(n) lgkmcnt(0)
        } else {
            __builtin_amdgcn_s_waitcnt(7 << 4);                                   // vmcnt(0) lgkmcnt(0)
        }
        asm volatile("s_barrier" ::: "memory");
        if (it + NBUF - 1 < nit) issue(it + NBUF - 1, (buf + NBUF - 1) % NBUF);
        int i0q;
        int64_t bh;
        tile_of(it, i0q, bh);
#pragma unroll
        for (int hf = 0; hf < QH; ++hf) {
            const int i0 = i0q + 32 * hf;
            // S = Q K^T, dP - D = dO V^T - D: register r holds query i0 + 16(r/8) + 8h + r%8,
            // key `key`; the dP accumulator starts from -D of its rows (two runs of 8
            // consecutive rows, 16-byte reads), so dS = P (dP - D) needs no further registers
            f32x16 s = f32x16{}, dp = f32x16{};
            if constexpr (PASS == 1) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const float4* pd = reinterpret_cast<const float4*>(&sD[buf][32 * hf + 16 * kk + 8 * h]);
                    const float4 x = pd[0], y = pd[1];
                    dp[8 * kk + 0] = -x.x; dp[8 * kk + 1] = -x.y; dp[8 * kk + 2] = -x.z; dp[8 * kk + 3] = -x.w;
                    dp[8 * kk + 4] = -y.x; dp[8 * kk + 5] = -y.y; dp[8 * kk + 6] = -y.z; dp[8 * kk + 7] = -y.w;
                }
            }
#pragma unroll
            for (int ks = 0; ks < TL::KS; ++ks) {
                s = Mfma<T>::mma(rd_rows<D>(sQ[buf][hf], ks, lane), kf[ks], s);
                if constexpr (PASS == 1) dp = Mfma<T>::mma(rd_rows<D>(sdO[buf][hf], ks, lane), vf[ks], dp);
            }
            // P (dV) or dS (dK) packed to 16 bit. The LSE of each run of 8 consecutive query
            // rows is read as two 16-byte vectors. Tiles away from the diagonal and the ends
            // need no mask: a uniform branch picks the mask-free form; on edge tiles every
            // exponential is taken and masked pairs are selected to 0 (no per-element branch).
            u32x4 bf[2];
            auto p_ds = [&](auto masked) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int q0 = 16 * kk + 8 * h;
                    const float4* pl = reinterpret_cast<const float4*>(&sL[buf][32 * hf + q0]);
                    const float4 a = pl[0], c = pl[1];
                    const float lq[8] = {a.x * kLog2eF, a.y * kLog2eF, a.z * kLog2eF, a.w * kLog2eF,
                                         c.x * kLog2eF, c.y * kLog2eF, c.z * kLog2eF, c.w * kLog2eF};
                    float v[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float x = fmaf(s[8 * kk + e], c2, -lq[e]);
                        if constexpr (decltype(masked)::value) {
                            const int qi = i0 + q0 + e;
                            const bool vis = qi < Nq && key < Nk && (!p.causal || key <= qi);
                            x = vis ? x : -INFINITY;   // exp2(-inf) = +0
                        }
                        const float pe = __builtin_amdgcn_exp2f(x);
                        v[e] = PASS == 1 ? pe * dp[8 * kk + e] : pe;
                    }
                    bf[kk] = u32x4{Mfma<T>::pack2(v[0], v[1]), Mfma<T>::pack2(v[2], v[3]),
                                   Mfma<T>::pack2(v[4], v[5]), Mfma<T>::pack2(v[6], v[7])};
                }
            };
            const bool inner = i0 + 32 <= Nq && kw0 + 32 <= Nk && (!p.causal || kw0 + 31 <= i0);
            if (inner) p_ds(std::false_type{});
            else p_ds(std::true_type{});
            // dV^T += dO^T P (PASS 0) or dK^T += Q^T dS (PASS 1)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int db = 0; db < TL::DB; ++db) {
                    if constexpr (PASS == 0) acc[db] = Mfma<T>::mma(rd_cols<D>(sdO[buf][hf], db, kk, lane), bf[kk], acc[db]);
                    else acc[db] = Mfma<T>::mma(rd_cols<D>(sQc[buf][hf], db, kk, lane), bf[kk], acc[db]);
                }
        }
    };
#pragma unroll
    for (int t = 0; t < NBUF - 1; ++t)
        if (t < nit) issue(t, t);
    for (int it = 0; it < nit; it += NBUF) {
#pragma unroll
        for (int t = 0; t < NBUF; ++t)
            if (it + t < nit) body(it + t, t);
    }
    if (key < Nk) {
        if constexpr (PASS == 1) store_rowT<T, D>(static_cast<T*>(p.dk) + kv_off + (int64_t)key * d, acc, p.scale, d, h);
        else store_rowT<T, D>(static_cast<T*>(p.dv) + kv_off + (int64_t)key * d, acc, 1.f, d, h);
    }
#endif
}

// dQ: wave w owns 32 query rows (its Q and dO rows held as B operands in registers, LSE_i and
// D_i per lane, D from the pre-pass) and one transposed accumulator dQ^T (d x 32 queries); the
// workgroup walks the key tiles (causal: up to its last row). The K and V tiles are copied
// global -> LDS by the buffer unit: per 32-key half, K in the ROWS and the COLS layout and V in
// the ROWS layout, one 16-byte chunk per lane each; KH halves per barrier, NBUF buffers, the
// copies of tile t + NBUF - 1 issued right after the barrier that starts tile t. Per half:
// S^T = K Q^T, dP^T = V dO^T with K / V rows in sigma order, then dQ^T += K^T dS^T with K^T
// read transposed; a wave skips the halves that lie wholly past its rows.
template <typename T, int D, int WQ, int KH, int NBUF>
__global__ __launch_bounds__(WQ * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bwd_dq_mfma_kernel(BwdProblem p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int NT = WQ * 64;
    using TL = Tile<D>;
    static_assert(32 * TL::CPR == NT, "one 16-byte chunk per thread per tile");
    static_assert(NBUF == 2 || NBUF == 3, "at most one later tile in flight at a barrier");
    constexpr int KR = 32 * KH;        // keys per tile
    constexpr int NCOPY = 3 * KH;      // copies per wave and tile
    __shared__ __attribute__((aligned(16))) char sK[NBUF][KH][TL::BYTES];    // ROWS
    __shared__ __attribute__((aligned(16))) char sKc[NBUF][KH][TL::BYTES];   // COLS
    __shared__ __attribute__((aligned(16))) char sV[NBUF][KH][TL::BYTES];    // ROWS

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5;
    const int Nq = p.seqlen_q, Nk = p.seqlen_k, d = p.head_dim;
    const uint32_t rs = (uint32_t)(d * (int)sizeof(T));
    // flat grid, query blocks slowest and (causal) last block first: the longest walks start
    // first. Within a block index the G query heads of one (batch, kv head) are
    // batch * heads_kv apart, which puts them on one XCD (sharing its L2 copy of that K/V)
    // when that count is a multiple of 8.
    const int per_qb = p.heads_q * p.batch;
    const int t_ = blockIdx.x / per_qb, rem = blockIdx.x - t_ * per_qb;
    const int nqb = (Nq + 32 * WQ - 1) / (32 * WQ);
    const int qblk = p.causal ? nqb - 1 - t_ : t_;
    const int nkvu = p.batch * p.heads_kv;
    const int gi = rem / nkvu, u = rem - gi * nkvu;
    const int b = u / p.heads_kv, hq = (u - b * p.heads_kv) * p.group + gi;
    const int i0 = qblk * 32 * WQ;
    const int hk = hq / p.group;
    const int qw0 = i0 + 32 * wave;                      // this wave's first query row
    const int qi = qw0 + (lane & 31);                    // this lane's query (B-operand column)
    const int64_t bh = (int64_t)b * p.heads_q + hq;
    const int64_t q_off = bh * Nq * d;
    const int64_t kv_off = ((int64_t)b * p.heads_kv + hk) * Nk * d;

    u32x4 qf[TL::KS], dof[TL::KS];
    fetch_operand<T, D>(qf, static_cast<const T*>(p.q) + q_off, qi, Nq, d, h);
    fetch_operand<T, D>(dof, static_cast<const T*>(p.do_) + q_off, qi, Nq, d, h);
    // D_i sits in the first 4 bytes of row i of dq until this kernel writes the row
    const float delta = qi < Nq ? *reinterpret_cast<const float*>(static_cast<const T*>(p.dq) + q_off + (int64_t)qi * d) : 0.f;
    const float lse2 = qi < Nq ? p.lse[bh * Nq + qi] * kLog2eF : 0.f;
    const float c2 = p.scale * kLog2eF;

    f32x16 dq[TL::DB];
#pragma unroll
    for (int db = 0; db < TL::DB; ++db) dq[db] = f32x16{};

    const int j_end = p.causal ? min(Nk, i0 + 32 * WQ) : Nk;
    const int nkt = (j_end + KR - 1) / KR;

    // this lane's chunk of a tile in each layout: slot wave * 64 + lane of the LDS image
    // holds chunk slot % CPR of row slot / CPR, which is global chunk (slot % CPR) ^ swz(row)
    uint32_t off_rows, off_cols;
    {
        const int slot = wave * 64 + lane;
        const int row = slot / TL::CPR, pc = slot % TL::CPR;
        const int cr = pc ^ swz<D, ROWS>(row), cc = pc ^ swz<D, COLS>(row);
        off_rows = cr * 8 < d ? row * rs + cr * 16 : kOobOffset;
        off_cols = cc * 8 < d ? row * rs + cc * 16 : kOobOffset;
    }
    auto lds_addr = [](const void* q) { return (uint32_t)(uintptr_t)(lds_void*)q; };
    const int nb = Nk * (int)rs;
    const i32x4 rk = buffer_desc(static_cast<const T*>(p.k) + kv_off, nb);
    const i32x4 rv = buffer_desc(static_cast<const T*>(p.v) + kv_off, nb);
    auto issue = [&](int t, int buf) {
        const uint32_t slot = (uint32_t)wave * 1024u;
#pragma unroll
        for (int hf = 0; hf < KH; ++hf) {
            const uint32_t base = (uint32_t)(KR * t + 32 * hf) * rs;
            lds_copy16(rk, off_rows + base, __builtin_amdgcn_readfirstlane(lds_addr(sK[buf][hf]) + slot));
            lds_copy16(rk, off_cols + base, __builtin_amdgcn_readfirstlane(lds_addr(sKc[buf][hf]) + slot));
            lds_copy16(rv, off_rows + base, __builtin_amdgcn_readfirstlane(lds_addr(sV[buf][hf]) + slot));
        }
    };
    auto body = [&](int t, int buf) {
        // tile t landed everywhere (the copies of tile t + 1 may still be in flight when
        // triple-buffered) and every wave is past tile t - 1, whose buffer takes the next copy
        if (NBUF > 2 && t + 1 < nkt) {
            constexpr int n = NCOPY * (NBUF - 2);
            __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4));   // vmcnt(n) lgkmcnt(0)
        } else {
            __builtin_amdgcn_s_waitcnt(7 << 4);                                   // vmcnt(0) lgkmcnt(0)
        }
        asm volatile("s_barrier" ::: "memory");
        if (t + NBUF - 1 < nkt) issue(t + NBUF - 1, (buf + NBUF - 1) % NBUF);
#pragma unroll
        for (int hf = 0; hf < KH; ++hf) {
            const int k0 = KR * t + 32 * hf;
            // wave-uniform: the half holds no key this wave's rows see
            if (k0 >= Nk || (p.causal && k0 > qw0 + 31)) continue;
            // S^T = K Q^T, dP^T = V dO^T: register r holds key k0 + 16(r/8) + 8h + r%8, query qi
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ks = 0; ks < TL::KS; ++ks) {
                s = Mfma<T>::mma(rd_rows<D>(sK[buf][hf], ks, lane), qf[ks], s);
                dp = Mfma<T>::mma(rd_rows<D>(sV[buf][hf], ks, lane), dof[ks], dp);
            }
            // dS packed to 16 bit. Halves before the diagonal and away from the ends need no
            // mask: a uniform branch picks the mask-free form; on edge halves every exponential
            // is taken and masked pairs are selected to 0 (no per-element branch).
            u32x4 dsf[2];
            auto ds_of = [&](auto masked) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    float dsv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float x = fmaf(s[8 * kk + e], c2, -lse2);
                        if constexpr (decltype(masked)::value) {
                            const int kj = k0 + 16 * kk + 8 * h + e;
                            const bool vis = qi < Nq && kj < Nk && (!p.causal || kj <= qi);
                            x = vis ? x : -INFINITY;   // exp2(-inf) = +0
                        }
                        dsv[e] = __builtin_amdgcn_exp2f(x) * (dp[8 * kk + e] - delta);
                    }
                    dsf[kk] = u32x4{Mfma<T>::pack2(dsv[0], dsv[1]), Mfma<T>::pack2(dsv[2], dsv[3]),
                                    Mfma<T>::pack2(dsv[4], dsv[5]), Mfma<T>::pack2(dsv[6], dsv[7])};
                }
            };
            const bool inner = qw0 + 32 <= Nq && k0 + 32 <= Nk && (!p.causal || k0 + 31 <= qw0);
            if (inner) ds_of(std::false_type{});
            else ds_of(std::true_type{});
            // dQ^T += K^T dS^T
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int db = 0; db < TL::DB; ++db)
                    dq[db] = Mfma<T>::mma(rd_cols<D>(sKc[buf][hf], db, kk, lane), dsf[kk], dq[db]);
        }
    };
#pragma unroll
    for (int t = 0; t < NBUF - 1; ++t)
        if (t < nkt) issue(t, t);
    for (int t = 0; t < nkt; t += NBUF) {
#pragma unroll
        for (int c = 0; c < NBUF; ++c)
            if (t + c < nkt) body(t + c, c);
    }
    if (qi < Nq) store_rowT<T, D>(static_cast<T*>(p.dq) + q_off + (int64_t)qi * d, dq, p.scale, d, h);
#endif
}

template <typename T, int D>
hipError_t launch_typed(const BwdProblem& p, hipStream_t stream) {
    // 8 waves per workgroup at head_dim 128 (a 32-row tile of 16-byte chunks then splits
    // evenly over 512 threads), 4 at 64: 32 keys (dK / dV) or query rows (dQ) per wave
    constexpr int WV = D == 128 ? 8 : 4;
    constexpr int RK = 32 * WV, R = 32 * WV;
    const int64_t nk = (int64_t)((p.seqlen_k + RK - 1) / RK) * p.heads_kv * p.batch;
    const int64_t nq = (int64_t)((p.seqlen_q + R - 1) / R) * p.heads_q * p.batch;
    if (nk > INT32_MAX || nq > INT32_MAX) return hipErrorInvalidConfiguration;
    const int64_t rows = (int64_t)p.batch * p.heads_q * p.seqlen_q;
    if ((rows + 15) / 16 > INT32_MAX) return hipErrorInvalidConfiguration;
    hipError_t e;
    if (rows > 0) {   // D into the rows of dq, before the dK pass reads it
        hipLaunchKernelGGL(attn_bwd_delta_kernel<T>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, stream, p, rows);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    dim3 gk((unsigned)nk);
    hipLaunchKernelGGL((attn_bwd_kv_mfma_kernel<T, D, 0, WV, kTiles, kBufs>), gk, dim3(WV * 64), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_kv_mfma_kernel<T, D, 1, WV, kTiles, kBufs>), gk, dim3(WV * 64), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess || p.seqlen_q == 0) return e;   // no query rows: dK = dV = 0, no dQ
    dim3 gq((unsigned)nq);
    hipLaunchKernelGGL((attn_bwd_dq_mfma_kernel<T, D, WV, kTiles, kBufs>), gq, dim3(WV * 64), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_dim(const BwdProblem& p, hipStream_t stream) {
    if (p.head_dim <= 64) return launch_typed<T, 64>(p, stream);
    return launch_typed<T, 128>(p, stream);
}

}  // namespace

hipError_t launch_attn_bwd_mfma(const BwdProblem& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::BF16) return launch_dim<bf16_t>(p, stream);
    if (dt == Dtype::F16) return launch_dim<f16_t>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace aule
