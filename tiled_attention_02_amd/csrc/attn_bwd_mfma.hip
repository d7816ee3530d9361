// Attention backward (dQ, dK, dV) on the matrix cores, fp16/bf16 inputs, fp32 accumulation.
//
// The score matrix is recomputed tile by tile from Q, K and the forward's per-row
// log-sum-exp (FlashAttention-T commentary, ai-stack.site, FAQ 4, training bullet). Per
// (query i, key j) pair: P = exp2(scale log2(e) q_i.k_j - LSE_i log2(e)) (0 where masked),
// dP = do_i.v_j, dS = P (dP - D_i) with D_i = do_i.o_i; dV_j += P dO_i,
// dK_j += scale dS q_i, dQ_i += scale dS k_j.
//
// Three launches, no atomics (deterministic), 32-row / 32-key steps:
//   * dV pass and dK pass (one kernel, two instantiations; WV = 8 waves per workgroup at
//     head_dim 128, 4 at 64): wave w owns 32 keys (its K rows and, for dK, its V rows held
//     as B operands in registers) and one transposed accumulator (dV^T or dK^T, d x 32
//     keys). The workgroup walks every query head of its GQA group and every 32-row query
//     tile (causal: from its first key on); Q and dO tiles go through LDS, double-buffered,
//     their global loads issued two iterations ahead. Per tile: S = Q K^T (and dP = dO V^T)
//     with Q / dO rows fed in sigma order, so P and dS leave the accumulators already in the
//     B-operand layout of dV^T += dO^T P and dK^T += Q^T dS, whose A operands (dO^T, Q^T)
//     are transposing LDS reads (ds_read_b64_tr_b16). The dK pass forms D_i from the O and
//     dO chunks as they are staged. The dV pass stages four 32-row query tiles per barrier.
//   * dQ (4 waves): wave w owns 32 query rows (Q and dO rows in registers, LSE_i and D_i per
//     lane); the workgroup walks the key tiles (causal: up to its last row). Per tile:
//     S^T = K Q^T, dP^T = V dO^T with K / V rows in sigma order, then dQ^T += K^T dS^T with
//     K^T read transposed from LDS.
// The dQ kernel keeps K / V tiles row-major [32][D] with one 16-byte pad per row; the dK / dV
// passes store each staged tile XOR-swizzled in the layout of the read that uses it.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "attn_bwd.h"
#include "attn_mfma.h"

namespace aule {
namespace {

constexpr int kWaves = 4;
// 32-row query tiles per iteration of the dV pass (one barrier per 128 rows; measured
// 3.44 -> 3.31 -> 3.25 ms per step of the bf16 causal GQA backward for 1, 2, 4). The dK pass
// keeps one: at 254 registers it has no room for a second score tile.
constexpr int kDvTiles = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kLog2eF = 1.4426950408889634f;

template <int D, int NT = kThreads>
struct Tile {
    static constexpr int RS = D * 2;                      // bytes per LDS row (swizzled layouts)
    static constexpr int RSP = D * 2 + 16;                // bytes per LDS row (PAD layout)
    static constexpr int CPR = D / 8;                     // 16-byte chunks per row
    static constexpr int BYTES = 32 * RS;
    static constexpr int BYTESP = 32 * RSP;
    static constexpr int NCH = 32 * CPR / NT;             // chunks per thread per tile
    static constexpr int KS = D / 16;                     // k-steps over head_dim
    static constexpr int DB = D / 32;                     // 32-row blocks of head_dim
    static_assert(NCH >= 1 && NCH * NT == 32 * CPR, "tile chunks must split evenly");
};

// Rows [r0, r0 + 32) of a [rows, d] slice as 16-byte chunks, this thread's share, through a
// buffer resource covering exactly the slice: rows past the end read as zero (the hardware's
// range check) and chunks past head_dim are sent past the range, so there is no branch and no
// zero fill (with those, the compiler waited for every load in flight before refilling a
// staging set, which undid the two-deep staging).
template <typename T, int D, int NT = kThreads>
__device__ __forceinline__ void fetch_rows_buf(u32x4 (&c)[(Tile<D, NT>::NCH)], __amdgpu_buffer_rsrc_t rs, int r0, int d) {
#pragma unroll
    for (int i = 0; i < Tile<D, NT>::NCH; ++i) {
        const int idx = (int)threadIdx.x + NT * i;
        const int row = idx / Tile<D>::CPR, ch = idx % Tile<D>::CPR;
        const uint32_t off = ch * 8 < d ? (uint32_t)(r0 + row) * (uint32_t)(d * (int)sizeof(T)) + (uint32_t)ch * 16u : kOobOffset;
        c[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
    }
}
// Resource for a [rows, d] slice of T (at most 1 GiB, checked by the host).
template <typename T>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const T* base, int rows, int d) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0, rows > 0 ? rows * d * (int)sizeof(T) : 0,
                                             (int)kBufferFlags);
}
// Two LDS layouts of a 32-row tile, one per read pattern, with the XOR swizzles of the
// forward kernel's K and V tiles (chunk c of row r stored at chunk c ^ swz(r)):
//   ROWS: rd_rows reads one chunk of rows sigma(0..31) per instruction -> kswz;
//   COLS: rd_cols reads 4 consecutive rows x 2 neighbouring chunks per 16 lanes -> vswz.
// A tile read both ways is stored twice. PAD: unswizzled rows padded by 16 bytes, read both
// ways from one copy (the transposed reads then conflict 2-way; the dQ kernel keeps it, where
// a second copy of K cost more than the conflicts).
enum Layout { ROWS = 0, COLS = 1, PAD = 2 };
template <int D, int L>
__device__ __forceinline__ int swz(int row) {
    if constexpr (L == ROWS) return kswz<D / 8>(row);
    else if constexpr (L == COLS) return vswz<D / 8>(row);
    else return 0;
}
template <int D, int L> constexpr int row_bytes() { return L == PAD ? Tile<D>::RSP : Tile<D>::RS; }
template <int D, int L, int NT = kThreads>
__device__ __forceinline__ void put_rows(char* tile, const u32x4 (&c)[(Tile<D, NT>::NCH)]) {
#pragma unroll
    for (int i = 0; i < Tile<D, NT>::NCH; ++i) {
        const int idx = (int)threadIdx.x + NT * i;
        const int row = idx / Tile<D>::CPR, ch = idx % Tile<D>::CPR;
        *reinterpret_cast<u32x4*>(tile + row * row_bytes<D, L>() + (ch ^ swz<D, L>(row)) * 16) = c[i];
    }
}

// A operand with rows in sigma order from a ROWS tile: lane l supplies row sigma(l % 32),
// k-chunk 2ks + h (stored at chunk (2ks + h) ^ kswz(sigma(l % 32)) = (2ks + h) ^ kx_lane(l % 32)).
template <int D, int L = ROWS>
__device__ __forceinline__ u32x4 rd_rows(const char* tile, int ks, int lane) {
    const int l32 = lane & 31;
    const int x = L == PAD ? 0 : kx_lane<Tile<D>::CPR>(l32);
    return *reinterpret_cast<const u32x4*>(tile + sigma(l32) * row_bytes<D, L>() + (((2 * ks + (lane >> 5)) ^ x) * 16));
}
// A operand of a transposed COLS tile: A[m = column 32db + l % 32][k = row 16kk + 8h .. + 7],
// two transposing 8-byte reads (each 16-lane group reads 4 rows x 16 columns); vswz depends
// on the row modulo 4 only, the same for both reads.
template <int D, int L = COLS>
__device__ __forceinline__ u32x4 rd_cols(const char* tile, int db, int kk, int lane) {
    const int tg = lane >> 4, tc = lane & 15;
    const int row0 = 16 * kk + 8 * (tg >> 1) + (tc >> 2);
    const int x = L == PAD ? 0 : vswz<D / 8>(row0);
    const int coff = ((4 * db + 2 * (tg & 1) + ((tc & 3) >> 1)) ^ x) * 16 + (tc & 1) * 8;
    u32x4 out;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const char* addr = tile + (row0 + 4 * t) * row_bytes<D, L>() + coff;
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

// PASS 0 accumulates dV only (S and dV^T += dO^T P: no V, O or D needed), PASS 1 dK only
// (S, dP and dK^T += Q^T dS). One gradient per pass halves the accumulators, so each pass
// fits two waves per SIMD, whose matrix products then overlap the other wave's
// exponentials; the price is S computed twice. WV waves own 32 keys each: the Q / dO / O
// rows of the group are read once per 32 * WV keys, so wider workgroups cut that traffic.
// QH 32-row query tiles are staged per iteration (one barrier per 32 * QH rows); within an
// iteration the halves' products and exponentials are independent until they accumulate.
template <typename T, int D, int PASS, int WV, int QH>
__global__ __launch_bounds__(WV * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bwd_dkdv_mfma_kernel(BwdProblem p) {
    constexpr int NT = WV * 64;
    constexpr int QR = 32 * QH;   // query rows per iteration
    using TL = Tile<D, NT>;
    // Q (ROWS) for S; dO (COLS) for dV^T in the dV pass, (ROWS) for dP in the dK pass; Q
    // again (COLS) for dK^T in the dK pass
    constexpr int DO_L = PASS == 0 ? COLS : ROWS;
    __shared__ __attribute__((aligned(16))) char sQ[2][QH][TL::BYTES];
    __shared__ __attribute__((aligned(16))) char sdO[2][QH][TL::BYTES];
    __shared__ __attribute__((aligned(16))) char sQc[PASS == 1 ? 2 : 1][QH][PASS == 1 ? TL::BYTES : 16];
    __shared__ __attribute__((aligned(16))) float sL[2][QR];
    __shared__ __attribute__((aligned(16))) float sD[2][QR];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, ln = lane & 31;
    const int Nq = p.seqlen_q, Nk = p.seqlen_k, d = p.head_dim, G = p.group;
    // flat grid, key blocks slowest: under causal masking block 0 walks every query tile and
    // later blocks fewer, so the longest workgroups start first; the key blocks of one
    // (batch, kv head) are heads_kv * batch apart, which keeps them on one XCD when that
    // count is a multiple of 8 (they read the same Q and dO tiles)
    const int per_kb = p.heads_kv * p.batch;
    const int kb = blockIdx.x / per_kb, rem = blockIdx.x - kb * per_kb;
    const int hk = rem % p.heads_kv, b = rem / p.heads_kv;
    const int j0 = kb * 32 * WV;
    const int key = j0 + 32 * wave + ln;                 // this lane's key (B-operand column)
    const int64_t kv_off = ((int64_t)b * p.heads_kv + hk) * Nk * d;
    // work: (QR-row query tile, query head g of the group), causal from the first key on.
    // The tiles are walked from the last one down, the group's heads inner, so that the
    // workgroups of one (batch, kv head) — which run on one XCD, whatever their first key —
    // read the same Q / dO / O tile at the same time and share it through that XCD's L2
    // (walked upwards from each block's first key, they read different rows: -2.5% time on the
    // bf16 causal GQA backward). With no query rows (nit == 0) only the zero gradients are
    // written: q, k, v, o, do and lse may then be null and are not read.
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

    // Register staging of one query tile's global loads. Two sets: tile it + 2 is fetched
    // into the set that held tile it while tile it + 1 (fetched an iteration earlier) is
    // committed to LDS, so each load has two iterations to arrive.
    struct Stage {
        u32x4 q[QH][TL::NCH], dO[QH][TL::NCH], o[QH][PASS == 1 ? TL::NCH : 1];
        float lse;
    };
    // (tile counted from the last, head) of the next fetch and of the current body: advanced
    // one step per iteration instead of dividing the iteration index by the group size
    int f_tr = 0, f_g = 0, b_tr = 0, b_g = 0;
    auto step = [&](int& tr, int& g) {
        if (++g == G) { g = 0; ++tr; }
    };
    const int64_t bh0 = (int64_t)b * p.heads_q + (int64_t)hk * G;
    auto fetch = [&](Stage& st) {
        const int i0 = i_start + QR * (ntile - 1 - f_tr);
        const int64_t bh = bh0 + f_g;
        const int64_t q_off = bh * Nq * d;
        step(f_tr, f_g);
        const __amdgpu_buffer_rsrc_t rq = slice_rsrc(static_cast<const T*>(p.q) + q_off, Nq, d);
        const __amdgpu_buffer_rsrc_t rdo = slice_rsrc(static_cast<const T*>(p.do_) + q_off, Nq, d);
#pragma unroll
        for (int hf = 0; hf < QH; ++hf) {
            fetch_rows_buf<T, D, NT>(st.q[hf], rq, i0 + 32 * hf, d);
            fetch_rows_buf<T, D, NT>(st.dO[hf], rdo, i0 + 32 * hf, d);
            if constexpr (PASS == 1)
                fetch_rows_buf<T, D, NT>(st.o[hf], slice_rsrc(static_cast<const T*>(p.o) + q_off, Nq, d), i0 + 32 * hf, d);
        }
        // every thread loads (rows past the end read as zero); the first QR are committed
        const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.lse) + bh * Nq, (short)0, Nq * 4, (int)kBufferFlags);
        const uint32_t loff = (int)threadIdx.x < QR ? (uint32_t)(i0 + (int)threadIdx.x) * 4u : kOobOffset;
        st.lse = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, (int)loff, 0, 0));
    };
    auto commit = [&](int buf, const Stage& st) {
#pragma unroll
        for (int hf = 0; hf < QH; ++hf) {
            put_rows<D, ROWS, NT>(sQ[buf][hf], st.q[hf]);
            put_rows<D, DO_L, NT>(sdO[buf][hf], st.dO[hf]);
            if constexpr (PASS == 1) put_rows<D, COLS, NT>(sQc[buf][hf], st.q[hf]);
            // D_i = do_i . o_i: a chunk pair per thread, summed over the CPR chunks of a row
            // (consecutive lanes)
            if constexpr (PASS == 1)
#pragma unroll
            for (int i = 0; i < TL::NCH; ++i) {
                float x = 0.f;
#pragma unroll
                for (int w = 0; w < 4; ++w) x = Mfma<T>::dot2(st.dO[hf][i][w], st.o[hf][i][w], x);
#pragma unroll
                for (int off = 1; off < TL::CPR; off <<= 1) x += __shfl_xor(x, off);
                const int idx = (int)threadIdx.x + NT * i;
                if (idx % TL::CPR == 0) sD[buf][32 * hf + idx / TL::CPR] = -x;   // -D
            }
        }
        if ((int)threadIdx.x < QR) sL[buf][threadIdx.x] = st.lse * kLog2eF;
    };

    const int kw0 = j0 + 32 * wave;   // this wave's first key
    auto body = [&](int it, Stage& mine, const Stage& other) {
        const int buf = it & 1;
        const int i0q = i_start + QR * (ntile - 1 - b_tr);
        step(b_tr, b_g);
        if (it + 2 < nit) fetch(mine);
#pragma unroll
        for (int hf = 0; hf < QH; ++hf) {
        const int i0 = i0q + 32 * hf;
        // S = Q K^T, dP - D = dO V^T - D: register r holds query i0 + 16(r/8) + 8h + r%8, key
        // `key`; the dP accumulator starts from -D of its rows (two runs of 8 consecutive rows,
        // 16-byte reads), so dS = P (dP - D) needs no further registers
        f32x16 s = f32x16{}, dp = f32x16{};
        if constexpr (PASS == 1) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const float4* pd = reinterpret_cast<const float4*>(&sD[buf][32 * hf + 16 * kk + 8 * h]);
                const float4 x = pd[0], y = pd[1];
                dp[8 * kk + 0] = x.x; dp[8 * kk + 1] = x.y; dp[8 * kk + 2] = x.z; dp[8 * kk + 3] = x.w;
                dp[8 * kk + 4] = y.x; dp[8 * kk + 5] = y.y; dp[8 * kk + 6] = y.z; dp[8 * kk + 7] = y.w;
            }
        }
#pragma unroll
        for (int ks = 0; ks < TL::KS; ++ks) {
            s = Mfma<T>::mma(rd_rows<D>(sQ[buf][hf], ks, lane), kf[ks], s);
            if constexpr (PASS == 1) dp = Mfma<T>::mma(rd_rows<D>(sdO[buf][hf], ks, lane), vf[ks], dp);
        }
        // P (and dS) packed to 16 bit. The row statistics of each run of 8 consecutive query
        // rows are read as two 16-byte vectors. Tiles away from the diagonal and the ends need
        // no mask: a uniform branch picks the mask-free form; on edge tiles every exponential
        // is taken and masked pairs are selected to 0 (no per-element branch).
        u32x4 pf[2], dsf[2];
        auto p_ds = [&](auto masked) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const int q0 = 16 * kk + 8 * h;
                float lq[8];
                {
                    const float4* pl = reinterpret_cast<const float4*>(&sL[buf][32 * hf + q0]);
                    const float4 a = pl[0], c = pl[1];
                    lq[0] = a.x; lq[1] = a.y; lq[2] = a.z; lq[3] = a.w;
                    lq[4] = c.x; lq[5] = c.y; lq[6] = c.z; lq[7] = c.w;
                }
                float pv[8], dsv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x = fmaf(s[8 * kk + e], c2, -lq[e]);
                    if constexpr (decltype(masked)::value) {
                        const int qi = i0 + q0 + e;
                        const bool vis = qi < Nq && key < Nk && (!p.causal || key <= qi);
                        x = vis ? x : -INFINITY;   // exp2(-inf) = +0
                    }
                    const float pe = __builtin_amdgcn_exp2f(x);
                    pv[e] = pe;
                    dsv[e] = PASS == 1 ? pe * dp[8 * kk + e] : 0.f;
                }
                if constexpr (PASS == 0)
                    pf[kk] = u32x4{Mfma<T>::pack2(pv[0], pv[1]), Mfma<T>::pack2(pv[2], pv[3]),
                                   Mfma<T>::pack2(pv[4], pv[5]), Mfma<T>::pack2(pv[6], pv[7])};
                else
                    dsf[kk] = u32x4{Mfma<T>::pack2(dsv[0], dsv[1]), Mfma<T>::pack2(dsv[2], dsv[3]),
                                    Mfma<T>::pack2(dsv[4], dsv[5]), Mfma<T>::pack2(dsv[6], dsv[7])};
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
                if constexpr (PASS == 0) acc[db] = Mfma<T>::mma(rd_cols<D>(sdO[buf][hf], db, kk, lane), pf[kk], acc[db]);
                else acc[db] = Mfma<T>::mma(rd_cols<D>(sQc[buf][hf], db, kk, lane), dsf[kk], acc[db]);
            }
        }
        if (it + 1 < nit) commit(buf ^ 1, other);
        __syncthreads();
    };

    Stage st0, st1;
    if (nit > 0) {
        fetch(st0);
        commit(0, st0);
    }
    if (nit > 1) fetch(st1);
    __syncthreads();
    for (int it = 0; it < nit; it += 2) {
        body(it, st0, st1);
        if (it + 1 < nit) body(it + 1, st1, st0);
    }
    if (key < Nk) {
        if constexpr (PASS == 1) store_rowT<T, D>(static_cast<T*>(p.dk) + kv_off + (int64_t)key * d, acc, p.scale, d, h);
        else store_rowT<T, D>(static_cast<T*>(p.dv) + kv_off + (int64_t)key * d, acc, 1.f, d, h);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bwd_dq_mfma_kernel(BwdProblem p) {
    using TL = Tile<D>;
    // K and V tiles in the PAD layout (K read both ways from one copy)
    __shared__ __attribute__((aligned(16))) char sK[2][TL::BYTESP];
    __shared__ __attribute__((aligned(16))) char sV[2][TL::BYTESP];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, ln = lane & 31;
    const int Nq = p.seqlen_q, Nk = p.seqlen_k, d = p.head_dim;
    // flat grid, query blocks slowest and (causal) last block first: the longest walks start
    // first. Within a block index the G query heads of one (batch, kv head) are
    // batch * heads_kv apart, which puts them on one XCD (sharing its L2 copy of that K/V)
    // when that count is a multiple of 8.
    const int per_qb = p.heads_q * p.batch;
    const int t_ = blockIdx.x / per_qb, rem = blockIdx.x - t_ * per_qb;
    const int nqb = (Nq + 32 * kWaves - 1) / (32 * kWaves);
    const int qblk = p.causal ? nqb - 1 - t_ : t_;
    const int nkvu = p.batch * p.heads_kv;
    const int gi = rem / nkvu, u = rem - gi * nkvu;
    const int b = u / p.heads_kv, hq = (u - b * p.heads_kv) * p.group + gi;
    const int i0 = qblk * 32 * kWaves;
    const int hk = hq / p.group;
    const int qi = i0 + 32 * wave + ln;                  // this lane's query (B-operand column)
    const int64_t bh = (int64_t)b * p.heads_q + hq;
    const int64_t q_off = bh * Nq * d;
    const int64_t kv_off = ((int64_t)b * p.heads_kv + hk) * Nk * d;
    const T* Kb = static_cast<const T*>(p.k) + kv_off;
    const T* Vb = static_cast<const T*>(p.v) + kv_off;

    u32x4 qf[TL::KS], dof[TL::KS];
    fetch_operand<T, D>(qf, static_cast<const T*>(p.q) + q_off, qi, Nq, d, h);
    fetch_operand<T, D>(dof, static_cast<const T*>(p.do_) + q_off, qi, Nq, d, h);
    float delta;
    {
        u32x4 of[TL::KS];
        fetch_operand<T, D>(of, static_cast<const T*>(p.o) + q_off, qi, Nq, d, h);
        float x = 0.f;
#pragma unroll
        for (int ks = 0; ks < TL::KS; ++ks)
#pragma unroll
            for (int w = 0; w < 4; ++w) x = Mfma<T>::dot2(dof[ks][w], of[ks][w], x);
        delta = x + __shfl_xor(x, 32);                    // the other half of the row
    }
    const float lse2 = qi < Nq ? p.lse[bh * Nq + qi] * kLog2eF : 0.f;
    const float c2 = p.scale * kLog2eF;

    f32x16 dq[TL::DB];
#pragma unroll
    for (int db = 0; db < TL::DB; ++db) dq[db] = f32x16{};

    const int j_end = p.causal ? min(Nk, i0 + 32 * kWaves) : Nk;
    const int nkt = (j_end + 31) / 32;
    // two register staging sets, as in the dK / dV kernel: key tile t + 2 is fetched while
    // tile t + 1 (fetched an iteration earlier) is committed to LDS
    struct Stage { u32x4 k[TL::NCH], v[TL::NCH]; };
    const __amdgpu_buffer_rsrc_t rk = slice_rsrc(Kb, Nk, d), rv = slice_rsrc(Vb, Nk, d);
    auto fetch = [&](int t, Stage& st) {
        fetch_rows_buf<T, D>(st.k, rk, 32 * t, d);
        fetch_rows_buf<T, D>(st.v, rv, 32 * t, d);
    };
    auto commit = [&](int buf, const Stage& st) {
        put_rows<D, PAD>(sK[buf], st.k);
        put_rows<D, PAD>(sV[buf], st.v);
    };
    const int qw0 = i0 + 32 * wave;   // this wave's first query row
    auto body = [&](int t, Stage& mine, const Stage& other) {
        const int buf = t & 1;
        if (t + 2 < nkt) fetch(t + 2, mine);
        // S^T = K Q^T, dP^T = V dO^T: register r holds key 32t + 16(r/8) + 8h + r%8, query qi
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < TL::KS; ++ks) {
            s = Mfma<T>::mma(rd_rows<D, PAD>(sK[buf], ks, lane), qf[ks], s);
            dp = Mfma<T>::mma(rd_rows<D, PAD>(sV[buf], ks, lane), dof[ks], dp);
        }
        // dS packed to 16 bit. Key tiles before the diagonal and away from the ends need no
        // mask: a uniform branch picks the mask-free form; on edge tiles every exponential is
        // taken and masked pairs are selected to 0 (no per-element branch).
        u32x4 dsf[2];
        auto ds_of = [&](auto masked) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                float dsv[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x = fmaf(s[8 * kk + e], c2, -lse2);
                    if constexpr (decltype(masked)::value) {
                        const int kj = 32 * t + 16 * kk + 8 * h + e;
                        const bool vis = qi < Nq && kj < Nk && (!p.causal || kj <= qi);
                        x = vis ? x : -INFINITY;   // exp2(-inf) = +0
                    }
                    const float pe = __builtin_amdgcn_exp2f(x);
                    dsv[e] = pe * (dp[8 * kk + e] - delta);
                }
                dsf[kk] = u32x4{Mfma<T>::pack2(dsv[0], dsv[1]), Mfma<T>::pack2(dsv[2], dsv[3]),
                                Mfma<T>::pack2(dsv[4], dsv[5]), Mfma<T>::pack2(dsv[6], dsv[7])};
            }
        };
        const bool inner = qw0 + 32 <= Nq && 32 * t + 32 <= Nk && (!p.causal || 32 * t + 31 <= qw0);
        if (inner) ds_of(std::false_type{});
        else ds_of(std::true_type{});
        // dQ^T += K^T dS^T
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int db = 0; db < TL::DB; ++db)
                dq[db] = Mfma<T>::mma(rd_cols<D, PAD>(sK[buf], db, kk, lane), dsf[kk], dq[db]);
        if (t + 1 < nkt) commit(buf ^ 1, other);
        __syncthreads();
    };
    Stage st0, st1;
    if (nkt > 0) {
        fetch(0, st0);
        commit(0, st0);
    }
    if (nkt > 1) fetch(1, st1);
    __syncthreads();
    for (int t = 0; t < nkt; t += 2) {
        body(t, st0, st1);
        if (t + 1 < nkt) body(t + 1, st1, st0);
    }
    if (qi < Nq) store_rowT<T, D>(static_cast<T*>(p.dq) + q_off + (int64_t)qi * d, dq, p.scale, d, h);
}

template <typename T, int D>
hipError_t launch_typed(const BwdProblem& p, hipStream_t stream) {
    constexpr int R = 32 * kWaves;
    // 256 keys per dK / dV workgroup at head_dim 128 (a 32-row tile of 16-byte chunks then
    // splits evenly over 512 threads), 128 at 64
    constexpr int WV = D == 128 ? 8 : 4;
    constexpr int RK = 32 * WV;
    const int64_t nk = (int64_t)((p.seqlen_k + RK - 1) / RK) * p.heads_kv * p.batch;
    const int64_t nq = (int64_t)((p.seqlen_q + R - 1) / R) * p.heads_q * p.batch;
    if (nk > INT32_MAX || nq > INT32_MAX) return hipErrorInvalidConfiguration;
    dim3 gk((unsigned)nk);
    hipLaunchKernelGGL((attn_bwd_dkdv_mfma_kernel<T, D, 0, WV, kDvTiles>), gk, dim3(WV * 64), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((attn_bwd_dkdv_mfma_kernel<T, D, 1, WV, 1>), gk, dim3(WV * 64), 0, stream, p);
    e = hipGetLastError();
    if (e != hipSuccess || p.seqlen_q == 0) return e;   // no query rows: dK = dV = 0, no dQ
    dim3 gq((unsigned)nq);
    hipLaunchKernelGGL((attn_bwd_dq_mfma_kernel<T, D>), gq, dim3(kThreads), 0, stream, p);
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
