// Matrix-core (MFMA) attention forward for fp16/bf16 on gfx950 (CDNA4).
//
// The FlashAttention block loop (xxqk.cn article "Attention算子实战：从CUDA优化到昇腾/CANN部署",
// section 2.2: Q tile on chip, K/V tiles streamed, numerically stable softmax kept in
// registers, partial P·V accumulated, only O written) with fp16/bf16 matrix products and
// fp32 softmax statistics (FlashAttention-T commentary, ai-stack.site, best practices 4-5),
// laid out for 64-wide wavefronts and v_mfma_f32_32x32x16_{bf16,f16}.
//
// Work split
//   workgroup = 4 waves; wave = 64 query rows (two 32-row blocks "nb") of one query head.
//   GH query heads that share one K/V head run in the same workgroup (GQA), the other
//   4/GH waves take further 64-row blocks, so one K/V tile in LDS serves 4 x 64 query rows.
//   K/V tiles of BN = 64 keys, double-buffered in LDS. They are copied global -> LDS with
//   buffer_load_dwordx4 ... lds (no register staging): each wave instruction fills 1 KiB of
//   LDS contiguously, and every lane picks the global 16-byte chunk that belongs at its LDS
//   slot, so the LDS image is XOR-swizzled against bank conflicts while the global reads stay
//   whole rows. The buffer descriptor's size check turns rows past the sequence end and
//   columns past head_dim into zeros.
//
// Transposed products
//   S^T = K Q^T : A = K tile rows (from LDS), B = Q^T (registers, loaded once). In the
//                 32x32 accumulator, lane n%32 holds query n and 16 keys in its registers,
//                 so row max / row sum are in-lane reductions plus one exchange with
//                 lane n^32.
//   O^T = V^T P^T : B = P^T taken straight from the S^T accumulator registers (converted to
//                 16-bit), A = V^T fragments read from the row-major V tile in LDS with
//                 ds_read_b64_tr_b16 (each 16-lane group reads a 4-key x 16-d block and
//                 receives it transposed: lane i gets the 4 keys of column d = i).
//   For the registers of S^T to line up with the k-slots of the P^T operand, the K tile
//   rows are fed to the first product in a permuted order: A-row m reads key sigma(m),
//   sigma swapping bits 2 and 3 of m. Then accumulator register r of lane (h = lane/32)
//   holds key 16*(r/8) + 8*h + r%8 of its 32-key block, i.e. 8 consecutive keys per
//   16-key chunk — exactly the k-slots of the second product, whose V^T fragment is then
//   two transposed 8-byte reads. (Any consistent order of the contraction index is valid.)
//
// Online softmax (fp32): t = s * c with c = |scale| * log2(e) (a negative scale is folded
// into Q by flipping its sign bits, exactly); P = exp2(t - m). The reference max m is only
// raised when some row's tile max exceeds it by more than kRescaleSlack (log2 units), so
// the O rescale is skipped for most tiles; P then stays <= 2^kRescaleSlack, well inside
// fp16/bf16 range, and the final O / l is unchanged mathematically.
#include <hip/hip_runtime.h>
#include <math.h>

#include <cstdlib>

#include "attn_device.h"

namespace aule {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kBN = 64;               // keys per K/V tile (two 32-key sub-steps)
[[maybe_unused]] constexpr float kRescaleSlack = 8.0f; // log2 units

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32)
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
    }
    // acc + lo + hi of a packed pair, in fp32 (v_dot2 against (1, 1))
    static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
        const bf16x2 one = {(bf16_t)1.0f, (bf16_t)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair), one, acc, false);
    }
};
template <> struct Mfma<f16_t> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    // two fp32 -> packed fp16 pair, round to nearest even (one v_cvt_pk_f16_f32)
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
    }
    static __device__ __forceinline__ float sum2(uint32_t pair, float acc) {
        const f16x2 one = {(f16_t)1.0f, (f16_t)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair), one, acc, false);
    }
};

// sigma: swap bits 2 and 3 (an involution on 0..31)
__device__ __forceinline__ int sigma(int m) {
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

// 16-byte chunk swizzles (XOR on the chunk index inside a row).
// K rows: the S^T reads of one instruction hit rows sigma(0..31) at one column; chunk c of
//   row r sits at c ^ (sigma(r % 32) % KC), so those reads spread over distinct chunks.
// V rows: a transposed read touches 4 consecutive rows x 2 (or 4) neighbouring chunks; the
//   per-row XOR masks below make those slots distinct modulo 8 and modulo 16 chunks.
template <int KC> __device__ __forceinline__ int kswz(int row) { return sigma(row & 31) & (KC - 1); }
template <int KC> __device__ __forceinline__ int vswz(int row) {
    if constexpr (KC == 16) return (0xCA60 >> (4 * (row & 3))) & 15;   // 0, 6, 10, 12
    else return 2 * (row & 3);
}

[[maybe_unused]] constexpr uint32_t kBufferFlags = 0x00020000u;   // raw buffer, 32-bit data format
[[maybe_unused]] constexpr uint32_t kOobOffset = 0x7FFFFFF0u;     // an offset past any slice: reads as zero

#if defined(__HIP_DEVICE_COMPILE__)
// Start the global -> LDS copy of K/V tile j: NI 16-byte loads per lane for each of K and
// V; wave w fills LDS chunk slots [(w*NI + i) * 64, +64) of the tile buffers.
template <int NI>
__device__ __forceinline__ void issue_tile(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv,
                                           const uint32_t (&koff)[NI], const uint32_t (&voff)[NI],
                                           uint32_t tile_k_bytes, uint32_t tile_v_bytes,
                                           lds_void* dK, lds_void* dV, int wave) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int slot = (wave * NI + i) * 64 * 16;   // bytes
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)((__attribute__((address_space(3))) char*)dK + slot),
                                                 16, koff[i] + tile_k_bytes, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)((__attribute__((address_space(3))) char*)dV + slot),
                                                 16, voff[i] + tile_v_bytes, 0, 0, 0);
    }
}
#endif  // __HIP_DEVICE_COMPILE__

// WAVES waves per workgroup (4: one per SIMD, 8: two per SIMD so one wave's softmax runs
// while the other's matrix products do); each wave owns NB blocks of 32 query rows of one
// query head.
template <typename T, int D, int WAVES, int NB, int GH, int LOOP, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(WAVES / 4)))
void attn_fwd_mfma_kernel(AttnProblem p, int n_qtiles) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int kThreads = WAVES * 64;
    constexpr int kRowsPerWave = 32 * NB;
    constexpr int RB = WAVES / GH;               // row blocks per workgroup
    constexpr int BMW = kRowsPerWave * RB;       // query rows per workgroup
    constexpr int KC = D / 8;                    // 16-byte chunks per K / V row
    constexpr int KS = D / 16;                   // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;                   // 32-row d-blocks of O^T
    constexpr int TILE_CHUNKS = kBN * KC;        // 16-byte chunks per K (or V) tile
    constexpr int NI = TILE_CHUNKS / kThreads;   // load instructions per wave per tile
    static_assert(NI >= 1 && TILE_CHUNKS % kThreads == 0, "tile must split evenly over the waves");

    __shared__ u32x4 sK0[TILE_CHUNKS], sK1[TILE_CHUNKS], sK2[TILE_CHUNKS];
    __shared__ u32x4 sV0[TILE_CHUNKS], sV1[TILE_CHUNKS], sV2[TILE_CHUNKS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int h = lane >> 5;
    const int ln = lane & 31;

    // ---------------------------------------------------------------- tile lookup
    int bidx, hq0, tile, Lq, Lk;
    int64_t tok0 = 0;
    if constexpr (VARLEN) {
        TileSlot s = locate_varlen_tile(p.cu_seqlens, p.batch, p.total_tokens, BMW, blockIdx.x, CAUSAL);
        if (!s.valid) return;
        bidx = s.seq; tok0 = s.tok0; tile = s.tile; Lq = s.len_q; Lk = s.len_k;
        hq0 = blockIdx.y * GH;
    } else {
        // groups = (batch, GH query heads sharing one kv head). Workgroup x runs on XCD
        // x % 8; when the groups split evenly, each XCD gets whole groups so their K/V stay
        // in that XCD's L2. Within an XCD (or the whole grid) the longest causal tiles go first.
        const int ngroups = p.heads_q / GH;
        const int NG = p.batch * ngroups;
        const int x = blockIdx.x;
        int t, g;
        if (NG % 8 == 0) {
            const int per = NG / 8, xcd = x & 7, l = x >> 3;
            t = l / per;
            g = xcd * per + (l - t * per);
        } else {
            t = x / NG;
            g = x - t * NG;
        }
        tile = CAUSAL ? (n_qtiles - 1 - t) : t;
        bidx = g / ngroups;
        hq0 = (g - bidx * ngroups) * GH;
        Lq = p.seqlen_q; Lk = p.seqlen_k;
    }
    const int hq = hq0 + (wave % GH);
    const int hk = hq0 / p.group;
    const int qr0 = tile * BMW + kRowsPerWave * (wave / GH);   // first row of this wave
    const int hd = p.head_dim;

    const T* qb = static_cast<const T*>(p.q) + (VARLEN ? tok0 * p.q_rstride : bidx * p.q_bstride) + hq * p.q_hstride;
    const T* kb = static_cast<const T*>(p.k) + (VARLEN ? tok0 * p.k_rstride : bidx * p.k_bstride) + hk * p.k_hstride;
    const T* vb = static_cast<const T*>(p.v) + (VARLEN ? tok0 * p.v_rstride : bidx * p.v_bstride) + hk * p.v_hstride;
    T* ob = static_cast<T*>(p.o) + (VARLEN ? tok0 * p.o_rstride : bidx * p.o_bstride) + hq * p.o_hstride;

    // ---------------------------------------------------------------- K/V copy set-up
    // Buffer descriptors cover exactly the Lk valid rows of this (sequence, kv head).
    const uint32_t k_rs = (uint32_t)(p.k_rstride * (int64_t)sizeof(T));   // row stride, bytes
    const uint32_t v_rs = (uint32_t)(p.v_rstride * (int64_t)sizeof(T));
    const int k_valid = Lk > 0 ? (int)((int64_t)(Lk - 1) * k_rs + hd * sizeof(T)) : 0;
    const int v_valid = Lk > 0 ? (int)((int64_t)(Lk - 1) * v_rs + hd * sizeof(T)) : 0;
    const __amdgpu_buffer_rsrc_t rsrc_k = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(kb), 0, k_valid, kBufferFlags);
    const __amdgpu_buffer_rsrc_t rsrc_v = __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(vb), 0, v_valid, kBufferFlags);
    // Per-lane byte offsets (tile-relative) of the global chunk that lands in this lane's
    // LDS slot, for each of the NI load instructions of this wave.
    uint32_t koff[NI], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int slot = (wave * NI + i) * 64 + lane;         // chunk slot in the LDS tile
        const int row = slot / KC, pos = slot % KC;
        const int kdc = pos ^ kswz<KC>(row), vdc = pos ^ vswz<KC>(row);
        koff[i] = kdc * 8 < hd ? row * k_rs + kdc * 16 : kOobOffset;
        voff[i] = vdc * 8 < hd ? row * v_rs + vdc * 16 : kOobOffset;
    }
    // ---------------------------------------------------------------- Q -> registers
    const bool neg = p.scale_log2 < 0.f;
    const float c = fmaxf(fabsf(p.scale_log2), 1e-30f);
    u32x4 qf[NB][KS];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const int row = qr0 + 32 * nb + ln;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int col = (2 * ks + h) * 8;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (row < Lq && col < hd) v = *reinterpret_cast<const u32x4*>(qb + (int64_t)row * p.q_rstride + col);
            if (neg) v ^= 0x80008000u;
            qf[nb][ks] = v;
        }
    }

    // ---------------------------------------------------------------- sub-step ranges
    // The key range is walked in 32-key sub-steps; sub-steps 2t and 2t+1 live in K/V tile t.
    // All waves of the workgroup walk the same sub-steps (a wave whose own rows end earlier
    // gets fully masked sub-steps at the end, which add exact zeros).
    const int wg_rows_end = min(tile * BMW + BMW, Lq);
    const int keys_needed = CAUSAL ? wg_rows_end : Lk;
    const int nsub = (keys_needed + 31) / 32;
    const int n_kt = (nsub + 1) / 2;

    // ---------------------------------------------------------------- accumulators
    f32x16 o[DB][NB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[db][nb] = f32x16{};
    float m_ref[NB], l_part[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) { m_ref[nb] = -INFINITY; l_part[nb] = 0.f; }

    // Per-lane LDS address terms of the fragment reads. They are rebuilt from `lane` where
    // they are used; pinning `lane` with an empty asm per iteration stops the compiler from
    // hoisting every buffer's addresses into registers for the whole loop.
    struct LaneAddr { int krow_sig, kx, h, tv_key, tv_chunk, tv_within, tv_swz; };
    auto lane_addr = [&](int ln_raw) {
        LaneAddr a;
        const int l32 = ln_raw & 31, tg = ln_raw >> 4, tc = ln_raw & 15;
        a.krow_sig = sigma(l32);
        a.kx = l32 & (KC - 1);
        a.h = ln_raw >> 5;
        a.tv_key = 8 * (tg >> 1) + (tc >> 2);          // + 16*kc + 4*t
        a.tv_chunk = 2 * (tg & 1) + ((tc & 3) >> 1);   // + 4*db
        a.tv_within = (tc & 1) * 8;                    // bytes
        a.tv_swz = vswz<KC>(a.tv_key);                 // (16*kc + 4*t + tv_key) % 4 == tv_key % 4
        return a;
    };

    // S^T = K Q^T for sub-step `sub` (32 keys x 32*NB queries) from K tile buffer cK
    auto qk = [&](int sub, const u32x4* cK, f32x16 (&acc)[NB], const LaneAddr& la) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
        const int krow = 32 * (sub & 1) + la.krow_sig;
#if defined(AULE_QK_PREFETCH)
        u32x4 af[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) af[ks] = cK[krow * KC + ((2 * ks + la.h) ^ la.kx)];
#endif
#if defined(AULE_SETPRIO)
        __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#if defined(AULE_QK_PREFETCH)
            const u32x4 a = af[ks];
#else
            const u32x4 a = cK[krow * KC + ((2 * ks + la.h) ^ la.kx)];
#endif
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = Mfma<T>::mma(a, qf[nb][ks], acc[nb]);
        }
#if defined(AULE_SETPRIO)
        __builtin_amdgcn_s_setprio(0);
#endif
    };
    // -inf for keys past the end and (causal) keys after the query; a uniform branch
    auto mask = [&](int sub, f32x16 (&acc)[NB]) {
        const int k0 = 32 * sub;
        if ((k0 + 32 > Lk) || (CAUSAL && k0 + 31 > qr0)) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int qi = qr0 + 32 * nb + ln;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 16 * (r >> 3) + 8 * h + (r & 7);
                    const bool masked = (key >= Lk) || (CAUSAL && key > qi);
                    acc[nb][r] = masked ? -INFINITY : acc[nb][r];
                }
            }
        }
    };
    // O^T += V^T P^T for sub-step `sub` from V tile buffer cV
    auto pv = [&](int sub, const u32x4* cV, const u32x4 (&pf)[2][NB], const LaneAddr& la) {
#if defined(AULE_SETPRIO)
        __builtin_amdgcn_s_setprio(1);
#endif
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int kc = 2 * (sub & 1) + cc;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                u32x4 a;
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int key = 16 * kc + 4 * t + la.tv_key;
                    const char* addr = reinterpret_cast<const char*>(cV + key * KC + ((4 * db + la.tv_chunk) ^ la.tv_swz)) + la.tv_within;
                    const i16x4_t part = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<char*>(addr)));
                    const u32x2 w = __builtin_bit_cast(u32x2, part);
                    a[2 * t] = w[0];
                    a[2 * t + 1] = w[1];
                }
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) o[db][nb] = Mfma<T>::mma(a, pf[cc][nb], o[db][nb]);
            }
        }
#if defined(AULE_SETPRIO)
        __builtin_amdgcn_s_setprio(0);
#endif
    };
    // online softmax of one sub-step: P (packed 16-bit) relative to the possibly raised
    // reference max; the O / l rescale is applied by finish() after this sub-step's
    // neighbours in the pipeline have been issued
    struct Soft { float m_new[NB], alpha[NB], lsum[NB]; bool raise[NB]; };
    auto softmax = [&](const f32x16 (&acc)[NB], u32x4 (&pf)[2][NB], Soft& st) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[nb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
            const bool any = __any(mt > m_ref[nb] + kRescaleSlack);
            const float m_new = any ? fmaxf(m_ref[nb], mt) : m_ref[nb];
            st.raise[nb] = any;
            st.m_new[nb] = m_new;
            st.alpha[nb] = __builtin_amdgcn_exp2f(m_ref[nb] - m_new);
            const float mneg = -m_new;
            float lsum = 0.f;
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                float pv8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) pv8[e] = __builtin_amdgcn_exp2f(fmaf(acc[nb][8 * cc + e], c, mneg));
                const u32x4 pk = {Mfma<T>::pack2(pv8[0], pv8[1]), Mfma<T>::pack2(pv8[2], pv8[3]),
                                  Mfma<T>::pack2(pv8[4], pv8[5]), Mfma<T>::pack2(pv8[6], pv8[7])};
                // the row sum uses the same rounded P that multiplies V, so O stays an
                // exact convex combination of V rows up to fp32 accumulation
#pragma unroll
                for (int w = 0; w < 4; ++w) lsum = Mfma<T>::sum2(pk[w], lsum);
                pf[cc][nb] = pk;
            }
            st.lsum[nb] = lsum;
        }
    };
    auto finish = [&](const Soft& st) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            if (st.raise[nb]) {
                l_part[nb] *= st.alpha[nb];
#pragma unroll
                for (int db = 0; db < DB; ++db) o[db][nb] *= st.alpha[nb];
            }
            l_part[nb] += st.lsum[nb];
            m_ref[nb] = st.m_new[nb];
        }
    };

    // ---------------------------------------------------------------- pipelined main loop
    // Iteration i issues, in one basic block, the matrix products of S(i+1) = K Q^T and of
    // O += V^T P(i-1) together with the softmax of S(i), so the vector ALU work of one
    // sub-step overlaps the matrix-core work of its neighbours. K/V tiles are triple
    // buffered (tile t in buffer t % 3): the copy of tile t+1 starts at the barrier before
    // the first iteration that reads tile t and must land by the next such barrier, one
    // tile later; by then tile t-2, which shared its buffer, has been read for the last
    // time. Iterations are unrolled by six so every buffer choice is a compile-time one.
    const uint32_t tk = kBN * k_rs, tv = kBN * v_rs;   // bytes per K / V tile
    lds_void* const lK[3] = {(lds_void*)sK0, (lds_void*)sK1, (lds_void*)sK2};
    lds_void* const lV[3] = {(lds_void*)sV0, (lds_void*)sV1, (lds_void*)sV2};
    const u32x4* const cKb[3] = {sK0, sK1, sK2};
    const u32x4* const cVb[3] = {sV0, sV1, sV2};

    f32x16 s_cur[NB], s_nxt[NB];
    u32x4 p_prev[2][NB], p_cur[2][NB];

    if constexpr (LOOP == 2) {
        // Ping-pong: the two waves of a SIMD (groups 0 and 1) alternate between a matrix
        // block M_m = {O += V^T P(m-1), S(m) = K Q^T} and a softmax block V_v, with a
        // workgroup barrier between phases. In phase p the group (p & 1) runs M_{p/2}
        // while the other group runs V_{p/2 - 1 + (p & 1)}, so one wave's vector work
        // hides under the other's matrix work. Tile t is read from phase 4t to phase 4t+5;
        // with three buffers the copy of tile t+2 starts at phase 4t+2 (tile t-1, its
        // buffer's previous tile, was last read in phase 4t+1) and is waited for at the
        // barrier before phase 4(t+2), when only the copy of tile t+3 may be newer.
        const int grp = (wave >> p.pp_shift) & 1;
        f32x16 sb[NB];
        u32x4 pb[2][NB];
        auto phase_barrier = [&](bool wait_tile, bool newer_pending) {
            if (wait_tile) {
                if (newer_pending) {
                    if constexpr (NI == 2) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
                    else asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
                } else {
                    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
                }
            } else {
                asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            }
        };
        issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, 0, 0, lK[0], lV[0], wave);
        if (n_kt > 1) issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, tk, tv, lK[1], lV[1], wave);
        phase_barrier(true, n_kt > 1);
        const int nphase = 2 * nsub + 2;
        for (int pg = 0; pg < nphase; pg += 12) {
#pragma unroll
            for (int q = 0; q < 12; ++q) {
                const int ph = pg + q;
                if (ph >= nphase) break;
                const int m = ph >> 1;
                if ((q & 3) == 2) {                           // phase 4u+2: copy tile u+2
                    const int t2 = (ph >> 2) + 2;
                    const int b2 = ((q >> 2) + 2) % 3;
                    if (t2 < n_kt) issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, t2 * tk, t2 * tv, lK[b2], lV[b2], wave);
                }
                if (grp == (q & 1)) {
                    // M_m: P(m-1) V and S(m) = K Q^T
                    const int kbuf = (q >> 2) % 3;            // tile m/2  (m/2 == ph/4)
                    const int vbuf = ((q + 10) >> 2) % 3;     // tile (m-1)/2 == (ph-2)/4, mod 3
                    const LaneAddr la = lane_addr(lane);
                    if (m < nsub) qk(m, cKb[kbuf], sb, la);
                    if (m >= 1 && m - 1 < nsub) pv(m - 1, cVb[vbuf], pb, la);
                } else {
                    const int v = m - 1 + (q & 1);
                    if (v >= 0 && v < nsub) {
                        mask(v, sb);
                        Soft st;
                        softmax(sb, pb, st);
                        finish(st);
                    }
                }
                const bool period_end = (q & 3) == 3;         // next phase starts tile (ph+1)/4
                const int tn = (ph + 1) >> 2;
                phase_barrier(period_end && tn < n_kt, tn + 1 < n_kt);
            }
        }
    } else if constexpr (LOOP == 0) {
        // Straight loop: per 32-key sub-step S = K Q^T, mask, softmax, P V. Tile t sits in
        // buffer t % 3. At the barrier before tile t each wave waits only for its copy of
        // tile t (the copy of tile t+1 may still be in flight), then starts the copy of
        // tile t+2 into the buffer of tile t-1, which every wave finished before this
        // barrier. Copies are thus requested two tiles ahead.
        issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, 0, 0, lK[0], lV[0], wave);
        if (n_kt > 1) issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, tk, tv, lK[1], lV[1], wave);
        for (int g = 0; 3 * g < n_kt; ++g) {
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int t = 3 * g + u;
                if (t >= n_kt) break;
                if (t + 1 < n_kt) {      // the copy of tile t+1 may stay outstanding
                    if constexpr (NI == 2) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
                    else asm volatile("s_waitcnt vmcnt(2) lgkmcnt(0)\n\ts_barrier" ::: "memory");
                } else {
                    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
                }
                if (t + 2 < n_kt)
                    issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, (t + 2) * tk, (t + 2) * tv,
                                   lK[(u + 2) % 3], lV[(u + 2) % 3], wave);
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int i = 2 * t + half;
                    if (i >= nsub) break;
                    const LaneAddr la = lane_addr(lane);
                    qk(i, cKb[u], s_cur, la);
                    mask(i, s_cur);
                    Soft st;
                    softmax(s_cur, p_cur, st);
                    finish(st);
                    pv(i, cVb[u], p_cur, la);
                }
            }
        }
    } else {

    // Instruction order of a full iteration (one basic block): a few LDS fragment reads up
    // front, then groups of one MFMA, a slice of the softmax VALU work and the next LDS
    // reads, so the matrix core and the vector ALU stay busy together and the fragment
    // registers stay short-lived.
    auto interleave = [&]() {
        constexpr int kMfma = NB * (KS + 2 * DB);      // matrix products per iteration
        constexpr int kDs = KS + 4 * DB;               // LDS fragment reads per iteration
        constexpr int kValu = (48 * NB + 32 + kMfma - 1) / kMfma;
        constexpr int kDsPer = (kDs - 4 + kMfma - 1) / kMfma;
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int k = 0; k < kMfma; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kValu, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, kDsPer, 0);
        }
    };

    issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, 0, 0, lK[0], lV[0], wave);
    __syncthreads();
    if (n_kt > 1) issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, tk, tv, lK[1], lV[1], wave);
    qk(0, cKb[0], s_cur, lane_addr(lane));
    mask(0, s_cur);
    {
        Soft st;
        if (nsub > 1) {
            qk(1, cKb[0], s_nxt, lane_addr(lane));
            softmax(s_cur, p_cur, st);
        } else {
            softmax(s_cur, p_cur, st);
        }
        finish(st);
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) p_prev[cc][nb] = p_cur[cc][nb];
        if (nsub > 1) {
            mask(1, s_nxt);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) s_cur[nb] = s_nxt[nb];
        }
    }
    for (int g = 0; 6 * g + 1 < nsub; ++g) {
#pragma unroll
        for (int u = 1; u <= 6; ++u) {
            const int i = 6 * g + u;
            if (i >= nsub) break;
            const int kb = ((u + 1) / 2) % 3;     // buffer of tile (i+1)/2
            const int vbuf = ((u - 1) / 2) % 3;   // buffer of tile (i-1)/2
            if (u & 1) {
                const int t = (i + 1) / 2;         // first iteration that reads tile t
                if (t < n_kt) {
                    __syncthreads();               // tile t landed; tile t-2 fully read
                    if (t + 1 < n_kt)
                        issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, (t + 1) * tk, (t + 1) * tv,
                                       lK[(kb + 1) % 3], lV[(kb + 1) % 3], wave);
                }
            }
            int lane_o = lane;
            asm volatile("" : "+v"(lane_o));
            const LaneAddr la = lane_addr(lane_o);
            Soft st;
            if (i + 1 < nsub) {
                qk(i + 1, cKb[kb], s_nxt, la);
                pv(i - 1, cVb[vbuf], p_prev, la);
                softmax(s_cur, p_cur, st);
                interleave();
            } else {
                pv(i - 1, cVb[vbuf], p_prev, la);
                softmax(s_cur, p_cur, st);
            }
            finish(st);
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) p_prev[cc][nb] = p_cur[cc][nb];
            if (i + 1 < nsub) {
                mask(i + 1, s_nxt);
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) s_cur[nb] = s_nxt[nb];
            }
        }
    }
    // the last sub-step's P^T V
    {
        const int last = nsub - 1;
        const int lb = (last / 2) % 3;
        pv(last, lb == 0 ? cVb[0] : lb == 1 ? cVb[1] : cVb[2], p_prev, lane_addr(lane));
    }
    }  // loop forms

    // ---------------------------------------------------------------- epilogue
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        const float l = l_part[nb] + __shfl_xor(l_part[nb], 32);
        const float inv = 1.f / l;
        const int row = qr0 + 32 * nb + ln;
        if (row < Lq) {
            T* orow = ob + (int64_t)row * p.o_rstride;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = 32 * db + 8 * g + 4 * h;
                    if (d0 < hd) {
                        u32x2 w = {Mfma<T>::pack2(o[db][nb][4 * g] * inv, o[db][nb][4 * g + 1] * inv),
                                   Mfma<T>::pack2(o[db][nb][4 * g + 2] * inv, o[db][nb][4 * g + 3] * inv)};
                        *reinterpret_cast<u32x2*>(orow + d0) = w;
                    }
                }
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

int heads_per_group(int group) { return (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1; }

int mfma_loop() {
    static const int v = [] {
        const char* e = std::getenv("AULE_MFMA_LOOP");
        const int v = e ? std::atoi(e) : 0;
        return (v >= 0 && v <= 2) ? v : 0;
    }();
    return v;
}
// which wave-index bit splits the ping-pong groups (waves w and w+4 share a SIMD: bit 2)
int pp_shift() {
    static const int v = [] {
        const char* e = std::getenv("AULE_PP_SHIFT");
        const int v = e ? std::atoi(e) : 2;
        return (v >= 0 && v <= 2) ? v : 2;
    }();
    return v;
}

template <typename T, int D, int WAVES, int NB, int GH, int LOOP, bool CAUSAL, bool VARLEN>
hipError_t launch_cfg(const AttnProblem& p, hipStream_t stream) {
    constexpr int BMW = 32 * NB * (WAVES / GH);
    dim3 block(WAVES * 64);
    AttnProblem pp = p;
    pp.pp_shift = pp_shift();
    if constexpr (VARLEN) {
        dim3 grid(varlen_grid_tiles(p.total_tokens, p.batch, BMW), p.heads_q / GH, 1);
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<T, D, WAVES, NB, GH, LOOP, CAUSAL, true>), grid, block, 0, stream, pp, 0);
    } else {
        const int n_qtiles = (p.seqlen_q + BMW - 1) / BMW;
        const int64_t nblocks = (int64_t)n_qtiles * p.batch * (p.heads_q / GH);
        if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
        dim3 grid((unsigned)nblocks);
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<T, D, WAVES, NB, GH, LOOP, CAUSAL, false>), grid, block, 0, stream, pp, n_qtiles);
    }
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, bool VARLEN>
hipError_t launch_gh(const AttnProblem& p, hipStream_t stream) {
    // loop form: AULE_MFMA_LOOP=0 straight (default), 1 software-pipelined, 2 ping-pong
    const int gh = VARLEN ? 1 : heads_per_group(p.group);
    const int g = gh == 4 ? 2 : gh == 2 ? 1 : 0;
    switch (mfma_loop() * 3 + g) {
        case 0: return launch_cfg<T, D, 8, 1, 1, 0, CAUSAL, VARLEN>(p, stream);
        case 1: return launch_cfg<T, D, 8, 1, 2, 0, CAUSAL, VARLEN>(p, stream);
        case 2: return launch_cfg<T, D, 8, 1, 4, 0, CAUSAL, VARLEN>(p, stream);
        case 3: return launch_cfg<T, D, 8, 1, 1, 1, CAUSAL, VARLEN>(p, stream);
        case 4: return launch_cfg<T, D, 8, 1, 2, 1, CAUSAL, VARLEN>(p, stream);
        case 5: return launch_cfg<T, D, 8, 1, 4, 1, CAUSAL, VARLEN>(p, stream);
        case 6: return launch_cfg<T, D, 8, 1, 1, 2, CAUSAL, VARLEN>(p, stream);
        case 7: return launch_cfg<T, D, 8, 1, 2, 2, CAUSAL, VARLEN>(p, stream);
        case 8: return launch_cfg<T, D, 8, 1, 4, 2, CAUSAL, VARLEN>(p, stream);
    }
    return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t launch_mode(const AttnProblem& p, hipStream_t stream) {
    const bool varlen = p.cu_seqlens != nullptr;
    if (p.causal) return varlen ? launch_gh<T, D, true, true>(p, stream) : launch_gh<T, D, true, false>(p, stream);
    return varlen ? launch_gh<T, D, false, true>(p, stream) : launch_gh<T, D, false, false>(p, stream);
}

template <typename T>
hipError_t launch_t(const AttnProblem& p, hipStream_t stream) {
    if (p.head_dim <= 64) return launch_mode<T, 64>(p, stream);
    return launch_mode<T, 128>(p, stream);
}

}  // namespace

bool mfma_supports(const AttnProblem& p, Dtype dt) {
    if (!(dt == Dtype::F16 || dt == Dtype::BF16) || p.head_dim > 128 || p.head_dim % 8 != 0) return false;
    // K/V copies address one (sequence, kv head) slice with 32-bit buffer offsets; keep the
    // slice plus one tile of offset headroom below 2^30 bytes.
    const int64_t rows = p.cu_seqlens ? p.total_tokens : p.seqlen_k;
    const int64_t stride = p.k_rstride > p.v_rstride ? p.k_rstride : p.v_rstride;
    const int64_t bytes = (rows + 128) * stride * 2;
    return bytes < (int64_t(1) << 30);
}

hipError_t launch_attn_fwd_mfma(const AttnProblem& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::BF16) return launch_t<bf16_t>(p, stream);
    if (dt == Dtype::F16) return launch_t<f16_t>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace aule
