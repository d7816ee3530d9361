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

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kBN = 64;               // keys per K/V tile
constexpr int kRowsPerWave = 64;      // two 32-row blocks
[[maybe_unused]] constexpr float kRescaleSlack = 8.0f; // log2 units

template <typename T> struct Mfma;
template <> struct Mfma<bf16_t> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        bf16_t a = static_cast<bf16_t>(lo), b = static_cast<bf16_t>(hi);
        return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
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
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        f16_t a = static_cast<f16_t>(lo), b = static_cast<f16_t>(hi);
        return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
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

template <typename T, int D, int GH, bool CAUSAL, bool VARLEN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_mfma_kernel(AttnProblem p, int n_qtiles) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int RB = kWaves / GH;              // 64-row blocks per workgroup
    constexpr int BMW = kRowsPerWave * RB;       // query rows per workgroup
    constexpr int KC = D / 8;                    // 16-byte chunks per K / V row
    constexpr int KS = D / 16;                   // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;                   // 32-row d-blocks of O^T
    constexpr int NB = 2;                        // 32-query blocks per wave
    constexpr int TILE_CHUNKS = kBN * KC;        // 16-byte chunks per K (or V) tile
    constexpr int NI = TILE_CHUNKS / kThreads;   // load instructions per wave per tile
    static_assert(NI >= 1 && TILE_CHUNKS % kThreads == 0, "tile must split evenly over the waves");

    __shared__ u32x4 sK0[TILE_CHUNKS], sK1[TILE_CHUNKS];
    __shared__ u32x4 sV0[TILE_CHUNKS], sV1[TILE_CHUNKS];

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
        const int ngroups = p.heads_q / GH;
        const int per_tile = p.batch * ngroups;
        const int x = blockIdx.x;
        const int t = x / per_tile;
        const int rest = x - t * per_tile;
        tile = CAUSAL ? (n_qtiles - 1 - t) : t;     // longest causal tiles first
        bidx = rest / ngroups;
        hq0 = (rest - bidx * ngroups) * GH;
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

    // ---------------------------------------------------------------- tile ranges
    const int wg_rows_end = min(tile * BMW + BMW, Lq);
    const int n_kt = CAUSAL ? (wg_rows_end - 1) / kBN + 1 : (Lk + kBN - 1) / kBN;
    int wave_last;   // last K/V tile this wave computes on (-1: none)
    if (qr0 >= Lq) wave_last = -1;
    else wave_last = CAUSAL ? (min(qr0 + kRowsPerWave, Lq) - 1) / kBN : n_kt - 1;

    // ---------------------------------------------------------------- accumulators
    f32x16 o[DB][NB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) o[db][nb] = f32x16{};
    float m_ref[NB], l_part[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) { m_ref[nb] = -INFINITY; l_part[nb] = 0.f; }

    // lane constants of the transposed V reads
    const int tg = lane >> 4, tc = lane & 15;
    const int t_key = 8 * (tg >> 1) + (tc >> 2);          // + 16*kc + 4*t
    const int t_chunk = 2 * (tg & 1) + ((tc & 3) >> 1);   // + 4*db
    const int t_within = (tc & 1) * 8;                     // bytes

    auto compute_tile = [&](int j, const u32x4* cK, const u32x4* cV) {
        // two 32-key sub-steps per LDS tile keep the live S / P registers small; the
        // online softmax is exact at any step size
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int k0 = j * kBN + 32 * mb;
            if (CAUSAL && k0 > qr0 + kRowsPerWave - 1) continue;   // all keys in the future
            // S^T = K Q^T: 32 keys x 64 queries
            f32x16 s[NB];
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) s[nb] = f32x16{};
            const int krow = 32 * mb + sigma(ln);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 a = cK[krow * KC + ((2 * ks + h) ^ (ln & (KC - 1)))];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) s[nb] = Mfma<T>::mma(a, qf[nb][ks], s[nb]);
            }
            // mask keys past the end and (causal) keys after the query
            const bool need_mask = (k0 + 32 > Lk) || (CAUSAL && k0 + 31 > qr0);
            if (need_mask) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int qi = qr0 + 32 * nb + ln;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 16 * (r >> 3) + 8 * h + (r & 7);
                        const bool masked = (key >= Lk) || (CAUSAL && key > qi);
                        if (masked) s[nb][r] = -INFINITY;
                    }
                }
            }
            // online softmax per 32-query block
            u32x4 pf[2][NB];   // [16-key chunk][nb] packed P^T operands
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                float mx = -INFINITY;
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                const float mt = (mx == -INFINITY) ? -INFINITY : mx * c;
                const bool raise = mt > m_ref[nb] + kRescaleSlack;
                if (__any(raise)) {
                    const float m_new = fmaxf(m_ref[nb], mt);
                    const float alpha = __builtin_amdgcn_exp2f(m_ref[nb] - m_new);
                    l_part[nb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) o[db][nb] *= alpha;
                    m_ref[nb] = m_new;
                }
                const float mneg = -m_ref[nb];
                float lsum = 0.f;
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    float pv[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(s[nb][8 * cc + e], c, mneg));
                    const u32x4 pk = {Mfma<T>::pack2(pv[0], pv[1]), Mfma<T>::pack2(pv[2], pv[3]),
                                      Mfma<T>::pack2(pv[4], pv[5]), Mfma<T>::pack2(pv[6], pv[7])};
                    // the row sum uses the same rounded P that multiplies V, so O stays an
                    // exact convex combination of V rows up to fp32 accumulation
#pragma unroll
                    for (int w = 0; w < 4; ++w) lsum = Mfma<T>::sum2(pk[w], lsum);
                    pf[cc][nb] = pk;
                }
                l_part[nb] += lsum;
            }
            // O^T += V^T P^T over these 32 keys
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) {
                const int kc = 2 * mb + cc;
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    u32x4 a;
#pragma unroll
                    for (int t = 0; t < 2; ++t) {
                        const int key = 16 * kc + 4 * t + t_key;
                        const int chunk = (4 * db + t_chunk) ^ vswz<KC>(key);
                        const char* addr = reinterpret_cast<const char*>(cV + key * KC + chunk) + t_within;
                        const i16x4_t part = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_i16x4*)(const_cast<char*>(addr)));
                        const u32x2 w = __builtin_bit_cast(u32x2, part);
                        a[2 * t] = w[0];
                        a[2 * t + 1] = w[1];
                    }
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) o[db][nb] = Mfma<T>::mma(a, pf[cc][nb], o[db][nb]);
                }
            }
        }
    };

    // ---------------------------------------------------------------- main loop
    // Even tiles live in buffers 0, odd tiles in buffers 1; the copy of tile j+1 is in
    // flight while tile j is computed.
    const uint32_t tk = kBN * k_rs, tv = kBN * v_rs;   // bytes per K / V tile
    lds_void* const lK0 = (lds_void*)sK0;
    lds_void* const lK1 = (lds_void*)sK1;
    lds_void* const lV0 = (lds_void*)sV0;
    lds_void* const lV1 = (lds_void*)sV1;
    issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, 0, 0, lK0, lV0, wave);
    __syncthreads();
    for (int j = 0; j < n_kt; j += 2) {
        if (j + 1 < n_kt) issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, (j + 1) * tk, (j + 1) * tv, lK1, lV1, wave);
        if (j <= wave_last) compute_tile(j, sK0, sV0);
        __syncthreads();
        if (j + 1 >= n_kt) break;
        if (j + 2 < n_kt) issue_tile<NI>(rsrc_k, rsrc_v, koff, voff, (j + 2) * tk, (j + 2) * tv, lK0, lV0, wave);
        if (j + 1 <= wave_last) compute_tile(j + 1, sK1, sV1);
        __syncthreads();
    }

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

template <typename T, int D, int GH, bool CAUSAL, bool VARLEN>
hipError_t launch_cfg(const AttnProblem& p, hipStream_t stream) {
    constexpr int BMW = kRowsPerWave * (kWaves / GH);
    dim3 block(kThreads);
    if constexpr (VARLEN) {
        dim3 grid(varlen_grid_tiles(p.total_tokens, p.batch, BMW), p.heads_q / GH, 1);
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<T, D, GH, CAUSAL, true>), grid, block, 0, stream, p, 0);
    } else {
        const int n_qtiles = (p.seqlen_q + BMW - 1) / BMW;
        const int64_t nblocks = (int64_t)n_qtiles * p.batch * (p.heads_q / GH);
        if (nblocks > INT32_MAX) return hipErrorInvalidConfiguration;
        dim3 grid((unsigned)nblocks);
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<T, D, GH, CAUSAL, false>), grid, block, 0, stream, p, n_qtiles);
    }
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, bool VARLEN>
hipError_t launch_gh(const AttnProblem& p, hipStream_t stream) {
    switch (VARLEN ? 1 : heads_per_group(p.group)) {
        case 4: return launch_cfg<T, D, 4, CAUSAL, VARLEN>(p, stream);
        case 2: return launch_cfg<T, D, 2, CAUSAL, VARLEN>(p, stream);
        default: return launch_cfg<T, D, 1, CAUSAL, VARLEN>(p, stream);
    }
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
    const int64_t bytes = (rows + kBN) * stride * 2;
    return bytes < (int64_t(1) << 30);
}

hipError_t launch_attn_fwd_mfma(const AttnProblem& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::BF16) return launch_t<bf16_t>(p, stream);
    if (dt == Dtype::F16) return launch_t<f16_t>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace aule
