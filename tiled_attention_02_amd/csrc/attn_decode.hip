// Split-KV attention of a few new queries against a long key/value cache (decoding), for
// fp16, bf16 and fp32.
//
// The FlashAttention-T commentary (ai-stack.site, FAQ 4) notes that at inference the KV
// cache is processed in blocks. With only Nq new queries per sequence the work per key is
// G * Nq dot products, far too little for the matrix cores to matter: the kernel is bound by
// streaming K and V from HBM once. So the key range is split across workgroups (the grid is
// splits x kv heads x batch, enough to fill the chip even at batch 1), each workgroup runs
// the online softmax over its keys for all G * Nq query rows that share its kv head, and
// writes a partial (m, l, O) in fp32; a second kernel merges the partials of each row with
// the same rescale the forward kernel applies between key blocks (xxqk.cn article, section
// 2.2: running max and sum, rescaled partial sums).
//
// Causal masking is bottom-right aligned: the new queries are the last Nq positions of the
// Nk-long sequence, so query i sees keys j <= i + Nk - Nq.
//
// Work split of the partial kernel (256 threads = 4 waves):
//   * K/V tiles of TK keys are staged in LDS (rows padded by 16 bytes so that one lane per
//     key reads conflict-free); the next tile is fetched into registers while the current
//     one is consumed, then written to LDS between two barriers;
//   * scores: lane j of every wave takes key j of the tile; wave w takes the query rows
//     r = w, w+4, ... (Q is held in LDS in fp32, pre-multiplied by scale * log2(e));
//   * softmax: row max by a wave-wide reduction, P = exp2(s - m); each lane keeps its own
//     partial row sum, reduced once at the end;
//   * P V: lane l accumulates columns D/64 * l ... of the wave's rows, reading P back from
//     LDS (one broadcast read per four keys) and one V element group per key.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_decode.h"

namespace aule {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
    // eight bf16 in a 16-byte chunk -> fp32 (a bf16 is the high half of an fp32)
    static __device__ __forceinline__ void chunk(u32x4 c, float* f) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            f[2 * w] = __builtin_bit_cast(float, c[w] << 16);
            f[2 * w + 1] = __builtin_bit_cast(float, c[w] & 0xFFFF0000u);
        }
    }
    static constexpr int kPerChunk = 8;
    static __device__ __forceinline__ bf16_t from_f32(float x) { return (bf16_t)x; }   // RNE
};
template <> struct Elem<f16_t> {
    static __device__ __forceinline__ void chunk(u32x4 c, float* f) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            f[2 * w] = (float)__builtin_bit_cast(f16_t, (uint16_t)(c[w] & 0xFFFFu));
            f[2 * w + 1] = (float)__builtin_bit_cast(f16_t, (uint16_t)(c[w] >> 16));
        }
    }
    static constexpr int kPerChunk = 8;
    static __device__ __forceinline__ f16_t from_f32(float x) { return (f16_t)x; }     // RNE
};
template <> struct Elem<float> {
    static __device__ __forceinline__ void chunk(u32x4 c, float* f) {
        // each element goes through a scalar first: a bit cast applied directly to the
        // vector element (an lvalue) was compiled as a cast of element 0 every time
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const uint32_t bits = c[w];
            f[w] = __builtin_bit_cast(float, bits);
        }
    }
    static constexpr int kPerChunk = 4;
    static __device__ __forceinline__ float from_f32(float x) { return x; }
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// T: element type; D: padded head dim (64 or 128); RMAX: query rows per workgroup (G * Nq).
template <typename T, int D, int RMAX>
__global__ __launch_bounds__(kThreads) void attn_decode_partial_kernel(DecodeProblem p) {
    constexpr int EPC = Elem<T>::kPerChunk;          // elements per 16-byte chunk
    constexpr int CPR = D / EPC;                     // chunks per K/V row
    constexpr int LDR = CPR + 1;                     // LDS row stride in chunks (padded)
    constexpr int TK = sizeof(T) == 4 ? 32 : 64;     // keys per tile
    constexpr int TILE_CHUNKS = TK * CPR;
    constexpr int NLD = TILE_CHUNKS / kThreads;      // staged chunks per thread, K and V each
    constexpr int RPW = RMAX / 4;                    // query rows per wave (upper bound)
    constexpr int CPL = D / 64;                      // output columns per lane
    static_assert(NLD * kThreads == TILE_CHUNKS, "tile must split over the threads");
    static_assert(TK <= 64, "one lane per key");

    // sQ and sP are read as 16-byte vectors: keep them 16-byte aligned
    __shared__ __attribute__((aligned(16))) float sQ[RMAX][D];
    __shared__ u32x4 sK[TK * LDR];
    __shared__ u32x4 sV[TK * LDR];
    __shared__ __attribute__((aligned(16))) float sP[RMAX][TK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int G = p.group, Nq = p.seqlen_q, Nk = p.seqlen_k, d = p.head_dim;
    const int R = G * Nq;                            // rows of this workgroup, <= RMAX
    const int shift = Nk - Nq;                       // query i is sequence position i + shift

    // key range of this split
    const int k_begin = split * p.keys_per_split;
    const int k_end = min(k_begin + p.keys_per_split, Nk);

    // Q rows -> LDS as fp32 times scale * log2(e); row r = g * Nq + i is query i of head
    // hk * G + g
    const float c = p.scale * kLog2e;
    for (int idx = tid; idx < RMAX * D; idx += kThreads) {
        const int r = idx / D, col = idx % D;
        float x = 0.f;
        if (r < R && col < d) {
            const int g = r / Nq, i = r - g * Nq;
            const T* qrow = static_cast<const T*>(p.q) +
                            (((int64_t)b * p.heads_q + hk * G + g) * Nq + i) * d;
            x = static_cast<float>(qrow[col]);
        }
        sQ[r][col] = x * c;
    }

    const T* kbase = static_cast<const T*>(p.k) + ((int64_t)b * p.heads_kv + hk) * (int64_t)Nk * d;
    const T* vbase = static_cast<const T*>(p.v) + ((int64_t)b * p.heads_kv + hk) * (int64_t)Nk * d;

    // staged chunk loads of one tile (zero outside [k_begin, k_end) and past head_dim)
    u32x4 stK[NLD], stV[NLD];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int id = u * kThreads + tid;
            const int row = id / CPR, cc = id % CPR;
            const int key = k0 + row;
            u32x4 a = {0u, 0u, 0u, 0u}, v = {0u, 0u, 0u, 0u};
            if (key < k_end && cc * EPC < d) {
                const int64_t off = (int64_t)key * d + cc * EPC;
                a = *reinterpret_cast<const u32x4*>(kbase + off);
                v = *reinterpret_cast<const u32x4*>(vbase + off);
            }
            stK[u] = a;
            stV[u] = v;
        }
    };
    auto stage = [&]() {
#pragma unroll
        for (int u = 0; u < NLD; ++u) {
            const int id = u * kThreads + tid;
            const int row = id / CPR, cc = id % CPR;
            sK[row * LDR + cc] = stK[u];
            sV[row * LDR + cc] = stV[u];
        }
    };

    // per-wave row state
    float m[RPW], lpart[RPW], o[RPW][CPL];
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        m[q] = -INFINITY;
        lpart[q] = 0.f;
#pragma unroll
        for (int e = 0; e < CPL; ++e) o[q][e] = 0.f;
    }

    if (k_begin < k_end) fetch(k_begin);
    for (int k0 = k_begin; k0 < k_end; k0 += TK) {
        __syncthreads();                              // previous tile fully consumed
        stage();
        __syncthreads();                              // tile visible (and sQ, first time)
        if (k0 + TK < k_end) fetch(k0 + TK);          // next tile in flight during compute

        // ---- scores: lane = key of the tile, wave rows r = wave + 4q
        const int key = k0 + lane;
        float s[RPW];
#pragma unroll
        for (int q = 0; q < RPW; ++q) s[q] = 0.f;
        if (lane < TK) {
#pragma unroll 4
            for (int cc = 0; cc < CPR; ++cc) {
                float kf[EPC];
                Elem<T>::chunk(sK[lane * LDR + cc], kf);
#pragma unroll
                for (int q = 0; q < RPW; ++q) {
                    const int r = wave + 4 * q;
                    if (r < R) {
                        const f32x4* qv = reinterpret_cast<const f32x4*>(&sQ[r][cc * EPC]);
#pragma unroll
                        for (int e4 = 0; e4 < EPC / 4; ++e4) {
                            const f32x4 qq = qv[e4];
                            s[q] = fmaf(kf[4 * e4], qq[0], s[q]);
                            s[q] = fmaf(kf[4 * e4 + 1], qq[1], s[q]);
                            s[q] = fmaf(kf[4 * e4 + 2], qq[2], s[q]);
                            s[q] = fmaf(kf[4 * e4 + 3], qq[3], s[q]);
                        }
                    }
                }
            }
        }
        // ---- online softmax per row (wave-uniform branches)
#pragma unroll
        for (int q = 0; q < RPW; ++q) {
            const int r = wave + 4 * q;
            if (r >= R) continue;
            const int i = r % Nq;
            const bool visible = lane < TK && key < k_end && (!p.causal || key <= i + shift);
            const float t = visible ? s[q] : -INFINITY;
            const float m_new = fmaxf(m[q], wave_max(t));
            float pj = 0.f;
            if (m_new != -INFINITY) {
                const float alpha = __builtin_amdgcn_exp2f(m[q] - m_new);
                pj = __builtin_amdgcn_exp2f(t - m_new);
                lpart[q] *= alpha;
#pragma unroll
                for (int e = 0; e < CPL; ++e) o[q][e] *= alpha;
                m[q] = m_new;
            }
            lpart[q] += pj;
            if (lane < TK) sP[r][lane] = pj;
        }
        // ---- O += P V: lane owns columns CPL * lane ...; P read back four keys at a time
        // (each wave reads only the rows it wrote, so no barrier is needed in between)
#pragma unroll 2
        for (int j4 = 0; j4 < TK; j4 += 4) {
            float vv[4][CPL];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j = j4 + jj;
                const int col0 = CPL * lane;                       // element column
                const T* vr = reinterpret_cast<const T*>(&sV[j * LDR + col0 / EPC]) + col0 % EPC;
#pragma unroll
                for (int e = 0; e < CPL; ++e) vv[jj][e] = static_cast<float>(vr[e]);
            }
#pragma unroll
            for (int q = 0; q < RPW; ++q) {
                const int r = wave + 4 * q;
                if (r >= R) continue;
                const f32x4 pp = *reinterpret_cast<const f32x4*>(&sP[r][j4]);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
#pragma unroll
                    for (int e = 0; e < CPL; ++e) o[q][e] = fmaf(pp[jj], vv[jj][e], o[q][e]);
            }
        }
    }

    // ---- partials: m (log2 units), l, unnormalised O, all fp32
    const int64_t rows_total = (int64_t)p.batch * p.heads_q * Nq;
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        const int r = wave + 4 * q;
        if (r >= R) continue;
        const int g = r / Nq, i = r - g * Nq;
        const int64_t row = ((int64_t)b * p.heads_q + hk * G + g) * Nq + i;
        const int64_t slot = (int64_t)split * rows_total + row;
        const float l = wave_sum(lpart[q]);
        if (lane == 0) {
            p.ws_ml[2 * slot] = m[q];
            p.ws_ml[2 * slot + 1] = l;
        }
#pragma unroll
        for (int e = 0; e < CPL; ++e) {
            const int col = CPL * lane + e;
            if (col < d) p.ws_o[slot * d + col] = o[q][e];
        }
    }
}

// Merge the splits of one output row: m = max m_s, l = sum l_s 2^(m_s - m),
// O = sum O_s 2^(m_s - m) / l. One workgroup of 64 threads per (batch, head, query) row.
template <typename T>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(DecodeProblem p) {
    const int64_t row = blockIdx.x;
    const int64_t rows_total = (int64_t)p.batch * p.heads_q * p.seqlen_q;
    const int d = p.head_dim;
    float mx = -INFINITY;
    for (int s = 0; s < p.num_splits; ++s) mx = fmaxf(mx, p.ws_ml[2 * (s * rows_total + row)]);
    float l = 0.f;
    float acc[2] = {0.f, 0.f};
    for (int s = 0; s < p.num_splits; ++s) {
        const int64_t slot = s * rows_total + row;
        const float ms = p.ws_ml[2 * slot];
        if (ms == -INFINITY) continue;              // a split with no visible key
        const float w = __builtin_amdgcn_exp2f(ms - mx);
        l = fmaf(p.ws_ml[2 * slot + 1], w, l);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int col = threadIdx.x + 64 * e;
            if (col < d) acc[e] = fmaf(p.ws_o[slot * d + col], w, acc[e]);
        }
    }
    const float inv = 1.f / l;
    T* orow = static_cast<T*>(p.o) + row * d;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int col = threadIdx.x + 64 * e;
        if (col < d) orow[col] = Elem<T>::from_f32(acc[e] * inv);
    }
}

template <typename T, int D>
hipError_t launch_partial(const DecodeProblem& p, hipStream_t stream) {
    dim3 grid(p.num_splits, p.heads_kv, p.batch);
    const int R = p.group * p.seqlen_q;
    if (R <= 16) hipLaunchKernelGGL((attn_decode_partial_kernel<T, D, 16>), grid, dim3(kThreads), 0, stream, p);
    else hipLaunchKernelGGL((attn_decode_partial_kernel<T, D, 64>), grid, dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const DecodeProblem& p, hipStream_t stream) {
    hipError_t e = p.head_dim <= 64 ? launch_partial<T, 64>(p, stream) : launch_partial<T, 128>(p, stream);
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)p.batch * p.heads_q * p.seqlen_q;
    hipLaunchKernelGGL((attn_decode_combine_kernel<T>), dim3((unsigned)rows), dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

int decode_keys_per_tile(Dtype dt) { return dt == Dtype::F32 ? 32 : 64; }

hipError_t launch_attn_decode(const DecodeProblem& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::BF16) return launch_t<bf16_t>(p, stream);
    if (dt == Dtype::F16) return launch_t<f16_t>(p, stream);
    return launch_t<float>(p, stream);
}

}  // namespace aule
