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
//   * scores (fp16/bf16): v_dot2 on packed pairs of K and raw Q, the scale applied to the
//     finished dot product; (fp32): fp32 FMAs against Q pre-multiplied by the scale;
//   * P V: lane l accumulates columns l and l + 64 of the wave's rows. fp16/bf16: P packed
//     in pairs (RNE, the same rounded values summed into l), V^T read from LDS with the
//     transposing ds_read_b64_tr_b16 (four keys of one column per lane), two v_dot2 per
//     four keys; fp32: fp32 FMAs, P read back from LDS four keys at a time.
#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>
#include <type_traits>

#include "attn_decode.h"

namespace aule {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

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
    // acc + a.lo * b.lo + a.hi * b.hi over packed pairs, in fp32
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
    }
    // two fp32 -> packed pair, round to nearest even
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
    }
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
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), acc, false);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, f16x2));
    }
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

    constexpr bool HALF = sizeof(T) == 2;            // 16-bit path: dot2 on packed pairs
    // Q rows: fp32 times scale * log2(e) (fp32 path) or the raw 16-bit chunks (16-bit path,
    // the scale multiplies the finished dot product). P: fp32 (fp32 path) or packed pairs
    // (16-bit path, the value that multiplies V). All read as vectors: 16-byte aligned.
    __shared__ __attribute__((aligned(16))) float sQ[HALF ? 1 : RMAX][D];
    __shared__ u32x4 sQh[HALF ? RMAX : 1][CPR];
    __shared__ u32x4 sK[TK * LDR];
    __shared__ u32x4 sV[TK * LDR];
    __shared__ __attribute__((aligned(16))) float sP[HALF ? 1 : RMAX][TK];
    __shared__ __attribute__((aligned(16))) uint32_t sPh[HALF ? RMAX : 1][TK / 2];

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
    if constexpr (HALF) {
        for (int idx = tid; idx < RMAX * CPR; idx += kThreads) {
            const int r = idx / CPR, cc = idx % CPR;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (r < R && cc * EPC < d) {
                const int g = r / Nq, i = r - g * Nq;
                const T* qrow = static_cast<const T*>(p.q) +
                                (((int64_t)b * p.heads_q + hk * G + g) * Nq + i) * d;
                x = *reinterpret_cast<const u32x4*>(qrow + cc * EPC);
            }
            sQh[r][cc] = x;
        }
    } else {
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

        // ---- scores: lane = key of the tile, wave rows r = wave + 4q (in log2 units)
        const int key = k0 + lane;
        float s[RPW];
        float s1[RPW], s2[RPW], s3[RPW];   // fp32: four partial sums, combined pairwise
#pragma unroll
        for (int q = 0; q < RPW; ++q) s[q] = s1[q] = s2[q] = s3[q] = 0.f;
        if (lane < TK) {
#pragma unroll 4
            for (int cc = 0; cc < CPR; ++cc) {
                const u32x4 kc = sK[lane * LDR + cc];
                if constexpr (HALF) {
#pragma unroll
                    for (int q = 0; q < RPW; ++q) {
                        const int r = wave + 4 * q;
                        if (r < R) {
                            const u32x4 qc = sQh[r][cc];
#pragma unroll
                            for (int w = 0; w < 4; ++w) s[q] = Elem<T>::dot2(kc[w], qc[w], s[q]);
                        }
                    }
                } else {
                    float kf[EPC];
                    Elem<T>::chunk(kc, kf);
#pragma unroll
                    for (int q = 0; q < RPW; ++q) {
                        const int r = wave + 4 * q;
                        if (r < R) {
                            const f32x4 qq = *reinterpret_cast<const f32x4*>(&sQ[r][cc * EPC]);
                            s[q] = fmaf(kf[0], qq[0], s[q]);
                            s1[q] = fmaf(kf[1], qq[1], s1[q]);
                            s2[q] = fmaf(kf[2], qq[2], s2[q]);
                            s3[q] = fmaf(kf[3], qq[3], s3[q]);
                        }
                    }
                }
            }
            if constexpr (HALF) {
#pragma unroll
                for (int q = 0; q < RPW; ++q) s[q] *= c;
            } else {
#pragma unroll
                for (int q = 0; q < RPW; ++q) s[q] = (s[q] + s1[q]) + (s2[q] + s3[q]);
            }
        }
        // ---- online softmax per row (wave-uniform branches). 16-bit path: P is packed in
        // pairs of neighbouring keys (even lanes store), and the row sum is taken over the
        // rounded pairs, so l matches the P that multiplies V.
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
            if constexpr (HALF) {
                const float pn = __shfl_xor(pj, 1);
                if ((lane & 1) == 0 && lane < TK) {
                    const uint32_t pk = Elem<T>::pack2(pj, pn);
                    sPh[r][lane >> 1] = pk;
                    lpart[q] = Elem<T>::dot2(pk, Elem<T>::pack2(1.f, 1.f), lpart[q]);
                }
            } else {
                lpart[q] += pj;
                if (lane < TK) sP[r][lane] = pj;
            }
        }
        // ---- O += P V; lane owns columns lane + 64 e. Each wave reads only the P rows it
        // wrote, so no barrier is needed in between.
        if constexpr (HALF) {
            // V^T from the row-major V tile: each 16-lane group reads a 4-key x 16-column
            // block transposed (lane c addresses key c/4, columns 4(c%4)..+3; lane i gets
            // the 4 keys of column i), then two dot2 against the matching P pairs.
            const int tg = lane >> 4, tc = lane & 15;
#pragma unroll 4
            for (int j4 = 0; j4 < TK; j4 += 4) {
                u32x2 vt[CPL];
#pragma unroll
                for (int e = 0; e < CPL; ++e) {
                    const int col = 64 * e + 16 * tg + 4 * (tc & 3);
                    const char* addr = reinterpret_cast<const char*>(&sV[(j4 + (tc >> 2)) * LDR + col / EPC]) +
                                       (col % EPC) * sizeof(T);
                    const i16x4_t part = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<char*>(addr)));
                    vt[e] = __builtin_bit_cast(u32x2, part);
                }
#pragma unroll
                for (int q = 0; q < RPW; ++q) {
                    const int r = wave + 4 * q;
                    if (r >= R) continue;
                    const u32x2 pp = *reinterpret_cast<const u32x2*>(&sPh[r][j4 >> 1]);
#pragma unroll
                    for (int e = 0; e < CPL; ++e) {
                        o[q][e] = Elem<T>::dot2(vt[e][0], pp[0], o[q][e]);
                        o[q][e] = Elem<T>::dot2(vt[e][1], pp[1], o[q][e]);
                    }
                }
            }
        } else {
#pragma unroll 2
            for (int j4 = 0; j4 < TK; j4 += 4) {
                float vv[4][CPL];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float* vr = reinterpret_cast<const float*>(&sV[(j4 + jj) * LDR]);
#pragma unroll
                    for (int e = 0; e < CPL; ++e) vv[jj][e] = vr[lane + 64 * e];
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
            const int col = lane + 64 * e;
            if (col < d) p.ws_o[slot * d + col] = o[q][e];
        }
    }
}

// Merge the splits of one output row: m = max m_s, l = sum l_s 2^(m_s - m),
// O = sum O_s 2^(m_s - m) / l. One wave per (batch, head, query) row: lane s holds split s's
// statistics (64 splits at a time), the weights go through wave reductions, and the
// partial outputs of all splits are loaded independently (columns lane and lane + 64).
template <typename T>
__global__ __launch_bounds__(64) void attn_decode_combine_kernel(DecodeProblem p) {
    const int64_t row = blockIdx.x;
    const int64_t rows_total = (int64_t)p.batch * p.heads_q * p.seqlen_q;
    const int d = p.head_dim;
    const int lane = threadIdx.x;
    const int S = p.num_splits;
    float mx = -INFINITY;
    for (int s0 = 0; s0 < S; s0 += 64) {
        const int s = s0 + lane;
        const float ms = s < S ? p.ws_ml[2 * (s * rows_total + row)] : -INFINITY;
        mx = fmaxf(mx, wave_max(ms));
    }
    float l = 0.f;
    float acc[2] = {0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += 64) {
        const int s = s0 + lane;
        float w = 0.f;
        if (s < S) {
            const int64_t slot = s * rows_total + row;
            const float ms = p.ws_ml[2 * slot];
            // a split without any visible key has m = -inf and weight 0
            w = ms == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms - mx);
            l = fmaf(p.ws_ml[2 * slot + 1], w, l);
        }
        const int n = min(64, S - s0);
        for (int j = 0; j < n; ++j) {   // independent loads: issued back to back
            const float wj = __shfl(w, j);
            const int64_t slot = (int64_t)(s0 + j) * rows_total + row;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int col = lane + 64 * e;
                if (col < d) acc[e] = fmaf(p.ws_o[slot * d + col], wj, acc[e]);
            }
        }
    }
    l = wave_sum(l);
    const float inv = 1.f / l;
    T* orow = static_cast<T*>(p.o) + row * d;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int col = lane + 64 * e;
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
    const Dtype dt = std::is_same<T, float>::value ? Dtype::F32 : std::is_same<T, bf16_t>::value ? Dtype::BF16 : Dtype::F16;
    hipError_t e = decode_mfma_supports(p, dt) ? launch_attn_decode_mfma_partial(p, dt, stream)
                   : p.head_dim <= 64          ? launch_partial<T, 64>(p, stream)
                                               : launch_partial<T, 128>(p, stream);
    if (e != hipSuccess) return e;
    const int64_t rows = (int64_t)p.batch * p.heads_q * p.seqlen_q;
    hipLaunchKernelGGL((attn_decode_combine_kernel<T>), dim3((unsigned)rows), dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

// Workspace of the entry point that allocates nothing: one fixed array per GPU, held from
// the library's first use on that GPU until the process ends. Every call on a GPU shares
// it, so calls that overlap in time on one GPU race. Nothing in it needs clearing: the
// partial kernel writes every (split, row) slot that the merge kernel reads.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void** ptr) {
    // In host code `scratch` only names the symbol; the array's address on the current
    // device comes from the runtime, once per device, and is what the kernels are given.
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!a) return hipErrorInvalidSymbol;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

int decode_keys_per_tile(Dtype dt) { return dt == Dtype::F32 ? 32 : 64; }

hipError_t launch_attn_decode(const DecodeProblem& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::BF16) return launch_t<bf16_t>(p, stream);
    if (dt == Dtype::F16) return launch_t<f16_t>(p, stream);
    return launch_t<float>(p, stream);
}

}  // namespace aule
