// Split-KV decoding on the matrix cores (fp16/bf16, at most 32 query rows per kv head).
//
// The same split-KV scheme as attn_decode.hip (FlashAttention-T commentary, ai-stack.site,
// FAQ 4: the KV cache processed in blocks; partials merged with the running-max rescale of
// the xxqk.cn article, section 2.2), with the per-split work moved off the vector ALUs: the
// G * Nq query rows of one kv head form one 32-row block, so S^T = K Q^T and O^T = V^T P^T
// are 32 x 32 products exactly as in the forward kernel (rows beyond G * Nq are zero and
// never written). A workgroup of 4 waves takes one (split, kv head, batch); wave w walks
// the split's 32-key tiles w, w + 4, ... on its own: each wave has a private two-stage LDS
// ring filled by buffer_load ... lds copies (the K and V tile swizzles of the forward
// kernel; marked non-temporal, since every cache byte is read once), so the loop has no
// barrier, and one copy is in flight while the other tile is consumed. At the end the four waves' (m, l, O) are merged through LDS and written to the
// workspace in the layout the merge kernel of attn_decode.hip reads.
#include <hip/hip_runtime.h>
#include <math.h>

#include "attn_decode.h"
#include "attn_mfma.h"

namespace aule {
namespace {

constexpr int kWaves = 4;
constexpr int kTileKeys = 32;                              // keys per wave step
[[maybe_unused]] constexpr float kLog2eF = 1.4426950408889634f;
[[maybe_unused]] constexpr float kRescaleSlack = 8.0f;     // log2 units, as the forward kernel

// vmcnt(N) only (lgkmcnt and expcnt not waited for)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N <= 63, "vmcnt field is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename T, int D>
__global__ __launch_bounds__(kWaves * 64) void attn_decode_mfma_kernel(DecodeProblem p) {
#if defined(__HIP_DEVICE_COMPILE__)
    constexpr int KC = D / 8;                 // 16-byte chunks per K / V row
    constexpr int KS = D / 16;                // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;                // 32-row d-blocks of O^T
    constexpr int TCH = kTileKeys * KC;       // chunks per K (or V) tile
    constexpr int NI = TCH / 64;              // copy instructions per wave per K (or V) tile
    static_assert(NI * 64 == TCH, "a tile splits into whole wave copies");
    // [wave][stage][K = 0, V = 1][chunk]; reused for the final merge
    __shared__ u32x4 sbuf[kWaves][2][2][TCH];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, ln = lane & 31;
    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int G = p.group, Nq = p.seqlen_q, Nk = p.seqlen_k, d = p.head_dim;
    const int R = G * Nq;                     // rows of this workgroup, <= 32
    const int shift = Nk - Nq;                // query i is sequence position i + shift
    const int k_begin = split * p.keys_per_split;
    const int k_end = min(k_begin + p.keys_per_split, Nk);
    const int ntiles = k_end > k_begin ? (k_end - k_begin + kTileKeys - 1) / kTileKeys : 0;
    const int nmine = ntiles > wave ? (ntiles - wave + kWaves - 1) / kWaves : 0;   // this wave's tiles

    // K / V of this (batch, kv head); the descriptors end at the split's last key, so rows
    // past it (and chunks past head_dim, sent past the range) read as zero
    const int64_t kv_off = ((int64_t)b * p.heads_kv + hk) * (int64_t)Nk * d;
    const T* kbase = static_cast<const T*>(p.k) + kv_off;
    const T* vbase = static_cast<const T*>(p.v) + kv_off;
    const uint32_t row_bytes = (uint32_t)d * (uint32_t)sizeof(T);
    const i32x4 rk = buffer_desc(kbase, (int)((uint32_t)k_end * row_bytes));
    const i32x4 rv = buffer_desc(vbase, (int)((uint32_t)k_end * row_bytes));
    // this lane's LDS slot in each copy instruction: the global chunk that belongs there
    uint32_t koff[NI], voff[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const int slot = i * 64 + lane;
        const int row = slot / KC, pos = slot % KC;
        const int kc = pos ^ kswz<KC>(row), vc = pos ^ vswz<KC>(row);
        koff[i] = kc * 8 < d ? (uint32_t)row * row_bytes + (uint32_t)kc * 16u : kOobOffset;
        voff[i] = vc * 8 < d ? (uint32_t)row * row_bytes + (uint32_t)vc * 16u : kOobOffset;
    }
    auto lds_of = [](const u32x4* q) { return (uint32_t)(uintptr_t)(lds_void*)q; };
    // copy of this wave's j-th tile into stage j & 1
    auto issue = [&](int j) {
        const int stg = j & 1;
        const uint32_t key0 = (uint32_t)(k_begin + kTileKeys * (wave + kWaves * j));
        const uint32_t kdst = lds_of(sbuf[wave][stg][0]), vdst = lds_of(sbuf[wave][stg][1]);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            lds_copy16_stream(rk, koff[i] + key0 * row_bytes, __builtin_amdgcn_readfirstlane(kdst + (uint32_t)i * 1024u));
            lds_copy16_stream(rv, voff[i] + key0 * row_bytes, __builtin_amdgcn_readfirstlane(vdst + (uint32_t)i * 1024u));
        }
    };
    if (nmine > 0) issue(0);

    // Q: B operand of S^T (lane column ln = local row r = g * Nq + i; chunk 2ks + h); a
    // negative scale flips Q's sign bits so that c = |scale| log2(e)
    const bool neg = p.scale < 0.f;
    const float c = fmaxf(fabsf(p.scale) * kLog2eF, 1e-30f);   // scale 0: no -inf * 0
    u32x4 qf[KS];
    {
        const int r = ln < R ? ln : 0;
        const int g = r / Nq, i = r - g * Nq;
        const T* qrow = static_cast<const T*>(p.q) + (((int64_t)b * p.heads_q + hk * G + g) * Nq + i) * d;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int col = (2 * ks + h) * 8;
            u32x4 x = u32x4{0u, 0u, 0u, 0u};
            if (ln < R && col < d) x = *reinterpret_cast<const u32x4*>(qrow + col);
            qf[ks] = neg ? (x ^ 0x80008000u) : x;
        }
    }
    // this lane's query row: position in the sequence for the causal test
    const int my_i = ln < R ? ln % Nq : 0;
    const int my_last = p.causal ? my_i + shift : INT32_MAX;   // last visible key

    // per-lane fragment addressing (as the forward kernel's)
    const int krow = sigma(ln), kx = kx_lane<KC>(ln);
    const int tg = lane >> 4, tc = lane & 15;
    const int tv_key = 8 * (tg >> 1) + (tc >> 2);
    const int tv_chunk = 2 * (tg & 1) + ((tc & 3) >> 1);
    const int tv_within = (tc & 1) * 8;
    const int tv_swz = vswz<KC>(tv_key);

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    float m_ref = -INFINITY, l_part = 0.f;

    for (int j = 0; j < nmine; ++j) {
        if (j + 1 < nmine) {
            issue(j + 1);
            wait_vmcnt<2 * NI>();            // tile j has landed; tile j + 1 stays in flight
        } else {
            wait_vmcnt<0>();
        }
        const int stg = j & 1;
        const u32x4* cK = sbuf[wave][stg][0];
        const u32x4* cV = sbuf[wave][stg][1];
        const int k0 = k_begin + kTileKeys * (wave + kWaves * j);
        // S^T = K Q^T: register r of half h holds key k0 + 16 (r / 8) + 8h + r % 8, row ln
        u32x4 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = cK[krow * KC + ((2 * ks + h) ^ kx)];
        f32x16 s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = Mfma<T>::mma(kf[ks], qf[ks], s);
        // V^T fragments: two transposed 8-byte reads per 16-key chunk and d-block
        u32x4 vf[2][DB];
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int key = 16 * cc + 4 * t + tv_key;
                    const char* addr = reinterpret_cast<const char*>(cV + key * KC + ((4 * db + tv_chunk) ^ tv_swz)) + tv_within;
                    const i16x4_t part = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<char*>(addr)));
                    const u32x2 w = __builtin_bit_cast(u32x2, part);
                    vf[cc][db][2 * t] = w[0];
                    vf[cc][db][2 * t + 1] = w[1];
                }
        // masks (keys past the split's end, causal), a uniform branch
        if (k0 + kTileKeys > k_end || (p.causal && k0 + kTileKeys - 1 > shift)) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + 16 * (r >> 3) + 8 * h + (r & 7);
                s[r] = (key >= k_end || key > my_last) ? -INFINITY : s[r];
            }
        }
        // online softmax of the tile in log2 units, reference max raised lazily
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mt = mx == -INFINITY ? -INFINITY : mx * c;
        const bool raise = __any(mt > m_ref + kRescaleSlack);
        const float m_new = raise ? fmaxf(m_ref, mt) : m_ref;
        const float mneg = m_new == -INFINITY ? 0.f : -m_new;   // no visible key yet: P = 0
        u32x4 pf[2];
        float lsum = 0.f;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            float pv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(s[8 * cc + e], c, mneg));
            pf[cc] = u32x4{Mfma<T>::pack2(pv[0], pv[1]), Mfma<T>::pack2(pv[2], pv[3]),
                           Mfma<T>::pack2(pv[4], pv[5]), Mfma<T>::pack2(pv[6], pv[7])};
#pragma unroll
            for (int w = 0; w < 4; ++w) lsum = Mfma<T>::sum2(pf[cc][w], lsum);   // the rounded P
        }
        if (raise) {
            const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
            l_part *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= alpha;
            m_ref = m_new;
        }
        l_part += lsum;
        // O^T += V^T P^T
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] = Mfma<T>::mma(vf[cc][db], pf[cc], o[db]);
    }

    // ---- merge the four waves' partials of each row through LDS, then write the
    // workgroup's partial (m in log2 units, l, unnormalised O, fp32) for the merge kernel
    __syncthreads();                          // every wave is done with its ring
    float* sm = reinterpret_cast<float*>(&sbuf[0][0][0][0]);   // [wave][32]: m
    float* sl = sm + kWaves * 32;                              // [wave][32]: l
    float* so = sl + kWaves * 32;                              // [wave][32][D + 1]: O
    constexpr int OS = D + 1;                                  // padded: a lane per bank
    const float l_row = l_part + __shfl_xor(l_part, 32);
    if (h == 0) {
        sm[wave * 32 + ln] = m_ref;
        sl[wave * 32 + ln] = l_row;
    }
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            so[(wave * 32 + ln) * OS + 32 * db + 8 * (r >> 2) + 4 * h + (r & 3)] = o[db][r];
    __syncthreads();
    const int64_t rows_total = (int64_t)p.batch * p.heads_q * Nq;
    // thread t merges row t / 8, columns (t % 8) * (D / 8) .. + D / 8
    constexpr int CPT = D / 8;
    const int r = (int)threadIdx.x >> 3, c0 = ((int)threadIdx.x & 7) * CPT;
    if (r < R) {
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm[w * 32 + r]);
        float wt[kWaves], l = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = sm[w * 32 + r];
            wt[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);
            l = fmaf(sl[w * 32 + r], wt[w], l);
        }
        const int g = r / Nq, i = r - g * Nq;
        const int64_t row = ((int64_t)b * p.heads_q + hk * G + g) * Nq + i;
        const int64_t slot = (int64_t)split * rows_total + row;
        if ((threadIdx.x & 7) == 0) {
            p.ws_ml[2 * slot] = M;
            p.ws_ml[2 * slot + 1] = l;
        }
#pragma unroll
        for (int e = 0; e < CPT; ++e) {
            const int col = c0 + e;
            float x = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) x = fmaf(so[(w * 32 + r) * OS + col], wt[w], x);
            if (col < d) p.ws_o[slot * d + col] = x;
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace

bool decode_mfma_eligible(Dtype dt, int rows_per_kv_head, int head_dim) {
    return (dt == Dtype::BF16 || dt == Dtype::F16) && rows_per_kv_head <= 32 && head_dim <= 128;
}

bool decode_mfma_supports(const DecodeProblem& p, Dtype dt) {
    return decode_mfma_eligible(dt, p.group * p.seqlen_q, p.head_dim) && p.keys_per_split % kTileKeys == 0;
}

int decode_mfma_keys_granule() { return kTileKeys * kWaves; }

hipError_t launch_attn_decode_mfma_partial(const DecodeProblem& p, Dtype dt, hipStream_t stream) {
    dim3 grid(p.num_splits, p.heads_kv, p.batch);
    dim3 block(kWaves * 64);
    if (dt == Dtype::BF16) {
        if (p.head_dim <= 64) hipLaunchKernelGGL((attn_decode_mfma_kernel<bf16_t, 64>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_decode_mfma_kernel<bf16_t, 128>), grid, block, 0, stream, p);
    } else {
        if (p.head_dim <= 64) hipLaunchKernelGGL((attn_decode_mfma_kernel<f16_t, 64>), grid, block, 0, stream, p);
        else hipLaunchKernelGGL((attn_decode_mfma_kernel<f16_t, 128>), grid, block, 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace aule
