// Short-sequence attention forward (fp16/bf16, at most 128 keys) on gfx950.
//
// For very short sequences and large batches, a single compact kernel that holds the whole
// score block of a head in one place beats the tiled block schedule, whose set-up and
// streaming machinery dominates such small matrices (xxqk.cn article
// "Attention算子实战：从CUDA优化到昇腾/CANN部署", section 2.3: the diffusion-model
// workload, sequences of at most ~64 tokens at large batch, e.g. 64 queries against 77
// keys, computed as one monolithic block with the row max and row sum exchanged between
// threads). Here that block is laid out for CDNA4:
//
//   * one workgroup per (batch, kv head): its whole K and V (at most 128 rows) are copied
//     global -> LDS once with buffer_load_dwordx4 ... lds, in the same swizzled layout the
//     tiled kernel uses, and read by every query head of the GQA group;
//   * each wave takes (query head, 32-row block) items; per item the full score row of
//     each query is formed in registers (S^T = K Q^T on v_mfma_f32_32x32x16, one 32x32
//     accumulator per 32 keys), so the softmax is the plain two-pass one: exact row max
//     (in-lane reduction plus one exchange with lane ^ 32), exp2, row sum over the rounded
//     P, then O^T = V^T P^T with P taken straight from the accumulators (K rows fed in
//     sigma order) and V^T read with ds_read_b64_tr_b16;
//   * causal rows skip the 32-key blocks after their diagonal.
// There is no online rescale, no double buffering and only one barrier (after the copy).
#include <hip/hip_runtime.h>
#include <math.h>


#include "attn_device.h"
#include "attn_mfma.h"

namespace aule {
namespace {

constexpr int kShortMaxKeys = 128;
[[maybe_unused]] constexpr int kMaxSub = kShortMaxKeys / 32;   // 32-key blocks of the score row
constexpr int kShortMaxItems = 16;            // (query head, 32-row block) items per workgroup

template <typename T, int D, int WAVES, bool CAUSAL>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_short_kernel(AttnProblem p, int n_rb) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int KC = D / 8;    // 16-byte chunks per K / V row
    constexpr int KS = D / 16;   // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;   // 32-row d-blocks of O^T
    extern __shared__ u32x4 smem[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int h = lane >> 5, ln = lane & 31;
    const int hd = p.head_dim, Lq = p.seqlen_q, Lk = p.seqlen_k;
    const int nsub = (Lk + 31) / 32;             // 1 .. kMaxSub (checked on the host)
    const int rows = nsub * 32;
    u32x4* sK = smem;
    u32x4* sV = smem + rows * KC;

    const int unit = blockIdx.x;                 // (batch, kv head)
    const int b = unit / p.heads_kv, hk = unit - b * p.heads_kv;
    const uint32_t k_rs = (uint32_t)(p.k_rstride * (int64_t)sizeof(T));
    const uint32_t v_rs = (uint32_t)(p.v_rstride * (int64_t)sizeof(T));
    const uint32_t q_rs = (uint32_t)(p.q_rstride * (int64_t)sizeof(T));
    const uint32_t o_rs = (uint32_t)(p.o_rstride * (int64_t)sizeof(T));

    // Q^T of an item as B operands: lane column = query qr0 + ln; rows past Lq and columns
    // past head_dim read as zero through the descriptor bound and the out-of-range offset
    const int n_items = p.group * n_rb;
    u32x4 qf[KS];
    auto load_q = [&](int it) {
        const int g = it / n_rb, rb = it - g * n_rb;
        const T* qb = static_cast<const T*>(p.q) + b * p.q_bstride + (hk * p.group + g) * p.q_hstride;
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T*>(qb), (short)0, (int)((int64_t)Lq * q_rs), (int)kBufferFlags);
        const uint32_t off = (uint32_t)(32 * rb + ln) * q_rs + (uint32_t)h * 16u;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint32_t o = (2 * ks + h) * 8 < hd ? off + (uint32_t)ks * 32u : kOobOffset;
            qf[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)o, 0, 0));
        }
    };
    // the first item's Q is fetched together with K and V, so that the two fetches overlap
    if (wave < n_items) load_q(wave);

    // ------------------------------------------------ K, V of the slice -> LDS (zero-padded)
    {
        const T* kb = static_cast<const T*>(p.k) + b * p.k_bstride + hk * p.k_hstride;
        const T* vb = static_cast<const T*>(p.v) + b * p.v_bstride + hk * p.v_hstride;
        const i32x4 rk = buffer_desc(kb, (int)((Lk - 1) * k_rs + hd * sizeof(T)));
        const i32x4 rv = buffer_desc(vb, (int)((Lk - 1) * v_rs + hd * sizeof(T)));
        // rows * KC chunks per tensor, a multiple of 64 * WAVES; each copy instruction fills
        // 1 KiB (64 lanes x 16 bytes) of LDS, every lane fetching the global chunk that
        // belongs at its slot (rows past Lk and columns past head_dim read as zero)
        const int per = rows * KC / (64 * WAVES);
        const uint32_t lK = (uint32_t)(uintptr_t)(lds_void*)sK, lV = (uint32_t)(uintptr_t)(lds_void*)sV;
        for (int i = 0; i < per; ++i) {
            const int blk = wave * per + i;
            const int slot = blk * 64 + lane;
            const int row = slot / KC, pos = slot % KC;
            const int kdc = pos ^ kswz<KC>(row), vdc = pos ^ vswz<KC>(row);
            const uint32_t ko = kdc * 8 < hd ? row * k_rs + kdc * 16 : kOobOffset;
            const uint32_t vo = vdc * 8 < hd ? row * v_rs + vdc * 16 : kOobOffset;
            lds_copy16(rk, ko, __builtin_amdgcn_readfirstlane(lK + blk * 1024u));
            lds_copy16(rv, vo, __builtin_amdgcn_readfirstlane(lV + blk * 1024u));
        }
        // the copies are invisible to the compiler: wait for them explicitly (vmcnt(0),
        // lgkmcnt(0)), then make every wave's part visible to all
        __builtin_amdgcn_s_waitcnt(0x70);
        asm volatile("s_barrier" ::: "memory");
    }

    // per-lane LDS address terms of the fragment reads
    const int krow_sig = sigma(ln), kx = kx_lane<KC>(ln);
    const int tg = lane >> 4, tc = lane & 15;
    const int tv_key = 8 * (tg >> 1) + (tc >> 2);
    const int tv_chunk = 2 * (tg & 1) + ((tc & 3) >> 1);
    const int tv_within = (tc & 1) * 8;
    const int tv_swz = vswz<KC>(tv_key);

    const bool neg = p.scale_log2 < 0.f;
    const float c = fmaxf(fabsf(p.scale_log2), 1e-30f);

    for (int it = wave; it < n_items; it += WAVES) {
        const int g = it / n_rb, rb = it - g * n_rb;
        const int hq = hk * p.group + g;
        const int qr0 = 32 * rb;
        T* ob = static_cast<T*>(p.o) + b * p.o_bstride + hq * p.o_hstride;

        if (it != wave) load_q(it);
        if (neg)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qf[ks] ^= 0x80008000u;   // a negative scale flips the sign of Q exactly

        // full score rows: block j holds keys 32j + 16(r/8) + 8h + r%8 of query qr0 + ln
        const int kend = CAUSAL ? min(Lk, qr0 + 32) : Lk;
        const int ns = (kend + 31) / 32;
        f32x16 s[kMaxSub];
#pragma unroll
        for (int j = 0; j < kMaxSub; ++j) {
            s[j] = f32x16{};
            if (j < ns) {
                u32x4 kf[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kf[ks] = sK[(32 * j + krow_sig) * KC + ((2 * ks + h) ^ kx)];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) s[j] = Mfma<T>::mma(kf[ks], qf[ks], s[j]);
                const int k0 = 32 * j;
                if (k0 + 32 > Lk || (CAUSAL && k0 + 31 > qr0)) {
                    const int qi = qr0 + ln;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int key = k0 + 16 * (r >> 3) + 8 * h + (r & 7);
                        const bool masked = key >= Lk || (CAUSAL && key > qi);
                        s[j][r] = masked ? -INFINITY : s[j][r];
                    }
                }
            }
        }
        // exact row max (every row has a visible key: key 0 is never masked)
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < kMaxSub; ++j)
            if (j < ns)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[j][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m = mx * c;

        // P = exp2(s c - m), packed RNE; l over the rounded P; O^T += V^T P^T
        f32x16 o[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db] = f32x16{};
        float lsum = 0.f;
#pragma unroll
        for (int j = 0; j < kMaxSub; ++j) {
            if (j < ns) {
                u32x4 pf[2];
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    float pv8[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) pv8[e] = __builtin_amdgcn_exp2f(fmaf(s[j][8 * cc + e], c, -m));
                    pf[cc] = u32x4{Mfma<T>::pack2(pv8[0], pv8[1]), Mfma<T>::pack2(pv8[2], pv8[3]),
                                   Mfma<T>::pack2(pv8[4], pv8[5]), Mfma<T>::pack2(pv8[6], pv8[7])};
#pragma unroll
                    for (int w = 0; w < 4; ++w) lsum = Mfma<T>::sum2(pf[cc][w], lsum);
                }
#pragma unroll
                for (int cc = 0; cc < 2; ++cc) {
                    const int kc = 2 * j + cc;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        u32x4 vf;
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            const int key = 16 * kc + 4 * t + tv_key;
                            const char* addr = reinterpret_cast<const char*>(sV + key * KC + ((4 * db + tv_chunk) ^ tv_swz)) + tv_within;
                            const i16x4_t part = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<char*>(addr)));
                            const u32x2 w2 = __builtin_bit_cast(u32x2, part);
                            vf[2 * t] = w2[0];
                            vf[2 * t + 1] = w2[1];
                        }
                        o[db] = Mfma<T>::mma(vf, pf[cc], o[db]);
                    }
                }
            }
        }

        // O = O^T / l through bounds-checked buffer stores (rows past Lq and columns past
        // head_dim are dropped by the hardware); optional natural-log LSE per row
        const float l = lsum + __shfl_xor(lsum, 32);
        const float inv = 1.f / l;
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            ob, (short)0, (int)((int64_t)Lq * o_rs), (int)kBufferFlags);
        const uint32_t rowoff = (uint32_t)(qr0 + ln) * o_rs;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int d0 = 32 * db + 8 * g4 + 4 * h;
                const u32x2 w = {Mfma<T>::pack2(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv),
                                 Mfma<T>::pack2(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv)};
                const uint32_t off = d0 < hd ? rowoff + (uint32_t)d0 * (uint32_t)sizeof(T) : kOobOffset;
                __builtin_amdgcn_raw_buffer_store_b64(w, ro, (int)off, 0, 0);
            }
        if (p.lse) {
            const int row = qr0 + ln;
            if (h == 0 && row < Lq)
                p.lse[((int64_t)b * p.heads_q + hq) * Lq + row] = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
        }
    }
#endif  // __HIP_DEVICE_COMPILE__
}

template <typename T, int D, int WAVES, bool CAUSAL>
hipError_t launch_short_cfg(const AttnProblem& p, hipStream_t stream) {
    const int n_rb = (p.seqlen_q + 31) / 32;
    const int nsub = (p.seqlen_k + 31) / 32;
    const size_t lds = (size_t)2 * nsub * 32 * D * sizeof(T);
    const int64_t units = (int64_t)p.batch * p.heads_kv;
    if (units > INT32_MAX) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((attn_fwd_short_kernel<T, D, WAVES, CAUSAL>), dim3((unsigned)units), dim3(WAVES * 64), lds,
                       stream, p, n_rb);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_short_d(const AttnProblem& p, hipStream_t stream) {
    const int items = p.group * ((p.seqlen_q + 31) / 32);
    if (items > 2) return p.causal ? launch_short_cfg<T, D, 4, true>(p, stream) : launch_short_cfg<T, D, 4, false>(p, stream);
    return p.causal ? launch_short_cfg<T, D, 2, true>(p, stream) : launch_short_cfg<T, D, 2, false>(p, stream);
}

template <typename T>
hipError_t launch_short_t(const AttnProblem& p, hipStream_t stream) {
    if (p.head_dim <= 64) return launch_short_d<T, 64>(p, stream);
    return launch_short_d<T, 128>(p, stream);
}

}  // namespace

bool short_supports(const AttnProblem& p, Dtype dt) {
    if (!(dt == Dtype::F16 || dt == Dtype::BF16) || p.cu_seqlens || p.mods) return false;
    if (p.head_dim > 128 || p.head_dim % 8 != 0) return false;
    if (p.seqlen_k < 1 || p.seqlen_k > kShortMaxKeys || p.seqlen_q < 1) return false;
    return (int64_t)p.group * ((p.seqlen_q + 31) / 32) <= kShortMaxItems;
}

hipError_t launch_attn_fwd_short(const AttnProblem& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::BF16) return launch_short_t<bf16_t>(p, stream);
    if (dt == Dtype::F16) return launch_short_t<f16_t>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace aule
