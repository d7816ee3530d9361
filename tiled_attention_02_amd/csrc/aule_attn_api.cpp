// C-ABI front end: argument validation, problem description, kernel selection.
//
// Every check happens on the host before any HIP call, so an invalid call returns its
// status without touching the device. Nothing here allocates or synchronises.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "aule_attn.h"
#include "attn_bwd.h"
#include "attn_decode.h"
#include "attn_problem.h"

namespace {

thread_local char g_last_error[512] = "";

aule_status_t fail(aule_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

size_t elem_size(aule_dtype_t dt) { return dt == AULE_DTYPE_F32 ? 4 : 2; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + nb && b0 < a0 + na;
}

aule_status_t check_common(int32_t head_dim, float scale, aule_dtype_t dtype) {
    if (dtype != AULE_DTYPE_F32 && dtype != AULE_DTYPE_F16 && dtype != AULE_DTYPE_BF16)
        return fail(AULE_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (head_dim <= 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "head_dim must be positive (got %d)", head_dim);
    if (head_dim > 128 || head_dim % 8 != 0)
        return fail(AULE_ERR_UNSUPPORTED, "head_dim must be a multiple of 8 and at most 128 (got %d)", head_dim);
    if (!std::isfinite(scale))
        return fail(AULE_ERR_INVALID_ARGUMENT, "scale must be finite");
    return AULE_OK;
}

// the backward on the matrix cores: fp16/bf16 kernels, and fp32 ones (the vector-ALU kernels
// take fp32 slices past the fp32 kernels' 32-bit offsets)
hipError_t launch_bwd(const aule::BwdProblem& p, aule_dtype_t dtype, hipStream_t stream) {
    const aule::Dtype dt = static_cast<aule::Dtype>(dtype);
    if (dt == aule::Dtype::F16 || dt == aule::Dtype::BF16) return aule::launch_attn_bwd_mfma(p, dt, stream);
    if (aule::bwd_f32_mfma_supports(p)) return aule::launch_attn_bwd_f32_mfma(p, stream);
    return aule::launch_attn_bwd(p, dt, stream);
}

// fp32 runs on the fp32 matrix-core kernel (the vector-ALU kernel takes score modifiers and
// slices past that kernel's 32-bit offsets); fp16/bf16 on the 16-bit matrix-core kernels: the
// short-sequence kernel for at most 128 keys, else the tiled kernel. A 16-bit problem that
// neither covers (a (sequence, head) slice of 1 GiB or more) is refused, never sent to
// another kernel.
aule_status_t dispatch(const aule::AttnProblem& p, aule_dtype_t dtype, hipStream_t stream) {
    aule::Dtype dt = static_cast<aule::Dtype>(dtype);
    hipError_t err;
    if (dt == aule::Dtype::F32)
        err = aule::f32_mfma_supports(p, dt) ? aule::launch_attn_fwd_f32_mfma(p, dt, stream)
                                             : aule::launch_attn_fwd_valu(p, dt, stream);
    else if (aule::short_supports(p, dt))
        err = aule::launch_attn_fwd_short(p, dt, stream);
    else if (aule::mfma_supports(p, dt))
        err = aule::launch_attn_fwd_mfma(p, dt, stream);
    else
        return fail(AULE_ERR_UNSUPPORTED, "fp16/bf16 slice too large for 32-bit offsets: one (%s, head) slice "
                    "must span less than 1 GiB", p.cu_seqlens ? "sequence" : "batch");
    if (err != hipSuccess)
        return fail(AULE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    g_last_error[0] = '\0';
    return AULE_OK;
}

const float kLog2e = 1.4426950408889634f;

// Split plan of the decoding path: how many key-range splits and how many keys each.
struct SplitPlan {
    int32_t splits;
    int32_t keys_per_split;
    size_t ml_bytes;   // workspace offset of the partial outputs (256-byte aligned)
    size_t bytes;      // total workspace
};

constexpr int64_t kSplitTargetWorkgroups = 1024;   // vector-ALU kernel: about four per CU on 256 CUs

// The matrix-core partial kernel holds one workgroup per CU (128 KiB of LDS at head_dim
// 128): one workgroup per CU, so that every split runs in the first and only round.
int64_t resident_cus() {
    static const int64_t n = [] {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess) return 256;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
        return cus;
    }();
    return n;
}

aule_status_t check_splitkv(int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t seqlen_q,
                            int32_t seqlen_k, int32_t head_dim, int32_t causal, aule_dtype_t dtype,
                            int32_t num_splits) {
    if (batch < 0 || seqlen_q < 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "batch and seqlen_q must be >= 0");
    if (num_splits < 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "num_splits must be >= 0 (got %d)", num_splits);
    if (aule_status_t st = check_common(head_dim, 1.f, dtype)) return st;
    if (heads_q <= 0 || heads_kv <= 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "heads_q and heads_kv must be positive");
    if (heads_q % heads_kv != 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "heads_q (%d) must be a multiple of heads_kv (%d)", heads_q, heads_kv);
    if (batch == 0 || seqlen_q == 0) return AULE_OK;
    if (seqlen_k <= 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "seqlen_k must be positive for a non-empty problem");
    if (causal && seqlen_q > seqlen_k)
        return fail(AULE_ERR_UNSUPPORTED, "causal decoding needs seqlen_q <= seqlen_k (got %d, %d)", seqlen_q, seqlen_k);
    if ((int64_t)(heads_q / heads_kv) * seqlen_q > 64)
        return fail(AULE_ERR_UNSUPPORTED, "at most 64 query rows per kv head (got %d); use aule_attn_fwd",
                    (heads_q / heads_kv) * seqlen_q);
    if ((int64_t)batch * heads_q * seqlen_q > INT32_MAX)
        return fail(AULE_ERR_INVALID_ARGUMENT, "too many output rows");
    if (dtype != AULE_DTYPE_F32 && (int64_t)seqlen_k * head_dim * 2 >= ((int64_t)1 << 30))
        return fail(AULE_ERR_UNSUPPORTED, "fp16/bf16 slice too large for 32-bit offsets: one (batch, kv head) "
                    "cache slice must span less than 1 GiB");
    if (batch > 65535 || heads_kv > 65535)   // grid z and y dimensions
        return fail(AULE_ERR_UNSUPPORTED, "batch and heads_kv must be at most 65535 for split-KV decoding");
    return AULE_OK;
}

SplitPlan plan_splits(int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t seqlen_q,
                      int32_t seqlen_k, int32_t head_dim, aule_dtype_t dtype, int32_t num_splits) {
    const aule::Dtype dt = static_cast<aule::Dtype>(dtype);
    const bool mfma = heads_kv > 0 && aule::decode_mfma_eligible(dt, heads_q / heads_kv * seqlen_q, head_dim);
    const int64_t tk = mfma ? aule::decode_mfma_keys_granule() : aule::decode_keys_per_tile(dt);
    const int64_t tiles = (seqlen_k + tk - 1) / tk;
    const int64_t groups = (int64_t)batch * heads_kv;
    const int64_t target = mfma ? resident_cus() : kSplitTargetWorkgroups;
    int64_t s = num_splits > 0 ? num_splits : (target + groups - 1) / groups;
    s = s < 1 ? 1 : (s > tiles ? tiles : s);
    const int64_t kps = (tiles + s - 1) / s * tk;           // whole tiles per split
    s = (seqlen_k + kps - 1) / kps;                         // no empty split
    const int64_t rows = (int64_t)batch * heads_q * seqlen_q;
    SplitPlan pl;
    pl.splits = (int32_t)s;
    pl.keys_per_split = (int32_t)kps;
    pl.ml_bytes = ((size_t)(s * rows * 2 * sizeof(float)) + 255) / 256 * 256;
    pl.bytes = pl.ml_bytes + (size_t)(s * rows * head_dim) * sizeof(float);
    return pl;
}

}  // namespace

namespace {

// The dense checks shared by the forward entry points and the backward.
aule_status_t check_dense(const void* q, const void* k, const void* v, const void* o,
                          int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t seqlen_q,
                          int32_t seqlen_k, int32_t head_dim, int32_t causal, float scale,
                          aule_dtype_t dtype, bool* empty) {
    *empty = false;
    if (batch < 0 || seqlen_q < 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "batch and seqlen_q must be >= 0");
    if (aule_status_t st = check_common(head_dim, scale, dtype)) return st;
    if (heads_q <= 0 || heads_kv <= 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "heads_q and heads_kv must be positive");
    if (heads_q % heads_kv != 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "heads_q (%d) must be a multiple of heads_kv (%d)", heads_q, heads_kv);
    if (causal && seqlen_q != seqlen_k)
        return fail(AULE_ERR_UNSUPPORTED, "causal attention needs seqlen_q == seqlen_k (got %d, %d)", seqlen_q, seqlen_k);
    if (batch == 0 || seqlen_q == 0) {
        *empty = true;
        return AULE_OK;
    }
    if (seqlen_k <= 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "seqlen_k must be positive for a non-empty problem");
    if (!q || !k || !v || !o)
        return fail(AULE_ERR_INVALID_ARGUMENT, "null tensor pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(AULE_ERR_INVALID_ARGUMENT, "tensor pointers must be 16-byte aligned");
    return AULE_OK;
}

aule_status_t fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                       int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t seqlen_q,
                       int32_t seqlen_k, int32_t head_dim, int32_t causal, float scale,
                       aule_dtype_t dtype, hipStream_t stream) {
    bool empty;
    if (aule_status_t st = check_dense(q, k, v, o, batch, heads_q, heads_kv, seqlen_q, seqlen_k,
                                       head_dim, causal, scale, dtype, &empty))
        return st;
    if (empty) {
        g_last_error[0] = '\0';
        return AULE_OK;  // empty problem
    }
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)batch * heads_q * seqlen_q * head_dim * es;
    const size_t nkv = (size_t)batch * heads_kv * seqlen_k * head_dim * es;
    if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv))
        return fail(AULE_ERR_INVALID_ARGUMENT, "output overlaps an input");
    if (lse) {
        const size_t nl = (size_t)batch * heads_q * seqlen_q * sizeof(float);
        if (reinterpret_cast<uintptr_t>(lse) & 3u)
            return fail(AULE_ERR_INVALID_ARGUMENT, "lse must be 4-byte aligned");
        if (overlaps(lse, nl, q, nq) || overlaps(lse, nl, k, nkv) || overlaps(lse, nl, v, nkv) ||
            overlaps(lse, nl, o, nq))
            return fail(AULE_ERR_INVALID_ARGUMENT, "lse overlaps a tensor");
    }

    aule::AttnProblem p{};
    p.q = q; p.k = k; p.v = v; p.o = o;
    p.q_rstride = head_dim; p.q_hstride = (int64_t)seqlen_q * head_dim; p.q_bstride = p.q_hstride * heads_q;
    p.k_rstride = head_dim; p.k_hstride = (int64_t)seqlen_k * head_dim; p.k_bstride = p.k_hstride * heads_kv;
    p.v_rstride = p.k_rstride; p.v_hstride = p.k_hstride; p.v_bstride = p.k_bstride;
    p.o_rstride = p.q_rstride; p.o_hstride = p.q_hstride; p.o_bstride = p.q_bstride;
    p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.group = heads_q / heads_kv;
    p.seqlen_q = seqlen_q; p.seqlen_k = seqlen_k; p.head_dim = head_dim;
    p.causal = causal ? 1 : 0;
    p.scale_log2 = scale * kLog2e;
    p.cu_seqlens = nullptr;
    p.total_tokens = 0;
    p.max_seqlen = seqlen_q;
    p.lse = lse;
    return dispatch(p, dtype, stream);
}

}  // namespace

namespace {

struct VarlenMods {
    int32_t win_left = -1, win_right = -1;
    float softcap = 0.f;
    const float* alibi = nullptr;
    int32_t alibi_sstride = 0;
};

aule_status_t varlen_impl(const void* qkv, const int32_t* cu_seqlens, void* o, int32_t num_seqs,
                          int32_t total_tokens, int32_t max_seqlen, int32_t heads,
                          int32_t head_dim, int32_t causal, float scale, aule_dtype_t dtype,
                          const VarlenMods& mods, hipStream_t stream) {
    if (total_tokens < 0 || max_seqlen < 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "total_tokens and max_seqlen must be >= 0");
    if (total_tokens > 0 && max_seqlen == 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "max_seqlen must be at least the longest sequence (got 0)");
    if (num_seqs <= 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "num_seqs must be positive (got %d)", num_seqs);
    if (heads <= 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "heads must be positive");
    if (aule_status_t st = check_common(head_dim, scale, dtype)) return st;
    if (total_tokens == 0) {
        g_last_error[0] = '\0';
        return AULE_OK;  // every sequence is empty
    }
    if (!qkv || !cu_seqlens || !o)
        return fail(AULE_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(qkv) || !aligned16(o) || (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u))
        return fail(AULE_ERR_INVALID_ARGUMENT, "qkv/o must be 16-byte aligned, cu_seqlens 4-byte aligned");
    const size_t es = elem_size(dtype);
    const size_t nqkv = (size_t)total_tokens * 3 * heads * head_dim * es;
    const size_t no = (size_t)total_tokens * heads * head_dim * es;
    if (overlaps(o, no, qkv, nqkv) || overlaps(o, no, cu_seqlens, (size_t)(num_seqs + 1) * 4))
        return fail(AULE_ERR_INVALID_ARGUMENT, "output overlaps an input");
    if ((int64_t)total_tokens + num_seqs > INT32_MAX)
        return fail(AULE_ERR_INVALID_ARGUMENT, "too many tokens");

    const int64_t hd = (int64_t)heads * head_dim;
    const char* base = static_cast<const char*>(qkv);
    aule::AttnProblem p{};
    p.q = base;
    p.k = base + hd * es;
    p.v = base + 2 * hd * es;
    p.o = o;
    p.q_rstride = p.k_rstride = p.v_rstride = 3 * hd;
    p.q_hstride = p.k_hstride = p.v_hstride = head_dim;
    p.q_bstride = p.k_bstride = p.v_bstride = 0;
    p.o_rstride = hd; p.o_hstride = head_dim; p.o_bstride = 0;
    p.batch = num_seqs; p.heads_q = heads; p.heads_kv = heads; p.group = 1;
    p.seqlen_q = max_seqlen; p.seqlen_k = max_seqlen; p.head_dim = head_dim;
    p.causal = causal ? 1 : 0;
    p.scale_log2 = scale * kLog2e;
    p.cu_seqlens = cu_seqlens;
    p.total_tokens = total_tokens;
    p.max_seqlen = max_seqlen;
    // causal already hides every key after the query: only a left edge remains. A window
    // of max_seqlen keys or more masks nothing (no sequence is longer; the kernels clamp
    // every sequence to max_seqlen), so it is unbounded: mapping it to -1 also keeps the
    // kernels' row + window sums far from int32 overflow.
    const int32_t wl = mods.win_left >= max_seqlen ? -1 : mods.win_left;
    const int32_t wr = (causal || mods.win_right >= max_seqlen) ? -1 : mods.win_right;
    p.mods = (wl >= 0 || wr >= 0 || mods.softcap > 0.f || mods.alibi) ? 1 : 0;
    p.win_left = wl;
    p.win_right = wr;
    p.softcap = mods.softcap;
    p.alibi = mods.alibi;
    p.alibi_sstride = mods.alibi_sstride;
    if (p.alibi) {
        const size_t na = ((size_t)(num_seqs - 1) * mods.alibi_sstride + heads) * sizeof(float);
        if (overlaps(o, no, p.alibi, na))
            return fail(AULE_ERR_INVALID_ARGUMENT, "output overlaps alibi_slopes");
    }
    return dispatch(p, dtype, stream);
}

}  // namespace

extern "C" {

aule_status_t aule_attn_fwd(const void* q, const void* k, const void* v, void* o,
                            int32_t batch, int32_t heads_q, int32_t heads_kv,
                            int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                            int32_t causal, float scale, aule_dtype_t dtype,
                            hipStream_t stream) {
    return fwd_impl(q, k, v, o, nullptr, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim,
                    causal, scale, dtype, stream);
}

aule_status_t aule_attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                                int32_t batch, int32_t heads_q, int32_t heads_kv,
                                int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                int32_t causal, float scale, aule_dtype_t dtype,
                                hipStream_t stream) {
    if (!lse && batch > 0 && seqlen_q > 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "null lse pointer");
    return fwd_impl(q, k, v, o, lse, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim,
                    causal, scale, dtype, stream);
}

aule_status_t aule_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            int32_t batch, int32_t heads_q, int32_t heads_kv,
                            int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                            int32_t causal, float scale, aule_dtype_t dtype,
                            hipStream_t stream) {
    bool empty;
    if (aule_status_t st = check_dense(q, k, v, o, batch, heads_q, heads_kv, seqlen_q, seqlen_k,
                                       head_dim, causal, scale, dtype, &empty))
        return st;
    // With no query rows but keys present, dK and dV are all zero and still written.
    const bool zero_kv_only = empty && batch > 0 && seqlen_q == 0 && seqlen_k > 0;
    if (empty && !zero_kv_only) {
        g_last_error[0] = '\0';
        return AULE_OK;
    }
    if (zero_kv_only) {
        if (!dk || !dv)
            return fail(AULE_ERR_INVALID_ARGUMENT, "null pointer");
        if (!aligned16(dk) || !aligned16(dv))
            return fail(AULE_ERR_INVALID_ARGUMENT, "misaligned pointer");
        const size_t nkv = (size_t)batch * heads_kv * seqlen_k * head_dim * elem_size(dtype);
        if (overlaps(dk, nkv, dv, nkv))
            return fail(AULE_ERR_INVALID_ARGUMENT, "gradient buffers overlap");
        if (batch > 65535)
            return fail(AULE_ERR_UNSUPPORTED, "batch must be at most 65535 for the backward");
        aule::BwdProblem p{};
        p.dk = dk; p.dv = dv;
        p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.group = heads_q / heads_kv;
        p.seqlen_q = 0; p.seqlen_k = seqlen_k; p.head_dim = head_dim;
        p.scale = scale;
        const hipError_t err = launch_bwd(p, dtype, stream);
        if (err != hipSuccess)
            return fail(AULE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
        g_last_error[0] = '\0';
        return AULE_OK;
    }
    if (!dout || !lse || !dq || !dk || !dv)
        return fail(AULE_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(AULE_ERR_INVALID_ARGUMENT, "misaligned pointer");
    if (batch > 65535 || heads_q > 65535)   // grid z and y dimensions
        return fail(AULE_ERR_UNSUPPORTED, "batch and heads_q must be at most 65535 for the backward");
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)batch * heads_q * seqlen_q * head_dim * es;
    const size_t nkv = (size_t)batch * heads_kv * seqlen_k * head_dim * es;
    const size_t nl = (size_t)batch * heads_q * seqlen_q * sizeof(float);
    const void* ins[] = {q, k, v, o, dout, lse};
    const size_t nin[] = {nq, nkv, nkv, nq, nq, nl};
    void* outs[] = {dq, dk, dv};
    const size_t nout[] = {nq, nkv, nkv};
    for (int a = 0; a < 3; ++a) {
        for (int b2 = 0; b2 < 6; ++b2)
            if (overlaps(outs[a], nout[a], ins[b2], nin[b2]))
                return fail(AULE_ERR_INVALID_ARGUMENT, "a gradient buffer overlaps an input");
        for (int b2 = a + 1; b2 < 3; ++b2)
            if (overlaps(outs[a], nout[a], outs[b2], nout[b2]))
                return fail(AULE_ERR_INVALID_ARGUMENT, "gradient buffers overlap");
    }
    // the matrix-core kernels address one (batch, head) slice with 32-bit buffer offsets
    const aule::Dtype dt16 = static_cast<aule::Dtype>(dtype);
    if ((dt16 == aule::Dtype::F16 || dt16 == aule::Dtype::BF16) &&
        (size_t)(seqlen_q > seqlen_k ? seqlen_q : seqlen_k) * head_dim * es >= ((size_t)1 << 30))
        return fail(AULE_ERR_UNSUPPORTED, "fp16/bf16 slice too large for 32-bit offsets: one (batch, head) slice "
                    "must span less than 1 GiB");
    aule::BwdProblem p{};
    p.q = q; p.k = k; p.v = v; p.o = o; p.do_ = dout; p.lse = lse;
    p.dq = dq; p.dk = dk; p.dv = dv;
    p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.group = heads_q / heads_kv;
    p.seqlen_q = seqlen_q; p.seqlen_k = seqlen_k; p.head_dim = head_dim;
    p.causal = causal ? 1 : 0;
    p.scale = scale;
    const hipError_t err = launch_bwd(p, dtype, stream);
    if (err != hipSuccess)
        return fail(AULE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    g_last_error[0] = '\0';
    return AULE_OK;
}

aule_status_t aule_attn_fwd_varlen(const void* qkv, const int32_t* cu_seqlens, void* o,
                                   int32_t num_seqs, int32_t total_tokens,
                                   int32_t max_seqlen, int32_t heads, int32_t head_dim,
                                   int32_t causal, float scale, aule_dtype_t dtype,
                                   hipStream_t stream) {
    return varlen_impl(qkv, cu_seqlens, o, num_seqs, total_tokens, max_seqlen, heads, head_dim,
                       causal, scale, dtype, VarlenMods{}, stream);
}

aule_status_t aule_attn_fwd_varlen_mods(const void* qkv, const int32_t* cu_seqlens, void* o,
                                        int32_t num_seqs, int32_t total_tokens,
                                        int32_t max_seqlen, int32_t heads, int32_t head_dim,
                                        int32_t causal, float scale, int32_t window_left,
                                        int32_t window_right, float softcap,
                                        const float* alibi_slopes, int32_t alibi_batch_stride,
                                        aule_dtype_t dtype, hipStream_t stream) {
    if (window_left < -1 || window_right < -1)
        return fail(AULE_ERR_INVALID_ARGUMENT, "window sizes must be >= -1 (got %d, %d)", window_left, window_right);
    if (causal && window_right > 0)
        return fail(AULE_ERR_INVALID_ARGUMENT, "causal attention takes window_right -1 or 0 (got %d)", window_right);
    if (!std::isfinite(softcap) || softcap < 0.f)
        return fail(AULE_ERR_INVALID_ARGUMENT, "softcap must be finite and >= 0");
    if (alibi_slopes) {
        if (reinterpret_cast<uintptr_t>(alibi_slopes) & 3u)
            return fail(AULE_ERR_INVALID_ARGUMENT, "alibi_slopes must be 4-byte aligned");
        if (alibi_batch_stride != 0 && alibi_batch_stride != heads)
            return fail(AULE_ERR_INVALID_ARGUMENT, "alibi_batch_stride must be 0 ([heads]) or heads ([batch, heads])");
    }
    VarlenMods m;
    m.win_left = window_left;
    m.win_right = window_right;
    m.softcap = softcap;
    m.alibi = alibi_slopes;
    m.alibi_sstride = alibi_slopes ? alibi_batch_stride : 0;
    return varlen_impl(qkv, cu_seqlens, o, num_seqs, total_tokens, max_seqlen, heads, head_dim,
                       causal, scale, dtype, m, stream);
}

}  // extern "C"

namespace {

// Shared by both split-KV entry points: validate, plan the splits, place the partials in
// `workspace` (the caller's buffer, or the library's device array when `own` is set), launch.
aule_status_t splitkv_impl(const void* q, const void* k, const void* v, void* o, int32_t batch,
                           int32_t heads_q, int32_t heads_kv, int32_t seqlen_q, int32_t seqlen_k,
                           int32_t head_dim, int32_t causal, float scale, aule_dtype_t dtype,
                           int32_t num_splits, void* workspace, size_t workspace_bytes, bool own,
                           hipStream_t stream) {
    if (aule_status_t st = check_splitkv(batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim,
                                         causal, dtype, num_splits))
        return st;
    if (!std::isfinite(scale))
        return fail(AULE_ERR_INVALID_ARGUMENT, "scale must be finite");
    if (batch == 0 || seqlen_q == 0) {
        g_last_error[0] = '\0';
        return AULE_OK;  // empty problem
    }
    if (!q || !k || !v || !o || (!own && !workspace))
        return fail(AULE_ERR_INVALID_ARGUMENT, "null pointer");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || (!own && !aligned16(workspace)))
        return fail(AULE_ERR_INVALID_ARGUMENT, "tensor and workspace pointers must be 16-byte aligned");
    const SplitPlan pl = plan_splits(batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, dtype, num_splits);
    if (own && pl.bytes > aule::decode_scratch_bytes())
        return fail(AULE_ERR_UNSUPPORTED, "the split partials need %zu bytes; the library's device array "
                    "holds %zu (use aule_attn_fwd_splitkv with a workspace, or fewer splits)",
                    pl.bytes, aule::decode_scratch_bytes());
    if (!own && workspace_bytes < pl.bytes)
        return fail(AULE_ERR_INVALID_ARGUMENT, "workspace of %zu bytes is smaller than the %zu needed",
                    workspace_bytes, pl.bytes);
    const size_t es = elem_size(dtype);
    const size_t nq = (size_t)batch * heads_q * seqlen_q * head_dim * es;
    const size_t nkv = (size_t)batch * heads_kv * seqlen_k * head_dim * es;
    if (overlaps(o, nq, q, nq) || overlaps(o, nq, k, nkv) || overlaps(o, nq, v, nkv))
        return fail(AULE_ERR_INVALID_ARGUMENT, "output overlaps an input");
    if (!own && (overlaps(workspace, pl.bytes, q, nq) || overlaps(workspace, pl.bytes, k, nkv) ||
                 overlaps(workspace, pl.bytes, v, nkv) || overlaps(workspace, pl.bytes, o, nq)))
        return fail(AULE_ERR_INVALID_ARGUMENT, "workspace overlaps a tensor");
    if (own) {
        const hipError_t e = aule::decode_scratch(&workspace);
        if (e != hipSuccess)
            return fail(AULE_ERR_HIP, "device workspace lookup failed: %s", hipGetErrorString(e));
    }

    aule::DecodeProblem p{};
    p.q = q; p.k = k; p.v = v; p.o = o;
    p.batch = batch; p.heads_q = heads_q; p.heads_kv = heads_kv; p.group = heads_q / heads_kv;
    p.seqlen_q = seqlen_q; p.seqlen_k = seqlen_k; p.head_dim = head_dim;
    p.causal = causal ? 1 : 0;
    p.scale = scale;
    p.num_splits = pl.splits;
    p.keys_per_split = pl.keys_per_split;
    p.ws_ml = static_cast<float*>(workspace);
    p.ws_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ml_bytes);
    const hipError_t err = aule::launch_attn_decode(p, static_cast<aule::Dtype>(dtype), stream);
    if (err != hipSuccess)
        return fail(AULE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(err));
    g_last_error[0] = '\0';
    return AULE_OK;
}

}  // namespace

extern "C" {

aule_status_t aule_attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o,
                                    int32_t batch, int32_t heads_q, int32_t heads_kv,
                                    int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                    int32_t causal, float scale, aule_dtype_t dtype,
                                    int32_t num_splits, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
    return splitkv_impl(q, k, v, o, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, causal,
                        scale, dtype, num_splits, workspace, workspace_bytes, false, stream);
}

aule_status_t aule_attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                            int32_t batch, int32_t heads_q, int32_t heads_kv,
                                            int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                            int32_t causal, float scale, aule_dtype_t dtype,
                                            int32_t num_splits, hipStream_t stream) {
    return splitkv_impl(q, k, v, o, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, causal,
                        scale, dtype, num_splits, nullptr, 0, true, stream);
}

size_t aule_attn_splitkv_workspace_size(int32_t batch, int32_t heads_q, int32_t heads_kv,
                                        int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                                        aule_dtype_t dtype, int32_t num_splits) {
    if (check_splitkv(batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, 0, dtype, num_splits) != AULE_OK)
        return 0;
    if (batch == 0 || seqlen_q == 0) return 0;
    return plan_splits(batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, dtype, num_splits).bytes;
}

const char* aule_status_string(aule_status_t status) {
    switch (status) {
        case AULE_OK: return "AULE_OK";
        case AULE_ERR_INVALID_ARGUMENT: return "AULE_ERR_INVALID_ARGUMENT";
        case AULE_ERR_UNSUPPORTED: return "AULE_ERR_UNSUPPORTED";
        case AULE_ERR_HIP: return "AULE_ERR_HIP";
    }
    return "AULE_STATUS_UNKNOWN";
}

const char* aule_last_error(void) { return g_last_error; }

}  // extern "C"
