// Matrix-core (MFMA) attention forward for fp16/bf16 on gfx950 (CDNA4).
//
// The FlashAttention block loop (xxqk.cn article "Attention算子实战：从CUDA优化到昇腾/CANN部署",
// section 2.2: Q tile on chip, K/V tiles streamed, numerically stable softmax kept in
// registers, partial P·V accumulated, only O written) with fp16/bf16 matrix products and
// fp32 softmax statistics (FlashAttention-T commentary, ai-stack.site, best practices 4-5),
// laid out for 64-wide wavefronts and v_mfma_f32_32x32x16_{bf16,f16}.
//
// Work split
//   Two kernel forms, chosen by shape (launch_gh):
//   * dense problems at head_dim 128: workgroup = 8 waves (two per SIMD, so one wave's
//     softmax can run under the other's matrix products); wave = 32 query rows of one query
//     head; GH query heads that share one K/V head run in the same workgroup (GQA) and the
//     other 8/GH waves take further 32-row blocks, so one K/V tile in LDS serves 256 query
//     rows. K/V tiles of 128 keys, double-buffered; persistent workgroups (one per CU), each
//     walking several work items.
//   * varlen problems and head_dim <= 64: workgroup = 4 waves over 128 query rows, K/V tiles
//     of 64 keys, double-buffered, two workgroups per CU, one workgroup per work item.
//   K/V tiles are copied global -> LDS with buffer_load_dwordx4 ... lds (no register
//   staging): each wave instruction fills 1 KiB of LDS contiguously, and every lane picks
//   the global 16-byte chunk that belongs at its LDS slot, so the LDS image is XOR-swizzled
//   against bank conflicts while the global reads stay whole rows. The buffer descriptor's
//   size check turns rows past the sequence end and columns past head_dim into zeros.
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

#include <type_traits>

#include "attn_device.h"
#include "attn_mfma.h"

namespace aule {
namespace {

[[maybe_unused]] constexpr float kRescaleSlack = 8.0f; // log2 units
[[maybe_unused]] constexpr float kSlackExp = 256.0f;   // 2^kRescaleSlack
[[maybe_unused]] constexpr int kCopyParts = 4;          // pieces of one K/V tile copy

#if defined(__HIP_DEVICE_COMPILE__)
// Start the global -> LDS copy of one K/V tile: NI 16-byte loads per lane for each of K and
// V; wave w fills LDS chunk slots [(w*NI + i) * 64, +64) of the tile buffers.
template <int NI>
__device__ __forceinline__ void issue_tile(i32x4 rk, i32x4 rv, const uint32_t (&koff)[NI],
                                           const uint32_t (&voff)[NI], uint32_t tile_k_bytes,
                                           uint32_t tile_v_bytes, uint32_t dK, uint32_t dV, int wave) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
        const uint32_t slot = (uint32_t)(wave * NI + i) * 64u * 16u;   // bytes
        lds_copy16(rk, koff[i] + tile_k_bytes, __builtin_amdgcn_readfirstlane(dK + slot));
        lds_copy16(rv, voff[i] + tile_v_bytes, __builtin_amdgcn_readfirstlane(dV + slot));
    }
}
// Part `part` of `parts` of the same copy: instructions [part * 2NI / parts, ...) of the
// 2NI (K first, then V). Spreading a tile's copy over several calls keeps a wave from
// stalling on a long run of copy instructions, which issue in order behind every other
// wave's copies.
template <int NI, int PARTS>
__device__ __forceinline__ void issue_tile_part(int part, i32x4 rk, i32x4 rv, const uint32_t (&koff)[NI],
                                                const uint32_t (&voff)[NI], uint32_t tile_k_bytes,
                                                uint32_t tile_v_bytes, uint32_t dK, uint32_t dV, int wave) {
    constexpr int PER = 2 * NI / PARTS;
    static_assert(PER * PARTS == 2 * NI, "copy parts must split the tile evenly");
#pragma unroll
    for (int j = 0; j < 2 * NI; ++j) {
        if (j / PER != part) continue;
        const int i = j % NI;
        const uint32_t slot = (uint32_t)(wave * NI + i) * 64u * 16u;   // bytes
        if (j < NI) lds_copy16(rk, koff[i] + tile_k_bytes, __builtin_amdgcn_readfirstlane(dK + slot));
        else lds_copy16(rv, voff[i] + tile_v_bytes, __builtin_amdgcn_readfirstlane(dV + slot));
    }
}
#endif  // __HIP_DEVICE_COMPILE__

// WAVES waves per workgroup (4: one per SIMD, 8: two per SIMD so one wave's softmax runs
// while the other's matrix products do); each wave owns NB blocks of 32 query rows of one
// query head.
// Wait until at most N of this wave's vector-memory operations are outstanding and for its
// LDS reads, then join the workgroup barrier.
// The wait is issued through the builtin so that the compiler's own wait-count tracking
// knows every LDS read has completed here (it cannot see waits inside inline asm and would
// otherwise keep inserting conservative waits for reads that have long finished); the
// barrier itself stays an asm statement with a memory clobber, which also keeps the
// compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
    static_assert(N >= 0 && N <= 63, "vmcnt field is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));   // vmcnt(N) lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}
// LDS reads done, then the workgroup barrier
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    asm volatile("s_barrier" ::: "memory");
}

// Parity of the LDS buffer that holds a work item's first K/V tile (persistent form), as a
// type so that every buffer index stays a compile-time constant.
template <int P> struct Parity { static constexpr int value = P; };

// TB: keys per K/V tile, double-buffered in LDS (the copy of tile t+1 runs during tile t).
// PERSIST (dense problems): the grid holds one workgroup per CU and each walks
// several work items, issuing the next item's first K/V tile copy and its Q loads while it
// finishes the current item, so that their latency and the workgroup launch gap are hidden.
template <typename T, int D, int WAVES, int NB, int GH, int TB, bool PERSIST, bool CAUSAL, bool VARLEN,
          bool MODS>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_fwd_mfma_kernel(AttnProblem p, int n_qtiles) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int kThreads = WAVES * 64;
    constexpr int kRowsPerWave = 32 * NB;
    constexpr int RB = WAVES / GH;               // row blocks per workgroup
    constexpr int BMW = kRowsPerWave * RB;       // query rows per workgroup
    constexpr int KC = D / 8;                    // 16-byte chunks per K / V row
    constexpr int KS = D / 16;                   // k-steps of S^T = K Q^T
    constexpr int DB = D / 32;                   // 32-row d-blocks of O^T
    constexpr int kBN = TB;                      // keys per K/V tile
    constexpr int SPT = TB / 32;                 // 32-key sub-steps per tile
    constexpr int NBUF = 2;                      // LDS tile buffers (double buffering)
    constexpr int AHEAD = 1;                     // tiles requested ahead
    constexpr int DMA_PARTS = kCopyParts < SPT ? kCopyParts : SPT;   // pieces of a tile copy
    constexpr int NSTORE = NB * (DB / 2) * 4;    // O store instructions per wave and item (slab path)
    static_assert(TB == 64 || TB == 128, "tile of 64 or 128 keys");
    static_assert(!PERSIST || !VARLEN, "persistent form: dense problems");
    constexpr int TILE_CHUNKS = kBN * KC;        // 16-byte chunks per K (or V) tile
    constexpr int NI = TILE_CHUNKS / kThreads;   // load instructions per wave per tile
    static_assert(NI >= 1 && TILE_CHUNKS % kThreads == 0, "tile must split evenly over the waves");

    __shared__ u32x4 sK[NBUF][TILE_CHUNKS];
    __shared__ u32x4 sV[NBUF][TILE_CHUNKS];
    // persistent form: a private 4 KiB slab per wave (32 rows x 128 bytes) through which O
    // is written out in whole row segments (the LDS left over next to the K/V buffers)
    constexpr int kSlab = PERSIST ? 256 : 1;
    __shared__ u32x4 sO[PERSIST ? WAVES : 1][kSlab];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform (an SGPR): everything derived from it (rows, heads, mask and barrier
    // conditions) stays scalar, so those branches are scalar branches
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = lane >> 5;
    const int ln = lane & 31;
    const int hd = p.head_dim;

    // ---------------------------------------------------------------- K/V copy set-up
    const uint32_t k_rs = (uint32_t)(p.k_rstride * (int64_t)sizeof(T));   // row strides, bytes
    const uint32_t v_rs = (uint32_t)(p.v_rstride * (int64_t)sizeof(T));
    const uint32_t o_rs = (uint32_t)(p.o_rstride * (int64_t)sizeof(T));
    const uint32_t q_rs = (uint32_t)(p.q_rstride * (int64_t)sizeof(T));
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

    // ---------------------------------------------------------------- work items
    // A work item is one q-tile of BMW rows of GH query heads that share one kv head (dense),
    // or of one head of one sequence (varlen).
    struct Item {
        int Lq, Lk, qr0, nsub, n_kt;   // lengths, first row of this wave, sub-steps, K/V tiles
        const T* qb;                   // this wave's Q slice and O slice
        T* ob;
        float* lseb;                   // this wave's log-sum-exp row (dense, optional)
        i32x4 rk, rv;                  // K / V slice descriptors, exactly the Lk valid rows
        int kb0;                       // first key walked (score modifiers: window start)
        float slope;                   // ALiBi slope of this wave's head (score modifiers)
    };
    const int ngroups = p.heads_q / GH;
    const int NG = p.batch * ngroups;
    // Varlen grid (virtual tile, head group): workgroups go to the 8 XCDs round-robin in
    // dispatch order (x fastest), so neighbouring tiles of one (sequence, head) would land
    // on different XCDs and each XCD's L2 would fetch that K/V again. When the head-group
    // count divides by 8 the linear block id is remapped (a bijection) so that every tile of
    // a head group runs on one XCD: XCD = group % 8, tiles in order within it.
    int vx = blockIdx.x, vy = blockIdx.y;
    if constexpr (VARLEN) {
        if ((gridDim.y & 7) == 0) {
            const int lin = blockIdx.x + gridDim.x * blockIdx.y;
            const int xcd = lin & 7, slot = lin >> 3, per = gridDim.y >> 3;
            vx = slot / per;
            vy = xcd + 8 * (slot - vx * per);
        }
    }
    auto make_item = [&](int x, Item& it) -> bool {
        int bidx, hq0, tile, Lq, Lk;
        int64_t tok0 = 0;
        if constexpr (VARLEN) {
            TileSlot s = locate_varlen_tile(p.cu_seqlens, p.batch, p.total_tokens, p.max_seqlen, BMW, x, CAUSAL);
            if (!s.valid) return false;
            bidx = s.seq; tok0 = s.tok0; tile = s.tile; Lq = s.len_q; Lk = s.len_k;
            hq0 = vy * GH;
        } else {
            // groups = (batch, GH query heads sharing one kv head). Item x runs on XCD x % 8
            // (workgroup x does, and a persistent workgroup only takes items of its own XCD);
            // when the groups split evenly, each XCD gets whole groups so that their K/V stay
            // in that XCD's L2. The longest causal tiles come first (within each group of an
            // XCD, or over the whole grid).
            if (x >= n_qtiles * NG) return false;
            int t, g;
            if (NG % 8 == 0) {
                // persistent: group-major within an XCD, all q-tiles of one group (longest
                // first), then the next group, so one group's K/V is live in the XCD's L2 at
                // a time (the snake order of the persistent workgroups keeps each one's
                // causal work equal over every two rounds of a group)
                const int per = NG / 8, xcd = x & 7, l = x >> 3;
                if constexpr (PERSIST) {
                    const int gl = l / n_qtiles;
                    t = l - gl * n_qtiles;
                    g = xcd * per + gl;
                } else {
                    // one workgroup per item, all resident at once when they fit: tile-rank
                    // major, the first half of the ranks longest first and the second half
                    // shortest first, so that the workgroups sharing a CU pair long with
                    // short tiles (group-major here put two longest tiles on one CU: -12%
                    // on the fp16 head_dim-64 causal workload; this order +5% over plain
                    // rank-major)
                    t = l / per;
                    g = xcd * per + (l - t * per);
                    const int half = (n_qtiles + 1) / 2;
                    if (t >= half) t = n_qtiles - 1 - (t - half);
                }
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
        it.Lq = Lq;
        it.Lk = Lk;
        it.qr0 = tile * BMW + kRowsPerWave * (wave / GH);
        it.qb = static_cast<const T*>(p.q) + (VARLEN ? tok0 * p.q_rstride : bidx * p.q_bstride) + hq * p.q_hstride;
        it.ob = static_cast<T*>(p.o) + (VARLEN ? tok0 * p.o_rstride : bidx * p.o_bstride) + hq * p.o_hstride;
        it.lseb = (!VARLEN && p.lse) ? p.lse + ((int64_t)bidx * p.heads_q + hq) * p.seqlen_q : nullptr;
        // Score modifiers: a sliding window's left edge lets the walk start at the 32-key
        // step holding the first key any row of this workgroup sees (the K/V descriptors
        // start there); the mask works in absolute key positions.
        int kb0 = 0;
        it.slope = 0.f;
        if constexpr (MODS) {
            if (p.win_left >= 0) kb0 = max(0, tile * BMW - p.win_left) & ~31;
            if (p.alibi) it.slope = p.alibi[(int64_t)bidx * p.alibi_sstride + hq];
        }
        it.kb0 = kb0;
        const T* kb = static_cast<const T*>(p.k) + (VARLEN ? tok0 * p.k_rstride : bidx * p.k_bstride) + hk * p.k_hstride + kb0 * p.k_rstride;
        const T* vb = static_cast<const T*>(p.v) + (VARLEN ? tok0 * p.v_rstride : bidx * p.v_bstride) + hk * p.v_hstride + kb0 * p.v_rstride;
        const int Lk_rel = Lk - kb0;
        const int k_valid = Lk_rel > 0 ? (int)((int64_t)(Lk_rel - 1) * k_rs + hd * sizeof(T)) : 0;
        const int v_valid = Lk_rel > 0 ? (int)((int64_t)(Lk_rel - 1) * v_rs + hd * sizeof(T)) : 0;
        it.rk = buffer_desc(kb, k_valid);
        it.rv = buffer_desc(vb, v_valid);
        // The key range is walked in 32-key sub-steps, SPT per K/V tile. All waves of the
        // workgroup walk the same sub-steps (a wave whose own rows end earlier gets fully
        // masked sub-steps at the end, which add exact zeros).
        const int wg_rows_end = min(tile * BMW + BMW, Lq);
        int keys_needed = CAUSAL ? wg_rows_end : Lk;
        if constexpr (MODS && !CAUSAL)
            if (p.win_right >= 0) keys_needed = min(Lk, wg_rows_end + p.win_right);
        it.nsub = (keys_needed - kb0 + 31) / 32;
        it.n_kt = (it.nsub + SPT - 1) / SPT;
        return true;
    };
    // Persistent form: the r-th item of this workgroup. Items of one XCD are dealt to its
    // workgroups in snake order (forward in even rounds, backward in odd ones), which with
    // the longest-first order balances the causal work across them.
    auto item_x = [&](int r) -> int {
        const int G = gridDim.x;
        if (NG % 8 == 0 && G % 8 == 0) {
            const int gx = G >> 3, w = blockIdx.x >> 3;
            const int l = r * gx + ((r & 1) ? gx - 1 - w : w);
            return l * 8 + (blockIdx.x & 7);
        }
        const int b = blockIdx.x;
        return r * G + ((r & 1) ? G - 1 - b : b);
    };

    Item cur;
    if (!make_item(PERSIST ? item_x(0) : vx, cur)) return;

    // ---------------------------------------------------------------- Q -> registers
    // Issued after the first K/V tile copy so that both latencies overlap; a negative scale
    // flips Q's sign bits in a separate uniform branch (the only place that waits for the
    // loads before the matrix products).
    const bool neg = p.scale_log2 < 0.f;
    const float c = fmaxf(fabsf(p.scale_log2), 1e-30f);
    // With score modifiers the mask step leaves the scores in log2 units already.
    const float cs = MODS ? 1.f : c;
    u32x4 qf[NB][KS];
    // Buffer loads whose descriptor covers the Lq valid rows: rows past the end read as
    // zero, and one lane offset serves all k-steps (a scalar offset adds 32 bytes per step).
    auto load_q = [&](const Item& it) {
        const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<T*>(it.qb), (short)0, it.Lq > 0 ? (int)((int64_t)it.Lq * q_rs) : 0, (int)kBufferFlags);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const uint32_t off = (uint32_t)(it.qr0 + 32 * nb + ln) * q_rs + (uint32_t)h * 16u;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[nb][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)off, ks * 32, 0));
        }
        if (hd < D) {   // columns past head_dim are zero (uniform branch)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    if ((2 * ks + h) * 8 >= hd) qf[nb][ks] = u32x4{0u, 0u, 0u, 0u};
        }
        if (neg) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) qf[nb][ks] ^= 0x80008000u;
        }
    };

    // ---------------------------------------------------------------- accumulators
    f32x16 o[DB][NB];
    float m_ref[NB], l_part[NB];
    auto reset_acc = [&]() {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) o[db][nb] = f32x16{};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) { m_ref[nb] = -INFINITY; l_part[nb] = 0.f; }
    };
    reset_acc();

    // Per-lane LDS address terms of the fragment reads. They are rebuilt from `lane` where
    // they are used; pinning `lane` with an empty asm per iteration stops the compiler from
    // hoisting every buffer's addresses into registers for the whole loop.
    struct LaneAddr { int krow_sig, kx, h, tv_key, tv_chunk, tv_within, tv_swz; };
    auto lane_addr = [&](int ln_raw) {
        LaneAddr a;
        const int l32 = ln_raw & 31, tg = ln_raw >> 4, tc = ln_raw & 15;
        a.krow_sig = sigma(l32);
        a.kx = kx_lane<KC>(l32);
        a.h = ln_raw >> 5;
        a.tv_key = 8 * (tg >> 1) + (tc >> 2);          // + 16*kc + 4*t
        a.tv_chunk = 2 * (tg & 1) + ((tc & 3) >> 1);   // + 4*db
        a.tv_within = (tc & 1) * 8;                    // bytes
        a.tv_swz = vswz<KC>(a.tv_key);                 // (16*kc + 4*t + tv_key) % 4 == tv_key % 4
        return a;
    };

    // K fragments of sub-step `sub` (A operands of S^T = K Q^T, rows in sigma order)
    auto load_k = [&](int sub, const u32x4* cK, const LaneAddr& la, u32x4 (&kf)[KS]) {
        const int krow = 32 * (sub % SPT) + la.krow_sig;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = cK[krow * KC + ((2 * ks + la.h) ^ la.kx)];
    };
    // S^T = K Q^T: 32 keys x 32*NB queries
    auto mma_qk = [&](const u32x4 (&kf)[KS], f32x16 (&acc)[NB]) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[nb] = Mfma<T>::mma(kf[ks], qf[nb][ks], acc[nb]);
    };
    // -inf for keys past the end and (causal) keys after the query; a uniform branch.
    // With score modifiers every score is rewritten into log2 units: soft cap
    // cap*log2(e)*tanh(x/cap) = cap_l2 - 2 cap_l2 / (exp2(2 x log2(e) / cap) + 1) with
    // x = |scale| q.k (Q carries the sign of the scale), then the ALiBi bias; the masks
    // (sequence end, causal, window edges) only on sub-steps that straddle an edge.
    const float cap = MODS ? p.softcap : 0.f;
    const float cap_l2 = cap * 1.4426950408889634f;
    const float cap_k = cap > 0.f ? 2.f * c / cap : 0.f;
    auto mask = [&](int sub, f32x16 (&acc)[NB]) {
        if constexpr (MODS) {
            const int k0 = cur.kb0 + 32 * sub;
            const int qlo = cur.qr0, qhi = cur.qr0 + 32 * NB - 1;
            const bool edge = (k0 + 32 > cur.Lk) || (CAUSAL && k0 + 31 > qlo) ||
                              (p.win_left >= 0 && k0 < qhi - p.win_left) ||
                              (!CAUSAL && p.win_right >= 0 && k0 + 31 > qlo + p.win_right);
            const float slope_l2 = cur.slope * 1.4426950408889634f;
            // The three conditions are uniform: each combination is a loop of its own (tested
            // inside the unrolled loop they cost scalar compares and branches per score).
            auto rewrite = [&](auto has_cap, auto has_slope, auto is_edge) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    const int qi = qlo + 32 * nb + ln;
                    const float fb = (float)(qi - k0 - 8 * h);   // qi - key = fb - (key offset)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int koff_r = 16 * (r >> 3) + (r & 7);
                        float x;
                        if constexpr (decltype(has_cap)::value) {
                            const float e = __builtin_amdgcn_exp2f(acc[nb][r] * cap_k);
                            x = fmaf(-2.f * cap_l2, __builtin_amdgcn_rcpf(e + 1.f), cap_l2);
                        } else {
                            x = acc[nb][r] * c;
                        }
                        if constexpr (decltype(has_slope)::value) x = fmaf(-slope_l2, fabsf(fb - (float)koff_r), x);
                        if constexpr (decltype(is_edge)::value) {
                            // keep the rewrite unconditional: left alone, the compiler moves it
                            // under a per-score branch on the mask
                            asm volatile("" : "+v"(x));
                            const int key = k0 + 8 * h + koff_r;
                            const bool masked = (key >= cur.Lk) || (CAUSAL && key > qi) ||
                                                (p.win_left >= 0 && key < qi - p.win_left) ||
                                                (!CAUSAL && p.win_right >= 0 && key > qi + p.win_right);
                            x = masked ? -INFINITY : x;
                        }
                        acc[nb][r] = x;
                    }
                }
            };
            using Y = std::true_type;
            using N = std::false_type;
            auto by_edge = [&](auto has_cap, auto has_slope) {
                if (edge) rewrite(has_cap, has_slope, Y{});
                else rewrite(has_cap, has_slope, N{});
            };
            if (cap > 0.f) {
                if (slope_l2 != 0.f) by_edge(Y{}, Y{});
                else by_edge(Y{}, N{});
            } else {
                if (slope_l2 != 0.f) by_edge(N{}, Y{});
                else by_edge(N{}, N{});
            }
            return;
        }
        const int k0 = 32 * sub;
        if ((k0 + 32 > cur.Lk) || (CAUSAL && k0 + 31 > cur.qr0)) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int qi = cur.qr0 + 32 * nb + ln;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 16 * (r >> 3) + 8 * h + (r & 7);
                    const bool masked = (key >= cur.Lk) || (CAUSAL && key > qi);
                    acc[nb][r] = masked ? -INFINITY : acc[nb][r];
                }
            }
        }
    };
    // Whether any of this wave's query rows sees a key of sub-step `sub` (wave-uniform).
    auto wave_sees = [&](int sub) -> bool {
        const int k0 = cur.kb0 + 32 * sub;
        const int qlo = cur.qr0, qhi = cur.qr0 + 32 * NB - 1;
        if (qlo >= cur.Lq) return false;
        if (CAUSAL && k0 > qhi) return false;
        if constexpr (MODS) {
            if (p.win_left >= 0 && k0 + 31 < qlo - p.win_left) return false;
            if (!CAUSAL && p.win_right >= 0 && k0 > qhi + p.win_right) return false;
        }
        return true;
    };
    // V^T fragments of sub-step `sub` (A operands of O^T = V^T P^T): two transposed 8-byte
    // reads per 16-key chunk and 32-row d-block
    auto load_v = [&](int sub, const u32x4* cV, const LaneAddr& la, u32x4 (&vf)[2][DB]) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int kc = 2 * (sub % SPT) + cc;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int key = 16 * kc + 4 * t + la.tv_key;
                    const char* addr = reinterpret_cast<const char*>(cV + key * KC + ((4 * db + la.tv_chunk) ^ la.tv_swz)) + la.tv_within;
                    const i16x4_t part = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const_cast<char*>(addr)));
                    const u32x2 w = __builtin_bit_cast(u32x2, part);
                    vf[cc][db][2 * t] = w[0];
                    vf[cc][db][2 * t + 1] = w[1];
                }
            }
        }
    };
    // O^T += V^T P^T over one sub-step
    auto mma_pv = [&](const u32x4 (&vf)[2][DB], const u32x4 (&pf)[2][NB]) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) o[db][nb] = Mfma<T>::mma(vf[cc][db], pf[cc][nb], o[db][nb]);
    };
    // online softmax of one sub-step: P (packed 16-bit) relative to the possibly raised
    // reference max; the O / l rescale is applied by finish() after this sub-step's
    // neighbours in the pipeline have been issued
    struct Soft { float m_new[NB], alpha[NB], lsum[NB]; bool raise[NB]; };
    // P = exp2(s * c - m) packed to 16 bit, with its row sum over the rounded values
    auto exp_pack = [&](const f32x16& a, float m, u32x4 (&pf)[2][NB], int nb) {
        // with a sliding window a row can have no visible key yet (m = -inf): its P are 0
        const float mneg = (MODS && m == -INFINITY) ? 0.f : -m;
        float lsum = 0.f;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            float pv8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) pv8[e] = __builtin_amdgcn_exp2f(fmaf(a[8 * cc + e], cs, mneg));
            const u32x4 pk = {Mfma<T>::pack2(pv8[0], pv8[1]), Mfma<T>::pack2(pv8[2], pv8[3]),
                              Mfma<T>::pack2(pv8[4], pv8[5]), Mfma<T>::pack2(pv8[6], pv8[7])};
            // the row sum uses the same rounded P that multiplies V, so O stays an exact
            // convex combination of V rows up to fp32 accumulation
#pragma unroll
            for (int w = 0; w < 4; ++w) lsum = Mfma<T>::sum2(pk[w], lsum);
            pf[cc][nb] = pk;
        }
        return lsum;
    };
    auto softmax = [&](const f32x16 (&acc)[NB], u32x4 (&pf)[2][NB], Soft& st) {
        // Fast path: exponentiate against the current reference max right away. If no
        // lane's partial row sum exceeds 2^slack, no single P does, so no score exceeds the
        // reference by more than the slack and the full path below would keep the reference
        // too (up to rounding exactly at the threshold, where either choice keeps P in
        // range): same P and sums, without the row max. Otherwise (and on the first
        // sub-step, where the reference is -inf and the sums are inf or NaN) the full path
        // recomputes everything.
        {
            bool ok = true;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                st.lsum[nb] = exp_pack(acc[nb], m_ref[nb], pf, nb);
                ok = ok && (st.lsum[nb] <= kSlackExp) && (!MODS || m_ref[nb] != -INFINITY);
            }
            if (__all(ok)) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) {
                    st.raise[nb] = false;
                    st.m_new[nb] = m_ref[nb];
                    st.alpha[nb] = 1.f;
                }
                return;
            }
        }
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[nb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mt = (mx == -INFINITY) ? -INFINITY : mx * cs;
            const bool any = __any(mt > m_ref[nb] + kRescaleSlack);
            const float m_new = any ? fmaxf(m_ref[nb], mt) : m_ref[nb];
            st.raise[nb] = any;
            st.m_new[nb] = m_new;
            st.alpha[nb] = (MODS && m_new == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m_ref[nb] - m_new);
            st.lsum[nb] = exp_pack(acc[nb], m_new, pf, nb);
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

    // ---------------------------------------------------------------- epilogue
    // O = O^T accumulators / l, rounded to T, through buffer stores whose descriptor covers
    // exactly the Lq valid rows of this wave's slice: rows past the end and columns past
    // head_dim (given an offset past the descriptor) are dropped by the hardware, so every
    // wave issues the same store instructions per item, with no branch (non-persistent forms).
    auto store_o = [&]() {
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            cur.ob, (short)0, cur.Lq > 0 ? (int)((int64_t)cur.Lq * o_rs) : 0, (int)kBufferFlags);
        float lse_row[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float l = l_part[nb] + __shfl_xor(l_part[nb], 32);
            const float inv = 1.f / l;
            // natural log-sum-exp of the scaled scores: t = scale * log2(e) * q.k, so
            // log(sum exp(scale q.k)) = (m + log2 l) * ln 2
            lse_row[nb] = (m_ref[nb] + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
            const uint32_t rowoff = (uint32_t)(cur.qr0 + 32 * nb + ln) * o_rs;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d0 = 32 * db + 8 * g + 4 * h;
                    const u32x2 w = {Mfma<T>::pack2(o[db][nb][4 * g] * inv, o[db][nb][4 * g + 1] * inv),
                                     Mfma<T>::pack2(o[db][nb][4 * g + 2] * inv, o[db][nb][4 * g + 3] * inv)};
                    const uint32_t off = d0 < hd ? rowoff + (uint32_t)d0 * (uint32_t)sizeof(T) : kOobOffset;
                    __builtin_amdgcn_raw_buffer_store_b64(w, ro, (int)off, 0, 0);
                }
        }
        // after the O stores: the persistent form's wait for the next item only needs every
        // store to be newer than that item's loads
        if (cur.lseb) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = cur.qr0 + 32 * nb + ln;
                if (h == 0 && row < cur.Lq) cur.lseb[row] = lse_row[nb];
            }
        }
    };

    // Persistent form: the same O, staged through the wave's LDS slab so that each store
    // instruction writes 8 whole 128-byte row segments (the accumulator layout above gives
    // every store 32 rows x 16 bytes: 32 cache lines per instruction, which left the memory
    // pipeline of every CU busy for thousands of cycles when all workgroups finished an item
    // at once, with the next item's loads and tile copies queued behind the stores). One
    // 64-column half of the rows at a time: 8 stores of 8 bytes per lane into the slab (16-byte
    // chunk c of row r sits at c ^ ((r / 2) % 8), its two 8-byte halves swapped in rows 16-31,
    // so that the 32 lanes of each write pass cover all 64 banks once), then 4 reads of 8 rows
    // x 128 contiguous bytes, each lane storing its chunk where it belongs (the reads of rows
    // 16-31 swap the halves back: a renaming of registers).
    // The slab is this wave's alone and LDS operations of one wave complete in order, so no
    // wait or barrier is needed between the writes, the reads and the next half's writes.
    auto store_o_slab = [&]() {
        const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
            cur.ob, (short)0, cur.Lq > 0 ? (int)((int64_t)cur.Lq * o_rs) : 0, (int)kBufferFlags);
        char* slab = reinterpret_cast<char*>(sO[PERSIST ? wave : 0]);   // called in the persistent form only
        float lse_row[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            const float l = l_part[nb] + __shfl_xor(l_part[nb], 32);
            const float inv = 1.f / l;
            lse_row[nb] = (m_ref[nb] + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
#pragma unroll
            for (int hr = 0; hr < DB / 2; ++hr) {
#pragma unroll
                for (int dbl = 0; dbl < 2; ++dbl)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x16& a = o[2 * hr + dbl][nb];
                        const u32x2 w = {Mfma<T>::pack2(a[4 * g] * inv, a[4 * g + 1] * inv),
                                         Mfma<T>::pack2(a[4 * g + 2] * inv, a[4 * g + 3] * inv)};
                        const int cs = (4 * dbl + g) ^ ((ln >> 1) & 7);
                        *reinterpret_cast<u32x2*>(slab + ln * 128 + cs * 16 + (h ^ (ln >> 4)) * 8) = w;
                    }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int row = 8 * k + (lane >> 3), slot = lane & 7;
                    u32x4 v = *reinterpret_cast<const u32x4*>(slab + row * 128 + slot * 16);
                    if (k >= 2) v = u32x4{v[2], v[3], v[0], v[1]};   // rows 16-31: halves swapped
                    const int d0 = 64 * hr + 8 * (slot ^ ((row >> 1) & 7));
                    const uint32_t off = d0 < hd ? (uint32_t)(cur.qr0 + 32 * nb + row) * o_rs + (uint32_t)d0 * (uint32_t)sizeof(T)
                                                 : kOobOffset;
                    // non-temporal: each instruction writes 8 whole lines that no one here
                    // reads again (-1.5 to -3% per launch on the bf16 causal GQA workload; the
                    // same policy on Q loads, read once too, was slower)
                    __builtin_amdgcn_raw_buffer_store_b128(v, ro, (int)off, 0, 2);
                }
            }
        }
        if (cur.lseb) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                const int row = cur.qr0 + 32 * nb + ln;
                if (h == 0 && row < cur.Lq) cur.lseb[row] = lse_row[nb];
            }
        }
    };

    // ---------------------------------------------------------------- main loop
    // Tile t of an item sits in buffer (t + parity) % NBUF. Every buffer choice is a
    // compile-time one after unrolling, and every tile-copy completion is ordered by an
    // explicit s_waitcnt vmcnt + s_barrier (the copies are invisible to the compiler).
    const uint32_t tk = kBN * k_rs, tv = kBN * v_rs;   // bytes per K / V tile
    auto lds_off = [](const u32x4* q) { return (uint32_t)(uintptr_t)(lds_void*)q; };
    uint32_t lK[NBUF], lV[NBUF];
    const u32x4* cKb[NBUF];
    const u32x4* cVb[NBUF];
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
        lK[b] = lds_off(sK[b]);
        lV[b] = lds_off(sV[b]);
        cKb[b] = sK[b];
        cVb[b] = sV[b];
    }
    f32x16 s_cur[NB];
    u32x4 p_cur[2][NB];

    // One item's tiles. `first`: no O stores of an earlier item are in flight; `more`: the
    // next item (persistent form) exists and its first tile copy is issued after the barrier
    // of this item's last tile (its Q loads follow the item, before the O stores).
    auto run_item = [&](auto parity, bool first, bool more, const Item& nxt) {
        constexpr int P = decltype(parity)::value;
        for (int g = 0; NBUF * g < cur.n_kt; ++g) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) {
                const int t = NBUF * g + u;
                if (t >= cur.n_kt) break;
                const int b = (u + P) % NBUF;
                const int bn = (u + P + AHEAD) % NBUF;          // buffer of tile t + AHEAD
                // at tile 0 of a later item the previous item's NSTORE O stores (and its LSE
                // stores after them) are the newest memory operations: vmcnt(NSTORE) still
                // waits for the copy and the Q loads issued before them
                if (PERSIST && t == 0 && !first) wait_vmcnt_barrier<NSTORE>();
                else wait_vmcnt_barrier<0>();
                // Fragment reads run one step ahead of their use: after the S^T products of
                // sub-step i are issued, the V fragments of i and the K fragments of i+1 are
                // requested, and arrive while the softmax of i runs. The copy of tile
                // t + AHEAD is issued in DMA_PARTS pieces, one after each of the first
                // DMA_PARTS sub-steps' S^T products (every sub-step of a tile that is not the
                // last one runs, so all pieces are issued before the next barrier).
                const bool copy_next = t + AHEAD < cur.n_kt;
                if (PERSIST && more && t + 1 == cur.n_kt)
                    issue_tile<NI>(nxt.rk, nxt.rv, koff, voff, 0, 0, lK[bn], lV[bn], wave);
                const LaneAddr la = lane_addr(lane);
                u32x4 kf[KS];
                u32x4 vf[2][DB];
                load_k(SPT * t, cKb[b], la, kf);
                // All K fragment reads of the tile's first sub-step are issued before its first
                // product: left to itself the scheduler chains them through one register quad,
                // read -> wait -> product, eight LDS round trips in a row after every barrier
                // (measured: -5% time on the fp16 head_dim-64 causal workload, -1% on the bf16
                // GQA ones, outputs bitwise unchanged).
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int hh = 0; hh < SPT; ++hh) {
                    const int i = SPT * t + hh;
                    if (i >= cur.nsub) break;
                    // varlen and score-modifier problems: a sub-step none of this wave's rows
                    // can see (a causal or window edge of the workgroup's other rows, or rows
                    // past the sequence) only does its share of the tile copy and the next
                    // fragment reads (measured: -5% time on the bf16 modifier workload, -3% on the
                    // bf16 varlen one). Not for dense problems: the persistent form's 64-row
                    // items leave one such sub-step to half of the waves and the branch costs it
                    // 17 registers; on the fp16 head_dim-64 causal workload it measured +3%.
                    const bool live = !VARLEN || wave_sees(i);
                    if (live) mma_qk(kf, s_cur);
                    if (hh < DMA_PARTS && copy_next)
                        issue_tile_part<NI, DMA_PARTS>(hh, cur.rk, cur.rv, koff, voff, (t + AHEAD) * tk, (t + AHEAD) * tv,
                                                       lK[bn], lV[bn], wave);
                    if (live) load_v(i, cVb[b], la, vf);
                    if (hh + 1 < SPT) load_k(i + 1, cKb[b], la, kf);
                    if (live) {
                        mask(i, s_cur);
                        Soft st;
                        softmax(s_cur, p_cur, st);
                        finish(st);
                        mma_pv(vf, p_cur);
                    }
                }
            }
        }
    };

    if constexpr (PERSIST) {
        issue_tile<NI>(cur.rk, cur.rv, koff, voff, 0, 0, lK[0], lV[0], wave);
        load_q(cur);
        int par = 0;   // buffer of the current item's first tile
        for (int r = 0;; ++r) {
            Item nxt;
            const bool more = make_item(item_x(r + 1), nxt);
            if (par == 0) run_item(Parity<0>{}, r == 0, more, nxt);
            else run_item(Parity<1>{}, r == 0, more, nxt);
            if (more) load_q(nxt);   // Q is dead after this item's last S^T products
            store_o_slab();
            if (!more) break;
            par = (par + cur.n_kt) & 1;
            cur = nxt;
            reset_acc();
        }
    } else {
#pragma unroll
        for (int a = 0; a < AHEAD; ++a)
            if (a < cur.n_kt) issue_tile<NI>(cur.rk, cur.rv, koff, voff, a * tk, a * tv, lK[a], lV[a], wave);
        load_q(cur);
        run_item(Parity<0>{}, true, false, cur);
        store_o();
    }
#endif  // __HIP_DEVICE_COMPILE__
}

int heads_per_group(int group) { return (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1; }

// workgroups that fit on the device at once for the persistent form (one per CU)
int resident_workgroups() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
    return n;
}

template <typename T, int D, int WAVES, int NB, int GH, int TB, bool PERSIST, bool CAUSAL, bool VARLEN,
          bool MODS = false>
hipError_t launch_cfg(const AttnProblem& p, hipStream_t stream) {
    constexpr int BMW = 32 * NB * (WAVES / GH);
    dim3 block(WAVES * 64);
    if constexpr (VARLEN) {
        dim3 grid(varlen_grid_tiles(p.total_tokens, p.batch, BMW), p.heads_q / GH, 1);
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<T, D, WAVES, NB, GH, TB, PERSIST, CAUSAL, true, MODS>), grid, block, 0, stream, p, 0);
    } else {
        const int n_qtiles = (p.seqlen_q + BMW - 1) / BMW;
        const int64_t nitems = (int64_t)n_qtiles * p.batch * (p.heads_q / GH);
        if (nitems > INT32_MAX) return hipErrorInvalidConfiguration;
        int64_t nblocks = nitems;
        if constexpr (PERSIST) {
            static const int resident = resident_workgroups();
            const int64_t g = resident >= 8 ? resident / 8 * 8 : resident;
            if (nblocks > g) nblocks = g;
        }
        dim3 grid((unsigned)nblocks);
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<T, D, WAVES, NB, GH, TB, PERSIST, CAUSAL, false, false>), grid, block, 0, stream, p, n_qtiles);
    }
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, bool VARLEN>
hipError_t launch_gh(const AttnProblem& p, hipStream_t stream) {
    const int gh = VARLEN ? 1 : heads_per_group(p.group);
    const int g = gh == 4 ? 2 : gh == 2 ? 1 : 0;
    if constexpr (VARLEN) {   // score modifiers: 4-wave workgroups, 64-key tiles (form 4)
        // 128-row workgroups balance the windowed causal work better than 256-row ones and
        // two share a CU: 0.529 -> 0.440 ms on the bf16 varlen workload with a 1024-key
        // window, soft cap 50 and ALiBi
        if (p.mods) return launch_cfg<T, D, 4, 1, 1, 64, false, CAUSAL, true, true>(p, stream);
    }
    // dense problems at head_dim 128: persistent 8-wave workgroups over 128-key tiles;
    // varlen problems and head_dim <= 64: 4-wave workgroups over 64-key tiles, where the
    // 128-row workgroups balance the causal work better (measured on the bf16 varlen and fp16
    // head_dim-64 causal workloads: +6% and +10% over the 8-wave form)
    if constexpr (VARLEN || D <= 64) {
        switch (g) {
            case 0: return launch_cfg<T, D, 4, 1, 1, 64, false, CAUSAL, VARLEN>(p, stream);
            case 1: return launch_cfg<T, D, 4, 1, 2, 64, false, CAUSAL, VARLEN>(p, stream);
            case 2: return launch_cfg<T, D, 4, 1, 4, 64, false, CAUSAL, VARLEN>(p, stream);
        }
    } else {
        switch (g) {
            case 0: return launch_cfg<T, D, 8, 1, 1, 128, true, CAUSAL, false>(p, stream);
            case 1: return launch_cfg<T, D, 8, 1, 2, 128, true, CAUSAL, false>(p, stream);
            case 2: return launch_cfg<T, D, 8, 1, 4, 128, true, CAUSAL, false>(p, stream);
        }
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
    // K/V copies, Q loads and O stores address one (sequence, head) slice with 32-bit buffer
    // offsets from the slice's first row (64-bit pointers get there); keep the slice plus
    // one tile of offset headroom below 2^30 bytes. A varlen slice is at most max_seqlen rows
    // (the kernels clamp every sequence to it).
    const int64_t rows_k = p.cu_seqlens ? p.max_seqlen : p.seqlen_k;
    const int64_t rows_q = p.cu_seqlens ? p.max_seqlen : p.seqlen_q;
    const int64_t stride_k = p.k_rstride > p.v_rstride ? p.k_rstride : p.v_rstride;
    const int64_t stride_q = p.q_rstride > p.o_rstride ? p.q_rstride : p.o_rstride;
    const int64_t limit = int64_t(1) << 30;
    return (rows_k + 256) * stride_k * 2 < limit && (rows_q + 256) * stride_q * 2 < limit;
}

hipError_t launch_attn_fwd_mfma(const AttnProblem& p, Dtype dt, hipStream_t stream) {
    if (dt == Dtype::BF16) return launch_t<bf16_t>(p, stream);
    if (dt == Dtype::F16) return launch_t<f16_t>(p, stream);
    return hipErrorInvalidValue;
}

}  // namespace aule
