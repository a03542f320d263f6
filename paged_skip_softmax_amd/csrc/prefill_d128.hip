// bf16 varlen prefill, head dim 128, for gfx950: the D = 128 path of attn_prefill_varlen and the
// long-query route of attn_decode_paged_multi ("Model-Optimizer: Add Triton unified attention kernel":
// variable-length batching, GQA, causal and non-causal; sequences packed THD with cu_seqlens, or K / V
// read through a block table from the paged cache).  One kernel template, prefill_d128_kernel<SKIP,
// PAGED>: SKIP adds skip-softmax on 32-key tiles ("TensorRT-LLM: Skip Softmax Attention",
// Description); PAGED takes K and V from [num_pages, Hkv, 16, D] caches instead of THD tensors.
//
// Work split.  A workgroup of 4 waves takes one query tile of one sequence for NH query heads of one
// KV head's group times RB blocks of 32 query rows (NH * RB = 4, NH the largest power of two dividing
// the group size, at most 4), so every K/V tile staged in LDS serves NH heads: the group's query heads
// share their KV head (GQA) and read it from LDS once.  Two workgroups share a CU.  Workgroups are
// numbered so that the hardware's round-robin over the 8 XCDs gives each XCD a contiguous run of work
// items ordered (KV head, sequence, query tile from the last): the query tiles of one sequence and KV
// head run together on one XCD and find their K and V in its L2.  Each wave keeps Q^T of its 32 rows in
// registers as the MFMA B operand for the whole loop.
//
// Per 64-key tile a wave computes
//   S^T[64 keys x 32 rows] = K[64 x 128] . Q^T[128 x 32]     16 MFMA 32x32x16 (bf16 in, fp32 acc)
//   online softmax in the log2 domain (scale * log2 e folded into one FMA)
//   O^T[128 x 32] += V^T[128 x 64] . P^T[64 x 32]            16 MFMA 32x32x16
// The key order inside P.V follows the S^T register layout, so P feeds the second product straight from
// registers.  The QK^T of tile t+1 is issued in the same basic block as the softmax of tile t.
//
// Memory pipeline.  K and V tiles travel HBM -> LDS with buffer loads that write LDS directly (no
// registers, no LDS store instructions), each in a two-stage ring with K one tile ahead of V: while the
// waves use K(t+1) and V(t), the loads of K(t+2) and V(t+1) are in flight.  Each load instruction of a
// wave fills 1 KB of LDS (4 key rows); rows past the sequence are outside the buffer resource and read
// as zero.  Paged: the four loads of wave w for tile t are exactly the 16 keys of one cache page (the
// block-table entry 4t + w), through a buffer resource built per page whose size ends at the sequence's
// last key; the block-table entries are read (scalar loads: the table is read through the constant
// address space) before the barrier that precedes the loads.
// LDS rows are not padded: the 16-byte chunks of a row are XOR-swizzled (slot = chunk ^ swz(row % 16)),
// which keeps both the 16-B reads of K and the transposed 8-B reads of V (ds_read_b64_tr_b16) free of
// bank conflicts.  Waits are explicit: vmcnt of the wave's own loads,
// then s_barrier.
//
// The running max used for the exponentials is only raised when a row's max exceeds it by more than 8
// (log2 units, a factor 2^8), so the O and l rescale is rare; the result is the same softmax computed
// with unnormalised weights P <= 2^8.
//
// Skip-softmax.  The two 32-key halves of a 64-key tile are the skip tiles (aligned to key 0).  Their
// row maxima come out of the same interleaved max as the dense tile max; each row keeps its exact
// running max beside the lazy one, and a half is skipped when the running max exists and its max is
// below it by more than -log2(threshold).  A skipped half contributes nothing and never raises the
// running max; its exponentials are left out by a wave-uniform branch when every row of the wave
// skips it, and the P.V products of a 64-key tile when every row skips both halves.
#include <type_traits>

#include "kcommon.h"
#include "launch.h"
#include "lds_dma.h"

namespace attn {
namespace {

constexpr int D = 128;
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBN = 64;                         // keys per tile
constexpr int kTileChunks = kBN * D / 8;        // 16-B chunks in one K (or V) tile
constexpr int kLoadsPerWave = kTileChunks / kThreads; // 1-KB load instructions per wave per tile
constexpr float kSlack = 8.f;
constexpr int kXcds = 8;

constexpr int kStages = 2;


// Two-stage rings for K and V, one LDS array per stage (64 KB per workgroup).
__shared__ __attribute__((aligned(1024))) uint4 k_st0[kTileChunks], k_st1[kTileChunks];
__shared__ __attribute__((aligned(1024))) uint4 v_st0[kTileChunks], v_st1[kTileChunks];

template <int ST> __device__ __forceinline__ uint4 *kbuf()
{
    return ST == 0 ? k_st0 : k_st1;
}
template <int ST> __device__ __forceinline__ uint4 *vbuf()
{
    return ST == 0 ? v_st0 : v_st1;
}

// Issues the direct-to-LDS loads of K and V tiles.  Contiguous K / V: one buffer resource over the
// sequence's rows of the KV head, tile t at a scalar offset.  Paged K / V: wave w loads the 16 keys of
// page 4 t + w of the sequence (one 4 KB slab of the cache) through a resource over that slab alone,
// cut at the sequence's last key; the page number comes from the block table.
template <bool PAGED>
struct Loader {
    i32x4 krs, vrs;
    uint32_t voff[kLoadsPerWave]; // this lane's byte offsets for its 4-row blocks
    uint32_t tile_bytes;          // global bytes between consecutive 64-key tiles
    uint32_t m0k[kStages], m0v[kStages]; // LDS byte address of this wave's first 4-row block per stage
    // paged only
    const __attribute__((address_space(4))) int32_t *btr; // the sequence's block-table row (read-only:
                                                          // scalar loads, outside the vector-memory count)
    const uint16_t *kc, *vc;      // the caches
    size_t head_off, page_elems;  // elements to the KV head's slab in a page; elements per page
    int Lk, w;                    // keys of the sequence; the (wave-uniform) wave index
    uint32_t zero;                // 0 in a scalar register (the buffer loads' scalar offset)

    // the wave's page of tile t (0 when the page lies past the sequence)
    __device__ __forceinline__ int page_of(int t) const { return 64 * t + 16 * w < Lk ? btr[4 * t + w] : 0; }
    __device__ __forceinline__ i32x4 page_rsrc(const uint16_t *cache, int t, int page) const
    {
        const int nkeys = max(0, min(16, Lk - 64 * t - 16 * w));
        const i32x4 r =
            make_rsrc(nkeys > 0 ? cache + (size_t)page * page_elems + head_off : cache, (uint32_t)nkeys * 256);
        // wave-uniform by construction; said explicitly so the words stay in scalar registers
        return i32x4{__builtin_amdgcn_readfirstlane(r[0]), __builtin_amdgcn_readfirstlane(r[1]),
                     __builtin_amdgcn_readfirstlane(r[2]), r[3]};
    }
    template <int P = 0>
    __device__ __forceinline__ void issue(const i32x4 &rs, uint32_t m0, uint32_t soff) const
    {
        if constexpr (P < kLoadsPerWave) {
            dma16_at<P * 1024>(m0, voff[P], rs, soff);
            issue<P + 1>(rs, m0, soff);
        }
    }
    template <int ST> __device__ __forceinline__ void issue_k(int t, int page) const
    {
        if (PAGED)
            issue(page_rsrc(kc, t, page), m0k[ST], zero);
        else
            issue(krs, m0k[ST], (uint32_t)t * tile_bytes);
    }
    template <int ST> __device__ __forceinline__ void issue_v(int t, int page) const
    {
        if (PAGED)
            issue(page_rsrc(vc, t, page), m0v[ST], zero);
        else
            issue(vrs, m0v[ST], (uint32_t)t * tile_bytes);
    }
};

struct Wave {
    bf16x8 qop[D / 16];
    f32x16 acc[D / 32];
    float m, l;
    uint32_t ka[D / 16];       // K operand read offsets within a tile (per k-step)
    uint32_t va[2][D / 32];    // V transposed-read offsets within a tile ([key half][d block])
};

template <int ST>
__device__ __forceinline__ void qk_tile(const Wave &wv, f32x16 sc[2])
{
    const char *kt = reinterpret_cast<const char *>(kbuf<ST>());
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            sc[kk][i] = 0.f;
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            sc[kk] = mfma32(as_bf16x8(ld16(kt + kk * 32 * 256 + wv.ka[s])), wv.qop[s], sc[kk]);
    }
}

// Masks keys at or past the row's limit (causal diagonal or sequence end).  key(kk, i) = kb + 32 kk +
// 8 (i / 4) + 4 J + i % 4.
__device__ __forceinline__ void mask_tile(f32x16 sc[2], int limit_minus_kb, int J)
{
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (32 * kk + 8 * (i / 4) + 4 * J + (i % 4) >= limit_minus_kb)
                sc[kk][i] = kNegInf;
}

struct IterCtx {
    int niter, Lk;
    bool causal;
    int first_row_w, diag, kend_row, J;
    float scale_log2;
    float log2_thr;  // log2(threshold), -inf when skipping is off
    uint8_t *map;      // skip map, or null
    uint32_t map_row;  // byte offset of this lane's map row; ~0u for lanes that write none
    int map_stride;
};

// Skip-softmax state of the lane's row: the exact running max (log2 units) and which 32-key halves of
// the current tile are kept.  A skipped half never raises the running max (threshold <= 1), so the max
// before any half is the max over all earlier halves, skipped or not: the decisions below are those of
// the sequential definition.
struct SkipState {
    float m_true;
    bool keep[2];
};

// Statistics of tile t from the lane's partial maxima t0, t1 of its two 32-key halves: the row max
// tm of the kept halves (log2 units) and whether it raises the exponent offset by more than the slack
// (then the O and l rescale is due before the tile's exponentials).  With SKIP, first the two skip
// decisions of the row: a visited half is skipped when the running max exists and
// tmax_half - running max < log2(threshold); the skip map gets 0 (kept), 1 (skipped) or 2 (no visible
// key).
template <bool SKIP>
__device__ __forceinline__ void tile_stats(float t0, float t1, int t, const IterCtx &c, const Wave &wv,
                                           SkipState &ss, float &tm, bool &raise)
{
    const float sl = c.scale_log2;
    if (!SKIP) {
        tm = fmaxf(t0, t1);
        tm = max_halves(tm) * sl;
    } else {
        const float h0 = max_halves(t0) * sl;
        const float h1 = max_halves(t1) * sl;
        const int kb = t * kBN;
        const bool vis0 = kb < c.kend_row, vis1 = kb + 32 < c.kend_row;
        const bool skip0 = vis0 && ss.m_true != kNegInf && h0 - ss.m_true < c.log2_thr;
        const float m1 = vis0 ? fmaxf(ss.m_true, h0) : ss.m_true;
        const bool skip1 = vis1 && m1 != kNegInf && h1 - m1 < c.log2_thr;
        ss.m_true = vis1 ? fmaxf(m1, h1) : m1;
        ss.keep[0] = vis0 && !skip0;
        ss.keep[1] = vis1 && !skip1;
        if (c.map && c.map_row != ~0u && t < c.niter) {
            uint8_t *mr = c.map + c.map_row;
            mr[2 * t] = vis0 ? (skip0 ? 1 : 0) : 2;
            if (2 * t + 1 < c.map_stride)
                mr[2 * t + 1] = vis1 ? (skip1 ? 1 : 0) : 2;
        }
        tm = fmaxf(ss.keep[0] ? h0 : kNegInf, ss.keep[1] ? h1 : kNegInf);
    }
    raise = tm > wv.m + kSlack;
}

__device__ __forceinline__ bool needs_mask(int t, const IterCtx &c)
{
    const int kb = t * kBN;
    return kb + kBN > c.Lk || (c.causal && kb + kBN - 1 > c.first_row_w + c.diag);
}

// Tile t held in stage ST = t % 2 (K(t+1) in the other stage).  K runs one tile ahead of V: when tile
// t starts, K(t+1) and V(t) must be resident.  t0, t1: the lane's partial maxima of the two 32-key
// halves of tile t on entry, of tile t+1 on return.
//   wait for the wave's loads, barrier (every wave is done with K(t) and V(t-1)); read the first two K
//   operands of (b), then start loading K(t+2) and V(t+1) into those two stages, and take the row
//   statistics (and skip decisions) of tile t while the reads are in flight;
//   (a) rescale O and l when the max rose by more than the slack;
//   (b) QK^T of tile t+1, with the exponentials and row sums of tile t placed between its MFMAs, at
//       raised wave priority (the two waves of a SIMD belong to different workgroups; the one in its
//       MFMA-and-exponential phase goes first, the other fills the gaps);
//   (c) mask tile t+1 where it crosses the diagonal or the sequence end;
//   (d) P.V of tile t, with the row max of tile t+1 placed between its MFMAs.
// On the last tile, (b)-(d) compute scores from a stale K stage that are never used.
// sc: the scores of tile t; the scores of tile t+1 go to nxo (the loop's two unrolled iterations pass two
// arrays in alternating roles, so no copy is needed between tiles).
template <int ST, bool SKIP, bool PAGED>
__device__ __forceinline__ void iteration(int t, const IterCtx &c, const Loader<PAGED> &ld, Wave &wv,
                                          f32x16 (&sc)[2], f32x16 (&nxo)[2], float &t0, float &t1,
                                          SkipState &ss)
{
    // paged: the block-table reads go out before the wait, so the barrier covers their latency
    int page_k = 0, page_v = 0;
    if (PAGED) {
        if (t + 2 < c.niter)
            page_k = ld.page_of(t + 2);
        if (t + 1 < c.niter)
            page_v = ld.page_of(t + 1);
    }
    wait_vmcnt<0>();
    barrier();
    constexpr int P = ST;
    const char *kt = reinterpret_cast<const char *>(kbuf<(P + 1) % kStages>());
    auto kop = [&](int step) { return ld16(kt + (step & 1) * 32 * 256 + wv.ka[step >> 1]); };
    uint4 k0 = kop(0), k1 = kop(1);
    sched_fence();
    if (t + 2 < c.niter)
        ld.template issue_k<ST>(t + 2, page_k);
    if (t + 1 < c.niter)
        ld.template issue_v<(ST + 1) % kStages>(t + 1, page_v);
    float tm;
    bool raise;
    tile_stats<SKIP>(t0, t1, t, c, wv, ss, tm, raise);

    // (a)
    if (__any(raise)) {
        const float m_new = raise ? tm : wv.m;
        // raising from m = -inf gives 0 (acc and l are still 0); rows that do not raise keep their state
        // (also rows that have seen no key yet, whose m - m_new would be -inf - -inf)
        const float alpha = raise ? exp2_fast(wv.m - m_new) : 1.f;
        wv.m = m_new;
        wv.l *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
            wv.acc[db] *= alpha;
    }
    const float m_use = wv.m == kNegInf ? 0.f : wv.m;
    const float sl = c.scale_log2;

    sched_fence();
    __builtin_amdgcn_s_setprio(1);
    sched_fence();
    // (b) 16 MFMA steps, alternating the two 32-key blocks of tile t+1; K operands read two steps ahead
    f32x16(&nx)[2] = nxo;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        nx[0][i] = 0.f;
        nx[1][i] = 0.f;
    }
    uint32_t pk[2][8];
    // SKIP: a skipped half gets p = 0 from an infinite reference max instead of a per-row branch, so
    // the interleave of MFMAs and exponentials stays one basic block; when no row of the wave keeps
    // either half, the steps run without exponentials
    float mk0 = m_use, mk1 = m_use;
    if constexpr (SKIP) {
        mk0 = ss.keep[0] ? m_use : __builtin_inff();
        mk1 = ss.keep[1] ? m_use : __builtin_inff();
    }
    auto steps_b = [&](auto with_exp) {
#pragma unroll
        for (int step = 0; step < 16; ++step) {
            const uint4 k2 = step + 2 < 16 ? kop(step + 2) : k0;
            nx[step & 1] = mfma32(as_bf16x8(k0), wv.qop[step >> 1], nx[step & 1]);
            const int kk = step >> 3, i = 2 * (step & 7);
            if constexpr (decltype(with_exp)::value) {
                const float mk = kk ? mk1 : mk0;
                const float p0 = exp2_fast(fmaf(sc[kk][i], sl, -mk));
                const float p1 = exp2_fast(fmaf(sc[kk][i + 1], sl, -mk));
                wv.l += p0 + p1;
                anchor(wv.l);
                pk[kk][i >> 1] = pack_bf16x2(p0, p1);
            } else {
                pk[kk][i >> 1] = 0u;
            }
            anchor(pk[kk][i >> 1]);
            sched_fence();
            k0 = k1;
            k1 = k2;
        }
    };
    if constexpr (!SKIP) {
#pragma unroll
        for (int step = 0; step < 16; ++step) {
            const uint4 k2 = step + 2 < 16 ? kop(step + 2) : k0;
            nx[step & 1] = mfma32(as_bf16x8(k0), wv.qop[step >> 1], nx[step & 1]);
            const int kk = step >> 3, i = 2 * (step & 7);
            const float p0 = exp2_fast(fmaf(sc[kk][i], sl, -m_use));
            const float p1 = exp2_fast(fmaf(sc[kk][i + 1], sl, -m_use));
            wv.l += p0 + p1;
            anchor(wv.l);
            pk[kk][i >> 1] = pack_bf16x2(p0, p1);
            anchor(pk[kk][i >> 1]);
            sched_fence();
            k0 = k1;
            k1 = k2;
        }
    } else if (__any(ss.keep[0] || ss.keep[1])) {
        steps_b(std::true_type{});
    } else {
        steps_b(std::false_type{});
    }

    sched_fence();
    __builtin_amdgcn_s_setprio(0);
    sched_fence();
    // (c)
    if (t + 1 < c.niter && needs_mask(t + 1, c))
        mask_tile(nx, c.kend_row - (t + 1) * kBN, c.J);

    // (d) 16 MFMA steps over (32-key block kk, 16-key half u, d block db), db fastest so consecutive
    // MFMAs use different accumulators; V operands read two steps ahead
    t0 = nx[0][0];
    t1 = nx[1][0];
    {
        const char *vt = reinterpret_cast<const char *>(vbuf<P>());
        auto vop = [&](int step) {
            const char *vk = vt + (32 * (step >> 3) + 16 * ((step >> 2) & 1)) * 256;
            const uint2 lo = lds_read_tr(vk + wv.va[0][step & 3]);
            const uint2 hi = lds_read_tr(vk + wv.va[1][step & 3]);
            return make_uint4(lo.x, lo.y, hi.x, hi.y);
        };
        if (!SKIP) {
            uint4 v0 = vop(0), v1 = vop(1);
#pragma unroll
            for (int step = 0; step < 16; ++step) {
                const uint4 v2 = step + 2 < 16 ? vop(step + 2) : v0;
                const int kk = step >> 3, u = (step >> 2) & 1;
                const bf16x8 pop = __builtin_bit_cast(bf16x8, make_uint4(pk[kk][4 * u], pk[kk][4 * u + 1],
                                                                          pk[kk][4 * u + 2], pk[kk][4 * u + 3]));
                wv.acc[step & 3] = mfma32(as_bf16x8(v0), pop, wv.acc[step & 3]);
                // two new elements per three-input max (v_max3_f32) on even steps, the last one alone
                if ((step & 1) == 0 && step < 14) {
                    t0 = fmaxf(t0, fmaxf(nx[0][step + 1], nx[0][step + 2]));
                    t1 = fmaxf(t1, fmaxf(nx[1][step + 1], nx[1][step + 2]));
                    anchor(t0);
                    anchor(t1);
                } else if (step == 14) {
                    t0 = fmaxf(t0, nx[0][15]);
                    t1 = fmaxf(t1, nx[1][15]);
                    anchor(t0);
                    anchor(t1);
                }
                sched_fence();
                v0 = v1;
                v1 = v2;
            }
        } else {
            // the row maxima of tile t+1 first; then a tile that no row of the wave keeps (both 32-key
            // halves skipped or unseen by every row: P = 0 throughout) leaves its P.V out by one uniform
            // branch
#pragma unroll
            for (int i = 1; i < 16; ++i) {
                t0 = fmaxf(t0, nx[0][i]);
                t1 = fmaxf(t1, nx[1][i]);
            }
            if (__any(ss.keep[0] || ss.keep[1])) {
                uint4 v0 = vop(0), v1 = vop(1);
#pragma unroll
                for (int step = 0; step < 16; ++step) {
                    const uint4 v2 = step + 2 < 16 ? vop(step + 2) : v0;
                    const int kk = step >> 3, u = (step >> 2) & 1;
                    const bf16x8 pop = __builtin_bit_cast(
                        bf16x8, make_uint4(pk[kk][4 * u], pk[kk][4 * u + 1], pk[kk][4 * u + 2], pk[kk][4 * u + 3]));
                    wv.acc[step & 3] = mfma32(as_bf16x8(v0), pop, wv.acc[step & 3]);
                    sched_fence();
                    v0 = v1;
                    v1 = v2;
                }
            }
        }
    }
}

template <bool SKIP, bool PAGED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_d128_kernel(PrefillArgs a, int NH, int RB, int nqt, int nunits)
{
    // XCD-aware work order: block i runs on XCD i % 8; XCD x takes units [x * per, (x + 1) * per)
    const int per = gridDim.x / kXcds;
    const int unit = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (unit >= nunits)
        return;
    const int hchunks = a.G / NH;
    const int gh = unit / (a.B * nqt), rem = unit % (a.B * nqt);
    const int b = rem / nqt;
    const int qt = nqt - 1 - rem % nqt;
    const int g = gh / hchunks, hc = gh % hchunks;
    const int rows_wg = 32 * RB;
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int k0 = PAGED ? 0 : a.cu_k[b];
    const int Lk = PAGED ? a.seq_lens[b] : a.cu_k[b + 1] - k0;
    const int m0 = qt * rows_wg;
    if (m0 >= Lq)
        return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, J = lane >> 5;
    const int h = g * a.G + hc * NH + (w % NH);
    const int rbk = w / NH;
    const int qi = m0 + 32 * rbk + n;
    const bool row_ok = qi < Lq;
    const int diag = Lk - Lq;
    const int last_row = min(m0 + rows_wg, Lq) - 1;
    const int kend = a.causal ? max(0, min(Lk, last_row + 1 + diag)) : Lk;
    const int kend_row = a.causal ? max(0, min(Lk, qi + 1 + diag)) : Lk;
    const int first_row_w = m0 + 32 * rbk;
    const int niter = (kend + kBN - 1) / kBN;


    // loads: wave w fills 4-row blocks rb0 .. rb0+3 of each tile; lane -> row 4 rb + lane/16, slot lane%16
    Loader<PAGED> ld;
    {
        const uint16_t *kg = static_cast<const uint16_t *>(a.k);
        const uint16_t *vg = static_cast<const uint16_t *>(a.v);
        // contiguous: rows of the KV head Hkv * D apart; paged: the 16 rows of a page slab are adjacent
        const uint32_t row_bytes = PAGED ? D * 2 : (uint32_t)a.Hkv * D * 2;
        if (!PAGED) {
            const size_t head0 = ((size_t)k0 * a.Hkv + (size_t)g) * D;
            const uint32_t seq_bytes = Lk > 0 ? ((uint32_t)(Lk - 1) * a.Hkv + 1) * D * 2 : 0;
            ld.krs = make_rsrc(kg + head0, seq_bytes);
            ld.vrs = make_rsrc(vg + head0, seq_bytes);
            ld.tile_bytes = kBN * row_bytes;
        } else {
            ld.btr = (const __attribute__((address_space(4))) int32_t *)(a.bt + (size_t)b * a.max_pages);
            ld.kc = kg;
            ld.vc = vg;
            ld.head_off = (size_t)g * 16 * D;
            ld.page_elems = (size_t)a.Hkv * 16 * D;
            ld.Lk = Lk;
            ld.w = __builtin_amdgcn_readfirstlane(w);
            asm volatile("s_mov_b32 %0, 0" : "=s"(ld.zero));
        }
        const int rb0 = kLoadsPerWave * w;
        const uint32_t wave_off = __builtin_amdgcn_readfirstlane(rb0 * 1024);
        ld.m0k[0] = lds_addr(k_st0) + wave_off;
        ld.m0k[1] = lds_addr(k_st1) + wave_off;
        ld.m0v[0] = lds_addr(v_st0) + wave_off;
        ld.m0v[1] = lds_addr(v_st1) + wave_off;
#pragma unroll
        for (int p = 0; p < kLoadsPerWave; ++p) {
            const int row = 4 * (rb0 + p) + (lane >> 4);
            const int chunk = (lane & 15) ^ swz(row & 15);
            // paged: the row within the wave's page (the tile row's swizzle is the same: 16 | 16 w)
            ld.voff[p] = (uint32_t)(PAGED ? row - 16 * w : row) * row_bytes + 16 * chunk;
        }
    }

    // the first K / V tiles go out before anything else
    if (niter > 0) {
        const int pg0 = PAGED ? ld.page_of(0) : 0;
        ld.template issue_k<0>(0, pg0);
        ld.template issue_v<0>(0, pg0);
        if (niter > 1)
            ld.template issue_k<1>(1, PAGED ? ld.page_of(1) : 0);
    }

    Wave wv;
    {
        const uint16_t *qg = static_cast<const uint16_t *>(a.q);
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            wv.qop[s] = row_ok ? as_bf16x8(ld16(qg + ((size_t)(q0 + qi) * a.Hq + h) * D + 16 * s + 8 * J))
                               : as_bf16x8(make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                wv.acc[db][i] = 0.f;
        wv.m = kNegInf;
        wv.l = 0.f;
        // settle the Q loads (and the first tiles) before the first barrier; no later compiler-inserted
        // wait inside the loop is then needed for them (such a wait would also drain the loads in flight)
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(0);
        barrier();
        // K operand (A of S^T): key row n of the 32-key block, dims 16 s + 8 J: chunk 2 s + J
        const uint32_t kA = n * 256 + 16 * (J ^ swz(n & 15));
#pragma unroll
        for (int s = 0; s < D / 16; ++s)
            wv.ka[s] = kA ^ (32 * s);
        // V operand (A of O^T) by transposed reads: lane (16-lane group G, index j) addresses key
        // 8 half + 4 J + j/4 of a 16-key block, dims 32 db + 16 (G % 2) + 4 (j % 4)
        const int G16 = lane >> 4, j = lane & 15;
        const int x = 2 * (G16 & 1) + ((j & 3) >> 1);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int r = 8 * hf + 4 * J + (j >> 2);
            const uint32_t vT = r * 256 + 8 * (j & 1) + 16 * (x ^ swz(r));
#pragma unroll
            for (int db = 0; db < D / 32; ++db)
                wv.va[hf][db] = vT ^ (64 * db);
        }
    }

    // skip map: the row's entries past the workgroup's last tile are "not visited" up front; the others
    // are written tile by tile
    uint8_t *maprow = nullptr;
    uint32_t map_row = ~0u;
    if (SKIP && a.skip_map && row_ok && J == 0) {
        map_row = (uint32_t)(((size_t)(q0 + qi) * a.Hq + h) * a.map_stride);
        maprow = a.skip_map + map_row;
        for (int e = 2 * niter; e < a.map_stride; ++e)
            maprow[e] = 2;
    }

    f32x16 sc[2], sc2[2];
    float t0 = kNegInf, t1 = kNegInf;
    SkipState ss{kNegInf, {true, true}};
    IterCtx c{niter, Lk, a.causal, first_row_w, diag, kend_row, J, a.scale_log2, a.log2_thr, SKIP ? a.skip_map : nullptr, map_row,
              a.map_stride};
    if (niter > 0) {
        // prologue: K(0), V(0), K(1) arrived with the Q rows; the masked scores of tile 0 and their row max
        qk_tile<0>(wv, sc);
        if (needs_mask(0, c))
            mask_tile(sc, kend_row, J);
        t0 = sc[0][0];
        t1 = sc[1][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) {
            t0 = fmaxf(t0, sc[0][i]);
            t1 = fmaxf(t1, sc[1][i]);
        }
    }
    for (int t = 0; t < niter; t += kStages) {
        iteration<0, SKIP, PAGED>(t, c, ld, wv, sc, sc2, t0, t1, ss);
        if (t + 1 < niter)
            iteration<1, SKIP, PAGED>(t + 1, c, ld, wv, sc2, sc, t0, t1, ss);
    }

    wv.l = sum_halves(wv.l);
    if (!row_ok)
        return;
    const float inv = wv.l > 0.f ? 1.f / wv.l : 0.f;
    uint16_t *og = static_cast<uint16_t *>(a.o) + ((size_t)(q0 + qi) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint2 pk;
            pk.x = pack_bf16x2(wv.acc[db][4 * r] * inv, wv.acc[db][4 * r + 1] * inv);
            pk.y = pack_bf16x2(wv.acc[db][4 * r + 2] * inv, wv.acc[db][4 * r + 3] * inv);
            *reinterpret_cast<uint2 *>(og + 32 * db + 8 * r + 4 * J) = pk;
        }
    if (a.lse && J == 0)
        a.lse[(size_t)(q0 + qi) * a.Hq + h] = wv.l > 0.f ? (wv.m + __log2f(wv.l)) * kLn2 : kNegInf;
}

} // namespace

// Heads per workgroup: the largest power of two dividing the group size, at most 4.
static int heads_per_wg(int G)
{
    int nh = 1;
    while (nh < kWaves && G % (2 * nh) == 0)
        nh *= 2;
    return nh;
}

hipError_t launch_prefill_d128(const PrefillArgs &a, hipStream_t stream)
{
    const int NH = heads_per_wg(a.G), RB = kWaves / NH;
    const int rows = 32 * RB;
    const int nqt = (a.max_q + rows - 1) / rows;
    const long units = (long)a.Hkv * (a.G / NH) * a.B * nqt;
    const long blocks = (units + kXcds - 1) / kXcds * kXcds;
    if (blocks > 0x7fffffff)
        return hipErrorInvalidValue;
    const bool skip = a.log2_thr != kNegInf || a.skip_map != nullptr;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (a.bt) {
        if (skip)
            ATTN_LAUNCH((prefill_d128_kernel<true, true>), grid, block, 0, stream, a, NH, RB, nqt, (int)units);
        else
            ATTN_LAUNCH((prefill_d128_kernel<false, true>), grid, block, 0, stream, a, NH, RB, nqt, (int)units);
    } else if (skip) {
        ATTN_LAUNCH((prefill_d128_kernel<true, false>), grid, block, 0, stream, a, NH, RB, nqt, (int)units);
    } else {
        ATTN_LAUNCH((prefill_d128_kernel<false, false>), grid, block, 0, stream, a, NH, RB, nqt, (int)units);
    }
    return hipGetLastError();
}

} // namespace attn
