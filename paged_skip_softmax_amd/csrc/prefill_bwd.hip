// Backward of the dense bf16 varlen prefill (head dim 128) for gfx950: dQ, dK, dV from Q, K, V, O, the
// output gradient dO and the forward's log-sum-exp.  The Triton kernel of "Model-Optimizer: Add Triton
// unified attention kernel with HuggingFace integration" (summary) has an autograd backward beside its
// forward; the gradients are those of the masked-softmax definition:
//   P = exp(scale Q K^T - lse),  dP = dO V^T,  Dsum = rowsum(dO * O),  dS = P * (dP - Dsum)
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K         (dK, dV summed over a KV head's group)
//
// Three kernels, no atomics (dK/dV and dQ run at the same time, dQ on a side stream of the device that the
// call forks from its stream after the prep kernel and joins back to it):
//  * bwd_prep: Dsum and lse * log2(e) per (token, query head), fp32, into the caller's workspace.
//  * bwd_dkdv: a workgroup of 8 waves (two per SIMD) owns 128 keys of one (sequence, KV head) as 4 wave
//    pairs of 32 keys.  It walks every 64-row query tile that sees any of its keys, for every query
//    head of the group, from the sequence's last tile backwards (so that the key blocks of a sequence,
//    dispatched together, share each tile through L2); Q and dO tiles go to LDS by direct-to-LDS loads
//    (XOR-swizzled 16-byte chunks).  With 32x32x16 MFMAs, per 32-row block, a pair's
//      P wave  (K in registers):  S = Q K^T, P = exp2(S scale log2(e) - lse2), dV^T += dO^T P
//      dS wave (V in registers):  dP = dO V^T, dS = P (dP - Dsum), dK^T += Q^T dS
//    with P passed through LDS; the dS wave runs one tile behind, so one barrier per tile serves both.
//    The key order inside the row contraction follows the S register layout, so P and dS feed the
//    MFMA B operand straight from registers (A operands: 16-byte and transposed LDS reads).
//  * bwd_dq: the forward's work split over 4 groups (one query head and 32 rows each, the heads of a
//    group sharing K/V tiles in LDS), three waves per group on one SIMD; per 32-key tile
//      S wave (Q^T in registers):   S^T = K Q^T, P^T
//      D wave (dO^T in registers):  dP^T = V dO^T, dS^T = P^T (dP^T - Dsum)
//      Q wave:                      dQ^T += K^T dS^T (K^T by transposed reads)
//    with P^T and dS^T passed through LDS, each wave one tile behind the one before it.
#include <mutex>

#include "kcommon.h"
#include "launch.h"
#include "lds_dma.h"

namespace attn {
namespace {

constexpr int D = 128;
constexpr int kRowBytes = D * 2; // one bf16 row of 128 dims

// ------------------------------------------------------------------ Dsum and lse in log2 units

constexpr int kPrepUnroll = 4; // rows a 16-lane group has in flight together

// The (token, query head) rows are contiguous in O, dO and the LSE ([T, Hq, ...]); a grid-stride loop
// over the T * Hq rows (T = cu_seqlens_q[B], read on the device), 16 lanes per row with 8 dims each and
// kPrepUnroll rows per group in flight.
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a)
{
    // valid cu_seqlens give T <= B * max_q, the rows the workspace holds; the bound keeps the writes in it
    const long rows = min((long)a.cu_q[a.B], (long)a.B * a.max_q) * a.Hq;
    const int c = threadIdx.x & 15;
    const long group = (long)blockIdx.x * 16 + (threadIdx.x >> 4), groups = (long)gridDim.x * 16;
    const uint16_t *o = static_cast<const uint16_t *>(a.o), *dout = static_cast<const uint16_t *>(a.dout);
    for (long r0 = group; r0 < rows; r0 += groups * kPrepUnroll) {
        uint4 x[kPrepUnroll], g[kPrepUnroll];
#pragma unroll
        for (int u = 0; u < kPrepUnroll; ++u) {
            const long row = r0 + u * groups;
            x[u] = g[u] = make_uint4(0, 0, 0, 0);
            if (row < rows) {
                x[u] = ld16(o + row * D + 8 * c);
                g[u] = ld16(dout + row * D + 8 * c);
            }
        }
#pragma unroll
        for (int u = 0; u < kPrepUnroll; ++u) {
            const long row = r0 + u * groups;
            const uint32_t xw[4] = {x[u].x, x[u].y, x[u].z, x[u].w}, gw[4] = {g[u].x, g[u].y, g[u].z, g[u].w};
            float s = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s = fmaf(bf16_lo(xw[e]), bf16_lo(gw[e]), s);
                s = fmaf(bf16_hi(xw[e]), bf16_hi(gw[e]), s);
            }
            s += __shfl_xor(s, 8);
            s += __shfl_xor(s, 4);
            s += __shfl_xor(s, 2);
            s += __shfl_xor(s, 1);
            if (row < rows && c == 0)
                a.dsum[row] = s;
            if (row < rows && c == 1)
                a.lse2[row] = a.lse[row] * kLog2e;
        }
    }
}

// ------------------------------------------------------------------ dK, dV

constexpr int kXcds = 8;
constexpr int kKvPairs = 4;                         // wave pairs per workgroup
constexpr int kKvWaves = 2 * kKvPairs;              // two waves per SIMD
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKeysPerPair = 32;
constexpr int kKeysPerWg = kKvPairs * kKeysPerPair; // 128
constexpr int kQRows = 64;                          // query rows per staged tile
constexpr int kQTileBytes = kQRows * kRowBytes;     // 16 KB
constexpr int kQLoads = kQTileBytes / 1024 / kKvWaves; // 1-KB direct-to-LDS loads per wave per tile
constexpr int kQStages = 3;

// One stage of the Q / dO ring: the two tiles (swizzled rows) and the rows' lse * log2(e) and Dsum.
struct alignas(1024) QStage {
    char q[kQTileBytes];
    char g[kQTileBytes];
    float lse[kQRows];
    float dsum[kQRows];
};
__shared__ QStage q_ring[kQStages];

// P of a 32-row block, passed from a pair's P wave to its dS wave: the 8 packed registers of each lane,
// as two 1-KB halves of 16 B per lane.  Two tiles in flight (the dS wave runs one tile behind), two
// blocks per tile.
constexpr int kXchgBlock = 2048;
__shared__ __attribute__((aligned(1024))) char p_xchg[2][kKvPairs][2 * kXchgBlock];

// A block's packed P or dS: word j of half u packs registers 8u + 2j, 8u + 2j + 1 (one 16-row half of the
// MFMA B operand per half).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
struct Packed {
    u32x4 h[2];
};

__device__ __forceinline__ void xchg_store(char *blk, int lane, const Packed &pk)
{
    *reinterpret_cast<u32x4 *>(blk + 16 * lane) = pk.h[0];
    *reinterpret_cast<u32x4 *>(blk + 1024 + 16 * lane) = pk.h[1];
}
__device__ __forceinline__ void xchg_load(const char *blk, int lane, Packed &pk)
{
    pk.h[0] = *reinterpret_cast<const u32x4 *>(blk + 16 * lane);
    pk.h[1] = *reinterpret_cast<const u32x4 *>(blk + 1024 + 16 * lane);
}

// s_waitcnt lgkmcnt(0): this wave's LDS writes are done (before a barrier that publishes them).
__device__ __forceinline__ void wait_lds()
{
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0xc07f); // vmcnt 63, expcnt 7, lgkmcnt 0
    compiler_fence();
}

// What one lane needs to issue the direct-to-LDS loads of a Q / dO tile.
struct QLoader {
    i32x4 qrs, grs, lrs, drs;  // buffer resources of Q, dO (from head 0 of the sequence), lse2, Dsum
    uint32_t voff[kQLoads];    // lane's byte offsets inside a tile of rows (4-row blocks of the wave)
    uint32_t loff;             // lane's byte offset of its LSE / Dsum row
    uint32_t row_bytes;        // global bytes between consecutive rows of one head
    int Hq, w;

    // rows [r0, r0 + 64) of head h into stage st (rows past the sequence read as zero)
    __device__ __forceinline__ void issue(int st, int r0, int h) const
    {
        const uint32_t soff = (uint32_t)r0 * row_bytes + (uint32_t)h * kRowBytes;
        const uint32_t wq = lds_addr(q_ring[st].q) + w * (kQLoads * 1024);
        const uint32_t wg = lds_addr(q_ring[st].g) + w * (kQLoads * 1024);
#pragma unroll
        for (int p = 0; p < kQLoads; ++p) {
            dma16(wq + p * 1024, voff[p], qrs, soff);
            dma16(wg + p * 1024, voff[p], grs, soff);
        }
        const uint32_t soff4 = ((uint32_t)r0 * Hq + h) * 4;
        if (w == 0)
            dma4(lds_addr(q_ring[st].lse), loff, lrs, soff4);
        else if (w == 1)
            dma4(lds_addr(q_ring[st].dsum), loff, drs, soff4);
    }
};

// A 32-row block of a staged tile: its Q and dO rows, their LSE and Dsum, and its first query row.
struct Blk {
    const char *q, *g;
    const float *lse, *dsum;
    int row0;
    bool full; // every row of the block sees every key of the pair
};

// A operand of S / dP, k-step s: 16 B of row n of the block, dims 16 s + 8 J.
__device__ __forceinline__ bf16x8 rd_rows(const char *rows, uint32_t rowA, int s)
{
    return as_bf16x8(ld16(rows + (rowA ^ (32 * s))));
}

// A operand of dV^T / dK^T for 16-row half u and 32-dim block db of a block, by transposed reads:
// dims 32 db + lane % 32, k-slot 8 J + e <-> row 16 u + 8 (e/4) + 4 J + e%4.
__device__ __forceinline__ bf16x8 rd_cols(const char *rows, const uint32_t trA[2], int u, int db)
{
    const char *base = rows + 16 * u * kRowBytes;
    const uint2 lo = lds_read_tr(base + (trA[0] ^ (64 * db)));
    const uint2 hi = lds_read_tr(base + (trA[1] ^ (64 * db)));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}


// Per-lane constants of a dK / dV wave.
struct KvLane {
    uint32_t rowA;    // A-operand read offset (row n, chunk J)
    uint32_t trA[2];  // transposed-read offsets (16-row halves' lower and upper 8 rows)
    int J;
    int lo_row, span; // the rows that see the lane's key: [lo_row, lo_row + span)
    float sl;         // scale * log2(e)
};

// One k-loop of a pair wave (8 k-steps, operands read two k-steps ahead).  With X: x = rows * bop, the
// first product of a new block (S = Q K^T for the P wave, dP = dO V^T for the dS wave).  With Y:
// acc += cols * yop, the second product of an older block (dV^T += dO^T P, dK^T += Q^T dS).  With F:
// two elements per k-step of a block whose first product is done (fin): the P wave forms
// P = exp2(scale log2(e) S - lse2), zeroed where the row does not see the key; the dS wave forms
// dS = P (dP - Dsum) from that P (pin).  Register i of a block <-> row 8 (i/4) + 4 J + i%4 of the block
// and the lane's key; fout[j] packs registers 2j, 2j+1.
constexpr int kPairAhead = 2; // k-steps of LDS operands in flight in a pair wave

template <bool PW, bool X, bool Y, bool F>
__device__ __forceinline__ void pair_phase(const KvLane &L, const bf16x8 bop[8], f32x16 acc[4], const char *xrows,
                                           f32x16 &x, const char *ycols, const Packed &yop, const Blk &bf,
                                           const f32x16 &fin, const Packed &pin, Packed &fout)
{
    if (X) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            x[i] = 0.f;
    }
    // operands of k-steps k .. k + kPairAhead - 1 in flight (xq[j], yq[j] hold k-step k + j)
    bf16x8 xq[kPairAhead + 1], yq[kPairAhead + 1];
#pragma unroll
    for (int j = 0; j < kPairAhead; ++j) {
        if (X)
            xq[j] = rd_rows(xrows, L.rowA, j);
        if (Y)
            yq[j] = rd_cols(ycols, L.trA, j >> 2, j & 3);
    }
    const float *fv = PW ? bf.lse : bf.dsum;
    float4 v4;
    if (F)
        v4 = *reinterpret_cast<const float4 *>(fv + 4 * L.J);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int u = k >> 2, db = k & 3;
        if (k + kPairAhead < 8) {
            if (X)
                xq[kPairAhead] = rd_rows(xrows, L.rowA, k + kPairAhead);
            if (Y)
                yq[kPairAhead] = rd_cols(ycols, L.trA, (k + kPairAhead) >> 2, (k + kPairAhead) & 3);
        }
        float4 v4n = v4;
        if (F && (k & 1) && k < 7)
            v4n = *reinterpret_cast<const float4 *>(fv + 8 * ((k + 1) >> 1) + 4 * L.J);
        if (X)
            x = mfma32(xq[0], bop[k], x);
        if (F) {
            // registers 2k, 2k+1: rows 8 (k/2) + 4 J + 2 (k%2) + {0, 1}
            const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
            float o[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * k + e, r = i & 3;
                if (PW)
                    o[e] = exp2_fast(fmaf(fin[i], L.sl, -vv[r]));
                else
                    o[e] = (e ? bf16_hi(pin.h[u][k & 3]) : bf16_lo(pin.h[u][k & 3])) * (fin[i] - vv[r]);
            }
            fout.h[u][k & 3] = pack_bf16x2(o[0], o[1]);
            anchor(fout.h[u][k & 3]);
        }
        if (Y)
            acc[db] = mfma32(yq[0], __builtin_bit_cast(bf16x8, yop.h[u]), acc[db]);
        sched_fence();
#pragma unroll
        for (int j = 0; j < kPairAhead; ++j) {
            xq[j] = xq[j + 1];
            yq[j] = yq[j + 1];
        }
        if (k & 1)
            v4 = v4n;
    }
    // The P wave, on blocks that cross the causal diagonal or an end of the sequence: zero the entries
    // whose row does not see the lane's key (their values above may be anything, infinities and NaN
    // included, since rows past the sequence and keys past the diagonal were not kept out of the
    // exponentials).  The dS wave needs no mask: its P is zero there and dP - Dsum is finite (rows past
    // the sequence and keys past it load as zero).
    if (F && PW && !bf.full) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t m = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * k + e;
                const int row = bf.row0 + 8 * (i >> 2) + 4 * L.J + (i & 3);
                if ((uint32_t)(row - L.lo_row) < (uint32_t)L.span)
                    m |= 0xffffu << (16 * e);
            }
            fout.h[k >> 2][k & 3] &= m;
        }
    }
}

// The P wave's work on one staged tile (blocks b0, b1): S of b0, with dV^T += dO^T P of the previous
// tile's second block when there is one (First false; its P in pl, its dO rows in gl); S of b1 with P of
// b0; dV^T of b0 with P of b1 (into pl, for the next tile).  Each block's P goes to the exchange (xb) as
// soon as it is formed.  The previous tile's stage is still in LDS: it is overwritten two tiles later.
template <bool First>
__device__ __forceinline__ void p_wave_tile(const KvLane &L, const bf16x8 kop[8], f32x16 dv[4], const Blk &b0,
                                            const Blk &b1, const char *gl, Packed &pl, char *xb, int lane)
{
    f32x16 s0, s1;
    Packed p0;
    pair_phase<true, true, !First, false>(L, kop, dv, b0.q, s0, gl, pl, b0, s0, pl, pl);
    pair_phase<true, true, false, true>(L, kop, dv, b1.q, s1, nullptr, p0, b0, s0, p0, p0);
    xchg_store(xb, lane, p0);
    pair_phase<true, false, true, true>(L, kop, dv, nullptr, s1, b0.g, p0, b1, s1, pl, pl);
    xchg_store(xb + kXchgBlock, lane, pl);
}

// The dS wave's work on one staged tile T, one tile behind its P wave (P of T in xb), whose first
// block's dP (dn) was formed during the step before: dP of b1 with dS of b0; dK^T += Q^T dS of b0 with dS
// of b1; dK^T of b1 with dP of the next tile's first block nb into dn (nb is already in LDS: it is the P
// wave's tile of this step; after the last tile nb is any resident block and dn goes unused).
__device__ __forceinline__ void ds_wave_tile(const KvLane &L, const bf16x8 vop[8], f32x16 dk[4], const Blk &b0,
                                             const Blk &b1, const Blk &nb, f32x16 &dn, const char *xb, int lane)
{
    f32x16 d1;
    Packed p0, p1, t0, t1;
    xchg_load(xb, lane, p0);
    xchg_load(xb + kXchgBlock, lane, p1);
    pair_phase<false, true, false, true>(L, vop, dk, b1.g, d1, nullptr, t0, b0, dn, p0, t0);
    pair_phase<false, false, true, true>(L, vop, dk, nullptr, d1, b0.q, t0, b1, d1, p1, t1);
    pair_phase<false, true, true, false>(L, vop, dk, nb.g, dn, b1.q, t1, nb, d1, p1, t1);
}

// dK, dV of 128 keys of one (sequence, KV head), two waves per SIMD: 4 pairs of waves, pair p owning keys
// kb0 + 32 p .. +31.  The pair's P wave keeps K of its keys in registers (the B operand of S = Q K^T),
// forms P and accumulates dV^T = sum dO^T P; its dS wave keeps V (the B operand of dP = dO V^T), takes P
// from the P wave through LDS, forms dS and accumulates dK^T = sum Q^T dS.  The loop runs over the query
// heads of the group and, per head, over the 64-row query tiles that see any of the keys, last tile
// first, staged in a three-stage direct-to-LDS ring; the dS waves run one tile behind the P waves, so
// one barrier per tile publishes both the tile and the P of the tile before it.  Both waves of a pair
// work through a tile's two 32-row blocks in the same four phases (first product of block 0; of block 1
// with the elementwise step of block 0; second product of block 0 with the elementwise step of block 1;
// second product of block 1); the other wave of the SIMD fills the gaps.
__global__ __launch_bounds__(kKvThreads) void bwd_dkdv_kernel(BwdArgs a, int nkt, int nunits)
{
    // XCD-aware order: block i runs on XCD i % 8, which takes a contiguous run of units ordered (KV
    // head, sequence, key block): each XCD serves whole KV heads of every sequence (even load), and the
    // key blocks of one (sequence, KV head) are dispatched together.  Every key block walks its query
    // tiles from the sequence's last one backwards (all key blocks see the last rows, under the causal
    // mask too), so the key blocks running together read the same Q and dO tiles at about the same
    // time and all but the first read of each come from the XCD's L2.
    const int per = gridDim.x / kXcds;
    const int unit = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (unit >= nunits)
        return;
    const int g = unit / (nkt * a.B), rem = unit % (nkt * a.B);
    const int b = rem / nkt, kt = rem % nkt;
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
    const int kb0 = kt * kKeysPerWg;
    if (kb0 >= Lk)
        return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = w % kKvPairs;
    const bool pwave = w < kKvPairs; // waves p and p + 4 form pair p
    const int n = lane & 31, J = lane >> 5;
    const int kw = kb0 + kKeysPerPair * pair; // the pair's first key
    const int key = kw + n;                   // the lane's key (MFMA column)
    const int diag = Lk - Lq;

    KvLane L;
    L.J = J;
    L.lo_row = key >= Lk ? Lq : (a.causal ? key - diag : 0);
    L.span = max(0, Lq - L.lo_row);
    L.sl = a.scale_log2;
    // A operand: row n, dims 16 s + 8 J at chunk 2 s + J; transposed reads: 16-lane group G16, index j
    // addresses row 8 hf + 4 J + j/4 of a 16-row half, dims 32 db + 16 (G16 % 2) + 4 (j % 4)
    L.rowA = n * kRowBytes + 16 * (J ^ swz(n & 15));
    {
        const int G16 = lane >> 4, j = lane & 15;
        const int x = 2 * (G16 & 1) + ((j & 3) >> 1);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int r = 8 * hf + 4 * J + (j >> 2);
            L.trA[hf] = r * kRowBytes + 8 * (j & 1) + 16 * (x ^ swz(r));
        }
    }

    // K (P wave) or V (dS wave) as the B operand: lane (key n, J) holds dims 16 s + 8 J .. +8
    bf16x8 bop[8];
    {
        const uint16_t *src = static_cast<const uint16_t *>(pwave ? a.k : a.v);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (key < Lk)
                v = ld16(src + ((size_t)(k0 + key) * a.Hkv + g) * D + 16 * s + 8 * J);
            bop[s] = as_bf16x8(v);
        }
    }
    // dV^T (P wave) or dK^T (dS wave) [128 dims x 32 keys] in blocks db of 32 dims: register i <-> dim
    // 32 db + 8 (i/4) + 4 J + i%4
    f32x16 acc[4];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            acc[db][i] = 0.f;

    QLoader ld;
    {
        const uint32_t row_bytes = (uint32_t)a.Hq * kRowBytes;
        const uint32_t seq_bytes = (uint32_t)Lq * row_bytes; // rows past the sequence read as zero
        ld.qrs = make_rsrc(static_cast<const uint16_t *>(a.q) + (size_t)q0 * a.Hq * D, seq_bytes);
        ld.grs = make_rsrc(static_cast<const uint16_t *>(a.dout) + (size_t)q0 * a.Hq * D, seq_bytes);
        ld.lrs = make_rsrc(a.lse2 + (size_t)q0 * a.Hq, (uint32_t)Lq * a.Hq * 4);
        ld.drs = make_rsrc(a.dsum + (size_t)q0 * a.Hq, (uint32_t)Lq * a.Hq * 4);
        ld.row_bytes = row_bytes;
        ld.Hq = a.Hq;
        ld.w = w;
        ld.loff = (uint32_t)lane * a.Hq * 4;
#pragma unroll
        for (int p = 0; p < kQLoads; ++p) {
            const int row = 4 * (kQLoads * w + p) + (lane >> 4);
            ld.voff[p] = (uint32_t)row * row_bytes + 16 * ((lane & 15) ^ swz(row & 15));
        }
    }

    // tiles: for every query head of the group, the 64-row tiles from the first that sees key kb0
    const int qt_first = (a.causal ? max(0, kb0 - diag) : 0) / kQRows;
    const int nq = (Lq + kQRows - 1) / kQRows - qt_first;
    const int ntiles = nq > 0 ? a.G * nq : 0;
    // a tile's place: ring stage, first row, query head (advanced one tile at a time: per head, from
    // the last tile down to the first)
    struct Tile {
        int st, row0, h;
    };
    const int row_first = qt_first * kQRows, row_last = (qt_first + nq - 1) * kQRows;
    auto advance = [&](Tile t) {
        t.st = t.st == kQStages - 1 ? 0 : t.st + 1;
        t.row0 -= kQRows;
        if (t.row0 < row_first) {
            t.row0 = row_last;
            ++t.h;
        }
        return t;
    };
    auto blk = [&](const Tile &t, int rb) {
        Blk x;
        x.q = q_ring[t.st].q + rb * 32 * kRowBytes;
        x.g = q_ring[t.st].g + rb * 32 * kRowBytes;
        x.lse = q_ring[t.st].lse + 32 * rb;
        x.dsum = q_ring[t.st].dsum + 32 * rb;
        x.row0 = t.row0 + 32 * rb;
        x.full = x.row0 + 32 <= Lq && kw + kKeysPerPair <= Lk &&
                 (!a.causal || kw + kKeysPerPair - 1 - diag <= x.row0);
        return x;
    };

    if (ntiles > 0) {
        // step s: the P waves work on tile s, the dS waves on tile s - 1.  At its barrier tile s is in LDS
        // and so is the P of tile s - 1, and every wave is done with tile s - 2 (stage and exchange).  Each
        // role runs its own loop (one set of registers for its accumulators); both pass ntiles + 1
        // barriers.
        Tile cur{0, row_last, g * a.G};
        ld.issue(cur.st, cur.row0, cur.h);
        auto sync = [&](int s, Tile &c) {
            wait_vmcnt<0>();
            wait_lds();
            barrier();
            if (s + 1 < ntiles) {
                c = advance(c);
                ld.issue(c.st, c.row0, c.h);
            }
        };
        if (pwave) {
            Packed pl; // P of the last tile's second block, whose dV^T product runs with the next tile
            const char *gl;
            {
                const Tile t = cur; // tile 0
                sync(0, cur);
                const Blk b0 = blk(t, 0), b1 = blk(t, 1);
                p_wave_tile<true>(L, bop, acc, b0, b1, nullptr, pl, p_xchg[0][pair], lane);
                gl = b1.g;
            }
            for (int s = 1; s < ntiles; ++s) {
                const Tile t = cur; // tile s
                sync(s, cur);
                const Blk b0 = blk(t, 0), b1 = blk(t, 1);
                p_wave_tile<false>(L, bop, acc, b0, b1, gl, pl, p_xchg[s & 1][pair], lane);
                gl = b1.g;
            }
            sync(ntiles, cur);
            f32x16 unused;
            pair_phase<true, false, true, false>(L, bop, acc, nullptr, unused, gl, pl, blk(cur, 0), unused, pl, pl);
        } else {
            Tile prev = cur;
            f32x16 dn; // dP of the first block of the next tile
            sync(0, cur);
            {
                Packed none;
                pair_phase<false, true, false, false>(L, bop, acc, blk(prev, 0).g, dn, nullptr, none, blk(prev, 0),
                                                      dn, none, none);
            }
            for (int s = 1; s <= ntiles; ++s) {
                const Tile t = prev; // tile s - 1
                prev = cur;          // tile s (when s < ntiles)
                sync(s, cur);
                ds_wave_tile(L, bop, acc, blk(t, 0), blk(t, 1), blk(prev, 0), dn, p_xchg[(s - 1) & 1][pair], lane);
            }
        }
    }

    if (key >= Lk)
        return;
    // the P wave writes dV, the dS wave dK = scale dS^T Q
    const float f = pwave ? 1.f : a.scale;
    uint16_t *dst = static_cast<uint16_t *>(pwave ? a.dv : a.dk) + ((size_t)(k0 + key) * a.Hkv + g) * D + 4 * J;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint2 pk;
            pk.x = pack_bf16x2(acc[db][4 * r] * f, acc[db][4 * r + 1] * f);
            pk.y = pack_bf16x2(acc[db][4 * r + 2] * f, acc[db][4 * r + 3] * f);
            *reinterpret_cast<uint2 *>(dst + 32 * db + 8 * r) = pk;
        }
}

// ------------------------------------------------------------------ dQ

constexpr int kDqGroups = 4;             // 32-row groups per workgroup
constexpr int kDqWaves = 3 * kDqGroups;  // three waves per SIMD: an S, a D and a Q wave per group
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kKTile = 32;                      // keys per staged tile
constexpr int kKTileBytes = kKTile * kRowBytes; // 8 KB
constexpr int kKLoaders = 8;                    // waves that issue a tile's loads: one 1-KB chunk of K and of V each
constexpr int kKStages = 4;
static_assert(kKTileBytes == kKLoaders * 1024, "one K and one V chunk per loading wave");

// One stage of the K / V ring (swizzled rows).
struct alignas(1024) KStage {
    char k[kKTileBytes];
    char v[kKTileBytes];
};
__shared__ KStage k_ring[kKStages];

// P^T (S wave -> D wave) and dS^T (D wave -> Q wave) of a group's 32-key tile, in the layout of p_xchg;
// two tiles in flight each.
__shared__ __attribute__((aligned(1024))) char pt_xchg[2][kDqGroups][kXchgBlock];
__shared__ __attribute__((aligned(1024))) char dst_xchg[2][kDqGroups][kXchgBlock];

struct KLoader {
    i32x4 krs, vrs;      // buffer resources of K, V (the sequence's rows of one KV head)
    uint32_t voff;       // lane's byte offset inside a tile of rows (the wave's 4-row block)
    uint32_t tile_bytes; // global bytes between consecutive tiles
    int w;

    // keys [32 t, 32 t + 32) into stage st (keys past the sequence read as zero); waves 0 .. 7
    __device__ __forceinline__ void issue(int st, int t) const
    {
        if (w >= kKLoaders)
            return;
        const uint32_t soff = (uint32_t)t * tile_bytes;
        dma16(lds_addr(k_ring[st].k) + w * 1024, voff, krs, soff);
        dma16(lds_addr(k_ring[st].v) + w * 1024, voff, vrs, soff);
    }
};

// A 32-key tile: its K and V rows and its first key.
struct KBlk {
    const char *k, *v;
    int kb;
    bool full; // every row of the group sees every key of the tile
};

// Per-lane constants of a dQ wave (lane: query row n of the group's 32, MFMA column).
struct QLane {
    uint32_t rowA, trA[2];
    int J;
    int kend_row;     // the lane's row sees keys [0, kend_row) (0 for rows past the sequence)
    float sl, lse2, dsum;
};

// One k-loop of a dQ wave (8 k-steps, operands read two k-steps ahead).  With X: x = rows * bop, the first
// product of a tile (S^T = K Q^T for the S wave, dP^T = V dO^T for the D wave).  With Y: acc += cols * yop,
// dQ^T += K^T dS^T (Q wave).  With F: the element-wise step on a tile whose first product is done (fin):
// the S wave forms P^T = exp2(scale log2(e) S^T - lse2), zeroed where the row does not see the key; the
// D wave forms dS^T = P^T (dP^T - Dsum) from that P^T (pin).  Register i of a tile <-> key 8 (i/4) + 4 J
// + i%4 of the tile and the lane's row.
template <bool PW, bool X, bool Y, bool F>
__device__ __forceinline__ void dq_phase(const QLane &L, const bf16x8 bop[8], f32x16 acc[4], const char *xrows,
                                         f32x16 &x, const char *ycols, const Packed &yop, const KBlk &bf,
                                         const f32x16 &fin, const Packed &pin, Packed &fout)
{
    if (X) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
            x[i] = 0.f;
    }
    bf16x8 xq[3], yq[3]; // operands of k-steps k, k + 1, k + 2
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        if (X)
            xq[j] = rd_rows(xrows, L.rowA, j);
        if (Y)
            yq[j] = rd_cols(ycols, L.trA, 0, j);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int u = k >> 2, db = k & 3;
        if (k + 2 < 8) {
            if (X)
                xq[2] = rd_rows(xrows, L.rowA, k + 2);
            if (Y)
                yq[2] = rd_cols(ycols, L.trA, (k + 2) >> 2, (k + 2) & 3);
        }
        if (X)
            x = mfma32(xq[0], bop[k], x);
        if (F) {
            float o[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * k + e;
                if (PW)
                    o[e] = exp2_fast(fmaf(fin[i], L.sl, -L.lse2));
                else
                    o[e] = (e ? bf16_hi(pin.h[u][k & 3]) : bf16_lo(pin.h[u][k & 3])) * (fin[i] - L.dsum);
            }
            fout.h[u][k & 3] = pack_bf16x2(o[0], o[1]);
            anchor(fout.h[u][k & 3]);
        }
        if (Y)
            acc[db] = mfma32(yq[0], __builtin_bit_cast(bf16x8, yop.h[u]), acc[db]);
        sched_fence();
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            xq[j] = xq[j + 1];
            yq[j] = yq[j + 1];
        }
    }
    // The S wave, on tiles that cross the causal diagonal or an end of the sequence: zero the entries
    // whose row does not see the key (their exponentials may be anything).  The D wave needs no mask: its
    // P^T is zero there and dP^T - Dsum is finite (keys and rows past the sequence load as zero).
    if (F && PW && !bf.full) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t m = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * k + e;
                if (bf.kb + 8 * (i >> 2) + 4 * L.J + (i & 3) < L.kend_row)
                    m |= 0xffffu << (16 * e);
            }
            fout.h[k >> 2][k & 3] &= m;
        }
    }
}

// dQ, three waves per SIMD: the forward's work split over 4 groups of 32 rows (NH query heads of one KV
// head's group times 4 / NH blocks of 32 rows; the group's heads share each K / V tile in LDS), XCD-aware
// order.  Each group has three waves, on one SIMD: the S wave keeps Q^T of the rows in registers (the B
// operand of S^T = K Q^T) and forms P^T; the D wave keeps dO^T (the B operand of dP^T = V dO^T), takes
// P^T through LDS and forms dS^T; the Q wave takes dS^T through LDS and accumulates dQ^T += K^T dS^T (K^T
// by transposed LDS reads).  Each issues 8 MFMAs per 32-key tile.  K and V tiles stream through a
// four-stage direct-to-LDS ring; at step s the S waves work on tile s, the D waves on tile s - 1 and the
// Q waves on tile s - 2, so one barrier per tile publishes the tile, the P^T of the tile before it and the
// dS^T of the one before that.
__global__ __launch_bounds__(kDqThreads) void bwd_dq_kernel(BwdArgs a, int NH, int RB, int nqt, int nunits)
{
    const int per = gridDim.x / kXcds;
    const int unit = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (unit >= nunits)
        return;
    const int hchunks = a.G / NH;
    const int gh = unit / (a.B * nqt), rem = unit % (a.B * nqt);
    const int b = rem / nqt, qt = nqt - 1 - rem % nqt;
    const int g = gh / hchunks, hc = gh % hchunks;
    const int rows_wg = 32 * RB;
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
    const int m0 = qt * rows_wg;
    if (m0 >= Lq)
        return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = w % kDqGroups;
    const int role = w / kDqGroups; // 0: S wave, 1: D wave, 2: Q wave
    const int n = lane & 31, J = lane >> 5;
    const int h = g * a.G + hc * NH + (grp % NH);
    const int row_w = m0 + 32 * (grp / NH); // the group's first row
    const int qi = row_w + n;               // the lane's row (MFMA column)
    const bool row_ok = qi < Lq;
    const int diag = Lk - Lq;
    const int last_row = min(m0 + rows_wg, Lq) - 1;
    const int kend = a.causal ? max(0, min(Lk, last_row + 1 + diag)) : Lk;

    QLane L;
    L.J = J;
    L.kend_row = !row_ok ? 0 : (a.causal ? max(0, min(Lk, qi + 1 + diag)) : Lk);
    L.sl = a.scale_log2;
    L.lse2 = row_ok ? a.lse2[(size_t)(q0 + qi) * a.Hq + h] : 0.f;
    L.dsum = row_ok ? a.dsum[(size_t)(q0 + qi) * a.Hq + h] : 0.f;
    L.rowA = n * kRowBytes + 16 * (J ^ swz(n & 15));
    {
        const int G16 = lane >> 4, j = lane & 15;
        const int x = 2 * (G16 & 1) + ((j & 3) >> 1);
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            const int r = 8 * hf + 4 * J + (j >> 2);
            L.trA[hf] = r * kRowBytes + 8 * (j & 1) + 16 * (x ^ swz(r));
        }
    }

    // Q^T (S wave) or dO^T (D wave) as the B operand: lane (row n, J) holds dims 16 s + 8 J .. +8
    bf16x8 bop[8];
    if (role < 2) {
        const uint16_t *src = static_cast<const uint16_t *>(role == 0 ? a.q : a.dout);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row_ok)
                v = ld16(src + ((size_t)(q0 + qi) * a.Hq + h) * D + 16 * s + 8 * J);
            bop[s] = as_bf16x8(v);
        }
    }
    f32x16 dq[4]; // dQ^T [128 dims x 32 rows] (Q wave): block db, register i <-> dim 32 db + 8 (i/4) + 4 J + i%4
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            dq[db][i] = 0.f;

    KLoader ld;
    {
        const uint16_t *kg = static_cast<const uint16_t *>(a.k), *vg = static_cast<const uint16_t *>(a.v);
        const size_t head0 = ((size_t)k0 * a.Hkv + g) * D;
        const uint32_t row_bytes = (uint32_t)a.Hkv * kRowBytes;
        const uint32_t seq_bytes = Lk > 0 ? ((uint32_t)(Lk - 1) * a.Hkv + 1) * kRowBytes : 0;
        ld.krs = make_rsrc(kg + head0, seq_bytes);
        ld.vrs = make_rsrc(vg + head0, seq_bytes);
        ld.tile_bytes = kKTile * row_bytes;
        ld.w = w;
        const int row = 4 * w + (lane >> 4); // waves 0 .. 7: rows 4 w .. 4 w + 3 of the tile
        ld.voff = (uint32_t)row * row_bytes + 16 * ((lane & 15) ^ swz(row & 15));
    }

    const int ntiles = (kend + kKTile - 1) / kKTile;
    auto blk = [&](int t) {
        const int st = t % kKStages;
        KBlk x;
        x.k = k_ring[st].k;
        x.v = k_ring[st].v;
        x.kb = t * kKTile;
        x.full = row_w + 32 <= Lq && x.kb + 32 <= Lk && (!a.causal || x.kb + 31 <= row_w + diag);
        return x;
    };
    // step s: S waves on tile s, D waves on tile s - 1, Q waves on tile s - 2.  At its barrier tile s is in
    // LDS, so are the P^T of tile s - 1 and the dS^T of tile s - 2, and every wave is done with tile s - 3
    // (stage) and with the exchange buffers of two tiles back.  Each role runs its own loop; all pass
    // ntiles + 2 barriers.
    auto sync = [&](int s) {
        wait_vmcnt<0>();
        wait_lds();
        barrier();
        if (s + 1 < ntiles)
            ld.issue((s + 1) % kKStages, s + 1);
    };

    if (ntiles > 0) {
        ld.issue(0, 0);
        Packed none;
        f32x16 fnone;
        if (role == 0) {
            for (int s = 0; s < ntiles; ++s) {
                sync(s);
                const KBlk bt = blk(s);
                f32x16 st;
                Packed p;
                dq_phase<true, true, false, false>(L, bop, dq, bt.k, st, nullptr, none, bt, st, none, none);
                dq_phase<true, false, false, true>(L, bop, dq, nullptr, fnone, nullptr, none, bt, st, none, p);
                xchg_store(pt_xchg[s & 1][grp], lane, p);
            }
            sync(ntiles);
            sync(ntiles + 1);
        } else if (role == 1) {
            sync(0);
            for (int s = 1; s <= ntiles; ++s) {
                sync(s);
                const KBlk bt = blk(s - 1);
                f32x16 dp;
                Packed p, ds;
                xchg_load(pt_xchg[(s - 1) & 1][grp], lane, p);
                dq_phase<false, true, false, false>(L, bop, dq, bt.v, dp, nullptr, none, bt, dp, none, none);
                dq_phase<false, false, false, true>(L, bop, dq, nullptr, fnone, nullptr, none, bt, dp, p, ds);
                xchg_store(dst_xchg[(s - 1) & 1][grp], lane, ds);
            }
            sync(ntiles + 1);
        } else {
            sync(0);
            sync(1);
            for (int s = 2; s <= ntiles + 1; ++s) {
                sync(s);
                const KBlk bt = blk(s - 2);
                Packed ds;
                xchg_load(dst_xchg[(s - 2) & 1][grp], lane, ds);
                dq_phase<false, false, true, false>(L, bop, dq, nullptr, fnone, bt.k, ds, bt, fnone, none, none);
            }
        }
    }

    if (role != 2 || !row_ok)
        return;
    uint16_t *dqg = static_cast<uint16_t *>(a.dq) + ((size_t)(q0 + qi) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint2 pk;
            pk.x = pack_bf16x2(dq[db][4 * r] * a.scale, dq[db][4 * r + 1] * a.scale);
            pk.y = pack_bf16x2(dq[db][4 * r + 2] * a.scale, dq[db][4 * r + 3] * a.scale);
            *reinterpret_cast<uint2 *>(dqg + 32 * db + 8 * r + 4 * J) = pk;
        }
}

} // namespace

static int heads_per_wg_bwd(int G)
{
    int nh = 1;
    while (nh < kDqGroups && G % (2 * nh) == 0)
        nh *= 2;
    return nh;
}

// The backward's side stream of one device (default priority, non-blocking) and its fork / join events,
// created on the first call for that device that is not under stream capture and kept until the
// process ends.
struct SideStream {
    std::mutex mu;
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxSideDevices = 64;

// The side stream of the device `stream` runs on, or null (then the kernels run on `stream` alone): when
// the device is not the calling thread's current one, when `stream` is being captured before the side
// stream exists, or when creating it fails.
static SideStream *side_stream(hipStream_t stream)
{
    static SideStream side[kMaxSideDevices];
    static std::mutex create_mu;
    int cur = -1;
    hipDevice_t dev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(stream, &dev) != hipSuccess || dev != cur ||
        dev < 0 || dev >= kMaxSideDevices)
        return nullptr;
    SideStream &ss = side[dev];
    std::lock_guard<std::mutex> lock(create_mu);
    if (!ss.s) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone)
            return nullptr;
        hipStream_t s = nullptr;
        hipEvent_t f = nullptr, j = nullptr;
        if (hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess ||
            hipEventCreateWithFlags(&f, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&j, hipEventDisableTiming) != hipSuccess) {
            if (j)
                (void)hipEventDestroy(j);
            if (f)
                (void)hipEventDestroy(f);
            if (s)
                (void)hipStreamDestroy(s);
            return nullptr;
        }
        ss.fork = f;
        ss.join = j;
        ss.s = s;
    }
    return &ss;
}

hipError_t launch_prefill_bwd(const BwdArgs &a, hipStream_t stream)
{
    const long slots = (long)a.B * a.max_q * a.Hq; // an upper bound of the T * Hq rows
    if (slots > 0x7fffffffL)
        return hipErrorInvalidValue;
    if (slots > 0)
        ATTN_LAUNCH(bwd_prep_kernel, dim3((unsigned)std::min<long>((slots + 15) / 16, 4096)), dim3(256), 0, stream,
                    a);
    const int nkt = (a.max_k + kKeysPerWg - 1) / kKeysPerWg;
    const long units_kv = (long)a.Hkv * a.B * nkt;
    const long blocks_kv = (units_kv + kXcds - 1) / kXcds * kXcds;
    const int NH = heads_per_wg_bwd(a.G), RB = kDqGroups / NH;
    const int nqt = (a.max_q + 32 * RB - 1) / (32 * RB);
    const long units_q = (long)a.Hkv * (a.G / NH) * a.B * nqt;
    const long blocks_q = (units_q + kXcds - 1) / kXcds * kXcds;
    if (blocks_kv > 0x7fffffff || blocks_q > 0x7fffffff)
        return hipErrorInvalidValue;
    // dK/dV and dQ are independent once the prep kernel is done: dQ runs on a side stream of the device,
    // forked from `stream` after the prep kernel and joined back after it, so each kernel's last
    // workgroups share the GPU with the other's (same-process A/B on the prefill shapes: 3.25 -> 3.15 ms)
    SideStream *ss = units_kv > 0 && units_q > 0 ? side_stream(stream) : nullptr;
    if (ss) {
        std::lock_guard<std::mutex> lock(ss->mu); // the fork / join events are shared by the device's callers
        hipError_t e = hipEventRecord(ss->fork, stream);
        if (e == hipSuccess)
            e = hipStreamWaitEvent(ss->s, ss->fork, 0);
        if (e != hipSuccess)
            return e;
        ATTN_LAUNCH(bwd_dq_kernel, dim3((unsigned)blocks_q), dim3(kDqThreads), 0, ss->s, a, NH, RB, nqt,
                    (int)units_q);
        ATTN_LAUNCH(bwd_dkdv_kernel, dim3((unsigned)blocks_kv), dim3(kKvThreads), 0, stream, a, nkt, (int)units_kv);
        e = hipEventRecord(ss->join, ss->s);
        if (e == hipSuccess)
            e = hipStreamWaitEvent(stream, ss->join, 0);
        if (e != hipSuccess)
            return e;
        return hipGetLastError();
    }
    if (units_kv > 0)
        ATTN_LAUNCH(bwd_dkdv_kernel, dim3((unsigned)blocks_kv), dim3(kKvThreads), 0, stream, a, nkt,
                           (int)units_kv);
    if (units_q > 0)
        ATTN_LAUNCH(bwd_dq_kernel, dim3((unsigned)blocks_q), dim3(kDqThreads), 0, stream, a, NH, RB, nqt,
                           (int)units_q);
    return hipGetLastError();
}

} // namespace attn
