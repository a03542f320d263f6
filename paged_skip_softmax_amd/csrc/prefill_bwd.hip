// Backward of the dense bf16 varlen prefill (head dim 128) for gfx950: dQ, dK, dV from Q, K, V, O, the
// output gradient dO and the forward's log-sum-exp.  The Triton kernel of "Model-Optimizer: Add Triton
// unified attention kernel with HuggingFace integration" (summary) has an autograd backward beside its
// forward; the gradients are those of the masked-softmax definition:
//   P = exp(scale Q K^T - lse),  dP = dO V^T,  Dsum = rowsum(dO * O),  dS = P * (dP - Dsum)
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K         (dK, dV summed over a KV head's group)
//
// Three kernels, no atomics:
//  * bwd_prep: Dsum and lse * log2(e) per (token, query head), fp32, into the caller's workspace.
//  * bwd_dkdv: a workgroup of 4 waves owns 64 keys of one (sequence, KV head), 16 keys per wave, whose
//    K and V stay in registers as MFMA B operands; it walks every query tile of 32 rows that sees any
//    of its keys, for every query head of the group.  The workgroup stages each Q and dO tile in LDS
//    once for its 4 waves (XOR-swizzled 16-byte chunks); per tile a wave computes, with 16x16x32 MFMAs,
//      S = Q K^T, dP = dO V^T           [32 rows x 16 keys]   (A operands: 16-byte LDS reads)
//      dV^T += dO^T P, dK^T += Q^T dS   [128 dims x 16 keys]  (A operands: transposed LDS reads)
//    so the key order inside the row contraction follows the S register layout and P, dS feed the
//    MFMA B operand straight from registers.
//  * bwd_dq: the forward's work split (4 waves, one query head and 32 rows each, the heads of a group
//    sharing K/V tiles in LDS); Q^T and dO^T stay in registers as B operands; per 32-key tile
//      S^T = K Q^T, dP^T = V dO^T   (32x32x16 MFMAs)
//      dQ^T += K^T dS^T             (K^T by transposed LDS reads)
#include "kcommon.h"
#include "launch.h"
#include "lds_dma.h"

namespace attn {
namespace {

constexpr int D = 128;
constexpr int kRowBytes = D * 2; // one bf16 row of 128 dims

// Byte offset of 16-byte chunk c of row r in a swizzled tile.
__device__ __forceinline__ uint32_t chunk_off(int r, int c) { return (uint32_t)(r * kRowBytes + 16 * (c ^ swz(r & 15))); }

// Copies rows [r0, r0 + nrows) of a [tokens, H, D] bf16 tensor (head h, rows past `valid` zero) into a
// swizzled LDS tile, cooperatively over the workgroup's threads.
__device__ __forceinline__ void stage_rows(char *tile, const uint16_t *src, size_t token0, int H, int h, int nrows,
                                           int valid, int tid, int nthreads)
{
    for (int idx = tid; idx < nrows * 16; idx += nthreads) {
        const int r = idx >> 4, c = idx & 15;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < valid)
            v = ld16(src + ((token0 + r) * H + h) * D + 8 * c);
        st16(tile + chunk_off(r, c), v);
    }
}

// ------------------------------------------------------------------ Dsum and lse in log2 units

__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a)
{
    // 16 lanes per (sequence, row, query head) slot of the padded [B, max_q, Hq] grid, 8 dims each
    const int slot = blockIdx.x * 16 + (threadIdx.x >> 4), c = threadIdx.x & 15;
    const int per_seq = a.max_q * a.Hq;
    const int b = slot / per_seq, i = (slot % per_seq) / a.Hq, h = slot % a.Hq;
    bool live = b < a.B;
    size_t row = 0;
    if (live) {
        const int q0 = a.cu_q[b];
        live = i < a.cu_q[b + 1] - q0;
        row = (size_t)(q0 + i) * a.Hq + h;
    }
    float s = 0.f;
    if (live) {
        const uint16_t *o = static_cast<const uint16_t *>(a.o), *dout = static_cast<const uint16_t *>(a.dout);
        const uint4 x = ld16(o + row * D + 8 * c), g = ld16(dout + row * D + 8 * c);
        const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            s = fmaf(bf16_lo(xw[e]), bf16_lo(gw[e]), s);
            s = fmaf(bf16_hi(xw[e]), bf16_hi(gw[e]), s);
        }
    }
    s += __shfl_xor(s, 8);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 1);
    if (live && c == 0)
        a.dsum[row] = s;
    if (live && c == 1)
        a.lse2[row] = a.lse[row] * kLog2e;
}

// ------------------------------------------------------------------ dK, dV

constexpr int kXcds = 8;
constexpr int kKvWaves = 4;
constexpr int kKvThreads = 64 * kKvWaves;
constexpr int kKeysPerWave = 32;
constexpr int kKeysPerWg = kKvWaves * kKeysPerWave; // 128
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
    bool full; // every row of the block sees every key of the wave
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

__device__ __forceinline__ bf16x8 half_op(const uint32_t x[8], int u)
{
    return as_bf16x8(make_uint4(x[4 * u], x[4 * u + 1], x[4 * u + 2], x[4 * u + 3]));
}

// Per-lane constants of the dK / dV wave.
struct KvLane {
    uint32_t rowA;    // A-operand read offset (row n, chunk J)
    uint32_t trA[2];  // transposed-read offsets (16-row halves' lower and upper 8 rows)
    int J;
    int lo_row, span; // the rows that see the lane's key: [lo_row, lo_row + span)
    float sl;         // scale * log2(e)
};

// One pipeline step of a wave over 32-row blocks: with C, dV^T += dO^T P and dK^T += Q^T dS of an
// older block (bc; its packed P and dS in pkc, skc); with S, S = Q K^T and dP = dO V^T of a new block
// (bs) into sc, dp; with P, P = exp(scale S - lse) and dS = P (dP - Dsum) of the block in between (bp;
// its scores scp, dpp) into pkn, skn, zero where the row does not see the key.  The 8 k-steps issue up to 4 MFMAs each, operands read two
// k-steps ahead, and two of the 16 P / dS elements are placed between the MFMAs of each k-step.
// Register i of a score block <-> row 8 (i/4) + 4 J + i%4 of the block; pk[j] packs registers 2j, 2j+1.
template <bool C, bool S, bool P>
__device__ __forceinline__ void kv_step(const KvLane &L, const bf16x8 kop[8], const bf16x8 vop[8], f32x16 dk[4],
                                        f32x16 dv[4], const Blk &bc, const uint32_t pkc[8], const uint32_t skc[8],
                                        const Blk &bs, f32x16 &sc, f32x16 &dp, const Blk &bp, const f32x16 &scp,
                                        const f32x16 &dpp, uint32_t pkn[8], uint32_t skn[8])
{
    if (S) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            sc[i] = 0.f;
            dp[i] = 0.f;
        }
    }
    bf16x8 cg0, cq0, cg1, cq1, aq0, ag0, aq1, ag1;
    if (C) {
        cg0 = rd_cols(bc.g, L.trA, 0, 0);
        cq0 = rd_cols(bc.q, L.trA, 0, 0);
        cg1 = rd_cols(bc.g, L.trA, 0, 1);
        cq1 = rd_cols(bc.q, L.trA, 0, 1);
    }
    if (S) {
        aq0 = rd_rows(bs.q, L.rowA, 0);
        ag0 = rd_rows(bs.g, L.rowA, 0);
        aq1 = rd_rows(bs.q, L.rowA, 1);
        ag1 = rd_rows(bs.g, L.rowA, 1);
    }
    float4 l4, d4;
    if (P) {
        l4 = *reinterpret_cast<const float4 *>(bp.lse + 4 * L.J);
        d4 = *reinterpret_cast<const float4 *>(bp.dsum + 4 * L.J);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int u = k >> 2, db = k & 3;
        bf16x8 cg2 = cg0, cq2 = cq0, aq2 = aq0, ag2 = ag0;
        if (k + 2 < 8) {
            if (C) {
                cg2 = rd_cols(bc.g, L.trA, (k + 2) >> 2, (k + 2) & 3);
                cq2 = rd_cols(bc.q, L.trA, (k + 2) >> 2, (k + 2) & 3);
            }
            if (S) {
                aq2 = rd_rows(bs.q, L.rowA, k + 2);
                ag2 = rd_rows(bs.g, L.rowA, k + 2);
            }
        }
        float4 l4n = l4, d4n = d4;
        if (P && (k & 1) && k < 7) {
            const int i4 = (k + 1) >> 1;
            l4n = *reinterpret_cast<const float4 *>(bp.lse + 8 * i4 + 4 * L.J);
            d4n = *reinterpret_cast<const float4 *>(bp.dsum + 8 * i4 + 4 * L.J);
        }
        if (C)
            dv[db] = mfma32(cg0, half_op(pkc, u), dv[db]);
        if (S)
            sc = mfma32(aq0, kop[k], sc);
        if (P) {
            // registers 2k, 2k+1: rows 8 (k/2) + 4 J + 2 (k%2) + {0, 1}
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dsv[4] = {d4.x, d4.y, d4.z, d4.w};
            float p[2], ds[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * k + e, r = i & 3;
                p[e] = exp2_fast(fmaf(scp[i], L.sl, -lv[r]));
                ds[e] = p[e] * (dpp[i] - dsv[r]);
            }
            pkn[k] = pack_bf16x2(p[0], p[1]);
            skn[k] = pack_bf16x2(ds[0], ds[1]);
            anchor(pkn[k]);
            anchor(skn[k]);
        }
        if (C)
            dk[db] = mfma32(cq0, half_op(skc, u), dk[db]);
        if (S)
            dp = mfma32(ag0, vop[k], dp);
        sched_fence();
        cg0 = cg1;
        cq0 = cq1;
        cg1 = cg2;
        cq1 = cq2;
        aq0 = aq1;
        ag0 = ag1;
        aq1 = aq2;
        ag1 = ag2;
        if (k & 1) {
            l4 = l4n;
            d4 = d4n;
        }
    }
    // Blocks that cross the causal diagonal or an end of the sequence: zero the entries whose row does
    // not see the lane's key (their values above may be anything, infinities and NaN included, since
    // rows past the sequence and keys past the diagonal were not kept out of the exponentials).
    if (P && !bp.full) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t m = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * k + e;
                const int row = bp.row0 + 8 * (i >> 2) + 4 * L.J + (i & 3);
                if ((uint32_t)(row - L.lo_row) < (uint32_t)L.span)
                    m |= 0xffffu << (16 * e);
            }
            pkn[k] &= m;
            skn[k] &= m;
        }
    }
}

// dK, dV of 128 keys of one (sequence, KV head): wave w owns keys kb0 + 32 w .. +31, whose K and V stay in
// registers as the B operands of S = Q K^T and dP = dO V^T.  The loop runs over the query heads of the
// group and, per head, over the 64-row query tiles that see any of the keys, staged in a three-stage
// direct-to-LDS ring.  A wave works in 32-row blocks through a three-deep software pipeline: while the
// MFMAs of S and dP [32 rows x 32 keys] of block j run (A operands: 16-B LDS reads of Q and dO rows),
// so do those of dV^T += dO^T P and dK^T += Q^T dS [128 dims x 32 keys] of block j-2 (A operands:
// transposed LDS reads), and P and dS of block j-1 are computed between them.  P and dS feed the B
// operand from registers in the S register order.
__global__ __launch_bounds__(kKvThreads) void bwd_dkdv_kernel(BwdArgs a, int nkt, int nunits)
{
    // XCD-aware order: block i runs on XCD i % 8, which takes a contiguous run of units ordered (KV
    // head, key block, sequence): each XCD serves whole KV heads of every sequence (even load), and
    // starts with the key blocks that see the most query rows (the first ones, under the causal mask);
    // the key blocks of one sequence that run at the same time stream the same Q and dO tiles through
    // the XCD's L2
    const int per = gridDim.x / kXcds;
    const int unit = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (unit >= nunits)
        return;
    const int g = unit / (nkt * a.B), rem = unit % (nkt * a.B);
    const int kt = rem / a.B, b = rem % a.B;
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
    const int kb0 = kt * kKeysPerWg;
    if (kb0 >= Lk)
        return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, J = lane >> 5;
    const int kw = kb0 + kKeysPerWave * w; // the wave's first key
    const int key = kw + n;                // the lane's key (MFMA column)
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

    // K and V as B operands: lane (key n, J) holds dims 16 s + 8 J .. +8
    bf16x8 kop[8], vop[8];
    {
        const uint16_t *kg = static_cast<const uint16_t *>(a.k), *vg = static_cast<const uint16_t *>(a.v);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
            if (key < Lk) {
                const size_t off = ((size_t)(k0 + key) * a.Hkv + g) * D + 16 * s + 8 * J;
                kv = ld16(kg + off);
                vv = ld16(vg + off);
            }
            kop[s] = as_bf16x8(kv);
            vop[s] = as_bf16x8(vv);
        }
    }
    f32x16 dk[4], dv[4]; // [128 dims x 32 keys] in blocks db of 32 dims: register i <-> dim 32 db + 8 (i/4) + 4 J + i%4
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            dk[db][i] = 0.f;
            dv[db][i] = 0.f;
        }

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
    // a tile's place: ring stage, first row, query head (advanced one tile at a time)
    struct Tile {
        int st, row0, h;
    };
    const int row_first = qt_first * kQRows, row_end = (qt_first + nq) * kQRows;
    auto advance = [&](Tile t) {
        t.st = t.st == kQStages - 1 ? 0 : t.st + 1;
        t.row0 += kQRows;
        if (t.row0 == row_end) {
            t.row0 = row_first;
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
        x.full = x.row0 + 32 <= Lq && kw + kKeysPerWave <= Lk &&
                 (!a.causal || kw + kKeysPerWave - 1 - diag <= x.row0);
        return x;
    };
    // tile t (in `cur`) was loaded one tile ahead; its stage is read until the step that finishes its
    // blocks, two tiles later
    auto next_tile = [&](const Tile &cur, int t) {
        wait_vmcnt<0>();
        barrier(); // tile t is in LDS for every wave; every wave is done with tile t - 2
        if (t + 1 < ntiles) {
            const Tile nx = advance(cur);
            ld.issue(nx.st, nx.row0, nx.h);
        }
    };

    if (ntiles > 0) {
        f32x16 sc, dp, scp, dpp;
        uint32_t pka[8], ska[8], pkb[8], skb[8];
        Tile prev{0, row_first, g * a.G};
        ld.issue(prev.st, prev.row0, prev.h);
        // steps 0 and 1: S of blocks 0, 1; P of block 0
        next_tile(prev, 0);
        {
            const Blk b0 = blk(prev, 0), b1 = blk(prev, 1);
            kv_step<false, true, false>(L, kop, vop, dk, dv, b0, pka, ska, b0, scp, dpp, b0, sc, dp, pkb, skb);
            kv_step<false, true, true>(L, kop, vop, dk, dv, b0, pka, ska, b1, sc, dp, b0, scp, dpp, pkb, skb);
        }
        // tile t: step 2t runs C of block 2t-2, S of block 2t, P of block 2t-1; step 2t+1 one block later.
        // At its start pkb/skb hold P, dS of block 2t-2 and sc, dp the scores of block 2t-1.
        for (int t = 1; t < ntiles; ++t) {
            const Tile cur = advance(prev);
            next_tile(cur, t);
            const Blk bm2 = blk(prev, 0), bm1 = blk(prev, 1), bj = blk(cur, 0), bj1 = blk(cur, 1);
            kv_step<true, true, true>(L, kop, vop, dk, dv, bm2, pkb, skb, bj, scp, dpp, bm1, sc, dp, pka, ska);
            kv_step<true, true, true>(L, kop, vop, dk, dv, bm1, pka, ska, bj1, sc, dp, bj, scp, dpp, pkb, skb);
            prev = cur;
        }
        // the last two steps: C of the last two blocks; P of the last block
        {
            const Blk bm2 = blk(prev, 0), bm1 = blk(prev, 1);
            kv_step<true, false, true>(L, kop, vop, dk, dv, bm2, pkb, skb, bm2, scp, dpp, bm1, sc, dp, pka, ska);
            kv_step<true, false, false>(L, kop, vop, dk, dv, bm1, pka, ska, bm1, scp, dpp, bm1, sc, dp, pkb, skb);
        }
    }

    if (key >= Lk)
        return;
    uint16_t *dkg = static_cast<uint16_t *>(a.dk) + ((size_t)(k0 + key) * a.Hkv + g) * D + 4 * J;
    uint16_t *dvg = static_cast<uint16_t *>(a.dv) + ((size_t)(k0 + key) * a.Hkv + g) * D + 4 * J;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint2 pk, pv;
            pk.x = pack_bf16x2(dk[db][4 * r] * a.scale, dk[db][4 * r + 1] * a.scale);
            pk.y = pack_bf16x2(dk[db][4 * r + 2] * a.scale, dk[db][4 * r + 3] * a.scale);
            pv.x = pack_bf16x2(dv[db][4 * r], dv[db][4 * r + 1]);
            pv.y = pack_bf16x2(dv[db][4 * r + 2], dv[db][4 * r + 3]);
            *reinterpret_cast<uint2 *>(dkg + 32 * db + 8 * r) = pk;
            *reinterpret_cast<uint2 *>(dvg + 32 * db + 8 * r) = pv;
        }
}

// ------------------------------------------------------------------ dQ

constexpr int kDqWaves = 4;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kKTile = 64;                            // keys per staged tile
constexpr int kKTileBytes = kKTile * kRowBytes;       // 16 KB
constexpr int kKLoads = kKTileBytes / 1024 / kDqWaves; // 1-KB direct-to-LDS loads per wave per tile
constexpr int kKStages = 3;

// One stage of the K / V ring (swizzled rows).
struct alignas(1024) KStage {
    char k[kKTileBytes];
    char v[kKTileBytes];
};
__shared__ KStage k_ring[kKStages];

struct KLoader {
    i32x4 krs, vrs;          // buffer resources of K, V (the sequence's rows of one KV head)
    uint32_t voff[kKLoads];  // lane's byte offsets inside a tile of rows (4-row blocks of the wave)
    uint32_t tile_bytes;     // global bytes between consecutive tiles
    int w;

    // keys [64 t, 64 t + 64) into stage st (keys past the sequence read as zero)
    __device__ __forceinline__ void issue(int st, int t) const
    {
        const uint32_t soff = (uint32_t)t * tile_bytes;
        const uint32_t wk = lds_addr(k_ring[st].k) + w * (kKLoads * 1024);
        const uint32_t wv = lds_addr(k_ring[st].v) + w * (kKLoads * 1024);
#pragma unroll
        for (int p = 0; p < kKLoads; ++p) {
            dma16(wk + p * 1024, voff[p], krs, soff);
            dma16(wv + p * 1024, voff[p], vrs, soff);
        }
    }
};

// A 32-key block of a staged tile: its K and V rows and its first key.
struct KBlk {
    const char *k, *v;
    int kb;
    bool full; // every row of the wave sees every key of the block
};

// Per-lane constants of the dQ wave.
struct QLane {
    uint32_t rowA, trA[2];
    int J;
    int kend_row;     // the lane's row sees keys [0, kend_row) (0 for rows past the sequence)
    float sl, lse2, dsum;
};

// One pipeline step of a dQ wave over 32-key blocks: with C, dQ^T += K^T dS^T of an older block (bc;
// its packed dS^T in skc); with S, S^T = K Q^T and dP^T = V dO^T of a new block (bs) into sc, dp; with
// P, dS^T = P (dP - Dsum), P = exp(scale S - lse), of the block in between (bp; its scores scp, dpp) into
// skn, zero where the row does not see the key.  Register i of a score block <-> key
// 8 (i/4) + 4 J + i%4 of the block; skn[j] packs registers 2j, 2j+1.
template <bool C, bool S, bool P>
__device__ __forceinline__ void q_step(const QLane &L, const bf16x8 qop[8], const bf16x8 gop[8], f32x16 dq[4],
                                       const KBlk &bc, const uint32_t skc[8], const KBlk &bs, f32x16 &sc, f32x16 &dp,
                                       const KBlk &bp, const f32x16 &scp, const f32x16 &dpp, uint32_t skn[8])
{
    if (S) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            sc[i] = 0.f;
            dp[i] = 0.f;
        }
    }
    bf16x8 ck0, ck1, ak0, av0, ak1, av1;
    if (C) {
        ck0 = rd_cols(bc.k, L.trA, 0, 0);
        ck1 = rd_cols(bc.k, L.trA, 0, 1);
    }
    if (S) {
        ak0 = rd_rows(bs.k, L.rowA, 0);
        av0 = rd_rows(bs.v, L.rowA, 0);
        ak1 = rd_rows(bs.k, L.rowA, 1);
        av1 = rd_rows(bs.v, L.rowA, 1);
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int u = k >> 2, db = k & 3;
        bf16x8 ck2 = ck0, ak2 = ak0, av2 = av0;
        if (k + 2 < 8) {
            if (C)
                ck2 = rd_cols(bc.k, L.trA, (k + 2) >> 2, (k + 2) & 3);
            if (S) {
                ak2 = rd_rows(bs.k, L.rowA, k + 2);
                av2 = rd_rows(bs.v, L.rowA, k + 2);
            }
        }
        if (S)
            sc = mfma32(ak0, qop[k], sc);
        if (P) {
            float d[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * k + e;
                const float p = exp2_fast(fmaf(scp[i], L.sl, -L.lse2));
                d[e] = p * (dpp[i] - L.dsum);
            }
            skn[k] = pack_bf16x2(d[0], d[1]);
            anchor(skn[k]);
        }
        if (C)
            dq[db] = mfma32(ck0, half_op(skc, u), dq[db]);
        if (S)
            dp = mfma32(av0, gop[k], dp);
        sched_fence();
        ck0 = ck1;
        ck1 = ck2;
        ak0 = ak1;
        av0 = av1;
        ak1 = ak2;
        av1 = av2;
    }
    if (P && !bp.full) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            uint32_t m = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int i = 2 * k + e;
                if (bp.kb + 8 * (i >> 2) + 4 * L.J + (i & 3) < L.kend_row)
                    m |= 0xffffu << (16 * e);
            }
            skn[k] &= m;
        }
    }
}

// dQ of 32 query rows per wave: the forward's work split (4 waves, NH query heads of one KV head's group
// times 4 / NH blocks of 32 rows; the group's heads share each K / V tile in LDS) and XCD-aware order.
// Q^T and dO^T of the wave's rows stay in registers as the B operands; K and V tiles of 64 keys stream
// through a three-stage direct-to-LDS ring.  Per 32-key block a wave computes S^T = K Q^T and
// dP^T = V dO^T (A operands: 16-B LDS reads of K and V rows), dS^T, and dQ^T += K^T dS^T (A operand:
// transposed LDS reads of K), in the three-deep block pipeline of the dK / dV kernel.
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
    const int n = lane & 31, J = lane >> 5;
    const int h = g * a.G + hc * NH + (w % NH);
    const int row_w = m0 + 32 * (w / NH); // the wave's first row
    const int qi = row_w + n;             // the lane's row (MFMA column)
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

    // Q^T and dO^T as B operands: lane (row n, J) holds dims 16 s + 8 J .. +8
    bf16x8 qop[8], gop[8];
    {
        const uint16_t *qg = static_cast<const uint16_t *>(a.q), *dog = static_cast<const uint16_t *>(a.dout);
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            uint4 qv = make_uint4(0, 0, 0, 0), gv = make_uint4(0, 0, 0, 0);
            if (row_ok) {
                const size_t off = ((size_t)(q0 + qi) * a.Hq + h) * D + 16 * s + 8 * J;
                qv = ld16(qg + off);
                gv = ld16(dog + off);
            }
            qop[s] = as_bf16x8(qv);
            gop[s] = as_bf16x8(gv);
        }
    }
    f32x16 dq[4]; // dQ^T [128 dims x 32 rows]: block db, register i <-> dim 32 db + 8 (i/4) + 4 J + i%4
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
#pragma unroll
        for (int p = 0; p < kKLoads; ++p) {
            const int row = 4 * (kKLoads * w + p) + (lane >> 4);
            ld.voff[p] = (uint32_t)row * row_bytes + 16 * ((lane & 15) ^ swz(row & 15));
        }
    }

    const int ntiles = (kend + kKTile - 1) / kKTile;
    auto blk = [&](int st, int t, int kk) {
        KBlk x;
        x.k = k_ring[st].k + kk * 32 * kRowBytes;
        x.v = k_ring[st].v + kk * 32 * kRowBytes;
        x.kb = t * kKTile + 32 * kk;
        x.full = row_w + 32 <= Lq && x.kb + 32 <= Lk && (!a.causal || x.kb + 31 <= row_w + diag);
        return x;
    };
    auto next_tile = [&](int st, int t) {
        wait_vmcnt<0>();
        barrier(); // tile t is in LDS for every wave; every wave is done with tile t - 2
        if (t + 1 < ntiles)
            ld.issue(st == kKStages - 1 ? 0 : st + 1, t + 1);
    };

    if (ntiles > 0) {
        f32x16 sc, dp, scp, dpp;
        uint32_t ska[8], skb[8];
        ld.issue(0, 0);
        next_tile(0, 0);
        {
            const KBlk b0 = blk(0, 0, 0), b1 = blk(0, 0, 1);
            q_step<false, true, false>(L, qop, gop, dq, b0, ska, b0, scp, dpp, b0, sc, dp, skb);
            q_step<false, true, true>(L, qop, gop, dq, b0, ska, b1, sc, dp, b0, scp, dpp, skb);
        }
        int sp = 0; // stage of tile t - 1
        for (int t = 1; t < ntiles; ++t) {
            const int st = sp == kKStages - 1 ? 0 : sp + 1;
            next_tile(st, t);
            const KBlk bm2 = blk(sp, t - 1, 0), bm1 = blk(sp, t - 1, 1), bj = blk(st, t, 0), bj1 = blk(st, t, 1);
            q_step<true, true, true>(L, qop, gop, dq, bm2, skb, bj, scp, dpp, bm1, sc, dp, ska);
            q_step<true, true, true>(L, qop, gop, dq, bm1, ska, bj1, sc, dp, bj, scp, dpp, skb);
            sp = st;
        }
        {
            const KBlk bm2 = blk(sp, ntiles - 1, 0), bm1 = blk(sp, ntiles - 1, 1);
            q_step<true, false, true>(L, qop, gop, dq, bm2, skb, bm2, scp, dpp, bm1, sc, dp, ska);
            q_step<true, false, false>(L, qop, gop, dq, bm1, ska, bm1, scp, dpp, bm1, sc, dp, skb);
        }
    }

    if (!row_ok)
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
    while (nh < kDqWaves && G % (2 * nh) == 0)
        nh *= 2;
    return nh;
}

hipError_t launch_prefill_bwd(const BwdArgs &a, hipStream_t stream)
{
    const long slots = (long)a.B * a.max_q * a.Hq;
    if (slots > 0x7fffffffL)
        return hipErrorInvalidValue;
    if (slots > 0)
        hipLaunchKernelGGL(bwd_prep_kernel, dim3((unsigned)((slots + 15) / 16)), dim3(256), 0, stream, a);
    const int nkt = (a.max_k + kKeysPerWg - 1) / kKeysPerWg;
    const long units_kv = (long)a.Hkv * a.B * nkt;
    const long blocks_kv = (units_kv + kXcds - 1) / kXcds * kXcds;
    const int NH = heads_per_wg_bwd(a.G), RB = kDqWaves / NH;
    const int nqt = (a.max_q + 32 * RB - 1) / (32 * RB);
    const long units_q = (long)a.Hkv * (a.G / NH) * a.B * nqt;
    const long blocks_q = (units_q + kXcds - 1) / kXcds * kXcds;
    if (blocks_kv > 0x7fffffff || blocks_q > 0x7fffffff)
        return hipErrorInvalidValue;
    if (units_kv > 0)
        hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)blocks_kv), dim3(kKvThreads), 0, stream, a, nkt,
                           (int)units_kv);
    if (units_q > 0)
        hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)blocks_q), dim3(kDqThreads), 0, stream, a, NH, RB, nqt,
                           (int)units_q);
    return hipGetLastError();
}

} // namespace attn
