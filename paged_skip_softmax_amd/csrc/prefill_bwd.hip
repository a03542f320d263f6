// Backward of the dense bf16 varlen prefill (head dim 128) for gfx950: dQ, dK, dV from Q, K, V, O, the
// output gradient dO and the forward's log-sum-exp.  The Triton kernel of "Model-Optimizer: Add Triton
// unified attention kernel with HuggingFace integration" (summary) has an autograd backward beside its
// forward; the gradients are those of the masked-softmax definition:
//   P = exp(scale Q K^T - lse),  dP = dO V^T,  Dsum = rowsum(dO * O),  dS = P * (dP - Dsum)
//   dV = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K         (dK, dV summed over a KV head's group)
//
// Three kernels, no atomics:
//  * bwd_prep: Dsum per (token, query head), fp32, into the caller's workspace.
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

namespace attn {
namespace {

constexpr int D = 128;
constexpr int kRowBytes = D * 2; // one bf16 row of 128 dims

typedef short i16x4 __attribute__((ext_vector_type(4)));

// XOR swizzle of the 16 chunk slots of a 256-B LDS row (as in the forward kernel).
__device__ __forceinline__ int swz(int r)
{
    return ((r & 1) ? 10 : 0) ^ ((r & 2) ? 4 : 0) ^ ((r & 4) ? 1 : 0) ^ ((r & 8) ? 2 : 0);
}

// Byte offset of 16-byte chunk c of row r in a swizzled tile.
__device__ __forceinline__ uint32_t chunk_off(int r, int c) { return (uint32_t)(r * kRowBytes + 16 * (c ^ swz(r & 15))); }

__device__ __forceinline__ uint2 lds_read_tr(const char *p)
{
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(uint2, r);
}

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

// ------------------------------------------------------------------ Dsum

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
}

// ------------------------------------------------------------------ dK, dV

constexpr int kKvWaves = 4;
constexpr int kKeysPerWave = 16;
constexpr int kKeysPerWg = kKvWaves * kKeysPerWave;
constexpr int kQRows = 32; // query rows per staged tile

__global__ __launch_bounds__(64 * kKvWaves) void bwd_dkdv_kernel(BwdArgs a, int nkt)
{
    // unit = (KV head g, sequence b, key block kt)
    const int unit = blockIdx.x;
    const int kt = unit % nkt, b = (unit / nkt) % a.B, g = unit / (nkt * a.B);
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
    const int kb0 = kt * kKeysPerWg;
    if (kb0 >= Lk)
        return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n16 = lane & 15, g4 = lane >> 4;
    const int kw = kb0 + kKeysPerWave * w;    // the wave's first key
    const int key = kw + n16;                 // the lane's key (MFMA column)
    const int diag = Lk - Lq;

    __shared__ __attribute__((aligned(16))) char q_t[kQRows * kRowBytes];
    __shared__ __attribute__((aligned(16))) char do_t[kQRows * kRowBytes];
    __shared__ float lse_t[kQRows], dsum_t[kQRows];

    // K^T and V^T as B operands: lane (key n16, group g4) holds dims 32 s + 8 g4 .. +8 of its key
    const uint16_t *kg = static_cast<const uint16_t *>(a.k), *vg = static_cast<const uint16_t *>(a.v);
    bf16x8 kop[4], vop[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
        if (key < Lk) {
            const size_t off = ((size_t)(k0 + key) * a.Hkv + g) * D + 32 * s + 8 * g4;
            kv = ld16(kg + off);
            vv = ld16(vg + off);
        }
        kop[s] = as_bf16x8(kv);
        vop[s] = as_bf16x8(vv);
    }
    f32x4 dk[8], dv[8]; // [16 dims x 16 keys] blocks db: lane holds dims 16 db + 4 g4 + i of its key
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        dk[db] = f32x4{0.f, 0.f, 0.f, 0.f};
        dv[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // the first query row that sees key kb0
    const int row_start = a.causal ? max(0, kb0 - diag) : 0;
    const int qt_first = row_start / kQRows, nqt = (Lq + kQRows - 1) / kQRows;
    const uint16_t *qg = static_cast<const uint16_t *>(a.q), *dog = static_cast<const uint16_t *>(a.dout);
    // transposed-read addresses (dims 16 db + lane's column, rows 4 g4 .. +3 and 16 + 4 g4 .. +3)
    const int trow_lo = 4 * g4 + (n16 >> 2), trow_hi = 16 + trow_lo;
    const int tcol_chunk = (n16 & 3) >> 1, tcol_half = 8 * (n16 & 1);

    for (int hh = 0; hh < a.G; ++hh) {
        const int h = g * a.G + hh;
        for (int qt = qt_first; qt < nqt; ++qt) {
            const int r0 = qt * kQRows;
            __syncthreads(); // the previous tile is no longer read
            stage_rows(q_t, qg, (size_t)q0 + r0, a.Hq, h, kQRows, Lq - r0, tid, 64 * kKvWaves);
            stage_rows(do_t, dog, (size_t)q0 + r0, a.Hq, h, kQRows, Lq - r0, tid, 64 * kKvWaves);
            if (tid < kQRows) {
                const int r = r0 + tid;
                lse_t[tid] = r < Lq ? a.lse[(size_t)(q0 + r) * a.Hq + h] * kLog2e : 0.f;
                dsum_t[tid] = r < Lq ? a.dsum[(size_t)(q0 + r) * a.Hq + h] : 0.f;
            }
            __syncthreads();

            // S and dP for the 2 row blocks of 16
            f32x4 s[2], dp[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                s[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
                dp[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int r = 16 * rb + n16;
#pragma unroll
                for (int st = 0; st < 4; ++st) {
                    const uint32_t off = chunk_off(r, 4 * st + g4);
                    s[rb] = mfma16(as_bf16x8(ld16(q_t + off)), kop[st], s[rb]);
                    dp[rb] = mfma16(as_bf16x8(ld16(do_t + off)), vop[st], dp[rb]);
                }
            }
            // P and dS: lane holds rows 16 rb + 4 g4 + i of its key
            float p[2][4], ds[2][4];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int rt = 16 * rb + 4 * g4 + i, row = r0 + rt;
                    const bool vis = row < Lq && key < Lk && (!a.causal || key <= row + diag);
                    const float pv = vis ? exp2_fast(fmaf(s[rb][i], a.scale_log2, -lse_t[rt])) : 0.f;
                    p[rb][i] = pv;
                    ds[rb][i] = pv * (dp[rb][i] - dsum_t[rt]);
                }
            // k-slot e of the row contraction <-> row 16 (e / 4) + 4 g4 + e % 4
            const bf16x8 pop = as_bf16x8(make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                                                    pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])));
            const bf16x8 dsop = as_bf16x8(make_uint4(pack_bf16x2(ds[0][0], ds[0][1]), pack_bf16x2(ds[0][2], ds[0][3]),
                                                     pack_bf16x2(ds[1][0], ds[1][1]), pack_bf16x2(ds[1][2], ds[1][3])));
#pragma unroll
            for (int db = 0; db < 8; ++db) {
                const int c = 2 * db + tcol_chunk;
                const uint32_t lo = chunk_off(trow_lo, c) + tcol_half, hi = chunk_off(trow_hi, c) + tcol_half;
                const uint2 glo = lds_read_tr(do_t + lo), ghi = lds_read_tr(do_t + hi);
                dv[db] = mfma16(as_bf16x8(make_uint4(glo.x, glo.y, ghi.x, ghi.y)), pop, dv[db]);
                const uint2 qlo = lds_read_tr(q_t + lo), qhi = lds_read_tr(q_t + hi);
                dk[db] = mfma16(as_bf16x8(make_uint4(qlo.x, qlo.y, qhi.x, qhi.y)), dsop, dk[db]);
            }
        }
    }

    if (key >= Lk)
        return;
    uint16_t *dkg = static_cast<uint16_t *>(a.dk) + ((size_t)(k0 + key) * a.Hkv + g) * D + 4 * g4;
    uint16_t *dvg = static_cast<uint16_t *>(a.dv) + ((size_t)(k0 + key) * a.Hkv + g) * D + 4 * g4;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        uint2 pk, pv;
        pk.x = pack_bf16x2(dk[db][0] * a.scale, dk[db][1] * a.scale);
        pk.y = pack_bf16x2(dk[db][2] * a.scale, dk[db][3] * a.scale);
        pv.x = pack_bf16x2(dv[db][0], dv[db][1]);
        pv.y = pack_bf16x2(dv[db][2], dv[db][3]);
        *reinterpret_cast<uint2 *>(dkg + 16 * db) = pk;
        *reinterpret_cast<uint2 *>(dvg + 16 * db) = pv;
    }
}

// ------------------------------------------------------------------ dQ

constexpr int kDqWaves = 4;
constexpr int kKeysPerTile = 32;

__global__ __launch_bounds__(64 * kDqWaves) void bwd_dq_kernel(BwdArgs a, int NH, int RB, int nqt)
{
    const int unit = blockIdx.x;
    const int hchunks = a.G / NH;
    const int qt = nqt - 1 - unit % nqt, b = (unit / nqt) % a.B, gh = unit / (nqt * a.B);
    const int g = gh / hchunks, hc = gh % hchunks;
    const int rows_wg = 32 * RB;
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
    const int m0 = qt * rows_wg;
    if (m0 >= Lq)
        return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, J = lane >> 5;
    const int h = g * a.G + hc * NH + (w % NH);
    const int qi = m0 + 32 * (w / NH) + n; // the lane's row (MFMA column)
    const bool row_ok = qi < Lq;
    const int diag = Lk - Lq;
    const int last_row = min(m0 + rows_wg, Lq) - 1;
    const int kend = a.causal ? max(0, min(Lk, last_row + 1 + diag)) : Lk;
    const int kend_row = a.causal ? max(0, min(Lk, qi + 1 + diag)) : Lk;

    __shared__ __attribute__((aligned(16))) char k_t[kKeysPerTile * kRowBytes];
    __shared__ __attribute__((aligned(16))) char v_t[kKeysPerTile * kRowBytes];

    // Q^T and dO^T as B operands: lane (row n, J) holds dims 16 s + 8 J .. +8
    const uint16_t *qg = static_cast<const uint16_t *>(a.q), *dog = static_cast<const uint16_t *>(a.dout);
    bf16x8 qop[8], gop[8];
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
    const float lse2 = row_ok ? a.lse[(size_t)(q0 + qi) * a.Hq + h] * kLog2e : 0.f;
    const float dsum = row_ok ? a.dsum[(size_t)(q0 + qi) * a.Hq + h] : 0.f;
    f32x16 dq[4]; // dQ^T [128 dims x 32 rows]: block db, register i -> dim 32 db + 8 (i / 4) + 4 J + i % 4
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            dq[db][i] = 0.f;

    // transposed reads of K (A operand of dQ^T): lane (16-lane group G16, index j) addresses key
    // 8 hf + 4 J + j / 4 of a 16-key block, dims 32 db + 16 (G16 % 2) + 4 (j % 4)
    const int G16 = lane >> 4, j = lane & 15;
    const int xcol = 2 * (G16 & 1) + ((j & 3) >> 1);
    const uint16_t *kg = static_cast<const uint16_t *>(a.k), *vg = static_cast<const uint16_t *>(a.v);

    for (int kb = 0; kb < kend; kb += kKeysPerTile) {
        __syncthreads();
        stage_rows(k_t, kg, (size_t)k0 + kb, a.Hkv, g, kKeysPerTile, Lk - kb, tid, 64 * kDqWaves);
        stage_rows(v_t, vg, (size_t)k0 + kb, a.Hkv, g, kKeysPerTile, Lk - kb, tid, 64 * kDqWaves);
        __syncthreads();
        // S^T and dP^T [32 keys x 32 rows]: A operand = key row n, dims 16 s + 8 J
        f32x16 s, dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            s[i] = 0.f;
            dp[i] = 0.f;
        }
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const uint32_t off = chunk_off(n, 2 * st + J);
            s = mfma32(as_bf16x8(ld16(k_t + off)), qop[st], s);
            dp = mfma32(as_bf16x8(ld16(v_t + off)), gop[st], dp);
        }
        // P^T, dS^T: register i <-> key kb + 8 (i / 4) + 4 J + i % 4 of the lane's row
        uint32_t dsk[8];
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            float d2[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int ii = i + e;
                const int keyi = kb + 8 * (ii / 4) + 4 * J + (ii % 4);
                const bool vis = row_ok && keyi < kend_row;
                const float pv = vis ? exp2_fast(fmaf(s[ii], a.scale_log2, -lse2)) : 0.f;
                d2[e] = pv * (dp[ii] - dsum);
            }
            dsk[i >> 1] = pack_bf16x2(d2[0], d2[1]);
        }
        // dQ^T += K^T dS^T over the two 16-key halves u
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8 dsop = as_bf16x8(make_uint4(dsk[4 * u], dsk[4 * u + 1], dsk[4 * u + 2], dsk[4 * u + 3]));
#pragma unroll
            for (int db = 0; db < 4; ++db) {
                uint2 lo, hi;
                {
                    const int rw = 16 * u + 4 * J + (j >> 2);
                    lo = lds_read_tr(k_t + chunk_off(rw, 4 * db + xcol) + 8 * (j & 1));
                }
                {
                    const int rw = 16 * u + 8 + 4 * J + (j >> 2);
                    hi = lds_read_tr(k_t + chunk_off(rw, 4 * db + xcol) + 8 * (j & 1));
                }
                dq[db] = mfma32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), dsop, dq[db]);
            }
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
    const int NH = heads_per_wg_bwd(a.G), RB = kDqWaves / NH;
    const int nqt = (a.max_q + 32 * RB - 1) / (32 * RB);
    const long units_q = (long)a.Hkv * (a.G / NH) * a.B * nqt;
    if (units_kv > 0x7fffffff || units_q > 0x7fffffff)
        return hipErrorInvalidValue;
    if (units_kv > 0)
        hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)units_kv), dim3(64 * kKvWaves), 0, stream, a, nkt);
    if (units_q > 0)
        hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)units_q), dim3(64 * kDqWaves), 0, stream, a, NH, RB, nqt);
    return hipGetLastError();
}

} // namespace attn
