// One-token paged-KV decode for gfx950: split-K (two kernels) and the sequential skip-softmax schedule.
//
// Schedules ("Model-Optimizer: Add split-k decode kernel for skip softmax", What does this PR do):
//  * skip-softmax off: the keys of a sequence are cut into 128-key tiles and the tiles into num_splits
//    contiguous runs of ceil(ntiles / num_splits) tiles.  Every (batch row, KV head, split) is one
//    workgroup that writes a partial (O_s, lse_s) for the G query heads of the KV head; a second small
//    kernel merges the partials of a row: lse = log sum_s e^{lse_s}, O = sum_s e^{lse_s - lse} O_s.
//    The KV head is the fastest grid dimension: the Hkv slabs of a page lie next to each other in the
//    cache, so the workgroups running together read whole pages rather than one slab of many pages.
//  * skip-softmax on: one sequential split over 32-key tiles.  Tile t of query row r is skipped (no exp,
//    no P.V, no rescale) when exp(tmax_t - m) < threshold, m the running max before the tile
//    ("TensorRT-LLM: Skip Softmax Attention", Description).  Because a skipped tile lies below the
//    running max (threshold <= 1), the running max before tile t always equals the max of tmax over
//    all earlier tiles, skipped or not.  So the waves of the workgroup take consecutive tiles in
//    rounds, publish their tile maxima in LDS, and each decides exactly from the prefix max -- the
//    decisions of one sequential pass, taken in parallel.  V of a tile is read only when at least one
//    query row of the group keeps it.  The K rows run two rounds ahead (requested after a round's V,
//    so that waiting for that V leaves them in flight), and batches of up to 128 rows are dispatched
//    longest first, so that the longest sequences (the critical path of a one-split-per-sequence
//    schedule) start at once and the short ones fill in behind them.
//
// Cache layout: [num_pages, Hkv, 16, D] bf16, so one (page, KV head) is a contiguous 4 KB slab.
//
// Per 32-key chunk (two pages) a wave computes, for the G query heads of its KV head:
//   S^T[32 keys x 16] = K[32 x 128] . Q^T[128 x 16]      8 MFMA 16x16x32 (columns >= G are zero)
//   online softmax in the log2 domain (scale * log2 e folded into one FMA)
//   O^T[128 x 16] += V^T[128 x 32] . P^T[32 x 16]         8 MFMA 16x16x32
// K goes straight from HBM into MFMA operand registers (each lane loads 16 B of one key row).  V is
// loaded with fully coalesced 16-B loads (each wave instruction reads 1 KB of a slab), stored to a
// wave-private LDS tile with a padded row pitch, and read back as the transposed operand with
// ds_read_b64_tr_b16 (two 8-B reads per MFMA).
// The key order inside the P.V contraction follows the S^T register layout (lane group j holds keys
// 4j..4j+3 of each page), so P needs no shuffle between the two products.  Each wave keeps its own
// online-softmax state; the states are merged through LDS at the end of the workgroup.
#include "kcommon.h"
#include "launch.h"

namespace attn {

constexpr int kPage = 16;
constexpr int kD = 128;
constexpr int kSplitTile = 128;
constexpr int kSplitWaves = 4;
constexpr int kSeqWaves = 8;
constexpr int kVPitch = kD + 16;                  // LDS row pitch (bf16 elements, 288 B)
constexpr int kVTile = 2 * kPage * kVPitch;       // one wave's V staging tile (elements)
// s_waitcnt immediate that waits for LDS / scalar memory only (vmcnt and expcnt at their maxima; gfx9
// layout: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int kWaitLdsOnly = 0xF | (0x7 << 4) | (0x3 << 14);

// Q^T operand: lane (n = lane%16, j = lane/16) holds head g*G+n, d = 32 s + 8 j .. +8.
__device__ __forceinline__ void load_q_operand(const uint16_t *q, int b, int g, int Hq, int G, int lane,
                                               bf16x8 qop[4])
{
    const int n = lane & 15, j = lane >> 4;
    if (n < G) {
        const uint16_t *qp = q + ((size_t)b * Hq + (size_t)g * G + n) * kD + 8 * j;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qop[s] = as_bf16x8(ld16(qp + 32 * s));
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qop[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
}

// K rows of two pages in MFMA A-operand order: key lane%16 of the page, d = 32 s + 8 (lane/16).
__device__ __forceinline__ void load_k_chunk(const uint16_t *kp0, const uint16_t *kp1, int lane, uint4 kr[2][4])
{
    const int off = (lane & 15) * kD + 8 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        kr[0][s] = ld16(kp0 + off + 32 * s);
        kr[1][s] = ld16(kp1 + off + 32 * s);
    }
}

// V slabs of two pages, coalesced: lane reads key lane/16 + 4 r, d = 8 (lane%16) .. +8.
__device__ __forceinline__ void load_v_chunk(const uint16_t *vp0, const uint16_t *vp1, int lane, uint4 vr[2][4])
{
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        vr[0][r] = ld16(vp0 + 8 * lane + 512 * r);
        vr[1][r] = ld16(vp1 + 8 * lane + 512 * r);
    }
}

// Raw scores q.k of the chunk: sc[pg][i] = key 16 pg + 4 j + i for head lane%16; keys at or past
// tend are set to -inf.  Returns the chunk max of the lane's head (raw units, across lane groups).
__device__ __forceinline__ float chunk_scores(const uint4 kr[2][4], const bf16x8 qop[4], int tok0, int tend,
                                              int lane, f32x4 sc[2])
{
    const int j = lane >> 4;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
        sc[pg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            sc[pg] = mfma16(as_bf16x8(kr[pg][s]), qop[s], sc[pg]);
    }
    const bool partial = tok0 + 2 * kPage > tend;
    float cmax = kNegInf;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (partial && tok0 + kPage * pg + 4 * j + i >= tend)
                sc[pg][i] = kNegInf;
            cmax = fmaxf(cmax, sc[pg][i]);
        }
    return max_across_groups16(cmax);
}

// Online-softmax state of one wave.  Lane (n, j) holds head n; m is in the log2 domain, l is this
// lane's partial sum (reduced over j at the end), acc[db][i] = O^T[d = 16 db + 4 j + i][n].
struct WaveState {
    float m, l;
    f32x4 acc[kD / 16];
};

__device__ __forceinline__ void state_init(WaveState &st)
{
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db)
        st.acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// 8-byte transposed LDS read (ds_read_b64_tr_b16): in each 16-lane group, lane i receives element i
// of the 16 consecutive columns the group addresses, from each of the 4 rows it addresses.
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t *p)
{
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(uint2, r);
}

// NVFP4 fake quantization ("Model-Optimizer: Add split-k decode kernel for skip softmax", What does this
// PR do and Usage: P and V quantized to NVFP4 and back in the sequential decode, each with an amax).
// A block of 16 values shares one E4M3 scale code; the elements are E2M1; enc = 448 / amax and
// dec = amax / 2688 (6 * 448) are the per-tensor fp32 factors.  For a block with max |x| = b:
//   s = e4m3(b * enc) * dec,   x^ = sign(x) * e2m1(|x| * (1 / s)) * s   (x^ = 0 when s = 0),
// every rounding to nearest even with saturation, in fp32.
struct Nvfp4 {
    float enc, dec;
};
struct Qdq {
    Nvfp4 p, v;
    bool p_on, v_on;
};

// E4M3 rounding of y >= 0 (3 mantissa bits, subnormals below 2^-6, nearest even, saturating at 448):
// gfx950's conversion to fp8 and back, after clamping to 448.
__device__ __forceinline__ float round_e4m3(float y)
{
    const int p = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(y, 448.f), 0.f, 0, false);
    return __builtin_amdgcn_cvt_f32_fp8(p, 0);
}

// E2M1 rounding of two fp32 values onto +-{0, 0.5, 1, 1.5, 2, 3, 4, 6} (nearest even, saturating at
// +-6): gfx950's conversion to packed fp4 and back, both at scale 1.
__device__ __forceinline__ f32x2 round_e2m1_pair(float a, float b)
{
    const uint32_t p = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.f, 0);
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(p, 1.f, 0);
}

struct BlockScale {
    float s, r; // block scale and its reciprocal (0 for an all-zero block)
};

__device__ __forceinline__ BlockScale nvfp4_block_scale(float bmax, Nvfp4 f)
{
    const float s = round_e4m3(bmax * f.enc) * f.dec;
    return {s, s > 0.f ? 1.f / s : 0.f};
}

// Two values of one block; sign(x) e2m1(|x| r) = e2m1(x r), the grid being symmetric.
__device__ __forceinline__ f32x2 nvfp4_qdq2(float x0, float x1, BlockScale b)
{
    const f32x2 q = round_e2m1_pair(x0 * b.r, x1 * b.r);
    return f32x2{q.x * b.s, q.y * b.s};
}

// Max of v over the lane pair (2i, 2i + 1) (DPP quad_perm [1, 0, 3, 2]).
__device__ __forceinline__ float max_lane_pair(float v)
{
    const int o = __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false);
    return fmaxf(v, __builtin_bit_cast(float, o));
}

// V of one key row slice (8 bf16, d = 8 (lane % 16) .. +8) fake-quantized in blocks of 16 along D: the
// block is the lane pair (2i, 2i + 1) of the 16-lane group, which holds one key.  Back to bf16.
__device__ __forceinline__ uint4 qdq_v8(uint4 v, Nvfp4 f)
{
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float x[8], bmax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        x[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
        bmax = fmaxf(bmax, fmaxf(fabsf(x[2 * i]), fabsf(x[2 * i + 1])));
    }
    const BlockScale b = nvfp4_block_scale(max_lane_pair(bmax), f);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f32x2 y = nvfp4_qdq2(x[2 * i], x[2 * i + 1], b);
        o[i] = pack_bf16x2(y.x, y.y);
    }
    return make_uint4(o[0], o[1], o[2], o[3]);
}

// Stages one chunk's V in the wave's LDS tile vt (keys at or past tend cleared, so that 0 * NaN never
// reaches the accumulator), fake-quantized per key in blocks of 16 along D when qq.v_on (QDQ).
template <bool QDQ = false>
__device__ __forceinline__ void stage_v(const uint4 vr[2][4], int tok0, int tend, uint16_t *vt, int lane,
                                        const Qdq &qq = Qdq{})
{
    // keys past tend: V cleared by an AND mask (no per-lane branch) under one wave-uniform branch
    const bool partial = tok0 + 2 * kPage > tend;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = (lane >> 4) + 4 * r;
            uint4 v = vr[pg][r];
            if (QDQ && qq.v_on)
                v = qdq_v8(v, qq.v);
            if (partial) {
                const uint32_t keep = tok0 + kPage * pg + key < tend ? ~0u : 0u;
                v = make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
            }
            st16(vt + (pg * kPage + key) * kVPitch + 8 * (lane & 15), v);
        }
}

// Folds one chunk, whose V is already staged in vt, into the state.  keep == false (per lane, i.e. per
// head) leaves that head's state untouched: p = 0 and no rescale.  cmax_l2: chunk max in log2 units.
// QDQ: fake-quantize P (blocks of the 16 keys of a page, per head; the row sum takes the unquantized P).
template <bool QDQ = false>
__device__ __forceinline__ void chunk_update_staged(WaveState &st, const f32x4 sc[2], float cmax_l2, bool keep,
                                                    float scale_log2, const uint16_t *vt, int lane,
                                                    const Qdq &qq = Qdq{})
{
    const int n = lane & 15, j = lane >> 4;
    const float m_new = keep ? fmaxf(st.m, cmax_l2) : st.m;
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = keep ? exp2_fast(st.m - m_use) : 1.f;
    float p[2][4], psum = 0.f;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[pg][i] = keep ? exp2_fast(fmaf(sc[pg][i], scale_log2, -m_use)) : 0.f;
            psum += p[pg][i];
        }
    st.l = fmaf(st.l, alpha, psum);
    st.m = m_new;
    if (QDQ && qq.p_on)
#pragma unroll
        for (int pg = 0; pg < 2; ++pg) {
            const float bm = fmaxf(fmaxf(p[pg][0], p[pg][1]), fmaxf(p[pg][2], p[pg][3]));
            const BlockScale b = nvfp4_block_scale(max_across_groups16(bm), qq.p);
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
                const f32x2 y = nvfp4_qdq2(p[pg][i], p[pg][i + 1], b);
                p[pg][i] = y.x;
                p[pg][i + 1] = y.y;
            }
        }
#pragma unroll
    for (int db = 0; db < kD / 16; ++db)
        st.acc[db] *= alpha;

    __builtin_amdgcn_wave_barrier();
    const bf16x8 pop = as_bf16x8(make_uint4(pack_bf16x2(p[0][0], p[0][1]), pack_bf16x2(p[0][2], p[0][3]),
                                            pack_bf16x2(p[1][0], p[1][1]), pack_bf16x2(p[1][2], p[1][3])));
    // V^T operand by transposed reads: in lane group j, lane (n) addresses key 4 j + n / 4 (then 16 +
    // 4 j + n / 4) and dims 16 db + 4 (n % 4) .. +3, and receives keys 4 j .. 4 j + 3 of dim 16 db + n
    const uint16_t *v0 = vt + (4 * j + (n >> 2)) * kVPitch + 4 * (n & 3);
    const uint16_t *v1 = v0 + kPage * kVPitch;
#pragma unroll
    for (int db = 0; db < kD / 16; ++db) {
        const uint2 lo = lds_read_tr(v0 + 16 * db);
        const uint2 hi = lds_read_tr(v1 + 16 * db);
        st.acc[db] = mfma16(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pop, st.acc[db]);
    }
    __builtin_amdgcn_wave_barrier();
}

// stage_v, then chunk_update_staged: V (read only when some head keeps the chunk) staged after the scores.
template <bool QDQ = false>
__device__ __forceinline__ void chunk_update(WaveState &st, const f32x4 sc[2], float cmax_l2, bool keep,
                                             const uint4 vr[2][4], int tok0, int tend, float scale_log2,
                                             uint16_t *vt, int lane, const Qdq &qq = Qdq{})
{
    stage_v<QDQ>(vr, tok0, tend, vt, lane, qq);
    chunk_update_staged<QDQ>(st, sc, cmax_l2, keep, scale_log2, vt, lane, qq);
}

// Merges the W wave states of the workgroup (through LDS at `smem`, which must hold
// W * 16 * (D + 2) floats and is reused after a barrier) and calls out(h, d, o, lse_natural) for
// every head h < G and d < D.  lse is -inf and o = 0 for a head that saw no key.
template <int W, typename Out>
__device__ __forceinline__ void merge_waves(WaveState &st, void *smem, int G, Out out)
{
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, j = lane >> 4;
    st.l = sum_across_groups16(st.l);
    __syncthreads();
    float *red_acc = static_cast<float *>(smem);
    float *red_m = red_acc + W * 16 * kD;
    float *red_l = red_m + W * 16;
    if (n < G) {
#pragma unroll
        for (int db = 0; db < kD / 16; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                red_acc[(w * 16 + n) * kD + 16 * db + 4 * j + i] = st.acc[db][i];
        if (j == 0) {
            red_m[w * 16 + n] = st.m;
            red_l[w * 16 + n] = st.l;
        }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < G * kD; idx += blockDim.x) {
        const int h = idx / kD, d = idx % kD;
        float M = kNegInf;
#pragma unroll
        for (int ww = 0; ww < W; ++ww)
            M = fmaxf(M, red_m[ww * 16 + h]);
        float o = 0.f, lse = kNegInf;
        if (M != kNegInf) {
            float den = 0.f, num = 0.f;
#pragma unroll
            for (int ww = 0; ww < W; ++ww) {
                const float e = exp2_fast(red_m[ww * 16 + h] - M);
                den = fmaf(e, red_l[ww * 16 + h], den);
                num = fmaf(e, red_acc[(ww * 16 + h) * kD + d], num);
            }
            o = num / den;
            lse = (M + __log2f(den)) * kLn2;
        }
        out(h, d, o, lse);
    }
}

// Runs compute(tok, kr, vr) over a wave's chunks tok = first, first + step, ... < end, with the K and V
// of the next chunk loaded (load(tok, kr, vr)) while the current one is computed.  The exit test comes
// before each prefetch, so no branch joins right after the loads (at such a join the compiler waits for
// every load in flight, the prefetch included), and the two buffer sets alternate by name (a register
// copy of a load in flight would wait for it).
template <typename Load, typename Compute>
__device__ __forceinline__ void chunk_pipeline(int first, int end, int step, Load load, Compute compute)
{
    uint4 ka[2][4], va[2][4], kb[2][4], vb[2][4];
    load(first, ka, va);
    for (int tok = first;;) {
        if (tok + step >= end) {
            compute(tok, ka, va);
            break;
        }
        load(tok + step, kb, vb);
        compute(tok, ka, va);
        tok += step;
        if (tok + step >= end) {
            compute(tok, kb, vb);
            break;
        }
        load(tok + step, ka, va);
        compute(tok, kb, vb);
        tok += step;
    }
}

// ------------------------------------------------------------------ split-K

__global__ __launch_bounds__(64 * kSplitWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void
decode_split_kernel(SplitArgs a)
{
    const int g = blockIdx.x, sp = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int S = a.num_splits;
    const int L = a.seq_lens[b];
    const int ntiles = (L + kSplitTile - 1) / kSplitTile;
    const int per = (ntiles + S - 1) / S;
    const int t0 = min(sp * per * kSplitTile, L);
    const int t1 = min((sp + 1) * per * kSplitTile, L);

    __shared__ __attribute__((aligned(16))) uint16_t smem[kSplitWaves * kVTile];
    static_assert(sizeof(smem) >= kSplitWaves * 16 * (kD + 2) * sizeof(float), "merge buffer");
    uint16_t *vt = smem + w * kVTile;

    bf16x8 qop[4];
    load_q_operand(a.q, b, g, a.Hq, a.G, lane, qop);
    WaveState st;
    state_init(st);
    const int32_t *btr = a.bt + (size_t)b * a.max_pages;
    const size_t slab = (size_t)kPage * kD;
    const int step = 2 * kPage * kSplitWaves;
    const int first = t0 + 2 * kPage * w;
    if (first < t1)
        chunk_pipeline(
            first, t1, step,
            [&](int tok0, uint4 (&kr)[2][4], uint4 (&vr)[2][4]) {
                const int p0 = btr[tok0 / kPage];
                const int p1 = tok0 + kPage < t1 ? btr[tok0 / kPage + 1] : p0;
                const size_t o0 = ((size_t)p0 * a.Hkv + g) * slab, o1 = ((size_t)p1 * a.Hkv + g) * slab;
                load_k_chunk(a.kc + o0, a.kc + o1, lane, kr);
                load_v_chunk(a.vc + o0, a.vc + o1, lane, vr);
            },
            [&](int tok0, const uint4 (&kr)[2][4], const uint4 (&vr)[2][4]) {
                // V goes to LDS first, so its registers are free before the scores are computed
                stage_v(vr, tok0, t1, vt, lane);
                f32x4 sc[2];
                const float cmax = chunk_scores(kr, qop, tok0, t1, lane, sc);
                chunk_update_staged(st, sc, cmax * a.scale_log2, true, a.scale_log2, vt, lane);
            });
    const size_t row0 = (size_t)b * a.Hq + (size_t)g * a.G;
    merge_waves<kSplitWaves>(st, smem, a.G, [&](int h, int d, float o, float lse) {
        a.ws_o[((row0 + h) * S + sp) * kD + d] = o;
        if (d == 0)
            a.ws_lse[(row0 + h) * S + sp] = lse;
    });
}

struct MergeArgs {
    const float *ws_o, *ws_lse;
    int rows, num_splits;
    uint16_t *o;   // [rows, D] bf16
    float *lse;    // nullable [rows]
};

constexpr int kMergeBatch = 16; // partial loads a merge wave has in flight together

// One wave per (batch row, query head): lse = log sum_s e^{lse_s}, O = sum_s e^{lse_s - lse} O_s.
__device__ __forceinline__ void merge_rows(const MergeArgs &a)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= a.rows)
        return;
    const int S = a.num_splits;
    const float ls = lane < S ? a.ws_lse[(size_t)row * S + lane] * kLog2e : kNegInf;
    const float M = wave_max(ls);
    float o0 = 0.f, o1 = 0.f, lse = kNegInf;
    if (M != kNegInf) {
        const float e = exp2_fast(ls - M);
        const float den = wave_sum(e);
        // every split wrote a finite partial (o = 0 where it saw no key, weight e = 0), so the loads go
        // out unconditionally, kMergeBatch at a time
        const float2 *src = reinterpret_cast<const float2 *>(a.ws_o + (size_t)row * S * kD) + lane;
        int s = 0;
        for (; s + kMergeBatch <= S; s += kMergeBatch) {
            float2 v[kMergeBatch];
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u)
                v[u] = src[(s + u) * (kD / 2)];
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                const float ws = __shfl(e, s + u);
                o0 = fmaf(ws, v[u].x, o0);
                o1 = fmaf(ws, v[u].y, o1);
            }
        }
        for (; s < S; ++s) {
            const float ws = __shfl(e, s);
            const float2 v = src[s * (kD / 2)];
            o0 = fmaf(ws, v.x, o0);
            o1 = fmaf(ws, v.y, o1);
        }
        o0 /= den;
        o1 /= den;
        lse = (M + __log2f(den)) * kLn2;
    }
    reinterpret_cast<uint32_t *>(a.o + (size_t)row * kD)[lane] = pack_bf16x2(o0, o1);
    if (a.lse && lane == 0)
        a.lse[row] = lse;
}

__global__ __launch_bounds__(256) void decode_merge_kernel(MergeArgs a) { merge_rows(a); }

// The same merge for the (token, head) rows of the multi-token decode (a name of its own in traces).
__global__ __launch_bounds__(256) void decode_merge_multi_kernel(MergeArgs a) { merge_rows(a); }

hipError_t launch_decode_split(const SplitArgs &a, int B, uint16_t *o, float *lse, hipStream_t stream)
{
    ATTN_LAUNCH(decode_split_kernel, dim3(a.Hkv, a.num_splits, B), dim3(64 * kSplitWaves), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    MergeArgs m{a.ws_o, a.ws_lse, B * a.Hq, a.num_splits, o, lse};
    ATTN_LAUNCH(decode_merge_kernel, dim3((B * a.Hq + 3) / 4), dim3(256), 0, stream, m);
    return hipGetLastError();
}

// ------------------------------------------------------------------ multi-token decode (split-K)

// Raw scores of a chunk for per-column key limits: keys at or past lim (the lane's column) are -inf;
// lim_min (wave-uniform) lets chunks below every column's limit skip the masking.
__device__ __forceinline__ float chunk_scores_lim(const uint4 kr[2][4], const bf16x8 qop[4], int tok0, int lim,
                                                  int lim_min, int lane, f32x4 sc[2])
{
    const int j = lane >> 4;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg) {
        sc[pg] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            sc[pg] = mfma16(as_bf16x8(kr[pg][s]), qop[s], sc[pg]);
    }
    const bool partial = tok0 + 2 * kPage > lim_min;
    float cmax = kNegInf;
#pragma unroll
    for (int pg = 0; pg < 2; ++pg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (partial && tok0 + kPage * pg + 4 * j + i >= lim)
                sc[pg][i] = kNegInf;
            cmax = fmaxf(cmax, sc[pg][i]);
        }
    return max_across_groups16(cmax);
}

// Multi-token decode: sequence b has Lq = cu_q[b+1] - cu_q[b] new tokens, the last Lq of its L cached
// keys; token i sees keys [0, L - Lq + i + 1) (bottom-right causal).  The Lq * G (token, head) rows of a
// KV head's group ride in the MFMA's 16 columns, 16 rows per workgroup (column n <-> row 16 cb + n:
// token (16 cb + n) / G, head g G + (16 cb + n) % G), so one read of the cache serves up to 16 rows;
// otherwise the same split-K schedule, chunk pipeline and partials as decode_split_kernel, over the
// keys the block's last token sees.
__global__ __launch_bounds__(64 * kSplitWaves) __attribute__((amdgpu_waves_per_eu(2, 2))) void
decode_multi_kernel(MultiArgs a)
{
    const int g = blockIdx.x, sp = blockIdx.y, b = blockIdx.z / a.ncb, cb = blockIdx.z % a.ncb;
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int r0 = 16 * cb;
    if (r0 >= Lq * a.G)
        return;
    const int nc = min(16, Lq * a.G - r0); // columns in use
    const int L = a.seq_lens[b];
    const int n = lane & 15, j = lane >> 4;
    const bool col_ok = n < nc;
    const int ti = (r0 + n) / a.G;         // the column's token
    auto key_end = [&](int i) { return max(0, min(L, L - Lq + i + 1)); };
    const int kend = key_end((r0 + nc - 1) / a.G); // keys the block's last token sees
    const int S = a.num_splits;
    const int ntiles = (kend + kSplitTile - 1) / kSplitTile;
    const int per = (ntiles + S - 1) / S;
    const int t0 = min(sp * per * kSplitTile, kend);
    const int t1 = min((sp + 1) * per * kSplitTile, kend);
    const int lim = col_ok ? min(key_end(ti), t1) : 0;
    const int lim_min = min(key_end(r0 / a.G), t1);

    __shared__ __attribute__((aligned(16))) uint16_t smem[kSplitWaves * kVTile];
    static_assert(sizeof(smem) >= kSplitWaves * 16 * (kD + 2) * sizeof(float), "merge buffer");
    uint16_t *vt = smem + w * kVTile;

    // Q^T operand: lane (n, j) holds the column's row, d = 32 s + 8 j .. +8
    bf16x8 qop[4];
    if (col_ok) {
        const uint16_t *qp = a.q + ((size_t)(q0 + ti) * a.Hq + (size_t)g * a.G + (r0 + n) % a.G) * kD + 8 * j;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qop[s] = as_bf16x8(ld16(qp + 32 * s));
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qop[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
    }
    WaveState st;
    state_init(st);
    const int32_t *btr = a.bt + (size_t)b * a.max_pages;
    const size_t slab = (size_t)kPage * kD;
    const int step = 2 * kPage * kSplitWaves;
    const int first = t0 + 2 * kPage * w;
    if (first < t1)
        chunk_pipeline(
            first, t1, step,
            [&](int tok0, uint4 (&kr)[2][4], uint4 (&vr)[2][4]) {
                const int p0 = btr[tok0 / kPage];
                const int p1 = tok0 + kPage < t1 ? btr[tok0 / kPage + 1] : p0;
                const size_t o0 = ((size_t)p0 * a.Hkv + g) * slab, o1 = ((size_t)p1 * a.Hkv + g) * slab;
                load_k_chunk(a.kc + o0, a.kc + o1, lane, kr);
                load_v_chunk(a.vc + o0, a.vc + o1, lane, vr);
            },
            [&](int tok0, const uint4 (&kr)[2][4], const uint4 (&vr)[2][4]) {
                stage_v(vr, tok0, t1, vt, lane);
                f32x4 sc[2];
                const float cmax = chunk_scores_lim(kr, qop, tok0, lim, lim_min, lane, sc);
                chunk_update_staged(st, sc, cmax * a.scale_log2, true, a.scale_log2, vt, lane);
            });
    merge_waves<kSplitWaves>(st, smem, nc, [&](int h, int d, float o, float lse) {
        const size_t row = (size_t)(q0 + (r0 + h) / a.G) * a.Hq + (size_t)g * a.G + (r0 + h) % a.G;
        a.ws_o[(row * S + sp) * kD + d] = o;
        if (d == 0)
            a.ws_lse[row * S + sp] = lse;
    });
}

hipError_t launch_decode_multi(const MultiArgs &a, int B, int total_q, uint16_t *o, float *lse, hipStream_t stream)
{
    ATTN_LAUNCH(decode_multi_kernel, dim3(a.Hkv, a.num_splits, B * a.ncb), dim3(64 * kSplitWaves), 0, stream,
                       a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    MergeArgs m{a.ws_o, a.ws_lse, total_q * a.Hq, a.num_splits, o, lse};
    ATTN_LAUNCH(decode_merge_multi_kernel, dim3((total_q * a.Hq + 3) / 4), dim3(256), 0, stream, m);
    return hipGetLastError();
}

// ------------------------------------------------------------------ sequential with skip-softmax

// Sequences of up to this batch size are scheduled longest first.  Beyond it the batch spans enough
// rounds of workgroups that the dispatch order matters little, while every workgroup ranking all B
// rows (O(B^2)) costs more than it saves.  Measured (Hq 32, Hkv 8, lengths 256..4096 unless noted),
// ranked against index order: B = 64 with lengths 1k..32k 0.705 / 0.848 ms, B = 128 0.225 / 0.234 ms,
// B = 256 0.471 / 0.444 ms; the earlier per-workgroup ranking over global memory at B = 1024 took
// 4.56 ms against 1.60 in index order.
constexpr int kLptMaxBatch = 128;

// Batch row of the workgroup at dispatch position `pos`: with B <= kLptMaxBatch the rows are taken
// in order of decreasing length (ties by index), so that the longest sequences start first and the
// short ones fill in behind them; otherwise in index order.  The lengths are staged in `lens` (LDS,
// 16-byte aligned, >= kLptMaxBatch ints, free again when this returns) and read four at a time.
__device__ __forceinline__ int lpt_row(const int32_t *seq_lens, int B, int pos, int *slot, int32_t *lens)
{
    if (B > kLptMaxBatch)
        return pos;
    const int Bp = (B + 3) & ~3;
    for (int i = threadIdx.x; i < Bp; i += blockDim.x)
        lens[i] = i < B ? seq_lens[i] : -1; // padding: below every length, so it never outranks a row
    if (threadIdx.x == 0)
        *slot = pos;
    __syncthreads();
    const int4 *l4 = reinterpret_cast<const int4 *>(lens);
    for (int i = threadIdx.x; i < B; i += blockDim.x) {
        const int Li = lens[i];
        int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
        for (int q = 0; q < Bp / 4; ++q) {
            const int4 v = l4[q];
            const int j = 4 * q;
            r0 += (v.x > Li) || (v.x == Li && j < i);
            r1 += (v.y > Li) || (v.y == Li && j + 1 < i);
            r2 += (v.z > Li) || (v.z == Li && j + 2 < i);
            r3 += (v.w > Li) || (v.w == Li && j + 3 < i);
        }
        if (r0 + r1 + r2 + r3 == pos)
            *slot = i;
    }
    __syncthreads();
    return *slot;
}

// QDQ: NVFP4 fake quantization of P and V.  P is then taken against the sequential pass's running max
// (the max over all earlier tiles and this one), not the wave's own, so that its blocks are quantized
// at the scale the one sequential pass sees; the wave's state is kept relative to that same max.
template <bool QDQ>
__device__ __forceinline__ void decode_seq(const SeqArgs &a)
{
    __shared__ int row_slot;
    __shared__ __attribute__((aligned(16))) uint16_t smem[kSeqWaves * kVTile];
    // the batch lengths for the dispatch order go to the V staging area, unused until the main loop
    const int g = blockIdx.x,
              b = lpt_row(a.seq_lens, gridDim.y, blockIdx.y, &row_slot, reinterpret_cast<int32_t *>(smem));
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, j = lane >> 4;
    const int L = a.seq_lens[b];
    const int ntiles = (L + kSkipTile - 1) / kSkipTile;

    static_assert(sizeof(smem) >= kSeqWaves * 16 * (kD + 2) * sizeof(float), "merge buffer");
    static_assert(sizeof(smem) >= kLptMaxBatch * sizeof(int32_t), "batch lengths");
    __shared__ float tmax_buf[2][kSeqWaves][16];
    uint16_t *vt = smem + w * kVTile;
    const size_t row0 = (size_t)b * a.Hq + (size_t)g * a.G;

    if (a.skip_map) // tiles with no key: "not visited"
        for (int idx = threadIdx.x; idx < a.G * a.map_stride; idx += blockDim.x) {
            const int h = idx / a.map_stride, t = idx % a.map_stride;
            if (t >= ntiles)
                a.skip_map[(row0 + h) * a.map_stride + t] = 2;
        }

    bf16x8 qop[4];
    load_q_operand(a.q, b, g, a.Hq, a.G, lane, qop);
    Qdq qq{};
    if constexpr (QDQ)
        qq = Qdq{{a.p_enc, a.p_dec}, {a.v_enc, a.v_dec}, a.p_qdq != 0, a.v_qdq != 0};
    WaveState st;
    state_init(st);
    float run_max = kNegInf; // max of tile maxima over all earlier rounds (log2 units), head n
    // the block table through the constant address space: read-only for the kernel, so its uniform reads
    // are scalar loads, which leave the vector-memory counter (and the loads in flight) alone
    const __attribute__((address_space(4))) int32_t *btr =
        (const __attribute__((address_space(4))) int32_t *)(a.bt + (size_t)b * a.max_pages);
    const size_t slab = (size_t)kPage * kD;
    const size_t head_off = (size_t)g * slab;
    const size_t page_stride = (size_t)a.Hkv * slab;
    // Slab offsets of the two pages of tile t; a tile past the end borrows the sequence's first tile,
    // so that every round can load unconditionally (a tile past the end is never used).
    auto tile_pages = [&](int t, size_t &o0, size_t &o1) {
        const int tt = t < ntiles ? t : 0;
        const int tok0 = tt * kSkipTile;
        const int p0 = btr[tok0 / kPage];
        const int p1 = tok0 + kPage < L ? btr[tok0 / kPage + 1] : p0;
        o0 = (size_t)p0 * page_stride + head_off;
        o1 = (size_t)p1 * page_stride + head_off;
    };
    // K rows run two rounds ahead: the K of round r+2 is requested after round r's V, so that waiting
    // for that V (loads complete in order) leaves the K of rounds r+1 and r+2 in flight.  The three K
    // buffers rotate by name (the loop is unrolled by three): a register copy would wait for its load.
    size_t o0 = 0, o1 = 0, n0 = 0, n1 = 0;
    uint4 kb[3][2][4];
    if (ntiles > 0) {
        tile_pages(w, o0, o1);
        load_k_chunk(a.kc + o0, a.kc + o1, lane, kb[0]);
        tile_pages(w + kSeqWaves, n0, n1);
        load_k_chunk(a.kc + n0, a.kc + n1, lane, kb[1]);
    }
    int parity = 0;
    // one round: scores of tile base + w from kc, the round's decisions, its V, the K of round r+2 into kq
    auto round = [&](int base, uint4 (&kc)[2][4], uint4 (&kq)[2][4]) {
        const int t = base + w;
        const int tok0 = t * kSkipTile;
        const bool active = t < ntiles;
        f32x4 sc[2];
        float tmax = kNegInf;
        if (active)
            tmax = chunk_scores(kc, qop, tok0, L, lane, sc) * a.scale_log2;
        if (j == 0)
            tmax_buf[parity][w][n] = tmax;
        // LDS write visible, then a plain barrier: the K loads of the next rounds stay in flight
        __builtin_amdgcn_s_waitcnt(kWaitLdsOnly);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        float prefix = run_max, round_max = run_max;
#pragma unroll
        for (int ww = 0; ww < kSeqWaves; ++ww) {
            const float tm = tmax_buf[parity][ww][n];
            if (ww < w)
                prefix = fmaxf(prefix, tm);
            round_max = fmaxf(round_max, tm);
        }
        run_max = round_max;
        bool keep = false, any_keep = false;
        uint4 vr[2][4];
        if (active) {
            // skip iff a running max exists and tmax - m < log2(threshold)
            const bool skip = prefix != kNegInf && tmax - prefix < a.log2_thr;
            keep = !skip;
            // V is needed when any real head of the group keeps the tile
            any_keep = __any(keep && n < a.G);
            if (any_keep)
                load_v_chunk(a.vc + o0, a.vc + o1, lane, vr);
            if (a.skip_map && j == 0 && n < a.G)
                a.skip_map[(row0 + n) * a.map_stride + t] = skip ? 1 : 0;
        }
        size_t q0, q1;
        tile_pages(t + 2 * kSeqWaves, q0, q1);
        load_k_chunk(a.kc + q0, a.kc + q1, lane, kq);
        if (active && any_keep) {
            if constexpr (QDQ)
                chunk_update<true>(st, sc, fmaxf(prefix, tmax), keep, vr, tok0, L, a.scale_log2, vt, lane, qq);
            else
                chunk_update(st, sc, tmax, keep, vr, tok0, L, a.scale_log2, vt, lane);
        }
        o0 = n0;
        o1 = n1;
        n0 = q0;
        n1 = q1;
        parity ^= 1;
    };
    for (int base = 0; base < ntiles;) {
        round(base, kb[0], kb[2]);
        base += kSeqWaves;
        if (base >= ntiles)
            break;
        round(base, kb[1], kb[0]);
        base += kSeqWaves;
        if (base >= ntiles)
            break;
        round(base, kb[2], kb[1]);
        base += kSeqWaves;
    }
    merge_waves<kSeqWaves>(st, smem, a.G, [&](int h, int d, float o, float lse) {
        a.o[(row0 + h) * kD + d] = f32_to_bf16(o);
        if (a.lse && d == 0)
            a.lse[row0 + h] = lse;
    });
}

__global__ __launch_bounds__(64 * kSeqWaves) void decode_seq_kernel(SeqArgs a) { decode_seq<false>(a); }
__global__ __launch_bounds__(64 * kSeqWaves) void decode_seq_qdq_kernel(SeqArgs a) { decode_seq<true>(a); }

hipError_t launch_decode_seq(const SeqArgs &a, int B, hipStream_t stream)
{
    if (a.p_qdq || a.v_qdq)
        ATTN_LAUNCH(decode_seq_qdq_kernel, dim3(a.Hkv, B), dim3(64 * kSeqWaves), 0, stream, a);
    else
        ATTN_LAUNCH(decode_seq_kernel, dim3(a.Hkv, B), dim3(64 * kSeqWaves), 0, stream, a);
    return hipGetLastError();
}

} // namespace attn
