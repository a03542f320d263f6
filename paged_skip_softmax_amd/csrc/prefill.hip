// Varlen prefill attention for gfx950 ("Model-Optimizer: Add Triton unified attention kernel":
// variable-length batching, GQA, causal and non-causal; sequences packed THD with cu_seqlens), with
// optional skip-softmax on 32-key tiles ("TensorRT-LLM: Skip Softmax Attention", Description).
//
// Head dim 128 in bf16 runs in prefill_d128.hip; this file holds the bf16 kernel for head dim 64 and
// the fp32 kernel.
//
// bf16 kernel: one workgroup of 4 waves per (query head, sequence, 128-row query tile); each wave owns
// 32 query rows and keeps Q^T in registers as the MFMA B operand for the whole loop.  Per 64-key
// iteration every wave computes
//   S^T[64 keys x 32 rows] = K[64 x D] . Q^T[D x 32]      2 x D/16 MFMA 32x32x16 (bf16, fp32 acc)
//   online softmax in the log2 domain (scale * log2 e folded into one FMA)
//   O^T[D x 32] += V^T[D x 64] . P^T[64 x 32]              D/32 x 4 MFMA 32x32x16
// K and V tiles are double-buffered in LDS: once a wave has issued the QK^T MFMAs of tile i, its
// lanes load tile i+1 into registers (coalesced 16-B buffer loads; rows past the sequence read as 0)
// and store it to the other buffer after the P.V product, so one barrier per iteration suffices and
// the load latency hides behind the softmax and P.V of tile i.  K is read back as the A operand with
// 16-B reads; V, stored key-major as loaded, is read back
// transposed with ds_read_b64_tr_b16 (lane j of each 16-lane group addresses key k0 + j/4, dims
// 4(j%4)..+3, and receives dims of its own column for keys k0..k0+3).  The key order inside P.V follows
// the S^T register layout, so P feeds the second product straight from registers.
// The running max used for the exponentials is only raised when a row's max exceeds it by more than 8
// (log2 units, a factor 2^8), so the O and l rescale is rare; the result is the same softmax, with
// unnormalised weights P <= 2^8.
// Query tiles are dispatched from the last (the most keys under a causal mask) to the first.  The two
// 32-key halves of an iteration are exactly the skip tiles (tiles aligned to key 0); skip decisions use
// the exact running max, and a tile skipped by every row of a wave costs no exp and no P.V.
//
// fp32 kernel: one lane per query row on the vector ALUs (exact fp32 products, no reduced-precision
// operand), 32-key K/V tiles staged in LDS, the same online softmax and the same skip rule.
#include "kcommon.h"
#include "launch.h"

namespace attn {

constexpr int kBM = 128;     // query rows per workgroup
constexpr int kBN = 64;      // keys per iteration
constexpr int kPrefWaves = 4;
constexpr float kRescaleSlack = 8.f; // log2 units the stale max may trail the true max

typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct PrefillSmem {
    static constexpr int kKP = D + 8;  // K row pitch (elements): 16-B row reads spread over all banks
    static constexpr int kVP = D + 16; // V row pitch (elements): transposed 8-B reads spread over banks
    uint16_t k[2][kBN * kKP];
    uint16_t v[2][kBN * kVP];
};

// Buffer-resource word 3 for gfx9-family raw buffers (32-bit data format, no swizzle).
constexpr int kBufWord3 = 0x00020000;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 buffer_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Transposed LDS read: 4 consecutive keys of one dim column (see the file comment).
__device__ __forceinline__ uint2 lds_read_tr(const uint16_t *p)
{
    const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4 *)(p));
    return __builtin_bit_cast(uint2, r);
}

template <int D, bool SKIP>
__global__ __launch_bounds__(64 * kPrefWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(PrefillArgs a)
{
    using Smem = PrefillSmem<D>;
    constexpr int KP = Smem::kKP, VP = Smem::kVP;
    constexpr int kSteps = D / 16;  // MFMA k-steps over D
    constexpr int kDB = D / 32;     // 32-wide d blocks of the output
    constexpr int kChunks = D / 8;  // 16-B chunks per key row
    constexpr int kRowsPerPass = 64 * kPrefWaves / kChunks;
    constexpr int kPasses = kBN / kRowsPerPass;
    __shared__ __attribute__((aligned(16))) Smem sm;

    const int h = blockIdx.x, b = blockIdx.y;
    const int qt = gridDim.z - 1 - blockIdx.z;
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
    const int m0 = qt * kBM;
    if (m0 >= Lq)
        return;
    const int g = h / a.G;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n = lane & 31, J = lane >> 5;
    const int diag = Lk - Lq;                 // row i sees keys j <= i + diag (causal)
    const int qi = m0 + 32 * w + n;           // this lane's query row
    const bool row_ok = qi < Lq;
    const uint16_t *qg = static_cast<const uint16_t *>(a.q);
    const uint16_t *kg = static_cast<const uint16_t *>(a.k);
    const uint16_t *vg = static_cast<const uint16_t *>(a.v);

    // keys the workgroup / this wave / this row can see
    const int last_row = min(m0 + kBM, Lq) - 1;
    const int kend = a.causal ? max(0, min(Lk, last_row + 1 + diag)) : Lk;
    const int wlast = min(m0 + 32 * w + 31, Lq - 1);
    const int kend_w = a.causal ? max(0, min(Lk, wlast + 1 + diag)) : Lk;
    const int kend_row = a.causal ? max(0, min(Lk, qi + 1 + diag)) : Lk;

    bf16x8 qop[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s)
        qop[s] = row_ok ? as_bf16x8(ld16(qg + ((size_t)(q0 + qi) * a.Hq + h) * D + 16 * s + 8 * J))
                        : as_bf16x8(make_uint4(0, 0, 0, 0));

    f32x16 acc[kDB];
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            acc[db][i] = 0.f;
    float m = kNegInf, l = 0.f;   // m: max used for the exponentials (may trail the true max)
    float m_true = kNegInf;       // exact running max over processed tiles (skip decisions)

    uint8_t *maprow = nullptr;
    if (SKIP && a.skip_map && row_ok) {
        maprow = a.skip_map + ((size_t)(q0 + qi) * a.Hq + h) * a.map_stride;
        if (J == 0)
            for (int t = (kend_row + kSkipTile - 1) / kSkipTile; t < a.map_stride; ++t)
                maprow[t] = 2;
    }

    // cooperative tile loads: thread -> (key tid / kChunks + p * kRowsPerPass, chunk tid % kChunks),
    // through buffer resources covering exactly this sequence's rows of KV head g: rows past the
    // sequence read as zero (range-checked by the hardware), so the loads need no branch or clamp.
    // The per-thread offset stays in one VGPR; the tile and pass offsets go in the scalar offset.
    const int ld_key = tid / kChunks, ld_c = tid % kChunks;
    const uint32_t row_bytes = (uint32_t)a.Hkv * D * 2;
    const uint32_t seq_bytes = Lk > 0 ? ((uint32_t)(Lk - 1) * a.Hkv + 1) * D * 2 : 0;
    const size_t head0 = ((size_t)k0 * a.Hkv + g) * D;
    const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)(kg + head0), 0, seq_bytes, kBufWord3);
    const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)(vg + head0), 0, seq_bytes, kBufWord3);
    const uint32_t voff = ld_key * row_bytes + 16 * ld_c;
    uint4 kn[kPasses], vn[kPasses];
    auto load_tile = [&](int kb) {
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const uint32_t soff = (uint32_t)(kb + p * kRowsPerPass) * row_bytes;
            kn[p] = buffer_ld16(krs, voff, soff);
            vn[p] = buffer_ld16(vrs, voff, soff);
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int p = 0; p < kPasses; ++p) {
            const int key = ld_key + p * kRowsPerPass;
            st16(sm.k[buf] + key * KP + 8 * ld_c, kn[p]);
            st16(sm.v[buf] + key * VP + 8 * ld_c, vn[p]);
        }
    };

    const int niter = (kend + kBN - 1) / kBN;
    if (niter > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();
    // transposed-read lane address: key offset j/4 within the 4-key group, dims 4 (j%4) of the
    // 16-dim half (lane/16) % 2 of the 32-dim block
    const int tr_key = (lane & 15) >> 2;
    const int tr_dim = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

    for (int it = 0; it < niter; ++it) {
        const int kb = it * kBN, cur = it & 1;
        if (kb < kend_w) {
            const uint16_t *Kl = sm.k[cur];
            const uint16_t *Vl = sm.v[cur];
            f32x16 sc[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint4 kop[kSteps];
#pragma unroll
                for (int s = 0; s < kSteps; ++s)
                    kop[s] = ld16(Kl + (32 * kk + n) * KP + 16 * s + 8 * J);
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    sc[kk][i] = 0.f;
#pragma unroll
                for (int s = 0; s < kSteps; ++s)
                    sc[kk] = mfma32(as_bf16x8(kop[s]), qop[s], sc[kk]);
            }
            if (it + 1 < niter)
                load_tile(kb + kBN);
            // mask keys past the sequence and past the causal diagonal
            const bool need_mask = kb + kBN > Lk || (a.causal && kb + kBN - 1 > m0 + 32 * w + diag);
            if (need_mask) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kb + 32 * kk + 8 * (i / 4) + 4 * J + (i % 4);
                        if (key >= kend_row)
                            sc[kk][i] = kNegInf;
                    }
            }
            float tmax[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                float t = sc[kk][0];
#pragma unroll
                for (int i = 1; i < 16; ++i)
                    t = fmaxf(t, sc[kk][i]);
                tmax[kk] = fmaxf(t, __shfl_xor(t, 32)) * a.scale_log2;
            }
            bool use[2] = {true, true};
            if (SKIP) {
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const bool visited = tmax[kk] != kNegInf;
                    const bool skip = visited && m_true != kNegInf && tmax[kk] - m_true < a.log2_thr;
                    use[kk] = visited && !skip;
                    if (use[kk])
                        m_true = fmaxf(m_true, tmax[kk]);
                    // tiles past the row's last visible key were marked 2 up front
                    if (maprow && J == 0 && visited)
                        maprow[(kb >> 5) + kk] = skip ? 1 : 0;
                }
            }
            const float m_tile = fmaxf(use[0] ? tmax[0] : kNegInf, use[1] ? tmax[1] : kNegInf);
            const bool raise = m_tile > m + kRescaleSlack;
            if (__any(raise)) {
                const float m_new = raise ? m_tile : m;
                // raising from m = -inf gives 0 (acc and l are still 0); rows that do not raise keep their
                // state (also rows that have seen no key yet, whose m - m_new would be -inf - -inf)
                const float alpha = raise ? exp2_fast(m - m_new) : 1.f;
                m = m_new;
                l *= alpha;
#pragma unroll
                for (int db = 0; db < kDB; ++db)
                    acc[db] *= alpha;
            }
            const float m_use = m == kNegInf ? 0.f : m;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if (SKIP && !__any(use[kk]))
                    continue; // no row of the wave keeps this tile: no exp, no P.V
                float p[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    p[i] = (!SKIP || use[kk]) ? exp2_fast(fmaf(sc[kk][i], a.scale_log2, -m_use)) : 0.f;
                    l += p[i];
                }
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    bf16x8 pop;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        pop[e] = (__bf16)p[8 * u + e];
                    const int ka = 32 * kk + 16 * u + 4 * J + tr_key; // keys k0..k0+3 of slots 0..3
#pragma unroll
                    for (int db = 0; db < kDB; ++db) {
                        const uint16_t *vp = Vl + ka * VP + 32 * db + tr_dim;
                        const uint2 lo = lds_read_tr(vp);
                        const uint2 hi = lds_read_tr(vp + 8 * VP); // keys k0+8..k0+11: slots 4..7
                        acc[db] = mfma32(as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y)), pop, acc[db]);
                    }
                }
            }
        }
        if (it + 1 < niter)
            store_tile(cur ^ 1);
        __syncthreads();
    }

    l += __shfl_xor(l, 32);
    if (!row_ok)
        return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t *og = static_cast<uint16_t *>(a.o) + ((size_t)(q0 + qi) * a.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < kDB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            uint2 pk;
            pk.x = pack_bf16x2(acc[db][4 * r] * inv, acc[db][4 * r + 1] * inv);
            pk.y = pack_bf16x2(acc[db][4 * r + 2] * inv, acc[db][4 * r + 3] * inv);
            *reinterpret_cast<uint2 *>(og + 32 * db + 8 * r + 4 * J) = pk;
        }
    if (a.lse && J == 0)
        a.lse[(size_t)(q0 + qi) * a.Hq + h] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
}

// ------------------------------------------------------------------ fp32

constexpr int kF32Tile = 32;                  // keys per LDS tile = skip tile
constexpr int kF32Rows = 64;                  // query rows per workgroup
constexpr int kF32Parts = 4;                  // lanes per row (a lane quad), each with D / 4 dims
constexpr int kF32Threads = kF32Rows * kF32Parts;

// fp32 on the VALU: a lane quad per query row, each lane holding a quarter of the dims of q and of the
// output; a score is the quad's four partial dot products summed across the quad.  K and V tiles of 32
// keys are double-buffered in LDS, the next one loaded into registers while the current one is used.
template <int D>
__global__ __launch_bounds__(kF32Threads) void prefill_f32_kernel(PrefillArgs a)
{
    constexpr int DP = D / kF32Parts;                   // dims per lane
    constexpr int kLd = kF32Tile * D / 4 / kF32Threads; // float4 loads per lane per tile, K and V each
    static_assert(kLd >= 1 && kF32Tile * D == kLd * 4 * kF32Threads, "whole float4 loads per lane");
    __shared__ float4 ks[2][kF32Tile][D / 4];
    __shared__ float4 vs[2][kF32Tile][D / 4];
    const int h = blockIdx.x, b = blockIdx.y;
    const int qt = gridDim.z - 1 - blockIdx.z;
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
    const int m0 = qt * kF32Rows;
    if (m0 >= Lq)
        return;
    const int g = h / a.G, tid = threadIdx.x;
    const int row = tid / kF32Parts, part = tid % kF32Parts;
    const int qi = m0 + row;
    const bool row_ok = qi < Lq;
    const int diag = Lk - Lq;
    const int last_row = min(m0 + kF32Rows, Lq) - 1;
    const int kend = a.causal ? max(0, min(Lk, last_row + 1 + diag)) : Lk;
    const int kend_row = !row_ok ? 0 : (a.causal ? max(0, min(Lk, qi + 1 + diag)) : Lk);
    const float *qg = static_cast<const float *>(a.q);
    const float4 *kg = static_cast<const float4 *>(a.k);
    const float4 *vg = static_cast<const float4 *>(a.v);

    float q[DP], acc[DP];
#pragma unroll
    for (int d = 0; d < DP; ++d) {
        q[d] = row_ok ? qg[((size_t)(q0 + qi) * a.Hq + h) * D + DP * part + d] : 0.f;
        acc[d] = 0.f;
    }
    float m = kNegInf, l = 0.f;
    uint8_t *maprow = (a.skip_map && row_ok && part == 0)
                          ? a.skip_map + ((size_t)(q0 + qi) * a.Hq + h) * a.map_stride : nullptr;
    if (maprow)
        for (int t = (kend_row + kF32Tile - 1) / kF32Tile; t < a.map_stride; ++t)
            maprow[t] = 2;

    // tile loads: float4 index e = tid + kF32Threads * i of the tile, key e / (D / 4), dims 4 (e % (D / 4))
    float4 kr[kLd], vr[kLd];
    auto load = [&](int kb) {
#pragma unroll
        for (int i = 0; i < kLd; ++i) {
            const int e = tid + kF32Threads * i, key = e / (D / 4), c = e % (D / 4);
            const bool in = kb + key < Lk;
            const size_t off = ((size_t)(k0 + kb + key) * a.Hkv + g) * (D / 4) + c;
            kr[i] = in ? kg[off] : make_float4(0.f, 0.f, 0.f, 0.f);
            vr[i] = in ? vg[off] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kLd; ++i) {
            const int e = tid + kF32Threads * i, key = e / (D / 4), c = e % (D / 4);
            ks[buf][key][c] = kr[i];
            vs[buf][key][c] = vr[i];
        }
    };
    const int ntiles = (kend + kF32Tile - 1) / kF32Tile;
    if (ntiles > 0) {
        load(0);
        store(0);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
        const int kb = t * kF32Tile, buf = t & 1;
        if (t + 1 < ntiles)
            load(kb + kF32Tile);
        if (kb < kend_row) {
            const int nk = min(kF32Tile, kend_row - kb);
            float s[kF32Tile];
            float tmax = kNegInf;
#pragma unroll
            for (int j = 0; j < kF32Tile; ++j) {
                float x = 0.f;
#pragma unroll
                for (int c = 0; c < DP / 4; ++c) {
                    const float4 kv = ks[buf][j][DP / 4 * part + c];
                    x = fmaf(q[4 * c], kv.x, x);
                    x = fmaf(q[4 * c + 1], kv.y, x);
                    x = fmaf(q[4 * c + 2], kv.z, x);
                    x = fmaf(q[4 * c + 3], kv.w, x);
                }
                x += __shfl_xor(x, 1);
                x += __shfl_xor(x, 2);
                s[j] = j < nk ? x * a.scale_log2 : kNegInf;
                tmax = fmaxf(tmax, s[j]);
            }
            const bool skip = m != kNegInf && tmax - m < a.log2_thr;
            if (maprow)
                maprow[kb / kF32Tile] = skip ? 1 : 0;
            if (!skip) {
                const float m_new = fmaxf(m, tmax);
                const float alpha = exp2_fast(m - m_new);
                l *= alpha;
#pragma unroll
                for (int d = 0; d < DP; ++d)
                    acc[d] *= alpha;
#pragma unroll
                for (int j = 0; j < kF32Tile; ++j) {
                    if (j < nk) {
                        const float p = exp2_fast(s[j] - m_new);
                        l += p;
#pragma unroll
                        for (int c = 0; c < DP / 4; ++c) {
                            const float4 vv = vs[buf][j][DP / 4 * part + c];
                            acc[4 * c] = fmaf(p, vv.x, acc[4 * c]);
                            acc[4 * c + 1] = fmaf(p, vv.y, acc[4 * c + 1]);
                            acc[4 * c + 2] = fmaf(p, vv.z, acc[4 * c + 2]);
                            acc[4 * c + 3] = fmaf(p, vv.w, acc[4 * c + 3]);
                        }
                    }
                }
                m = m_new;
            }
        }
        // the other buffer was last read during tile t - 1, which every lane finished before the barrier
        // that ended it
        if (t + 1 < ntiles)
            store(buf ^ 1);
        __syncthreads();
    }
    if (!row_ok)
        return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *og = static_cast<float *>(a.o) + ((size_t)(q0 + qi) * a.Hq + h) * D + DP * part;
#pragma unroll
    for (int d = 0; d < DP; ++d)
        og[d] = acc[d] * inv;
    if (a.lse && part == 0)
        a.lse[(size_t)(q0 + qi) * a.Hq + h] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
}

hipError_t launch_prefill(const PrefillArgs &a, bool bf16, int D, hipStream_t stream)
{
    const bool skip = a.log2_thr != kNegInf || a.skip_map != nullptr;
    if (bf16) {
        dim3 grid(a.Hq, a.B, (a.max_q + kBM - 1) / kBM), block(64 * kPrefWaves);
        if (D == 128) {
            return launch_prefill_d128(a, stream);
        } else if (D == 64) {
            if (skip)
                ATTN_LAUNCH((prefill_bf16_kernel<64, true>), grid, block, 0, stream, a);
            else
                ATTN_LAUNCH((prefill_bf16_kernel<64, false>), grid, block, 0, stream, a);
        } else {
            return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (D != 64)
        return hipErrorNotSupported;
    dim3 grid(a.Hq, a.B, (a.max_q + kF32Rows - 1) / kF32Rows);
    ATTN_LAUNCH((prefill_f32_kernel<64>), grid, dim3(kF32Threads), 0, stream, a);
    return hipGetLastError();
}

} // namespace attn
