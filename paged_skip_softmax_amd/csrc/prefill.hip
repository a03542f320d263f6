// Varlen prefill attention for gfx950 ("Model-Optimizer: Add Triton unified attention kernel":
// variable-length batching, GQA, causal and non-causal; sequences packed THD with cu_seqlens), with
// optional skip-softmax on 32-key tiles ("TensorRT-LLM: Skip Softmax Attention", Description).
//
// bf16 kernel: one workgroup of 4 waves per (query head, sequence, 128-row query tile); each wave owns
// 32 query rows and keeps Q^T in registers as the MFMA B operand for the whole loop.  Per 64-key
// iteration the workgroup stages the K and V tiles in LDS (coalesced 16-B loads, padded rows) and
// every wave computes
//   S^T[64 keys x 32 rows] = K[64 x D] . Q^T[D x 32]      2 x D/16 MFMA 32x32x16 (bf16, fp32 acc)
//   online softmax in the log2 domain (scale * log2 e folded into one FMA)
//   O^T[D x 32] += V^T[D x 64] . P^T[64 x 32]              D/32 x 4 MFMA 32x32x16
// The key order inside P.V follows the S^T register layout, so P feeds the second product straight
// from registers.  Query tiles are dispatched from the last (the most keys under a causal mask) to the
// first.  The two 32-key halves of an iteration are exactly the skip tiles (tiles aligned to key 0);
// a tile skipped by every row of a wave costs no exp and no P.V.
//
// fp32 kernel: one lane per query row on the vector ALUs (exact fp32 products, no reduced-precision
// operand), 32-key K/V tiles staged in LDS, the same online softmax and the same skip rule.
#include "kcommon.h"
#include "launch.h"

namespace attn {

constexpr int kBM = 128;     // query rows per workgroup
constexpr int kBN = 64;      // keys per iteration
constexpr int kPrefWaves = 4;

template <int D>
struct PrefillSmem {
    static constexpr int kPitch = D + 8; // bf16 elements per LDS row (16-B aligned, conflict-free)
    uint16_t k[kBN * kPitch];
    uint16_t v[kBN * kPitch];
};

template <int D, bool SKIP>
__global__ __launch_bounds__(64 * kPrefWaves) void prefill_bf16_kernel(PrefillArgs a)
{
    constexpr int kPitch = PrefillSmem<D>::kPitch;
    constexpr int kSteps = D / 16;  // MFMA k-steps over D
    constexpr int kDB = D / 32;     // 32-wide d blocks of the output
    __shared__ __attribute__((aligned(16))) PrefillSmem<D> sm;

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
    float m = kNegInf, l = 0.f;

    uint8_t *maprow = nullptr;
    if (SKIP && a.skip_map && row_ok) {
        maprow = a.skip_map + ((size_t)(q0 + qi) * a.Hq + h) * a.map_stride;
        if (J == 0)
            for (int t = (kend_row + kSkipTile - 1) / kSkipTile; t < a.map_stride; ++t)
                maprow[t] = 2;
    }

    constexpr int kChunks = D / 8;               // 16-B chunks per key row
    constexpr int kRowsPerPass = 256 / kChunks;
    for (int kb = 0; kb < kend; kb += kBN) {
        __syncthreads();
#pragma unroll
        for (int p = 0; p < kBN / kRowsPerPass; ++p) {
            const int key = tid / kChunks + p * kRowsPerPass, c = tid % kChunks;
            uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
            if (kb + key < Lk) {
                const size_t off = ((size_t)(k0 + kb + key) * a.Hkv + g) * D + 8 * c;
                kv = ld16(kg + off);
                vv = ld16(vg + off);
            }
            st16(sm.k + key * kPitch + 8 * c, kv);
            st16(sm.v + key * kPitch + 8 * c, vv);
        }
        __syncthreads();
        if (kb >= kend_w)
            continue; // every row of this wave is past the diagonal

        f32x16 sc[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sc[kk][i] = 0.f;
#pragma unroll
            for (int s = 0; s < kSteps; ++s) {
                const bf16x8 ka = as_bf16x8(ld16(sm.k + (32 * kk + n) * kPitch + 16 * s + 8 * J));
                sc[kk] = mfma32(ka, qop[s], sc[kk]);
            }
        }
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
        float m_new = m;
        if (SKIP) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bool visited = tmax[kk] != kNegInf;
                const bool skip = visited && m_new != kNegInf && tmax[kk] - m_new < a.log2_thr;
                use[kk] = visited && !skip;
                if (use[kk])
                    m_new = fmaxf(m_new, tmax[kk]);
                // tiles past the row's last visible key were marked 2 up front
                if (maprow && J == 0 && visited)
                    maprow[(kb >> 5) + kk] = skip ? 1 : 0;
            }
        } else {
            m_new = fmaxf(m, fmaxf(tmax[0], tmax[1]));
        }
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = exp2_fast(m - m_use);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < kDB; ++db)
            acc[db] *= alpha;
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
#pragma unroll
                for (int db = 0; db < kDB; ++db) {
                    const int d = 32 * db + n;
                    bf16x8 va;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int key = 32 * kk + 16 * u + 8 * (e / 4) + 4 * J + (e % 4);
                        va[e] = __builtin_bit_cast(__bf16, sm.v[key * kPitch + d]);
                    }
                    acc[db] = mfma32(va, pop, acc[db]);
                }
            }
        }
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

constexpr int kF32Tile = 32; // keys per LDS tile = skip tile

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a)
{
    __shared__ float ks[kF32Tile][D];
    __shared__ float vs[kF32Tile][D];
    const int h = blockIdx.x, b = blockIdx.y;
    const int qt = gridDim.z - 1 - blockIdx.z;
    const int q0 = a.cu_q[b], Lq = a.cu_q[b + 1] - q0;
    const int k0 = a.cu_k[b], Lk = a.cu_k[b + 1] - k0;
    const int m0 = qt * 64;
    if (m0 >= Lq)
        return;
    const int g = h / a.G, lane = threadIdx.x;
    const int qi = m0 + lane;
    const bool row_ok = qi < Lq;
    const int diag = Lk - Lq;
    const int last_row = min(m0 + 64, Lq) - 1;
    const int kend = a.causal ? max(0, min(Lk, last_row + 1 + diag)) : Lk;
    const int kend_row = !row_ok ? 0 : (a.causal ? max(0, min(Lk, qi + 1 + diag)) : Lk);
    const float *qg = static_cast<const float *>(a.q);
    const float *kg = static_cast<const float *>(a.k);
    const float *vg = static_cast<const float *>(a.v);

    float q[D], acc[D];
#pragma unroll
    for (int d = 0; d < D; ++d) {
        q[d] = row_ok ? qg[((size_t)(q0 + qi) * a.Hq + h) * D + d] : 0.f;
        acc[d] = 0.f;
    }
    float m = kNegInf, l = 0.f;
    uint8_t *maprow = (a.skip_map && row_ok) ? a.skip_map + ((size_t)(q0 + qi) * a.Hq + h) * a.map_stride : nullptr;
    if (maprow)
        for (int t = (kend_row + kF32Tile - 1) / kF32Tile; t < a.map_stride; ++t)
            maprow[t] = 2;

    for (int kb = 0; kb < kend; kb += kF32Tile) {
        __syncthreads();
        for (int idx = lane; idx < kF32Tile * D; idx += 64) {
            const int key = idx / D, d = idx % D;
            const bool in = kb + key < Lk;
            const size_t off = ((size_t)(k0 + kb + key) * a.Hkv + g) * D + d;
            ks[key][d] = in ? kg[off] : 0.f;
            vs[key][d] = in ? vg[off] : 0.f;
        }
        __syncthreads();
        if (kb >= kend_row)
            continue;
        const int nk = min(kF32Tile, kend_row - kb);
        float s[kF32Tile];
        float tmax = kNegInf;
#pragma unroll
        for (int j = 0; j < kF32Tile; ++j) {
            float t = 0.f;
#pragma unroll
            for (int d = 0; d < D; ++d)
                t = fmaf(q[d], ks[j][d], t);
            s[j] = j < nk ? t * a.scale_log2 : kNegInf;
            tmax = fmaxf(tmax, s[j]);
        }
        const bool skip = m != kNegInf && tmax - m < a.log2_thr;
        if (maprow)
            maprow[kb / kF32Tile] = skip ? 1 : 0;
        if (skip)
            continue;
        const float m_new = fmaxf(m, tmax);
        const float alpha = exp2_fast(m - m_new);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < D; ++d)
            acc[d] *= alpha;
#pragma unroll
        for (int j = 0; j < kF32Tile; ++j) {
            if (j < nk) {
                const float p = exp2_fast(s[j] - m_new);
                l += p;
#pragma unroll
                for (int d = 0; d < D; ++d)
                    acc[d] = fmaf(p, vs[j][d], acc[d]);
            }
        }
        m = m_new;
    }
    if (!row_ok)
        return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float *og = static_cast<float *>(a.o) + ((size_t)(q0 + qi) * a.Hq + h) * D;
#pragma unroll
    for (int d = 0; d < D; ++d)
        og[d] = acc[d] * inv;
    if (a.lse)
        a.lse[(size_t)(q0 + qi) * a.Hq + h] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
}

hipError_t launch_prefill(const PrefillArgs &a, bool bf16, int D, hipStream_t stream)
{
    const bool skip = a.log2_thr != kNegInf || a.skip_map != nullptr;
    if (bf16) {
        dim3 grid(a.Hq, a.B, (a.max_q + kBM - 1) / kBM), block(64 * kPrefWaves);
        if (D == 128) {
            if (skip)
                hipLaunchKernelGGL((prefill_bf16_kernel<128, true>), grid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((prefill_bf16_kernel<128, false>), grid, block, 0, stream, a);
        } else if (D == 64) {
            if (skip)
                hipLaunchKernelGGL((prefill_bf16_kernel<64, true>), grid, block, 0, stream, a);
            else
                hipLaunchKernelGGL((prefill_bf16_kernel<64, false>), grid, block, 0, stream, a);
        } else {
            return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (D != 64)
        return hipErrorNotSupported;
    dim3 grid(a.Hq, a.B, (a.max_q + 63) / 64);
    hipLaunchKernelGGL((prefill_f32_kernel<64>), grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

} // namespace attn
