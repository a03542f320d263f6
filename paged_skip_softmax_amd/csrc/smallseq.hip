// Small-seq cross-attention for gfx950: one query token per sequence and at most 16 keys, huge batch
// ("ROCm TransformerEngine: Integrate CK varlen cross attention for small-seq (s_q=1, s_kv<=16)",
// change list: scores, mask + softmax, output, and the attention weights [tokens_q, h_q, 1, max_s_kv]).
//
// The op is a gather of at most 16 key and value rows per (sequence, head) -- HBM-bound with ~1 flop per
// byte -- so it runs on the vector ALUs, fused into one kernel: one workgroup of 256 lanes per sequence
// and per block of 16 heads; lane (h = lane/16, c = lane%16) owns the 8 dims [8c, 8c+8) of head h.
// Every key row of a sequence is one contiguous H x 128 bf16 block, so each wave instruction reads a
// contiguous 1 KB and all key and value rows of the sequence are in flight at once.  Scores are reduced
// over the 16 lanes of a head with xor shuffles; softmax runs in registers in the log2 domain.
#include "kcommon.h"
#include "launch.h"

namespace attn {

constexpr int kSmallD = 128;
constexpr int kSmallMaxS = 16;

__device__ __forceinline__ float dot8_bf16(uint4 a, const float qf[8])
{
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        s = fmaf(bf16_lo(w[e]), qf[2 * e], s);
        s = fmaf(bf16_hi(w[e]), qf[2 * e + 1], s);
    }
    return s;
}

__device__ __forceinline__ float sum16(float v)
{
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 2);
    return v + __shfl_xor(v, 1);
}

__global__ __launch_bounds__(256) void smallseq_kernel(SmallArgs a)
{
    const int b = blockIdx.x;
    const int h = blockIdx.y * 16 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    if (h >= a.H)
        return; // whole 16-lane head groups exit together
    const int kv0 = a.cu[b];
    const int s = min(a.cu[b + 1] - kv0, kSmallMaxS);
    const size_t rowq = (size_t)b * a.H + h;
    const size_t stride = (size_t)a.H * kSmallD; // elements between consecutive key rows

    float qf[8];
    {
        const uint4 qv = ld16(a.q + rowq * kSmallD + 8 * c);
        const uint32_t w[4] = {qv.x, qv.y, qv.z, qv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qf[2 * e] = bf16_lo(w[e]);
            qf[2 * e + 1] = bf16_hi(w[e]);
        }
    }
    const uint16_t *kp = a.k + ((size_t)kv0 * a.H + h) * kSmallD + 8 * c;
    const uint16_t *vp = a.v + ((size_t)kv0 * a.H + h) * kSmallD + 8 * c;
    uint4 kr[kSmallMaxS], vr[kSmallMaxS];
#pragma unroll
    for (int j = 0; j < kSmallMaxS; ++j)
        if (j < s)
            kr[j] = ld16(kp + j * stride);
#pragma unroll
    for (int j = 0; j < kSmallMaxS; ++j)
        if (j < s)
            vr[j] = ld16(vp + j * stride);

    float sc[kSmallMaxS];
    float m = kNegInf;
#pragma unroll
    for (int j = 0; j < kSmallMaxS; ++j) {
        sc[j] = kNegInf;
        if (j < s) {
            sc[j] = sum16(dot8_bf16(kr[j], qf)) * a.scale_log2;
            m = fmaxf(m, sc[j]);
        }
    }
    float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float den = 0.f, inv = 0.f;
    if (s > 0) {
#pragma unroll
        for (int j = 0; j < kSmallMaxS; ++j) {
            if (j < s) {
                sc[j] = exp2_fast(sc[j] - m); // sc now holds unnormalised probabilities
                den += sc[j];
                const uint32_t w[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[2 * e] = fmaf(sc[j], bf16_lo(w[e]), o[2 * e]);
                    o[2 * e + 1] = fmaf(sc[j], bf16_hi(w[e]), o[2 * e + 1]);
                }
            }
        }
        inv = 1.f / den;
    }
    uint4 ov;
    ov.x = pack_bf16x2(o[0] * inv, o[1] * inv);
    ov.y = pack_bf16x2(o[2] * inv, o[3] * inv);
    ov.z = pack_bf16x2(o[4] * inv, o[5] * inv);
    ov.w = pack_bf16x2(o[6] * inv, o[7] * inv);
    st16(a.o + rowq * kSmallD + 8 * c, ov);
    if (a.w && c < a.max_s) {
        float pc = 0.f;
#pragma unroll
        for (int j = 0; j < kSmallMaxS; ++j)
            if (j == c && j < s)
                pc = sc[j] * inv;
        a.w[rowq * a.max_s + c] = f32_to_bf16(pc);
    }
    if (a.lse && c == 0)
        a.lse[rowq] = s > 0 ? (m + __log2f(den)) * kLn2 : kNegInf;
}

// Backward from the stored weights w (the change list's grad_V, grad_attn, softmax backward,
// grad_Q / grad_K): per (sequence, head), dv_j = w_j dO, dw_j = dO . v_j, ds_j = w_j (dw_j - sum_j' w_j' dw_j'),
// dq = scale sum_j ds_j k_j, dk_j = scale ds_j q.  Same layout as the forward: one workgroup per
// sequence and 16 heads, lane (h, c) owns dims [8c, 8c+8) of head h; dw_j is reduced over the 16 lanes
// of a head; every input row is read once and every output row written once (HBM-bound).
__global__ __launch_bounds__(256) void smallseq_bwd_kernel(SmallBwdArgs a)
{
    const int b = blockIdx.x;
    const int h = blockIdx.y * 16 + (threadIdx.x >> 4);
    const int c = threadIdx.x & 15;
    if (h >= a.H)
        return; // whole 16-lane head groups exit together
    const int kv0 = a.cu[b];
    const int s = min(a.cu[b + 1] - kv0, kSmallMaxS);
    const size_t rowq = (size_t)b * a.H + h;
    const size_t stride = (size_t)a.H * kSmallD; // elements between consecutive key rows

    float qf[8], gf[8];
    {
        const uint4 qv = ld16(a.q + rowq * kSmallD + 8 * c), gv = ld16(a.dout + rowq * kSmallD + 8 * c);
        const uint32_t qw[4] = {qv.x, qv.y, qv.z, qv.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qf[2 * e] = bf16_lo(qw[e]);
            qf[2 * e + 1] = bf16_hi(qw[e]);
            gf[2 * e] = bf16_lo(gw[e]);
            gf[2 * e + 1] = bf16_hi(gw[e]);
        }
    }
    // lane c holds weight c of its head; the others come by shuffles within the 16-lane group
    const float wc = c < s ? __uint_as_float((uint32_t)a.w[rowq * a.max_s + c] << 16) : 0.f;
    const int base = threadIdx.x & 48;
    const uint16_t *kp = a.k + ((size_t)kv0 * a.H + h) * kSmallD + 8 * c;
    const uint16_t *vp = a.v + ((size_t)kv0 * a.H + h) * kSmallD + 8 * c;
    uint4 kr[kSmallMaxS], vr[kSmallMaxS];
#pragma unroll
    for (int j = 0; j < kSmallMaxS; ++j)
        if (j < s)
            vr[j] = ld16(vp + j * stride);
#pragma unroll
    for (int j = 0; j < kSmallMaxS; ++j)
        if (j < s)
            kr[j] = ld16(kp + j * stride);

    float wj[kSmallMaxS], dw[kSmallMaxS];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < kSmallMaxS; ++j) {
        wj[j] = __shfl(wc, base + j);
        dw[j] = 0.f;
        if (j < s) {
            dw[j] = sum16(dot8_bf16(vr[j], gf));
            sum = fmaf(wj[j], dw[j], sum);
        }
    }
    float dq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    uint16_t *dkp = a.dk + ((size_t)kv0 * a.H + h) * kSmallD + 8 * c;
    uint16_t *dvp = a.dv + ((size_t)kv0 * a.H + h) * kSmallD + 8 * c;
#pragma unroll
    for (int j = 0; j < kSmallMaxS; ++j) {
        if (j < s) {
            const float ds = wj[j] * (dw[j] - sum) * a.scale;
            const uint32_t kw[4] = {kr[j].x, kr[j].y, kr[j].z, kr[j].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dq[2 * e] = fmaf(ds, bf16_lo(kw[e]), dq[2 * e]);
                dq[2 * e + 1] = fmaf(ds, bf16_hi(kw[e]), dq[2 * e + 1]);
            }
            uint4 ok, ov;
            ok.x = pack_bf16x2(ds * qf[0], ds * qf[1]);
            ok.y = pack_bf16x2(ds * qf[2], ds * qf[3]);
            ok.z = pack_bf16x2(ds * qf[4], ds * qf[5]);
            ok.w = pack_bf16x2(ds * qf[6], ds * qf[7]);
            ov.x = pack_bf16x2(wj[j] * gf[0], wj[j] * gf[1]);
            ov.y = pack_bf16x2(wj[j] * gf[2], wj[j] * gf[3]);
            ov.z = pack_bf16x2(wj[j] * gf[4], wj[j] * gf[5]);
            ov.w = pack_bf16x2(wj[j] * gf[6], wj[j] * gf[7]);
            st16(dkp + j * stride, ok);
            st16(dvp + j * stride, ov);
        }
    }
    uint4 oq;
    oq.x = pack_bf16x2(dq[0], dq[1]);
    oq.y = pack_bf16x2(dq[2], dq[3]);
    oq.z = pack_bf16x2(dq[4], dq[5]);
    oq.w = pack_bf16x2(dq[6], dq[7]);
    st16(a.dq + rowq * kSmallD + 8 * c, oq);
}

hipError_t launch_smallseq_bwd(const SmallBwdArgs &a, hipStream_t stream)
{
    ATTN_LAUNCH(smallseq_bwd_kernel, dim3(a.B, (a.H + 15) / 16), dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_smallseq(const SmallArgs &a, hipStream_t stream)
{
    ATTN_LAUNCH(smallseq_kernel, dim3(a.B, (a.H + 15) / 16), dim3(256), 0, stream, a);
    return hipGetLastError();
}

} // namespace attn
