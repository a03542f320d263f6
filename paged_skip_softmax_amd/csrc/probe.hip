// Measurement only (not part of the attention library's ABI): the bf16 matrix-core rate a plain MFMA loop
// sustains with every CU busy, the achievable peak the contraction-bound kernels are set against next to
// the published one.  Built into libattn_probe.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4; // independent accumulators per wave

// Each wave issues kChains independent 32x32x16 bf16 MFMAs per iteration on operands of ordinary
// magnitude (values in +-[1, 2), so the matrix core does not run on zeros); two waves per SIMD.
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void mfma_loop_kernel(float *out,
                                                                                                 int iters)
{
    const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
    uint16_t av[8], bv[8];
    for (int i = 0; i < 8; ++i) {
        const uint32_t h = (tid * 2654435761u) ^ (0x9e3779b9u * (i + 1));
        av[i] = (uint16_t)(0x3f80u | ((h >> 9) & 0x7fu) | ((h & 1u) << 15));
        bv[i] = (uint16_t)(0x3f80u | ((h >> 17) & 0x7fu) | (((h >> 1) & 1u) << 15));
    }
    const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(av));
    const bf16x8 b = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(bv));
    f32x16 c[kChains];
    for (int k = 0; k < kChains; ++k)
        for (int e = 0; e < 16; ++e)
            c[k][e] = 0.f;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int k = 0; k < kChains; ++k)
            c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
    }
    float s = 0.f;
    for (int k = 0; k < kChains; ++k)
        s += c[k][0] + c[k][15];
    out[tid] = s;
}

} // namespace

// blocks workgroups of 256 lanes, iters iterations each: blocks * 4 * iters * kChains * 32768 FLOP.  out:
// blocks * 256 floats of device memory.  Returns 0, or the HIP error code of the launch.
extern "C" int attn_probe_mfma_bf16(float *out, int blocks, int iters, void *stream)
{
    hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
    return (int)hipGetLastError();
}

extern "C" double attn_probe_mfma_bf16_flop(int blocks, int iters)
{
    return (double)blocks * 4 * iters * kChains * 32768.0;
}
