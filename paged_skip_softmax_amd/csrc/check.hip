// Device-side validation of the index arrays the entry points take as preconditions (ATTN_CHECK=1):
// cu_seqlens monotone from 0 and within the host's max_seqlen bounds, seq_lens within the block table,
// block-table entries of every visible page inside the page pool.  It runs before the attention kernels
// of the call, on the call's stream, then synchronizes; a call whose arrays fail is rejected with
// ATTN_ERR_INVALID and launches nothing else.  ("Model-Optimizer: Add split-k decode kernel for skip
// softmax", What does this PR do: the host validates its arguments before launching; the device contents
// are checked here only on request because the check costs a synchronization.)
//
// The verdict of a check goes to a small file-scope device array (one per GPU, no allocation): the
// kernels store an error code there with plain vector stores; any nonzero value rejects the call.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "launch.h"

namespace attn {
namespace {

// [0]: error code (0 = none), [1]: the batch row it was found in (any one of them when several fail)
static __device__ int check_result[2];

__global__ void check_clear_kernel(int *res)
{
    if (threadIdx.x < 2)
        res[threadIdx.x] = 0;
}

__device__ __forceinline__ void report(int *res, int code, int b)
{
    res[0] = code;
    res[1] = b;
}

// cu[0] == 0, 0 <= cu[b + 1] - cu[b] <= max_len, and cu[B] == total when total >= 0.
__global__ void check_cu_kernel(const int32_t *cu, int B, int max_len, int total, int code_base, int *res)
{
    for (int b = blockIdx.x * blockDim.x + threadIdx.x; b < B; b += gridDim.x * blockDim.x) {
        const int lo = cu[b], hi = cu[b + 1];
        if (b == 0 && lo != 0)
            report(res, code_base + 0, b);
        if (hi < lo)
            report(res, code_base + 1, b);
        else if (hi - lo > max_len)
            report(res, code_base + 2, b);
        if (b == B - 1 && total >= 0 && hi != total)
            report(res, code_base + 3, b);
    }
}

// 0 <= seq_lens[b] <= max_pages * page and every page of the first ceil(seq_lens[b] / page) entries of
// row b in [0, num_pages).  One wave per batch row.
__global__ void check_pages_kernel(const int32_t *bt, const int32_t *seq_lens, int B, int max_pages, int page,
                                   int num_pages, int *res)
{
    const int lane = threadIdx.x & 63;
    for (int b = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6); b < B; b += gridDim.x * (blockDim.x / 64)) {
        const int L = seq_lens[b];
        if (L < 0 || (int64_t)L > (int64_t)max_pages * page) {
            if (lane == 0)
                report(res, kCheckSeqLen, b);
            continue;
        }
        const int np = (L + page - 1) / page;
        const int32_t *row = bt + (size_t)b * max_pages;
        for (int j = lane; j < np; j += 64) {
            const int p = row[j];
            if (p < 0 || p >= num_pages)
                report(res, kCheckPage, b);
        }
    }
}

// The verdict of the checks queued on `stream`, after waiting for them.
hipError_t verdict(hipStream_t stream, int *res_dev, CheckResult *out)
{
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess)
        return e;
    int res[2] = {0, 0};
    e = hipMemcpy(res, res_dev, sizeof res, hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return e;
    out->code = res[0];
    out->row = res[1];
    return hipSuccess;
}

hipError_t result_ptr(int **p)
{
    // looked up on every call: the check is a debugging aid that synchronizes anyway
    return hipGetSymbolAddress(reinterpret_cast<void **>(p), HIP_SYMBOL(check_result));
}

unsigned grid_for(int n, int per_block) { return (unsigned)std::max(1, std::min(1024, (n + per_block - 1) / per_block)); }

} // namespace

hipError_t check_indices(const CheckSpec &s, hipStream_t stream, CheckResult *out)
{
    int *res = nullptr;
    hipError_t e = result_ptr(&res);
    if (e != hipSuccess)
        return e;
    ATTN_LAUNCH(check_clear_kernel, dim3(1), dim3(64), 0, stream, res);
    if (s.cu_a)
        ATTN_LAUNCH(check_cu_kernel, dim3(grid_for(s.B, 256)), dim3(256), 0, stream, s.cu_a, s.B, s.max_a,
                           s.total_a, kCheckCuA, res);
    if (s.cu_b)
        ATTN_LAUNCH(check_cu_kernel, dim3(grid_for(s.B, 256)), dim3(256), 0, stream, s.cu_b, s.B, s.max_b,
                           -1, kCheckCuB, res);
    if (s.bt)
        ATTN_LAUNCH(check_pages_kernel, dim3(grid_for(s.B, 4)), dim3(256), 0, stream, s.bt, s.seq_lens, s.B,
                           s.max_pages, s.page, s.num_pages, res);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    return verdict(stream, res, out);
}

} // namespace attn
