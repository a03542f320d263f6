// Kernel argument blocks and launchers shared by the C ABI (api.cpp) and the kernel sources.
// Plain structs passed by value as kernel arguments.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

constexpr int kSkipTile = 32; // keys per skip decision

// Split-K paged decode (num_splits > 1): partials into the workspace, then the merge.
struct SplitArgs {
    const uint16_t *q;      // [B, Hq, D] bf16
    const uint16_t *kc;     // [pages, Hkv, 16, D] bf16
    const uint16_t *vc;
    const int32_t *bt;      // [B, max_pages]
    const int32_t *seq_lens;
    int Hq, Hkv, G, max_pages, num_splits;
    float scale_log2;       // scale * log2(e)
    float *ws_o;            // [B, Hq, S, D]
    float *ws_lse;          // [B, Hq, S], natural log
};

// Multi-token paged decode: split-K over the cache for the (token, head) rows of each KV head's group.
struct MultiArgs {
    const uint16_t *q;      // [total_q, Hq, D] bf16
    const int32_t *cu_q;    // [B + 1]
    const uint16_t *kc, *vc;
    const int32_t *bt, *seq_lens;
    int Hq, Hkv, G, max_pages, num_splits, ncb; // ncb: 16-row blocks per (sequence, KV head)
    float scale_log2;
    float *ws_o;            // [total_q, Hq, S, D]
    float *ws_lse;          // [total_q, Hq, S]
};

// Sequential paged decode with skip-softmax over 32-key tiles (num_splits == 1).
struct SeqArgs {
    const uint16_t *q, *kc, *vc;
    const int32_t *bt, *seq_lens;
    int Hq, Hkv, G, max_pages;
    float scale_log2;
    float log2_thr;         // log2(threshold); -inf disables skipping
    uint16_t *o;            // [B, Hq, D] bf16
    float *lse;             // nullable [B, Hq]
    uint8_t *skip_map;      // nullable [B, Hq, map_stride]
    int map_stride;
    // NVFP4 fake quantization of P / V (on when p_qdq / v_qdq): enc = 448 / amax, dec = amax / 2688
    float p_enc, p_dec, v_enc, v_dec;
    int p_qdq, v_qdq;
};

// Small-seq cross-attention (s_q = 1, s_kv <= 16).
struct SmallArgs {
    const uint16_t *q, *k, *v; // [B, H, D], [T, H, D] x2
    const int32_t *cu;         // [B + 1]
    int B, H, max_s;
    float scale_log2;
    uint16_t *o;               // [B, H, D]
    uint16_t *w;               // nullable [B, H, 1, max_s]
    float *lse;                // nullable [B, H]
};

// Small-seq backward from the stored attention weights.
struct SmallBwdArgs {
    const uint16_t *q, *k, *v, *w, *dout; // [B, H, D], [T, H, D] x2, [B, H, 1, max_s], [B, H, D]
    const int32_t *cu;                    // [B + 1]
    int B, H, max_s;
    float scale;
    uint16_t *dq, *dk, *dv;               // [B, H, D], [T, H, D] x2
};

// Varlen prefill.
struct PrefillArgs {
    const void *q, *k, *v;
    const int32_t *cu_q, *cu_k;
    int B, max_q, max_k, Hq, Hkv, G;
    bool causal;
    float scale_log2;
    float log2_thr;
    void *o;
    float *lse;
    uint8_t *skip_map;
    int map_stride;
    // paged K / V (null bt: contiguous THD k, v with cu_k): k, v are [num_pages, Hkv, 16, D] caches,
    // sequence b's key j in page bt[b * max_pages + j / 16], and it has seq_lens[b] keys
    const int32_t *bt, *seq_lens;
    int max_pages;
};

// Backward of the dense bf16 varlen prefill (D = 128).
struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;          // [tq, Hq] natural log, from the forward
    float *dsum;               // [tq, Hq] workspace: rowsum(dO * O)
    float *lse2;               // [tq, Hq] workspace: lse * log2(e)
    const int32_t *cu_q, *cu_k;
    int B, max_q, max_k, Hq, Hkv, G;
    bool causal;
    float scale, scale_log2;
    void *dq, *dk, *dv;        // bf16, like q, k, v
};

// ATTN_CHECK=1: device-side validation of a call's index arrays before its kernels (check.hip).  cu_a
// (nullable): [B + 1] prefix sums, each difference at most max_a, cu_a[B] == total_a when total_a >= 0;
// cu_b likewise with max_b; bt / seq_lens (nullable): a [B, max_pages] block table over num_pages pages
// of `page` keys and the row lengths it covers.
struct CheckSpec {
    int B;
    const int32_t *cu_a;
    int max_a, total_a;
    const int32_t *cu_b;
    int max_b;
    const int32_t *bt, *seq_lens;
    int max_pages, page, num_pages;
};
enum CheckCode {
    kCheckCuA = 1,   // +0 cu_a[0] != 0, +1 decreasing, +2 a length above max_a, +3 cu_a[B] != total_a
    kCheckCuB = 5,   // the same for cu_b
    kCheckSeqLen = 9, // seq_lens[b] outside [0, max_pages * page]
    kCheckPage = 10,  // a visible block-table entry outside [0, num_pages)
};
struct CheckResult {
    int code, row; // code 0: every check passed
};
// Queues the checks on `stream`, waits for them and reports the verdict.
hipError_t check_indices(const CheckSpec &s, hipStream_t stream, CheckResult *out);

// ATTN_LOG=1: every kernel launch (name, grid, block) and every rejected call (its message) is printed
// to stderr.  Both variables are read on every call.
bool log_enabled();
void log_launch(const char *kernel, dim3 grid, dim3 block);

// hipLaunchKernelGGL plus the ATTN_LOG line.
#define ATTN_LAUNCH(kernel, grid, block, lds, stream, ...)                                                        \
    do {                                                                                                          \
        if (::attn::log_enabled())                                                                                \
            ::attn::log_launch(#kernel, dim3(grid), dim3(block));                                                 \
        hipLaunchKernelGGL(kernel, grid, block, lds, stream, __VA_ARGS__);                                        \
    } while (0)

hipError_t launch_decode_split(const SplitArgs &a, int B, uint16_t *o, float *lse, hipStream_t stream);
hipError_t launch_decode_seq(const SeqArgs &a, int B, hipStream_t stream);
hipError_t launch_decode_multi(const MultiArgs &a, int B, int total_q, uint16_t *o, float *lse, hipStream_t stream);
hipError_t launch_smallseq(const SmallArgs &a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &a, bool bf16, int D, hipStream_t stream);
hipError_t launch_prefill_d128(const PrefillArgs &a, hipStream_t stream); // bf16, D = 128
hipError_t launch_prefill_bwd(const BwdArgs &a, hipStream_t stream);
hipError_t launch_smallseq_bwd(const SmallBwdArgs &a, hipStream_t stream);

} // namespace attn
