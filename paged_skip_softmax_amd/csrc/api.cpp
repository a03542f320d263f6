// C ABI of libattn.so (declared in include/attn.h): host-side validation, schedule choice and launch.
// Every check runs before the first HIP runtime call, so a rejected call never touches the device.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "launch.h"

namespace {

thread_local std::string g_last_error;

// A diagnostics switch: set, non-empty and not "0".
bool env_on(const char *name)
{
    const char *v = std::getenv(name);
    return v && v[0] && std::strcmp(v, "0") != 0;
}

attn_status_t fail(attn_status_t s, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    if (attn::log_enabled())
        std::fprintf(stderr, "[attn] rejected (status %d): %s\n", (int)s, buf);
    return s;
}

attn_status_t ok()
{
    g_last_error.clear();
    return ATTN_OK;
}

attn_status_t hip_status(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

const char *check_what(int code)
{
    switch (code) {
    case attn::kCheckCuA + 0: return "cu_seqlens (queries / kv) does not start at 0";
    case attn::kCheckCuA + 1: return "cu_seqlens (queries / kv) decreases";
    case attn::kCheckCuA + 2: return "a sequence is longer than max_seqlen (queries / kv)";
    case attn::kCheckCuA + 3: return "cu_seqlens_q[B] differs from total_q";
    case attn::kCheckCuB + 0: return "cu_seqlens_k does not start at 0";
    case attn::kCheckCuB + 1: return "cu_seqlens_k decreases";
    case attn::kCheckCuB + 2: return "a sequence has more keys than max_seqlen_k";
    case attn::kCheckSeqLen: return "seq_lens outside [0, max_pages_per_seq * page_size]";
    case attn::kCheckPage: return "a block-table entry of a visible page is outside [0, num_pages)";
    }
    return "unknown check failure";
}

// ATTN_CHECK=1: the call's index arrays are validated on the device (on the call's stream, which is
// then synchronized) before anything else is launched; a failure rejects the call.
attn_status_t device_check(const char *fn, const attn::CheckSpec &spec, void *stream)
{
    if (!env_on("ATTN_CHECK"))
        return ATTN_OK;
    attn::CheckResult r{};
    const hipError_t e = attn::check_indices(spec, static_cast<hipStream_t>(stream), &r);
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, "%s: ATTN_CHECK: %s", fn, hipGetErrorString(e));
    if (r.code != 0)
        return fail(ATTN_ERR_INVALID, "%s: ATTN_CHECK: %s (batch row %d)", fn, check_what(r.code), r.row);
    return ATTN_OK;
}

attn::CheckSpec cu_spec(int B, const int32_t *cu_a, int max_a, int total_a, const int32_t *cu_b, int max_b)
{
    attn::CheckSpec c{};
    c.B = B;
    c.cu_a = cu_a;
    c.max_a = max_a;
    c.total_a = total_a;
    c.cu_b = cu_b;
    c.max_b = max_b;
    return c;
}

attn::CheckSpec page_spec(attn::CheckSpec c, const int32_t *bt, const int32_t *seq_lens, int max_pages, int page,
                          int num_pages)
{
    c.bt = bt;
    c.seq_lens = seq_lens;
    c.max_pages = max_pages;
    c.page = page;
    c.num_pages = num_pages;
    return c;
}

bool bad_threshold(float thr) { return !(thr >= 0.f && thr <= 1.f); } // also rejects NaN

// The kernels mask keys with -inf before scaling and take a tile's maximum of the raw scores, so the
// logit scale must be positive (0 turns -inf * 0 into NaN, a negative scale turns the maximum into the
// minimum) and scale * log2(e) must stay finite.
bool bad_scale(float scale) { return !(scale > 0.f && std::isfinite(scale * 1.4426950408889634f)); }

// log2(threshold): the kernels compare in the log2 domain, tile_max - running_max < log2(thr) (both in
// log2 units); thr = 0 gives -inf, which never skips.
float log2_threshold(float thr) { return thr > 0.f ? std::log2(thr) : -INFINITY; }

constexpr int kDefaultSplits = 32;
constexpr int kMaxSplits = 64;
constexpr int64_t kMaxGridYZ = 65535; // largest y or z grid dimension a launch here may use
// NVFP4 amax range: keeps 448 / amax, amax / 2688 and every block scale and its reciprocal normal fp32
constexpr float kMinQdqAmax = 1e-20f;
constexpr float kMaxQdqAmax = 1e20f;

int resolve_splits(int num_splits, float thr) { return num_splits != 0 ? num_splits : (thr == 0.f ? kDefaultSplits : 1); }

} // namespace

namespace attn {

bool log_enabled() { return env_on("ATTN_LOG"); }

void log_launch(const char *kernel, dim3 grid, dim3 block)
{
    std::fprintf(stderr, "[attn] launch %s grid (%u, %u, %u) block (%u, %u, %u)\n", kernel, grid.x, grid.y, grid.z,
                 block.x, block.y, block.z);
}

} // namespace attn

extern "C" {

const char *attn_status_string(attn_status_t s)
{
    switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP runtime error";
    default: break;
    }
    return "unknown status";
}

const char *attn_last_error_message(void) { return g_last_error.c_str(); }

size_t attn_decode_paged_workspace_size(int32_t B, int32_t Hq, int32_t D, int32_t num_splits)
{
    const int S = num_splits == 0 ? kDefaultSplits : num_splits;
    if (B <= 0 || Hq <= 0 || D <= 0 || S <= 1)
        return 0;
    return (size_t)B * Hq * S * ((size_t)D + 1) * sizeof(float);
}

} // extern "C"

namespace {

// Scratch memory of attn_decode_paged_noalloc: file-scope device memory, one copy per GPU the library
// runs on, held until the process ends.  In host code `scratch` is only a host-side handle: every use
// goes through the device address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];

// Device address of the current device's copy of `scratch`, looked up once per device.
attn_status_t current_scratch(void **ptr)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return fail(ATTN_ERR_HIP, "attn_decode_paged_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxScratchDevices)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_noalloc: device %d beyond %d", dev, kMaxScratchDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(ATTN_ERR_HIP, "attn_decode_paged_noalloc: hipGetSymbolAddress(scratch): %s",
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return ATTN_OK;
}

// attn_decode_paged with its split-K partials in `workspace`; when use_scratch is set the workspace
// arguments are ignored and the current device's scratch (kScratchBytes) takes their place.
attn_status_t decode_paged(const char *fn, const void *q, const void *k_cache, const void *v_cache,
                           const int32_t *block_table, const int32_t *seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t page_size, int32_t num_pages, int32_t max_pages_per_seq, float scale,
                           float skip_threshold, int32_t num_splits, bool use_scratch, void *workspace,
                           size_t workspace_bytes, void *o, float *lse, uint8_t *skip_map, int32_t skip_map_stride,
                           void *stream)
{
    if (B < 0)
        return fail(ATTN_ERR_INVALID, "%s: B = %d < 0", fn, B);
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv)
        return fail(ATTN_ERR_INVALID, "%s: Hq = %d must be a positive multiple of Hkv = %d", fn, Hq, Hkv);
    if (bad_threshold(skip_threshold))
        return fail(ATTN_ERR_INVALID, "%s: skip_threshold %g outside [0, 1]", fn, (double)skip_threshold);
    if (num_splits < 0 || num_splits > kMaxSplits)
        return fail(ATTN_ERR_INVALID, "%s: num_splits %d outside [0, %d]", fn, num_splits, kMaxSplits);
    const int S = resolve_splits(num_splits, skip_threshold);
    if (skip_threshold > 0.f && S > 1)
        return fail(ATTN_ERR_INVALID, "%s: skip_threshold > 0 needs one sequential split, got %d", fn, S);
    if (bad_scale(scale))
        return fail(ATTN_ERR_INVALID, "%s: scale must be positive and finite", fn);
    if (num_pages <= 0 || max_pages_per_seq <= 0 || page_size <= 0)
        return fail(ATTN_ERR_INVALID, "%s: num_pages, max_pages_per_seq and page_size must be > 0", fn);
    if (skip_map && S > 1)
        return fail(ATTN_ERR_INVALID, "%s: skip_map needs the sequential schedule (num_splits = 1)", fn);
    if (skip_map && (int64_t)skip_map_stride * attn::kSkipTile < (int64_t)max_pages_per_seq * page_size)
        return fail(ATTN_ERR_INVALID, "%s: skip_map_stride %d < ceil(max_pages_per_seq * page_size / 32)", fn,
                    skip_map_stride);
    if (D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: D = %d (built for 128)", fn, D);
    if (page_size != 16)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: page_size = %d (built for 16)", fn, page_size);
    if (Hq / Hkv > 16)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: Hq / Hkv = %d > 16", fn, Hq / Hkv);
    if (B > kMaxGridYZ)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: B = %d above %d (a grid dimension)", fn, B, (int)kMaxGridYZ);
    if (B == 0)
        return ok();
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
        return fail(ATTN_ERR_INVALID, "%s: a required pointer is NULL", fn);
    const float scale_log2 = scale * 1.4426950408889634f;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (S > 1 && use_scratch && attn_decode_paged_workspace_size(B, Hq, D, S) > kScratchBytes)
        return fail(ATTN_ERR_WORKSPACE, "%s: the split-K partials need %zu bytes, above the %zu-byte scratch "
                                        "(B * Hq * num_splits * (D + 1) * 4 must stay within it)", fn,
                    attn_decode_paged_workspace_size(B, Hq, D, S), kScratchBytes);
    if (S > 1 && !use_scratch && (!workspace || workspace_bytes < attn_decode_paged_workspace_size(B, Hq, D, S)))
        return fail(ATTN_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes,
                    attn_decode_paged_workspace_size(B, Hq, D, S));
    {
        const attn_status_t c = device_check(
            fn, page_spec(cu_spec(B, nullptr, 0, -1, nullptr, 0), block_table, seq_lens, max_pages_per_seq, page_size,
                          num_pages), stream);
        if (c != ATTN_OK)
            return c;
    }
    if (S > 1) {
        const size_t need = attn_decode_paged_workspace_size(B, Hq, D, S);
        if (use_scratch) { // its size was checked above, before any HIP call
            const attn_status_t sc = current_scratch(&workspace);
            if (sc != ATTN_OK)
                return sc;
            workspace_bytes = kScratchBytes;
        }
        if (!workspace || workspace_bytes < need)
            return fail(ATTN_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, workspace_bytes, need);
        attn::SplitArgs a{};
        a.q = static_cast<const uint16_t *>(q);
        a.kc = static_cast<const uint16_t *>(k_cache);
        a.vc = static_cast<const uint16_t *>(v_cache);
        a.bt = block_table;
        a.seq_lens = seq_lens;
        a.Hq = Hq;
        a.Hkv = Hkv;
        a.G = Hq / Hkv;
        a.max_pages = max_pages_per_seq;
        a.num_splits = S;
        a.scale_log2 = scale_log2;
        a.ws_o = static_cast<float *>(workspace);
        a.ws_lse = a.ws_o + (size_t)B * Hq * S * D;
        return hip_status(attn::launch_decode_split(a, B, static_cast<uint16_t *>(o), lse, st), "decode split-K launch");
    }
    attn::SeqArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.kc = static_cast<const uint16_t *>(k_cache);
    a.vc = static_cast<const uint16_t *>(v_cache);
    a.bt = block_table;
    a.seq_lens = seq_lens;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.max_pages = max_pages_per_seq;
    a.scale_log2 = scale_log2;
    a.log2_thr = log2_threshold(skip_threshold);
    a.o = static_cast<uint16_t *>(o);
    a.lse = lse;
    a.skip_map = skip_map;
    a.map_stride = skip_map_stride;
    return hip_status(attn::launch_decode_seq(a, B, st), "decode sequential launch");
}

} // namespace

extern "C" {

attn_status_t attn_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *block_table, const int32_t *seq_lens, int32_t B, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                int32_t max_pages_per_seq, float scale, float skip_threshold,
                                int32_t num_splits, void *workspace, size_t workspace_bytes, void *o,
                                float *lse, uint8_t *skip_map, int32_t skip_map_stride, void *stream)
{
    return decode_paged("attn_decode_paged", q, k_cache, v_cache, block_table, seq_lens, B, Hq, Hkv, D, page_size,
                        num_pages, max_pages_per_seq, scale, skip_threshold, num_splits, false, workspace,
                        workspace_bytes, o, lse, skip_map, skip_map_stride, stream);
}

attn_status_t attn_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *block_table, const int32_t *seq_lens, int32_t B, int32_t Hq,
                                        int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                        int32_t max_pages_per_seq, float scale, float skip_threshold,
                                        int32_t num_splits, void *o, float *lse, uint8_t *skip_map,
                                        int32_t skip_map_stride, void *stream)
{
    return decode_paged("attn_decode_paged_noalloc", q, k_cache, v_cache, block_table, seq_lens, B, Hq, Hkv, D,
                        page_size, num_pages, max_pages_per_seq, scale, skip_threshold, num_splits, true, nullptr, 0,
                        o, lse, skip_map, skip_map_stride, stream);
}

attn_status_t attn_decode_paged_qdq(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_table, const int32_t *seq_lens, int32_t B, int32_t Hq,
                                    int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                    int32_t max_pages_per_seq, float scale, float skip_threshold, float p_amax,
                                    float v_amax, void *o, float *lse, uint8_t *skip_map, int32_t skip_map_stride,
                                    void *stream)
{
    if (B < 0)
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_qdq: B = %d < 0", B);
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv)
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_qdq: Hq = %d must be a positive multiple of Hkv = %d", Hq,
                    Hkv);
    if (bad_threshold(skip_threshold))
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_qdq: skip_threshold %g outside [0, 1]",
                    (double)skip_threshold);
    if (bad_scale(scale))
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_qdq: scale must be positive and finite");
    for (float amax : {p_amax, v_amax})
        if (!(amax == 0.f || (amax >= kMinQdqAmax && amax <= kMaxQdqAmax)))
            return fail(ATTN_ERR_INVALID, "attn_decode_paged_qdq: amax %g is neither 0 (off) nor in [%g, %g]",
                        (double)amax, (double)kMinQdqAmax, (double)kMaxQdqAmax);
    if (num_pages <= 0 || max_pages_per_seq <= 0 || page_size <= 0)
        return fail(ATTN_ERR_INVALID,
                    "attn_decode_paged_qdq: num_pages, max_pages_per_seq and page_size must be > 0");
    if (skip_map && (int64_t)skip_map_stride * attn::kSkipTile < (int64_t)max_pages_per_seq * page_size)
        return fail(ATTN_ERR_INVALID,
                    "attn_decode_paged_qdq: skip_map_stride %d < ceil(max_pages_per_seq * page_size / 32)",
                    skip_map_stride);
    if (D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_qdq: D = %d (built for 128)", D);
    if (page_size != 16)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_qdq: page_size = %d (built for 16)", page_size);
    if (Hq / Hkv > 16)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_qdq: Hq / Hkv = %d > 16", Hq / Hkv);
    if (B > kMaxGridYZ)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_qdq: B = %d above %d (a grid dimension)", B,
                    (int)kMaxGridYZ);
    if (B == 0)
        return ok();
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_qdq: a required pointer is NULL");
    {
        const attn_status_t c = device_check(
            "attn_decode_paged_qdq",
            page_spec(cu_spec(B, nullptr, 0, -1, nullptr, 0), block_table, seq_lens, max_pages_per_seq, page_size,
                      num_pages), stream);
        if (c != ATTN_OK)
            return c;
    }
    attn::SeqArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.kc = static_cast<const uint16_t *>(k_cache);
    a.vc = static_cast<const uint16_t *>(v_cache);
    a.bt = block_table;
    a.seq_lens = seq_lens;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.max_pages = max_pages_per_seq;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.log2_thr = log2_threshold(skip_threshold);
    a.o = static_cast<uint16_t *>(o);
    a.lse = lse;
    a.skip_map = skip_map;
    a.map_stride = skip_map_stride;
    a.p_qdq = p_amax > 0.f;
    a.v_qdq = v_amax > 0.f;
    if (a.p_qdq) {
        a.p_enc = 448.f / p_amax;
        a.p_dec = p_amax / 2688.f;
    }
    if (a.v_qdq) {
        a.v_enc = 448.f / v_amax;
        a.v_dec = v_amax / 2688.f;
    }
    return hip_status(attn::launch_decode_seq(a, B, static_cast<hipStream_t>(stream)), "decode QDQ launch");
}

size_t attn_prefill_varlen_backward_workspace_size(int32_t B, int32_t max_seqlen_q, int32_t Hq)
{
    if (B <= 0 || max_seqlen_q <= 0 || Hq <= 0)
        return 0;
    // rowsum(dO * O) and lse * log2(e) per (token, query head); B * max_seqlen_q bounds the token count
    return 2 * (size_t)B * max_seqlen_q * Hq * sizeof(float);
}

attn_status_t attn_prefill_varlen_backward(attn_dtype_t dtype, const void *q, const void *k, const void *v,
                                           const void *o, const void *dout, const float *lse,
                                           const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t B,
                                           int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv,
                                           int32_t D, float scale, int32_t causal, void *dq, void *dk, void *dv,
                                           void *workspace, size_t workspace_bytes, void *stream)
{
    if (dtype != ATTN_F32 && dtype != ATTN_BF16)
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen_backward: unknown dtype %d", (int)dtype);
    if (B < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen_backward: negative B or max_seqlen");
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv)
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen_backward: Hq = %d must be a positive multiple of Hkv = %d",
                    Hq, Hkv);
    if (bad_scale(scale))
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen_backward: scale must be positive and finite");
    if (dtype != ATTN_BF16 || D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_varlen_backward: built for bf16 with D = 128");
    if ((int64_t)B * max_seqlen_q * Hq >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_varlen_backward: B * max_seqlen_q * Hq must stay below 2^31");
    // the kernels address one sequence's rows of all heads with 32-bit byte offsets
    if ((int64_t)max_seqlen_q * Hq * D * 2 >= ((int64_t)1 << 31) || (int64_t)max_seqlen_k * Hkv * D * 2 >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_varlen_backward: max_seqlen * heads * D * 2 must stay below 2^31");
    if (B == 0)
        return ok();
    if (!q || !k || !v || !o || !dout || !lse || !cu_seqlens_q || !cu_seqlens_k || !dq || !dk || !dv)
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen_backward: a required pointer is NULL");
    const size_t need = attn_prefill_varlen_backward_workspace_size(B, max_seqlen_q, Hq);
    if (need && (!workspace || workspace_bytes < need))
        return fail(ATTN_ERR_WORKSPACE, "attn_prefill_varlen_backward: workspace %zu bytes, need %zu", workspace_bytes,
                    need);
    {
        const attn_status_t c = device_check(
            "attn_prefill_varlen_backward", cu_spec(B, cu_seqlens_q, max_seqlen_q, -1, cu_seqlens_k, max_seqlen_k),
            stream);
        if (c != ATTN_OK)
            return c;
    }
    attn::BwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.dsum = static_cast<float *>(workspace);
    a.lse2 = a.dsum + (size_t)B * max_seqlen_q * Hq;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.B = B;
    a.max_q = max_seqlen_q;
    a.max_k = max_seqlen_k;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.causal = causal != 0;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    return hip_status(attn::launch_prefill_bwd(a, static_cast<hipStream_t>(stream)),
                      "prefill backward launch");
}

// Query rows per KV head up to which the multi-token call runs the split-K decode kernel (rows packed
// into 16-column MFMA blocks, each block reading the cache once); beyond it, the paged prefill kernel.
constexpr int kMultiSplitRows = 64;

size_t attn_decode_paged_multi_workspace_size(int32_t total_q, int32_t max_seqlen_q, int32_t Hq, int32_t Hkv,
                                              int32_t D, int32_t num_splits)
{
    if (total_q <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || D <= 0 || max_seqlen_q <= 0)
        return 0;
    if ((int64_t)max_seqlen_q * (Hq / Hkv) > kMultiSplitRows)
        return 0; // the paged prefill kernel needs no workspace
    const int S = num_splits == 0 ? kDefaultSplits : num_splits;
    return (size_t)total_q * Hq * S * (D + 1) * sizeof(float);
}

attn_status_t attn_decode_paged_multi(const void *q, const int32_t *cu_seqlens_q, int32_t total_q,
                                      int32_t max_seqlen_q, const void *k_cache, const void *v_cache,
                                      const int32_t *block_table, const int32_t *seq_lens, int32_t B, int32_t Hq,
                                      int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                      int32_t max_pages_per_seq, float scale, float skip_threshold,
                                      int32_t num_splits, void *workspace, size_t workspace_bytes, void *o,
                                      float *lse, uint8_t *skip_map, int32_t skip_map_stride, void *stream)
{
    if (B < 0 || total_q < 0 || max_seqlen_q < 0)
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_multi: negative B, total_q or max_seqlen_q");
    if (bad_threshold(skip_threshold))
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_multi: skip_threshold %g outside [0, 1]",
                    (double)skip_threshold);
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv)
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_multi: Hq = %d must be a positive multiple of Hkv = %d", Hq,
                    Hkv);
    if (num_splits < 0 || num_splits > kMaxSplits)
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_multi: num_splits %d outside [0, %d]", num_splits,
                    kMaxSplits);
    if (bad_scale(scale))
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_multi: scale must be positive and finite");
    if (num_pages <= 0 || max_pages_per_seq <= 0 || page_size <= 0)
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_multi: num_pages, max_pages_per_seq and page_size must be > 0");
    if (D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_multi: D = %d (built for 128)", D);
    if (page_size != 16)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_multi: page_size = %d (built for 16)", page_size);
    if ((int64_t)B * max_seqlen_q * Hq >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_multi: B * max_seqlen_q * Hq must stay below 2^31");
    if (skip_map && (int64_t)skip_map_stride * attn::kSkipTile < (int64_t)max_pages_per_seq * page_size)
        return fail(ATTN_ERR_INVALID,
                    "attn_decode_paged_multi: skip_map_stride %d < ceil(max_pages_per_seq * page_size / 32)",
                    skip_map_stride);
    if (skip_map && (uint64_t)total_q * (uint64_t)Hq * (uint64_t)skip_map_stride >= ((uint64_t)1 << 32))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_multi: a skip map of total_q * Hq * stride bytes must "
                                          "stay below 2^32");
    if (B == 0 || total_q == 0)
        return ok();
    if (!q || !cu_seqlens_q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
        return fail(ATTN_ERR_INVALID, "attn_decode_paged_multi: a required pointer is NULL");
    const int G = Hq / Hkv;
    const bool skip = skip_threshold > 0.f || skip_map;
    if (!skip && (int64_t)max_seqlen_q * G <= kMultiSplitRows) {
        // the split-K schedule: its grid limit and workspace are checked before the device check
        const int S0 = num_splits == 0 ? kDefaultSplits : num_splits;
        const int ncb0 = std::max(1, (max_seqlen_q * G + 15) / 16);
        if ((int64_t)B * ncb0 > kMaxGridYZ)
            return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_multi: B * ceil(max_seqlen_q * Hq / Hkv / 16) = %lld "
                                              "above %d (a grid dimension)", (long long)B * ncb0, (int)kMaxGridYZ);
        const size_t need0 = attn_decode_paged_multi_workspace_size(total_q, max_seqlen_q, Hq, Hkv, D, S0);
        if (!workspace || workspace_bytes < need0)
            return fail(ATTN_ERR_WORKSPACE, "attn_decode_paged_multi: workspace %zu bytes, need %zu", workspace_bytes,
                        need0);
    }
    {
        const attn_status_t c = device_check(
            "attn_decode_paged_multi",
            page_spec(cu_spec(B, cu_seqlens_q, max_seqlen_q, total_q, nullptr, 0), block_table, seq_lens,
                      max_pages_per_seq, page_size, num_pages), stream);
        if (c != ATTN_OK)
            return c;
    }
    if (skip || (int64_t)max_seqlen_q * G > kMultiSplitRows) {
        // long query chunks, or skip-softmax: the prefill kernel with K / V tiles gathered page by page
        attn::PrefillArgs a{};
        a.q = q;
        a.k = k_cache;
        a.v = v_cache;
        a.cu_q = cu_seqlens_q;
        a.cu_k = nullptr;
        a.B = B;
        a.max_q = max_seqlen_q;
        a.max_k = max_pages_per_seq * page_size;
        a.Hq = Hq;
        a.Hkv = Hkv;
        a.G = G;
        a.causal = true;
        a.scale_log2 = scale * 1.4426950408889634f;
        a.log2_thr = log2_threshold(skip_threshold);
        a.o = o;
        a.lse = lse;
        a.skip_map = skip_map;
        a.map_stride = skip_map ? skip_map_stride : 0;
        a.bt = block_table;
        a.seq_lens = seq_lens;
        a.max_pages = max_pages_per_seq;
        return hip_status(attn::launch_prefill_d128(a, static_cast<hipStream_t>(stream)), "paged prefill launch");
    }
    const int S = num_splits == 0 ? kDefaultSplits : num_splits;
    const int ncb = std::max(1, (max_seqlen_q * G + 15) / 16);
    if ((int64_t)B * ncb > kMaxGridYZ)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_paged_multi: B * ceil(max_seqlen_q * Hq / Hkv / 16) = %lld above %d "
                                          "(a grid dimension)", (long long)B * ncb, (int)kMaxGridYZ);
    const size_t need = attn_decode_paged_multi_workspace_size(total_q, max_seqlen_q, Hq, Hkv, D, S);
    if (!workspace || workspace_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "attn_decode_paged_multi: workspace %zu bytes, need %zu", workspace_bytes,
                    need);
    attn::MultiArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.cu_q = cu_seqlens_q;
    a.kc = static_cast<const uint16_t *>(k_cache);
    a.vc = static_cast<const uint16_t *>(v_cache);
    a.bt = block_table;
    a.seq_lens = seq_lens;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = G;
    a.max_pages = max_pages_per_seq;
    a.num_splits = S;
    a.ncb = ncb;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.ws_o = static_cast<float *>(workspace);
    a.ws_lse = a.ws_o + (size_t)total_q * Hq * S * D;
    return hip_status(attn::launch_decode_multi(a, B, total_q, static_cast<uint16_t *>(o), lse,
                                                static_cast<hipStream_t>(stream)),
                      "multi-token decode launch");
}

attn_status_t attn_smallseq_cross(const void *q, const void *k, const void *v, const int32_t *cu_seqlens_kv,
                                  int32_t B, int32_t H, int32_t D, int32_t max_seqlen_kv, float scale,
                                  void *o, void *attn_weights, float *lse, void *stream)
{
    if (B < 0)
        return fail(ATTN_ERR_INVALID, "attn_smallseq_cross: B = %d < 0", B);
    if (H <= 0)
        return fail(ATTN_ERR_INVALID, "attn_smallseq_cross: H = %d", H);
    if (max_seqlen_kv < 0 || max_seqlen_kv > 16)
        return fail(ATTN_ERR_INVALID, "attn_smallseq_cross: max_seqlen_kv = %d outside [0, 16]", max_seqlen_kv);
    if (bad_scale(scale))
        return fail(ATTN_ERR_INVALID, "attn_smallseq_cross: scale must be positive and finite");
    if (D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_smallseq_cross: D = %d (built for 128)", D);
    if (B == 0)
        return ok();
    if (!q || !k || !v || !cu_seqlens_kv || !o)
        return fail(ATTN_ERR_INVALID, "attn_smallseq_cross: a required pointer is NULL");
    {
        const attn_status_t c =
            device_check("attn_smallseq_cross", cu_spec(B, cu_seqlens_kv, max_seqlen_kv, -1, nullptr, 0), stream);
        if (c != ATTN_OK)
            return c;
    }
    attn::SmallArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.cu = cu_seqlens_kv;
    a.B = B;
    a.H = H;
    a.max_s = max_seqlen_kv;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.o = static_cast<uint16_t *>(o);
    a.w = static_cast<uint16_t *>(attn_weights);
    a.lse = lse;
    return hip_status(attn::launch_smallseq(a, static_cast<hipStream_t>(stream)), "small-seq launch");
}

attn_status_t attn_smallseq_cross_backward(const void *q, const void *k, const void *v, const void *attn_weights,
                                           const void *dout, const int32_t *cu_seqlens_kv, int32_t B, int32_t H,
                                           int32_t D, int32_t max_seqlen_kv, float scale, void *dq, void *dk,
                                           void *dv, void *stream)
{
    if (B < 0)
        return fail(ATTN_ERR_INVALID, "attn_smallseq_cross_backward: B = %d < 0", B);
    if (H <= 0)
        return fail(ATTN_ERR_INVALID, "attn_smallseq_cross_backward: H = %d", H);
    if (max_seqlen_kv < 0 || max_seqlen_kv > 16)
        return fail(ATTN_ERR_INVALID, "attn_smallseq_cross_backward: max_seqlen_kv = %d outside [0, 16]",
                    max_seqlen_kv);
    if (bad_scale(scale))
        return fail(ATTN_ERR_INVALID, "attn_smallseq_cross_backward: scale must be positive and finite");
    if (D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_smallseq_cross_backward: D = %d (built for 128)", D);
    if (B == 0)
        return ok();
    if (!q || !k || !v || !dout || !cu_seqlens_kv || !dq || !dk || !dv || (max_seqlen_kv > 0 && !attn_weights))
        return fail(ATTN_ERR_INVALID, "attn_smallseq_cross_backward: a required pointer is NULL");
    {
        const attn_status_t c = device_check("attn_smallseq_cross_backward",
                                             cu_spec(B, cu_seqlens_kv, max_seqlen_kv, -1, nullptr, 0), stream);
        if (c != ATTN_OK)
            return c;
    }
    attn::SmallBwdArgs a{};
    a.q = static_cast<const uint16_t *>(q);
    a.k = static_cast<const uint16_t *>(k);
    a.v = static_cast<const uint16_t *>(v);
    a.w = static_cast<const uint16_t *>(attn_weights);
    a.dout = static_cast<const uint16_t *>(dout);
    a.cu = cu_seqlens_kv;
    a.B = B;
    a.H = H;
    a.max_s = max_seqlen_kv;
    a.scale = scale;
    a.dq = static_cast<uint16_t *>(dq);
    a.dk = static_cast<uint16_t *>(dk);
    a.dv = static_cast<uint16_t *>(dv);
    return hip_status(attn::launch_smallseq_bwd(a, static_cast<hipStream_t>(stream)), "small-seq backward launch");
}

attn_status_t attn_prefill_varlen(attn_dtype_t dtype, const void *q, const void *k, const void *v,
                                  const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t B,
                                  int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv,
                                  int32_t D, float scale, int32_t causal, float skip_threshold, void *o,
                                  float *lse, uint8_t *skip_map, int32_t skip_map_stride, void *stream)
{
    if (dtype != ATTN_F32 && dtype != ATTN_BF16)
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen: unknown dtype %d", (int)dtype);
    if (B < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen: negative B or max_seqlen");
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv)
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen: Hq = %d must be a positive multiple of Hkv = %d", Hq, Hkv);
    if (bad_threshold(skip_threshold))
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen: skip_threshold %g outside [0, 1]", (double)skip_threshold);
    if (bad_scale(scale))
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen: scale must be positive and finite");
    if (skip_map && (int64_t)skip_map_stride * attn::kSkipTile < (int64_t)max_seqlen_k)
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen: skip_map_stride %d < ceil(max_seqlen_k / 32)", skip_map_stride);
    if (dtype == ATTN_BF16 && D != 64 && D != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_varlen: bf16 D = %d (built for 64 and 128)", D);
    if (dtype == ATTN_F32 && D != 64)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_varlen: fp32 D = %d (built for 64)", D);
    if (dtype == ATTN_BF16 && (int64_t)max_seqlen_k * Hkv * D * 2 >= ((int64_t)1 << 31))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_varlen: max_seqlen_k * Hkv * D * 2 must stay below 2^31 bytes");
    if (dtype == ATTN_BF16 && D == 128 && skip_map &&
        (uint64_t)B * (uint64_t)max_seqlen_q * (uint64_t)Hq * (uint64_t)skip_map_stride >= ((uint64_t)1 << 32))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_varlen: a skip map of B * max_seqlen_q * Hq * stride bytes must "
                                          "stay below 2^32");
    if (D == 64 && (B > kMaxGridYZ || ((int64_t)max_seqlen_q + 63) / 64 > kMaxGridYZ))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_prefill_varlen: D = 64 needs B <= %d and max_seqlen_q <= %lld (grid "
                                          "dimensions)", (int)kMaxGridYZ, (long long)kMaxGridYZ * 64);
    if (B == 0 || max_seqlen_q == 0)
        return ok();
    if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k || !o)
        return fail(ATTN_ERR_INVALID, "attn_prefill_varlen: a required pointer is NULL");
    {
        const attn_status_t c = device_check(
            "attn_prefill_varlen", cu_spec(B, cu_seqlens_q, max_seqlen_q, -1, cu_seqlens_k, max_seqlen_k), stream);
        if (c != ATTN_OK)
            return c;
    }
    attn::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.cu_q = cu_seqlens_q;
    a.cu_k = cu_seqlens_k;
    a.B = B;
    a.max_q = max_seqlen_q;
    a.max_k = max_seqlen_k;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.G = Hq / Hkv;
    a.causal = causal != 0;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.log2_thr = log2_threshold(skip_threshold);
    a.o = o;
    a.lse = lse;
    a.skip_map = skip_map;
    a.map_stride = skip_map_stride;
    return hip_status(attn::launch_prefill(a, dtype == ATTN_BF16, D, static_cast<hipStream_t>(stream)),
                      "prefill launch");
}

} // extern "C"
