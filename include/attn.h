/*
 * attn.h -- C ABI of libattn.so, FlashAttention-style tiled attention with online softmax for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations are the ones the source pages describe:
 *   - varlen prefill: "Model-Optimizer: Add Triton unified attention kernel with HuggingFace integration"
 *     (variable-length batching, GQA, causal and non-causal masking), sequences packed THD with
 *     cu_seqlens as in "ROCm TransformerEngine: Integrate CK varlen cross attention", change list;
 *   - one-token paged decode with split-K and skip-softmax: "Model-Optimizer: Add split-k decode kernel
 *     for skip softmax", What does this PR do (one sequential split of 32-token tiles when skip-softmax
 *     is on, 32 splits of 128-token tiles when it is off, threshold validated and passed at run time)
 *     and Usage (query, key_cache, value_cache, block_table, sequence_lengths, threshold);
 *   - skip-softmax itself: "TensorRT-LLM: Skip Softmax Attention", Description -- a whole KV tile is
 *     skipped (no exp, no P.V, no rescale) when exp(tile_max - running_max) < threshold;
 *   - small-seq cross-attention: "ROCm TransformerEngine: Integrate CK varlen cross attention for
 *     small-seq (s_q=1, s_kv<=16)", change list (one query per sequence, 2..16 keys, huge batch,
 *     head_dim 128, BF16, attention weights written as [tokens_q, h_q, 1, max_seqlen_kv]).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer, owned by the caller, to a dense row-major array.  The
 *     library never allocates device memory, never synchronizes the stream, keeps no state besides a
 *     thread-local error message, the allocation-free decode's scratch and the prefill backward's side
 *     stream (below), and is reentrant.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is enqueued on it
 *     and the call returns before the GPU finishes.  The prefill backward forks part of its work onto
 *     a side stream of the device and joins it back before returning (events recorded on `stream` and
 *     on the side stream), so its work is ordered with `stream` like the rest; the side stream (default
 *     priority) and two events are created on the first such call for a device that is not under
 *     stream capture, and kept until the process ends.
 *   - Arguments are validated on the host before any HIP runtime call; a rejected call launches
 *     nothing and returns ATTN_ERR_INVALID / _UNSUPPORTED / _WORKSPACE.  Device-side contents
 *     (monotone cu_seqlens, in-range block_table entries, seq_lens within the table) are
 *     preconditions and are not checked.  ATTN_ERR_HIP reports a failed launch.
 *   - GQA: query head h reads KV head h / (Hq / Hkv).
 *   - Logits are scale * q.k; LSE outputs are the natural-log log-sum-exp of those logits, fp32; a row
 *     that sees no key gets o = 0 and lse = -inf.  scale must be positive with scale * log2(e) finite
 *     (else ATTN_ERR_INVALID): masked keys are -inf before scaling and tile maxima are taken of the
 *     unscaled scores.
 *   - skip_threshold must lie in [0, 1]; 0 reproduces dense attention.  Skip decisions are taken per
 *     (query row, 32-key tile), tiles aligned to key 0 and visited in ascending order; the first
 *     visited tile is never skipped.  Skip maps hold one byte per (row, tile):
 *     0 = processed, 1 = skipped, 2 = not visited (no visible key).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID = 1,     /* bad argument value or a required pointer is NULL            */
    ATTN_ERR_UNSUPPORTED = 2, /* valid request this build has no kernel for (dtype, D, page) */
    ATTN_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the size query returned   */
    ATTN_ERR_HIP = 4,         /* the HIP runtime reported an error while launching           */
    ATTN_STATUS_INT_RANGE = 0x7fffffff /* not a status: makes every int32 a value of the type   */
} attn_status_t;

/* ATTN_DTYPE_INT_RANGE is not a dtype: it makes every int32 a value of the type, so that a code a C
 * caller passes outside {0, 1} is well defined in the library and rejected (ATTN_ERR_INVALID). */
typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1, ATTN_DTYPE_INT_RANGE = 0x7fffffff } attn_dtype_t;

/* Width of the tiles skip decisions are taken on, in keys. */
#define ATTN_SKIP_TILE 32

/*
 * Varlen prefill.
 *   q [tq, Hq, D], k and v [tk, Hkv, D], o [tq, Hq, D], all of `dtype` (fp32 or bf16); tq = cu_seqlens_q[B],
 *   tk = cu_seqlens_k[B].  cu_seqlens_q / cu_seqlens_k: int32 [B + 1], non-decreasing, starting at 0.
 *   max_seqlen_q / max_seqlen_k: host upper bounds of the per-sequence lengths (size the launch grid).
 *   causal != 0: query i of a sequence with Lq queries and Lk keys sees keys j <= i + Lk - Lq.
 *   skip_threshold: see above; accumulation is fp32 and the P.V product is bf16 for bf16 inputs.
 *   lse: nullable fp32 [tq, Hq].  skip_map: nullable uint8 [tq, Hq, skip_map_stride] with
 *   skip_map_stride >= ceil(max_seqlen_k / 32); every entry of a row is written (2 past its visible keys).
 *   Supported: bf16 with D in {64, 128}; fp32 with D = 64.  B == 0 is a no-op.  bf16 needs
 *   max_seqlen_k * Hkv * D * 2 < 2^31 and, for D = 128 with a skip map, B * max_seqlen_q * Hq *
 *   skip_map_stride < 2^32; D = 64 needs B <= 65535 and max_seqlen_q <= 65535 * 64 (grid dimensions)
 *   (else ATTN_ERR_UNSUPPORTED).
 */
attn_status_t attn_prefill_varlen(attn_dtype_t dtype, const void *q, const void *k, const void *v,
                                  const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t B,
                                  int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv,
                                  int32_t D, float scale, int32_t causal, float skip_threshold, void *o,
                                  float *lse, uint8_t *skip_map, int32_t skip_map_stride, void *stream);

/*
 * Bytes of workspace attn_decode_paged needs for the split-K schedule (num_splits > 1):
 * per-split fp32 outputs [B, Hq, num_splits, D] and fp32 LSEs [B, Hq, num_splits].  0 when
 * num_splits <= 1 (the sequential schedule needs none).  num_splits = 0 means the default for a
 * dense call (32).
 */
size_t attn_decode_paged_workspace_size(int32_t B, int32_t Hq, int32_t D, int32_t num_splits);

/*
 * One-token paged decode: the single query token of batch row b attends to all seq_lens[b] cached keys.
 *   q [B, Hq, D] bf16;  o [B, Hq, D] bf16;  lse nullable fp32 [B, Hq].
 *   k_cache, v_cache: bf16 [num_pages, Hkv, page_size, D] -- one (page, kv head) is a contiguous
 *   page_size x D slab.  Key j of row b is slot j % page_size of page block_table[b][j / page_size].
 *   block_table: int32 [B, max_pages_per_seq], row-major; entries past ceil(seq_lens[b] / page_size)
 *   are never read.  seq_lens: int32 [B], each in [0, max_pages_per_seq * page_size].
 *   Cache slots past seq_lens[b] in the last page may hold anything (NaN included); they are masked.
 *   num_splits: 0 = default (32 when skip_threshold == 0, else 1).  num_splits > 1 runs split-K over
 *   128-key tiles: each split takes a contiguous run of ceil(ntiles / num_splits) tiles, writes
 *   (O_s, lse_s) to the workspace and a second kernel merges them by log-sum-exp.  num_splits == 1
 *   runs one sequential split over 32-key tiles with skip-softmax at `skip_threshold`; skip_threshold
 *   > 0 requires num_splits == 1.  num_splits must be in [0, 64].
 *   workspace: device buffer of at least attn_decode_paged_workspace_size() bytes (may be NULL when
 *   that size is 0).  skip_map: nullable uint8 [B, Hq, skip_map_stride], sequential schedule only,
 *   skip_map_stride >= ceil(max_pages_per_seq * page_size / 32).
 *   Supported: D = 128, page_size = 16, Hq / Hkv <= 16, B <= 65535 (a grid dimension; else
 *   ATTN_ERR_UNSUPPORTED).  B == 0 is a no-op.
 */
attn_status_t attn_decode_paged(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *block_table, const int32_t *seq_lens, int32_t B, int32_t Hq,
                                int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                int32_t max_pages_per_seq, float scale, float skip_threshold,
                                int32_t num_splits, void *workspace, size_t workspace_bytes, void *o,
                                float *lse, uint8_t *skip_map, int32_t skip_map_stride, void *stream);

/*
 * attn_decode_paged for callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops and harnesses that forbid allocation.  Same arguments, layouts, schedules,
 * kernels and results as attn_decode_paged, minus the workspace: the split-K partials
 * (B * Hq * num_splits * (D + 1) * 4 bytes) go to a scratch array that the library keeps in device
 * memory, ATTN_NOALLOC_SCRATCH_BYTES per GPU it runs on, held until the process ends.  A call that
 * would need more returns ATTN_ERR_WORKSPACE before any HIP call (e.g. 64 MiB covers B = 64, Hq = 32
 * with the default 32 splits, 33.8 MB).  The sequential schedule (num_splits == 1) uses no scratch.
 * The scratch used is the one of the calling thread's current device, so `stream` must belong to
 * that device.  The call allocates nothing (the first call on a device looks the scratch address up
 * once).  Every call on one GPU shares that GPU's scratch and it keeps the last call's contents:
 * calls that overlap on one GPU (different streams, or different threads) race and must be
 * serialized by the caller; calls on one stream are ordered and safe.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
attn_status_t attn_decode_paged_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                        const int32_t *block_table, const int32_t *seq_lens, int32_t B, int32_t Hq,
                                        int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                        int32_t max_pages_per_seq, float scale, float skip_threshold,
                                        int32_t num_splits, void *o, float *lse, uint8_t *skip_map,
                                        int32_t skip_map_stride, void *stream);

/*
 * One-token paged decode with NVFP4 fake quantization of P and V ("Model-Optimizer: Add split-k decode
 * kernel for skip softmax", What does this PR do: skip-softmax together with NVFP4 P/V quantize-dequantize
 * in the sequential schedule; Usage: p_qdq / v_qdq with p_qdq_amax / v_qdq_amax).  The sequential
 * schedule of attn_decode_paged (num_splits = 1, 32-key tiles, skip_threshold in [0, 1], 0 = dense) with:
 *   - V (v_amax > 0): every key's D values fake-quantized in blocks of 16 consecutive values along D and
 *     rounded back to bf16 before the P.V product;
 *   - P (p_amax > 0): the unnormalized probabilities exp(s - m) of a kept tile, m the sequential pass's
 *     running max including the tile (P in [0, 1]), fake-quantized in blocks of the 16 keys of a page
 *     (keys 16 i .. 16 i + 15 of the sequence) before P.V; the softmax denominator sums the unquantized P.
 * NVFP4 (the pages give no recipe; this is the format read plainly): E2M1 elements {0, 0.5, 1, 1.5, 2, 3,
 * 4, 6}, one E4M3 scale code per block (largest 448), per-tensor factors enc = 448 / amax and
 * dec = amax / 2688, all in fp32: block scale s = e4m3(max |x| * enc) * dec, x^ = sign(x) *
 * e2m1(|x| * (1 / s)) * s (0 when s = 0), each rounding to nearest even, saturating.  Values above amax
 * saturate at about amax.
 *   amax: 0 turns that side off; otherwise in [1e-20, 1e20] (else ATTN_ERR_INVALID).  With both 0 the
 *   result is attn_decode_paged's with num_splits = 1, from the same schedule.
 *   Every other argument, layout, ownership and error as for attn_decode_paged with num_splits = 1 (no
 *   workspace).  Stream-ordered, asynchronous.
 */
attn_status_t attn_decode_paged_qdq(const void *q, const void *k_cache, const void *v_cache,
                                    const int32_t *block_table, const int32_t *seq_lens, int32_t B, int32_t Hq,
                                    int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                    int32_t max_pages_per_seq, float scale, float skip_threshold, float p_amax,
                                    float v_amax, void *o, float *lse, uint8_t *skip_map, int32_t skip_map_stride,
                                    void *stream);

/*
 * Multi-token paged decode (several new tokens per sequence over the paged cache; "Model-Optimizer: Add
 * split-k decode kernel for skip softmax", description: multi-token decode stays on the shared
 * attention kernel, whose summary gives causal masking over variable-length batches).  Sequence b has
 * Lq_b = cu_seqlens_q[b + 1] - cu_seqlens_q[b] new query tokens, the last Lq_b of its seq_lens[b]
 * cached keys (already in the cache); its token i sees keys j < seq_lens[b] - Lq_b + i + 1 (bottom-right
 * causal; none when that is <= 0).  Skip-softmax as in attn_prefill_varlen ("TensorRT-LLM: Skip Softmax
 * Attention", Description): per (token, head) row and 32-key tile, tiles aligned to key 0 of the cache.
 *   q, o [total_q, Hq, D] bf16 THD (total_q = cu_seqlens_q[B]); cu_seqlens_q int32 [B + 1];
 *   max_seqlen_q >= every Lq_b; caches, block_table, seq_lens, page_size as for attn_decode_paged.
 *   skip_threshold in [0, 1] (0 = dense).  num_splits in [0, 64] (0 = 32; the split-K schedule only).
 *   workspace: at least attn_decode_paged_multi_workspace_size(total_q, max_seqlen_q, Hq, Hkv, D,
 *   num_splits) bytes (caller-owned, no initialisation; may be NULL when that is 0; unused when
 *   skip-softmax is on).  lse: nullable fp32 [total_q, Hq] (natural log; -inf for a token that sees no
 *   key, whose output is 0).  skip_map: nullable uint8 [total_q, Hq, skip_map_stride] with
 *   skip_map_stride >= ceil(max_pages_per_seq * page_size / 32); 0 = kept, 1 = skipped, 2 = not visited
 *   (every entry of a row is written).
 *   Schedules: dense with max_seqlen_q * Hq / Hkv <= 64 query rows per KV head, split-K over the cache
 *   with the rows in 16-row blocks (each block reads the cache once) and a merge kernel; otherwise (a
 *   chunked prefill, or skip_threshold > 0, or a skip map) the prefill kernel with its K / V tiles
 *   gathered page by page, no split, no workspace.  Supported: D = 128, page_size = 16,
 *   B * max_seqlen_q * Hq < 2^31, a skip map below 2^32 bytes and, on the split-K schedule,
 *   B * ceil(max_seqlen_q * Hq / Hkv / 16) <= 65535 (a grid dimension) (else ATTN_ERR_UNSUPPORTED).
 *   B == 0 or total_q == 0 is a no-op.
 */
size_t attn_decode_paged_multi_workspace_size(int32_t total_q, int32_t max_seqlen_q, int32_t Hq, int32_t Hkv,
                                              int32_t D, int32_t num_splits);
attn_status_t attn_decode_paged_multi(const void *q, const int32_t *cu_seqlens_q, int32_t total_q,
                                      int32_t max_seqlen_q, const void *k_cache, const void *v_cache,
                                      const int32_t *block_table, const int32_t *seq_lens, int32_t B, int32_t Hq,
                                      int32_t Hkv, int32_t D, int32_t page_size, int32_t num_pages,
                                      int32_t max_pages_per_seq, float scale, float skip_threshold,
                                      int32_t num_splits, void *workspace, size_t workspace_bytes, void *o,
                                      float *lse, uint8_t *skip_map, int32_t skip_map_stride, void *stream);

/*
 * Small-seq cross-attention (s_q = 1): sequence b has one query token and
 * s_b = cu_seqlens_kv[b + 1] - cu_seqlens_kv[b] keys, non-causal, H query heads = H KV heads.
 *   q [B, H, D], k and v [cu_seqlens_kv[B], H, D], o [B, H, D], all bf16.
 *   max_seqlen_kv: host value in [0, 16], >= every s_b; it is the last dimension of the weights.
 *   attn_weights: nullable bf16 [B, H, 1, max_seqlen_kv]; entry j < s_b is softmax probability j,
 *   entries s_b <= j < max_seqlen_kv are 0.  lse: nullable fp32 [B, H].
 *   Supported: D = 128.  B == 0 is a no-op.
 */
attn_status_t attn_smallseq_cross(const void *q, const void *k, const void *v, const int32_t *cu_seqlens_kv,
                                  int32_t B, int32_t H, int32_t D, int32_t max_seqlen_kv, float scale,
                                  void *o, void *attn_weights, float *lse, void *stream);

/*
 * Backward of the small-seq cross-attention from the attention weights its forward stored
 * ("ROCm TransformerEngine: Integrate CK varlen cross attention for small-seq (s_q=1, s_kv<=16)",
 * change list: grad_V, grad_attn, the softmax backward and grad_Q / grad_K; the weights buffer is
 * written by the forward and read by the backward).  Per (sequence b, head h) with s_b keys, stored
 * weights w_j and output gradient dout:
 *   dv_j = w_j dout,  dw_j = dout . v_j,  ds_j = w_j (dw_j - sum_j' w_j' dw_j'),
 *   dq = scale sum_j ds_j k_j,  dk_j = scale ds_j q.
 *   q, dout, dq [B, H, D]; k, v, dk, dv [cu_seqlens_kv[B], H, D]; attn_weights [B, H, 1, max_seqlen_kv]
 *   (as attn_smallseq_cross writes it; entries j >= s_b are not read); all bf16.  dq, dk, dv are fully
 *   written.  max_seqlen_kv in [0, 16], >= every s_b.  Supported: D = 128.  B == 0 is a no-op.
 */
attn_status_t attn_smallseq_cross_backward(const void *q, const void *k, const void *v, const void *attn_weights,
                                           const void *dout, const int32_t *cu_seqlens_kv, int32_t B, int32_t H,
                                           int32_t D, int32_t max_seqlen_kv, float scale, void *dq, void *dk,
                                           void *dv, void *stream);

/*
 * Backward of the dense varlen prefill: the gradients dq, dk, dv of the masked-softmax attention
 * o = softmax(scale q k^T + mask) v for an output gradient dout ("Model-Optimizer: Add Triton unified
 * attention kernel with HuggingFace integration", summary: the Triton kernel has an autograd backward
 * beside its forward).  With P = exp(scale q k^T - lse) over the visible keys:
 *   dv = P^T dout,  dk = scale dS^T q,  dq = scale dS k,  dS = P * (dout v^T - rowsum(dout * o))
 * with dk and dv summed over the query heads of each KV head's group.
 *   q, o, dout, dq [tq, Hq, D]; k, v, dk, dv [tk, Hkv, D]; all bf16; cu_seqlens_q / cu_seqlens_k,
 *   max_seqlen_q / max_seqlen_k, causal and scale as for the forward call that produced o and lse.
 *   lse: fp32 [tq, Hq], the forward's natural-log LSE (-inf for rows with no visible key).
 *   workspace: at least attn_prefill_varlen_backward_workspace_size(B, max_seqlen_q, Hq) bytes
 *   (B * max_seqlen_q * Hq * 8) of device memory owned by the caller; no initialisation needed; it
 *   receives rowsum(dout * o) and lse * log2(e) per (token, query head).  dq, dk, dv are fully written (rows with no
 *   visible key and keys no query sees get 0).
 *   Supported: bf16 with D = 128, B * max_seqlen_q * Hq < 2^31, max_seqlen_q * Hq * D * 2 < 2^31 and
 *   max_seqlen_k * Hkv * D * 2 < 2^31 (else ATTN_ERR_UNSUPPORTED).
 *   B == 0 is a no-op.  Asynchronous on `stream`, like the forward.
 */
size_t attn_prefill_varlen_backward_workspace_size(int32_t B, int32_t max_seqlen_q, int32_t Hq);
attn_status_t attn_prefill_varlen_backward(attn_dtype_t dtype, const void *q, const void *k, const void *v,
                                           const void *o, const void *dout, const float *lse,
                                           const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int32_t B,
                                           int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t Hq, int32_t Hkv,
                                           int32_t D, float scale, int32_t causal, void *dq, void *dk, void *dv,
                                           void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *attn_status_string(attn_status_t s);

/* Detail of the calling thread's last failed call ("" if none). */
const char *attn_last_error_message(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
