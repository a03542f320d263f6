"""GPU parity at the full workload sizes, in the launch configuration the benchmark times.

The oracle checks sampled outputs (prefill: a fixed sample of query rows of every sequence, all heads;
decode: a sample of batch rows, all heads) or every output where the fp64 work stays within seconds
(skip decode maps and outputs, small-seq).  Same tolerances as the small parity tests: 2e-2 max-abs
for bf16 outputs, 1e-3 for LSE, >= 99.9 % skip-map agreement with exact visited sets, skip outputs
compared against the oracle replaying the GPU's decisions.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_skip_softmax_amd as attn
from paged_skip_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
LSE_TOL = 1e-3
DEV = "cuda"


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_map(g, o, min_agree=0.999):
    assert g.shape == o.shape
    assert np.array_equal(g == 2, o == 2), "visited tiles differ"
    vis = o != 2
    agree = float((g[vis] == o[vis]).mean())
    assert agree >= min_agree, f"skip-map agreement {agree:.5f}"
    return agree


def test_full_varlen_prefill_sampled_rows():
    x = W.varlen_prefill(seed=1001, device=DEV)           # 16 sequences, L in [256, 4096], Hq 32, Hkv 8, D 128
    o = torch.empty_like(x.q)
    _, lse, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=True, out=o,
                                         return_lse=True)
    torch.cuda.synchronize()
    on, ln = _np(o), _np(lse)
    assert np.isfinite(on).all()
    cu = x.cu_q.cpu().tolist()
    rng = np.random.default_rng(11)
    toks = []
    for b in range(x.B):
        L = cu[b + 1] - cu[b]
        # the first rows, the rows around the 32/64-row tile edges, the last rows and a random sample
        pick = {0, 1, 31, 32, 63, 64, L // 2, L - 2, L - 1}
        pick |= set(rng.choice(L, size=min(L, 40), replace=False).tolist())
        toks += [cu[b] + i for i in sorted(p for p in pick if 0 <= p < L)]
    rows = [(t, h) for t in toks for h in range(x.Hq)]
    od, ld, _ = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), x.Hq, x.Hkv, x.scale,
                               True, rows=rows)
    r = np.array(rows)
    assert np.max(np.abs(on[r[:, 0], r[:, 1]] - od)) <= BF16_TOL
    assert np.max(np.abs(ln[r[:, 0], r[:, 1]] - ld)) <= LSE_TOL


@pytest.fixture(scope="module", params=["hot", "sink"])
def prefill_hot(request):
    # the full prefill shapes plus hot keys; "sink": the coherent attention-sink variant
    if request.param == "sink":
        return W.varlen_prefill_sink(seed=1001, device=DEV)
    return W.varlen_prefill_hot(seed=1001, device=DEV)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("thr", [0.01, 0.1])
def test_full_skip_prefill_sampled_rows(prefill_hot, thr, causal):
    x = prefill_hot
    print(f"full skip prefill thr {thr} causal {causal}", flush=True)
    o, lse, smap = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=causal,
                                            skip_threshold=thr, return_lse=True, return_skip_map=True)
    # the same call without a map (the timed configuration) gives the same output
    o2, _, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=causal,
                                        skip_threshold=thr)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    on, ln, g = _np(o), _np(lse), smap.cpu().numpy()
    assert np.isfinite(on).all()
    cu = x.cu_q.cpu().tolist()
    rng = np.random.default_rng(12)
    toks = []
    for b in range(x.B):
        L = cu[b + 1] - cu[b]
        pick = {0, 31, 32, 63, 64, L // 2, L - 1} | set(rng.choice(L, size=min(L, 24), replace=False).tolist())
        toks += [cu[b] + i for i in sorted(p for p in pick if 0 <= p < L)]
    rows = [(t, h) for t in toks for h in range(x.Hq)]
    r = np.array(rows)
    gm = g[r[:, 0], r[:, 1]]
    qc, kc, vc = x.q.cpu(), x.k.cpu(), x.v.cpu()
    _, _, om = oracle.prefill(qc, kc, vc, x.cu_q.cpu(), x.cu_k.cpu(), x.Hq, x.Hkv, x.scale, causal, mode="skip",
                              thr=thr, rows=rows, stride=g.shape[-1])
    _check_map(gm, om)
    assert (gm == 1).sum() / (gm != 2).sum() > 0.3, "the hot-key prefill input should make tiles skippable"
    od, ld, _ = oracle.prefill(qc, kc, vc, x.cu_q.cpu(), x.cu_k.cpu(), x.Hq, x.Hkv, x.scale, causal, mode="skip",
                               rows=rows, replay=np.where(gm == 2, 0, gm), stride=g.shape[-1])
    assert np.max(np.abs(on[r[:, 0], r[:, 1]] - od)) <= BF16_TOL
    assert np.max(np.abs(ln[r[:, 0], r[:, 1]] - ld)) <= LSE_TOL


@pytest.fixture(scope="module")
def decode_host():
    """The full paged-decode workload (B 64, L in [1024, 32768], 140,000-page pool) and its host copy."""
    x = W.paged_decode(seed=1002, device=DEV)
    host = dict(q=x.q.cpu(), k=x.k_cache.cpu(), v=x.v_cache.cpu(), bt=x.block_table.cpu(), sl=x.seq_lens.cpu())
    return x, host


def test_full_paged_decode_split_k_sampled_rows(decode_host):
    x, h = decode_host
    ws = torch.empty(attn.attn_decode_paged_workspace_size(x.B, x.Hq, x.D, 32), dtype=torch.uint8, device=DEV)
    o, lse, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=32,
                                       workspace=ws, return_lse=True)
    torch.cuda.synchronize()
    on, ln = _np(o), _np(lse)
    assert np.isfinite(on).all(), "NaN poison reached the output"
    L = h["sl"].numpy()
    bs = sorted({int(np.argmax(L)), int(np.argmin(L))} | set(range(0, x.B, 5)))
    rows = [(b, hh) for b in bs for hh in range(x.Hq)]
    od, ld, _ = oracle.decode(h["q"], h["k"], h["v"], h["bt"], h["sl"], x.scale, rows=rows)
    r = np.array(rows)
    assert np.max(np.abs(on[r[:, 0], r[:, 1]] - od)) <= BF16_TOL
    assert np.max(np.abs(ln[r[:, 0], r[:, 1]] - ld)) <= LSE_TOL


@pytest.fixture(scope="module")
def hot_host():
    x = W.paged_decode_hot(seed=1002, device=DEV)
    host = dict(q=x.q.cpu(), k=x.k_cache.cpu(), v=x.v_cache.cpu(), bt=x.block_table.cpu(), sl=x.seq_lens.cpu())
    return x, host


@pytest.mark.parametrize("thr", [0.0, 0.01, 0.1])
def test_full_skip_decode_all_rows(hot_host, thr):
    x, h = hot_host
    o, lse, smap = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=1,
                                          skip_threshold=thr, return_lse=True, return_skip_map=True)
    torch.cuda.synchronize()
    on, ln = _np(o), _np(lse)
    assert np.isfinite(on).all()
    g = smap.cpu().numpy()
    _, _, om = oracle.decode(h["q"], h["k"], h["v"], h["bt"], h["sl"], x.scale, mode="skip", thr=thr, tile=32,
                             stride=g.shape[-1])
    _check_map(g, om)
    if thr == 0.0:
        assert set(np.unique(g)) <= {0, 2}
    if thr == 0.1:
        assert (g == 1).sum() / (g != 2).sum() > 0.5, "the hot-key workload should make most tiles skippable"
    orp, lrp, _ = oracle.decode(h["q"], h["k"], h["v"], h["bt"], h["sl"], x.scale, mode="skip", tile=32,
                                replay=np.where(g == 2, 0, g).reshape(-1, g.shape[-1]), stride=g.shape[-1])
    assert np.max(np.abs(on - orp)) <= BF16_TOL
    assert np.max(np.abs(ln - lrp)) <= LSE_TOL


@pytest.mark.parametrize("thr", [0.0, 0.1])
def test_full_skip_decode_nvfp4_sampled_rows(hot_host, thr):
    # the benchmark's NVFP4 decode call (amax 1 for P and V) on the full hot-key workload; sampled batch
    # rows (the longest, the shortest, every fifth) against the oracle replaying the GPU's skip map
    x, h = hot_host
    o, lse, smap = attn.attn_decode_paged_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                              skip_threshold=thr, p_amax=1.0, v_amax=1.0, return_lse=True,
                                              return_skip_map=True)
    torch.cuda.synchronize()
    on, ln = _np(o), _np(lse)
    assert np.isfinite(on).all()
    g = smap.cpu().numpy()
    L = h["sl"].numpy()
    bs = sorted({int(np.argmax(L)), int(np.argmin(L))} | set(range(0, x.B, 5)))
    rows = [(b, hh) for b in bs for hh in range(x.Hq)]
    r = np.array(rows)
    gm = g[r[:, 0], r[:, 1]]
    _, _, om = oracle.decode_qdq(h["q"], h["k"], h["v"], h["bt"], h["sl"], x.scale, thr=thr, p_amax=1.0, v_amax=1.0,
                                 rows=rows)
    _check_map(gm, om[:, :gm.shape[-1]])
    od, ld, _ = oracle.decode_qdq(h["q"], h["k"], h["v"], h["bt"], h["sl"], x.scale, p_amax=1.0, v_amax=1.0,
                                  rows=rows, replay=np.where(gm == 1, 1, 0))
    assert np.max(np.abs(on[r[:, 0], r[:, 1]] - od)) <= BF16_TOL
    assert np.max(np.abs(ln[r[:, 0], r[:, 1]] - ld)) <= LSE_TOL


def test_decode_largest_batch():
    # B = 65535, the largest grid dimension the decode launches use (split-K in z, sequential in y):
    # sampled rows at both ends of the batch against the oracle, for split-K, the sequential skip decode
    # and the NVFP4 decode
    B = 65535
    lens = torch.randint(1, 49, (B,), generator=torch.Generator().manual_seed(120)).tolist()
    pool = sum((L + 15) // 16 for L in lens) + 5
    x = W.paged_decode(seed=121, device=DEV, B=B, Hq=4, Hkv=1, D=128, lengths=lens, lmax=48, pool=pool)
    rows = [(b, h) for b in list(range(40)) + list(range(B - 40, B)) for h in range(4)]
    r = np.array(rows)
    h = dict(q=x.q.cpu(), k=x.k_cache.cpu(), v=x.v_cache.cpu(), bt=x.block_table.cpu(), sl=x.seq_lens.cpu())
    print("largest batch: split-K", flush=True)
    o, _, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=32)
    torch.cuda.synchronize()
    od, _, _ = oracle.decode(h["q"], h["k"], h["v"], h["bt"], h["sl"], x.scale, rows=rows)
    assert np.max(np.abs(_np(o)[r[:, 0], r[:, 1]] - od)) <= BF16_TOL
    print("largest batch: sequential skip", flush=True)
    o, _, smap = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=1,
                                        skip_threshold=0.1, return_skip_map=True)
    torch.cuda.synchronize()
    g = smap.cpu().numpy()[r[:, 0], r[:, 1]]
    orp, _, _ = oracle.decode(h["q"], h["k"], h["v"], h["bt"], h["sl"], x.scale, mode="skip", tile=32, rows=rows,
                              replay=np.where(g == 2, 0, g), stride=g.shape[-1])
    assert np.max(np.abs(_np(o)[r[:, 0], r[:, 1]] - orp)) <= BF16_TOL
    print("largest batch: NVFP4", flush=True)
    o, _, smap = attn.attn_decode_paged_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                            skip_threshold=0.1, p_amax=1.0, v_amax=1.0, return_skip_map=True)
    torch.cuda.synchronize()
    g = smap.cpu().numpy()[r[:, 0], r[:, 1]]
    oq, _, _ = oracle.decode_qdq(h["q"], h["k"], h["v"], h["bt"], h["sl"], x.scale, p_amax=1.0, v_amax=1.0,
                                 rows=rows, replay=np.where(g == 1, 1, 0))
    assert np.max(np.abs(_np(o)[r[:, 0], r[:, 1]] - oq)) <= BF16_TOL


def test_full_smallseq_all_rows():
    x = W.smallseq_cross(seed=1004, device=DEV)              # B 30720, s_kv in {2..16}, H 16, D 128
    o, w, lse = attn.attn_smallseq_cross(x.q, x.k, x.v, x.cu_kv, x.max_s, return_lse=True)
    torch.cuda.synchronize()
    od, wd, ld = oracle.smallseq(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_kv.cpu(), x.max_s, x.scale, with_lse=True)
    assert np.max(np.abs(_np(o) - od)) <= BF16_TOL
    assert np.max(np.abs(_np(w) - wd)) <= BF16_TOL
    assert np.max(np.abs(_np(lse) - ld)) <= 1e-3


def test_empty_batch_is_a_no_op():
    # B = 0 for every entry point: nothing is launched, nothing fails
    z32 = torch.zeros(1, dtype=torch.int32, device=DEV)
    e = torch.empty((0, 4, 128), dtype=torch.bfloat16, device=DEV)
    o, _, _ = attn.attn_prefill_varlen(e, torch.empty((0, 1, 128), dtype=torch.bfloat16, device=DEV),
                                       torch.empty((0, 1, 128), dtype=torch.bfloat16, device=DEV), z32, z32, 0, 0)
    assert o.shape == (0, 4, 128)
    kc = torch.zeros((1, 1, 16, 128), dtype=torch.bfloat16, device=DEV)
    o, _, _ = attn.attn_decode_paged(e, kc, kc, torch.zeros((0, 1), dtype=torch.int32, device=DEV),
                                     torch.zeros(0, dtype=torch.int32, device=DEV))
    assert o.shape == (0, 4, 128)
    o, w, _ = attn.attn_smallseq_cross(e, torch.empty((0, 4, 128), dtype=torch.bfloat16, device=DEV),
                                       torch.empty((0, 4, 128), dtype=torch.bfloat16, device=DEV), z32, 16)
    torch.cuda.synchronize()
    assert o.shape == (0, 4, 128) and w.shape == (0, 4, 1, 16)


def test_prefill_one_long_sequence_sampled():
    # one causal sequence of 131,072 tokens (Hq 8, Hkv 1): 2,048 key tiles per row at the end, 4,096
    # query tiles (the offsets at the 2^31-byte limit are the next test's); sampled rows, all heads
    L = 131072
    x = W.varlen_prefill(seed=1011, device=DEV, lengths=[L], Hq=8, Hkv=1)
    o, lse, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=True,
                                         return_lse=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(13)
    toks = sorted({0, 1, 31, 32, 63, 64, 4095, 4096, L // 2, L - 65, L - 64, L - 2, L - 1}
                  | set(rng.choice(L, size=24, replace=False).tolist()))
    rows = [(t, h) for t in toks for h in range(x.Hq)]
    od, ld, _ = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), x.Hq, x.Hkv, x.scale,
                               True, rows=rows)
    r = np.array(rows)
    assert np.max(np.abs(_np(o)[r[:, 0], r[:, 1]] - od)) <= BF16_TOL
    assert np.max(np.abs(_np(lse)[r[:, 0], r[:, 1]] - ld)) <= LSE_TOL


def test_prefill_kv_offsets_at_the_limit():
    # one sequence whose K / V rows of a KV head span just under 2^31 bytes, the host's limit for
    # max_seqlen_k * Hkv * D * 2: 1,048,000 keys with Hkv 8 (2.15 GB each for K and V), 64 queries,
    # bottom-right causal and non-causal; the buffer sizes and tile offsets of the direct-to-LDS loads
    # sit near the top of 32 bits.  Sampled rows (the oracle sums a million keys per row).
    Lk, Lq, Hq, Hkv, D = 1_048_000, 64, 8, 8, 128
    assert Lk * Hkv * D * 2 < 2 ** 31 <= (Lk + 1024) * Hkv * D * 2
    g = torch.Generator(device=DEV).manual_seed(21)
    q = torch.randn(Lq, Hq, D, generator=g, device=DEV).bfloat16()
    k = torch.randn(Lk, Hkv, D, generator=g, device=DEV).bfloat16()
    v = torch.randn(Lk, Hkv, D, generator=g, device=DEV).bfloat16()
    cq = torch.tensor([0, Lq], dtype=torch.int32, device=DEV)
    ck = torch.tensor([0, Lk], dtype=torch.int32, device=DEV)
    kc, vc = k.cpu(), v.cpu()
    rows = [(t, h) for t in (0, 31, 32, 63) for h in range(Hq)]
    r = np.array(rows)
    for causal in (True, False):
        o, lse, _ = attn.attn_prefill_varlen(q, k, v, cq, ck, Lq, Lk, causal=causal, return_lse=True)
        torch.cuda.synchronize()
        od, ld, _ = oracle.prefill(q.cpu(), kc, vc, cq.cpu(), ck.cpu(), Hq, Hkv, 1 / math.sqrt(D), causal,
                                   rows=rows)
        assert np.max(np.abs(_np(o)[r[:, 0], r[:, 1]] - od)) <= BF16_TOL
        assert np.max(np.abs(_np(lse)[r[:, 0], r[:, 1]] - ld)) <= LSE_TOL


def test_prefill_many_short_sequences():
    # 4,096 sequences of 1..16 tokens: every query tile is partial, most workgroups see one key tile;
    # every row against the oracle
    g = torch.Generator().manual_seed(14)
    lens = torch.randint(1, 17, (4096,), generator=g).tolist()
    x = W.varlen_prefill(seed=1012, device=DEV, lengths=lens, Hq=32, Hkv=8)
    o, lse, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=True,
                                         return_lse=True)
    torch.cuda.synchronize()
    od, ld, _ = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), x.Hq, x.Hkv, x.scale,
                               True)
    assert np.max(np.abs(_np(o) - od)) <= BF16_TOL
    assert np.max(np.abs(_np(lse) - ld)) <= LSE_TOL


@pytest.mark.parametrize("splits", [64, 1])
def test_decode_one_long_context(splits):
    # one sequence of 262,144 cached tokens (16,384 pages): 2,048 128-key tiles over 64 splits, or the
    # sequential schedule's 8,192 32-key tiles; every head against the oracle
    L = 262144
    x = W.paged_decode(seed=1013, device=DEV, B=1, lengths=[L], lmax=L, pool=L // 16 + 8)
    ws = torch.empty(attn.attn_decode_paged_workspace_size(x.B, x.Hq, x.D, splits), dtype=torch.uint8, device=DEV)
    o, lse, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=splits,
                                       workspace=ws, return_lse=True)
    torch.cuda.synchronize()
    od, ld, _ = oracle.decode(x.q.cpu(), x.k_cache.cpu(), x.v_cache.cpu(), x.block_table.cpu(), x.seq_lens.cpu(),
                              x.scale)
    assert np.isfinite(_np(o)).all()
    assert np.max(np.abs(_np(o) - od)) <= BF16_TOL
    assert np.max(np.abs(_np(lse) - ld)) <= LSE_TOL
