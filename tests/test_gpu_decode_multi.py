"""GPU parity of the multi-token paged decode (bottom-right causal over the paged cache) against the fp64
oracle, through the C ABI.  Same bars as the one-token decode: 2e-2 max-abs on the bf16 outputs (unit
variance V), 1e-3 on the LSE, exact agreement on which rows see no key."""
import numpy as np
import pytest
import torch

import oracle
import paged_skip_softmax_amd as attn
from paged_skip_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16_TOL = 2e-2
LSE_TOL = 1e-3


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _compare(x, o, lse, rows=None):
    od, ld = oracle.decode_multi(x.q.cpu(), x.cu_q.cpu(), x.k_cache.cpu(), x.v_cache.cpu(), x.block_table.cpu(),
                                 x.seq_lens.cpu(), x.scale, rows=rows)
    on, ln = _np(o), _np(lse)
    if rows is not None:
        r = np.array(rows)
        on, ln = on[r[:, 0], r[:, 1]], ln[r[:, 0], r[:, 1]]
    assert np.isfinite(on).all(), "NaN poison reached the output"
    assert np.max(np.abs(on - od)) <= BF16_TOL
    fin = np.isfinite(ld)
    assert np.array_equal(fin, np.isfinite(ln))
    if fin.any():
        assert np.max(np.abs(ln[fin] - ld[fin])) <= LSE_TOL
    assert np.all(on[~fin] == 0)


@pytest.mark.parametrize("splits", [1, 7, 32])
def test_decode_multi_small(splits):
    # 12 sequences of 1..300 cached keys, 1..8 new tokens each (G = 4: up to 2 blocks of 16 rows)
    x = W.paged_decode_multi(seed=61, device=DEV, B=12, Hq=8, Hkv=2, lmin=1, lmax=300, pool=400, qmin=1, qmax=8)
    o, lse, _ = attn.attn_decode_paged_multi(x.q, x.cu_q, x.max_q, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                          num_splits=splits, return_lse=True)
    torch.cuda.synchronize()
    _compare(x, o, lse)


@pytest.mark.parametrize("Hq,Hkv,qmax", [(8, 8, 64), (32, 2, 4), (12, 3, 16)])
def test_decode_multi_groupings(Hq, Hkv, qmax):
    # G = 1 with up to 64 tokens, G = 16 with up to 4, G = 4 with up to 16: every row-block count 1..4
    x = W.paged_decode_multi(seed=62, device=DEV, B=6, Hq=Hq, Hkv=Hkv, lmin=40, lmax=500, pool=300, qmin=1,
                             qmax=qmax)
    o, lse, _ = attn.attn_decode_paged_multi(x.q, x.cu_q, x.max_q, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                          return_lse=True)
    torch.cuda.synchronize()
    _compare(x, o, lse)


def test_decode_multi_tokens_without_keys():
    # more new tokens than cached keys: the leading tokens see no key (o = 0, lse = -inf); a one-key
    # sequence and an empty one
    x = W.paged_decode_multi(seed=63, device=DEV, B=4, Hq=8, Hkv=2, lengths=[5, 1, 0, 40], pool=64, qmin=1, qmax=1)
    lq = torch.tensor([9, 3, 2, 16])
    cu = torch.cat([torch.zeros(1, dtype=torch.int64), lq.cumsum(0)])
    g = torch.Generator(device=DEV).manual_seed(64)
    x.q = torch.randn(int(cu[-1]), x.Hq, x.D, generator=g, device=DEV).bfloat16()
    x.cu_q = cu.to(torch.int32).to(DEV)
    o, lse, _ = attn.attn_decode_paged_multi(x.q, x.cu_q, 16, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                          num_splits=4, return_lse=True)
    torch.cuda.synchronize()
    _compare(x, o, lse)
    assert not np.isfinite(_np(lse)).all()


def test_decode_multi_full_size_sampled():
    # the full paged-decode cache (B 64, L in [1024, 32768], 140,000-page pool) with 1..4 new tokens per
    # sequence, 32 splits (the benchmark's configuration); every token and head of a sample of sequences
    x = W.paged_decode_multi(seed=1002, device=DEV)
    o, lse, _ = attn.attn_decode_paged_multi(x.q, x.cu_q, x.max_q, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                          num_splits=32, return_lse=True)
    torch.cuda.synchronize()
    L = x.lens.numpy()
    cu = x.cu_q.cpu().tolist()
    bs = sorted({int(np.argmax(L)), int(np.argmin(L))} | set(range(0, x.B, 7)))
    rows = [(t, h) for b in bs for t in range(cu[b], cu[b + 1]) for h in range(x.Hq)]
    _compare(x, o, lse, rows=rows)


# ------------------------------------------------------------------ long query chunks: the paged prefill kernel

@pytest.mark.parametrize("Hq,Hkv,qmin,qmax", [(8, 2, 20, 200), (8, 8, 65, 130), (32, 8, 17, 70)])
def test_paged_prefill_chunks(Hq, Hkv, qmin, qmax):
    # Lq * G > 64 rows per KV head: the prefill kernel with page-gathered K / V tiles (ragged chunks and
    # contexts, every tile-edge case: partial pages, partial 64-key tiles, the causal diagonal)
    x = W.paged_decode_multi(seed=65, device=DEV, B=7, Hq=Hq, Hkv=Hkv, lmin=70, lmax=1500, pool=800, qmin=qmin,
                             qmax=qmax)
    assert x.max_q * (Hq // Hkv) > 64
    o, lse, _ = attn.attn_decode_paged_multi(x.q, x.cu_q, x.max_q, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                          return_lse=True)
    torch.cuda.synchronize()
    _compare(x, o, lse)


def test_paged_prefill_whole_sequences_and_tokens_without_keys():
    # Lq = L (the whole sequence is new), Lq > L (leading tokens without a key), and an empty cache
    x = W.paged_decode_multi(seed=66, device=DEV, B=4, Hq=8, Hkv=2, lengths=[100, 33, 0, 64], pool=64, qmin=1,
                             qmax=1)
    lq = torch.tensor([100, 50, 20, 64])
    cu = torch.cat([torch.zeros(1, dtype=torch.int64), lq.cumsum(0)])
    g = torch.Generator(device=DEV).manual_seed(67)
    x.q = torch.randn(int(cu[-1]), x.Hq, x.D, generator=g, device=DEV).bfloat16()
    x.cu_q = cu.to(torch.int32).to(DEV)
    o, lse, _ = attn.attn_decode_paged_multi(x.q, x.cu_q, 100, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                          return_lse=True)
    torch.cuda.synchronize()
    _compare(x, o, lse)


def test_paged_prefill_full_size_sampled():
    # the full paged-decode cache with 256-token chunks (a chunked prefill over contexts of 1k-32k keys);
    # the first, last and a sample of tokens of several sequences, all heads
    x = W.paged_decode_multi(seed=1002, device=DEV, qmin=256, qmax=256)
    o, lse, _ = attn.attn_decode_paged_multi(x.q, x.cu_q, x.max_q, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                          return_lse=True)
    torch.cuda.synchronize()
    L = x.lens.numpy()
    cu = x.cu_q.cpu().tolist()
    rng = np.random.default_rng(68)
    bs = sorted({int(np.argmax(L)), int(np.argmin(L))} | set(range(0, x.B, 16)))
    rows = []
    for b in bs:
        n = cu[b + 1] - cu[b]
        toks = {0, 1, 63, 64, n - 1} | set(rng.choice(n, size=6, replace=False).tolist())
        rows += [(cu[b] + t, h) for t in sorted(toks) for h in range(x.Hq)]
    _compare(x, o, lse, rows=rows)


# ------------------------------------------------------------------ skip-softmax over the paged cache

def _gather_thd(x):
    """Each sequence's cached keys and values gathered through the block table (key j of sequence b is slot
    j % 16 of page block_table[b][j // 16]) and packed THD, with cu_seqlens_k = prefix sums of seq_lens."""
    kc, vc, bt, sl = x.k_cache.cpu(), x.v_cache.cpu(), x.block_table.cpu(), x.seq_lens.cpu()
    ks, vs = [], []
    for b in range(len(sl)):
        j = torch.arange(int(sl[b]))
        pages = bt[b, j // 16].long()
        ks.append(kc[pages, :, j % 16, :])
        vs.append(vc[pages, :, j % 16, :])
    cu_k = torch.zeros(len(sl) + 1, dtype=torch.int32)
    cu_k[1:] = sl.cumsum(0)
    return torch.cat(ks).contiguous(), torch.cat(vs).contiguous(), cu_k


def _check_map(g, o, min_agree=0.999):
    assert g.shape == o.shape
    assert np.array_equal(g == 2, o == 2), "visited tiles differ"
    vis = o != 2
    agree = (g[vis] == o[vis]).mean() if vis.any() else 1.0
    assert agree >= min_agree, f"skip-map agreement {agree:.5f}"


def test_decode_multi_skip_threshold_zero_is_dense():
    # thr 0 with a skip map: the paged prefill kernel's skip instantiation, which must equal dense attention
    # and mark every visited tile kept
    x = W.paged_decode_multi(seed=65, device=DEV, B=8, Hq=8, Hkv=2, lmin=1, lmax=400, pool=300, qmin=1, qmax=24)
    o, lse, smap = attn.attn_decode_paged_multi(x.q, x.cu_q, x.max_q, x.k_cache, x.v_cache, x.block_table,
                                                x.seq_lens, return_lse=True, return_skip_map=True)
    torch.cuda.synchronize()
    _compare(x, o, lse)
    k, v, cu_k = _gather_thd(x)
    _, _, om = oracle.prefill(x.q.cpu(), k, v, x.cu_q.cpu(), cu_k, x.Hq, x.Hkv, x.scale, True, mode="skip",
                              thr=0.0, stride=smap.shape[-1])
    g = smap.cpu().numpy()
    assert set(np.unique(g)) <= {0, 2}
    _check_map(g, om)


@pytest.mark.parametrize("qmax", [4, 100])
@pytest.mark.parametrize("thr", [0.5, 0.9])
def test_decode_multi_skip(qmax, thr):
    # short chunks (which would take split-K when dense) and long ones; random logits skip many tiles at
    # these thresholds.  Decisions agree with the oracle's on >= 99.9 % of visited (row, tile) pairs; the
    # outputs equal the oracle replaying the GPU's own decisions.
    x = W.paged_decode_multi(seed=66, device=DEV, B=6, Hq=8, Hkv=2, lmin=1, lmax=700, pool=400, qmin=1, qmax=qmax)
    o, lse, smap = attn.attn_decode_paged_multi(x.q, x.cu_q, x.max_q, x.k_cache, x.v_cache, x.block_table,
                                                x.seq_lens, skip_threshold=thr, return_lse=True,
                                                return_skip_map=True)
    torch.cuda.synchronize()
    k, v, cu_k = _gather_thd(x)
    stride = smap.shape[-1]
    _, _, om = oracle.prefill(x.q.cpu(), k, v, x.cu_q.cpu(), cu_k, x.Hq, x.Hkv, x.scale, True, mode="skip",
                              thr=thr, stride=stride)
    g = smap.cpu().numpy()
    _check_map(g, om)
    assert (g == 1).mean() > 0.05, "these thresholds should skip tiles"
    orp, lrp, _ = oracle.prefill(x.q.cpu(), k, v, x.cu_q.cpu(), cu_k, x.Hq, x.Hkv, x.scale, True, mode="skip",
                                 replay=np.where(g == 2, 0, g).reshape(-1, stride), stride=stride)
    on, ln = _np(o), _np(lse)
    assert np.isfinite(on).all()
    assert np.max(np.abs(on - orp)) <= BF16_TOL
    fin = np.isfinite(lrp)
    assert np.array_equal(fin, np.isfinite(ln))
    assert np.max(np.abs(ln[fin] - lrp[fin])) <= LSE_TOL
