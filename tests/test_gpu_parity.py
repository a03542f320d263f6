"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle, element by element.

Tolerances: max-abs error 1e-5 for fp32 outputs and 2e-2 for bf16 outputs (unit-variance V).  Skip-softmax
decisions come from fp32 scores on the GPU and fp64 scores in the oracle, so near a threshold several
skip sets are correct: the test requires >= 99.9 % agreement of the GPU skip map with the oracle's own
decisions over visited (row, tile) pairs, an exact match of which tiles are visited at all, and compares
the outputs against the oracle replaying the GPU's skip map.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_skip_softmax_amd as attn
from paged_skip_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu

F32_TOL = 1e-5
BF16_TOL = 2e-2
DEV = "cuda"


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check_map(gpu_map, ora_map, min_agree=0.999):
    g = gpu_map.cpu().numpy() if isinstance(gpu_map, torch.Tensor) else gpu_map
    o = ora_map
    assert g.shape == o.shape
    # the visited set is pure indexing: exact
    assert np.array_equal(g == 2, o == 2), "visited tiles differ"
    vis = o != 2
    agree = (g[vis] == o[vis]).mean() if vis.any() else 1.0
    assert agree >= min_agree, f"skip-map agreement {agree:.5f}"
    return g, agree


# ------------------------------------------------------------------ prefill

@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("thr", [0.0, 0.1])
def test_tiny_dense_fp32(causal, thr):
    x = W.tiny_dense(seed=1000, device=DEV)
    o, lse, smap = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, scale=x.scale,
                                            causal=causal, skip_threshold=thr, return_lse=True,
                                            return_skip_map=True)
    torch.cuda.synchronize()
    mode = "skip"
    oo, ol, om = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), x.Hq, x.Hkv, x.scale,
                                causal, mode=mode, thr=thr, tile=32, stride=smap.shape[-1])
    g, _ = _check_map(smap, om)
    if thr == 0:
        assert set(np.unique(g)) <= {0, 2}
        od, ld, _ = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), x.Hq, x.Hkv,
                                   x.scale, causal)
        assert np.max(np.abs(_np(o) - od)) <= F32_TOL
    else:
        assert (g == 1).any(), "threshold 0.1 skipped nothing"
    # compare against the oracle replaying the GPU's decisions
    orp, lrp, _ = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), x.Hq, x.Hkv, x.scale,
                                 causal, mode="skip", tile=32, replay=np.where(g == 2, 0, g).reshape(-1, g.shape[-1]),
                                 stride=g.shape[-1])
    assert np.max(np.abs(_np(o) - orp)) <= F32_TOL
    assert np.max(np.abs(_np(lse) - lrp)) <= F32_TOL


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("thr", [0.0, 0.1])
def test_fp32_varlen_ragged_cross(causal, thr):
    # fp32 over several 64-row blocks and 32-key tiles: ragged lengths, an empty sequence, and queries
    # fewer than keys (bottom-right causal) or more (rows that see no key)
    lk = [1, 17, 128, 0, 129, 300, 64, 255, 40]
    lq = [1, 5, 128, 0, 70, 300, 1, 200, 100]
    kv = W.tiny_dense(seed=1010, device=DEV, lengths=lk)
    qq = W.tiny_dense(seed=1011, device=DEV, lengths=lq)
    o, lse, smap = attn.attn_prefill_varlen(qq.q, kv.k, kv.v, qq.cu_q, kv.cu_k, qq.max_q, kv.max_k,
                                            scale=kv.scale, causal=causal, skip_threshold=thr, return_lse=True,
                                            return_skip_map=True)
    torch.cuda.synchronize()
    args = (qq.q.cpu(), kv.k.cpu(), kv.v.cpu(), qq.cu_q.cpu(), kv.cu_k.cpu(), kv.Hq, kv.Hkv, kv.scale, causal)
    _, _, om = oracle.prefill(*args, mode="skip", thr=thr, tile=32, stride=smap.shape[-1])
    g, _ = _check_map(smap, om)
    if thr == 0:
        od, ld, _ = oracle.prefill(*args)
        assert np.max(np.abs(_np(o) - od)) <= F32_TOL
        fin = np.isfinite(ld)
        assert np.array_equal(fin, np.isfinite(_np(lse)))
        assert np.max(np.abs(_np(lse)[fin] - ld[fin])) <= F32_TOL
    orp, lrp, _ = oracle.prefill(*args, mode="skip", tile=32, replay=np.where(g == 2, 0, g).reshape(-1, g.shape[-1]),
                                 stride=g.shape[-1])
    assert np.max(np.abs(_np(o) - orp)) <= F32_TOL
    fin = np.isfinite(lrp)
    assert np.array_equal(fin, np.isfinite(_np(lse)))
    assert np.max(np.abs(_np(lse)[fin] - lrp[fin])) <= F32_TOL


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_bf16_varlen_ragged(D, causal):
    lens = [1, 17, 128, 0, 129, 300, 64, 255]
    x = W.varlen_prefill(seed=31, device=DEV, lengths=lens, Hq=8, Hkv=2, D=D)
    o, lse, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=causal,
                                         return_lse=True)
    torch.cuda.synchronize()
    od, ld, _ = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), 8, 2, x.scale, causal)
    assert np.max(np.abs(_np(o) - od)) <= BF16_TOL
    assert np.max(np.abs(_np(lse) - ld)) <= 1e-3


@pytest.mark.parametrize("B", [256, 300])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_bf16_batch_schedules(B, causal):
    # large batches of short ragged sequences (most units of the grid past their sequence's end), with
    # empty and one-row sequences, against the oracle
    rng = np.random.default_rng(71 + B)
    lens = rng.integers(0, 160, size=B)
    lens[::37] = 0
    lens[5::41] = 1
    x = W.varlen_prefill(seed=37, device=DEV, lengths=lens.tolist(), Hq=8, Hkv=2, D=128)
    o, lse, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=causal,
                                         return_lse=True)
    torch.cuda.synchronize()
    od, ld, _ = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), 8, 2, x.scale, causal)
    assert np.max(np.abs(_np(o) - od)) <= BF16_TOL
    ok = np.isfinite(ld)
    assert np.max(np.abs(_np(lse)[ok] - ld[ok])) <= 1e-3
    assert np.all(np.isneginf(_np(lse)[~ok]))


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2), (32, 2), (12, 3), (6, 2)])
@pytest.mark.parametrize("thr", [0.0, 0.1])
def test_prefill_bf16_gqa_groupings(Hq, Hkv, thr):
    # group sizes 1, 8, 16 and non-powers of two (the workgroup takes the largest power of two dividing
    # the group size as its number of heads)
    lens = [77, 200, 33]
    x = W.varlen_prefill(seed=35, device=DEV, lengths=lens, Hq=Hq, Hkv=Hkv, D=128)
    o, lse, smap = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=True,
                                            skip_threshold=thr, return_lse=True, return_skip_map=thr > 0)
    torch.cuda.synchronize()
    if thr == 0:
        od, ld, _ = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), Hq, Hkv, x.scale,
                                   True)
    else:
        g = smap.cpu().numpy()
        _, _, om = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), Hq, Hkv, x.scale,
                                  True, mode="skip", thr=thr, stride=g.shape[-1])
        _check_map(g, om)
        od, ld, _ = oracle.prefill(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), Hq, Hkv, x.scale,
                                   True, mode="skip", replay=np.where(g == 2, 0, g).reshape(-1, g.shape[-1]),
                                   stride=g.shape[-1])
    assert np.max(np.abs(_np(o) - od)) <= BF16_TOL
    assert np.max(np.abs(_np(lse) - ld)) <= 1e-3


def test_prefill_bf16_cross_lengths_and_empty_keys():
    # Lq != Lk (bottom-right causal alignment) and a sequence with queries but no keys
    Hq, Hkv, D = 4, 4, 128
    lq, lk = [5, 70, 33, 8], [40, 70, 0, 200]
    g = torch.Generator(device=DEV).manual_seed(3)
    q = torch.randn(sum(lq), Hq, D, generator=g, device=DEV).bfloat16()
    k = torch.randn(sum(lk), Hkv, D, generator=g, device=DEV).bfloat16()
    v = torch.randn(sum(lk), Hkv, D, generator=g, device=DEV).bfloat16()
    cq = torch.tensor([0] + list(np.cumsum(lq)), dtype=torch.int32, device=DEV)
    ck = torch.tensor([0] + list(np.cumsum(lk)), dtype=torch.int32, device=DEV)
    for causal in (True, False):
        o, lse, _ = attn.attn_prefill_varlen(q, k, v, cq, ck, max(lq), max(lk), causal=causal, return_lse=True)
        torch.cuda.synchronize()
        od, ld, _ = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), cq.cpu(), ck.cpu(), Hq, Hkv, 1 / math.sqrt(D), causal)
        assert np.max(np.abs(_np(o) - od)) <= BF16_TOL
        fin = np.isfinite(ld)
        assert np.array_equal(fin, np.isfinite(_np(lse)))
        assert np.max(np.abs(_np(lse)[fin] - ld[fin])) <= 1e-3
        assert np.all(_np(o)[75:108] == 0)  # the sequence with no keys


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("thr", [0.0, 0.1])
def test_prefill_bf16_causal_more_queries_than_keys(D, thr):
    # bottom-right causal with Lq > Lk: the first Lq - Lk rows see no key while later rows of the same
    # 32-row block do; those rows must come out as o = 0, lse = -inf (no NaN from an empty running max)
    Hq, Hkv = 4, 2
    lq, lk = [70, 100, 45], [40, 3, 45]
    g = torch.Generator(device=DEV).manual_seed(8)
    q = torch.randn(sum(lq), Hq, D, generator=g, device=DEV).bfloat16()
    k = torch.randn(sum(lk), Hkv, D, generator=g, device=DEV).bfloat16()
    v = torch.randn(sum(lk), Hkv, D, generator=g, device=DEV).bfloat16()
    cq = torch.tensor([0] + list(np.cumsum(lq)), dtype=torch.int32, device=DEV)
    ck = torch.tensor([0] + list(np.cumsum(lk)), dtype=torch.int32, device=DEV)
    o, lse, smap = attn.attn_prefill_varlen(q, k, v, cq, ck, max(lq), max(lk), causal=True, skip_threshold=thr,
                                            return_lse=True, return_skip_map=True)
    torch.cuda.synchronize()
    on, ln = _np(o), _np(lse)
    assert np.isfinite(on).all()
    g_map = smap.cpu().numpy()
    _, _, om = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), cq.cpu(), ck.cpu(), Hq, Hkv, 1 / math.sqrt(D), True,
                              mode="skip", thr=thr, stride=g_map.shape[-1])
    _check_map(g_map, om)
    od, ld, _ = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), cq.cpu(), ck.cpu(), Hq, Hkv, 1 / math.sqrt(D), True,
                               mode="skip", replay=np.where(g_map == 2, 0, g_map).reshape(-1, g_map.shape[-1]),
                               stride=g_map.shape[-1])
    assert np.max(np.abs(on - od)) <= BF16_TOL
    fin = np.isfinite(ld)
    assert not fin.all(), "some rows should see no key"
    assert np.array_equal(fin, np.isfinite(ln))
    assert np.max(np.abs(ln[fin] - ld[fin])) <= 1e-3
    assert np.all(on[~fin] == 0)
    if thr == 0.0:
        # without a skip map the dense path runs (the D = 128 fast kernel for D = 128)
        o2, l2, _ = attn.attn_prefill_varlen(q, k, v, cq, ck, max(lq), max(lk), causal=True, return_lse=True)
        torch.cuda.synchronize()
        o2n, l2n = _np(o2), _np(l2)
        assert np.isfinite(o2n).all()
        assert np.max(np.abs(o2n - od)) <= BF16_TOL
        assert np.array_equal(fin, np.isfinite(l2n))
        assert np.max(np.abs(l2n[fin] - ld[fin])) <= 1e-3
        assert np.all(o2n[~fin] == 0)


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("thr", [0.01, 0.1])
def test_prefill_bf16_noncausal_skip(D, thr):
    # non-causal skip-softmax: every row visits every key tile of its sequence, the last one ragged.
    # Lq != Lk, a sequence with no queries, one with queries but no keys, several query tiles and a
    # ragged query tail; two hot 32-key runs per sequence make the tiles after them skippable.
    Hq, Hkv = 8, 2
    lq, lk = [37, 0, 130, 64, 5, 200], [300, 50, 97, 0, 517, 64]
    gen = torch.Generator(device=DEV).manual_seed(13)
    u = torch.randn(D, generator=gen, device=DEV)
    u = u / u.norm()
    q = (torch.randn(sum(lq), Hq, D, generator=gen, device=DEV) + 3 * u).bfloat16().contiguous()
    k = torch.randn(sum(lk), Hkv, D, generator=gen, device=DEV)
    v = torch.randn(sum(lk), Hkv, D, generator=gen, device=DEV).bfloat16().contiguous()
    ck_l = [0] + list(np.cumsum(lk))
    for b in range(len(lk)):
        for t in (1, 4):
            if 32 * (t + 1) <= lk[b]:
                k[ck_l[b] + 32 * t:ck_l[b] + 32 * (t + 1)] += 25 * u
    k = k.bfloat16().contiguous()
    cq = torch.tensor([0] + list(np.cumsum(lq)), dtype=torch.int32, device=DEV)
    ck = torch.tensor(ck_l, dtype=torch.int32, device=DEV)
    print(f"non-causal skip prefill D {D} thr {thr}", flush=True)
    o, lse, smap = attn.attn_prefill_varlen(q, k, v, cq, ck, max(lq), max(lk), causal=False, skip_threshold=thr,
                                            return_lse=True, return_skip_map=True)
    o2, _, _ = attn.attn_prefill_varlen(q, k, v, cq, ck, max(lq), max(lk), causal=False, skip_threshold=thr)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)  # writing the map does not change the result
    g = smap.cpu().numpy()
    scale = 1 / math.sqrt(D)
    _, _, om = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), cq.cpu(), ck.cpu(), Hq, Hkv, scale, False, mode="skip",
                              thr=thr, stride=g.shape[-1])
    _check_map(g, om)
    assert (g == 1).sum() / (g != 2).sum() > 0.2, "the hot keys should make tiles skippable"
    od, ld, _ = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), cq.cpu(), ck.cpu(), Hq, Hkv, scale, False, mode="skip",
                               replay=np.where(g == 2, 0, g).reshape(-1, g.shape[-1]), stride=g.shape[-1])
    on, ln = _np(o), _np(lse)
    assert np.max(np.abs(on - od)) <= BF16_TOL
    fin = np.isfinite(ld)
    assert np.array_equal(fin, np.isfinite(ln))
    assert np.max(np.abs(ln[fin] - ld[fin])) <= 1e-3
    assert np.all(on[~fin] == 0)
    # rows of the sequence with no keys: nothing visited, o = 0, lse = -inf
    r0 = sum(lq[:3])
    assert np.all(g[r0:r0 + lq[3]] == 2) and np.all(on[r0:r0 + lq[3]] == 0)


def test_prefill_bf16_skip_replay():
    lens = [300, 517, 64]
    x = W.varlen_prefill(seed=41, device=DEV, lengths=lens, Hq=4, Hkv=1, D=128)
    # hot keys: queries share a component along one direction u; two 32-key runs of every sequence get a
    # large component along u, so their logits sit ~4 above the rest and later tiles become skippable
    g = torch.Generator(device=DEV).manual_seed(4)
    u = torch.randn(128, generator=g, device=DEV)
    u = u / u.norm()
    qb = (x.q.float() + 3 * u).bfloat16().contiguous()
    k = x.k.float()
    cu = x.cu_q.tolist()
    for b in range(3):
        for t0 in (cu[b] + 32, cu[b] + 96):
            if t0 + 32 <= cu[b + 1]:
                k[t0:t0 + 32, 0] += 15 * u
    kb = k.bfloat16().contiguous()
    x.q = qb
    for thr in (0.01, 0.1):
        o, lse, smap = attn.attn_prefill_varlen(x.q, kb, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=True,
                                                skip_threshold=thr, return_lse=True, return_skip_map=True)
        torch.cuda.synchronize()
        _, _, om = oracle.prefill(x.q.cpu(), kb.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), 4, 1, x.scale, True,
                                  mode="skip", thr=thr, stride=smap.shape[-1])
        g, _ = _check_map(smap, om)
        if thr == 0.1:
            assert (g == 1).mean() > 0.05, "the hot-key input should make tiles skippable"
        orp, _, _ = oracle.prefill(x.q.cpu(), kb.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), 4, 1, x.scale, True,
                                   mode="skip", replay=np.where(g == 2, 0, g).reshape(-1, g.shape[-1]),
                                   stride=g.shape[-1])
        assert np.max(np.abs(_np(o) - orp)) <= BF16_TOL


# ------------------------------------------------------------------ paged decode

def _small_decode(hot=False, seed=51):
    lengths = [1, 15, 16, 17, 127, 128, 129, 1000, 4097, 33]
    return W.paged_decode(seed=seed, device=DEV, B=len(lengths), Hq=8, Hkv=2, D=128, page=16, pool=1000,
                          lengths=lengths, lmax=4112, hot=hot)


def _decode_oracle(x, **kw):
    return oracle.decode(x.q.cpu(), x.k_cache.cpu(), x.v_cache.cpu(), x.block_table.cpu(), x.seq_lens.cpu(),
                         x.scale, **kw)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2), (32, 2), (12, 4)])
@pytest.mark.parametrize("splits", [1, 32])
def test_decode_gqa_groupings(Hq, Hkv, splits):
    # group sizes 1, 8, 16 (the largest supported) and 3
    lengths = [1, 33, 500, 1000]
    x = W.paged_decode(seed=53, device=DEV, B=len(lengths), Hq=Hq, Hkv=Hkv, D=128, page=16, pool=300,
                       lengths=lengths, lmax=1024)
    o, lse, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=splits,
                                       return_lse=True)
    torch.cuda.synchronize()
    od, ld, _ = _decode_oracle(x)
    assert np.isfinite(_np(o)).all()
    assert np.max(np.abs(_np(o) - od)) <= BF16_TOL
    assert np.max(np.abs(_np(lse) - ld)) <= 1e-3


@pytest.mark.parametrize("splits", [2, 7, 32, 64])
def test_decode_split_k(splits):
    x = _small_decode()
    o, lse, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=splits,
                                       return_lse=True)
    torch.cuda.synchronize()
    od, ld, _ = _decode_oracle(x)
    assert np.isfinite(_np(o)).all(), "NaN poison reached the output"
    assert np.max(np.abs(_np(o) - od)) <= BF16_TOL
    assert np.max(np.abs(_np(lse) - ld)) <= 1e-3


def test_decode_zero_length_and_block_table_permutation():
    x = _small_decode()
    sl = x.seq_lens.clone()
    sl[3] = 0
    o, lse, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, sl, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o[3] == 0) and torch.all(torch.isneginf(lse[3]))
    # permuting the pool and remapping the table gives bit-identical output
    o1, _, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens)
    perm = torch.randperm(x.pool, generator=torch.Generator().manual_seed(5)).to(DEV)
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(x.pool, device=DEV)
    bt2 = x.block_table.clone()
    m = bt2 >= 0
    bt2[m] = inv[bt2[m].long()].to(torch.int32)
    o2, _, _ = attn.attn_decode_paged(x.q, x.k_cache[perm].contiguous(), x.v_cache[perm].contiguous(), bt2,
                                      x.seq_lens)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("B", [100, 200])
@pytest.mark.parametrize("thr", [0.0, 0.1])
def test_decode_sequential_batch_order(B, thr):
    # the sequential decode takes up to 128 batch rows longest first (each workgroup ranks the lengths in
    # LDS) and larger batches in index order: both against the oracle, with empty and one-token rows and
    # ties among the lengths
    rng = np.random.default_rng(81 + B)
    lengths = rng.integers(0, 700, size=B)
    lengths[::23] = 0
    lengths[1::29] = 1
    lengths[2::31] = 256
    x = W.paged_decode(seed=57, device=DEV, B=B, Hq=8, Hkv=2, D=128, page=16, pool=64 * B, lengths=lengths.tolist(),
                       lmax=720, hot=True)
    o, lse, smap = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=1,
                                          skip_threshold=thr, return_lse=True, return_skip_map=True)
    torch.cuda.synchronize()
    _, _, om = _decode_oracle(x, mode="skip", thr=thr, tile=32, stride=smap.shape[-1])
    g, _ = _check_map(smap, om)
    orp, lrp, _ = _decode_oracle(x, mode="skip", tile=32, replay=np.where(g == 2, 0, g).reshape(-1, g.shape[-1]),
                                 stride=g.shape[-1])
    assert np.max(np.abs(_np(o) - orp)) <= BF16_TOL
    ok = np.isfinite(lrp)
    assert np.max(np.abs(_np(lse)[ok] - lrp[ok])) <= 1e-3
    assert np.all(np.isneginf(_np(lse)[~ok]))


@pytest.mark.parametrize("thr", [0.0, 0.01, 0.1, 0.5])
def test_decode_sequential_skip(thr):
    x = _small_decode(hot=True)
    o, lse, smap = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=1,
                                          skip_threshold=thr, return_lse=True, return_skip_map=True)
    torch.cuda.synchronize()
    assert np.isfinite(_np(o)).all()
    _, _, om = _decode_oracle(x, mode="skip", thr=thr, tile=32, stride=smap.shape[-1])
    g, _ = _check_map(smap, om)
    if thr == 0:
        assert set(np.unique(g)) <= {0, 2}
        od, _, _ = _decode_oracle(x)
        assert np.max(np.abs(_np(o) - od)) <= BF16_TOL
    orp, lrp, _ = _decode_oracle(x, mode="skip", tile=32, replay=np.where(g == 2, 0, g).reshape(-1, g.shape[-1]),
                                 stride=g.shape[-1])
    assert np.max(np.abs(_np(o) - orp)) <= BF16_TOL
    assert np.max(np.abs(_np(lse) - lrp)) <= 1e-3


def test_decode_deterministic():
    x = _small_decode()
    a1, _, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens)
    a2, _, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens)
    s1, _, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=1,
                                      skip_threshold=0.1)
    s2, _, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=1,
                                      skip_threshold=0.1)
    torch.cuda.synchronize()
    assert torch.equal(a1, a2) and torch.equal(s1, s2)


# ------------------------------------------------------------------ small-seq

@pytest.mark.parametrize("fixed", [None, 2, 4, 6, 8, 12, 16])
def test_smallseq(fixed):
    x = W.smallseq_cross(seed=61, device=DEV, B=3000, fixed=fixed)
    o, w, lse = attn.attn_smallseq_cross(x.q, x.k, x.v, x.cu_kv, x.max_s, return_lse=True)
    torch.cuda.synchronize()
    rows = [(b, h) for b in range(0, 3000, 7) for h in range(16)]
    oo, ow, ol = oracle.smallseq(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_kv.cpu(), x.max_s, x.scale, rows=rows,
                                 with_lse=True)
    r = np.array(rows)
    assert np.max(np.abs(_np(o)[r[:, 0], r[:, 1]] - oo)) <= BF16_TOL
    assert np.max(np.abs(_np(w)[r[:, 0], r[:, 1], 0] - ow)) <= BF16_TOL
    # the fp32 LSE output: natural log of the row's sum of exp(logits)
    assert np.max(np.abs(_np(lse)[r[:, 0], r[:, 1]] - ol)) <= 1e-3
    # padding weights are exactly zero
    s = x.lens.numpy()
    wn = _np(w)[:, :, 0]
    for b in range(0, 3000, 97):
        assert np.all(wn[b, :, s[b]:] == 0)


def test_smallseq_zero_length():
    x = W.smallseq_cross(seed=62, device=DEV, B=64)
    lens = x.lens.clone()
    lens[5] = 0  # sequence 5 has no keys
    cu = torch.zeros(65, dtype=torch.int32)
    cu[1:] = torch.cumsum(lens, 0)
    T = int(cu[-1])
    o, w, lse = attn.attn_smallseq_cross(x.q, x.k[:T].contiguous(), x.v[:T].contiguous(), cu.to(DEV), 16,
                                         return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o[5] == 0) and torch.all(w[5] == 0) and torch.all(torch.isneginf(lse[5]))
