"""ATTN_CHECK=1 and ATTN_LOG=1 on the GPU.

With ATTN_CHECK=1 every entry point validates its index arrays on the device before launching its
attention kernels (cu_seqlens monotone from 0 within max_seqlen, cu_seqlens_q[B] == total_q, seq_lens
within the block table, visible block-table entries inside the pool) and rejects a call that fails with
ATTN_ERR_INVALID, having launched nothing else: the outputs keep their sentinel.  The invalid arrays
below are only ever read by the validation kernels, whose reads stay inside the arrays.  Valid inputs give
the same results as without the check.  ATTN_LOG=1 prints one line per kernel launch."""
import pytest
import torch

import paged_skip_softmax_amd as attn
from paged_skip_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rejected(fn, match):
    with pytest.raises(attn.AttnError) as ei:
        fn()
    assert ei.value.status == 1 and match in str(ei.value), str(ei.value)


def test_check_rejects_bad_block_tables_and_lengths(monkeypatch):
    x = W.paged_decode(seed=71, device=DEV, B=4, Hq=8, Hkv=2, lengths=[40, 700, 0, 1500], lmax=2048, pool=300)
    monkeypatch.setenv("ATTN_CHECK", "1")
    ref, _, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=8)
    torch.cuda.synchronize()
    monkeypatch.delenv("ATTN_CHECK")
    plain, _, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=8)
    torch.cuda.synchronize()
    assert torch.equal(ref, plain)
    monkeypatch.setenv("ATTN_CHECK", "1")
    num_pages = x.k_cache.shape[0]
    print("ATTN_CHECK: page index past the pool", flush=True)
    bt = x.block_table.clone()
    bt[1, 3] = num_pages + 3  # a page row 1 reads (it has 44 pages)
    out = torch.full_like(x.q, 7.0)
    for splits in (8, 1):
        _rejected(lambda: attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, bt, x.seq_lens, num_splits=splits,
                                                 out=out), "block-table entry")
    _rejected(lambda: attn.attn_decode_paged_qdq(x.q, x.k_cache, x.v_cache, bt, x.seq_lens, p_amax=1.0, out=out),
              "block-table entry")
    _rejected(lambda: attn.attn_decode_paged_noalloc(x.q, x.k_cache, x.v_cache, bt, x.seq_lens, out=out),
              "block-table entry")
    torch.cuda.synchronize()
    assert torch.all(out == 7.0), "a rejected call wrote its output"
    # a negative entry past the sequence's pages is never read, so it passes
    bt2 = x.block_table.clone()
    bt2[0, 10] = -5
    o2, _, _ = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, bt2, x.seq_lens, num_splits=8)
    torch.cuda.synchronize()
    assert torch.equal(o2, ref)
    print("ATTN_CHECK: sequence longer than its table row", flush=True)
    sl = x.seq_lens.clone()
    sl[3] = x.block_table.shape[1] * 16 + 1
    _rejected(lambda: attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, sl, out=out), "seq_lens")
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_check_rejects_bad_cu_seqlens(monkeypatch):
    monkeypatch.setenv("ATTN_CHECK", "1")
    x = W.varlen_prefill(seed=72, device=DEV, lengths=[50, 130, 7], Hq=8, Hkv=2)
    o_ok, _, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k)
    torch.cuda.synchronize()
    out = torch.full_like(x.q, 3.0)
    print("ATTN_CHECK: decreasing cu_seqlens_q", flush=True)
    bad = torch.tensor([0, 50, 40, 57], dtype=torch.int32, device=DEV)  # lengths 50, -10, 17
    _rejected(lambda: attn.attn_prefill_varlen(x.q, x.k, x.v, bad, x.cu_k, x.max_q, x.max_k, out=out), "decreases")
    print("ATTN_CHECK: a sequence above max_seqlen_k", flush=True)
    _rejected(lambda: attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, 100, out=out),
              "more keys than max_seqlen_k")
    print("ATTN_CHECK: cu_seqlens not starting at 0", flush=True)
    shifted = x.cu_k.clone()
    shifted[0] = 1
    _rejected(lambda: attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, shifted, x.max_q, x.max_k, out=out),
              "does not start at 0")
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)
    o2, _, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k)
    torch.cuda.synchronize()
    assert torch.equal(o_ok, o2)
    # small-seq: the first of 64 sequences has 9 keys, max_seqlen_kv says 8
    g = torch.Generator(device=DEV).manual_seed(73)
    sq = torch.randn(64, 16, 128, generator=g, device=DEV).bfloat16()
    sk = torch.randn(513, 16, 128, generator=g, device=DEV).bfloat16()
    cu = torch.arange(0, 65, dtype=torch.int32, device=DEV) * 8
    cu[1:] += 1
    print("ATTN_CHECK: small-seq length above max_seqlen_kv", flush=True)
    _rejected(lambda: attn.attn_smallseq_cross(sq, sk, sk, cu, 8), "longer than max_seqlen")
    # multi-token decode: cu_seqlens_q[B] must equal total_q
    d = W.paged_decode_multi(seed=74, device=DEV, B=3, lengths=[100, 300, 50], lmax=512, pool=100, qmin=1, qmax=3)
    cq = d.cu_q.clone()
    cq[-1] -= 1
    print("ATTN_CHECK: multi-token cu_seqlens_q[B] != total_q", flush=True)
    _rejected(lambda: attn.attn_decode_paged_multi(d.q, cq, d.max_q, d.k_cache, d.v_cache, d.block_table,
                                                   d.seq_lens), "total_q")


def test_log_prints_launches(monkeypatch, capfd):
    x = W.varlen_prefill(seed=75, device=DEV, lengths=[64, 100], Hq=4, Hkv=1)
    monkeypatch.setenv("ATTN_LOG", "1")
    attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k)
    d = W.paged_decode(seed=76, device=DEV, B=2, Hq=8, Hkv=2, lengths=[300, 20], lmax=512, pool=64)
    attn.attn_decode_paged(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens, num_splits=4)
    torch.cuda.synchronize()
    err = capfd.readouterr().err
    assert "[attn] launch (prefill_d128_kernel<false, false>)" in err
    assert "[attn] launch decode_split_kernel grid (2, 4, 2) block (256, 1, 1)" in err
    assert "[attn] launch decode_merge_kernel" in err
