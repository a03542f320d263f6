"""GPU parity of the one-token paged decode with NVFP4 fake quantization of P and V (attn_decode_paged_qdq)
against the fp64 oracle's sequential pass with the same quantizer.

The quantizer's rounding decisions are taken in fp32 on both sides.  With integer scores (Q and K small
integers, scale ln 2 so that the kernel's log2-domain scale is exactly 1) every P value is an exact power
of two on both sides, so both take identical decisions, skip maps included: those cases compare the skip
map exactly and the output to the bf16 bar.  With Gaussian inputs P comes from fp32 exponentials on the
GPU and fp64 ones in the oracle, so a P value within rounding of a code boundary may round the other way;
with thousands of keys per row one such flip moves the output far less than the bf16 bar, and the skip
maps are checked as in the other skip tests (>= 99.9 % agreement, outputs against the oracle replaying
the GPU's map).
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
DEV = "cuda"
LN2 = math.log(2)


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _exact(lengths, Hq=32, Hkv=8, seed=110, q_nnz=16):
    pool = sum((L + 15) // 16 for L in lengths) + 7
    return W.paged_decode_exact(seed=seed, device=DEV, B=len(lengths), Hq=Hq, Hkv=Hkv, D=128, lengths=lengths,
                                lmax=max(lengths), pool=pool, q_nnz=q_nnz)


LENGTHS = [1, 15, 16, 17, 31, 32, 33, 64, 100, 257, 1000, 2049, 4097, 0, 513]


def test_qdq_off_is_the_sequential_decode():
    x = W.paged_decode(seed=111, device=DEV, B=6, Hq=32, Hkv=8, D=128, lengths=[1, 33, 100, 600, 2000, 40],
                       lmax=2048, pool=300)
    for thr in (0.0, 0.1):
        a, la, ma = attn.attn_decode_paged_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                               skip_threshold=thr, return_lse=True, return_skip_map=True)
        b, lb, mb = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, num_splits=1,
                                           skip_threshold=thr, return_lse=True, return_skip_map=True)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and torch.equal(la, lb) and torch.equal(ma, mb)


@pytest.mark.parametrize("thr", [0.0, 0.1])
@pytest.mark.parametrize("p_amax,v_amax", [(1.0, 0.0), (0.0, "max"), (1.0, 1.0), (1.0, "max"), (0.5, 3.0)])
def test_qdq_exact_scores(thr, p_amax, v_amax):
    x = _exact(LENGTHS)
    if v_amax == "max":
        vc = x.v_cache.float()
        v_amax = float(vc[~torch.isnan(vc)].abs().max())
    o, lse, smap = attn.attn_decode_paged_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, scale=LN2,
                                              skip_threshold=thr, p_amax=p_amax, v_amax=v_amax, return_lse=True,
                                              return_skip_map=True)
    torch.cuda.synchronize()
    print(f"exact scores thr={thr} p_amax={p_amax} v_amax={v_amax}", flush=True)
    od, ld, om = oracle.decode_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, LN2, thr=thr,
                                   p_amax=p_amax, v_amax=v_amax)
    assert np.array_equal(smap.cpu().numpy()[..., :om.shape[-1]], om), "skip decisions differ"
    if thr > 0:
        assert (om == 1).any()
    go = _np(o)
    assert np.isfinite(go).all()
    err = np.max(np.abs(go - od))
    assert err <= BF16_TOL, err
    fin = np.isfinite(ld)
    assert np.array_equal(np.isfinite(_np(lse)), fin)
    assert np.max(np.abs(_np(lse)[fin] - ld[fin])) <= 1e-3
    # the quantization is visible: the output differs from the unquantized pass by much more than the bar
    # wherever P or V is quantized (a check that the quantizer is switched on at all)
    ou, _, _ = oracle.decode_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, LN2, thr=thr)
    assert np.max(np.abs(od - ou)) > BF16_TOL


def test_qdq_exact_scores_group_of_1_and_deterministic():
    x = _exact([1, 17, 64, 999, 2500, 0, 48], Hq=8, Hkv=8, seed=114)
    args = (x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens)
    o1, _, m1 = attn.attn_decode_paged_qdq(*args, scale=LN2, skip_threshold=0.2, p_amax=1.0, v_amax=2.5,
                                           return_skip_map=True)
    o2, _, m2 = attn.attn_decode_paged_qdq(*args, scale=LN2, skip_threshold=0.2, p_amax=1.0, v_amax=2.5,
                                           return_skip_map=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(m1, m2)
    od, _, om = oracle.decode_qdq(*args, LN2, thr=0.2, p_amax=1.0, v_amax=2.5)
    assert np.array_equal(m1.cpu().numpy()[..., :om.shape[-1]], om)
    assert np.max(np.abs(_np(o1) - od)) <= BF16_TOL
    assert torch.all(o1[5] == 0)  # the empty sequence


def test_qdq_exact_scores_group_of_16():
    x = _exact([1, 40, 300, 1500, 33], Hq=16, Hkv=1, seed=112)
    o, _, smap = attn.attn_decode_paged_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, scale=LN2,
                                            skip_threshold=0.05, p_amax=1.0, v_amax=2.0, return_skip_map=True)
    torch.cuda.synchronize()
    od, _, om = oracle.decode_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, LN2, thr=0.05, p_amax=1.0,
                                  v_amax=2.0)
    assert np.array_equal(smap.cpu().numpy()[..., :om.shape[-1]], om)
    assert np.max(np.abs(_np(o) - od)) <= BF16_TOL


@pytest.mark.parametrize("thr", [0.0, 0.1])
def test_qdq_gaussian(thr):
    # the pages' usage: amax 1 for both P and V (V ~ N(0, 1) then saturates above 1)
    lengths = [600, 1000, 2500, 4096, 3000, 777]
    x = W.paged_decode(seed=113, device=DEV, B=len(lengths), Hq=32, Hkv=8, D=128, lengths=lengths, lmax=4096,
                       pool=1000)
    o, lse, smap = attn.attn_decode_paged_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens,
                                              skip_threshold=thr, p_amax=1.0, v_amax=1.0, return_lse=True,
                                              return_skip_map=True)
    torch.cuda.synchronize()
    print(f"gaussian thr={thr}", flush=True)
    _, _, om = oracle.decode_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, thr=thr, p_amax=1.0,
                                 v_amax=1.0)
    g = smap.cpu().numpy()[..., :om.shape[-1]]
    assert np.array_equal(g == 2, om == 2)
    vis = om != 2
    assert (g[vis] == om[vis]).mean() >= 0.999
    rp = np.where(g == 1, 1, 0).reshape(-1, g.shape[-1])
    od, ld, _ = oracle.decode_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, p_amax=1.0,
                                  v_amax=1.0, replay=rp)
    go = _np(o)
    assert np.isfinite(go).all()
    assert np.max(np.abs(go - od)) <= BF16_TOL
    assert np.max(np.abs(_np(lse) - ld)) <= 1e-3


def test_qdq_invalid_amax_is_rejected():
    x = _exact([40])
    for bad in (-1.0, float("nan"), float("inf"), 1e-30, 1e30):
        with pytest.raises(attn.AttnError):
            attn.attn_decode_paged_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, p_amax=bad)
        with pytest.raises(attn.AttnError):
            attn.attn_decode_paged_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, v_amax=bad)
