"""The allocation-free decode entry point (attn_decode_paged_noalloc) through the C ABI, against
attn_decode_paged on the same inputs: the same kernels run, so outputs and LSEs must be bit-identical.
Two split-K calls in a row, the second smaller (its partials overwrite only part of what the first left
in the scratch), then the sequential skip schedule, which uses no scratch."""
import numpy as np
import pytest
import torch

import paged_skip_softmax_amd as attn
from paged_skip_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(x, **kw):
    ref, lref, mref = attn.attn_decode_paged(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, return_lse=True,
                                             **kw)
    out = torch.full_like(x.q, float("nan"))
    lse = torch.full((x.B, x.Hq), float("nan"), dtype=torch.float32, device=DEV)
    smap = None
    if mref is not None:
        smap = torch.full_like(mref, 7)
    attn.attn_decode_paged_noalloc(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, out=out, lse=lse,
                                   skip_map=smap, skip_threshold=kw.get("skip_threshold", 0.0),
                                   num_splits=kw.get("num_splits", 0))
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "outputs differ from attn_decode_paged"
    assert torch.equal(torch.isneginf(lse), torch.isneginf(lref))
    fin = torch.isfinite(lref)
    assert torch.equal(lse[fin], lref[fin]), "LSEs differ from attn_decode_paged"
    if mref is not None:
        assert torch.equal(smap, mref)
    assert np.isfinite(out.float().cpu().numpy()).all()


def test_noalloc_decode_matches_two_calls_then_sequential():
    # first call: 48 sequences, Hq 32, Hkv 8, 32 splits (25 MB of partials)
    print("noalloc: large split-K call", flush=True)
    big = W.paged_decode(seed=91, device=DEV, B=48, lmin=100, lmax=9000, pool=30000)
    _both(big, num_splits=32)
    # second call, smaller: 5 sequences (one empty, one of a single key), 7 splits, G = 4
    print("noalloc: small split-K call", flush=True)
    small = W.paged_decode(seed=92, device=DEV, B=5, Hq=8, Hkv=2, lengths=[0, 1, 300, 2049, 77], lmax=2100,
                           pool=400)
    _both(small, num_splits=7)
    # the default split count, then the sequential schedule with skip-softmax (no scratch) on hot keys
    print("noalloc: default splits and the sequential schedule", flush=True)
    _both(small)
    hot = W.paged_decode(seed=93, device=DEV, B=6, Hq=8, Hkv=2, lengths=[5, 700, 3000, 64, 1, 4096], lmax=4096,
                         pool=900, hot=True)
    _both(hot, num_splits=1, skip_threshold=0.1, return_skip_map=True)
