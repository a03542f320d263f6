"""GPU parity of the prefill backward (dq, dk, dv) against the fp64 oracle, through the C ABI.

Inputs: the backward reads a stored forward output o (bf16) and LSE (fp32).  The parity tests give both
sides the same o, the oracle's forward output rounded to bf16, and the GPU the oracle's LSE in fp32;
the oracle then forms dS from the same row dots dO.o as the GPU.  One test chains the GPU forward into
the GPU backward, as a training step does (see its comment for what it checks).

Tolerance, derived from the arithmetic: each gradient element is a sum over rows (dk, dv) or keys (dq)
of products whose factors the kernels round to bf16 (P and dS, relative 2^-9 each; dS is formed from
the rounded P, which adds one more 2^-9 to it) before fp32 accumulation, and the result is rounded to
bf16 once more.  The rounding error of such a sum grows like
the root of the summed squared terms, which is shared by the whole (token, head) row of D elements (the
row's rms), not like the element itself, which cancellation can make small.  So every element must
satisfy
    |gpu - oracle| <= 2e-2 * max(1, |oracle|, rms of the oracle over its (token, head) row)
(2e-2 is the forward's bf16 bound for unit-scale values; the rounded factors alone give about 1e-2 at
the tail of these sums), and the relative L2 error of each whole gradient must stay <= 1e-2, which any
indexing or missing-term mistake exceeds by far.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_skip_softmax_amd as attn
from paged_skip_softmax_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
REL_TOL = 2e-2
L2_TOL = 1e-2


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(name, gpu, ref, elementwise=True):
    g = _np(gpu)
    assert np.isfinite(g).all(), f"{name}: non-finite values"
    if not ref.size:
        return
    if elementwise:
        err = np.abs(g - ref)
        row_rms = np.sqrt(np.mean(ref ** 2, axis=-1, keepdims=True))
        worst = float(np.max(err / np.maximum(1.0, np.maximum(np.abs(ref), row_rms))))
        assert worst <= REL_TOL, f"{name}: max |err| / max(1, |ref|, row rms) = {worst:.4f}"
    nrm = np.linalg.norm(ref)
    if nrm > 0:
        rel = float(np.linalg.norm(g - ref) / nrm)
        assert rel <= L2_TOL, f"{name}: relative L2 error {rel:.2e}"


def _stored_forward(q, k, v, cq, ck, Hq, Hkv, scale, causal):
    """The oracle's forward output rounded to bf16 and its LSE in fp32 (the stored forward state)."""
    o, lse, _ = oracle.prefill(q.cpu(), k.cpu(), v.cpu(), cq.cpu(), ck.cpu(), Hq, Hkv, scale, causal)
    return torch.from_numpy(o).to(torch.bfloat16), torch.from_numpy(lse).to(torch.float32)


def _run(q, k, v, do, cq, ck, mq, mk, Hq, Hkv, scale, causal):
    """GPU backward on the oracle's stored forward state, and the oracle's gradients for the same o."""
    o, lse = _stored_forward(q, k, v, cq, ck, Hq, Hkv, scale, causal)
    got = attn.attn_prefill_varlen_backward(q, k, v, o.to(DEV), do, lse.to(DEV), cq, ck, mq, mk, scale=scale,
                                            causal=causal)
    torch.cuda.synchronize()
    ref = oracle.prefill_backward(q.cpu(), k.cpu(), v.cpu(), do.cpu(), cq.cpu(), ck.cpu(), Hq, Hkv, scale, causal,
                                  o=o)
    return got, ref


def _grads(got, ref):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        _check(name, g, r)


@pytest.mark.parametrize("causal", [True, False])
def test_backward_varlen_ragged(causal):
    # lengths cover a 1-row sequence, an empty one, and tails of every size around the 32/64 tiles
    lens = [1, 17, 128, 0, 129, 300, 64, 255]
    x = W.varlen_prefill(seed=31, device=DEV, lengths=lens, Hq=8, Hkv=2)
    do = W.grad_output(x, seed=32, device=DEV)
    _grads(*_run(x.q, x.k, x.v, do, x.cu_q, x.cu_k, x.max_q, x.max_k, 8, 2, x.scale, causal))


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2), (32, 2), (12, 3), (6, 2)])
def test_backward_gqa_groupings(Hq, Hkv):
    lens = [77, 200, 33]
    x = W.varlen_prefill(seed=41, device=DEV, lengths=lens, Hq=Hq, Hkv=Hkv)
    do = W.grad_output(x, seed=42, device=DEV)
    _grads(*_run(x.q, x.k, x.v, do, x.cu_q, x.cu_k, x.max_q, x.max_k, Hq, Hkv, x.scale, True))


@pytest.mark.parametrize("causal", [True, False])
def test_backward_cross_lengths(causal):
    # Lq != Lk with bottom-right causal alignment: Lq > Lk (leading rows see no key: dq = 0), a sequence
    # without keys (dq = 0) and one without queries (dk = dv = 0)
    Hq, Hkv, D = 4, 2, 128
    lq, lk = [70, 5, 33, 0, 100], [40, 90, 0, 50, 3]
    g = torch.Generator(device=DEV).manual_seed(9)
    q = torch.randn(sum(lq), Hq, D, generator=g, device=DEV).bfloat16()
    k = torch.randn(sum(lk), Hkv, D, generator=g, device=DEV).bfloat16()
    v = torch.randn(sum(lk), Hkv, D, generator=g, device=DEV).bfloat16()
    do = torch.randn(sum(lq), Hq, D, generator=g, device=DEV).bfloat16()
    cq = torch.tensor([0] + list(np.cumsum(lq)), dtype=torch.int32, device=DEV)
    ck = torch.tensor([0] + list(np.cumsum(lk)), dtype=torch.int32, device=DEV)
    got, ref = _run(q, k, v, do, cq, ck, max(lq), max(lk), Hq, Hkv, D ** -0.5, causal)
    _grads(got, ref)
    dq, dk, dv = (_np(t) for t in got)
    assert np.all(dq[75:108] == 0)  # the sequence with no keys
    assert np.all(dk[130:180] == 0) and np.all(dv[130:180] == 0)  # the keys no query sees
    if causal:
        assert np.all(dq[:30] == 0)  # rows 0..29 of the first sequence precede every key


def test_backward_chained_after_gpu_forward():
    # o and lse from the GPU forward, as in training.  dv does not depend on o and meets the elementwise
    # bound; dq and dk also carry the forward's own bf16 rounding of o through the row dots dO.o (a shift
    # of dS by p times dO.(o_gpu - o)), so for them the whole-tensor relative L2 bound is checked.
    lens = [1, 17, 128, 0, 129, 300, 64, 255]
    x = W.varlen_prefill(seed=61, device=DEV, lengths=lens, Hq=8, Hkv=2)
    do = W.grad_output(x, seed=62, device=DEV)
    o, lse, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=True,
                                         return_lse=True)
    dq, dk, dv = attn.attn_prefill_varlen_backward(x.q, x.k, x.v, o, do, lse, x.cu_q, x.cu_k, x.max_q, x.max_k,
                                                   causal=True)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.prefill_backward(x.q.cpu(), x.k.cpu(), x.v.cpu(), do.cpu(), x.cu_q.cpu(), x.cu_k.cpu(), 8, 2,
                                         x.scale, True)
    _check("dv", dv, rv)
    _check("dq", dq, rq, elementwise=False)
    _check("dk", dk, rk, elementwise=False)


def test_backward_deterministic():
    # no atomics: two calls give the same bits
    x = W.varlen_prefill(seed=51, device=DEV, lengths=[300, 65, 129], Hq=8, Hkv=2)
    do = W.grad_output(x, seed=52, device=DEV)
    o, lse, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, return_lse=True)
    a = attn.attn_prefill_varlen_backward(x.q, x.k, x.v, o, do, lse, x.cu_q, x.cu_k, x.max_q, x.max_k)
    b = attn.attn_prefill_varlen_backward(x.q, x.k, x.v, o, do, lse, x.cu_q, x.cu_k, x.max_q, x.max_k)
    torch.cuda.synchronize()
    for s, t in zip(a, b):
        assert torch.equal(s, t)


def test_backward_stream_ordered_with_two_callers():
    # part of the backward runs on a side stream that the call forks from and joins back to its stream:
    # copies taken on the caller's stream right after the call (no host synchronization in between) hold
    # the finished gradients, also with two callers' streams (default priority) working at once
    x = W.varlen_prefill(seed=53, device=DEV, lengths=[300, 65, 129, 700], Hq=8, Hkv=2)
    do = W.grad_output(x, seed=54, device=DEV)
    o, lse, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, return_lse=True)
    ref = attn.attn_prefill_varlen_backward(x.q, x.k, x.v, o, do, lse, x.cu_q, x.cu_k, x.max_q, x.max_k)
    torch.cuda.synchronize()
    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    outs = []
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            g = attn.attn_prefill_varlen_backward(x.q, x.k, x.v, o, do, lse, x.cu_q, x.cu_k, x.max_q, x.max_k)
            outs.append([t.clone() for t in g])
    torch.cuda.synchronize()
    for got in outs:
        for s_, t in zip(got, ref):
            assert torch.equal(s_, t)


def test_backward_full_size_sampled_sequences():
    # the full prefill workload (16 sequences of 935..4083 tokens, Hq 32, Hkv 8) in one backward call.  The
    # stored state is the GPU forward's, except for three whole sequences (the shortest, a middle and the
    # longest) whose o and lse rows are the oracle's; the oracle checks every gradient of those three
    # (sequences are independent).
    x = W.varlen_prefill(seed=1001, device=DEV)
    do = W.grad_output(x, seed=1005, device=DEV)
    o, lse, _ = attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k, causal=True,
                                         return_lse=True)
    lens = x.lens.tolist()
    cu = x.cu_q.cpu().tolist()
    order = sorted(range(x.B), key=lambda b: lens[b])
    picked = (order[0], order[len(order) // 2], order[-1])
    c1 = {b: torch.tensor([0, lens[b]], dtype=torch.int32) for b in picked}
    stored = {}
    for b in picked:
        s = slice(cu[b], cu[b + 1])
        stored[b] = _stored_forward(x.q[s], x.k[s], x.v[s], c1[b], c1[b], x.Hq, x.Hkv, x.scale, True)
        o[s] = stored[b][0].to(DEV)
        lse[s] = stored[b][1].to(DEV)
    dq, dk, dv = attn.attn_prefill_varlen_backward(x.q, x.k, x.v, o, do, lse, x.cu_q, x.cu_k, x.max_q, x.max_k,
                                                   causal=True)
    torch.cuda.synchronize()
    for b in picked:
        s = slice(cu[b], cu[b + 1])
        ref = oracle.prefill_backward(x.q[s].cpu(), x.k[s].cpu(), x.v[s].cpu(), do[s].cpu(), c1[b], c1[b], x.Hq,
                                      x.Hkv, x.scale, True, o=stored[b][0])
        for name, g, r in zip(("dq", "dk", "dv"), (dq[s], dk[s], dv[s]), ref):
            _check(f"{name} of sequence {b} (L {lens[b]})", g, r)


# ------------------------------------------------------------------ small-seq backward

def _smallseq_stored(x):
    """The oracle's attention weights rounded to bf16 (the stored forward state)."""
    _, w = oracle.smallseq(x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_kv.cpu(), x.max_s, x.scale)
    return torch.from_numpy(w).to(torch.bfloat16)


def _smallseq_check(x, do, w):
    got = attn.attn_smallseq_cross_backward(x.q, x.k, x.v, w.to(DEV), do, x.cu_kv, x.max_s, scale=x.scale)
    torch.cuda.synchronize()
    ref = oracle.smallseq_backward(x.q.cpu(), x.k.cpu(), x.v.cpu(), w, do.cpu(), x.cu_kv.cpu(), x.max_s, x.scale)
    _grads(got, ref)
    return got, ref


@pytest.mark.parametrize("H", [16, 20])
@pytest.mark.parametrize("fixed", [None, 1, 16])
def test_smallseq_backward(H, fixed):
    # key counts from {2..16} (or all 1 / all 16), plus H = 20 for a partial block of 16 heads
    x = W.smallseq_cross(seed=71, device=DEV, B=257, H=H, fixed=fixed)
    do = W.grad_output(x, seed=72, device=DEV)
    _smallseq_check(x, do, _smallseq_stored(x))


def test_smallseq_backward_zero_length():
    # sequences without keys: dq = 0; the other sequences are unaffected
    g = torch.Generator(device=DEV).manual_seed(5)
    lens = [3, 0, 16, 0, 1]
    H, D = 16, 128
    q = torch.randn(len(lens), H, D, generator=g, device=DEV).bfloat16()
    k = torch.randn(sum(lens), H, D, generator=g, device=DEV).bfloat16()
    v = torch.randn(sum(lens), H, D, generator=g, device=DEV).bfloat16()
    do = torch.randn(len(lens), H, D, generator=g, device=DEV).bfloat16()
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32, device=DEV)
    from types import SimpleNamespace
    x = SimpleNamespace(q=q, k=k, v=v, cu_kv=cu, max_s=16, scale=D ** -0.5)
    got, _ = _smallseq_check(x, do, _smallseq_stored(x))
    dq = _np(got[0])
    assert np.all(dq[1] == 0) and np.all(dq[3] == 0)


def test_smallseq_backward_full_size_chained():
    # the full small-seq workload (B 30720, s_kv in {2..16}, H 16): every gradient against the oracle on
    # the oracle's stored weights; then the GPU forward's own weights chained into the GPU backward (its
    # weights differ from the oracle's by bf16 rounding, so the chained gradients get the L2 bound)
    x = W.smallseq_cross(seed=1004, device=DEV)
    do = W.grad_output(x, seed=1006, device=DEV)
    _, ref = _smallseq_check(x, do, _smallseq_stored(x))
    _, w_gpu, _ = attn.attn_smallseq_cross(x.q, x.k, x.v, x.cu_kv, x.max_s)
    chained = attn.attn_smallseq_cross_backward(x.q, x.k, x.v, w_gpu, do, x.cu_kv, x.max_s)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), chained, ref):
        _check(f"chained {name}", g, r, elementwise=False)
