"""Seeded synthetic inputs for the attention hot path.

This module holds no attention arithmetic at all: only random draws, prefix sums that pack sequences
(cu_seqlens), the page-pool layout and NaN poison.  The HIP path (tests, bench) and the fp64 oracle both
read exactly the tensors built here, so the two sides see identical bytes.

Every random stream is its own ``torch.Generator`` seeded from ``(seed, stream)``; sequence lengths,
tile choices and the page permutation are always drawn on the CPU so that shapes do not depend on the
device, while bulk N(0,1) values are drawn on ``device`` (Philox on the GPU, so that multi-GB pools take
milliseconds).  Values are drawn in fp32 and rounded to bf16 with round-to-nearest-even where the
workload is bf16.

Workloads (sizes are the defaults; tests pass reduced sizes):

* ``tiny_dense``        B=2, Hq=4, Hkv=2, D=64, S=128, fp32, cu_seqlens [0,128,256].
* ``varlen_prefill``    16 sequences, lengths uniform in [256, 4096], THD packed, Hq=32, Hkv=8, D=128, bf16.
* ``varlen_prefill_hot`` ``varlen_prefill`` plus an attention-sink run and 2 % hot 32-key runs per
                        sequence aligned with the queries of each KV head's group (prefill skip-softmax).
* ``paged_decode``      B=64, Hq=32, Hkv=8, D=128, context lengths uniform in [1024, 32768], 16-token pages
                        in a 140,000-page pool laid out [page, kv_head, slot, D]; the block table holds
                        consecutive slices of one seeded permutation of the pool, padded with -1.  Pages no
                        sequence uses, and the slots past the last token of each sequence's last page, hold
                        NaN, so a wrong gather or a missing mask shows up as NaN.
* ``paged_decode_hot``  ``paged_decode`` plus "hot" keys: in each sequence a seeded set of
                        max(1, round(0.02 * L / 32)) distinct 32-aligned full 32-token runs gets
                        ``4 * sum_h q_h / |q_h|`` (sum over the query heads of the KV head's group) added to
                        every key of the run, before rounding to bf16.
* ``paged_decode_exact`` ``paged_decode`` with integer Q (16 entries of +-1 per head row) and K (entries in
                        {-1, 0, 1}), so that every score is an exact integer.
* ``smallseq_cross``    B=30720 sequences with s_q=1 and s_kv drawn from {2,4,6,8,12,16}, H=16, D=128, bf16,
                        THD packed K/V with cu_seqlens_kv.
"""
from __future__ import annotations

import math
from types import SimpleNamespace

import torch

# stream ids: one independent generator per purpose
_S_LEN, _S_Q, _S_K, _S_V, _S_PERM, _S_HOT, _S_DO, _S_QLEN, _S_EXACT = range(9)


def _gen(seed: int, stream: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + stream)
    return g


def _randn(shape, seed, stream, device, dtype):
    g = _gen(seed, stream, device)
    x = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    return x if dtype == torch.float32 else x.to(dtype)


def _uniform_int(n, lo, hi, seed, stream=_S_LEN):
    """n integers uniform on the inclusive range [lo, hi] (CPU)."""
    g = _gen(seed, stream)
    return torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64)


def _cu(lengths: torch.Tensor) -> torch.Tensor:
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(lengths.to(torch.int64), 0).to(torch.int32)
    return cu


def tiny_dense(seed=1000, device="cpu", B=2, Hq=4, Hkv=2, D=64, S=128, lengths=None):
    """fp32 THD inputs; every sequence has S tokens unless explicit ``lengths`` are given."""
    lens = torch.tensor(lengths if lengths is not None else [S] * B, dtype=torch.int64)
    cu = _cu(lens)
    T = int(cu[-1])
    q = _randn((T, Hq, D), seed, _S_Q, device, torch.float32)
    k = _randn((T, Hkv, D), seed, _S_K, device, torch.float32)
    v = _randn((T, Hkv, D), seed, _S_V, device, torch.float32)
    return SimpleNamespace(q=q, k=k, v=v, cu_q=cu.to(device), cu_k=cu.to(device), lens=lens,
                           B=len(lens), Hq=Hq, Hkv=Hkv, D=D, max_q=int(lens.max()) if len(lens) else 0,
                           max_k=int(lens.max()) if len(lens) else 0, scale=1.0 / math.sqrt(D),
                           dtype=torch.float32)


def varlen_prefill(seed=1001, device="cpu", nseq=16, lmin=256, lmax=4096, Hq=32, Hkv=8, D=128,
                   dtype=torch.bfloat16, lengths=None):
    """THD-packed self-attention prefill inputs (same lengths for Q and K/V)."""
    lens = (torch.tensor(lengths, dtype=torch.int64) if lengths is not None
            else _uniform_int(nseq, lmin, lmax, seed))
    cu = _cu(lens)
    T = int(cu[-1])
    q = _randn((T, Hq, D), seed, _S_Q, device, dtype)
    k = _randn((T, Hkv, D), seed, _S_K, device, dtype)
    v = _randn((T, Hkv, D), seed, _S_V, device, dtype)
    return SimpleNamespace(q=q, k=k, v=v, cu_q=cu.to(device), cu_k=cu.to(device), lens=lens,
                           B=len(lens), Hq=Hq, Hkv=Hkv, D=D, max_q=int(lens.max()), max_k=int(lens.max()),
                           scale=1.0 / math.sqrt(D), dtype=dtype)


def varlen_prefill_hot(seed=1001, device="cpu", q_align=2.0, k_boost=24.0, hot_frac=0.02, hot_run=32, **kw):
    """``varlen_prefill`` plus hot keys that most later key tiles fall far below (prefill skip-softmax).

    Per sequence b and KV head g a seeded unit direction u is drawn; every query of the group's heads
    gets ``q_align * u`` added and every key of the sequence's hot runs gets ``k_boost * u`` added (before
    rounding to bf16), which lifts the hot logits by about q_align * k_boost / sqrt(D) (4.2 at the
    defaults).  The hot runs are the first 32 keys of the sequence (an attention sink) plus
    max(0, round(hot_frac * L / hot_run) - 1) further distinct 32-aligned full runs chosen by seed.  With
    the same seed the lengths, V and the unperturbed parts of Q and K equal ``varlen_prefill``'s."""
    x = varlen_prefill(seed=seed, device=device, **kw)
    G = x.Hq // x.Hkv
    g = _gen(seed, _S_HOT)
    u = torch.randn(x.B, x.Hkv, x.D, generator=g, dtype=torch.float32)
    u = (u / u.norm(dim=-1, keepdim=True)).to(device)
    q = x.q.float()
    k = x.k.float()
    cu = x.cu_q.cpu().tolist()
    hot_tiles = []
    for b in range(x.B):
        L = cu[b + 1] - cu[b]
        q[cu[b]:cu[b + 1]].view(L, x.Hkv, G, x.D).add_(q_align * u[b][None, :, None, :])
        nfull = L // hot_run
        extra = max(0, int(round(hot_frac * L / hot_run)) - 1)
        tiles = [0] if L > 0 else []
        if nfull > 1 and extra > 0:
            tiles += sorted((1 + torch.randperm(nfull - 1, generator=g)[:extra]).tolist())
        hot_tiles.append(tiles)
        for t in tiles:
            j0, j1 = cu[b] + t * hot_run, min(cu[b] + (t + 1) * hot_run, cu[b + 1])
            k[j0:j1].add_(k_boost * u[b][None, :, :])
    x.q = q.to(x.dtype)
    x.k = k.to(x.dtype)
    x.hot_tiles = hot_tiles
    return x


def grad_output(x, seed=1005, device="cpu"):
    """A seeded standard-normal output gradient dO shaped like x.q (backward inputs)."""
    return _randn(tuple(x.q.shape), seed, _S_DO, device, x.q.dtype)


def varlen_prefill_sink(seed=1001, device="cpu", **kw):
    """``varlen_prefill_hot`` with a coherent attention sink: queries lean harder towards the shared
    direction (q_align 8) and hot keys less (k_boost 12), so the hot logits rise by about 8.5 with a row
    spread of about 1 (against about 2 at the defaults): nearly every query row of a sequence sees the
    sink far above its ordinary tiles, as with the attention sinks of trained models."""
    return varlen_prefill_hot(seed=seed, device=device, q_align=8.0, k_boost=12.0, **kw)


def _page_table(lens, page, pool, max_pages, seed):
    """Block table of consecutive slices of one seeded permutation of the pool, padded with -1."""
    g = _gen(seed, _S_PERM)
    perm = torch.randperm(pool, generator=g, dtype=torch.int64)
    npages = [(int(L) + page - 1) // page for L in lens]
    if sum(npages) > pool:
        raise ValueError("page pool too small for the drawn lengths")
    bt = torch.full((len(lens), max_pages), -1, dtype=torch.int32)
    off = 0
    for b, n in enumerate(npages):
        bt[b, :n] = perm[off:off + n].to(torch.int32)
        off += n
    return bt, perm[:off], npages


def paged_decode(seed=1002, device="cpu", B=64, Hq=32, Hkv=8, D=128, lmin=1024, lmax=32768, page=16,
                 pool=140000, lengths=None, hot=False, hot_mag=4.0, hot_frac=0.02, hot_run=32):
    """One-token paged decode inputs; ``hot=True`` builds the hot-key variant (see module doc)."""
    lens = (torch.tensor(lengths, dtype=torch.int64) if lengths is not None
            else _uniform_int(B, lmin, lmax, seed))
    max_pages = (max(int(lmax), int(lens.max()) if len(lens) else 0) + page - 1) // page
    bt, used, npages = _page_table(lens, page, pool, max_pages, seed)
    q = _randn((B, Hq, D), seed, _S_Q, device, torch.bfloat16)
    nused = len(used)
    # K and V values of the used pages, drawn in page-list order (sequence-major), in fp32
    kf = _randn((nused, Hkv, page, D), seed, _S_K, device, torch.float32)
    hot_tiles = []
    if hot:
        G = Hq // Hkv
        qf = q.float()
        qn = qf / qf.norm(dim=-1, keepdim=True)                        # [B, Hq, D]
        direction = hot_mag * qn.view(B, Hkv, G, D).sum(2)             # [B, Hkv, D]
        g = _gen(seed, _S_HOT)
        off = 0
        for b in range(B):
            L = int(lens[b])
            nfull = L // hot_run
            nh = max(1, int(round(hot_frac * L / hot_run)))
            nh = min(nh, nfull)
            tiles = torch.randperm(nfull, generator=g)[:nh].sort().values.tolist() if nfull else []
            hot_tiles.append(tiles)
            for t in tiles:
                j0, j1 = t * hot_run, (t + 1) * hot_run
                for p in range(j0 // page, (j1 - 1) // page + 1):
                    s0, s1 = max(j0, p * page) - p * page, min(j1, (p + 1) * page) - p * page
                    kf[off + p, :, s0:s1, :] += direction[b][:, None, :]
            off += npages[b]
    v_used = _randn((nused, Hkv, page, D), seed, _S_V, device, torch.bfloat16)
    k_used = kf.to(torch.bfloat16)
    del kf
    nan = float("nan")
    k_cache = torch.full((pool, Hkv, page, D), nan, dtype=torch.bfloat16, device=device)
    v_cache = torch.full((pool, Hkv, page, D), nan, dtype=torch.bfloat16, device=device)
    # poison the slots past the end of each sequence's last page
    off = 0
    for b in range(B):
        n, L = npages[b], int(lens[b])
        tail = n * page - L
        if tail:
            k_used[off + n - 1, :, page - tail:, :] = nan
            v_used[off + n - 1, :, page - tail:, :] = nan
        off += n
    idx = used.to(device)
    k_cache[idx] = k_used
    v_cache[idx] = v_used
    del k_used, v_used
    return SimpleNamespace(q=q, k_cache=k_cache, v_cache=v_cache, block_table=bt.to(device),
                           seq_lens=lens.to(torch.int32).to(device), lens=lens, B=B, Hq=Hq, Hkv=Hkv, D=D,
                           page=page, pool=pool, max_pages=max_pages, scale=1.0 / math.sqrt(D),
                           hot_tiles=hot_tiles, dtype=torch.bfloat16)


def paged_decode_hot(seed=1002, device="cpu", **kw):
    """The hot-key decode workload; with the same seed its lengths, Q, V and table equal paged_decode's."""
    return paged_decode(seed=seed, device=device, hot=True, **kw)


def paged_decode_exact(seed=1006, device="cpu", q_nnz=16, **kw):
    """``paged_decode`` (built on the CPU, then moved) with small-integer Q and K: each query head row has
    q_nnz entries +-1 at random positions and zeros elsewhere, every key entry is -1, 0 or +1 (the slots
    past a sequence's end stay NaN).  Every score q.k is then an integer in [-q_nnz, q_nnz], which bf16
    products and an fp32 sum give exactly; V is paged_decode's."""
    x = paged_decode(seed=seed, device="cpu", **kw)
    g = _gen(seed, _S_EXACT)
    B, Hq, D = x.q.shape
    pos = torch.rand((B, Hq, D), generator=g).argsort(-1)[..., :q_nnz]
    sign = (torch.randint(0, 2, (B, Hq, q_nnz), generator=g) * 2 - 1).float()
    q = torch.zeros(B, Hq, D).scatter_(-1, pos, sign)
    kint = torch.randint(-1, 2, tuple(x.k_cache.shape), generator=g).to(torch.bfloat16)
    kc = torch.where(torch.isnan(x.k_cache), x.k_cache, kint)
    x.q = q.to(torch.bfloat16).to(device)
    x.k_cache = kc.to(device)
    x.v_cache = x.v_cache.to(device)
    x.block_table = x.block_table.to(device)
    x.seq_lens = x.seq_lens.to(device)
    return x


def paged_decode_multi(seed=1002, device="cpu", qmin=1, qmax=4, **kw):
    """Multi-token paged decode: ``paged_decode``'s cache (the same one for the same seed) plus
    Lq_b ~ U{qmin..qmax} new query tokens per sequence (at most L_b), packed THD with cu_seqlens_q; they
    are the last Lq_b of the L_b cached keys."""
    x = paged_decode(seed=seed, device=device, **kw)
    g = _gen(seed, _S_QLEN)
    ql = torch.randint(qmin, qmax + 1, (x.B,), generator=g, dtype=torch.int64)
    ql = torch.minimum(ql, x.lens)
    cu = _cu(ql)
    x.q = _randn((int(cu[-1]), x.Hq, x.D), seed, _S_Q, device, torch.bfloat16)
    x.cu_q = cu.to(device)
    x.qlens = ql
    x.max_q = int(ql.max()) if x.B else 0
    return x


def smallseq_cross(seed=1004, device="cpu", B=30720, H=16, D=128, choices=(2, 4, 6, 8, 12, 16),
                   fixed=None, dtype=torch.bfloat16):
    """s_q = 1 cross-attention inputs; ``fixed`` forces every s_kv to one value."""
    if fixed is not None:
        lens = torch.full((B,), int(fixed), dtype=torch.int64)
    else:
        idx = _uniform_int(B, 0, len(choices) - 1, seed)
        lens = torch.tensor(choices, dtype=torch.int64)[idx]
    cu = _cu(lens)
    T = int(cu[-1])
    q = _randn((B, H, D), seed, _S_Q, device, dtype)
    k = _randn((T, H, D), seed, _S_K, device, dtype)
    v = _randn((T, H, D), seed, _S_V, device, dtype)
    return SimpleNamespace(q=q, k=k, v=v, cu_kv=cu.to(device), lens=lens, B=B, H=H, D=D,
                           max_s=int(lens.max()) if B else 0, scale=1.0 / math.sqrt(D), dtype=dtype)
