"""Pins for the fp64 oracle: brute force, a library special case, closed forms and invariants.

Each test checks the oracle against something other than itself, so that a dropped term, a wrong sign,
a wrong index or a transposed operand in oracle/oracle.c fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import brute
import oracle
from paged_skip_softmax_amd import workloads as W

TOL = 1e-12


def _f64(x):
    return x.detach().cpu().double().numpy() if isinstance(x, torch.Tensor) else np.asarray(x, np.float64)


# ---------------------------------------------------------------- brute force, tiny inputs

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_dense_matches_brute_force(causal, dtype):
    lens = [5, 1, 17, 33]
    x = W.varlen_prefill(seed=7, lengths=lens, Hq=4, Hkv=2, D=8, dtype=dtype)
    o, lse, _ = oracle.prefill(x.q, x.k, x.v, x.cu_q, x.cu_k, 4, 2, 0.37, causal)
    q, k, v = _f64(x.q), _f64(x.k), _f64(x.v)
    start = 0
    for L in lens:
        for i in range(L):
            for h in range(4):
                g = h // 2
                nvis = i + 1 if causal else L
                keys = [list(k[start + j, g]) for j in range(nvis)]
                vals = [list(v[start + j, g]) for j in range(nvis)]
                ob, lb, _ = brute.softmax_attend(brute.scores(list(q[start + i, h]), keys, 0.37), vals)
                assert np.max(np.abs(o[start + i, h] - ob)) < TOL
                assert abs(lse[start + i, h] - lb) < TOL
        start += L


def test_decode_dense_matches_brute_force():
    x = W.paged_decode(seed=3, B=3, Hq=4, Hkv=2, D=8, page=4, pool=64, lengths=[1, 6, 13], lmax=16)
    o, lse, _ = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, 0.5)
    q, kc, vc = _f64(x.q), _f64(x.k_cache), _f64(x.v_cache)
    bt = x.block_table.numpy()
    for b, L in enumerate([1, 6, 13]):
        for h in range(4):
            keys = [list(kc[bt[b, j // 4], h // 2, j % 4]) for j in range(L)]
            vals = [list(vc[bt[b, j // 4], h // 2, j % 4]) for j in range(L)]
            ob, lb, _ = brute.softmax_attend(brute.scores(list(q[b, h]), keys, 0.5), vals)
            assert np.max(np.abs(o[b, h] - ob)) < TOL and abs(lse[b, h] - lb) < TOL


@pytest.mark.parametrize("thr", [0.0, 0.05, 0.3, 0.9])
@pytest.mark.parametrize("tile", [4, 7])
def test_skip_matches_brute_force(thr, tile):
    # a few large-logit keys make skipping common
    lens = [3, 29, 40]
    x = W.varlen_prefill(seed=11, lengths=lens, Hq=2, Hkv=1, D=6, dtype=torch.float32)
    kk = x.k.clone()
    kk[10:13] += 3.0 * x.q[10:13, :1].sign()
    o, lse, mp = oracle.prefill(x.q, kk, x.v, x.cu_q, x.cu_k, 2, 1, 0.8, True, mode="skip", thr=thr,
                                tile=tile)
    q, k, v = _f64(x.q), _f64(kk), _f64(x.v)
    start = 0
    for L in lens:
        for i in range(L):
            for h in range(2):
                keys = [list(k[start + j, 0]) for j in range(i + 1)]
                vals = [list(v[start + j, 0]) for j in range(i + 1)]
                ob, lb, dec = brute.skip_attend(brute.scores(list(q[start + i, h]), keys, 0.8), vals, tile, thr)
                assert np.max(np.abs(o[start + i, h] - ob)) < TOL and abs(lse[start + i, h] - lb) < TOL
                got = list(mp[start + i, h, :len(dec)])
                assert got == dec
                assert all(c == 2 for c in mp[start + i, h, len(dec):])
        start += L


def test_skip_replay_imposes_decisions():
    x = W.varlen_prefill(seed=12, lengths=[64], Hq=1, Hkv=1, D=4, dtype=torch.float32)
    o0, _, m0 = oracle.prefill(x.q, x.k, x.v, x.cu_q, x.cu_k, 1, 1, 0.5, False, mode="skip", thr=0.0, tile=8)
    rng = np.random.default_rng(0)
    rep = (rng.random(m0.shape) < 0.4).astype(np.uint8)
    rep[..., 0] = 0
    o1, lse1, m1 = oracle.prefill(x.q, x.k, x.v, x.cu_q, x.cu_k, 1, 1, 0.5, False, mode="skip", tile=8,
                                  replay=rep.reshape(64, -1), stride=m0.shape[-1])
    assert np.array_equal(m1, rep)
    q, k, v = _f64(x.q), _f64(x.k), _f64(x.v)
    for i in range(64):
        keep = [j for j in range(64) if rep[i, 0, j // 8] == 0]
        ob, lb, _ = brute.softmax_attend(brute.scores(list(q[i, 0]), [list(k[j, 0]) for j in keep], 0.5),
                                         [list(v[j, 0]) for j in keep])
        assert np.max(np.abs(o1[i, 0] - ob)) < TOL and abs(lse1[i, 0] - lb) < TOL


def test_smallseq_matches_brute_force():
    x = W.smallseq_cross(seed=5, B=6, H=3, D=8)
    o, w, lse = oracle.smallseq(x.q, x.k, x.v, x.cu_kv, x.max_s, 0.3, with_lse=True)
    q, k, v = _f64(x.q), _f64(x.k), _f64(x.v)
    cu = x.cu_kv.numpy()
    for b in range(6):
        for h in range(3):
            keys = [list(k[j, h]) for j in range(cu[b], cu[b + 1])]
            vals = [list(v[j, h]) for j in range(cu[b], cu[b + 1])]
            ob, lb, p = brute.softmax_attend(brute.scores(list(q[b, h]), keys, 0.3), vals)
            assert np.max(np.abs(o[b, h] - ob)) < TOL
            assert np.max(np.abs(w[b, h, 0, :len(p)] - p)) < TOL
            assert np.all(w[b, h, 0, len(p):] == 0)
            assert abs(lse[b, h] - lb) < TOL
    # the rows= form returns the same LSE per (b, head), and a sequence with no key gives -inf
    _, _, lr = oracle.smallseq(x.q, x.k, x.v, x.cu_kv, x.max_s, 0.3, rows=[(5, 2), (0, 1)], with_lse=True)
    assert lr[0] == lse[5, 2] and lr[1] == lse[0, 1]
    cu0 = torch.tensor([0, 0], dtype=torch.int32)
    o0, _, l0 = oracle.smallseq(x.q[:1], x.k, x.v, cu0, 16, 0.3, with_lse=True)
    assert l0[0, 0] == -np.inf and np.all(o0 == 0)


# ---------------------------------------------------------------- library special case

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_prefill_matches_torch_sdpa_fp64(causal, dtype):
    lens = [37, 128, 64]
    x = W.varlen_prefill(seed=21, lengths=lens, Hq=8, Hkv=2, D=32, dtype=dtype)
    o, lse, _ = oracle.prefill(x.q, x.k, x.v, x.cu_q, x.cu_k, 8, 2, x.scale, causal)
    cu = x.cu_q.tolist()
    for b in range(3):
        q = x.q[cu[b]:cu[b + 1]].double().transpose(0, 1)
        k = x.k[cu[b]:cu[b + 1]].double().transpose(0, 1).repeat_interleave(4, 0)
        v = x.v[cu[b]:cu[b + 1]].double().transpose(0, 1).repeat_interleave(4, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=x.scale)
        assert np.max(np.abs(o[cu[b]:cu[b + 1]] - ref.transpose(0, 1).numpy())) < TOL


# ---------------------------------------------------------------- closed forms

def test_closed_forms():
    # worked by hand: q=(1,0), keys e1,e2, values e1,e2, scale 1 -> p = (e, 1)/(e+1)
    q = torch.tensor([[[1.0, 0.0]]])
    k = torch.tensor([[[1.0, 0.0]], [[0.0, 1.0]]])
    cu_q, cu_k = torch.tensor([0, 1], dtype=torch.int32), torch.tensor([0, 2], dtype=torch.int32)
    o, lse, _ = oracle.prefill(q, k, k.clone(), cu_q, cu_k, 1, 1, 1.0, False)
    e = math.e
    assert np.allclose(o[0, 0], [e / (e + 1), 1 / (e + 1)], atol=TOL, rtol=0)
    assert abs(lse[0, 0] - math.log(e + 1)) < TOL

    x = W.varlen_prefill(seed=2, lengths=[9], Hq=2, Hkv=1, D=5, dtype=torch.float32)
    v = x.v
    # identical keys -> mean of V
    kk = x.k[:1].expand(9, 1, 5).contiguous()
    o, lse, _ = oracle.prefill(x.q, kk, v, x.cu_q, x.cu_k, 2, 1, 0.7, False)
    assert np.max(np.abs(o - _f64(v).mean(0)[None, 0:1])) < TOL
    # q = 0 -> mean of V and lse = log n
    o, lse, _ = oracle.prefill(torch.zeros_like(x.q), x.k, v, x.cu_q, x.cu_k, 2, 1, 0.7, False)
    assert np.max(np.abs(o - _f64(v).mean(0)[None, 0:1])) < TOL
    assert np.max(np.abs(lse - math.log(9))) < TOL
    # constant V -> that constant
    o, _, _ = oracle.prefill(x.q, x.k, torch.full_like(v, 1.25), x.cu_q, x.cu_k, 2, 1, 0.7, True)
    assert np.max(np.abs(o - 1.25)) < TOL
    # a single visible key (causal row 0) -> that key's value, lse = its logit
    o, lse, _ = oracle.prefill(x.q, x.k, v, x.cu_q, x.cu_k, 2, 1, 0.7, True)
    assert np.max(np.abs(o[0] - _f64(v)[0, 0])) < TOL
    s00 = 0.7 * float(_f64(x.q)[0, 0] @ _f64(x.k)[0, 0])
    assert abs(lse[0, 0] - s00) < TOL


def test_probabilities_sum_to_one_and_lse_normalises():
    x = W.varlen_prefill(seed=4, lengths=[50], Hq=2, Hkv=2, D=16, dtype=torch.bfloat16)
    o, lse, _ = oracle.prefill(x.q, x.k, x.v, x.cu_q, x.cu_k, 2, 2, 0.25, False)
    s = 0.25 * np.einsum("ihd,jhd->hij", _f64(x.q), _f64(x.k))
    tot = np.exp(s - lse.T[:, :, None]).sum(-1)
    assert np.max(np.abs(tot - 1)) < TOL
    # o is the probability-weighted sum of V
    p = np.exp(s - lse.T[:, :, None])
    assert np.max(np.abs(np.einsum("hij,jhd->ihd", p, _f64(x.v)) - o)) < 1e-10
    xs = W.smallseq_cross(seed=9, B=40, H=2, D=16)
    _, w = oracle.smallseq(xs.q, xs.k, xs.v, xs.cu_kv, xs.max_s, xs.scale)
    assert np.max(np.abs(w.sum(-1) - 1)) < TOL


# ---------------------------------------------------------------- invariants

def test_varlen_equals_per_sequence_and_empty_sequences():
    lens_q, lens_k = [3, 0, 6, 2], [5, 4, 0, 2]
    Hq, Hkv, D = 4, 2, 8
    gq = torch.Generator().manual_seed(1)
    q = torch.randn(sum(lens_q), Hq, D, generator=gq)
    k = torch.randn(sum(lens_k), Hkv, D, generator=gq)
    v = torch.randn(sum(lens_k), Hkv, D, generator=gq)
    cu_q = torch.tensor([0, 3, 3, 9, 11], dtype=torch.int32)
    cu_k = torch.tensor([0, 5, 9, 9, 11], dtype=torch.int32)
    for causal in (False, True):
        o, lse, _ = oracle.prefill(q, k, v, cu_q, cu_k, Hq, Hkv, 0.3, causal)
        for b in range(4):
            sq, sk = slice(int(cu_q[b]), int(cu_q[b + 1])), slice(int(cu_k[b]), int(cu_k[b + 1]))
            one = torch.tensor([0, lens_q[b]], dtype=torch.int32)
            onek = torch.tensor([0, lens_k[b]], dtype=torch.int32)
            ob, lb, _ = oracle.prefill(q[sq], k[sk], v[sk], one, onek, Hq, Hkv, 0.3, causal)
            assert np.array_equal(o[sq], ob) and np.array_equal(lse[sq], lb)
        # the sequence with no keys gives zeros and lse = -inf
        assert np.all(o[cu_q[2]:cu_q[3]] == 0) and np.all(np.isneginf(lse[cu_q[2]:cu_q[3]]))
    # causal with Lq < Lk is bottom-right aligned: the last query row sees every key
    o, _, _ = oracle.prefill(q, k, v, cu_q, cu_k, Hq, Hkv, 0.3, True)
    on, _, _ = oracle.prefill(q, k, v, cu_q, cu_k, Hq, Hkv, 0.3, False)
    assert np.array_equal(o[2], on[2])


def test_gqa_equals_mha_with_repeated_kv():
    x = W.varlen_prefill(seed=8, lengths=[20, 7], Hq=8, Hkv=2, D=8, dtype=torch.float32)
    o, lse, _ = oracle.prefill(x.q, x.k, x.v, x.cu_q, x.cu_k, 8, 2, 0.4, True)
    k4, v4 = x.k.repeat_interleave(4, 1), x.v.repeat_interleave(4, 1)
    om, lm, _ = oracle.prefill(x.q, k4, v4, x.cu_q, x.cu_k, 8, 8, 0.4, True)
    assert np.array_equal(o, om) and np.array_equal(lse, lm)
    # a transposed head map (h % Hkv instead of h // G) would differ
    kt, vt = x.k.repeat(1, 4, 1), x.v.repeat(1, 4, 1)
    ot, _, _ = oracle.prefill(x.q, kt, vt, x.cu_q, x.cu_k, 8, 8, 0.4, True)
    assert not np.allclose(o, ot)


def test_causal_row_equals_prefix_attention():
    x = W.varlen_prefill(seed=10, lengths=[24], Hq=2, Hkv=1, D=8, dtype=torch.float32)
    o, lse, _ = oracle.prefill(x.q, x.k, x.v, x.cu_q, x.cu_k, 2, 1, 0.6, True)
    for i in (0, 5, 23):
        cu_q = torch.tensor([0, 1], dtype=torch.int32)
        cu_k = torch.tensor([0, i + 1], dtype=torch.int32)
        oi, li, _ = oracle.prefill(x.q[i:i + 1], x.k[:i + 1], x.v[:i + 1], cu_q, cu_k, 2, 1, 0.6, False)
        assert np.max(np.abs(oi[0] - o[i])) < TOL and np.max(np.abs(li[0] - lse[i])) < TOL


def _small_paged(seed=13, hot=False):
    return W.paged_decode(seed=seed, B=4, Hq=4, Hkv=2, D=16, page=16, pool=200, lengths=[1, 100, 700, 33],
                          lmax=1024, hot=hot)


def test_paged_block_table_permutation_invariance():
    x = _small_paged()
    o, lse, _ = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale)
    perm = torch.randperm(x.pool, generator=torch.Generator().manual_seed(99))
    inv = torch.empty_like(perm)
    inv[perm] = torch.arange(x.pool)
    kc2, vc2 = x.k_cache[perm].contiguous(), x.v_cache[perm].contiguous()   # page p moves to inv[p]
    bt2 = x.block_table.clone()
    m = bt2 >= 0
    bt2[m] = inv[bt2[m].long()].to(torch.int32)
    o2, lse2, _ = oracle.decode(x.q, kc2, vc2, bt2, x.seq_lens, x.scale)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # a table that is not remapped reads other pages and changes the result
    o3, _, _ = oracle.decode(x.q, kc2, vc2, x.block_table, x.seq_lens, x.scale)
    assert not np.allclose(o[1:], o3[1:])


def test_paged_equals_contiguous():
    x = _small_paged()
    lens = x.lens.tolist()
    kk, vv = [], []
    for b, L in enumerate(lens):
        for j in range(L):
            p = int(x.block_table[b, j // 16])
            kk.append(x.k_cache[p, :, j % 16])
            vv.append(x.v_cache[p, :, j % 16])
    k, v = torch.stack(kk), torch.stack(vv)
    cu_k = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    cu_q = torch.arange(5, dtype=torch.int32)
    o, lse, _ = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale)
    op, lp, _ = oracle.prefill(x.q, k, v, cu_q, cu_k, 4, 2, x.scale, False)
    assert np.max(np.abs(o - op)) < TOL and np.max(np.abs(lse - lp)) < TOL


@pytest.mark.parametrize("S", [1, 2, 7, 32, 64])
def test_split_merge_equals_unsplit(S):
    x = _small_paged()
    o, lse, _ = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale)
    os_, ls_, _ = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, mode="split",
                                tile=128, splits=S)
    assert np.max(np.abs(o - os_)) < TOL and np.max(np.abs(lse - ls_)) < TOL


def test_skip_threshold_zero_is_dense():
    x = _small_paged(hot=True)
    o, lse, _ = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale)
    o0, l0, m0 = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, mode="skip", thr=0.0)
    assert np.max(np.abs(o - o0)) < TOL and np.max(np.abs(lse - l0)) < TOL
    assert set(np.unique(m0)) <= {0, 2}
    xp = W.tiny_dense(seed=1000)
    for causal in (False, True):
        od, ld, _ = oracle.prefill(xp.q, xp.k, xp.v, xp.cu_q, xp.cu_k, 4, 2, xp.scale, causal)
        os_, ls_, ms = oracle.prefill(xp.q, xp.k, xp.v, xp.cu_q, xp.cu_k, 4, 2, xp.scale, causal, mode="skip",
                                      thr=0.0)
        assert np.max(np.abs(od - os_)) < TOL and np.max(np.abs(ld - ls_)) < TOL
        assert set(np.unique(ms)) <= {0, 2}


def _decode_scores(x, b, h):
    L = int(x.lens[b])
    g = h // (x.Hq // x.Hkv)
    q = _f64(x.q[b, h])
    ks = np.stack([_f64(x.k_cache[int(x.block_table[b, j // x.page]), g, j % x.page]) for j in range(L)])
    vs = np.stack([_f64(x.v_cache[int(x.block_table[b, j // x.page]), g, j % x.page]) for j in range(L)])
    return x.scale * ks @ q, vs


def test_skip_prefix_max_lemma_nesting_and_error_bound():
    x = _small_paged(hot=True)
    maps = {}
    outs = {}
    for thr in (0.01, 0.1, 0.5):
        o, lse, m = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, mode="skip",
                                  thr=thr)
        maps[thr], outs[thr] = m, o
    od, _, _ = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale)
    nskip = 0
    for b in range(x.B):
        L = int(x.lens[b])
        nt = (L + 31) // 32
        for h in range(x.Hq):
            s, vs = _decode_scores(x, b, h)
            tmax = np.array([s[32 * t:32 * t + 32].max() for t in range(nt)])
            for thr, m in maps.items():
                # decisions follow the prefix max of all earlier tiles, skipped ones included
                pref = np.concatenate([[-np.inf], np.maximum.accumulate(tmax)[:-1]])
                want = (pref > -np.inf) & (np.exp(tmax - pref) < thr)
                assert np.array_equal(m[b, h, :nt] == 1, want)
                assert np.all(m[b, h, nt:] == 2)
                # the tile holding the global max is never skipped
                assert m[b, h, int(np.argmax(tmax))] == 0
                # error bound against dense attention
                M = s.max()
                skipped = np.repeat(m[b, h, :nt] == 1, 32)[:L]
                A = np.exp(s[~skipped] - M).sum()
                Bd = np.exp(s[skipped] - M).sum()
                assert Bd < thr * max(1, skipped.sum())
                bound = Bd / (A + Bd) * (vs.max(0) - vs.min(0))
                assert np.all(np.abs(outs[thr][b, h] - od[b, h]) <= bound + 1e-12)
                nskip += int(skipped.any())
    # skip sets are nested as the threshold grows
    assert np.all((maps[0.01] == 1) <= (maps[0.1] == 1)) and np.all((maps[0.1] == 1) <= (maps[0.5] == 1))
    assert nskip > 0


def test_smallseq_invariants():
    xs = W.smallseq_cross(seed=17, B=64, H=4, D=32)
    o, w = oracle.smallseq(xs.q, xs.k, xs.v, xs.cu_kv, 16, xs.scale)
    cu = xs.cu_kv.tolist()
    v = _f64(xs.v)
    for b in range(64):
        s = cu[b + 1] - cu[b]
        assert np.all(w[b, :, 0, s:] == 0)
        # o = W . V
        assert np.max(np.abs(np.einsum("hj,jhd->hd", w[b, :, 0, :s], v[cu[b]:cu[b + 1]]) - o[b])) < 1e-12
    # equals dense prefill with one query per sequence
    cu_q = torch.arange(65, dtype=torch.int32)
    op, _, _ = oracle.prefill(xs.q, xs.k, xs.v, cu_q, xs.cu_kv, 4, 4, xs.scale, False)
    assert np.max(np.abs(o - op)) < TOL
    # a zero-length sequence gives zero output and zero weights
    cu0 = xs.cu_kv.clone()
    cu0[1] = cu0[0]
    o0, w0 = oracle.smallseq(xs.q[:1], xs.k, xs.v, cu0[:2], 16, xs.scale)
    assert np.all(o0 == 0) and np.all(w0 == 0)


def test_hot_key_workload_makes_most_tiles_skippable():
    x = W.paged_decode(seed=5, B=2, Hq=8, Hkv=2, D=128, page=16, pool=1200, lengths=[4000, 6000], lmax=8192,
                       hot=True)
    _, _, m = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, mode="skip", thr=0.1)
    visited = m != 2
    frac = (m == 1).sum() / visited.sum()
    assert frac > 0.5, frac


def test_hot_key_prefill_workload():
    # same seed: V and the unperturbed keys equal the plain workload's; the sink run is always hot; and
    # the skip-softmax definition then skips most (row, tile) pairs at threshold 0.1 (parity unpinned
    # beyond these properties: the generator is a reading of the pages)
    lens = [1500, 2100]
    x = W.varlen_prefill_hot(seed=9, lengths=lens, Hq=8, Hkv=2, D=128)
    y = W.varlen_prefill(seed=9, lengths=lens, Hq=8, Hkv=2, D=128)
    assert torch.equal(x.v, y.v)
    assert all(t[0] == 0 for t in x.hot_tiles)
    cu = y.cu_q.tolist()
    hot = torch.zeros(cu[-1], dtype=torch.bool)
    for b, tiles in enumerate(x.hot_tiles):
        for t in tiles:
            hot[cu[b] + 32 * t: cu[b] + 32 * (t + 1)] = True
    assert torch.equal(x.k[~hot], y.k[~hot]) and not torch.equal(x.k[hot], y.k[hot])
    rows = [(t, h) for t in range(0, cu[-1], 7) for h in range(8)]
    _, _, m = oracle.prefill(x.q, x.k, x.v, x.cu_q, x.cu_k, 8, 2, x.scale, True, mode="skip", thr=0.1,
                             rows=rows, stride=(max(lens) + 31) // 32)
    visited = m != 2
    assert (m == 1).sum() / visited.sum() > 0.5


# ---------------------------------------------------------------- backward (gradients of the dense definition)

@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    # library special case: float64 SDPA with the KV heads repeated, per sequence; the gradients of the
    # repeated K/V are summed over each KV head's group
    lens, Hq, Hkv, D = [5, 17, 33], 4, 2, 16
    G = Hq // Hkv
    x = W.varlen_prefill(seed=71, lengths=lens, Hq=Hq, Hkv=Hkv, D=D, dtype=torch.float32)
    dout = W.varlen_prefill(seed=72, lengths=lens, Hq=Hq, Hkv=Hkv, D=D, dtype=torch.float32).q
    scale = 0.3
    dq, dk, dv = oracle.prefill_backward(x.q, x.k, x.v, dout, x.cu_q, x.cu_k, Hq, Hkv, scale, causal)
    cu = x.cu_q.tolist()
    for b, L in enumerate(lens):
        sl = slice(cu[b], cu[b + 1])
        q = x.q[sl].double().permute(1, 0, 2).clone().requires_grad_(True)
        k = x.k[sl].double().permute(1, 0, 2).clone().requires_grad_(True)
        v = x.v[sl].double().permute(1, 0, 2).clone().requires_grad_(True)
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None], k.repeat_interleave(G, 0)[None], v.repeat_interleave(G, 0)[None], is_causal=causal,
            scale=scale)[0]
        (o * dout[sl].double().permute(1, 0, 2)).sum().backward()
        assert np.max(np.abs(dq[sl] - q.grad.permute(1, 0, 2).numpy())) < 1e-10
        assert np.max(np.abs(dk[sl] - k.grad.permute(1, 0, 2).numpy())) < 1e-10
        assert np.max(np.abs(dv[sl] - v.grad.permute(1, 0, 2).numpy())) < 1e-10


@pytest.mark.parametrize("causal", [True, False])
def test_backward_with_stored_output_matches_autograd(causal):
    # with a stored output o' the row dot dO.o' replaces sum_j p_j dP_j; that equals the gradient of
    # sum(dO * O) - sum_i delta_i * LSE_i with the constant delta_i = dO_i.(o'_i - O_i), since
    # d LSE_i / d s_ij = p_ij.  Autograd of float64 torch ops (masked logsumexp and softmax) pins it.
    lens, Hq, Hkv, D = [5, 17, 33], 4, 2, 16
    G = Hq // Hkv
    x = W.varlen_prefill(seed=76, lengths=lens, Hq=Hq, Hkv=Hkv, D=D, dtype=torch.float32)
    dout = W.varlen_prefill(seed=77, lengths=lens, Hq=Hq, Hkv=Hkv, D=D, dtype=torch.float32).q
    scale = 0.3
    o_exact, _, _ = oracle.prefill(x.q, x.k, x.v, x.cu_q, x.cu_k, Hq, Hkv, scale, causal)
    rng = np.random.default_rng(78)
    o_st = (o_exact + 0.05 * rng.standard_normal(o_exact.shape)).astype(np.float32)
    dq, dk, dv = oracle.prefill_backward(x.q, x.k, x.v, dout, x.cu_q, x.cu_k, Hq, Hkv, scale, causal,
                                         o=torch.from_numpy(o_st))
    cu = x.cu_q.tolist()
    for b, L in enumerate(lens):
        sl = slice(cu[b], cu[b + 1])
        q = x.q[sl].double().permute(1, 0, 2).clone().requires_grad_(True)
        k = x.k[sl].double().permute(1, 0, 2).clone().requires_grad_(True)
        v = x.v[sl].double().permute(1, 0, 2).clone().requires_grad_(True)
        s = scale * q @ k.repeat_interleave(G, 0).transpose(1, 2)
        if causal:
            s = s.masked_fill(torch.ones(L, L, dtype=torch.bool).triu(1), -math.inf)
        lse = torch.logsumexp(s, dim=-1)
        o = torch.softmax(s, dim=-1) @ v.repeat_interleave(G, 0)
        g = dout[sl].double().permute(1, 0, 2)
        delta = (g * (torch.from_numpy(o_st[sl]).double().permute(1, 0, 2) - o.detach())).sum(-1)
        ((o * g).sum() - (delta * lse).sum()).backward()
        assert np.max(np.abs(dq[sl] - q.grad.permute(1, 0, 2).numpy())) < 1e-10
        assert np.max(np.abs(dk[sl] - k.grad.permute(1, 0, 2).numpy())) < 1e-10
        assert np.max(np.abs(dv[sl] - v.grad.permute(1, 0, 2).numpy())) < 1e-10
    # the stored output shifts dq and dk, never dv
    dq0, dk0, dv0 = oracle.prefill_backward(x.q, x.k, x.v, dout, x.cu_q, x.cu_k, Hq, Hkv, scale, causal)
    assert np.array_equal(dv, dv0) and np.max(np.abs(dq - dq0)) > 1e-3


def test_backward_matches_finite_differences():
    # central differences of L = sum(O * dO) with the forward oracle, on inputs that are multiples of
    # 2^-10 so that x +- 2^-10 is exact in fp32; the error of the difference is O(eps^2)
    rng = np.random.default_rng(3)
    L, Hq, Hkv, D = 9, 2, 1, 8
    q = (np.round(rng.standard_normal((L, Hq, D)) * 1024) / 1024).astype(np.float32)
    k = (np.round(rng.standard_normal((L, Hkv, D)) * 1024) / 1024).astype(np.float32)
    v = (np.round(rng.standard_normal((L, Hkv, D)) * 1024) / 1024).astype(np.float32)
    g = rng.standard_normal((L, Hq, D)).astype(np.float32)
    cu = np.array([0, L], dtype=np.int32)
    scale = 0.5

    def loss(q_, k_, v_):
        o, _, _ = oracle.prefill(q_, k_, v_, cu, cu, Hq, Hkv, scale, True)
        return float(np.sum(o * g.astype(np.float64)))

    dq, dk, dv = oracle.prefill_backward(q, k, v, g, cu, cu, Hq, Hkv, scale, True)
    eps = 2.0 ** -10
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for idx in [(0, 0, 0), (3, 0, 5), (8, arr.shape[1] - 1, 7), (5, 0, 2)]:
            plus, minus = arr.copy(), arr.copy()
            plus[idx] += eps
            minus[idx] -= eps
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = plus, minus
            fd = (loss(args_p["q"], args_p["k"], args_p["v"]) - loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * eps)
            assert abs(fd - grad[idx]) < 1e-5, (name, idx, fd, grad[idx])


def test_backward_rows_without_keys_and_unseen_keys():
    # causal with Lq > Lk: the first Lq - Lk rows see no key and get dq = 0; with Lk > Lq every key is
    # seen by some row, and a row's gradient does not depend on keys past its diagonal
    x = W.varlen_prefill(seed=74, lengths=[12], Hq=2, Hkv=1, D=8, dtype=torch.float32)
    dout = W.varlen_prefill(seed=75, lengths=[12], Hq=2, Hkv=1, D=8, dtype=torch.float32).q
    cq = torch.tensor([0, 12], dtype=torch.int32)
    ck = torch.tensor([0, 7], dtype=torch.int32)
    dq, dk, dv = oracle.prefill_backward(x.q, x.k[:7], x.v[:7], dout, cq, ck, 2, 1, 0.4, True)
    assert np.all(dq[:5] == 0) and np.any(dq[5:] != 0)
    # the last key is seen only by the last row: its dv is that row's p times dO, summed over the heads
    o, lse, _ = oracle.prefill(x.q, x.k[:7], x.v[:7], cq, ck, 2, 1, 0.4, True, rows=[(11, 0), (11, 1)])
    s = np.array([0.4 * float(x.q[11, h].double() @ x.k[6, 0].double()) for h in range(2)])
    p_last = np.exp(s - lse)
    expect = sum(p_last[h] * dout[11, h].double().numpy() for h in range(2))
    assert np.max(np.abs(dv[6, 0] - expect)) < 1e-12


def _smallseq_fixture(lens, H=3, D=16, seed=81):
    """fp32 small-seq inputs with the given key counts, the exact softmax weights (float64 torch,
    stored as fp32, zero padded) and an output gradient."""
    g = torch.Generator().manual_seed(seed)
    B, T, ms = len(lens), sum(lens), max(lens)
    q = torch.randn(B, H, D, generator=g)
    k = torch.randn(T, H, D, generator=g)
    v = torch.randn(T, H, D, generator=g)
    do = torch.randn(B, H, D, generator=g)
    cu = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    scale = D ** -0.5
    w = torch.zeros(B, H, 1, ms, dtype=torch.float64)
    for b, n in enumerate(lens):
        if n:
            s = scale * torch.einsum("hd,jhd->hj", q[b].double(), k[cu[b]:cu[b + 1]].double())
            w[b, :, 0, :n] = torch.softmax(s, dim=-1)
    return q, k, v, do, cu, ms, scale, w.float()


def test_smallseq_backward_matches_torch_autograd():
    # the stored weights are the exact softmax rounded to fp32; float64 autograd of o = softmax(scale q k^T) v
    # differs from the stored-weights backward only by that rounding (relative ~6e-8)
    lens = [1, 3, 16, 0, 7, 2]
    q, k, v, do, cu, ms, scale, w = _smallseq_fixture(lens)
    dq, dk, dv = oracle.smallseq_backward(q, k, v, w, do, cu, ms, scale)
    for b, n in enumerate(lens):
        qb = q[b].double().clone().requires_grad_(True)
        kb = k[cu[b]:cu[b + 1]].double().clone().requires_grad_(True)
        vb = v[cu[b]:cu[b + 1]].double().clone().requires_grad_(True)
        if n == 0:
            assert np.all(dq[b] == 0)
            continue
        p = torch.softmax(scale * torch.einsum("hd,jhd->hj", qb, kb), dim=-1)
        o = torch.einsum("hj,jhd->hd", p, vb)
        (o * do[b].double()).sum().backward()
        assert np.max(np.abs(dq[b] - qb.grad.numpy())) < 1e-5
        assert np.max(np.abs(dk[cu[b]:cu[b + 1]] - kb.grad.numpy())) < 1e-5
        assert np.max(np.abs(dv[cu[b]:cu[b + 1]] - vb.grad.numpy())) < 1e-5


def test_smallseq_backward_padding_and_closed_forms():
    lens = [1, 5, 0, 4]
    q, k, v, do, cu, ms, scale, w = _smallseq_fixture(lens, seed=82)
    dq, dk, dv = oracle.smallseq_backward(q, k, v, w, do, cu, ms, scale)
    # weights past a sequence's key count are padding and never read
    w2 = w.clone()
    for b, n in enumerate(lens):
        w2[b, :, 0, n:] = 7.0
    assert all(np.array_equal(x, y) for x, y in zip((dq, dk, dv), oracle.smallseq_backward(q, k, v, w2, do, cu, ms,
                                                                                           scale)))
    # one key: w = 1, so dv = dO, and the softmax backward leaves ds = 0 (dq = dk = 0)
    assert np.max(np.abs(dv[0] - do[0].double().numpy())) < 1e-12
    assert np.all(dq[0] == 0) and np.all(dk[0] == 0)
    # a sequence with no key: dq = 0
    assert np.all(dq[2] == 0)
    # the weights enter dv linearly: doubling w doubles dv
    _, _, dv2 = oracle.smallseq_backward(q, k, v, w * 2, do, cu, ms, scale)
    assert np.max(np.abs(dv2 - 2 * dv)) < 1e-12


def _paged_from_contiguous(k, v, lens, Hkv, D, page=16, seed=91):
    """A bf16 paged cache [pages, Hkv, page, D] holding the contiguous k, v [sum(lens), Hkv, D] through a
    permuted block table; unused slots NaN."""
    g = torch.Generator().manual_seed(seed)
    npg = [(L + page - 1) // page for L in lens]
    pool = sum(npg) + 3
    perm = torch.randperm(pool, generator=g)
    maxp = max(npg)
    bt = torch.full((len(lens), maxp), -1, dtype=torch.int32)
    kc = torch.full((pool, Hkv, page, D), float("nan"), dtype=torch.bfloat16)
    vc = kc.clone()
    off, tok = 0, 0
    for b, L in enumerate(lens):
        for p in range(npg[b]):
            pg = int(perm[off + p])
            bt[b, p] = pg
            n = min(page, L - p * page)
            kc[pg, :, :n] = k[tok + p * page:tok + p * page + n].transpose(0, 1)
            vc[pg, :, :n] = v[tok + p * page:tok + p * page + n].transpose(0, 1)
        off += npg[b]
        tok += L
    return kc, vc, bt


def test_decode_multi_equals_contiguous_causal_prefill():
    # the paged multi-token rows equal the (separately pinned) contiguous varlen prefill with bottom-right
    # causal alignment, Lq != Lk, over the same keys
    lens, qlens, Hq, Hkv, D = [20, 33, 5, 16], [3, 1, 5, 16], 4, 2, 16
    g = torch.Generator().manual_seed(90)
    k = torch.randn(sum(lens), Hkv, D, generator=g).bfloat16()
    v = torch.randn(sum(lens), Hkv, D, generator=g).bfloat16()
    q = torch.randn(sum(qlens), Hq, D, generator=g).bfloat16()
    kc, vc, bt = _paged_from_contiguous(k, v, lens, Hkv, D)
    cu_q = torch.tensor([0] + list(np.cumsum(qlens)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(lens)), dtype=torch.int32)
    sl = torch.tensor(lens, dtype=torch.int32)
    om, lm = oracle.decode_multi(q, cu_q, kc, vc, bt, sl, 0.25)
    op, lp, _ = oracle.prefill(q, k, v, cu_q, cu_k, Hq, Hkv, 0.25, True)
    assert np.max(np.abs(om - op)) < 1e-12
    assert np.max(np.abs(lm - lp)) < 1e-12


def test_decode_multi_one_token_equals_decode():
    # with one new token per sequence the rows are the (separately pinned) one-token paged decode
    x = W.paged_decode(seed=93, B=5, Hq=8, Hkv=2, D=32, lmin=1, lmax=70, pool=64)
    cu_q = torch.arange(x.B + 1, dtype=torch.int32)
    om, lm = oracle.decode_multi(x.q, cu_q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale)
    od, ld, _ = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale)
    assert np.max(np.abs(om - od)) < 1e-12
    assert np.max(np.abs(lm - ld)) < 1e-12


# ---------------------------------------------------------------- NVFP4 fake quantization of P and V

E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]  # the format's table of magnitudes


def test_e2m1_grid_ties_and_saturation():
    assert list(oracle.fp_round("e2m1", E2M1)) == E2M1
    # midpoints go to the code with an even mantissa bit: 0, 1, 2 and 4 are even, 0.5, 1.5, 3 and 6 odd
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    assert list(oracle.fp_round("e2m1", mids)) == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    assert list(oracle.fp_round("e2m1", [0.26, 0.74, 2.51, 4.99, 5.01])) == [0.5, 0.5, 3.0, 4.0, 6.0]
    assert list(oracle.fp_round("e2m1", [6.0, 6.9, 7.0, 1e3, 3e38])) == [6.0] * 5


def test_e4m3_matches_torch_float8_in_range():
    # in [0, 448] the rounding is torch's float32 -> float8_e4m3fn conversion (round to nearest even)
    g = torch.Generator().manual_seed(5)
    y = torch.cat([torch.rand(20000, generator=g) * 448, torch.rand(20000, generator=g) * 2.0 ** -5,
                   torch.rand(5000, generator=g) * 2.0 ** -8, torch.tensor([0.0, 2.0 ** -10, 3 * 2.0 ** -10,
                                                                             2.0 ** -9, 2.0 ** -6, 448.0, 440.0])])
    ref = y.to(torch.float8_e4m3fn).float().numpy()
    assert np.array_equal(oracle.fp_round("e4m3", y.numpy()), ref)


def test_e4m3_grid_and_saturation():
    r = oracle.fp_round("e4m3", [448.0, 460.0, 464.0, 1e6, 2.0 ** -9, 2.0 ** -10, 1.5 * 2.0 ** -10, 248.0])
    # 448 is the largest finite value; the saturating rounding keeps everything above it at 448; the
    # smallest subnormal is 2^-9, its half-way point goes to 0 (even), 248 lies between 240 (odd mantissa)
    # and 256 (even) and goes to 256
    assert list(r) == [448.0, 448.0, 448.0, 448.0, 2.0 ** -9, 0.0, 2.0 ** -9, 256.0]
    sweep = np.concatenate([np.linspace(0, 460, 400001, dtype=np.float32),
                            np.linspace(0, 2.0 ** -5, 100001, dtype=np.float32)])
    assert len(np.unique(oracle.fp_round("e4m3", sweep))) == 127  # 0 and the 126 positive finite codes


def test_nvfp4_identity_on_the_grid_and_sign():
    # amax = 6 * 448 gives enc = 1/6 and dec = 1: a block with max 6 gets scale code 1, and values on the
    # E2M1 grid come back unchanged, with their signs
    x = np.array([6.0, -3.0, 1.5, 0.5, 0.0, -6.0, 4.0, 2.0, 1.0, -0.5, 3.0, -1.5, 0.0, 4.0, -2.0, 1.0], np.float32)
    assert np.array_equal(oracle.nvfp4_qdq(x, 2688.0), x)


def test_nvfp4_hand_worked_block():
    # amax 1: a block with max 1 gets scale code e4m3(448) = 448 and block scale 448 / 2688 = 1/6, so the
    # values are 6x rounded to E2M1, divided by 6: 0.3 -> 1.8 -> 2, -0.05 -> -0.3 -> -0.5, 0.7 -> 4.2 -> 4,
    # 0.9 -> 5.4 -> 6, 0.04 -> 0.24 -> 0
    x = np.array([1.0, 0.3, -0.05, 0.7, 0.9, 0.04] + [0.0] * 10, np.float32)
    want = np.array([1.0, 2 / 6, -0.5 / 6, 4 / 6, 1.0, 0.0] + [0.0] * 10)
    assert np.max(np.abs(oracle.nvfp4_qdq(x, 1.0) - want)) < 1e-6


def test_nvfp4_saturates_at_amax_and_zero_block():
    # a block whose max exceeds amax gets the largest scale code, and its largest values come back as amax
    x = np.array([5.0, -2.0, 0.5] + [0.0] * 13, np.float32)
    out = oracle.nvfp4_qdq(x, 1.0)
    assert abs(out[0] - 1.0) < 1e-6 and abs(out[1] + 1.0) < 1e-6
    assert np.array_equal(oracle.nvfp4_qdq(np.zeros(16, np.float32), 1.0), np.zeros(16))


def test_nvfp4_blocks_are_16_along_the_last_dim_and_scale_by_powers_of_two():
    g = np.random.default_rng(7)
    x = g.standard_normal((3, 40)).astype(np.float32)
    out = oracle.nvfp4_qdq(x, 4.0)
    # blocks [0,16), [16,32), [32,40) of each row are independent
    for r in range(3):
        for b0, b1 in ((0, 16), (16, 32), (32, 40)):
            assert np.array_equal(out[r, b0:b1], oracle.nvfp4_qdq(x[r, b0:b1], 4.0))
    # every value is sign * (E2M1 magnitude) * (its block's scale), and the block scale is
    # e4m3(block max * 448 / amax) * amax / 2688: the error is at most half the widest step, 1 * scale
    for r in range(3):
        blk = x[r, :16]
        s = oracle.fp_round("e4m3", [np.float32(np.abs(blk).max()) * np.float32(448 / 4.0)])[0] * (4.0 / 2688)
        assert np.all(np.abs(blk - out[r, :16]) <= s * (1 + 1e-6))
        codes = np.abs(out[r, :16]) / s
        assert np.all(np.min(np.abs(codes[:, None] - np.array(E2M1)[None]), axis=1) < 1e-5)
    # a power-of-two factor on both x and amax commutes with the quantizer
    assert np.array_equal(oracle.nvfp4_qdq(x * 8, 32.0), out * 8)
    assert np.array_equal(oracle.nvfp4_qdq(x / 4, 1.0), out / 4)


def _exact_decode(seed, lengths, Hq=4, Hkv=2, D=32, q_nnz=8):
    return W.paged_decode_exact(seed=seed, B=len(lengths), Hq=Hq, Hkv=Hkv, D=D, lengths=lengths,
                                lmax=max(lengths), pool=sum((L + 15) // 16 for L in lengths) + 5, q_nnz=q_nnz)


def test_decode_qdq_off_is_the_dense_decode():
    x = W.paged_decode(seed=95, B=4, Hq=8, Hkv=2, D=32, lmin=1, lmax=150, pool=64)
    o, lse, m = oracle.decode_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale)
    od, ld, _ = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale)
    assert np.max(np.abs(o - od)) < 1e-12 and np.max(np.abs(lse - ld)) < 1e-12


def test_decode_qdq_v_only_is_decode_of_the_quantized_cache():
    # V fake-quantized per key in blocks of 16 along D and rounded back to bf16, then the plain decode
    x = W.paged_decode(seed=96, B=3, Hq=4, Hkv=2, D=48, lmin=1, lmax=90, pool=40)
    vq = torch.from_numpy(oracle.nvfp4_qdq(x.v_cache.float().numpy(), 1.5)).to(torch.bfloat16)
    o, lse, _ = oracle.decode_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, x.scale, v_amax=1.5)
    od, ld, _ = oracle.decode(x.q, x.k_cache, vq, x.block_table, x.seq_lens, x.scale)
    assert np.max(np.abs(o - od)) < 1e-12 and np.max(np.abs(lse - ld)) < 1e-12


def test_decode_qdq_p_brute_force_sequential_tiles():
    # brute force of the sequential pass on tiny rows: per 32-key tile, P = exp(s - m) with m the running
    # max including the tile, quantized in 16-key blocks, accumulated with the rescale exp(m_old - m);
    # the denominator sums the unquantized P
    lens = [1, 15, 16, 17, 32, 33, 70, 100]
    x = W.paged_decode(seed=97, B=len(lens), Hq=4, Hkv=1, D=16, lengths=lens, lmax=100, pool=40)
    scale = 0.9
    o, lse, _ = oracle.decode_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, scale, p_amax=1.0)
    q, kc, vc, bt = _f64(x.q), _f64(x.k_cache), _f64(x.v_cache), x.block_table.numpy()
    for b, L in enumerate(lens):
        keys = [bt[b, j // 16] for j in range(L)]
        K = np.stack([kc[keys[j], 0, j % 16] for j in range(L)])
        V = np.stack([vc[keys[j], 0, j % 16] for j in range(L)])
        for h in range(4):
            s = scale * (K @ q[b, h])
            m, l, acc = -np.inf, 0.0, np.zeros(16)
            for j0 in range(0, L, 32):
                st = s[j0:j0 + 32]
                mn = max(m, st.max())
                p = np.exp(st - mn)
                pq = np.concatenate([oracle.nvfp4_qdq(p[i:i + 16].astype(np.float32), 1.0).astype(np.float64)
                                     for i in range(0, len(p), 16)])
                a = 0.0 if m == -np.inf else math.exp(m - mn)
                l = l * a + p.sum()
                acc = acc * a + pq @ V[j0:j0 + 32]
                m = mn
            assert np.max(np.abs(o[b, h] - acc / l)) < 1e-12
            assert abs(lse[b, h] - (m + math.log(l))) < 1e-12


def test_decode_qdq_p_top_block_on_the_sixths_grid():
    # one tile, one key block: the block holding the tile max has P max 1, scale code 448 and block scale
    # 1/6, so the quantized P takes only values of the E2M1 grid / 6; with V = e_d the output row times l
    # shows those values directly
    lens = [16]
    x = _exact_decode(98, lens, Hq=1, Hkv=1, D=16)
    vc = torch.zeros_like(x.v_cache)
    pg = int(x.block_table[0, 0])
    vc[pg, 0, :16] = torch.eye(16, dtype=torch.bfloat16)
    o, lse, _ = oracle.decode_qdq(x.q, x.k_cache, vc, x.block_table, x.seq_lens, math.log(2), p_amax=1.0)
    # o = sum_j pq_j e_j / l with l = sum_j exp(s_j - max s) = exp(lse - max s)
    l = math.exp(lse[0, 0] - np.max(math.log(2) * _f64(x.k_cache)[pg, 0, :16] @ _f64(x.q)[0, 0]))
    vals = np.sort(o[0, 0] * l)
    assert abs(vals[-1] - 1.0) < 1e-6
    grid6 = np.array(E2M1) / 6
    assert np.all(np.min(np.abs(vals[:, None] - grid6[None]), axis=1) < 1e-6)


def test_decode_qdq_skip_decisions_unchanged_by_quantization():
    # the decisions depend on the scores alone: the map with P and V quantized equals the unquantized one
    x = _exact_decode(99, [40, 200, 333, 64], Hq=4, Hkv=2, D=32, q_nnz=8)
    _, _, m0 = oracle.decode_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, math.log(2), thr=0.1)
    _, _, m1 = oracle.decode_qdq(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, math.log(2), thr=0.1,
                                 p_amax=1.0, v_amax=1.0)
    assert np.array_equal(m0, m1) and (m0 == 1).any()
    od, _, md = oracle.decode(x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, math.log(2), mode="skip",
                              thr=0.1, stride=m0.shape[-1])
    assert np.array_equal(md, m0)


def test_decode_qdq_replay():
    # replaying the pass's own decisions reproduces it; replaying "keep everything" is the thr = 0 pass
    x = _exact_decode(100, [40, 200, 333], Hq=4, Hkv=2, D=32, q_nnz=8)
    args = (x.q, x.k_cache, x.v_cache, x.block_table, x.seq_lens, math.log(2))
    o1, l1, m1 = oracle.decode_qdq(*args, thr=0.2, p_amax=1.0, v_amax=2.0)
    o2, l2, _ = oracle.decode_qdq(*args, p_amax=1.0, v_amax=2.0, replay=np.where(m1 == 1, 1, 0).reshape(-1, m1.shape[-1]))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3, _ = oracle.decode_qdq(*args, thr=0.0, p_amax=1.0, v_amax=2.0)
    o4, l4, _ = oracle.decode_qdq(*args, thr=0.9, p_amax=1.0, v_amax=2.0, replay=np.zeros_like(m1).reshape(-1, m1.shape[-1]))
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)
