"""Benchmark of the attention hot path on one MI355X.

One step = one pass of every hot-path kernel over its synthetic workload, inputs resident in HBM:
  prefill  varlen causal prefill, bf16: 16 sequences, lengths uniform in [256, 4096], THD, Hq=32, Hkv=8,
           D=128 (the workload the headline metric is quoted on)
  decode   paged one-token decode, split-K: B=64, Hq=32, Hkv=8, D=128, contexts uniform in [1024, 32768],
           16-token pages in a 140,000-page pool, 32 splits of 128-key tiles (+ the merge kernel)
  skip     the same decode shapes with hot keys, one sequential split of 32-key tiles, threshold
           0, 0.01 and 0.1; and at threshold 0 and 0.1 with NVFP4 fake quantization of P and V (amax 1)
  smallseq small-seq cross-attention: 30720 sequences, s_q=1, s_kv in {2,4,6,8,12,16}, H=16, D=128

value = prefill TFLOP/s (algorithmic FLOPs 4 D Hq sum_b L_b (L_b + 1) / 2 over the kernel's event time);
the decode, skip and small-seq figures ride along in the same JSON line.  Kernel times come from HIP
events recorded on the stream the kernels are launched on (torch's current stream).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
FLUSH_BYTES = 512 << 20     # read between timed calls: twice the 256 MB last-level cache


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", default="",
                   help="comma list of tiny,prefill,prefill_skip,decode,skip,smallseq,prefill_bwd,smallseq_bwd,"
                        "decode_multi,prefill_paged (profiling runs)")
    p.add_argument("--launch-log", metavar="PATH", default="",
                   help="write the bench's calls, in launch order, to PATH (JSON; profiling runs)")
    p.add_argument("--calib-copy", action="store_true",
                   help="also run one plain 1 GiB device-to-device copy (scales HBM byte counters)")
    p.add_argument("--summarize-profiles", metavar="DIR", default="",
                   help="no GPU work: turn the rocprofv3 csv output under DIR/prof_trace, DIR/prof_fetch and "
                        "DIR/prof_write into the summaries under profiles/")
    return p.parse_args()


# Every library call the bench makes, in launch order (its name is the call's role in the profiles).
LAUNCH_LOG = []


def _logged(name, fn):
    def call():
        LAUNCH_LOG.append(name)
        return fn()
    return call


def _traffic_from_profiles(kernel: str):
    """HBM bytes per launch measured by rocprofv3 counters, if a summary for this kernel build exists."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
        ent = data.get(kernel)
        if not ent:
            return None
        if _sources_digest(ent["sources"]) != ent.get("sources_sha256"):
            return None  # the kernel changed since the counters were taken
        return float(ent["bytes_per_launch"])
    except Exception:
        return None


def _sources_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def main():
    args = _parse()
    if args.summarize_profiles:
        _summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (every path here runs on a "
              "single MI355X)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import paged_skip_softmax_amd as attn
    from paged_skip_softmax_amd import workloads as W

    only = (set(args.only.split(",")) if args.only
            else {"tiny", "prefill", "prefill_skip", "decode", "skip", "smallseq", "prefill_bwd", "smallseq_bwd",
                  "decode_multi", "prefill_paged"})
    dev = "cuda:0"
    torch.cuda.set_device(0)
    t_gen = time.time()
    work = {}
    if "tiny" in only:
        work["tiny"] = W.tiny_dense(seed=1000 + args.seed, device=dev)
    if "prefill" in only:
        work["prefill"] = W.varlen_prefill(seed=1001 + args.seed, device=dev)
    if "prefill_skip" in only:
        work["prefill_skip"] = W.varlen_prefill_hot(seed=1001 + args.seed, device=dev)
        work["prefill_sink"] = W.varlen_prefill_sink(seed=1001 + args.seed, device=dev)
    if "decode" in only:
        work["decode"] = W.paged_decode(seed=1002 + args.seed, device=dev)
    if "skip" in only:
        work["skip"] = W.paged_decode_hot(seed=1002 + args.seed, device=dev)
    if "smallseq" in only:
        work["smallseq"] = W.smallseq_cross(seed=1004 + args.seed, device=dev)
    torch.cuda.synchronize()
    print(f"# inputs generated in {time.time() - t_gen:.1f} s", file=sys.stderr, flush=True)

    # rows past the hot path (timed after it, outside the step, each call in a loop of its own): the prefill
    # backward, ...; `last` runs after all of them
    nxt = {}
    last = {}
    if "prefill_bwd" in only:
        xb = work.get("prefill") or W.varlen_prefill(seed=1001 + args.seed, device=dev)
        work["prefill_bwd"] = xb
        do_b = W.grad_output(xb, seed=1005 + args.seed, device=dev)
        LAUNCH_LOG.append("setup_prefill_fwd")
        o_b, lse_b, _ = attn.attn_prefill_varlen(xb.q, xb.k, xb.v, xb.cu_q, xb.cu_k, xb.max_q, xb.max_k, causal=True,
                                                 return_lse=True)
        ws_b = torch.empty(attn.attn_prefill_varlen_backward_workspace_size(xb.B, xb.max_q, xb.Hq),
                           dtype=torch.uint8, device=dev)
        g_b = (torch.empty_like(xb.q), torch.empty_like(xb.k), torch.empty_like(xb.v))
        nxt["prefill_bwd"] = lambda: attn.attn_prefill_varlen_backward(
            xb.q, xb.k, xb.v, o_b, do_b, lse_b, xb.cu_q, xb.cu_k, xb.max_q, xb.max_k, causal=True, workspace=ws_b,
            dq=g_b[0], dk=g_b[1], dv=g_b[2])

    if "smallseq_bwd" in only:
        cb = work.get("smallseq") or W.smallseq_cross(seed=1004 + args.seed, device=dev)
        work["smallseq_bwd"] = cb
        do_s = W.grad_output(cb, seed=1006 + args.seed, device=dev)
        LAUNCH_LOG.append("setup_smallseq_fwd")
        _, w_s, _ = attn.attn_smallseq_cross(cb.q, cb.k, cb.v, cb.cu_kv, cb.max_s)
        gs = (torch.empty_like(cb.q), torch.empty_like(cb.k), torch.empty_like(cb.v))
        nxt["smallseq_bwd"] = lambda: attn.attn_smallseq_cross_backward(
            cb.q, cb.k, cb.v, w_s, do_s, cb.cu_kv, cb.max_s, dq=gs[0], dk=gs[1], dv=gs[2])

    if "decode_multi" in only:
        dm = W.paged_decode_multi(seed=1002 + args.seed, device=dev)
        work["decode_multi"] = dm
        ws_m = torch.empty(attn.attn_decode_paged_multi_workspace_size(dm.q.shape[0], dm.max_q, dm.Hq, dm.Hkv, dm.D,
                                                                       32), dtype=torch.uint8, device=dev)
        o_m = torch.empty_like(dm.q)
        nxt["decode_multi"] = lambda: attn.attn_decode_paged_multi(
            dm.q, dm.cu_q, dm.max_q, dm.k_cache, dm.v_cache, dm.block_table, dm.seq_lens, num_splits=32,
            workspace=ws_m, out=o_m)

    if "prefill_paged" in only:
        pp = W.paged_decode_multi(seed=1002 + args.seed, device=dev, qmin=256, qmax=256)
        work["prefill_paged"] = pp
        o_pp = torch.empty_like(pp.q)
        nxt["prefill_paged"] = lambda: attn.attn_decode_paged_multi(
            pp.q, pp.cu_q, pp.max_q, pp.k_cache, pp.v_cache, pp.block_table, pp.seq_lens, out=o_pp)

    calls = {}  # name -> zero-arg launcher
    if "tiny" in only:
        # the tiny fp32 workload, each call in a loop of its own after every other call: short calls changed
        # the clocks the calls after them ran at (measured: the hot-key skip-softmax prefill calls took 7-10 %
        # longer in kernel time with the tiny calls in the step)
        xt = work["tiny"]
        o_t = torch.empty_like(xt.q)
        for causal in (True, False):
            for thr in (0.0, 0.1):
                last[f"tiny_{'causal' if causal else 'noncausal'}_{thr}"] = (
                    lambda causal=causal, thr=thr: attn.attn_prefill_varlen(
                        xt.q, xt.k, xt.v, xt.cu_q, xt.cu_k, xt.max_q, xt.max_k, scale=xt.scale, causal=causal,
                        skip_threshold=thr, out=o_t))
    if "prefill" in only:
        x = work["prefill"]
        o_pf = torch.empty_like(x.q)
        calls["prefill"] = lambda: attn.attn_prefill_varlen(x.q, x.k, x.v, x.cu_q, x.cu_k, x.max_q, x.max_k,
                                                            causal=True, out=o_pf)
    if "prefill_skip" in only:
        xh = work["prefill_skip"]
        o_ph = torch.empty_like(xh.q)
        # the speedup curve of skip-softmax prefill over dense on the same input (hot keys here, a coherent sink
        # below), each call timed in a loop of its own after the step: in the step, the calls' times depended on
        # the calls before them (the clocks the GPU ran at), by more than the differences being measured
        for thr in (0.0, 0.01, 0.1):
            nxt[f"prefill_skip_{thr}"] = (lambda thr=thr: attn.attn_prefill_varlen(
                xh.q, xh.k, xh.v, xh.cu_q, xh.cu_k, xh.max_q, xh.max_k, causal=True, skip_threshold=thr, out=o_ph))
        # the coherent-sink input
        xs = work["prefill_sink"]
        for thr in (0.0, 0.01, 0.1):
            nxt[f"prefill_sink_{thr}"] = (lambda thr=thr: attn.attn_prefill_varlen(
                xs.q, xs.k, xs.v, xs.cu_q, xs.cu_k, xs.max_q, xs.max_k, causal=True, skip_threshold=thr, out=o_ph))
    if "decode" in only:
        d = work["decode"]
        ws = torch.empty(attn.attn_decode_paged_workspace_size(d.B, d.Hq, d.D, 32), dtype=torch.uint8, device=dev)
        o_dc = torch.empty_like(d.q)
        calls["decode"] = lambda: attn.attn_decode_paged(d.q, d.k_cache, d.v_cache, d.block_table, d.seq_lens,
                                                         num_splits=32, workspace=ws, out=o_dc)
    if "skip" in only:
        s = work["skip"]
        o_sk = torch.empty_like(s.q)
        for thr in (0.0, 0.01, 0.1):
            calls[f"skip_{thr}"] = (lambda thr=thr: attn.attn_decode_paged(
                s.q, s.k_cache, s.v_cache, s.block_table, s.seq_lens, num_splits=1, skip_threshold=thr, out=o_sk))
        # NVFP4 fake quantization of P and V (amax 1 for both, as in the usage the pages print)
        for thr in (0.0, 0.1):
            calls[f"qdq_{thr}"] = (lambda thr=thr: attn.attn_decode_paged_qdq(
                s.q, s.k_cache, s.v_cache, s.block_table, s.seq_lens, skip_threshold=thr, p_amax=1.0, v_amax=1.0,
                out=o_sk))
    if "smallseq" in only:
        c = work["smallseq"]
        o_ss = torch.empty_like(c.q)
        w_ss = torch.empty((c.B, c.H, 1, c.max_s), dtype=torch.bfloat16, device=dev)
        calls["smallseq"] = lambda: attn.attn_smallseq_cross(c.q, c.k, c.v, c.cu_kv, c.max_s, out=o_ss)

    calls = {k: _logged(k, f) for k, f in calls.items()}
    nxt.update(last)
    nxt = {k: _logged(k, f) for k, f in nxt.items()}
    names = list(calls)
    stream = torch.cuda.current_stream()
    # Between timed calls (outside each event pair) a 512 MiB buffer is read, which evicts what the
    # previous call left in the L2s (4 MB per XCD) and the 256 MB last-level cache, so every call starts
    # cold.  A read, not a write: written lines would stay dirty in the caches and their write-back would
    # land inside the next timed call (measured: +5 to +14 % on the HBM-bound kernels).
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def flush():
        flush_buf.sum()

    def step(record):
        for nm in names:
            flush()
            if record is None:
                calls[nm]()
            else:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                calls[nm]()
                e1.record(stream)
                record[nm].append((e0, e1))

    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()
    rec = {nm: [] for nm in names}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(rec)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = {nm: float(np.mean([a.elapsed_time(b) for a, b in rec[nm]])) for nm in names}
    ms_min = {nm: float(np.min([a.elapsed_time(b) for a, b in rec[nm]])) for nm in names}
    ms_med = {nm: float(np.median([a.elapsed_time(b) for a, b in rec[nm]])) for nm in names}
    ms_max = {nm: float(np.max([a.elapsed_time(b) for a, b in rec[nm]])) for nm in names}
    ms_per_step = (t1 - t0) * 1e3 / max(1, args.steps)
    for nm, fn in nxt.items():
        for _ in range(args.warmup):
            flush()
            fn()
        torch.cuda.synchronize()
        evs = []
        for _ in range(args.steps):
            flush()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ms[nm] = float(np.mean([a.elapsed_time(b) for a, b in evs]))
        ms_min[nm] = float(np.min([a.elapsed_time(b) for a, b in evs]))
        ms_med[nm] = float(np.median([a.elapsed_time(b) for a, b in evs]))
        ms_max[nm] = float(np.max([a.elapsed_time(b) for a, b in evs]))
    del flush_buf

    def spread(nm):
        return {"ms_min": ms_min[nm], "ms_median": ms_med[nm], "ms_max": ms_max[nm]}

    print(f"# kernel ms (mean over {args.steps} steps): " + ", ".join(f"{k}={v:.4f}" for k, v in ms.items()),
          file=sys.stderr, flush=True)

    if args.calib_copy:
        # a plain device-to-device copy of 1 GiB: 2^20 KiB read and 2^20 KiB written
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    achievable = _achievable(torch, dev)

    out = {}
    rooflines = []
    if "tiny" in only:
        xt = work["tiny"]
        res = {}
        for causal in (True, False):
            fl = _tiny_flops(xt, causal)
            for thr in (0.0, 0.1):
                nm = f"tiny_{'causal' if causal else 'noncausal'}_{thr}"
                res[nm[5:]] = {"ms": ms[nm], **spread(nm), "flop_dense_equiv": fl,
                               "gflops_dense_equiv": fl / (ms[nm] * 1e-3) / 1e9}
        res["note"] = ("fp32, B=2, Hq=4, Hkv=2, D=64, S=128, 32-key skip tiles; latency-bound (a few hundred "
                       "workgroups), reported for completeness")
        out["tiny_fp32"] = res
    if "prefill" in only:
        L = work["prefill"].lens.double()
        flops = 4.0 * 128 * 32 * float((L * (L + 1) / 2).sum())
        tflops = flops / (ms["prefill"] * 1e-3) / 1e12
        out["prefill"] = {"ms": ms["prefill"], **spread("prefill"), "flop": flops, "tflops": tflops,
                          "frac_peak": tflops / PEAK_BF16_TFLOPS}
        if achievable.get("mfma_bf16_loop_TFLOPs"):
            out["prefill"]["frac_of_mfma_loop"] = tflops / achievable["mfma_bf16_loop_TFLOPs"]
        rooflines.append({"kernel": PF, "bound": "mfma", "achieved": tflops,
                          "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tflops / PEAK_BF16_TFLOPS,
                          "traffic": _traffic_from_profiles(PF), "ms": ms["prefill"]})
    if "prefill_skip" in only:
        res = {}
        curve = []
        for inp, key in (("hot", "prefill_skip"), ("sink", "prefill_sink")):
            xh = work[key]
            L = xh.lens.double()
            flops = 4.0 * 128 * 32 * float((L * (L + 1) / 2).sum())
            sub = {}
            for thr in (0.0, 0.01, 0.1):
                t = ms[f"{key}_{thr}"]
                ent = {"ms": t, **spread(f"{key}_{thr}"), "dense_equiv_tflops": flops / (t * 1e-3) / 1e12}
                if thr > 0:
                    LAUNCH_LOG.append(f"map_{key}_{thr}")
                    _, _, smap = attn.attn_prefill_varlen(xh.q, xh.k, xh.v, xh.cu_q, xh.cu_k, xh.max_q, xh.max_k,
                                                          causal=True, skip_threshold=thr, return_skip_map=True)
                    torch.cuda.synchronize()
                    row_frac, wave_frac = _skip_fractions(torch, xh, smap)
                    del smap
                    ent["row_subtile_skip_frac"] = row_frac
                    # the kernel leaves out a 64-key tile's P.V (half the MFMA work) when no row of the
                    # wave's 32 rows keeps it
                    ent["wave_tile_skip_frac"] = wave_frac
                    ent["ideal_speedup_pv_only"] = 1.0 / (1.0 - 0.5 * wave_frac)
                    ent["speedup_vs_dense"] = ms[f"{key}_0.0"] / t
                    curve.append({"input": inp, "thr": thr, "row_skip": row_frac, "wave_tile_skip": wave_frac,
                                  "speedup": ent["speedup_vs_dense"]})
                sub[str(thr)] = ent
            res[inp] = sub
        res["curve"] = curve
        out["prefill_skip"] = res
    if "decode" in only:
        d = work["decode"]
        kv = 4.0 * d.Hkv * d.D * float(d.lens.sum())
        gbps = kv / (ms["decode"] * 1e-3) / 1e9
        part = d.B * d.Hq * 32 * (d.D + 1) * 4 * 2
        out["decode"] = {"ms": ms["decode"], **spread("decode"), "kv_bytes": kv, "kv_GBps": gbps,
                         "frac_peak": gbps / PEAK_HBM_GBPS, "split_partial_bytes": part,
                         "note": "time covers the split kernel and the merge kernel"}
        if achievable.get("read_1GiB_int64_sum_GBps"):
            out["decode"]["frac_of_plain_read"] = gbps / achievable["read_1GiB_int64_sum_GBps"]
        rooflines.append({"kernel": "decode_split_kernel+decode_merge_kernel", "bound": "hbm", "achieved": gbps,
                          "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
                          "traffic": _traffic_from_profiles("decode_split_kernel"), "ms": ms["decode"]})
    if "skip" in only:
        s = work["skip"]
        G = s.Hq // s.Hkv
        res = {}
        kbytes = 2.0 * s.Hkv * s.D * float(s.lens.sum())
        for thr in (0.0, 0.01, 0.1):
            LAUNCH_LOG.append(f"map_skip_{thr}")
            _, _, smap = attn.attn_decode_paged(s.q, s.k_cache, s.v_cache, s.block_table, s.seq_lens, num_splits=1,
                                                skip_threshold=thr, return_skip_map=True)
            torch.cuda.synchronize()
            m = smap.view(s.B, s.Hkv, G, -1)
            vis = m[:, :, 0] != 2
            f_r = float((smap == 1).sum()) / float((smap != 2).sum())
            vskip = (m == 1).all(2) & vis
            f_v = float(vskip.sum()) / float(vis.sum())
            # algorithmic bytes: all K, V of the tiles some row of the group keeps (32-key tiles)
            kept_tiles_v = float((vis & ~vskip).sum())
            vbytes_kept = kbytes * (kept_tiles_v / float(vis.sum()))
            t = ms[f"skip_{thr}"]
            res[str(thr)] = {"ms": t, **spread(f"skip_{thr}"), "row_tile_skip_frac": f_r,
                             "group_v_tile_skip_frac": f_v, "bytes_read_alg": kbytes + vbytes_kept,
                             "GBps_alg": (kbytes + vbytes_kept) / (t * 1e-3) / 1e9,
                             "dense_equiv_GBps": 2 * kbytes / (t * 1e-3) / 1e9,
                             "ideal_speedup_vs_thr0": 2.0 / (2.0 - f_v)}
        for thr in ("0.01", "0.1"):
            res[thr]["speedup_vs_thr0"] = res["0.0"]["ms"] / res[thr]["ms"]
            if "decode" in out:
                res[thr]["speedup_vs_splitk_dense"] = out["decode"]["ms"] / res[thr]["ms"]
        for thr in ("0.0", "0.1"):
            t = ms[f"qdq_{thr}"]
            by = res[thr]["bytes_read_alg"]
            res[thr]["nvfp4_qdq"] = {"ms": t, **spread(f"qdq_{thr}"), "GBps_alg": by / (t * 1e-3) / 1e9,
                                     "time_over_unquantized": t / res[thr]["ms"]}
        out["skip"] = res
        gq = res["0.0"]["nvfp4_qdq"]["GBps_alg"]
        rooflines.append({"kernel": "decode_seq_qdq_kernel(thr=0, P and V NVFP4)", "bound": "hbm", "achieved": gq,
                          "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": gq / PEAK_HBM_GBPS,
                          "traffic": _traffic_from_profiles("decode_seq_qdq_kernel"),
                          "ms": res["0.0"]["nvfp4_qdq"]["ms"]})
        g0 = res["0.0"]["GBps_alg"]
        rooflines.append({"kernel": "decode_seq_kernel(thr=0)", "bound": "hbm", "achieved": g0,
                          "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": g0 / PEAK_HBM_GBPS,
                          "traffic": _traffic_from_profiles("decode_seq_kernel"), "ms": res["0.0"]["ms"]})
    if "smallseq" in only:
        c = work["smallseq"]
        kv = 4.0 * c.H * c.D * float(c.lens.sum())
        tot = kv + 2.0 * 2 * c.B * c.H * c.D + 2.0 * c.B * c.H * c.max_s
        gbps = kv / (ms["smallseq"] * 1e-3) / 1e9
        out["smallseq"] = {"ms": ms["smallseq"], **spread("smallseq"), "kv_bytes": kv, "kv_GBps": gbps,
                           "all_bytes": tot, "all_GBps": tot / (ms["smallseq"] * 1e-3) / 1e9,
                           "frac_peak": gbps / PEAK_HBM_GBPS}
        rooflines.append({"kernel": "smallseq_kernel", "bound": "hbm", "achieved": gbps, "peak": PEAK_HBM_GBPS,
                          "unit": "GB/s", "frac": gbps / PEAK_HBM_GBPS,
                          "traffic": _traffic_from_profiles("smallseq_kernel"), "ms": ms["smallseq"]})

    if "prefill_bwd" in only:
        L = work["prefill_bwd"].lens.double()
        fwd_flops = 4.0 * 128 * 32 * float((L * (L + 1) / 2).sum())
        t = ms["prefill_bwd"]
        # algorithmic: the five products S (recomputed), dP, dV, dK, dQ = 2.5x the forward's two; the dQ
        # kernel recomputes S and dP once more (executed: 3.5x)
        tf = 2.5 * fwd_flops / (t * 1e-3) / 1e12
        out["prefill_bwd"] = {"ms": t, **spread("prefill_bwd"), "flop_alg": 2.5 * fwd_flops, "tflops_alg": tf,
                              "tflops_executed": 3.5 * fwd_flops / (t * 1e-3) / 1e12,
                              "frac_peak": tf / PEAK_BF16_TFLOPS,
                              "note": "one call: bwd_prep + bwd_dkdv + bwd_dq; timed outside the step"}
        if "prefill" in out:
            out["prefill_bwd"]["bwd_over_fwd_time"] = t / out["prefill"]["ms"]

    if "smallseq_bwd" in only:
        c = work["smallseq_bwd"]
        nk = float(c.lens.sum())
        # read K, V and write dK, dV per key; read q, dO and write dq per sequence; the stored weights read
        byts = 4.0 * c.H * c.D * 2 * nk + 3.0 * c.B * c.H * c.D * 2 + 2.0 * c.H * nk
        t = ms["smallseq_bwd"]
        gb = byts / (t * 1e-3) / 1e9
        out["smallseq_bwd"] = {"ms": t, **spread("smallseq_bwd"), "bytes_alg": byts, "GBps": gb,
                               "frac_peak": gb / PEAK_HBM_GBPS, "note": "one launch; timed outside the step"}

    if "decode_multi" in only:
        dm = work["decode_multi"]
        # every cached key of every KV head once (one 16-row block per group when Lq * G <= 16)
        kv = 4.0 * dm.Hkv * dm.D * float(dm.lens.sum())
        t = ms["decode_multi"]
        gb = kv / (t * 1e-3) / 1e9
        out["decode_multi"] = {"ms": t, **spread("decode_multi"), "kv_bytes": kv, "kv_GBps": gb,
                               "frac_peak": gb / PEAK_HBM_GBPS, "tokens": int(dm.q.shape[0]),
                               "note": "split kernel + merge; timed outside the step"}
        if "decode" in out:
            out["decode_multi"]["time_over_one_token_decode"] = t / out["decode"]["ms"]

    if "prefill_paged" in only:
        pp = work["prefill_paged"]
        Lk = pp.lens.double()
        Lq = pp.qlens.double()
        # token i of a sequence sees L - Lq + i + 1 keys
        pairs = float((Lq * (Lk - Lq) + Lq * (Lq + 1) / 2).sum())
        flops = 4.0 * pp.D * pp.Hq * pairs
        t = ms["prefill_paged"]
        tf = flops / (t * 1e-3) / 1e12
        out["prefill_paged"] = {"ms": t, **spread("prefill_paged"), "flop": flops, "tflops": tf,
                                "frac_peak": tf / PEAK_BF16_TFLOPS, "tokens": int(pp.q.shape[0]),
                                "note": "the prefill kernel with page-gathered K/V; timed outside the step"}
        if "prefill" in out:
            out["prefill_paged"]["tflops_over_contiguous_prefill"] = tf / out["prefill"]["tflops"]

    # the dominant kernel: the largest share of the step
    dom = max(rooflines, key=lambda r: r["ms"]) if rooflines else None
    roofline = None
    if dom:
        roofline = {k: dom[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
        roofline["kernel"] = dom["kernel"]

    cpu = None
    if not args.no_cpu_baseline and "prefill" in only:
        cpu = _cpu_baseline(work["prefill"])
    if not args.no_cpu_baseline:
        # the oracle on a bounded sample of every other workload too (a baseline only, never the target)
        if "decode" in out:
            out["decode"]["cpu_oracle"] = _cpu_decode(work["decode"], "dense", 0.0)
        if "skip" in out:
            out["skip"]["cpu_oracle_thr0.1"] = _cpu_decode(work["skip"], "skip", 0.1)
            out["skip"]["cpu_oracle_nvfp4_thr0.1"] = _cpu_decode(work["skip"], "nvfp4", 0.1)
        if "smallseq" in out:
            out["smallseq"]["cpu_oracle"] = _cpu_smallseq(work["smallseq"])
        if "tiny_fp32" in out:
            for causal in (True, False):
                for thr in (0.0, 0.1):
                    out["tiny_fp32"][f"{'causal' if causal else 'noncausal'}_{thr}"]["cpu_oracle"] = _cpu_tiny(
                        work["tiny"], causal, thr)

    headline = out.get("prefill", {}).get("tflops")
    line = {
        "metric": "prefill TFLOP/s & decode KV GB/s vs MI355X peak; skip-softmax speedup",
        "value": headline,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "varlen causal prefill bf16: 16 seqs, L~U[256,4096] THD, Hq=32, Hkv=8, D=128",
                   "step_also_runs": ["paged decode split-K B=64 L~U[1024,32768] page 16, 32x128-key splits",
                                      "sequential skip decode thr {0,0.01,0.1} on hot keys",
                                      "small-seq cross B=30720 s_kv in {2..16} H=16 D=128"],
                   "timed_after_the_step": ["skip-softmax prefill thr {0,0.01,0.1} on the prefill shapes with hot "
                                            "keys and on the coherent-sink input",
                                            "the prefill backward (dq, dk, dv) on the prefill shapes",
                                            "the small-seq backward from the stored weights on the small-seq shapes",
                                            "multi-token paged decode: the paged-decode cache with 1..4 new tokens "
                                            "per sequence, 32 splits",
                                            "chunked prefill over the paged-decode cache: 256 new tokens per "
                                            "sequence",
                                            "tiny fp32 B=2 Hq=4 Hkv=2 D=64 S=128, {causal, non-causal} x thr {0, 0.1}"],
                   "seed": args.seed},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": out,
        "rooflines": rooflines,
        "achievable_context": achievable,
    }
    print(json.dumps(line), flush=True)
    if args.launch_log:
        os.makedirs(os.path.dirname(os.path.abspath(args.launch_log)), exist_ok=True)
        with open(args.launch_log, "w") as f:
            json.dump(LAUNCH_LOG, f)


def _skip_fractions(torch, x, smap):
    """Fractions of visited (row, 32-key half) pairs skipped, and of (32-row wave block, 64-key tile)
    pairs in which no row keeps either half (the unit whose P.V the kernel leaves out)."""
    vis = smap != 2
    row = float((smap == 1).sum()) / float(vis.sum())
    cu = x.cu_q.cpu().tolist()
    ws = wv = 0
    for b in range(x.B):
        n = cu[b + 1] - cu[b]
        m = smap[cu[b]:cu[b + 1]]                                  # [n, H, S]
        nb, S = (n + 31) // 32, m.shape[-1]
        pad_r = torch.full((nb * 32 - n, m.shape[1], S), 2, dtype=m.dtype, device=m.device)
        m = torch.cat([m, pad_r])
        if S % 2:
            m = torch.cat([m, torch.full((m.shape[0], m.shape[1], 1), 2, dtype=m.dtype, device=m.device)], -1)
        m = m.view(nb, 32, m.shape[1], -1, 2)                      # [blocks, 32 rows, H, tiles, halves]
        kept = (m == 0).any(-1).any(1)                             # some row keeps some half
        seen = (m != 2).any(-1).any(1)
        ws += int((seen & ~kept).sum())
        wv += int(seen.sum())
    return row, ws / max(1, wv)


def _achievable(torch, dev):
    """What plain library kernels reach on this GPU in the same session (context for the fractions of
    the published peaks): a 1 GiB device copy (HBM read + write) and a large bf16 GEMM (hipBLASLt)."""
    res = {}
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    res["copy_1GiB_GBps"] = 2.0 * (1 << 30) / (ms * 1e-3) / 1e9
    # a plain read: torch's sum over 1 GiB viewed as int64 (reads the bytes once, writes one scalar; of the
    # library reductions tried it reads fastest here: float32 sum and amax reach about 4 TB/s)
    x64 = src.view(torch.int64)
    for _ in range(3):
        x64.sum()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        x64.sum()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    res["read_1GiB_int64_sum_GBps"] = float(1 << 30) / (ms * 1e-3) / 1e9
    del src, dst, x64
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        c = a @ b
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 10
    res["gemm_bf16_8192_TFLOPs"] = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    # a plain 32x32x16 bf16 MFMA loop on every CU (two waves per SIMD, operands of ordinary magnitude): the
    # matrix-core rate this chip sustains, clock drop included (measurement-only library, built beside
    # libattn.so)
    probe = os.path.join(ROOT, "paged_skip_softmax_amd", "libattn_probe.so")
    if os.path.exists(probe):
        import ctypes
        lib = ctypes.CDLL(probe)
        lib.attn_probe_mfma_bf16.restype = ctypes.c_int
        lib.attn_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        lib.attn_probe_mfma_bf16_flop.restype = ctypes.c_double
        lib.attn_probe_mfma_bf16_flop.argtypes = [ctypes.c_int, ctypes.c_int]
        blocks, iters = 1024, 10000
        out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
        st = torch.cuda.current_stream().cuda_stream
        for _ in range(2):
            assert lib.attn_probe_mfma_bf16(out.data_ptr(), blocks, iters, st) == 0
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            assert lib.attn_probe_mfma_bf16(out.data_ptr(), blocks, iters, st) == 0
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        res["mfma_bf16_loop_TFLOPs"] = lib.attn_probe_mfma_bf16_flop(blocks, iters) / (ms * 1e-3) / 1e12
        del out
    torch.cuda.empty_cache()
    return res


def _threads():
    return int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)


def _cpu_model():
    """The host CPU's model name (as lscpu reports it), from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _cpu_tiny(x, causal, thr):
    """The fp64 oracle on the whole tiny fp32 workload (every row, every head), repeated until about
    0.2 s have passed; GFLOP/s of the dense-equivalent work, and the mean time of one run."""
    import oracle
    q, k, v, cq, ck = x.q.cpu(), x.k.cpu(), x.v.cpu(), x.cu_q.cpu(), x.cu_k.cpu()
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.prefill(q, k, v, cq, ck, x.Hq, x.Hkv, x.scale, causal, mode="skip", thr=thr, tile=32)
        n += 1
        dt = time.perf_counter() - t0
        if dt > 0.2:
            break
    fl = _tiny_flops(x, causal)
    return {"value": fl * n / dt / 1e9, "unit": "GFLOP/s", "cores": _threads(), "kind": "oracle",
            "cpu_model": _cpu_model(), "ms": dt / n * 1e3,
            "sample": f"the whole workload ({x.q.shape[0] * x.Hq} rows), skip mode with thr {thr} and 32-key tiles, "
                      f"mean of {n} runs"}


def _tiny_flops(x, causal):
    """4 D Hq per visible (query, key) pair."""
    L = x.lens.double()
    pairs = float((L * (L + 1) / 2).sum()) if causal else float((L * L).sum())
    return 4.0 * x.D * x.Hq * pairs


def _cpu_decode(d, mode, thr):
    """The fp64 oracle on the eight longest batch rows of a paged-decode workload, all heads, in GB/s of
    KV read (dense accounting); mode "nvfp4" is the decode with NVFP4 P and V (amax 1).  Only the pages of
    those rows are copied to the host."""
    import numpy as np
    import torch

    import oracle
    L = d.lens.numpy()
    bs = [int(b) for b in np.argsort(-L)[:8]]
    bt = d.block_table[bs]
    used = torch.unique(bt[bt >= 0])
    bt_h = torch.full_like(bt, -1)
    m = bt >= 0
    bt_h[m] = torch.searchsorted(used, bt[m]).to(torch.int32)
    kc, vc = d.k_cache[used].cpu(), d.v_cache[used].cpu()
    q, sl = d.q[bs].cpu(), d.seq_lens[bs].cpu()
    t0 = time.perf_counter()
    if mode == "nvfp4":
        oracle.decode_qdq(q, kc, vc, bt_h.cpu(), sl, d.scale, thr=thr, p_amax=1.0, v_amax=1.0)
    else:
        oracle.decode(q, kc, vc, bt_h.cpu(), sl, d.scale, mode=mode, thr=thr, tile=32)
    dt = time.perf_counter() - t0
    kv = 4.0 * d.Hkv * d.D * float(sl.sum())
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": _threads(), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"the 8 longest batch rows (L = {[int(L[b]) for b in bs]}), all {d.Hq} heads, mode {mode}"
                      f"{' thr ' + str(thr) if mode in ('skip', 'nvfp4') else ''}"
                      f"{' (P and V amax 1)' if mode == 'nvfp4' else ''}: {kv / 1e9:.2f} GB of KV in {dt:.2f} s"}


def _cpu_smallseq(c):
    """The fp64 oracle on the first 4096 sequences of the small-seq workload, all heads, in GB/s of KV."""
    import oracle
    n = 4096
    T = int(c.cu_kv[n])
    q, k, v, cu = c.q[:n].cpu(), c.k[:T].cpu(), c.v[:T].cpu(), c.cu_kv[:n + 1].cpu()
    t0 = time.perf_counter()
    oracle.smallseq(q, k, v, cu, c.max_s, c.scale)
    dt = time.perf_counter() - t0
    kv = 4.0 * c.H * c.D * T
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": _threads(), "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"the first {n} sequences ({T} keys), all {c.H} heads: {kv / 1e9:.3f} GB of KV in {dt:.2f} s"}


def _cpu_baseline(x):
    """The fp64 oracle on a bounded sample of the prefill workload, on this host's cores: every causal
    query row and head of the three longest sequences (about 10 s of CPU work on the GPU machine's host)."""
    import numpy as np

    import oracle
    threads = _threads()
    q, k, v = x.q.cpu(), x.k.cpu(), x.v.cpu()
    cu = x.cu_q.cpu()
    L = x.lens.numpy()
    picked = [int(b) for b in np.argsort(-L, kind="stable")[:3]]
    rows = [(int(cu[b]) + i, h) for b in picked for i in range(int(L[b])) for h in range(x.Hq)]
    t0 = time.perf_counter()
    oracle.prefill(q, k, v, x.cu_q.cpu(), x.cu_k.cpu(), x.Hq, x.Hkv, x.scale, True, rows=rows)
    dt = time.perf_counter() - t0
    flops = sum(4.0 * x.D * (i + 1) for b in picked for i in range(int(L[b]))) * x.Hq
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "sample": f"every causal query row of the three longest sequences (L={[int(L[b]) for b in picked]}), "
                      f"all {x.Hq} heads: {len(rows)} rows, {flops:.3e} FLOP in {dt:.2f} s"}


# ---- rocprofv3 summaries -------------------------------------------------------------------------------

# kernel -> (workload the bench runs it on, summary file stem, sources it is built from)
_KSRC = ["paged_skip_softmax_amd/csrc/kcommon.h", "paged_skip_softmax_amd/csrc/launch.h"]
_LDS = "paged_skip_softmax_amd/csrc/lds_dma.h"
_BWD = ["paged_skip_softmax_amd/csrc/prefill_bwd.hip", _LDS] + _KSRC
_BWD_W = "prefill backward on the prefill shapes (16 seqs L~U[256,4096], Hq=32, Hkv=8, D=128, causal)"
PF = "prefill_d128_kernel<false, false>"   # dense prefill, contiguous K / V
PS = "prefill_d128_kernel<true, false>"    # skip-softmax prefill
PP = "prefill_d128_kernel<false, true>"    # dense prefill, page-gathered K / V

# kernel -> (workload, summary file stem, source files, headline role: the bench call whose launches
# the summary's traffic figure and traffic.json refer to)
PROFILED = {
    PF: ("varlen causal prefill bf16, 16 seqs L~U[256,4096], Hq=32, Hkv=8, D=128",
         "prefill_d128_kernel.varlen_causal_16seq_L256-4096_Hq32_Hkv8_D128",
         ["paged_skip_softmax_amd/csrc/prefill_d128.hip", _LDS] + _KSRC, "prefill"),
    PS: ("skip-softmax prefill on the hot-key and the coherent-sink prefill inputs (same shapes), thresholds "
         "0.01 and 0.1", "prefill_d128_kernel_skip.varlen_causal_hot_sink_16seq_thr0.01-0.1",
         ["paged_skip_softmax_amd/csrc/prefill_d128.hip", _LDS] + _KSRC, "prefill_skip_0.1"),
    PP: ("chunked prefill over the paged-decode cache (B=64, L~U[1024,32768], page 16), 256 new tokens per "
         "sequence", "prefill_d128_kernel_paged.paged_cache_B64_L1k-32k_q256",
         ["paged_skip_softmax_amd/csrc/prefill_d128.hip", _LDS] + _KSRC, "prefill_paged"),
    "decode_split_kernel": ("paged decode B=64, L~U[1024,32768], page 16, 32 splits of 128-key tiles",
                            "decode_split_kernel.paged_decode_B64_L1k-32k_page16_32splits",
                            ["paged_skip_softmax_amd/csrc/decode.hip"] + _KSRC, "decode"),
    "decode_merge_kernel": ("merge of the 32 split partials, B=64, Hq=32, D=128",
                            "decode_merge_kernel.paged_decode_B64_Hq32_32splits",
                            ["paged_skip_softmax_amd/csrc/decode.hip"] + _KSRC, "decode"),
    "decode_multi_kernel": ("multi-token paged decode: the paged-decode cache (B=64, L~U[1024,32768]) with 1..4 new "
                            "tokens per sequence, 32 splits", "decode_multi_kernel.paged_decode_B64_L1k-32k_q1-4_32splits",
                            ["paged_skip_softmax_amd/csrc/decode.hip"] + _KSRC, "decode_multi"),
    "decode_merge_multi_kernel": ("merge of the 32 split partials of the multi-token decode (1..4 tokens x 32 heads "
                                  "per sequence, B=64)", "decode_merge_multi_kernel.paged_decode_B64_q1-4_32splits",
                                  ["paged_skip_softmax_amd/csrc/decode.hip"] + _KSRC, "decode_multi"),
    "decode_seq_kernel": ("sequential skip decode on hot keys, B=64, L~U[1024,32768], 32-key tiles, "
                          "threshold 0 / 0.01 / 0.1", "decode_seq_kernel.paged_decode_hot_B64_thr0-0.01-0.1",
                          ["paged_skip_softmax_amd/csrc/decode.hip"] + _KSRC, "skip_0.0"),
    "decode_seq_qdq_kernel": ("sequential decode with NVFP4 fake quantization of P and V (amax 1) on hot keys, "
                              "B=64, L~U[1024,32768], 32-key tiles, threshold 0 / 0.1",
                              "decode_seq_qdq_kernel.paged_decode_hot_B64_nvfp4_pv_thr0-0.1",
                              ["paged_skip_softmax_amd/csrc/decode.hip"] + _KSRC, "qdq_0.0"),
    "smallseq_kernel": ("small-seq cross-attention B=30720, s_kv in {2,4,6,8,12,16}, H=16, D=128",
                        "smallseq_kernel.smallseq_cross_B30720_H16_D128",
                        ["paged_skip_softmax_amd/csrc/smallseq.hip"] + _KSRC, "smallseq"),
    "smallseq_bwd_kernel": ("small-seq backward from the stored weights, B=30720, s_kv in {2,4,6,8,12,16}, H=16, "
                            "D=128", "smallseq_bwd_kernel.smallseq_cross_B30720_H16_D128",
                            ["paged_skip_softmax_amd/csrc/smallseq.hip"] + _KSRC, "smallseq_bwd"),
    "bwd_prep_kernel": (_BWD_W + ": rowsum(dO * O) and lse * log2(e)",
                        "bwd_prep_kernel.varlen_causal_16seq_L256-4096_Hq32", _BWD, "prefill_bwd"),
    "bwd_dkdv_kernel": (_BWD_W + ": dK, dV", "bwd_dkdv_kernel.varlen_causal_16seq_L256-4096_Hq32_Hkv8_D128", _BWD,
                        "prefill_bwd"),
    "bwd_dq_kernel": (_BWD_W + ": dQ", "bwd_dq_kernel.varlen_causal_16seq_L256-4096_Hq32_Hkv8_D128", _BWD,
                      "prefill_bwd"),
}


def call_kernels(call):
    """The kernels one bench call launches, in order (keys of PROFILED)."""
    if call in ("prefill", "setup_prefill_fwd", "prefill_skip_0.0", "prefill_sink_0.0"):
        return [PF]
    if call.startswith(("prefill_skip_", "prefill_sink_", "map_prefill_")):
        return [PS]
    if call == "prefill_paged":
        return [PP]
    if call == "decode":
        return ["decode_split_kernel", "decode_merge_kernel"]
    if call.startswith(("skip_", "map_skip_")):
        return ["decode_seq_kernel"]
    if call.startswith("qdq_"):
        return ["decode_seq_qdq_kernel"]
    if call in ("smallseq", "setup_smallseq_fwd"):
        return ["smallseq_kernel"]
    if call == "smallseq_bwd":
        return ["smallseq_bwd_kernel"]
    if call == "prefill_bwd":
        return ["bwd_prep_kernel", "bwd_dkdv_kernel", "bwd_dq_kernel"]
    if call == "decode_multi":
        return ["decode_multi_kernel", "decode_merge_multi_kernel"]
    return []


PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d {out}/prof_trace -o run -- "
             "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --launch-log {out}/prof_trace/launch_log.json",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d {out}/prof_fetch -o run -- "
             "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --calib-copy "
             "--launch-log {out}/prof_fetch/launch_log.json",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d {out}/prof_write -o run -- "
             "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --calib-copy "
             "--launch-log {out}/prof_write/launch_log.json",
    "mfma": "rocprofv3 --pmc MfmaUtil SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_BUSY_CYCLES -f csv -d {out}/prof_mfma -o run -- "
            "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --launch-log {out}/prof_mfma/launch_log.json",
    "sq": "rocprofv3 --pmc MfmaUtil VALUBusy LdsUtil LdsBankConflict SQ_VALU_MFMA_BUSY_CYCLES SQ_VALU_MFMA_COEXEC_CYCLES "
          "SQ_WAIT_INST_LDS SQ_WAVE_CYCLES -f csv -d {out}/prof_sq -o run -- "
          "python3 bench.py --steps 2 --warmup 1 --no-cpu-baseline --launch-log {out}/prof_sq/launch_log.json",
    "summary": "python3 bench.py --summarize-profiles {out}",
}


def _csv(dirpath, suffix):
    import csv
    import glob
    hits = sorted(glob.glob(os.path.join(dirpath, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {dirpath}")
    with open(hits[0]) as f:
        return list(csv.DictReader(f))


def _match(name):
    for k in PROFILED:
        if k + "(" in name or k + "<" in name:
            return k
    if "copyBuffer" in name:
        return "copy"
    return None


def _per_dispatch_counter(rows, counter, reduce=sum):
    """kernel key -> list of per-dispatch values (reduced over the counter's instances, summed by
    default), dispatch order."""
    vals, key, order = {}, {}, []
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        d = int(r["Dispatch_Id"])
        if d not in vals:
            vals[d] = []
            key[d] = _match(r["Kernel_Name"])
            order.append(d)
        vals[d].append(float(r["Counter_Value"]))
    agg = {d: float(reduce(v)) for d, v in vals.items()}
    out = {}
    for d in sorted(order):
        if key[d]:
            out.setdefault(key[d], []).append(agg[d])
    return out


def _roles(base, run, k, n):
    """The role (bench call) of each of the n dispatches of kernel k in one profiled run, from the run's
    launch log; None when there is no log or it does not account for exactly n dispatches."""
    path = os.path.join(base, run, "launch_log.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        log = json.load(f)
    roles = [c for c in log for kk in call_kernels(c) if kk == k]
    return roles if len(roles) == n else None


def _by_role(values, roles):
    """role -> values, roles in first-launch order."""
    out = {}
    for v, r in zip(values, roles):
        out.setdefault(r, []).append(v)
    return out


def _summarize_profiles(base):
    import numpy as np
    trace = _csv(os.path.join(base, "prof_trace"), "kernel_trace.csv")
    stats = _csv(os.path.join(base, "prof_trace"), "kernel_stats.csv")
    fetch = _per_dispatch_counter(_csv(os.path.join(base, "prof_fetch"), "counter_collection.csv"), "FETCH_SIZE")
    write = _per_dispatch_counter(_csv(os.path.join(base, "prof_write"), "counter_collection.csv"), "WRITE_SIZE")
    if "copy" not in fetch or "copy" not in write:
        raise RuntimeError("the 1 GiB calibration copy is missing from the counter runs")
    kib = float(1 << 20)
    # the 1 GiB copy is the largest copy dispatch of each run
    c_fetch, c_write = max(fetch["copy"]), max(write["copy"])
    f_fetch = kib / c_fetch
    f_write = kib / c_write
    durs, spans = {}, {}
    for r in sorted(trace, key=lambda r: int(r["Start_Timestamp"])):
        k = _match(r["Kernel_Name"])
        if k and k != "copy":
            durs.setdefault(k, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
            spans.setdefault(k, []).append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    # dK/dV and dQ of one backward call run at the same time (dQ on a side stream): the i-th dispatches of
    # the two belong to the i-th call; the pair's span runs from the earlier start to the later end
    pair = None
    kv, dq = spans.get("bwd_dkdv_kernel", []), spans.get("bwd_dq_kernel", [])
    if kv and len(kv) == len(dq):
        pair = np.array([max(a[1], b[1]) - min(a[0], b[0]) for a, b in zip(kv, dq)], dtype=np.float64) / 1e3
    outdir = os.path.join(ROOT, "profiles")
    os.makedirs(outdir, exist_ok=True)
    traffic = {}
    cmds = "\n".join(f"#   {k}: {v.format(out=base)}" for k, v in PROFILE_COMMANDS.items())
    for k, (workload, stem, srcs, headline) in PROFILED.items():
        if k not in durs:
            continue
        st = [r for r in stats if _match(r["Name"]) == k]
        lines = [f"# {k} on: {workload}",
                 "# commands (repository root, TMPDIR=/tmp; the summary step runs on any host):", cmds, ""]
        for r in st:
            lines.append(f"kernel-trace --stats: calls {r['Calls']}, average {float(r['AverageNs']) / 1e3:.2f} us, "
                         f"min {float(r['MinNs']) / 1e3:.2f} us, max {float(r['MaxNs']) / 1e3:.2f} us, "
                         f"{float(r['Percentage']):.2f}% of GPU kernel time")
        d = np.array(durs[k], dtype=np.float64) / 1e3
        lines.append(f"kernel_trace.csv: {len(d)} dispatches, mean {d.mean():.2f} us, median {np.median(d):.2f} us")
        if k in ("bwd_dkdv_kernel", "bwd_dq_kernel") and pair is not None:
            lines.append("  dK/dV and dQ run at the same time (dQ on a side stream forked after the prep kernel), "
                         "so each one's duration")
            lines.append(f"  spans time shared with the other; the two together: mean {pair.mean():.2f} us, "
                         f"median {np.median(pair):.2f} us per call (earlier start to later end)")
        roles = _roles(base, "prof_trace", k, len(d))
        if roles:
            lines.append("  per bench call (from the run's launch log):")
            for role, v in _by_role(list(d), roles).items():
                lines.append(f"    {role}: mean {np.mean(v):.2f} us over {len(v)} dispatches")
        fk = fetch.get(k, [])
        wk = write.get(k, [])
        if fk and wk:
            fm, wm = float(np.mean(fk)), float(np.mean(wk))
            byts = (fm * f_fetch + wm * f_write) * 1024.0
            lines += [f"FETCH_SIZE {fm:.0f} KiB / dispatch (mean of {len(fk)}), WRITE_SIZE {wm:.0f} KiB / dispatch "
                      f"(mean of {len(wk)})",
                      f"calibration: the 1 GiB copy read FETCH_SIZE {c_fetch:.0f} KiB and WRITE_SIZE "
                      f"{c_write:.0f} KiB, factors {f_fetch:.4f} (fetch) and {f_write:.4f} (write)",
                      f"HBM traffic per launch (scaled), all dispatches: {byts / 1e6:.1f} MB"]
            rf, rw = _roles(base, "prof_fetch", k, len(fk)), _roles(base, "prof_write", k, len(wk))
            if rf and rw:
                bf, bw = _by_role(fk, rf), _by_role(wk, rw)
                lines.append("  per bench call:")
                for role in bf:
                    if role in bw:
                        b_i = (np.mean(bf[role]) * f_fetch + np.mean(bw[role]) * f_write) * 1024.0
                        lines.append(f"    {role}: {b_i / 1e6:.1f} MB per launch")
                if headline in bf and headline in bw:
                    fm, wm = float(np.mean(bf[headline])), float(np.mean(bw[headline]))
                    byts = (fm * f_fetch + wm * f_write) * 1024.0
                    lines.append(f"traffic.json: the {headline} launches, {byts / 1e6:.1f} MB per launch")
            traffic[k] = {"bytes_per_launch": float(byts), "fetch_kib": fm, "write_kib": wm, "role": headline,
                          "fetch_factor": f_fetch, "write_factor": f_write, "sources": srcs,
                          "sources_sha256": _sources_digest(srcs), "summary": f"profiles/{stem}.txt"}
        with open(os.path.join(outdir, stem + ".txt"), "w") as f:
            f.write("\n".join(lines) + "\n")
        print(f"wrote profiles/{stem}.txt")
    with open(os.path.join(outdir, "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1, sort_keys=True)
    print("wrote profiles/traffic.json")
    if os.path.isdir(os.path.join(base, "prof_mfma")):
        _summarize_mfma(base, durs)
    if os.path.isdir(os.path.join(base, "prof_sq")):
        _summarize_sq(base)


# kernels whose matrix-core use the MFMA-busy summary reports (the contraction-bound ones)
MFMA_KERNELS = [PF, PS, PP, "bwd_dkdv_kernel", "bwd_dq_kernel"]


def _summarize_mfma(base, durs):
    """MFMA busy % (rocprofv3's derived MfmaUtil: SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE times
    the SIMD count), executed bf16 MFMA FLOPs per dispatch (SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512) and the
    SQ busy cycles, per kernel and bench call, into profiles/mfma_busy.<workload>.txt."""
    import numpy as np
    rows = _csv(os.path.join(base, "prof_mfma"), "counter_collection.csv")
    util = _per_dispatch_counter(rows, "MfmaUtil", reduce=np.mean)
    mops = _per_dispatch_counter(rows, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    busy = _per_dispatch_counter(rows, "SQ_BUSY_CYCLES", reduce=max)
    lines = ["# MFMA busy per kernel, rocprofv3 counters (one dispatch = one launch), bench workloads as in the",
             "# kernel summaries of this folder",
             "# commands (repository root, TMPDIR=/tmp; the summary step runs on any host):",
             "\n".join(f"#   {k}: {v.format(out=base)}" for k, v in PROFILE_COMMANDS.items()),
             "# MfmaUtil = 100 * sum(SQ_VALU_MFMA_BUSY_CYCLES) / (max(GRBM_GUI_ACTIVE) * SIMDs); executed FLOP =",
             "# SQ_INSTS_VALU_MFMA_MOPS_BF16 * 512 (includes masked and recomputed work); SQ_BUSY_CYCLES as the",
             "# counter reports it (aggregated over the shader engines)", ""]
    for k in MFMA_KERNELS:
        if k not in util:
            continue
        u = util[k]
        lines.append(f"{k}: MfmaUtil mean {np.mean(u):.1f} % over {len(u)} dispatches (min {np.min(u):.1f}, max "
                     f"{np.max(u):.1f})")
        roles = _roles(base, "prof_mfma", k, len(u))
        if roles:
            bu = _by_role(u, roles)
            bm = _by_role(mops.get(k, [0.0] * len(u)), roles) if len(mops.get(k, [])) == len(u) else {}
            bb = _by_role(busy.get(k, [0.0] * len(u)), roles) if len(busy.get(k, [])) == len(u) else {}
            for role, v in bu.items():
                ln = f"    {role}: MfmaUtil {np.mean(v):.1f} %"
                if role in bm:
                    ln += f", executed bf16 MFMA {np.mean(bm[role]) * 512:.4e} FLOP per launch"
                if role in bb:
                    ln += f", SQ_BUSY_CYCLES {np.mean(bb[role]):.0f}"
                lines.append(ln)
    path = os.path.join(ROOT, "profiles", "mfma_busy.bench_workloads.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/mfma_busy.bench_workloads.txt")


def _summarize_sq(base):
    """Where the contraction-bound kernels spend their cycles, from rocprofv3's derived counters (MfmaUtil,
    VALUBusy, LdsUtil, LdsBankConflict) and three SQ counters: the share of MFMA-busy cycles in which a
    VALU instruction issued too (SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES), and the share of
    wave cycles spent waiting for LDS instructions (SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES); per kernel and
    bench call, into profiles/sq_counters.bench_workloads.txt."""
    import numpy as np
    rows = _csv(os.path.join(base, "prof_sq"), "counter_collection.csv")
    mean = dict(reduce=np.mean)
    cols = {"MfmaUtil": _per_dispatch_counter(rows, "MfmaUtil", **mean),
            "VALUBusy": _per_dispatch_counter(rows, "VALUBusy", **mean),
            "LdsUtil": _per_dispatch_counter(rows, "LdsUtil", **mean),
            "LdsBankConflict": _per_dispatch_counter(rows, "LdsBankConflict", **mean)}
    coexec = _per_dispatch_counter(rows, "SQ_VALU_MFMA_COEXEC_CYCLES")
    mbusy = _per_dispatch_counter(rows, "SQ_VALU_MFMA_BUSY_CYCLES")
    wlds = _per_dispatch_counter(rows, "SQ_WAIT_INST_LDS")
    wcyc = _per_dispatch_counter(rows, "SQ_WAVE_CYCLES")
    # dispatch duration (ns) from the rows' timestamps, for the shader clock: GRBM_GUI_ACTIVE cycles,
    # recovered from MfmaUtil = 100 * MFMA-busy cycles / (GRBM_GUI_ACTIVE * SIMDs), over the duration
    span = {}
    for r in rows:
        if r["Counter_Name"] == "MfmaUtil":
            span[int(r["Dispatch_Id"])] = (_match(r["Kernel_Name"]),
                                           int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    durs = {}
    for d in sorted(span):
        if span[d][0]:
            durs.setdefault(span[d][0], []).append(span[d][1])
    simds = 4 * 256
    lines = ["# SQ counters per kernel, rocprofv3 (one dispatch = one launch), bench workloads as in the kernel",
             "# summaries of this folder",
             "# commands (repository root, TMPDIR=/tmp; the summary step runs on any host):",
             "\n".join(f"#   {k}: {v.format(out=base)}" for k, v in PROFILE_COMMANDS.items()),
             "# MfmaUtil, VALUBusy, LdsUtil (%) and LdsBankConflict (conflict cycles per LDS access) as rocprofv3",
             "# derives them; coexec = SQ_VALU_MFMA_COEXEC_CYCLES / SQ_VALU_MFMA_BUSY_CYCLES (the share of",
             "# MFMA-busy cycles in which a VALU instruction also issued); LDS wait = SQ_WAIT_INST_LDS /",
             "# SQ_WAVE_CYCLES (the share of wave cycles spent waiting to issue an LDS instruction); clock =",
             "# GRBM_GUI_ACTIVE cycles (100 * MFMA-busy cycles / (MfmaUtil * 1024 SIMDs)) over the dispatch's",
             "# duration under counter collection: the shader clock the kernel ran at (published maximum",
             "# 2.4 GHz)", ""]
    for k in MFMA_KERNELS:
        if k not in cols["MfmaUtil"]:
            continue
        n = len(cols["MfmaUtil"][k])
        roles = _roles(base, "prof_sq", k, n) or ["all"] * n

        def part(vals, r):
            return [v for v, x in zip(vals, roles) if x == r] if len(vals) == n else []

        lines.append(f"{k}: {n} dispatches")
        for r in dict.fromkeys(roles):
            f = []
            for name, c in cols.items():
                v = part(c.get(k, []), r)
                if v:
                    f.append(f"{name} {np.mean(v):.3g}" + (" %" if name != "LdsBankConflict" else ""))
            ce, mb = part(coexec.get(k, []), r), part(mbusy.get(k, []), r)
            if ce and mb and sum(mb) > 0:
                f.append(f"coexec {sum(ce) / sum(mb):.2f}")
            wl, wc = part(wlds.get(k, []), r), part(wcyc.get(k, []), r)
            if wl and wc and sum(wc) > 0:
                f.append(f"LDS wait {100 * sum(wl) / sum(wc):.1f} %")
            mu, du = part(cols["MfmaUtil"].get(k, []), r), part(durs.get(k, []), r)
            if mb and mu and du and len(mb) == len(mu) == len(du):
                ghz = [100 * b / (u * simds) / t for b, u, t in zip(mb, mu, du) if u > 0 and t > 0]
                if ghz:
                    f.append(f"clock {np.mean(ghz):.2f} GHz")
            lines.append(f"    {r}: " + ", ".join(f))
    path = os.path.join(ROOT, "profiles", "sq_counters.bench_workloads.txt")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("wrote profiles/sq_counters.bench_workloads.txt")


if __name__ == "__main__":
    main()
