"""Python binding of the fp64 CPU oracle (``oracle/oracle.c``).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library and never imports it.

All functions take CPU torch tensors or numpy arrays holding the exact input bytes (fp32, or bf16), and
return fp64 numpy arrays.  ``rows`` selects which output rows to compute (default: all of them), so that
full-size workloads can be checked on a sample.

Modes: ``"dense"`` (the plain masked-softmax definition), ``"skip"`` (skip-softmax over ``tile``-key
tiles in ascending order with threshold ``thr``, optionally replaying a given skip map) and ``"split"``
(split-K over ``tile``-key tiles in ``splits`` contiguous chunks merged by log-sum-exp).
Skip-map codes: 0 processed, 1 skipped, 2 not visited.

``prefill_backward`` gives the gradients (dq, dk, dv) of the dense varlen prefill for an output gradient.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_MODES = {"dense": 0, "skip": 1, "split": 2}
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c with gcc (fp64, OpenMP) into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
        lib.orc_prefill_rows.argtypes = [I, P, P, P, P, P, I, I, I, I, D, I, I, D, I, I, P, I, P, I, P, P, P]
        lib.orc_decode_rows.argtypes = [P, P, P, P, P, I, I, I, I, I, I, D, I, D, I, I, P, I, P, I, P, P, P]
        lib.orc_smallseq_rows.argtypes = [I, P, P, P, P, I, I, I, I, D, P, I, P, P, P]
        lib.orc_prefill_bwd.argtypes = [I, P, P, P, P, P, P, P, I, I, I, I, D, I, P, P, P]
        lib.orc_smallseq_bwd.argtypes = [I, P, P, P, P, P, P, I, I, I, I, D, P, P, P]
        lib.orc_paged_multi_rows.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, D, P, I, P, P]
        F = ctypes.c_float
        lib.orc_decode_qdq_rows.argtypes = [P, P, P, P, P, I, I, I, I, I, I, D, D, F, F, P, I, P, I, P, P, P]
        lib.orc_fp_round.argtypes = [I, P, P, ctypes.c_size_t]
        lib.orc_nvfp4_qdq.argtypes = [P, ctypes.c_size_t, I, F, P]
        for f in (lib.orc_prefill_rows, lib.orc_decode_rows, lib.orc_smallseq_rows, lib.orc_prefill_bwd,
                  lib.orc_smallseq_bwd, lib.orc_paged_multi_rows, lib.orc_decode_qdq_rows, lib.orc_fp_round,
                  lib.orc_nvfp4_qdq):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _np(x):
    """Contiguous numpy view of the raw bytes; bf16 becomes uint16.  Returns (array, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), 1
            if x.dtype == torch.float32:
                return x.numpy(), 0
            if x.dtype in (torch.int32, torch.int64):
                return np.ascontiguousarray(x.numpy().astype(np.int32)), -1
            raise TypeError("unsupported dtype %s" % x.dtype)
    except ImportError:
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, 0
    if x.dtype == np.uint16:
        return x, 1
    if x.dtype in (np.int32, np.int64):
        return np.ascontiguousarray(x.astype(np.int32)), -1
    raise TypeError("unsupported dtype %s" % x.dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _rows_arg(rows, default):
    r = np.ascontiguousarray(np.asarray(default if rows is None else rows, dtype=np.int32).reshape(-1, 2))
    return r


def _map_args(mode, replay, stride, n_rows, ntile_default):
    if mode != "skip":
        return None, 1, None
    stride = int(stride if stride is not None else max(1, ntile_default))
    rp = None
    if replay is not None:
        rp = np.ascontiguousarray(np.asarray(replay, dtype=np.uint8).reshape(n_rows, stride))
    return rp, stride, np.empty((n_rows, stride), dtype=np.uint8)


def prefill(q, k, v, cu_q, cu_k, Hq, Hkv, scale, causal, mode="dense", thr=0.0, tile=32, splits=1,
            rows=None, replay=None, stride=None):
    """Varlen THD attention.  rows: (token, head) pairs; default all, in token-major order."""
    qa, dt = _np(q)
    ka, dk = _np(k)
    va, dv = _np(v)
    assert dt == dk == dv and dt in (0, 1)
    cq, _ = _np(cu_q)
    ck, _ = _np(cu_k)
    T, D = qa.shape[0], qa.shape[-1]
    B = len(cq) - 1
    allrows = [(t, h) for t in range(T) for h in range(Hq)] if rows is None else None
    r = _rows_arg(rows, allrows)
    n = len(r)
    maxk = int(np.max(np.diff(ck))) if B > 0 else 0
    rp, stride, mp = _map_args(mode, replay, stride, n, (maxk + tile - 1) // tile)
    o = np.zeros((n, D))
    lse = np.zeros(n)
    rc = _load().orc_prefill_rows(dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(cq), _ptr(ck), B, Hq, Hkv, D,
                                  float(scale), int(bool(causal)), _MODES[mode], float(thr), int(tile),
                                  int(splits), _ptr(r), n, _ptr(rp), stride, _ptr(o), _ptr(lse), _ptr(mp))
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments")
    if rows is None:
        o = o.reshape(T, Hq, D)
        lse = lse.reshape(T, Hq)
        if mp is not None:
            mp = mp.reshape(T, Hq, stride)
    return o, lse, mp


def decode(q, k_cache, v_cache, block_table, seq_lens, scale, mode="dense", thr=0.0, tile=32, splits=1,
           rows=None, replay=None, stride=None):
    """One-token paged decode over [num_pages, Hkv, page, D] caches.  rows: (b, head) pairs."""
    qa, dt = _np(q)
    ka, dk = _np(k_cache)
    va, dv = _np(v_cache)
    assert dt == dk == dv == 1, "paged decode is bf16"
    bt, _ = _np(block_table)
    sl, _ = _np(seq_lens)
    B, Hq, D = qa.shape
    Hkv, page = ka.shape[1], ka.shape[2]
    max_pages = bt.shape[1]
    allrows = [(b, h) for b in range(B) for h in range(Hq)] if rows is None else None
    r = _rows_arg(rows, allrows)
    n = len(r)
    maxk = int(sl.max()) if B else 0
    rp, stride, mp = _map_args(mode, replay, stride, n, (max(maxk, max_pages * page) + tile - 1) // tile)
    o = np.zeros((n, D))
    lse = np.zeros(n)
    rc = _load().orc_decode_rows(_ptr(qa), _ptr(ka), _ptr(va), _ptr(bt), _ptr(sl), B, Hq, Hkv, D, page,
                                 max_pages, float(scale), _MODES[mode], float(thr), int(tile), int(splits),
                                 _ptr(r), n, _ptr(rp), stride, _ptr(o), _ptr(lse), _ptr(mp))
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    if rows is None:
        o = o.reshape(B, Hq, D)
        lse = lse.reshape(B, Hq)
        if mp is not None:
            mp = mp.reshape(B, Hq, stride)
    return o, lse, mp


def decode_qdq(q, k_cache, v_cache, block_table, seq_lens, scale, thr=0.0, p_amax=0.0, v_amax=0.0, rows=None,
               replay=None):
    """One-token paged decode in one sequential pass of 32-key tiles with skip threshold ``thr`` (or the
    decisions of ``replay`` [rows, stride], 1 = skip) and NVFP4 fake quantization of P (``p_amax`` > 0) and
    V (``v_amax`` > 0).  Returns (o, lse, skip map)."""
    qa, dt = _np(q)
    ka, dk = _np(k_cache)
    va, dv = _np(v_cache)
    assert dt == dk == dv == 1, "paged decode is bf16"
    bt, _ = _np(block_table)
    sl, _ = _np(seq_lens)
    B, Hq, D = qa.shape
    Hkv, page = ka.shape[1], ka.shape[2]
    max_pages = bt.shape[1]
    allrows = [(b, h) for b in range(B) for h in range(Hq)] if rows is None else None
    r = _rows_arg(rows, allrows)
    n = len(r)
    maxk = int(sl.max()) if B else 0
    stride = max(1, (max(maxk, max_pages * page) + 31) // 32)
    rp = None
    if replay is not None:
        rp = np.ascontiguousarray(np.asarray(replay, dtype=np.uint8).reshape(n, -1))
        stride = rp.shape[1]
    o = np.zeros((n, D))
    lse = np.zeros(n)
    mp = np.zeros((n, stride), dtype=np.uint8)
    rc = _load().orc_decode_qdq_rows(_ptr(qa), _ptr(ka), _ptr(va), _ptr(bt), _ptr(sl), B, Hq, Hkv, D, page,
                                     max_pages, float(scale), float(thr), float(p_amax), float(v_amax), _ptr(r), n,
                                     _ptr(rp), stride, _ptr(o), _ptr(lse), _ptr(mp))
    if rc != 0:
        raise ValueError("oracle decode_qdq rejected its arguments")
    if rows is None:
        o = o.reshape(B, Hq, D)
        lse = lse.reshape(B, Hq)
        mp = mp.reshape(B, Hq, stride)
    return o, lse, mp


def fp_round(fmt, y):
    """Nearest value of the E2M1 (``fmt="e2m1"``) or E4M3 (``"e4m3"``) grid to each y >= 0 (fp32), ties to
    the even code, saturating at the top."""
    ya = np.ascontiguousarray(np.asarray(y, dtype=np.float32))
    out = np.empty_like(ya)
    if _load().orc_fp_round({"e2m1": 0, "e4m3": 1}[fmt], _ptr(ya), _ptr(out), ya.size) != 0:
        raise ValueError("fp_round: values must be >= 0")
    return out


def nvfp4_qdq(x, amax):
    """NVFP4 fake quantization (fp32) of x along its last dimension, in blocks of 16, tensor amax ``amax``."""
    xa = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty_like(xa)
    length = xa.shape[-1]
    if _load().orc_nvfp4_qdq(_ptr(xa), xa.size // max(length, 1), length, float(amax), _ptr(out)) != 0:
        raise ValueError("nvfp4_qdq rejected its arguments")
    return out


def smallseq(q, k, v, cu_kv, max_s, scale, rows=None, with_lse=False):
    """s_q = 1 cross-attention with attention weights.  rows: (b, head) pairs.  Returns (o, w), or
    (o, w, lse) with ``with_lse`` (lse [B, H], or [n_rows] for given rows; -inf with no key)."""
    qa, dt = _np(q)
    ka, dk = _np(k)
    va, dv = _np(v)
    assert dt == dk == dv and dt in (0, 1)
    cu, _ = _np(cu_kv)
    B, H, D = qa.shape
    allrows = [(b, h) for b in range(B) for h in range(H)] if rows is None else None
    r = _rows_arg(rows, allrows)
    n = len(r)
    o = np.zeros((n, D))
    w = np.zeros((n, max(int(max_s), 0)))
    lse = np.zeros(n)
    rc = _load().orc_smallseq_rows(dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(cu), B, H, D, int(max_s),
                                   float(scale), _ptr(r), n, _ptr(o), _ptr(w), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle smallseq rejected its arguments")
    if rows is None:
        o = o.reshape(B, H, D)
        w = w.reshape(B, H, 1, max(int(max_s), 0))
        lse = lse.reshape(B, H)
    return (o, w, lse) if with_lse else (o, w)


def decode_multi(q, cu_q, k_cache, v_cache, block_table, seq_lens, scale, rows=None):
    """Multi-token paged decode: q [total_q, Hq, D] THD with cu_q; rows: (token, head) pairs."""
    qa, dt = _np(q)
    ka, dk = _np(k_cache)
    va, dv = _np(v_cache)
    assert dt == dk == dv == 1, "paged decode is bf16"
    cq, _ = _np(cu_q)
    bt, _ = _np(block_table)
    sl, _ = _np(seq_lens)
    T, Hq, D = qa.shape
    B = len(sl)
    Hkv, page = ka.shape[1], ka.shape[2]
    allrows = [(t, h) for t in range(T) for h in range(Hq)] if rows is None else None
    r = _rows_arg(rows, allrows)
    n = len(r)
    o = np.zeros((n, D))
    lse = np.zeros(n)
    rc = _load().orc_paged_multi_rows(_ptr(qa), _ptr(cq), _ptr(ka), _ptr(va), _ptr(bt), _ptr(sl), B, Hq, Hkv, D,
                                      page, bt.shape[1], float(scale), _ptr(r), n, _ptr(o), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle multi-token decode rejected its arguments")
    if rows is None:
        o = o.reshape(T, Hq, D)
        lse = lse.reshape(T, Hq)
    return o, lse


def smallseq_backward(q, k, v, w, dout, cu_kv, max_s, scale):
    """Gradients (dq, dk, dv) of the small-seq cross-attention from the stored weights w [B, H, 1, max_s]."""
    qa, dt = _np(q)
    ka, dk_ = _np(k)
    va, dv_ = _np(v)
    wa, dw_ = _np(w)
    ga, dg = _np(dout)
    assert dt == dk_ == dv_ == dw_ == dg and dt in (0, 1)
    cu, _ = _np(cu_kv)
    B, H, D = qa.shape
    assert wa.shape == (B, H, 1, int(max_s)) and ga.shape == qa.shape
    dq = np.zeros(qa.shape, dtype=np.float64)
    dk = np.zeros(ka.shape, dtype=np.float64)
    dv = np.zeros(va.shape, dtype=np.float64)
    rc = _load().orc_smallseq_bwd(dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(wa), _ptr(ga), _ptr(cu), B, H, D,
                                  int(max_s), float(scale), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle smallseq backward rejected its arguments")
    return dq, dk, dv


def prefill_backward(q, k, v, dout, cu_q, cu_k, Hq, Hkv, scale, causal, o=None):
    """Gradients (dq, dk, dv) of the dense varlen prefill for the output gradient ``dout`` (all rows).

    o (optional, dout's dtype and shape): a stored forward output; the row dots dO.o then replace the exact
    sum_j p_j dP_j in dS, as a backward that reads the saved output computes them."""
    qa, dt = _np(q)
    ka, dk_ = _np(k)
    va, dv_ = _np(v)
    ga, dg = _np(dout)
    assert dt == dk_ == dv_ == dg and dt in (0, 1)
    oa = None
    if o is not None:
        oa, do_ = _np(o)
        assert do_ == dt and oa.shape == ga.shape
    cq, _ = _np(cu_q)
    ck, _ = _np(cu_k)
    B = len(cq) - 1
    D = qa.shape[-1]
    dq = np.zeros(qa.shape, dtype=np.float64)
    dk = np.zeros(ka.shape, dtype=np.float64)
    dv = np.zeros(va.shape, dtype=np.float64)
    rc = _load().orc_prefill_bwd(dt, _ptr(qa), _ptr(ka), _ptr(va), _ptr(ga), None if oa is None else _ptr(oa),
                                 _ptr(cq), _ptr(ck), B, Hq, Hkv, D, float(scale), int(bool(causal)), _ptr(dq),
                                 _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle backward rejected its arguments")
    return dq, dk, dv

