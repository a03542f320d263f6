"""The C ABI without a GPU: the library loads, exports every declared entry point, and rejects bad
arguments with the documented status before any HIP runtime call (no compute call is made here)."""
import ctypes
import math
import os
import re

import pytest

from paged_skip_softmax_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUPPORTED, WORKSPACE = _lib.ATTN_ERR_INVALID, _lib.ATTN_ERR_UNSUPPORTED, _lib.ATTN_ERR_WORKSPACE
FAKE = 0x1000  # a non-NULL pointer value; validation fails before anything could dereference it


def _declared():
    text = open(os.path.join(ROOT, "include", "attn.h")).read()
    return sorted(set(re.findall(r"^\w[\w \*]*?\b(attn_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n)


def _decode(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, B=2, Hq=8, Hkv=2, D=128, page=16, pages=100, maxp=10,
             scale=0.1, thr=0.0, splits=0, ws=FAKE, wsb=1 << 30, o=FAKE, lse=None, map=None, stride=5, stream=None)
    a.update(kw)
    return lib.attn_decode_paged(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                 a["page"], a["pages"], a["maxp"], a["scale"], a["thr"], a["splits"], a["ws"],
                                 a["wsb"], a["o"], a["lse"], a["map"], a["stride"], a["stream"])


def test_decode_validation(lib):
    assert _decode(lib, B=-1) == INVALID
    assert _decode(lib, Hq=7) == INVALID
    for thr in (float("nan"), -0.01, 1.01, math.inf):
        assert _decode(lib, thr=thr) == INVALID
    assert _decode(lib, splits=65) == INVALID
    assert _decode(lib, splits=-1) == INVALID
    assert _decode(lib, thr=0.1, splits=32) == INVALID
    assert _decode(lib, scale=math.nan) == INVALID
    assert _decode(lib, map=FAKE, splits=32) == INVALID
    assert _decode(lib, map=FAKE, splits=1, stride=4) == INVALID
    assert _decode(lib, D=64) == UNSUPPORTED
    assert _decode(lib, page=32) == UNSUPPORTED
    assert _decode(lib, Hq=34, Hkv=2) == UNSUPPORTED
    assert _decode(lib, q=None) == INVALID
    assert _decode(lib, wsb=100) == WORKSPACE
    assert _decode(lib, ws=None) == WORKSPACE
    assert _decode(lib, B=0) == _lib.ATTN_OK
    # B is a grid dimension of both schedules
    assert _decode(lib, B=65536) == UNSUPPORTED
    assert _decode(lib, B=65536, thr=0.1, splits=1) == UNSUPPORTED
    _decode(lib, splits=99)
    assert b"num_splits" in lib.attn_last_error_message()


def _decode_qdq(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, B=2, Hq=8, Hkv=2, D=128, page=16, pages=100, maxp=10,
             scale=0.1, thr=0.0, pa=1.0, va=1.0, o=FAKE, lse=None, map=None, stride=5, stream=None)
    a.update(kw)
    return lib.attn_decode_paged_qdq(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                     a["page"], a["pages"], a["maxp"], a["scale"], a["thr"], a["pa"], a["va"],
                                     a["o"], a["lse"], a["map"], a["stride"], a["stream"])


def test_decode_qdq_validation(lib):
    for bad in (-1.0, math.nan, math.inf, 1e-30, 1e30):
        assert _decode_qdq(lib, pa=bad) == INVALID
        assert _decode_qdq(lib, va=bad) == INVALID
    assert b"amax" in lib.attn_last_error_message()
    for thr in (math.nan, -0.01, 1.01):
        assert _decode_qdq(lib, thr=thr) == INVALID
    assert _decode_qdq(lib, B=-1) == INVALID
    assert _decode_qdq(lib, Hq=7) == INVALID
    assert _decode_qdq(lib, scale=math.nan) == INVALID
    assert _decode_qdq(lib, map=FAKE, stride=4) == INVALID
    assert _decode_qdq(lib, D=64) == UNSUPPORTED
    assert _decode_qdq(lib, page=32) == UNSUPPORTED
    assert _decode_qdq(lib, Hq=34, Hkv=2) == UNSUPPORTED
    assert _decode_qdq(lib, B=65536) == UNSUPPORTED
    assert _decode_qdq(lib, vc=None) == INVALID
    assert _decode_qdq(lib, B=0) == _lib.ATTN_OK
    assert _decode_qdq(lib, B=0, pa=0.0, va=0.0) == _lib.ATTN_OK


def test_workspace_size(lib):
    assert lib.attn_decode_paged_workspace_size(64, 32, 128, 32) == 64 * 32 * 32 * 129 * 4
    assert lib.attn_decode_paged_workspace_size(64, 32, 128, 0) == 64 * 32 * 32 * 129 * 4
    assert lib.attn_decode_paged_workspace_size(64, 32, 128, 1) == 0
    assert lib.attn_decode_paged_workspace_size(0, 32, 128, 32) == 0


def _prefill(lib, **kw):
    a = dict(dt=_lib.ATTN_BF16, q=FAKE, k=FAKE, v=FAKE, cq=FAKE, ck=FAKE, B=2, mq=10, mk=10, Hq=8, Hkv=2, D=128,
             scale=0.1, causal=1, thr=0.0, o=FAKE, lse=None, map=None, stride=1, stream=None)
    a.update(kw)
    return lib.attn_prefill_varlen(a["dt"], a["q"], a["k"], a["v"], a["cq"], a["ck"], a["B"], a["mq"], a["mk"],
                                   a["Hq"], a["Hkv"], a["D"], a["scale"], a["causal"], a["thr"], a["o"], a["lse"],
                                   a["map"], a["stride"], a["stream"])


def test_prefill_validation(lib):
    assert _prefill(lib, dt=7) == INVALID
    assert _prefill(lib, B=-1) == INVALID
    assert _prefill(lib, Hkv=3) == INVALID
    assert _prefill(lib, thr=2.0) == INVALID
    assert _prefill(lib, thr=float("nan")) == INVALID
    assert _prefill(lib, map=FAKE, mk=100, stride=3) == INVALID
    assert _prefill(lib, D=96) == UNSUPPORTED
    assert _prefill(lib, dt=_lib.ATTN_F32, D=128) == UNSUPPORTED
    assert _prefill(lib, k=None) == INVALID
    assert _prefill(lib, B=0) == _lib.ATTN_OK
    assert _prefill(lib, mq=0) == _lib.ATTN_OK
    # size limits of the bf16 kernels: K/V rows of one sequence addressed in 31 bits, skip-map offsets in 32
    assert _prefill(lib, mk=1 << 20, Hkv=8, Hq=8) == UNSUPPORTED
    assert _prefill(lib, map=FAKE, B=4096, mq=4096, mk=4096, Hq=32, Hkv=8, stride=128) == UNSUPPORTED
    assert b"2^32" in lib.attn_last_error_message()
    # the D = 64 kernels put B and the query tiles in grid dimensions; the D = 128 kernel uses one
    for dt in (_lib.ATTN_BF16, _lib.ATTN_F32):
        assert _prefill(lib, dt=dt, D=64, B=65536) == UNSUPPORTED
        assert _prefill(lib, dt=dt, D=64, mq=65535 * 64 + 1) == UNSUPPORTED
    assert _prefill(lib, B=0, D=128, mq=65535 * 64 + 1) == _lib.ATTN_OK


def _backward(lib, **kw):
    a = dict(dt=_lib.ATTN_BF16, q=FAKE, k=FAKE, v=FAKE, o=FAKE, do=FAKE, lse=FAKE, cq=FAKE, ck=FAKE, B=2, mq=10,
             mk=10, Hq=8, Hkv=2, D=128, scale=0.1, causal=1, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE, wsb=1 << 20,
             stream=None)
    a.update(kw)
    return lib.attn_prefill_varlen_backward(a["dt"], a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["cq"],
                                            a["ck"], a["B"], a["mq"], a["mk"], a["Hq"], a["Hkv"], a["D"], a["scale"],
                                            a["causal"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], a["stream"])


def test_backward_validation(lib):
    assert lib.attn_prefill_varlen_backward_workspace_size(3, 100, 8) == 3 * 100 * 8 * 8
    assert lib.attn_prefill_varlen_backward_workspace_size(0, 100, 8) == 0
    assert _backward(lib, dt=5) == INVALID
    assert _backward(lib, B=-1) == INVALID
    assert _backward(lib, Hq=6, Hkv=4) == INVALID
    assert _backward(lib, scale=math.inf) == INVALID
    assert _backward(lib, D=64) == UNSUPPORTED
    assert _backward(lib, dt=_lib.ATTN_F32) == UNSUPPORTED
    assert _backward(lib, B=1 << 16, mq=1 << 12, Hq=8) == UNSUPPORTED
    assert _backward(lib, mq=1 << 17, Hq=64, Hkv=8) == UNSUPPORTED
    assert _backward(lib, mk=1 << 20, Hq=8, Hkv=8) == UNSUPPORTED
    assert _backward(lib, lse=None) == INVALID
    assert _backward(lib, dv=None) == INVALID
    assert _backward(lib, wsb=2 * 10 * 8 * 8 - 1) == WORKSPACE
    assert _backward(lib, ws=None) == WORKSPACE
    assert _backward(lib, B=0) == _lib.ATTN_OK
    _backward(lib, D=96)
    assert b"D = 128" in lib.attn_last_error_message()


def _small(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, cu=FAKE, B=4, H=16, D=128, ms=16, scale=0.1, o=FAKE, w=None, lse=None,
             stream=None)
    a.update(kw)
    return lib.attn_smallseq_cross(a["q"], a["k"], a["v"], a["cu"], a["B"], a["H"], a["D"], a["ms"], a["scale"],
                                   a["o"], a["w"], a["lse"], a["stream"])


def test_smallseq_validation(lib):
    assert _small(lib, ms=17) == INVALID
    assert _small(lib, ms=-1) == INVALID
    assert _small(lib, B=-2) == INVALID
    assert _small(lib, H=0) == INVALID
    assert _small(lib, D=64) == UNSUPPORTED
    assert _small(lib, cu=None) == INVALID
    assert _small(lib, B=0) == _lib.ATTN_OK


def test_smallseq_backward_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, w=FAKE, do=FAKE, cu=FAKE, B=4, H=16, D=128, ms=16, scale=0.1, dq=FAKE,
                 dk=FAKE, dv=FAKE, stream=None)
        a.update(kw)
        return lib.attn_smallseq_cross_backward(a["q"], a["k"], a["v"], a["w"], a["do"], a["cu"], a["B"], a["H"],
                                                a["D"], a["ms"], a["scale"], a["dq"], a["dk"], a["dv"], a["stream"])
    assert call(ms=17) == INVALID
    assert call(B=-1) == INVALID
    assert call(H=0) == INVALID
    assert call(scale=math.nan) == INVALID
    assert call(D=64) == UNSUPPORTED
    assert call(w=None) == INVALID
    assert call(dk=None) == INVALID
    assert call(B=0) == _lib.ATTN_OK


def test_decode_multi_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, cq=FAKE, tq=10, mq=4, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, B=4, Hq=32, Hkv=8, D=128, page=16,
                 pages=100, maxp=10, scale=0.1, thr=0.0, splits=0, ws=FAKE, wsb=1 << 30, o=FAKE, lse=None, map=None,
                 stride=5, stream=None)
        a.update(kw)
        return lib.attn_decode_paged_multi(a["q"], a["cq"], a["tq"], a["mq"], a["kc"], a["vc"], a["bt"], a["sl"],
                                           a["B"], a["Hq"], a["Hkv"], a["D"], a["page"], a["pages"], a["maxp"],
                                           a["scale"], a["thr"], a["splits"], a["ws"], a["wsb"], a["o"], a["lse"],
                                           a["map"], a["stride"], a["stream"])
    assert lib.attn_decode_paged_multi_workspace_size(10, 4, 32, 8, 128, 0) == 10 * 32 * 32 * 129 * 4
    assert lib.attn_decode_paged_multi_workspace_size(10, 4, 32, 8, 128, 7) == 10 * 32 * 7 * 129 * 4
    assert lib.attn_decode_paged_multi_workspace_size(10, 17, 32, 8, 128, 0) == 0  # the paged prefill path
    assert call(B=-1) == INVALID
    assert call(Hkv=5) == INVALID
    assert call(splits=65) == INVALID
    assert call(scale=math.inf) == INVALID
    assert call(D=64) == UNSUPPORTED
    assert call(page=32) == UNSUPPORTED
    assert call(mq=1 << 20, B=1 << 10) == UNSUPPORTED
    # 8 tokens x 4 heads = 2 blocks of 16 rows per sequence: B * 2 grid blocks in z
    assert call(B=32768, mq=8) == UNSUPPORTED
    assert call(B=32767, mq=8, wsb=100) == WORKSPACE  # within the grid; fails on the workspace next
    for thr in (float("nan"), -0.5, 1.5):
        assert call(thr=thr) == INVALID
    assert call(map=FAKE, stride=4) == INVALID  # 10 pages of 16 keys need 5 tiles
    assert call(map=FAKE, tq=1 << 17, B=4, mq=1 << 9, maxp=1 << 11, stride=1 << 10) == UNSUPPORTED  # 2^32 B map
    # skip-softmax takes the paged prefill kernel: no workspace needed, and no split-K grid limit
    assert call(thr=0.1, ws=None, wsb=0, B=0) == _lib.ATTN_OK
    assert call(cq=None) == INVALID
    assert call(wsb=100) == WORKSPACE
    assert call(B=0) == _lib.ATTN_OK
    assert call(tq=0) == _lib.ATTN_OK


def test_status_strings(lib):
    for s in range(5):
        assert lib.attn_status_string(s)
    assert lib.attn_status_string(99) == b"unknown status"


def test_python_binding_raises_without_gpu_tensors():
    import torch
    import paged_skip_softmax_amd as attn
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        attn.attn_decode_paged(q, q, q, q, q)


@pytest.mark.parametrize("scale", [0.0, -0.1, -math.inf, math.nan, 3.0e38])
def test_scale_must_be_positive_and_finite(lib, scale):
    """A zero scale makes the kernels' masked -inf * 0 a NaN and a negative one turns tile maxima into
    minima, so every entry point rejects scale <= 0 (and a scale whose log2-domain value overflows)."""
    assert _decode(lib, scale=scale) == INVALID
    assert _decode_qdq(lib, scale=scale) == INVALID
    assert _prefill(lib, scale=scale) == INVALID
    assert _backward(lib, scale=scale) == INVALID
    assert _small(lib, scale=scale) == INVALID
    assert b"scale" in lib.attn_last_error_message()


def test_python_binding_checks_out_shapes():
    """A caller-supplied out= of the wrong shape is refused before anything is launched."""
    import torch
    import paged_skip_softmax_amd as attn
    from unittest import mock

    # the binding's device checks run first; patch is_cuda so the shape check is what fails
    q = torch.zeros(2, 8, 128, dtype=torch.bfloat16)
    kc = torch.zeros(4, 2, 16, 128, dtype=torch.bfloat16)
    bt = torch.zeros(2, 2, dtype=torch.int32)
    sl = torch.zeros(2, dtype=torch.int32)
    cu = torch.zeros(3, dtype=torch.int32)
    bad = torch.zeros(1, 8, 128, dtype=torch.bfloat16)
    with mock.patch.object(torch.Tensor, "is_cuda", new=property(lambda self: True)):
        with pytest.raises(ValueError, match="out"):
            attn.attn_decode_paged(q, kc, kc, bt, sl, out=bad)
        with pytest.raises(ValueError, match="out"):
            attn.attn_decode_paged_qdq(q, kc, kc, bt, sl, out=bad)
        with pytest.raises(ValueError, match="out"):
            attn.attn_decode_paged_multi(q, cu, 1, kc, kc, bt, sl, out=bad)
        with pytest.raises(ValueError, match="out"):
            attn.attn_smallseq_cross(q, q, q, cu, 1, out=bad)


def test_decode_noalloc_validation(lib):
    """The allocation-free decode: the decode's argument checks, and partials beyond the scratch rejected
    with ATTN_ERR_WORKSPACE, all before any HIP call."""
    def call(**kw):
        a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, B=2, Hq=8, Hkv=2, D=128, page=16, pages=100, maxp=10,
                 scale=0.1, thr=0.0, splits=0, o=FAKE, lse=None, map=None, stride=5, stream=None)
        a.update(kw)
        return lib.attn_decode_paged_noalloc(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["B"], a["Hq"], a["Hkv"],
                                             a["D"], a["page"], a["pages"], a["maxp"], a["scale"], a["thr"],
                                             a["splits"], a["o"], a["lse"], a["map"], a["stride"], a["stream"])
    assert _lib.NOALLOC_SCRATCH_BYTES == 64 << 20
    assert call(B=-1) == INVALID
    assert call(scale=0.0) == INVALID
    assert call(thr=0.1, splits=32) == INVALID
    assert call(D=64) == UNSUPPORTED
    assert call(q=None) == INVALID
    assert call(B=0) == _lib.ATTN_OK
    # 128 x 32 heads x 32 splits x 129 floats = 67.6 MB > 64 MiB; 64 rows fit (33.8 MB)
    assert call(B=128, Hq=32, Hkv=8) == WORKSPACE
    assert b"scratch" in lib.attn_last_error_message()
    assert call(B=64, Hq=32, Hkv=8, splits=64) == WORKSPACE


def test_attn_log_prints_rejections(lib, capfd, monkeypatch):
    """ATTN_LOG=1 prints every rejected call's reason to stderr (and every launch, on a GPU); unset, the
    library prints nothing.  The variable is read on every call."""
    monkeypatch.delenv("ATTN_LOG", raising=False)
    assert _decode(lib, B=-1) == INVALID
    assert capfd.readouterr().err == ""
    monkeypatch.setenv("ATTN_LOG", "1")
    assert _decode(lib, D=64) == UNSUPPORTED
    assert _prefill(lib, thr=2.0) == INVALID
    err = capfd.readouterr().err
    assert "[attn] rejected (status 2): attn_decode_paged: D = 64" in err
    assert "[attn] rejected (status 1): attn_prefill_varlen: skip_threshold" in err
    monkeypatch.setenv("ATTN_LOG", "0")
    assert _decode(lib, B=-1) == INVALID
    assert capfd.readouterr().err == ""


def test_attn_check_runs_after_the_host_checks(lib, monkeypatch):
    """With ATTN_CHECK=1 the host-side validation still comes first: a call it rejects returns its
    status without touching the device (so this runs without a GPU)."""
    monkeypatch.setenv("ATTN_CHECK", "1")
    assert _decode(lib, B=-1) == INVALID
    assert _decode(lib, wsb=100) == WORKSPACE
    assert _prefill(lib, D=96) == UNSUPPORTED
    assert _small(lib, ms=17) == INVALID
    assert _decode(lib, B=0) == _lib.ATTN_OK
