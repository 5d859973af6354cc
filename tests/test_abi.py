"""The C-ABI library without a GPU: exports, argument checks, host-side score derivation."""
import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
import integer_image_reductions_amd as iir
from integer_image_reductions_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    hdr = open(os.path.join(ROOT, "include", "iir.h")).read()
    return re.findall(r"IIR_API\s+[\w\s\*]*?\b(iir_\w+)\s*\(", hdr)


@pytest.fixture(scope="module")
def lib():
    return iir.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(n for n, _, _ in B.SIGNATURES) == sorted(names)


def test_strerror_all_codes(lib):
    for code in range(0, -8, -1):
        assert lib.iir_strerror(code).decode() not in ("", "unknown error")
    assert lib.iir_strerror(-99).decode() == "unknown error"


def _create(lib, **kw):
    cfg = B.Config(kw.get("w", 64), kw.get("h", 32), kw.get("bpc", 8), kw.get("chroma", 420),
                   kw.get("max_batch", 4), kw.get("flags", 0))
    h = ctypes.c_void_p()
    return lib.iir_create(ctypes.byref(cfg), kw.get("device", 0), None, ctypes.byref(h))


@pytest.mark.parametrize("kw", [dict(bpc=7), dict(bpc=17), dict(chroma=444), dict(w=2),
                                dict(h=2), dict(w=40000), dict(max_batch=0),
                                dict(max_batch=70000), dict(flags=16)])
def test_create_rejects_bad_config(lib, kw):
    assert _create(lib, **kw) == B.IIR_EINVAL
    assert lib.iir_last_error().decode()


def test_create_null_out(lib):
    cfg = B.Config(64, 32, 8, 420, 4, 0)
    assert lib.iir_create(ctypes.byref(cfg), 0, None, None) == B.IIR_EINVAL
    assert lib.iir_create(None, 0, None, ctypes.byref(ctypes.c_void_p())) == B.IIR_EINVAL


def test_create_without_device(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert _create(lib) == B.IIR_ENODEV


def test_null_context_calls(lib):
    out = (B.Result * 1)()
    n = ctypes.c_int32()
    f = B.Frame()
    assert lib.iir_submit(None, ctypes.byref(f), ctypes.byref(f)) == B.IIR_EINVAL
    assert lib.iir_submit_clip(None, ctypes.byref(f), ctypes.byref(f), 1) == B.IIR_EINVAL
    assert lib.iir_collect(None, out, 1, ctypes.byref(n)) == B.IIR_EINVAL
    assert lib.iir_run_clip(None, ctypes.byref(f), ctypes.byref(f), 1, out) == B.IIR_EINVAL
    assert lib.iir_reset(None) == B.IIR_EINVAL
    assert lib.iir_set_coalesce(None, 2) == B.IIR_EINVAL
    assert lib.iir_export_blur(None, None, 0) == B.IIR_EINVAL
    assert lib.iir_kernel_time(None, ctypes.byref(ctypes.c_float())) == B.IIR_EINVAL
    assert lib.iir_kernel_stats(None, 0, ctypes.byref(ctypes.c_int64()),
                                ctypes.byref(ctypes.c_double())) == B.IIR_EINVAL
    assert lib.iir_get_geometry(None, ctypes.byref(B.Geometry())) == B.IIR_EINVAL
    assert lib.iir_plan_chunks(None, 1, ctypes.byref(n)) == B.IIR_EINVAL
    lib.iir_destroy(None)


def test_probe_rejects_bad_arguments(lib):
    ms = ctypes.c_float()
    assert lib.iir_probe_bandwidth(0, None, 3, None, None, 4096, 1, ctypes.byref(ms)) == B.IIR_EINVAL
    assert lib.iir_probe_bandwidth(0, None, 0, None, None, 4096, 1, ctypes.byref(ms)) == B.IIR_EINVAL
    assert lib.iir_probe_bandwidth(0, None, 1, None, ctypes.c_void_p(4096), 100, 1,
                                   ctypes.byref(ms)) == B.IIR_EINVAL


def test_scores_of_rejects(lib):
    r, s = B.Result(), B.Scores()
    assert lib.iir_scores_of(None, ctypes.byref(r), ctypes.byref(s)) == B.IIR_EINVAL
    for bpc in (7, 17):
        cfg = B.Config(8, 8, bpc, 420, 1, 0)
        assert lib.iir_scores_of(ctypes.byref(cfg), ctypes.byref(r), ctypes.byref(s)) == B.IIR_EINVAL


def _close(a, b):
    if math.isinf(a) or math.isinf(b):
        return a == b
    return abs(a - b) <= 1e-12 * max(abs(a), abs(b), 1e-300)


@pytest.mark.parametrize("bpc", [8, 10, 12, 16])
def test_scores_match_oracle(bpc):
    """Host score derivation in the library equals the oracle's within 1e-12 relative."""
    r = np.random.default_rng(bpc)
    for w, h in ((3840, 2160), (576, 324), (5, 3), (1283, 723)):
        for _ in range(20):
            sums = [int(v) for v in r.integers(0, 2 ** 40, size=4)]
            if r.random() < 0.2:
                sums[1 + int(r.integers(0, 3))] = 0
            hm = int(r.integers(0, 2))
            a = iir.scores(w, h, bpc, sums, hm)
            b = oracle.scores(w, h, bpc, sums, hm)
            assert _close(a["motion"], b["motion"])
            for c in range(3):
                assert _close(a["mse"][c], b["mse"][c])
                assert _close(a["psnr"][c], b["psnr"][c])


def test_clip_functions_reject(lib):
    dp = ctypes.POINTER(ctypes.c_double)
    m = (ctypes.c_double * 2)()
    assert lib.iir_motion2(None, 2, m) == B.IIR_EINVAL
    assert lib.iir_motion2(m, 0, m) == B.IIR_EINVAL
    assert lib.iir_motion2(ctypes.cast(m, dp), 2, None) == B.IIR_EINVAL
    cfg = B.Config(8, 8, 8, 420, 1, 0)
    r, a = (B.Result * 1)(), B.Aggregate()
    assert lib.iir_aggregate_of(None, r, 1, ctypes.byref(a)) == B.IIR_EINVAL
    assert lib.iir_aggregate_of(ctypes.byref(cfg), r, 0, ctypes.byref(a)) == B.IIR_EINVAL
    assert lib.iir_aggregate_of(ctypes.byref(cfg), r, 1, None) == B.IIR_EINVAL
    bad = B.Config(8, 8, 17, 420, 1, 0)
    assert lib.iir_aggregate_of(ctypes.byref(bad), r, 1, ctypes.byref(a)) == B.IIR_EINVAL


@pytest.mark.parametrize("n", [1, 2, 3, 17, 300])
def test_motion2_matches_oracle(n):
    """The library's motion2 equals the oracle's exactly (min is exact), ties and zeros included."""
    r = np.random.default_rng(n)
    m = r.random(n) * 20.0
    m[r.random(n) < 0.3] = 0.0
    if n > 3:
        m[2] = m[3]
    assert np.array_equal(iir.motion2(m), oracle.motion2(m))


@pytest.mark.parametrize("bpc", [8, 10, 16])
@pytest.mark.parametrize("n", [1, 2, 5, 64])
def test_aggregate_matches_oracle(bpc, n):
    """Clip aggregates: totals exact, apsnr and the motion means within 1e-12 relative of the
    oracle, also with a plane whose error is zero on every frame (+infinity)."""
    r = np.random.default_rng(100 * bpc + n)
    for w, h in ((3840, 2160), (576, 324), (5, 3)):
        sums = r.integers(0, 2 ** 40, size=(n, 4)).astype(np.uint64)
        hm = np.ones(n, np.int32)
        hm[0] = int(r.integers(0, 2))
        if n > 1:
            sums[:, 2] = 0
        a = iir.aggregate(w, h, bpc, sums, hm)
        b = oracle.aggregate(w, h, bpc, sums, hm)
        assert a["sse"] == [int(sums[:, c + 1].sum()) for c in range(3)]
        for c in range(3):
            assert _close(a["apsnr"][c], b["apsnr"][c])
        assert _close(a["mean_motion"], b["mean_motion"])
        assert _close(a["mean_motion2"], b["mean_motion2"])


def test_scores_moments():
    """moment[k] of the scores is the k-th luma moment sum over W * H samples."""
    w, h = 37, 19
    row = [5, 1, 2, 3, 4 * w * h, 7 * w * h, 16 * w * h, 49 * w * h]
    s = iir.scores(w, h, 8, row, 1)
    assert s["moment"] == [4.0, 7.0, 16.0, 49.0]
    assert iir.scores(w, h, 8, row[:4], 1)["moment"] == [0.0, 0.0, 0.0, 0.0]


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    """No fallback: without the built library the binding raises, naming how to build it."""
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(ImportError) as e:
        B.load_library(str(tmp_path / "libiir.so"))
    assert "build" in str(e.value)


def test_static_rejects_before_device_work(lib):
    # argument errors are found on the host before any device is touched
    cfg = B.Config(64, 32, 8, B.IIR_CHROMA_420, 1, 0)
    f = (B.Frame * 1)()
    out = (B.Result * 1)()
    assert lib.iir_run_clip_static(ctypes.byref(cfg), 0, None, f, f, 1, None) == B.IIR_EINVAL
    assert lib.iir_run_clip_static(None, 0, None, f, f, 1, out) == B.IIR_EINVAL
    for n in (0, -1, B.STATIC_MAX_FRAMES + 1):
        assert lib.iir_run_clip_static(ctypes.byref(cfg), 0, None, f, f, n, out) == B.IIR_EINVAL
        assert str(B.STATIC_MAX_FRAMES) in lib.iir_last_error().decode()
    bad = B.Config(64, 32, 7, B.IIR_CHROMA_420, 1, 0)
    assert lib.iir_run_clip_static(ctypes.byref(bad), 0, None, f, f, 1, out) == B.IIR_EINVAL
    # the debug input-range check needs per-submission state the static entry does not keep
    checked = B.Config(64, 32, 10, B.IIR_CHROMA_420, 1, B.IIR_FLAG_CHECK_RANGE)
    assert lib.iir_run_clip_static(ctypes.byref(checked), 0, None, f, f, 1, out) == B.IIR_EINVAL
    assert "IIR_FLAG_CHECK_RANGE" in lib.iir_last_error().decode()


def test_unpack_results_matches_struct():
    # the numpy view of iir_result rows reads the same fields as ctypes
    out = (B.Result * 4)()
    for i in range(4):
        out[i].sad = 3 * i + 1
        out[i].sse[0], out[i].sse[1], out[i].sse[2] = 2 ** 64 - 1 - i, 7 * i, 2 ** 40 + i
        for k in range(4):
            out[i].moment[k] = 100 * i + k
        out[i].has_motion = i % 2
    for moments in (False, True):
        sums, hm = B._unpack_results(out, 3, moments)
        assert sums.shape == (3, 8 if moments else 4) and sums.dtype == np.uint64
        for i in range(3):
            row = [out[i].sad] + list(out[i].sse) + (list(out[i].moment) if moments else [])
            assert [int(v) for v in sums[i]] == row
            assert hm[i] == out[i].has_motion
