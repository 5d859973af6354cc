"""ctypes marshalling for the C oracle in iir_oracle.c (test infrastructure only).

The functions take numpy arrays on the host, check shapes and dtypes, and call the C code. They do
no arithmetic of the method themselves. ``OracleLib(path)`` wraps any build of iir_oracle.c (the
mutation tests load deliberately broken copies); the module-level functions use the real build.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "iir_oracle.c")
_LIB = os.path.join(_HERE, "libiir_oracle.so")
_lock = threading.Lock()
_default = None

# Plain build: no fast-math, no FMA contraction, so the host doubles are IEEE-exact per operation.
CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math"]


class OracleError(RuntimeError):
    pass


def library_path() -> str:
    return _LIB


def compile_source(src: str, out: str) -> str:
    """Compile a C source file with the oracle's flags into a shared library at ``out``."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile iir_oracle.c into libiir_oracle.so next to it."""
    global _default
    with _lock:
        if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
            compile_source(SOURCE, _LIB)
            _default = None
    return _LIB


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str):
    if rc != 0:
        raise OracleError(f"{what} failed with code {rc}")


def _dtype(bpc: int):
    if bpc == 8:
        return np.uint8
    if 9 <= bpc <= 16:
        return np.uint16
    raise OracleError(f"bpc must be 8 to 16, got {bpc}")


def _plane(a: np.ndarray, bpc: int) -> np.ndarray:
    a = np.asarray(a)
    if a.ndim != 2 or a.dtype != _dtype(bpc):
        raise OracleError(f"expected a 2-D {_dtype(bpc).__name__} plane, got {a.dtype} {a.shape}")
    return np.ascontiguousarray(a)


class OracleLib:
    """One loaded build of iir_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.iiro_taps.argtypes = [vp]
        lib.iiro_sse.argtypes = [vp, i64, vp, i64, i32, i32, i32, vp]
        lib.iiro_blur.argtypes = [vp, i64, i32, i32, i32, vp, i64]
        lib.iiro_sad.argtypes = [vp, vp, i32, i32, vp]
        lib.iiro_clip.argtypes = [vp] * 6 + [i32, i32, i32, i32, vp, vp, vp, vp]
        lib.iiro_scores.argtypes = [i32, i32, i32, vp, i32, vp]
        lib.iiro_moments.argtypes = [vp, i64, i32, i32, i32, vp]
        lib.iiro_motion2.argtypes = [vp, i32, vp]
        lib.iiro_aggregate.argtypes = [i32, i32, i32, vp, vp, i32, vp]
        lib.iiro_diff_blur.argtypes = [vp, vp, i64, i32, i32, i32, vp, i64]
        lib.iiro_clip_v2.argtypes = [vp] * 6 + [i32, i32, i32, i32, vp, vp, vp]
        for f in (lib.iiro_taps, lib.iiro_sse, lib.iiro_blur, lib.iiro_sad, lib.iiro_clip,
                  lib.iiro_scores, lib.iiro_moments, lib.iiro_motion2, lib.iiro_aggregate,
                  lib.iiro_diff_blur, lib.iiro_clip_v2):
            f.restype = ctypes.c_int
        self.path = path
        self._lib = lib

    def taps(self) -> np.ndarray:
        g = np.zeros(5, dtype=np.int32)
        _check(self._lib.iiro_taps(_ptr(g)), "taps")
        return g

    def sse(self, ref: np.ndarray, dist: np.ndarray, bpc: int) -> int:
        r, d = _plane(ref, bpc), _plane(dist, bpc)
        if r.shape != d.shape:
            raise OracleError("ref and dist shapes differ")
        out = np.zeros(1, dtype=np.uint64)
        h, w = r.shape
        _check(self._lib.iiro_sse(_ptr(r), r.strides[0], _ptr(d), d.strides[0], w, h, bpc,
                                  _ptr(out)), "sse")
        return int(out[0])

    def blur(self, plane: np.ndarray, bpc: int) -> np.ndarray:
        x = _plane(plane, bpc)
        h, w = x.shape
        out = np.zeros((h, w), dtype=np.uint16)
        _check(self._lib.iiro_blur(_ptr(x), x.strides[0], w, h, bpc, _ptr(out), w), "blur")
        return out

    def sad(self, a: np.ndarray, b: np.ndarray) -> int:
        a = np.ascontiguousarray(a, dtype=np.uint16)
        b = np.ascontiguousarray(b, dtype=np.uint16)
        if a.shape != b.shape or a.ndim != 2:
            raise OracleError("sad needs two equal 2-D planes")
        out = np.zeros(1, dtype=np.uint64)
        _check(self._lib.iiro_sad(_ptr(a), _ptr(b), a.shape[1], a.shape[0], _ptr(out)), "sad")
        return int(out[0])

    def clip(self, ref, dist, bpc: int, prev_blur: np.ndarray | None = None,
             want_last_blur: bool = False):
        """Run a clip. ref and dist are (Y, U, V) tuples of (F, H, W) / (F, Hc, Wc) arrays.

        Returns (sums, has_motion[, last_blur]) with sums an (F, 4) uint64 array of
        {SAD, SSE_Y, SSE_U, SSE_V}.
        """
        dt = _dtype(bpc)
        planes = [np.ascontiguousarray(p) for p in (*ref, *dist)]
        for p in planes:
            if p.dtype != dt or p.ndim != 3:
                raise OracleError("clip planes must be 3-D arrays of the bit depth's dtype")
        f, h, w = planes[0].shape
        hc, wc = (h + 1) // 2, (w + 1) // 2
        for i, p in enumerate(planes):
            want = (f, h, w) if i % 3 == 0 else (f, hc, wc)
            if p.shape != want:
                raise OracleError(f"plane {i} has shape {p.shape}, expected {want}")
        out = np.zeros((f, 4), dtype=np.uint64)
        hm = np.zeros(f, dtype=np.int32)
        pb = None
        if prev_blur is not None:
            pb = np.ascontiguousarray(prev_blur, dtype=np.uint16)
            if pb.shape != (h, w):
                raise OracleError("prev_blur must be an (H, W) uint16 plane")
        last = np.zeros((h, w), dtype=np.uint16) if want_last_blur else None
        rc = self._lib.iiro_clip(*[_ptr(p) for p in planes], f, w, h, bpc,
                                 _ptr(pb) if pb is not None else None, _ptr(out), _ptr(hm),
                                 _ptr(last) if last is not None else None)
        _check(rc, "clip")
        if want_last_blur:
            return out, hm, last
        return out, hm

    def diff_blur(self, prev: np.ndarray, cur: np.ndarray, bpc: int) -> np.ndarray:
        """Motion v2 filter F of prev - cur, an (H, W) int32 array."""
        p, c = _plane(prev, bpc), _plane(cur, bpc)
        if p.shape != c.shape or p.strides != c.strides:
            raise OracleError("prev and cur must be planes of one shape")
        h, w = p.shape
        out = np.zeros((h, w), dtype=np.int32)
        _check(self._lib.iiro_diff_blur(_ptr(p), _ptr(c), p.strides[0], w, h, bpc, _ptr(out), w),
               "diff_blur")
        return out

    def clip_v2(self, ref, dist, bpc: int, prev_luma: np.ndarray | None = None):
        """Run a clip with motion v2: (sums (F, 4) uint64 {SAD2, SSE_Y, SSE_U, SSE_V},
        has_motion). prev_luma is the reference luma of the frame before the clip, if any."""
        dt = _dtype(bpc)
        planes = [np.ascontiguousarray(p) for p in (*ref, *dist)]
        for p in planes:
            if p.dtype != dt or p.ndim != 3:
                raise OracleError("clip planes must be 3-D arrays of the bit depth's dtype")
        f, h, w = planes[0].shape
        hc, wc = (h + 1) // 2, (w + 1) // 2
        for i, p in enumerate(planes):
            want = (f, h, w) if i % 3 == 0 else (f, hc, wc)
            if p.shape != want:
                raise OracleError(f"plane {i} has shape {p.shape}, expected {want}")
        pl = None
        if prev_luma is not None:
            pl = np.ascontiguousarray(prev_luma)
            if pl.dtype != dt or pl.shape != (h, w):
                raise OracleError("prev_luma must be an (H, W) plane of the bit depth's dtype")
        out = np.zeros((f, 4), dtype=np.uint64)
        hm = np.zeros(f, dtype=np.int32)
        _check(self._lib.iiro_clip_v2(*[_ptr(p) for p in planes], f, w, h, bpc,
                                      _ptr(pl) if pl is not None else None, _ptr(out), _ptr(hm)),
               "clip_v2")
        return out, hm

    def scores(self, w: int, h: int, bpc: int, sums, has_motion: int) -> dict:
        s = np.ascontiguousarray(np.asarray(sums, dtype=np.uint64).reshape(4))
        out = np.zeros(7, dtype=np.float64)
        _check(self._lib.iiro_scores(w, h, bpc, _ptr(s), int(has_motion), _ptr(out)), "scores")
        return {"motion": float(out[0]), "mse": [float(x) for x in out[1:4]],
                "psnr": [float(x) for x in out[4:7]]}

    def moments(self, plane: np.ndarray, bpc: int):
        """(sum x, sum x^2) of one plane."""
        p = _plane(plane, bpc)
        out = np.zeros(2, dtype=np.uint64)
        _check(self._lib.iiro_moments(_ptr(p), p.strides[0], p.shape[1], p.shape[0], bpc,
                                      _ptr(out)), "moments")
        return int(out[0]), int(out[1])

    def motion2(self, motion) -> np.ndarray:
        m = np.ascontiguousarray(np.asarray(motion, dtype=np.float64).reshape(-1))
        out = np.zeros_like(m)
        _check(self._lib.iiro_motion2(_ptr(m), m.size, _ptr(out)), "motion2")
        return out

    def aggregate(self, w: int, h: int, bpc: int, sums, has_motion) -> dict:
        s = np.ascontiguousarray(np.asarray(sums, dtype=np.uint64).reshape(-1, 4))
        hm = np.ascontiguousarray(np.asarray(has_motion, dtype=np.int32).reshape(-1))
        out = np.zeros(5, dtype=np.float64)
        _check(self._lib.iiro_aggregate(w, h, bpc, _ptr(s), _ptr(hm), s.shape[0], _ptr(out)),
               "aggregate")
        return {"apsnr": [float(x) for x in out[:3]], "mean_motion": float(out[3]),
                "mean_motion2": float(out[4])}


def default() -> OracleLib:
    """The real oracle, built on first use if the library is missing or stale."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(SOURCE):
            build(force=False)
        with _lock:
            if _default is None:
                _default = OracleLib(_LIB)
    return _default


def taps():
    return default().taps()


def sse(ref, dist, bpc):
    return default().sse(ref, dist, bpc)


def blur(plane, bpc):
    return default().blur(plane, bpc)


def sad(a, b):
    return default().sad(a, b)


def clip(ref, dist, bpc, prev_blur=None, want_last_blur=False):
    return default().clip(ref, dist, bpc, prev_blur, want_last_blur)


def scores(w, h, bpc, sums, has_motion):
    return default().scores(w, h, bpc, sums, has_motion)


def diff_blur(prev, cur, bpc):
    return default().diff_blur(prev, cur, bpc)


def clip_v2(ref, dist, bpc, prev_luma=None):
    return default().clip_v2(ref, dist, bpc, prev_luma)


def moments(plane, bpc):
    return default().moments(plane, bpc)


def motion2(motion):
    return default().motion2(motion)


def aggregate(w, h, bpc, sums, has_motion):
    return default().aggregate(w, h, bpc, sums, has_motion)
