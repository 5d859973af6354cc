"""Thin ctypes binding of libiir.so (include/iir.h). Argument marshalling only.

Every step of the computation runs in the library's HIP kernels. torch supplies device memory and
the current HIP stream; nothing here computes a sum. The library must have been built
(``python -m integer_image_reductions_amd.build``); loading fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libiir.so")

IIR_OK, IIR_EINVAL, IIR_ENODEV, IIR_ENOMEM, IIR_EDEVICE, IIR_EBUSY, IIR_ESTATE = 0, -1, -2, -3, -4, -5, -6
IIR_ERANGE = -7
IIR_CHROMA_420 = 420
IIR_FLAG_TIMING = 1
IIR_FLAG_MOMENTS = 2
IIR_FLAG_MOTION_V2 = 4
IIR_FLAG_CHECK_RANGE = 8
PLANE_ALIGN = 16  # bytes: plane data and pitch must be multiples of this

c_i32, c_i64, c_u32, c_u64, c_vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                    ctypes.c_uint64, ctypes.c_void_p)


class Plane(ctypes.Structure):
    _fields_ = [("data", c_vp), ("pitch", c_i64), ("width", c_i32), ("height", c_i32)]


class Frame(ctypes.Structure):
    _fields_ = [("plane", Plane * 3)]


class Config(ctypes.Structure):
    _fields_ = [("width", c_i32), ("height", c_i32), ("bpc", c_i32), ("chroma", c_i32),
                ("max_batch", c_i32), ("flags", c_u32)]


class Result(ctypes.Structure):
    _fields_ = [("sad", c_u64), ("sse", c_u64 * 3), ("moment", c_u64 * 4), ("has_motion", c_i32),
                ("reserved", c_i32)]


class Scores(ctypes.Structure):
    _fields_ = [("motion", ctypes.c_double), ("mse", ctypes.c_double * 3),
                ("psnr", ctypes.c_double * 3), ("moment", ctypes.c_double * 4)]


class Aggregate(ctypes.Structure):
    _fields_ = [("sse", c_u64 * 3), ("apsnr", ctypes.c_double * 3),
                ("mean_motion", ctypes.c_double), ("mean_motion2", ctypes.c_double),
                ("frames", c_i32), ("reserved", c_i32)]


class Geometry(ctypes.Structure):
    _fields_ = [("rows_per_tile", c_i32), ("lanes_out", c_i32), ("strips", c_i32),
                ("row_tiles", c_i32), ("tiles", c_i32), ("sum_slots", c_i32),
                ("max_chunks", c_i32)]


class IIRError(RuntimeError):
    """A library call's error code and iir_last_error(). `results` is set where the call still
    returned results (iir_collect's IIR_ERANGE: the (sums, has_motion) of every frame)."""

    def __init__(self, code: int, func: str, detail: str):
        self.code = code
        self.results = None
        super().__init__(f"{func} failed: {detail} (code {code})")


_lib = None

# (name, argtypes, restype) for every function include/iir.h declares
SIGNATURES = [
    ("iir_create", [ctypes.POINTER(Config), c_i32, c_vp, ctypes.POINTER(c_vp)], ctypes.c_int),
    ("iir_submit", [c_vp, ctypes.POINTER(Frame), ctypes.POINTER(Frame)], ctypes.c_int),
    ("iir_submit_clip", [c_vp, ctypes.POINTER(Frame), ctypes.POINTER(Frame), c_i32], ctypes.c_int),
    ("iir_collect", [c_vp, ctypes.POINTER(Result), c_i32, ctypes.POINTER(c_i32)], ctypes.c_int),
    ("iir_run_clip", [c_vp, ctypes.POINTER(Frame), ctypes.POINTER(Frame), c_i32,
                      ctypes.POINTER(Result)], ctypes.c_int),
    ("iir_scores_of", [ctypes.POINTER(Config), ctypes.POINTER(Result), ctypes.POINTER(Scores)],
     ctypes.c_int),
    ("iir_motion2", [ctypes.POINTER(ctypes.c_double), c_i32, ctypes.POINTER(ctypes.c_double)],
     ctypes.c_int),
    ("iir_aggregate_of", [ctypes.POINTER(Config), ctypes.POINTER(Result), c_i32,
                          ctypes.POINTER(Aggregate)], ctypes.c_int),
    ("iir_reset", [c_vp], ctypes.c_int),
    ("iir_set_coalesce", [c_vp, c_i32], ctypes.c_int),
    ("iir_export_blur", [c_vp, c_vp, c_i64], ctypes.c_int),
    ("iir_kernel_time", [c_vp, ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
    ("iir_kernel_stats", [c_vp, c_i32, ctypes.POINTER(c_i64), ctypes.POINTER(ctypes.c_double)],
     ctypes.c_int),
    ("iir_get_geometry", [c_vp, ctypes.POINTER(Geometry)], ctypes.c_int),
    ("iir_plan_chunks", [c_vp, c_i32, ctypes.POINTER(c_i32)], ctypes.c_int),
    ("iir_probe_bandwidth", [c_i32, c_vp, c_i32, c_vp, c_vp, c_i64, c_i32,
                             ctypes.POINTER(ctypes.c_float)], ctypes.c_int),
    ("iir_run_clip_static", [ctypes.POINTER(Config), c_i32, c_vp, ctypes.POINTER(Frame),
                             ctypes.POINTER(Frame), c_i32, ctypes.POINTER(Result)], ctypes.c_int),
    ("iir_destroy", [c_vp], None),
    ("iir_strerror", [ctypes.c_int], ctypes.c_char_p),
    ("iir_last_error", [], ctypes.c_char_p),
]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libiir.so from the package directory, or raise with how to build it."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python -m integer_image_reductions_amd.build` (needs ROCm hipcc)")
    lib = ctypes.CDLL(path)
    for name, args, res in SIGNATURES:
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(rc: int, func: str):
    if rc != IIR_OK:
        lib = load_library()
        detail = lib.iir_last_error().decode() or lib.iir_strerror(rc).decode()
        raise IIRError(rc, func, detail)


def _torch():
    import torch
    return torch


def sample_dtype(bpc: int):
    """torch dtype holding the samples of a bit depth (10-bit: int16 carrying the uint16 bits)."""
    torch = _torch()
    return torch.uint8 if bpc == 8 else torch.int16


def _plane_of(t, width: int, height: int) -> Plane:
    """A 2-D (rows, cols) device tensor with unit column stride, as an iir_plane."""
    if t.dim() != 2 or t.stride(1) != 1 or not t.is_cuda:
        raise ValueError("planes must be 2-D CUDA tensors with contiguous rows")
    return Plane(t.data_ptr(), t.stride(0) * t.element_size(), width, height)


def frame_of(planes, width: int, height: int) -> Frame:
    wc, hc = (width + 1) // 2, (height + 1) // 2
    f = Frame()
    f.plane[0] = _plane_of(planes[0], width, height)
    f.plane[1] = _plane_of(planes[1], wc, hc)
    f.plane[2] = _plane_of(planes[2], wc, hc)
    return f


def upload_planes(arrays, device="cuda", align: int = PLANE_ALIGN):
    """Copy host planes (numpy uint8 / uint16, shape (..., h, w)) into device tensors whose rows
    start on `align`-byte boundaries (padded pitch); returns views of shape (..., h, w). 16-bit
    samples are held in int16 tensors (same bits), so no uint16 torch kernels are needed."""
    torch = _torch()
    out = []
    for a in arrays:
        a = np.ascontiguousarray(a)
        w = a.shape[-1]
        per = align // a.dtype.itemsize
        wp = -(-w // per) * per
        if a.dtype == np.uint8:
            src, dt = torch.from_numpy(a), torch.uint8
        elif a.dtype == np.uint16:
            src, dt = torch.from_numpy(a.view(np.int16)), torch.int16
        else:
            raise ValueError(f"unsupported sample dtype {a.dtype}")
        buf = torch.zeros(a.shape[:-1] + (wp,), dtype=dt, device=device)
        buf[..., :w].copy_(src)
        out.append(buf[..., :w])
    return tuple(out)


class Context:
    """One library context (iir_ctx): a frame geometry, a device and a stream."""

    def __init__(self, width: int, height: int, bpc: int, max_batch: int = 64, device=None,
                 stream=None, timing: bool = False, moments: bool = False,
                 motion_v2: bool = False, check_range: bool = False, coalesce: int = 1):
        torch = _torch()
        lib = load_library()
        self._lib = lib
        dev = torch.device("cuda", torch.cuda.current_device() if device is None else device)
        self.device = dev
        self.stream = stream if stream is not None else torch.cuda.current_stream(dev)
        self.config = Config(width, height, bpc, IIR_CHROMA_420, max_batch,
                             (IIR_FLAG_TIMING if timing else 0) |
                             (IIR_FLAG_MOMENTS if moments else 0) |
                             (IIR_FLAG_MOTION_V2 if motion_v2 else 0) |
                             (IIR_FLAG_CHECK_RANGE if check_range else 0))
        self.moments = bool(moments)
        h = c_vp()
        _check(lib.iir_create(ctypes.byref(self.config), dev.index, c_vp(self.stream.cuda_stream),
                              ctypes.byref(h)), "iir_create")
        self._h = h
        self._keep = []  # tensors referenced by pending submissions
        self._coalesce = 1
        if coalesce != 1:
            self.set_coalesce(coalesce)

    @property
    def width(self):
        return self.config.width

    @property
    def height(self):
        return self.config.height

    @property
    def bpc(self):
        return self.config.bpc

    def close(self):
        if getattr(self, "_h", None):
            self._lib.iir_destroy(self._h)
            self._h = None
            self._keep = []

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def geometry(self) -> dict:
        g = Geometry()
        _check(self._lib.iir_get_geometry(self._h, ctypes.byref(g)), "iir_get_geometry")
        return {k: getattr(g, k) for k, _ in Geometry._fields_ if k != "reserved"}

    def plan_chunks(self, nframes: int) -> int:
        n = c_i32()
        _check(self._lib.iir_plan_chunks(self._h, nframes, ctypes.byref(n)), "iir_plan_chunks")
        return n.value

    def submit(self, ref, dist):
        """Enqueue one frame pair; ref and dist are (Y, U, V) 2-D device tensors."""
        fr = frame_of(ref, self.width, self.height)
        fd = frame_of(dist, self.width, self.height)
        _check(self._lib.iir_submit(self._h, ctypes.byref(fr), ctypes.byref(fd)), "iir_submit")
        self._keep.append((ref, dist))

    def _frames(self, planes):
        n = planes[0].shape[0]
        arr = (Frame * n)()
        for t in range(n):
            arr[t] = frame_of([p[t] for p in planes], self.width, self.height)
        return arr, n

    def prepare_clip(self, ref, dist):
        """Build the frame descriptors of a clip once; pass the result to submit_prepared()."""
        fr, n = self._frames(ref)
        fd, m = self._frames(dist)
        if n != m:
            raise ValueError("ref and dist have different frame counts")
        return (fr, fd, n, ref, dist)

    def submit_prepared(self, prepared):
        fr, fd, n, ref, dist = prepared
        _check(self._lib.iir_submit_clip(self._h, fr, fd, n), "iir_submit_clip")
        self._keep.append((ref, dist))
        return n

    def submit_clip(self, ref, dist):
        """Enqueue a clip; ref and dist are (Y, U, V) device tensors of shape (F, h, w)."""
        return self.submit_prepared(self.prepare_clip(ref, dist))

    def submit_frames(self, ref_frames, dist_frames):
        """Enqueue frames given as lists of (Y, U, V) 2-D device tensors (any addresses)."""
        n = len(ref_frames)
        if n != len(dist_frames):
            raise ValueError("ref and dist have different frame counts")
        fr, fd = (Frame * n)(), (Frame * n)()
        for t in range(n):
            fr[t] = frame_of(ref_frames[t], self.width, self.height)
            fd[t] = frame_of(dist_frames[t], self.width, self.height)
        _check(self._lib.iir_submit_clip(self._h, fr, fd, n), "iir_submit_clip")
        self._keep.append((ref_frames, dist_frames))
        return n

    def _unpack(self, out, n):
        return _unpack_results(out, n, self.moments)

    def collect(self, max_results: int = 1 << 20):
        """Wait for pending work; returns (sums (n, 4) uint64 [SAD, SSE_Y, SSE_U, SSE_V] -- (n, 8)
        with moments, adding [sum ref Y, sum dist Y, sum ref Y^2, sum dist Y^2] --, has_motion
        (n,) int32)."""
        n_cap = min(max_results, self.config.max_batch)
        out = (Result * n_cap)()
        got = c_i32()
        rc = self._lib.iir_collect(self._h, out, n_cap, ctypes.byref(got))
        # at most 64 launches stay pending, each of up to `coalesce` submissions
        keep = 64 * max(self._coalesce, 1)
        if len(self._keep) > keep:
            self._keep = self._keep[-keep:]
        return self._results_or_raise(rc, "iir_collect", out, got.value)

    def run_clip(self, ref, dist):
        """Submit a clip and wait for its sums; same return as collect()."""
        fr, n = self._frames(ref)
        fd, m = self._frames(dist)
        if n != m:
            raise ValueError("ref and dist have different frame counts")
        out = (Result * n)()
        rc = self._lib.iir_run_clip(self._h, fr, fd, n, out)
        return self._results_or_raise(rc, "iir_run_clip", out, n)

    def _results_or_raise(self, rc: int, func: str, out, n: int):
        """The n results in `out`, or IIRError; IIR_ERANGE still returned them, so that error
        carries them as `results`."""
        if rc == IIR_ERANGE:
            try:
                _check(rc, func)
            except IIRError as e:
                e.results = self._unpack(out, n)
                raise
        _check(rc, func)
        return self._unpack(out, n)

    def reset(self):
        _check(self._lib.iir_reset(self._h), "iir_reset")

    def set_coalesce(self, frames: int):
        """Enqueue one-frame submissions `frames` at a time as one launch (1: each on its own)."""
        _check(self._lib.iir_set_coalesce(self._h, frames), "iir_set_coalesce")
        self._coalesce = frames

    def export_blur(self):
        """The blurred reference luma of the last submitted frame, as an (H, W) uint16 tensor
        (an int16 view of the same bits is returned where torch lacks uint16 kernels)."""
        torch = _torch()
        w2 = -(-2 * self.width // 16) * 16
        buf = torch.empty((self.height, w2 // 2), dtype=torch.int16, device=self.device)
        _check(self._lib.iir_export_blur(self._h, c_vp(buf.data_ptr()), w2), "iir_export_blur")
        return buf[:, :self.width]

    def kernel_stats(self, reset: bool = False):
        """(launches, total kernel ms) of collected timed submissions since create / last reset."""
        n, ms = c_i64(), ctypes.c_double()
        _check(self._lib.iir_kernel_stats(self._h, 1 if reset else 0, ctypes.byref(n),
                                          ctypes.byref(ms)), "iir_kernel_stats")
        return n.value, ms.value

    def kernel_time_ms(self) -> float:
        ms = ctypes.c_float()
        _check(self._lib.iir_kernel_time(self._h, ctypes.byref(ms)), "iir_kernel_time")
        return ms.value


# iir_result as a numpy record (the C layout: eight u64, then two i32)
RESULT_DTYPE = np.dtype([("sad", "<u8"), ("sse", "<u8", (3,)), ("moment", "<u8", (4,)),
                         ("has_motion", "<i4"), ("reserved", "<i4")])


def _unpack_results(out, n: int, moments: bool):
    """(sums (n, 4 or 8) uint64, has_motion (n,) int32) from the first n iir_result of `out`."""
    assert ctypes.sizeof(Result) == RESULT_DTYPE.itemsize
    rec = np.frombuffer(out, dtype=RESULT_DTYPE, count=n)
    cols = [rec["sad"][:, None], rec["sse"]] + ([rec["moment"]] if moments else [])
    return np.concatenate(cols, axis=1).astype(np.uint64), rec["has_motion"].astype(np.int32)


STATIC_MAX_FRAMES = 256  # IIR_STATIC_MAX_FRAMES


def run_clip_static(width: int, height: int, bpc: int, ref, dist, moments: bool = False,
                    motion_v2: bool = False, device=None, stream=None):
    """iir_run_clip_static: the sums of a standalone clip with no context (the library allocates
    nothing). ref and dist are (Y, U, V) device tensors of shape (F, h, w), or lists of per-frame
    (Y, U, V) 2-D tensors (any addresses); same return as Context.collect()."""
    torch = _torch()
    lib = load_library()
    dev = torch.device("cuda", torch.cuda.current_device() if device is None else device)
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    cfg = Config(width, height, bpc, IIR_CHROMA_420, 1,
                 (IIR_FLAG_MOMENTS if moments else 0) | (IIR_FLAG_MOTION_V2 if motion_v2 else 0))
    if isinstance(ref, (list, tuple)) and isinstance(ref[0], (list, tuple)):
        n = len(ref)
        fr, fd = (Frame * n)(), (Frame * n)()
        for t in range(n):
            fr[t] = frame_of(ref[t], width, height)
            fd[t] = frame_of(dist[t], width, height)
    else:
        n = ref[0].shape[0]
        fr, fd = (Frame * n)(), (Frame * n)()
        for t in range(n):
            fr[t] = frame_of([p[t] for p in ref], width, height)
            fd[t] = frame_of([p[t] for p in dist], width, height)
    out = (Result * n)()
    _check(lib.iir_run_clip_static(ctypes.byref(cfg), dev.index, c_vp(s.cuda_stream), fr, fd, n,
                                   out), "iir_run_clip_static")
    return _unpack_results(out, n, moments)


def _result(row, has_motion) -> Result:
    r = Result()
    row = [int(v) for v in row]
    r.sad, r.sse[0], r.sse[1], r.sse[2] = row[:4]
    for k, v in enumerate(row[4:8]):
        r.moment[k] = v
    r.has_motion = int(has_motion)
    return r


def scores(width: int, height: int, bpc: int, sums, has_motion: int) -> dict:
    """iir_scores_of for one result row (4 sums, or 8 with moments): {motion, mse[3], psnr[3],
    moment[4]}."""
    lib = load_library()
    cfg = Config(width, height, bpc, IIR_CHROMA_420, 1, 0)
    r = _result(sums, has_motion)
    s = Scores()
    _check(lib.iir_scores_of(ctypes.byref(cfg), ctypes.byref(r), ctypes.byref(s)), "iir_scores_of")
    return {"motion": s.motion, "mse": list(s.mse), "psnr": list(s.psnr),
            "moment": list(s.moment)}


def motion2(motion) -> np.ndarray:
    """iir_motion2: each frame's second motion score from the clip's motion scores."""
    lib = load_library()
    m = np.ascontiguousarray(motion, dtype=np.float64)
    out = np.empty_like(m)
    dp = ctypes.POINTER(ctypes.c_double)
    _check(lib.iir_motion2(m.ctypes.data_as(dp), m.size, out.ctypes.data_as(dp)), "iir_motion2")
    return out


def aggregate(width: int, height: int, bpc: int, sums, has_motion) -> dict:
    """iir_aggregate_of over a clip's results: {sse[3], apsnr[3], mean_motion, mean_motion2}."""
    lib = load_library()
    n = len(sums)
    cfg = Config(width, height, bpc, IIR_CHROMA_420, 1, 0)
    arr = (Result * n)()
    for i in range(n):
        arr[i] = _result(sums[i], has_motion[i])
    a = Aggregate()
    _check(lib.iir_aggregate_of(ctypes.byref(cfg), arr, n, ctypes.byref(a)), "iir_aggregate_of")
    return {"sse": [int(v) for v in a.sse], "apsnr": list(a.apsnr), "mean_motion": a.mean_motion,
            "mean_motion2": a.mean_motion2}


def probe_bandwidth(mode: int, src, dst, iters: int = 20, stream=None) -> float:
    """Mean ms per launch of the memory-ceiling probe (0 read, 1 write, 2 copy) over `nbytes` of
    the given device tensors."""
    torch = _torch()
    lib = load_library()
    nbytes = dst.numel() * dst.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(dst.device)
    ms = ctypes.c_float()
    _check(lib.iir_probe_bandwidth(dst.device.index, c_vp(s.cuda_stream), mode,
                                   c_vp(src.data_ptr() if src is not None else 0),
                                   c_vp(dst.data_ptr()), nbytes, iters, ctypes.byref(ms)),
           "iir_probe_bandwidth")
    return ms.value
