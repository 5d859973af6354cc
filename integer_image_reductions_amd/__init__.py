"""Integer motion (blurred-luma SAD) and PSNR (per-plane SSE) sums on AMD MI355X.

The computation lives in libiir.so (HIP kernels for gfx950 behind the C ABI in include/iir.h);
this package is its Python binding. Import is cheap: the library loads on first use.
"""
from .binding import (  # noqa: F401
    IIR_CHROMA_420,
    IIR_ERANGE,
    IIR_FLAG_CHECK_RANGE,
    IIR_FLAG_MOMENTS,
    IIR_FLAG_MOTION_V2,
    IIR_FLAG_TIMING,
    LIB_PATH,
    PLANE_ALIGN,
    SIGNATURES,
    STATIC_MAX_FRAMES,
    aggregate,
    motion2,
    Context,
    IIRError,
    frame_of,
    load_library,
    probe_bandwidth,
    run_clip_static,
    sample_dtype,
    scores,
    upload_planes,
)
