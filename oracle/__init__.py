"""CPU oracle for the integer motion and PSNR sums (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import this package. The GPU
library never does, and this package never imports the GPU library: the two share no code.

`iir_oracle.c` holds the arithmetic; `oracle.py` builds it with gcc and marshals numpy arrays.
"""
from .oracle import (  # noqa: F401
    SOURCE,
    OracleError,
    OracleLib,
    aggregate,
    blur,
    build,
    clip,
    clip_v2,
    compile_source,
    default,
    diff_blur,
    library_path,
    moments,
    motion2,
    sad,
    scores,
    sse,
    taps,
)
