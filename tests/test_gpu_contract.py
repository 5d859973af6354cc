"""Device-resident contract of a submission, counted on the GPU.

"ADR-1380: The CUDA SpEED twins are device-resident ...", Consequences, counts per frame the
kernel launches, device-to-host copies and stream synchronisations of its extractors, and pins the
design with a contract test (its Neutral / follow-ups item). Here: N iir_submit calls enqueue
exactly N frames-kernel dispatches and no memory copy, and return before the GPU has run them;
the one wait is iir_collect's.
"""
import sys

import numpy as np
import pytest

import oracle
import synth
import integer_image_reductions_amd as iir

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def test_submits_dispatch_once_each_and_copy_nothing():
    import torch
    from torch.profiler import ProfilerActivity, profile
    clip = synth.make_clip("c1", 10)
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    n = 8
    _say("contract: dispatches")
    with iir.Context(clip.width, clip.height, 8, max_batch=16) as ctx:
        ctx.submit([p[0] for p in ref], [p[0] for p in dist])  # first launch loads the code
        ctx.collect()
        ctx.reset()
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CPU, ProfilerActivity.CUDA]) as prof:
            for t in range(n):
                ctx.submit([p[t] for p in ref], [p[t] for p in dist])
            torch.cuda.synchronize()
        sums, hm = ctx.collect()
    events = list(prof.events())
    gpu = [e for e in events if str(e.device_type).endswith("CUDA")]
    if not gpu:
        pytest.skip("the PyTorch profiler recorded no device activity here")
    kernels = [e for e in gpu if "frames_kernel" in e.name]
    copies = [e for e in gpu if "memcpy" in e.name.lower() or "memset" in e.name.lower()]
    assert len(kernels) == n, [e.name for e in gpu]
    assert not copies, [e.name for e in copies]
    want, want_hm = oracle.clip(tuple(p[:n] for p in clip.ref), tuple(p[:n] for p in clip.dist), 8)
    assert np.array_equal(sums, want) and list(hm) == list(want_hm)


def test_submits_do_not_wait():
    import torch
    clip = synth.make_clip("c3", 4)
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    stream = torch.cuda.current_stream()
    _say("contract: no wait")
    with iir.Context(clip.width, clip.height, 8, max_batch=64) as ctx:
        ctx.submit([p[0] for p in ref], [p[0] for p in dist])
        ctx.collect()
        torch.cuda.synchronize()
        # 48 one-frame 4K launches are milliseconds of GPU work; the submits only enqueue them
        for k in range(48):
            t = k % 4
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        pending = not stream.query()
        sums, hm = ctx.collect()
        assert stream.query()
    assert pending
    assert len(sums) == 48 and all(hm)
