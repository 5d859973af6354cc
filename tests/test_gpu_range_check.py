"""GPU tests of the debug input-range check (IIR_FLAG_CHECK_RANGE), through the C ABI.

At 9 to 15 bits a sample >= 2^bpc anywhere inside a plane's width makes iir_collect return
IIR_ERANGE (the results are still returned), naming the frame and the plane; samples past the
width (pitch padding) are never looked at. Clean input gives exactly the sums of an unchecked
context, which equal the oracle's.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
import integer_image_reductions_amd as iir

pytestmark = pytest.mark.gpu

PLANES = ["ref Y", "ref U", "ref V", "dist Y", "dist U", "dist V"]


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _upload_dirty_padding(arrays):
    """Like iir.upload_planes, but the pitch padding of every row holds 0xFFFF (or 0xFF)."""
    out = []
    for a in arrays:
        w = a.shape[-1]
        per = iir.PLANE_ALIGN // a.dtype.itemsize
        wp = -(-w // per) * per + per  # at least one whole group of padding
        if a.dtype == np.uint8:
            buf = torch.full(a.shape[:-1] + (wp,), 255, dtype=torch.uint8, device="cuda")
            buf[..., :w].copy_(torch.from_numpy(np.ascontiguousarray(a)))
        else:
            buf = torch.full(a.shape[:-1] + (wp,), -1, dtype=torch.int16, device="cuda")
            buf[..., :w].copy_(torch.from_numpy(np.ascontiguousarray(a).view(np.int16)))
        out.append(buf[..., :w])
    return tuple(out)


def _want(clip):
    base, hm = oracle.clip(clip.ref, clip.dist, clip.bpc)
    return np.asarray(base, np.uint64), hm


@pytest.mark.parametrize("bpc", [10, 12])
@pytest.mark.parametrize("w,h", [(131, 17), (512, 48), (3, 3)])
def test_clean_input_passes_with_dirty_padding(w, h, bpc):
    clip = synth.random_clip(w, h, bpc, 3, seed=40 + w + h + bpc, kind="extreme")
    ref, dist = _upload_dirty_padding(clip.ref), _upload_dirty_padding(clip.dist)
    _say("range clean", w, h, bpc)
    with iir.Context(w, h, bpc, max_batch=4, check_range=True) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    want, want_hm = _want(clip)
    assert np.array_equal(sums, want) and list(hm) == list(want_hm)


@pytest.mark.parametrize("bpc", [10, 12, 15])
@pytest.mark.parametrize("plane", range(6))
def test_one_bad_sample_is_named(plane, bpc):
    w, h, f = 131, 17, 4
    clip = synth.random_clip(w, h, bpc, f, seed=7 * plane + bpc, kind="uniform")
    arrs = [np.array(a) for a in clip.ref + clip.dist]
    bad_t = 2
    a = arrs[plane]
    a[bad_t, a.shape[1] - 1, a.shape[2] - 1] = 1 << bpc  # the last sample inside the width
    ref, dist = iir.upload_planes(arrs[:3]), iir.upload_planes(arrs[3:])
    _say("range bad", plane, bpc)
    with iir.Context(w, h, bpc, max_batch=f, check_range=True) as ctx:
        with pytest.raises(iir.IIRError) as ei:
            ctx.run_clip(ref, dist)
        e = ei.value
        assert e.code == iir.IIR_ERANGE
        assert f"frame {bad_t} of its launch" in str(e) and PLANES[plane] in str(e)
        sums, hm = e.results
        assert sums.shape[0] == f
        # frames before the bad one are untouched by it
        want, want_hm = _want(clip)
        assert np.array_equal(sums[:bad_t], want[:bad_t])
        # the context stays usable: after a reset, clean frames pass
        ctx.reset()
        clean_ref, clean_dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
        sums, hm = ctx.run_clip(clean_ref, clean_dist)
        assert np.array_equal(sums, want) and list(hm) == list(want_hm)


def test_limit_is_exactly_two_to_the_bpc():
    w, h, bpc = 64, 8, 12
    clip = synth.random_clip(w, h, bpc, 2, seed=3)
    for value, bad in ((4095, False), (4096, True), (65535, True)):
        arrs = [np.array(a) for a in clip.ref + clip.dist]
        arrs[0][1, 3, 5] = value
        ref, dist = iir.upload_planes(arrs[:3]), iir.upload_planes(arrs[3:])
        _say("range limit", value)
        with iir.Context(w, h, bpc, max_batch=2, check_range=True) as ctx:
            if bad:
                with pytest.raises(iir.IIRError) as ei:
                    ctx.run_clip(ref, dist)
                assert ei.value.code == iir.IIR_ERANGE and "ref Y" in str(ei.value)
            else:
                ctx.run_clip(ref, dist)


def test_streaming_names_the_right_result_and_later_frames_pass():
    w, h, bpc, f = 96, 20, 10, 6
    clip = synth.random_clip(w, h, bpc, f, seed=11)
    arrs = [np.array(a) for a in clip.ref + clip.dist]
    arrs[4][3, 0, 0] = 1023 + 1  # dist U of frame 3
    ref, dist = iir.upload_planes(arrs[:3]), iir.upload_planes(arrs[3:])
    want, want_hm = _want(clip)
    _say("range streaming")
    with iir.Context(w, h, bpc, max_batch=f, check_range=True) as ctx:
        for t in range(f):
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        s1, _ = ctx.collect(2)  # frames 0-1: clean
        assert np.array_equal(s1, want[:2])
        with pytest.raises(iir.IIRError) as ei:
            ctx.collect()
        assert ei.value.code == iir.IIR_ERANGE
        assert "result 1 (frame 0 of its launch): dist U" in str(ei.value)
        sums, hm = ei.value.results
        assert sums.shape[0] == f - 2 and np.array_equal(sums[0], want[2])


def test_frame_table_path_is_checked():
    """Frames at unrelated addresses go through the descriptor table; the check reads it too."""
    w, h, bpc, f = 70, 9, 10, 3
    clip = synth.random_clip(w, h, bpc, f, seed=5)
    rf, df = [], []
    for t in range(f):
        planes = [np.array(a[t]) for a in clip.ref + clip.dist]
        if t == 1:
            planes[5][2, 1] = 2000  # dist V
        rf.append(iir.upload_planes(planes[:3]))
        df.append(iir.upload_planes(planes[3:]))
    _say("range table")
    with iir.Context(w, h, bpc, max_batch=f, check_range=True) as ctx:
        ctx.submit_frames(rf, df)
        with pytest.raises(iir.IIRError) as ei:
            ctx.collect()
    assert ei.value.code == iir.IIR_ERANGE and "frame 1 of its launch): dist V" in str(ei.value)


@pytest.mark.parametrize("bpc", [8, 10, 16])
def test_check_kernel_runs_only_where_values_can_be_invalid(bpc):
    """At 8 and 16 bits every stored value is a sample: the flag is accepted and no check kernel
    runs; at 10 bits one runs before the frames kernel. The sums are the unchecked ones."""
    w, h = 64, 12
    clip = synth.random_clip(w, h, bpc, 2, seed=bpc, kind="extreme")
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    _say("range kernels", bpc)
    with iir.Context(w, h, bpc, max_batch=2, check_range=True) as ctx:
        ctx.run_clip(ref, dist)  # warm
        ctx.reset()
        torch.cuda.synchronize()
        with torch.profiler.profile(activities=[torch.profiler.ProfilerActivity.CUDA]) as prof:
            sums, hm = ctx.run_clip(ref, dist)
            torch.cuda.synchronize()
    names = [e.name for e in prof.events() if e.device_type == torch.autograd.DeviceType.CUDA]
    if not names:
        pytest.skip("the PyTorch profiler recorded no device activity here")
    checks = sum("check_range" in n for n in names)
    assert checks == (1 if bpc == 10 else 0), names
    assert sum("frames_kernel" in n for n in names) == 1, names
    want, want_hm = _want(clip)
    assert np.array_equal(sums, want) and list(hm) == list(want_hm)


@pytest.mark.parametrize("moments,motion_v2", [(True, False), (False, True), (True, True)])
def test_check_with_other_flags(moments, motion_v2):
    """The check runs before the frames kernel whatever that kernel sums: clean input gives the
    sums of a context without the check."""
    w, h, bpc, f = 200, 30, 10, 3
    clip = synth.random_clip(w, h, bpc, f, seed=17)
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    _say("range flags", moments, motion_v2)
    kw = dict(max_batch=f, moments=moments, motion_v2=motion_v2)
    with iir.Context(w, h, bpc, **kw) as ctx:
        want, want_hm = ctx.run_clip(ref, dist)
    with iir.Context(w, h, bpc, check_range=True, **kw) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    assert np.array_equal(sums, want) and list(hm) == list(want_hm)
