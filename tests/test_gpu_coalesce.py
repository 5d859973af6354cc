"""GPU tests of opt-in submission coalescing (iir_set_coalesce), through the C ABI.

With K > 1, one-frame submissions are recorded on the host and enqueued K at a time as one launch.
Every sum must equal the oracle's exactly as without coalescing; collect, reset, export and
submit_clip first enqueue what is recorded; a recorded frame counts as pending.
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


def _want(clip, v2=False):
    base, hm = (oracle.clip_v2 if v2 else oracle.clip)(clip.ref, clip.dist, clip.bpc)
    return np.asarray(base, np.uint64), list(hm)


@pytest.mark.parametrize("bpc", [8, 10])
@pytest.mark.parametrize("k", [2, 3, 8])
@pytest.mark.parametrize("moments,v2", [(False, False), (True, False), (False, True)])
def test_coalesced_stream_equals_oracle(k, bpc, moments, v2):
    w, h, f = 300, 70, 11
    clip = synth.random_clip(w, h, bpc, f, seed=31 * k + bpc, kind="uniform")
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    want, want_hm = _want(clip, v2)
    _say("coalesce", k, bpc, moments, v2)
    with iir.Context(w, h, bpc, max_batch=16, moments=moments, motion_v2=v2, coalesce=k) as ctx:
        for t in range(f):
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        sums, hm = ctx.collect()
    assert np.array_equal(sums[:, :4], want) and list(hm) == want_hm


def test_partial_collect_reset_and_export():
    w, h, f = 257, 40, 9
    clip = synth.random_clip(w, h, 8, f, seed=77)
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    want, want_hm = _want(clip)
    _say("coalesce partial/reset/export")
    with iir.Context(w, h, 8, max_batch=16, coalesce=4) as ctx:
        for t in range(5):  # one launch of 4, one frame recorded
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        s1, h1 = ctx.collect(3)  # enqueues the recorded frame first
        s2, h2 = ctx.collect()
        assert len(s1) == 3 and len(s2) == 2
        assert np.array_equal(np.concatenate([s1, s2]), want[:5])
        # the exported blurred plane is the last submitted frame's, recorded or not
        ctx.submit([p[5] for p in ref], [p[5] for p in dist])
        blur = ctx.export_blur()
        _, _, last = oracle.clip(tuple(p[:6] for p in clip.ref),
                                 tuple(p[:6] for p in clip.dist), 8, want_last_blur=True)
        import torch
        torch.cuda.synchronize()
        assert np.array_equal(blur.cpu().numpy().view(np.uint16), last)
        # a reset first enqueues what is recorded, which still follows frame 4
        ctx.submit([p[6] for p in ref], [p[6] for p in dist])
        ctx.reset()
        ctx.submit([p[7] for p in ref], [p[7] for p in dist])
        ctx.submit([p[8] for p in ref], [p[8] for p in dist])
        sums, hm = ctx.collect()
    assert np.array_equal(sums[:2], want[5:7]) and list(hm[:2]) == [1, 1]
    after, after_hm = _want(synth.Clip("tail", w, h, 8, tuple(p[7:] for p in clip.ref),
                                       tuple(p[7:] for p in clip.dist)))
    assert np.array_equal(sums[2:], after) and list(hm[2:]) == after_hm == [0, 1]


def test_recorded_frames_count_as_pending():
    w, h = 64, 12
    clip = synth.random_clip(w, h, 8, 6, seed=5)
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    _say("coalesce pending")
    with iir.Context(w, h, 8, max_batch=4, coalesce=4) as ctx:
        for t in range(3):
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        with pytest.raises(iir.IIRError) as ei:
            ctx.run_clip(tuple(p[:2] for p in ref), tuple(p[:2] for p in dist))
        assert ei.value.code == iir.binding.IIR_ESTATE
        ctx.submit([p[3] for p in ref], [p[3] for p in dist])  # the fourth: one launch of 4
        with pytest.raises(iir.IIRError) as ei:
            ctx.submit([p[4] for p in ref], [p[4] for p in dist])
        assert ei.value.code == iir.binding.IIR_EBUSY
        sums, hm = ctx.collect()
        assert len(sums) == 4
        for bad in (0, 5):
            with pytest.raises(iir.IIRError):
                ctx.set_coalesce(bad)


def test_pitch_change_sends_the_record_out():
    """A launch takes one set of pitches: a frame with other pitches sends the record out first."""
    w, h, f = 100, 20, 6
    clip = synth.random_clip(w, h, 10, f, seed=9)
    narrow = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    wide = iir.upload_planes(clip.ref, align=256), iir.upload_planes(clip.dist, align=256)
    assert narrow[0][0].stride(-2) != wide[0][0].stride(-2)
    want, want_hm = _want(clip)
    _say("coalesce pitches")
    with iir.Context(w, h, 10, max_batch=8, coalesce=4) as ctx:
        for t in range(f):
            r, d = (wide if t in (2, 3) else narrow)
            ctx.submit([p[t] for p in r], [p[t] for p in d])
        sums, hm = ctx.collect()
    assert np.array_equal(sums, want) and list(hm) == want_hm


def test_dispatches_per_coalesced_launch():
    import torch
    from torch.profiler import ProfilerActivity, profile
    clip = synth.make_clip("c1", 9)
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    _say("coalesce dispatches")
    with iir.Context(clip.width, clip.height, 8, max_batch=16, coalesce=4) as ctx:
        ctx.submit([p[0] for p in ref], [p[0] for p in dist])
        ctx.collect()  # the first launch loads the code
        ctx.reset()
        torch.cuda.synchronize()
        with profile(activities=[ProfilerActivity.CPU, ProfilerActivity.CUDA]) as prof:
            for t in range(9):  # launches of 4 and 4, one frame recorded
                ctx.submit([p[t] for p in ref], [p[t] for p in dist])
            sums, hm = ctx.collect()  # enqueues the ninth
            torch.cuda.synchronize()
    names = [e.name for e in prof.events() if str(e.device_type).endswith("CUDA")]
    if not names:
        pytest.skip("the PyTorch profiler recorded no device activity here")
    assert sum("frames_kernel" in n for n in names) == 3, names
    want, want_hm = _want(synth.Clip("c1", clip.width, clip.height, 8, clip.ref, clip.dist))
    assert np.array_equal(sums, want) and list(hm) == want_hm


def test_range_check_names_the_result_across_coalesced_launches():
    """IIR_FLAG_CHECK_RANGE with coalescing: the error names the collected result that held the
    sample, whichever launch carried it."""
    w, h, f = 96, 20, 7
    clip = synth.random_clip(w, h, 10, f, seed=13)
    arrs = [np.array(a) for a in clip.ref + clip.dist]
    arrs[3][5, 2, 7] = 1024  # dist Y of frame 5, carried by the second launch of 4
    ref, dist = iir.upload_planes(arrs[:3]), iir.upload_planes(arrs[3:])
    _say("coalesce range")
    with iir.Context(w, h, 10, max_batch=8, coalesce=4, check_range=True) as ctx:
        for t in range(f):
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        with pytest.raises(iir.IIRError) as ei:
            ctx.collect()
    assert ei.value.code == iir.IIR_ERANGE
    assert "result 5 (frame 1 of its launch): dist Y" in str(ei.value)
    sums, hm = ei.value.results
    want, _ = _want(clip)
    assert len(sums) == f and np.array_equal(sums[:5], want[:5])
