"""iir_run_clip_static, the entry point that allocates nothing, against iir_run_clip.

Each case calls the static entry point twice in a row through the C ABI, the second time with a
smaller clip (fewer frames, a smaller frame), and compares every sum with what iir_run_clip of a
fresh context returns for the same clip (exact equality); the small clips are also checked against
the oracle. The static working memory keeps the previous call's contents, so the second, smaller
call shows that it clears what it must.
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


def _context_sums(clip, moments, motion_v2, ref, dist):
    with iir.Context(clip.width, clip.height, clip.bpc, max_batch=clip.frames, moments=moments,
                     motion_v2=motion_v2) as ctx:
        return ctx.run_clip(ref, dist)


def _per_frame(planes):
    return [tuple(p[t] for p in planes) for t in range(planes[0].shape[0])]


def _one(clip, moments=False, motion_v2=False, table=False):
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    args = (_per_frame(ref), _per_frame(dist)) if table else (ref, dist)
    got, hm = iir.run_clip_static(clip.width, clip.height, clip.bpc, *args, moments=moments,
                                  motion_v2=motion_v2)
    want, want_hm = _context_sums(clip, moments, motion_v2, ref, dist)
    assert list(hm) == list(want_hm)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (bad[0], got[bad[0][0]], want[bad[0][0]])
    if clip.width * clip.height * clip.frames <= 600_000:
        ofn = oracle.clip_v2 if motion_v2 else oracle.clip
        o, o_hm = ofn(clip.ref, clip.dist, clip.bpc)
        assert np.array_equal(got[:, :4], o)
        assert list(hm) == list(o_hm)


CASES = [
    # (first clip, second smaller clip, moments, motion_v2, table)
    (("c1", None), ("rand", 37, 19, 8, 3), False, False, False),
    (("rand", 300, 70, 10, 5), ("rand", 37, 19, 10, 2), False, False, False),
    (("rand", 270, 36, 16, 4), ("rand", 40, 12, 16, 2), True, False, False),
    (("rand", 513, 40, 12, 4), ("rand", 9, 5, 12, 3), True, False, False),
    (("c1", None), ("rand", 64, 5, 8, 2), False, True, False),
    (("rand", 300, 70, 10, 5), ("rand", 37, 19, 10, 2), False, True, False),
    (("rand", 513, 7, 8, 4), ("rand", 17, 23, 8, 3), False, False, True),
    (("c2", 12), ("c1", 5), False, False, False),
    # one 8-bit frame pair per call: the one-frame kernels, without a previous state
    (("rand", 300, 70, 8, 1), ("rand", 257, 40, 8, 1), False, False, False),
    (("rand", 256, 48, 8, 1), ("rand", 64, 12, 8, 1), True, False, False),
]


def _make(spec, seed):
    if spec[0] == "rand":
        _, w, h, bpc, f = spec
        return synth.random_clip(w, h, bpc, f, seed=seed)
    return synth.make_clip(spec[0], spec[1])


@pytest.mark.parametrize("first,second,moments,motion_v2,table", CASES,
                         ids=[f"case{i}" for i in range(len(CASES))])
def test_static_matches_run_clip(first, second, moments, motion_v2, table):
    for i, spec in enumerate((first, second)):
        clip = _make(spec, 4242 + i)
        _say("static", spec, "moments" if moments else "", "v2" if motion_v2 else "",
             "table" if table else "")
        _one(clip, moments, motion_v2, table)


def test_static_rejects_too_many_frames():
    clip = synth.random_clip(16, 8, 8, 1, seed=1)
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    one_r, one_d = _per_frame(ref)[0], _per_frame(dist)[0]
    n = iir.STATIC_MAX_FRAMES + 1
    with pytest.raises(iir.IIRError) as e:
        iir.run_clip_static(16, 8, 8, [one_r] * n, [one_d] * n)
    assert e.value.code == -1
