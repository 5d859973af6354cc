"""GPU parity at the size limits of the C ABI, through the C ABI.

iir_create accepts frames of 3 to 32768 samples on each side, and iir_submit planes whose rows
times pitch stay below 4 GiB. These cases take each limit one at a time:
- the widest and tallest frames (32768 samples), narrow in the other direction, at every bit
  depth class, plain, with moments and with motion v2;
- planes whose pitch puts their last rows more than 2^31 bytes past the plane's start (row
  offsets near the 4 GiB bound), so the kernels' unsigned 32-bit row offsets are exercised past
  the signed range.
Every sum equals the oracle's exactly, and so does the exported blurred plane where it exists.
"""
import gc
import sys

import numpy as np
import pytest

import oracle
import synth
import integer_image_reductions_amd as iir

pytestmark = pytest.mark.gpu

MAX_SIDE = 32768
SHAPES = [(MAX_SIDE, 3), (MAX_SIDE, 20), (3, MAX_SIDE), (4, MAX_SIDE), (36, MAX_SIDE)]
MODES = ["plain", "moments", "v2"]


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _run(clip, mode, ref, dist):
    moments, v2 = mode == "moments", mode == "v2"
    with iir.Context(clip.width, clip.height, clip.bpc, max_batch=clip.frames,
                     moments=moments, motion_v2=v2) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
        blur = None
        if not v2:
            b = ctx.export_blur()
            import torch
            torch.cuda.synchronize()
            blur = b.cpu().numpy().view(np.uint16)
    return sums, hm, blur


def _compare(clip, mode, sums, hm, blur, what):
    if mode == "v2":
        want, want_hm = oracle.clip_v2(clip.ref, clip.dist, clip.bpc)
    else:
        want, want_hm, last = oracle.clip(clip.ref, clip.dist, clip.bpc, want_last_blur=True)
        assert np.array_equal(blur, last), f"blurred plane {what}"
    assert list(hm) == list(want_hm), what
    assert np.array_equal(sums[:, :4], np.asarray(want, np.uint64)), what
    if mode == "moments":
        for t in range(clip.frames):
            (r1, r2), (d1, d2) = (oracle.moments(p[0][t], clip.bpc) for p in (clip.ref, clip.dist))
            assert tuple(int(x) for x in sums[t, 4:]) == (r1, d1, r2, d2), (what, t)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("bpc", [8, 10, 16])
@pytest.mark.parametrize("w,h", SHAPES, ids=[f"{w}x{h}" for w, h in SHAPES])
def test_largest_side(w, h, bpc, mode):
    clip = synth.random_clip(w, h, bpc, 3, seed=w + 3 * h + bpc, kind="uniform")
    _say("largest side", w, h, bpc, mode)
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    sums, hm, blur = _run(clip, mode, ref, dist)
    _compare(clip, mode, sums, hm, blur, f"{w}x{h} {bpc} {mode}")


# Row pitches (bytes) that put the plane's last row just below the 4 GiB bound: 16384 luma rows
# of 261,888 bytes and 8192 chroma rows of twice that end 4,290,772,992 bytes past the plane start.
BIG_H, BIG_LUMA_PITCH = 16384, 261_888
assert BIG_H * BIG_LUMA_PITCH < 2**32 and (BIG_H // 2) * 2 * BIG_LUMA_PITCH < 2**32


@pytest.mark.parametrize("bpc,w,mode", [(8, 256, "plain"), (8, 300, "v2"), (16, 64, "plain"),
                                        (10, 96, "moments")])
def test_row_offsets_past_2gib(bpc, w, mode):
    """Two frames whose planes span almost 4 GiB each (about 51 GB of device memory in all)."""
    clip = synth.random_clip(w, BIG_H, bpc, 2, seed=4242 + w, kind="uniform")
    _say("row offsets past 2 GiB", bpc, w, mode)
    ref = (iir.upload_planes(clip.ref[:1], align=BIG_LUMA_PITCH)
           + iir.upload_planes(clip.ref[1:], align=2 * BIG_LUMA_PITCH))
    dist = (iir.upload_planes(clip.dist[:1], align=BIG_LUMA_PITCH)
            + iir.upload_planes(clip.dist[1:], align=2 * BIG_LUMA_PITCH))
    item = 1 if bpc == 8 else 2
    assert ref[0].stride(-2) * item == BIG_LUMA_PITCH
    assert ref[1].stride(-2) * item == 2 * BIG_LUMA_PITCH
    try:
        sums, hm, blur = _run(clip, mode, ref, dist)
    finally:
        del ref, dist
        gc.collect()
        import torch
        torch.cuda.empty_cache()
    _compare(clip, mode, sums, hm, blur, f"{w}x{BIG_H} {bpc} {mode} big pitch")
