"""GPU parity at the bit depths beyond 8 and 10 (9 to 16 bits in 16-bit storage), through the C ABI.

These depths take the 16-bit kernel: samples are scaled to 16 bits by a launch-time shift and the
squares are summed per lane in 64 bits. Every sum equals the oracle's exactly, on small and ragged
clips, on every tile height and path, with moments, and on a full-size 4K 16-bit clip.
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


def _dev(clip):
    return iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)


def _blur_np(ctx):
    b = ctx.export_blur()
    import torch
    torch.cuda.synchronize()
    return b.cpu().numpy().view(np.uint16)


def _check(sums, hm, want, want_hm, what):
    assert list(hm) == list(want_hm), what
    bad = np.argwhere(sums != want)
    assert bad.size == 0, f"{what}: first mismatch frame {bad[0][0]} sum {bad[0][1]}: " \
                          f"{sums[bad[0][0]]} vs {want[bad[0][0]]}"


SIZES = [(3, 3), (9, 5), (17, 23), (64, 5), (131, 17), (255, 33), (257, 9), (260, 4), (513, 7),
         (1283, 723)]


@pytest.mark.parametrize("bpc", [9, 12, 16])
@pytest.mark.parametrize("w,h", SIZES, ids=[f"{w}x{h}" for w, h in SIZES])
def test_depth_small(w, h, bpc):
    for i, kind in enumerate(["uniform", "extreme", "checker"]):
        frames = 3 if w * h < 200_000 else 2
        clip = synth.random_clip(w, h, bpc, frames, seed=9000 + 5 * w + h + i, kind=kind)
        _say("depth", w, h, bpc, kind)
        ref, dist = _dev(clip)
        with iir.Context(w, h, bpc, max_batch=4) as ctx:
            sums, hm = ctx.run_clip(ref, dist)
            blur = _blur_np(ctx)
        want, want_hm, last = oracle.clip(clip.ref, clip.dist, bpc, want_last_blur=True)
        _check(sums, hm, want, want_hm, f"{kind} {w}x{h} {bpc}")
        assert np.array_equal(blur, last), f"blurred plane {kind} {w}x{h} {bpc}"


DEPTH_PATHS = [(504, 36), (512, 48), (257, 40), (512, 50), (768, 60)]


@pytest.mark.parametrize("bpc", [12, 16])
@pytest.mark.parametrize("th", ["12", "16", "20"])
@pytest.mark.parametrize("w,h", DEPTH_PATHS, ids=[f"{w}x{h}" for w, h in DEPTH_PATHS])
def test_depth_each_tile_height_and_path(w, h, th, bpc, monkeypatch):
    monkeypatch.setenv("IIR_ROWS_PER_TILE", th)
    clip = synth.random_clip(w, h, bpc, 3, seed=3 * w + h + int(th) + bpc, kind="uniform")
    ref, dist = _dev(clip)
    _say("depth path", w, h, th, bpc)
    with iir.Context(w, h, bpc, max_batch=4) as ctx:
        assert ctx.geometry()["rows_per_tile"] == int(th)
        sums, hm = ctx.run_clip(ref, dist)
        blur = _blur_np(ctx)
    want, want_hm, last = oracle.clip(clip.ref, clip.dist, bpc, want_last_blur=True)
    _check(sums, hm, want, want_hm, f"{w}x{h} th={th} bpc={bpc}")
    assert np.array_equal(blur, last)


@pytest.mark.parametrize("bpc", [12, 16])
@pytest.mark.parametrize("w,h", [(257, 40), (512, 40), (1283, 723)])
def test_depth_moments(w, h, bpc, monkeypatch):
    """Moments and squared errors at full 16-bit scale, tallest tile: the per-lane 64-bit squares
    and their split wavefront sums stay exact with every sample at the peak."""
    monkeypatch.setenv("IIR_ROWS_PER_TILE", "20")
    for kind in ("uniform", "extreme"):
        clip = synth.random_clip(w, h, bpc, 2, seed=w + h + bpc, kind=kind)
        ref, dist = _dev(clip)
        _say("depth moments", w, h, bpc, kind)
        with iir.Context(w, h, bpc, max_batch=2, moments=True) as ctx:
            sums, hm = ctx.run_clip(ref, dist)
        base, want_hm = oracle.clip(clip.ref, clip.dist, bpc)
        _check(sums[:, :4], hm, base, want_hm, f"{kind} {w}x{h} {bpc}")
        for t in range(2):
            r1, r2 = oracle.moments(clip.ref[0][t], bpc)
            d1, d2 = oracle.moments(clip.dist[0][t], bpc)
            assert [int(v) for v in sums[t, 4:]] == [r1, d1, r2, d2], (kind, t)
    peak = (1 << bpc) - 1
    hc, wc = (h + 1) // 2, (w + 1) // 2
    full = tuple(np.full((2, a, b), peak, np.uint16) for a, b in ((h, w), (hc, wc), (hc, wc)))
    zero = tuple(np.zeros_like(p) for p in full)
    ref, dist = iir.upload_planes(full), iir.upload_planes(zero)
    with iir.Context(w, h, bpc, max_batch=2, moments=True) as ctx:
        sums, _ = ctx.run_clip(ref, dist)
    n, nc = w * h, wc * hc
    assert [int(v) for v in sums[1]] == [0, n * peak ** 2, nc * peak ** 2, nc * peak ** 2,
                                        n * peak, 0, n * peak ** 2, 0]


def test_depth_full_4k():
    """The 4K 16-bit clip at full size, every frame, in the benchmark's launch configuration."""
    _say("depth 4k generate")
    clip = synth.make_clip("c6")
    ref, dist = _dev(clip)
    _say("depth 4k gpu")
    with iir.Context(clip.width, clip.height, clip.bpc, max_batch=clip.frames) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
        blur = _blur_np(ctx)
    _say("depth 4k oracle")
    want, want_hm, last = oracle.clip(clip.ref, clip.dist, clip.bpc, want_last_blur=True)
    _check(sums, hm, want, want_hm, "c6")
    assert np.array_equal(blur, last)


def test_depth_full_4k_moments():
    """The 4K 16-bit clip with the luma moments, every frame, in one launch."""
    _say("depth 4k moments generate")
    clip = synth.make_clip("c6")
    ref, dist = _dev(clip)
    _say("depth 4k moments gpu")
    with iir.Context(clip.width, clip.height, clip.bpc, max_batch=clip.frames, moments=True) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    _say("depth 4k moments oracle")
    want, want_hm = oracle.clip(clip.ref, clip.dist, clip.bpc)
    _check(sums[:, :4], hm, want, want_hm, "c6 moments")
    for t in range(0, clip.frames, 7):
        r1, r2 = oracle.moments(clip.ref[0][t], clip.bpc)
        d1, d2 = oracle.moments(clip.dist[0][t], clip.bpc)
        assert [int(v) for v in sums[t, 4:]] == [r1, d1, r2, d2], t
