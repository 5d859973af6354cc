"""GPU parity of the optional luma moments (IIR_FLAG_MOMENTS) and of the clip functions applied to
GPU results, through the C ABI.

With moments on, every frame returns eight exact sums: SAD, SSE_Y, SSE_U, SSE_V, then the sum and
the sum of squares of the reference and the distorted luma. All eight equal the oracle's: the first
four from its clip function, the moments from its per-plane moment function.
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


def _want(clip, prev_blur=None):
    """(n, 8) oracle sums and has_motion of a clip with moments."""
    base, hm = oracle.clip(clip.ref, clip.dist, clip.bpc, prev_blur=prev_blur)
    n = len(base)
    mom = np.zeros((n, 4), np.uint64)
    for t in range(n):
        r1, r2 = oracle.moments(clip.ref[0][t], clip.bpc)
        d1, d2 = oracle.moments(clip.dist[0][t], clip.bpc)
        mom[t] = (r1, d1, r2, d2)
    return np.concatenate([np.asarray(base, np.uint64), mom], axis=1), hm


def _check(sums, hm, want, want_hm, what):
    assert sums.shape == want.shape, (what, sums.shape, want.shape)
    assert list(hm) == list(want_hm), what
    bad = np.argwhere(sums != want)
    assert bad.size == 0, f"{what}: first mismatch frame {bad[0][0]} sum {bad[0][1]}: " \
                          f"{sums[bad[0][0]]} vs {want[bad[0][0]]}"


def _flat_clip(w, h, bpc, frames, value_ref, value_dist):
    dt = np.uint8 if bpc == 8 else np.uint16
    hc, wc = (h + 1) // 2, (w + 1) // 2
    ref = tuple(np.full((frames, a, b), value_ref, dt) for a, b in ((h, w), (hc, wc), (hc, wc)))
    dist = tuple(np.full((frames, a, b), value_dist, dt) for a, b in ((h, w), (hc, wc), (hc, wc)))
    return synth.Clip(f"flat{w}x{h}", w, h, bpc, ref, dist)


SMALL = [(3, 3), (9, 5), (17, 23), (70, 3), (131, 17), (255, 33), (257, 9), (260, 4), (513, 7),
         (1283, 723)]


@pytest.mark.parametrize("bpc", [8, 10])
@pytest.mark.parametrize("w,h", SMALL, ids=[f"{w}x{h}" for w, h in SMALL])
def test_moments_small(w, h, bpc):
    for i, kind in enumerate(["uniform", "extreme", "impulse"]):
        frames = 3 if w * h < 200_000 else 2
        clip = synth.random_clip(w, h, bpc, frames, seed=5000 + 3 * w + h + i, kind=kind)
        _say("moments", w, h, bpc, kind)
        ref, dist = _dev(clip)
        with iir.Context(w, h, bpc, max_batch=4, moments=True) as ctx:
            sums, hm = ctx.run_clip(ref, dist)
        want, want_hm = _want(clip)
        _check(sums, hm, want, want_hm, f"{kind} {w}x{h} {bpc}")


MOM_PATHS = [(504, 36), (512, 48), (257, 40), (512, 50), (8, 12), (768, 60)]


@pytest.mark.parametrize("bpc", [8, 10])
@pytest.mark.parametrize("th", ["12", "16", "20"])
@pytest.mark.parametrize("w,h", MOM_PATHS, ids=[f"{w}x{h}" for w, h in MOM_PATHS])
def test_moments_each_tile_height_and_path(w, h, th, bpc, monkeypatch):
    monkeypatch.setenv("IIR_ROWS_PER_TILE", th)
    clip = synth.random_clip(w, h, bpc, 3, seed=7 * w + h + int(th), kind="uniform")
    ref, dist = _dev(clip)
    _say("moments path", w, h, th, bpc)
    with iir.Context(w, h, bpc, max_batch=4, moments=True) as ctx:
        assert ctx.geometry()["rows_per_tile"] == int(th)
        sums, hm = ctx.run_clip(ref, dist)
    want, want_hm = _want(clip)
    _check(sums, hm, want, want_hm, f"{w}x{h} th={th} bpc={bpc}")


@pytest.mark.parametrize("bpc", [8, 10])
@pytest.mark.parametrize("w,h", [(512, 40), (513, 41)])
def test_moments_at_peak(w, h, bpc, monkeypatch):
    """Every sample at the peak, tallest tile: the largest per-lane partial sums the kernel
    forms (20 rows x 4 samples of 1023^2 per lane at 10 bits) stay exact."""
    monkeypatch.setenv("IIR_ROWS_PER_TILE", "20")
    peak = (1 << bpc) - 1
    clip = _flat_clip(w, h, bpc, 2, peak, 0)
    ref, dist = _dev(clip)
    _say("moments peak", w, h, bpc)
    with iir.Context(w, h, bpc, max_batch=2, moments=True) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    want, want_hm = _want(clip)
    _check(sums, hm, want, want_hm, f"peak {w}x{h} {bpc}")
    n = w * h
    assert int(sums[0, 4]) == peak * n and int(sums[0, 6]) == peak * peak * n
    assert int(sums[0, 5]) == 0 and int(sums[0, 7]) == 0


def test_moments_streaming_and_chunks(monkeypatch):
    """Moments per frame are the same streamed one frame at a time, in one launch, and in time
    chunks (whose prologue frame is blurred again but must not be counted twice)."""
    w, h, f = 200, 48, 11
    clip = synth.random_clip(w, h, 8, f, seed=91)
    ref, dist = _dev(clip)
    want, want_hm = _want(clip)
    _say("moments streaming")
    with iir.Context(w, h, 8, max_batch=16, moments=True) as ctx:
        for t in range(f):
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        sums, hm = ctx.collect()
    _check(sums, hm, want, want_hm, "streaming")
    monkeypatch.setenv("IIR_TARGET_WAVES", "100000")
    monkeypatch.setenv("IIR_MIN_CHUNK", "2")
    _say("moments chunks")
    with iir.Context(w, h, 8, max_batch=16, moments=True) as ctx:
        assert ctx.plan_chunks(f) > 1
        sums, hm = ctx.run_clip(ref, dist)
    _check(sums, hm, want, want_hm, "chunks")


@pytest.mark.parametrize("name", ["c1", "c2", "c5", "c3", "c4"])
def test_moments_workload_full(name):
    """Every frame of a named workload at full size with moments on; the clip aggregates of the
    GPU sums equal the oracle's aggregates of its own sums."""
    _say("moments workload", name, "generate")
    clip = synth.make_clip(name)
    ref, dist = _dev(clip)
    _say("moments workload", name, "gpu")
    with iir.Context(clip.width, clip.height, clip.bpc, max_batch=clip.frames,
                     moments=True) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    _say("moments workload", name, "oracle")
    want, want_hm = _want(clip)
    _check(sums, hm, want, want_hm, name)
    a = iir.aggregate(clip.width, clip.height, clip.bpc, sums, hm)
    b = oracle.aggregate(clip.width, clip.height, clip.bpc, want[:, :4], want_hm)
    for x, y in list(zip(a["apsnr"], b["apsnr"])) + [(a["mean_motion"], b["mean_motion"]),
                                                      (a["mean_motion2"], b["mean_motion2"])]:
        assert x == y or abs(x - y) <= 1e-12 * abs(y), (name, x, y)
    m = [iir.scores(clip.width, clip.height, clip.bpc, sums[t], hm[t])["motion"]
         for t in range(len(sums))]
    assert np.array_equal(iir.motion2(m), oracle.motion2(m))
