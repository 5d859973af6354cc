"""GPU parity of motion v2 (IIR_FLAG_MOTION_V2), through the C ABI.

Motion v2 filters the difference prev - cur of consecutive reference luma frames with the same
separable taps (floor shifts) and sums the absolute values. Every sum equals the oracle's
(oracle.clip_v2) exactly: small and ragged clips at 8 to 16 bits, every tile height and path,
streamed frame by frame (the last frame's luma crossing launches), split clips, time chunks, with
moments, the five named workloads at full size, and full-size 4K clips at 15 and 16 bits.
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


def _check(sums, hm, want, want_hm, what):
    assert list(hm) == list(want_hm), what
    bad = np.argwhere(sums != want)
    assert bad.size == 0, f"{what}: first mismatch frame {bad[0][0]} sum {bad[0][1]}: " \
                          f"{sums[bad[0][0]]} vs {want[bad[0][0]]}"


SIZES = [(3, 3), (4, 7), (9, 5), (17, 23), (64, 5), (70, 3), (131, 17), (250, 40), (255, 33),
         (256, 5), (257, 9), (258, 35), (259, 6), (260, 4), (513, 7), (1283, 723)]


@pytest.mark.parametrize("bpc", [8, 10, 12, 15, 16])
@pytest.mark.parametrize("w,h", SIZES, ids=[f"{w}x{h}" for w, h in SIZES])
def test_v2_small(w, h, bpc):
    for i, kind in enumerate(["uniform", "extreme", "checker", "impulse"]):
        frames = 3 if w * h < 200_000 else 2
        clip = synth.random_clip(w, h, bpc, frames, seed=7000 + 3 * w + h + i, kind=kind)
        _say("v2", w, h, bpc, kind)
        ref, dist = _dev(clip)
        with iir.Context(w, h, bpc, max_batch=4, motion_v2=True) as ctx:
            sums, hm = ctx.run_clip(ref, dist)
        want, want_hm = oracle.clip_v2(clip.ref, clip.dist, bpc)
        _check(sums, hm, want, want_hm, f"{kind} {w}x{h} {bpc}")


V2_PATHS = [(504, 36), (1000, 80), (248, 60), (8, 12), (64, 240), (512, 48), (768, 60),
            (257, 40), (513, 24), (512, 50)]


@pytest.mark.parametrize("bpc", [8, 10])
@pytest.mark.parametrize("th", ["12", "16", "20"])
@pytest.mark.parametrize("w,h", V2_PATHS, ids=[f"{w}x{h}" for w, h in V2_PATHS])
def test_v2_each_tile_height_and_path(w, h, th, bpc, monkeypatch):
    monkeypatch.setenv("IIR_ROWS_PER_TILE", th)
    clip = synth.random_clip(w, h, bpc, 3, seed=11 * w + h + int(th), kind="uniform")
    ref, dist = _dev(clip)
    _say("v2 path", w, h, th, bpc)
    with iir.Context(w, h, bpc, max_batch=4, motion_v2=True) as ctx:
        assert ctx.geometry()["rows_per_tile"] == int(th)
        sums, hm = ctx.run_clip(ref, dist)
    want, want_hm = oracle.clip_v2(clip.ref, clip.dist, bpc)
    _check(sums, hm, want, want_hm, f"{w}x{h} th={th} bpc={bpc}")


@pytest.mark.parametrize("bpc", [8, 10, 12, 16])
@pytest.mark.parametrize("w,h", [(300, 70), (512, 48), (257, 33)])
def test_v2_streaming_split_and_chunks(w, h, bpc, monkeypatch):
    """Frame by frame (every frame's previous luma comes from the saved plane of the launch
    before), in two submissions, in one launch, and in time chunks all give the same sums."""
    f = 9
    clip = synth.random_clip(w, h, bpc, f, seed=w + h + bpc, kind="uniform")
    ref, dist = _dev(clip)
    want, want_hm = oracle.clip_v2(clip.ref, clip.dist, bpc)
    _say("v2 streaming", w, h, bpc)
    with iir.Context(w, h, bpc, max_batch=16, motion_v2=True) as ctx:
        for t in range(f):
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        sums, hm = ctx.collect()
        _check(sums, hm, want, want_hm, "streaming")
        ctx.reset()
        ctx.submit_clip(tuple(p[:4] for p in ref), tuple(p[:4] for p in dist))
        ctx.submit_clip(tuple(p[4:] for p in ref), tuple(p[4:] for p in dist))
        sums, hm = ctx.collect()
        _check(sums, hm, want, want_hm, "split")
        with pytest.raises(iir.IIRError) as e:
            ctx.export_blur()
        assert e.value.code == -6
    monkeypatch.setenv("IIR_TARGET_WAVES", "100000")
    monkeypatch.setenv("IIR_MIN_CHUNK", "2")
    _say("v2 chunks", w, h, bpc)
    with iir.Context(w, h, bpc, max_batch=16, motion_v2=True) as ctx:
        assert ctx.plan_chunks(f) > 1
        ctx.run_clip(tuple(p[:1] for p in ref), tuple(p[:1] for p in dist))
        sums, hm = ctx.run_clip(tuple(p[1:] for p in ref), tuple(p[1:] for p in dist))
    _check(sums, hm, want[1:], want_hm[1:], "chunks")


@pytest.mark.parametrize("bpc", [8, 10, 12, 15, 16])
@pytest.mark.parametrize("w,h", [(131, 17), (512, 48), (1283, 723)])
def test_v2_with_moments(w, h, bpc):
    clip = synth.random_clip(w, h, bpc, 3, seed=3 * w + h, kind="extreme")
    ref, dist = _dev(clip)
    _say("v2 moments", w, h, bpc)
    with iir.Context(w, h, bpc, max_batch=4, motion_v2=True, moments=True) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    want, want_hm = oracle.clip_v2(clip.ref, clip.dist, bpc)
    _check(sums[:, :4], hm, want, want_hm, f"v2 moments {w}x{h} {bpc}")
    for t in range(3):
        r1, r2 = oracle.moments(clip.ref[0][t], bpc)
        d1, d2 = oracle.moments(clip.dist[0][t], bpc)
        assert [int(v) for v in sums[t, 4:]] == [r1, d1, r2, d2]


@pytest.mark.parametrize("name", ["c1", "c2", "c5", "c3", "c4"])
def test_v2_workload_full(name):
    """Every frame of a named workload at full size with motion v2, in one launch."""
    _say("v2 workload", name, "generate")
    clip = synth.make_clip(name)
    ref, dist = _dev(clip)
    _say("v2 workload", name, "gpu")
    with iir.Context(clip.width, clip.height, clip.bpc, max_batch=clip.frames,
                     motion_v2=True) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    _say("v2 workload", name, "oracle")
    want, want_hm = oracle.clip_v2(clip.ref, clip.dist, clip.bpc)
    _check(sums, hm, want, want_hm, name)


@pytest.mark.parametrize("bpc", [9, 12, 15, 16])
@pytest.mark.parametrize("w,h", V2_PATHS, ids=[f"{w}x{h}" for w, h in V2_PATHS])
def test_v2_deep_tiles(w, h, bpc, monkeypatch):
    """16-bit storage (9 to 16 bits): one kernel, the 12-row tile on every shape; a forced other
    tile height is refused at create."""
    clip = synth.random_clip(w, h, bpc, 3, seed=13 * w + h + bpc, kind="uniform")
    ref, dist = _dev(clip)
    _say("v2 deep", w, h, bpc)
    with iir.Context(w, h, bpc, max_batch=4, motion_v2=True) as ctx:
        assert ctx.geometry()["rows_per_tile"] == 12
        sums, hm = ctx.run_clip(ref, dist)
    want, want_hm = oracle.clip_v2(clip.ref, clip.dist, bpc)
    _check(sums, hm, want, want_hm, f"{w}x{h} bpc={bpc}")
    monkeypatch.setenv("IIR_ROWS_PER_TILE", "16")
    with pytest.raises(iir.IIRError) as e:
        iir.Context(w, h, bpc, max_batch=4, motion_v2=True)
    assert e.value.code == -1


def test_v2_full_4k_15bit():
    """The 4K 16-bit clip halved to 15 bits, every frame, in one launch, with motion v2."""
    _say("v2 4k 15-bit generate")
    clip = synth.make_clip("c6")
    ref_np = tuple(p >> 1 for p in clip.ref)
    dist_np = tuple(p >> 1 for p in clip.dist)
    ref, dist = iir.upload_planes(ref_np), iir.upload_planes(dist_np)
    _say("v2 4k 15-bit gpu")
    with iir.Context(clip.width, clip.height, 15, max_batch=clip.frames, motion_v2=True) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    _say("v2 4k 15-bit oracle")
    want, want_hm = oracle.clip_v2(ref_np, dist_np, 15)
    _check(sums, hm, want, want_hm, "c6 >> 1")


def test_v2_full_4k_16bit():
    """The 4K 16-bit clip, every frame, in one launch, with motion v2 (halved differences)."""
    _say("v2 4k 16-bit generate")
    clip = synth.make_clip("c6")
    ref, dist = _dev(clip)
    _say("v2 4k 16-bit gpu")
    with iir.Context(clip.width, clip.height, 16, max_batch=clip.frames, motion_v2=True) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    _say("v2 4k 16-bit oracle")
    want, want_hm = oracle.clip_v2(clip.ref, clip.dist, 16)
    _check(sums, hm, want, want_hm, "c6")


def test_v2_16bit_extremes():
    """Differences of +-65535 everywhere and in checkerboards: every halved sum at its bound."""
    w, h = 264, 40
    peak = 65535
    yy, xx = np.mgrid[0:h, 0:w]
    chk = (((yy + xx) % 2) * peak).astype(np.uint16)
    frames_y = np.stack([np.full((h, w), peak, np.uint16), np.zeros((h, w), np.uint16), chk,
                         peak - chk, np.full((h, w), peak, np.uint16)])
    hc, wc = (h + 1) // 2, (w + 1) // 2
    cz = np.zeros((5, hc, wc), np.uint16)
    ref_np = (frames_y, cz, cz)
    dist_np = (frames_y[::-1].copy(), cz, cz)
    ref, dist = iir.upload_planes(ref_np), iir.upload_planes(dist_np)
    with iir.Context(w, h, 16, max_batch=5, motion_v2=True) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    want, want_hm = oracle.clip_v2(ref_np, dist_np, 16)
    _check(sums, hm, want, want_hm, "16-bit extremes")
    # flat frames 65535 then 0: every output is 65535 (d 2^(16 - bpc) at 16 bits)
    assert int(sums[1, 0]) == w * h * peak


def test_v2_full_4k_16bit_moments():
    """The 4K 16-bit clip with motion v2 and the luma moments (the generic 16-bit v2 kernel)."""
    _say("v2 4k 16-bit moments generate")
    clip = synth.make_clip("c6")
    ref, dist = _dev(clip)
    _say("v2 4k 16-bit moments gpu")
    with iir.Context(clip.width, clip.height, 16, max_batch=clip.frames, motion_v2=True,
                     moments=True) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
    _say("v2 4k 16-bit moments oracle")
    want, want_hm = oracle.clip_v2(clip.ref, clip.dist, 16)
    _check(sums[:, :4], hm, want, want_hm, "c6 v2 moments")
    for t in range(0, clip.frames, 7):
        r1, r2 = oracle.moments(clip.ref[0][t], 16)
        d1, d2 = oracle.moments(clip.dist[0][t], 16)
        assert [int(v) for v in sums[t, 4:]] == [r1, d1, r2, d2], t


@pytest.mark.parametrize("th", ["12", "16"])
@pytest.mark.parametrize("w,h", [(512, 48), (257, 40), (768, 60)])
def test_v2_moments_10bit_tiles(w, h, th, monkeypatch):
    """10-bit motion v2 with moments has its 12- and 16-row tiles at two wavefronts per SIMD
    (no scratch); each matches the oracle on the fast and the generic path."""
    monkeypatch.setenv("IIR_ROWS_PER_TILE", th)
    clip = synth.random_clip(w, h, 10, 3, seed=5 * w + h + int(th), kind="extreme")
    ref, dist = _dev(clip)
    _say("v2 moments 10-bit", w, h, th)
    with iir.Context(w, h, 10, max_batch=4, motion_v2=True, moments=True) as ctx:
        assert ctx.geometry()["rows_per_tile"] == int(th)
        sums, hm = ctx.run_clip(ref, dist)
    want, want_hm = oracle.clip_v2(clip.ref, clip.dist, 10)
    _check(sums[:, :4], hm, want, want_hm, f"v2 moments 10-bit {w}x{h} th={th}")
    for t in range(3):
        r1, r2 = oracle.moments(clip.ref[0][t], 10)
        d1, d2 = oracle.moments(clip.dist[0][t], 10)
        assert [int(v) for v in sums[t, 4:]] == [r1, d1, r2, d2]


def test_v2_moments_10bit_has_no_20_row_tile(monkeypatch):
    monkeypatch.setenv("IIR_ROWS_PER_TILE", "20")
    with pytest.raises(iir.IIRError) as e:
        iir.Context(512, 40, 10, max_batch=2, motion_v2=True, moments=True)
    assert e.value.code == -1
