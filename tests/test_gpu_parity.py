"""GPU parity: every sum of the HIP path equals the oracle's exactly, through the C ABI.

Small clips span several tiles with ragged tails in both directions; the five named workloads run
at full size in the launch configuration the benchmark uses (one submit_clip per clip), and every
frame of every workload is compared with the oracle.
"""
import math
import os
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


def _oracle(clip, prev_blur=None, last=False):
    return oracle.clip(clip.ref, clip.dist, clip.bpc, prev_blur=prev_blur, want_last_blur=last)


def _blur_np(ctx):
    b = ctx.export_blur()
    import torch
    torch.cuda.synchronize()
    return b.cpu().numpy().view(np.uint16)


def _check(clip, sums, hm, want, want_hm, what):
    assert list(hm) == list(want_hm), what
    bad = np.argwhere(sums != want)
    assert bad.size == 0, f"{what}: first mismatch frame {bad[0][0]} sum {bad[0][1]}: " \
                          f"{sums[bad[0][0]]} vs {want[bad[0][0]]}"


TINY = [(3, 3), (4, 7), (9, 5), (17, 23), (5, 64), (64, 5), (70, 3), (33, 18), (131, 17),
        (250, 40), (255, 33), (256, 5), (257, 9), (258, 35), (259, 6), (260, 4), (500, 17),
        (513, 7), (1283, 723)]


@pytest.mark.parametrize("bpc", [8, 10])
@pytest.mark.parametrize("w,h", TINY, ids=[f"{w}x{h}" for w, h in TINY])
def test_tiny_sweep(w, h, bpc):
    kinds = ["uniform", "extreme", "checker", "impulse"]
    for i, kind in enumerate(kinds):
        frames = 3 if w * h < 200_000 else 2
        clip = synth.random_clip(w, h, bpc, frames, seed=1000 + 7 * w + h + i, kind=kind)
        _say("tiny", w, h, bpc, kind)
        ref, dist = _dev(clip)
        with iir.Context(w, h, bpc, max_batch=8) as ctx:
            sums, hm = ctx.run_clip(ref, dist)
            want, want_hm, last = _oracle(clip, last=True)
            _check(clip, sums, hm, want, want_hm, f"{kind} {w}x{h} {bpc}")
            assert np.array_equal(_blur_np(ctx), last), f"blurred plane {kind} {w}x{h} {bpc}"


@pytest.mark.parametrize("w,h", TINY, ids=[f"{w}x{h}" for w, h in TINY])
def test_tiny_sweep_streamed(w, h):
    """The same tiny shapes submitted one 8-bit frame pair at a time (the one-frame kernels, whose
    state crosses launches), with and without moments."""
    for i, (kind, moments) in enumerate([("uniform", False), ("extreme", True)]):
        clip = synth.random_clip(w, h, 8, 3, seed=2000 + 7 * w + h + i, kind=kind)
        _say("tiny streamed", w, h, kind, moments)
        ref, dist = _dev(clip)
        want, want_hm, last = _oracle(clip, last=True)
        with iir.Context(w, h, 8, max_batch=4, moments=moments) as ctx:
            for t in range(3):
                ctx.submit([p[t] for p in ref], [p[t] for p in dist])
            sums, hm = ctx.collect()
            _check(clip, sums[:, :4], hm, want, want_hm, f"{kind} {w}x{h} streamed")
            assert np.array_equal(_blur_np(ctx), last), f"blurred plane {kind} {w}x{h}"


# 256-column strips: right frame edge at a strip boundary (512, 768), inside the last strip
# (504, 1000, 248, 8, 64), one column past a boundary (257, 513), ragged rows (512x50)
PATH_SIZES = [(504, 36), (1000, 80), (248, 60), (8, 12), (64, 240), (512, 48), (768, 60),
              (257, 40), (513, 24), (512, 50)]


@pytest.mark.parametrize("bpc", [8, 10])
@pytest.mark.parametrize("th", ["12", "16", "20"])
@pytest.mark.parametrize("w,h", PATH_SIZES, ids=[f"{w}x{h}" for w, h in PATH_SIZES])
def test_each_tile_height_and_path(w, h, th, bpc, monkeypatch):
    """Every tile height on sizes where the uniform fast path applies (W % 8 == 0, H a multiple of
    the tile height) and where it does not, across several strips and row tiles."""
    monkeypatch.setenv("IIR_ROWS_PER_TILE", th)
    clip = synth.random_clip(w, h, bpc, 3, seed=w + h + int(th), kind="uniform")
    ref, dist = _dev(clip)
    _say("path", w, h, th, bpc)
    with iir.Context(w, h, bpc, max_batch=4) as ctx:
        assert ctx.geometry()["rows_per_tile"] == int(th)
        sums, hm = ctx.run_clip(ref, dist)
        blur = _blur_np(ctx)
    want, want_hm, last = _oracle(clip, last=True)
    _check(clip, sums, hm, want, want_hm, f"{w}x{h} th={th} bpc={bpc}")
    assert np.array_equal(blur, last)


@pytest.mark.parametrize("bpc", [8, 10, 12])
@pytest.mark.parametrize("moments", [False, True])
@pytest.mark.parametrize("th", ["12", "16", "20"])
@pytest.mark.parametrize("w,h", PATH_SIZES, ids=[f"{w}x{h}" for w, h in PATH_SIZES])
def test_one_frame_launches_each_tile_height_and_path(w, h, th, moments, bpc, monkeypatch):
    """Frames submitted one at a time: at 8 bits the one-frame kernels, which load the previous
    launch's blurred tile behind the frame's own; at 10 and 12 bits the batch kernels with one
    frame. Every tile height, the fast and the generic path, with and without moments, ragged row
    tiles, and frames after a batch and a reset."""
    monkeypatch.setenv("IIR_ROWS_PER_TILE", th)
    f = 4
    clip = synth.random_clip(w, h, bpc, f, seed=3 * w + h + int(th) + bpc, kind="uniform")
    ref, dist = _dev(clip)
    want, want_hm, last = _oracle(clip, last=True)
    if moments:  # the sums, then the sums of squares, of the reference and distorted luma
        mom = np.zeros((f, 4), np.uint64)
        for t in range(f):
            (r1, r2), (d1, d2) = (oracle.moments(c[0][t], bpc) for c in (clip.ref, clip.dist))
            mom[t] = (r1, d1, r2, d2)
        want = np.concatenate([np.asarray(want, np.uint64), mom], axis=1)
    _say("one-frame", w, h, th, moments, bpc)
    with iir.Context(w, h, bpc, max_batch=f, moments=moments) as ctx:
        assert ctx.geometry()["rows_per_tile"] == int(th)
        for t in range(f):
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        sums, hm = ctx.collect()
        _check(clip, sums, hm, want, want_hm, f"streamed {w}x{h} th={th}")
        assert np.array_equal(_blur_np(ctx), last)
        ctx.reset()
        ctx.submit_clip(tuple(p[:2] for p in ref), tuple(p[:2] for p in dist))
        for t in (2, 3):
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        sums, hm = ctx.collect()
        _check(clip, sums, hm, want, want_hm, f"batch then streamed {w}x{h} th={th}")


@pytest.mark.parametrize("bpc", [8, 10])
def test_streaming_equals_batch_equals_split(bpc):
    w, h = 300, 70
    clip = synth.random_clip(w, h, bpc, 9, seed=77, kind="uniform")
    ref, dist = _dev(clip)
    want, want_hm = _oracle(clip)
    _say("streaming/batch/split", bpc)
    with iir.Context(w, h, bpc, max_batch=16) as ctx:
        for t in range(9):
            ctx.submit([p[t] for p in ref], [p[t] for p in dist])
        sums, hm = ctx.collect()
        _check(clip, sums, hm, want, want_hm, "streaming")
    with iir.Context(w, h, bpc, max_batch=16) as ctx:
        ctx.submit_clip(tuple(p[:4] for p in ref), tuple(p[:4] for p in dist))
        ctx.submit_clip(tuple(p[4:] for p in ref), tuple(p[4:] for p in dist))
        sums, hm = ctx.collect()
        _check(clip, sums, hm, want, want_hm, "split")
        # partial collects keep the rest queued
        ctx.reset()
        ctx.submit_clip(ref, dist)
        s1, h1 = ctx.collect(4)
        s2, h2 = ctx.collect()
        assert len(s1) == 4 and len(s2) == 5
        _check(clip, np.concatenate([s1, s2]), np.concatenate([h1, h2]), want, want_hm, "partial")


def test_pipelined_submissions():
    """Several submissions in flight; each collect waits only for what it returns, and the result
    slots wrap around."""
    w, h, f = 128, 36, 11
    clip = synth.random_clip(w, h, 8, f, seed=44)
    ref, dist = _dev(clip)
    want, want_hm = _oracle(clip)
    _say("pipelined")
    got, got_hm = [], []
    part = lambda a, b: (tuple(p[a:b] for p in ref), tuple(p[a:b] for p in dist))  # noqa: E731
    with iir.Context(w, h, 8, max_batch=8, timing=True) as ctx:
        ctx.submit_clip(*part(0, 3))    # slots 0-2
        ctx.submit_clip(*part(3, 7))    # slots 3-6
        s, hm = ctx.collect(3)
        got.append(s); got_hm.append(hm)
        ctx.submit_clip(*part(7, 8))    # slot 7
        ctx.submit_clip(*part(8, 11))   # wraps to slots 0-2
        with pytest.raises(iir.IIRError) as e:
            ctx.submit_clip(*part(0, 1))  # 8 frames pending already
        assert e.value.code == -5
        s, hm = ctx.collect(2)
        got.append(s); got_hm.append(hm)
        s, hm = ctx.collect()
        got.append(s); got_hm.append(hm)
        n, ms = ctx.kernel_stats()
        assert n == 4 and ms > 0
    _check(clip, np.concatenate(got), np.concatenate(got_hm), want, want_hm, "pipelined")


def test_reset_restarts_motion():
    w, h = 64, 40
    clip = synth.random_clip(w, h, 8, 4, seed=5)
    ref, dist = _dev(clip)
    _say("reset")
    with iir.Context(w, h, 8, max_batch=8) as ctx:
        ctx.run_clip(tuple(p[:2] for p in ref), tuple(p[:2] for p in dist))
        ctx.reset()
        sums, hm = ctx.run_clip(tuple(p[2:] for p in ref), tuple(p[2:] for p in dist))
    want, want_hm = _oracle(clip.slice(2, 4))
    _check(clip, sums, hm, want, want_hm, "after reset")


def test_frame_table_path():
    """Frames at unrelated addresses (descriptor table copied to the device)."""
    w, h, f = 260, 50, 6
    clip = synth.random_clip(w, h, 10, f, seed=9, kind="extreme")
    order = [3, 0, 5, 1, 4, 2]
    ref, dist = _dev(clip)
    rf = [tuple(p[t] for p in ref) for t in order]
    df = [tuple(p[t] for p in dist) for t in order]
    perm = clip.__class__(clip.name, w, h, 10, tuple(p[order] for p in clip.ref),
                          tuple(p[order] for p in clip.dist))
    want, want_hm = _oracle(perm)
    _say("table path")
    with iir.Context(w, h, 10, max_batch=8) as ctx:
        ctx.submit_frames(rf, df)
        sums, hm = ctx.collect()
    _check(perm, sums, hm, want, want_hm, "table")


@pytest.mark.parametrize("target", ["1", "100000"])
def test_time_chunks_match(target, monkeypatch):
    """Splitting a clip into time chunks (each re-blurring the frame before it) changes nothing."""
    monkeypatch.setenv("IIR_TARGET_WAVES", target)
    monkeypatch.setenv("IIR_MIN_CHUNK", "2")
    w, h, f = 200, 48, 11
    clip = synth.random_clip(w, h, 8, f, seed=31)
    ref, dist = _dev(clip)
    want, want_hm = _oracle(clip)
    _say("chunks", target)
    with iir.Context(w, h, 8, max_batch=16) as ctx:
        chunks = ctx.plan_chunks(f)
        assert (chunks == 1) == (target == "1")
        ctx.run_clip(tuple(p[:1] for p in ref), tuple(p[:1] for p in dist))
        sums, hm = ctx.run_clip(tuple(p[1:] for p in ref), tuple(p[1:] for p in dist))
    _check(clip, sums, hm, want[1:], want_hm[1:], f"chunks={chunks}")


def test_errors_on_device():
    import torch
    w, h = 64, 32
    clip = synth.random_clip(w, h, 8, 3, seed=2)
    ref, dist = _dev(clip)
    _say("errors")
    with iir.Context(w, h, 8, max_batch=2) as ctx:
        with pytest.raises(iir.IIRError) as e:
            ctx.export_blur()
        assert e.value.code == -6
        with pytest.raises(iir.IIRError) as e:
            ctx.submit_clip(ref, dist)  # 3 > max_batch
        assert e.value.code == -1
        ctx.submit_clip(tuple(p[:2] for p in ref), tuple(p[:2] for p in dist))
        with pytest.raises(iir.IIRError) as e:
            ctx.submit([p[2] for p in ref], [p[2] for p in dist])
        assert e.value.code == -5
        with pytest.raises(iir.IIRError) as e:
            ctx.run_clip(tuple(p[:1] for p in ref), tuple(p[:1] for p in dist))
        assert e.value.code == -6
        ctx.collect()
        # misaligned plane: a view starting one byte in
        bad = torch.zeros((h, w + 16), dtype=torch.uint8, device="cuda")[:, 1:w + 1]
        with pytest.raises(iir.IIRError) as e:
            ctx.submit([bad, ref[1][0], ref[2][0]], [p[0] for p in dist])
        assert e.value.code == -1


def test_empty_submissions():
    """Zero frames is an argument error and launches nothing; a collect with nothing pending
    returns no rows; the context then works as usual."""
    w, h = 64, 32
    clip = synth.random_clip(w, h, 8, 2, seed=3)
    ref, dist = _dev(clip)
    empty = tuple(p[:0] for p in ref), tuple(p[:0] for p in dist)
    _say("empty submissions")
    with iir.Context(w, h, 8, max_batch=4) as ctx:
        sums, hm = ctx.collect()
        assert len(sums) == 0 and len(hm) == 0
        for call in (ctx.submit_clip, ctx.run_clip):
            with pytest.raises(iir.IIRError) as e:
                call(*empty)
            assert e.value.code == iir.binding.IIR_EINVAL
        sums, hm = ctx.collect()
        assert len(sums) == 0
        sums, hm = ctx.run_clip(ref, dist)
    with pytest.raises(iir.IIRError) as e:
        iir.run_clip_static(w, h, 8, *empty)
    assert e.value.code == iir.binding.IIR_EINVAL
    want, want_hm = _oracle(clip)
    _check(clip, sums, hm, want, want_hm, "after empty submissions")

def _score_check(clip, sums, hm):
    for t in range(len(sums)):
        a = iir.scores(clip.width, clip.height, clip.bpc, sums[t], hm[t])
        b = oracle.scores(clip.width, clip.height, clip.bpc, sums[t], hm[t])
        for x, y in [(a["motion"], b["motion"])] + list(zip(a["psnr"] + a["mse"],
                                                             b["psnr"] + b["mse"])):
            assert (x == y) or abs(x - y) <= 1e-12 * abs(y)


@pytest.mark.parametrize("name", ["c1", "c2", "c5", "c3", "c4"])
def test_workload_full(name):
    """Every frame of a named workload, at full size, in the benchmark's launch configuration."""
    _say("workload", name, "generate")
    clip = synth.make_clip(name)
    ref, dist = _dev(clip)
    _say("workload", name, "gpu")
    with iir.Context(clip.width, clip.height, clip.bpc, max_batch=clip.frames) as ctx:
        sums, hm = ctx.run_clip(ref, dist)
        blur = _blur_np(ctx)
    _say("workload", name, "oracle")
    want, want_hm, last = _oracle(clip, last=True)
    _check(clip, sums, hm, want, want_hm, name)
    assert np.array_equal(blur, last)
    _score_check(clip, sums, hm)


def test_bit_depth_invariance_4k():
    """The 10-bit 4K reference is exactly 4x the 8-bit one (same seed), so the two workloads'
    per-frame SADs from the GPU are identical. Both clips are made and run here."""
    n = 8
    sads = []
    for name in ("c3", "c4"):
        _say("bit depth invariance", name)
        clip = synth.make_clip(name, n)
        ref, dist = _dev(clip)
        with iir.Context(clip.width, clip.height, clip.bpc, max_batch=n) as ctx:
            sums, hm = ctx.run_clip(ref, dist)
        assert list(hm) == [0] + [1] * (n - 1)
        sads.append(sums[:, 0])
    assert np.array_equal(sads[0], sads[1])
    assert sads[0][1:].min() > 0  # the clips move, so the identity is not between zeros


@pytest.mark.parametrize("moments", [False, True])
def test_varying_batches_reuse_slots(moments):
    """Consecutive submissions of different lengths on one context: each launch accumulates into
    the slot buffer the launch before cleared, so a clearing that missed rows would leak partial
    sums into later results. Every frame still equals the oracle."""
    w, h = 520, 70
    clip = synth.random_clip(w, h, 8, 40, seed=515, kind="uniform")
    ref, dist = _dev(clip)
    want, want_hm = _oracle(clip)
    _say("varying batches", moments)
    got, got_hm = [], []
    with iir.Context(w, h, 8, max_batch=40, moments=moments) as ctx:
        t = 0
        for n in (7, 2, 13, 1, 9, 3, 5):
            sums, hm = ctx.run_clip(tuple(p[t:t + n] for p in ref), tuple(p[t:t + n] for p in dist))
            got.append(sums[:, :4])
            got_hm.append(hm)
            t += n
    _check(clip, np.concatenate(got), np.concatenate(got_hm), want, want_hm, "varying batches")
