"""GPU parity on seeded random configurations, through the C ABI.

Each case draws a frame size (3 to 1400 columns, 3 to 300 rows), a bit depth (8, 9, 10, 12, 15 or
16), a clip length, the moments, motion v2 and input-range-check flags, a sample pattern, a
submission pattern (one launch, one frame pair per submission, or two launches) and a coalescing
factor, and compares every sum with the oracle's.
A second set draws shapes on the uniform fast path (W a multiple of 8, H a multiple of the tile
height, which each case forces), where the last strip's tiles hold the frame's right edge whenever
W % 256 != 0.
The draws are fixed by the seed, so a failure names a reproducible case.
"""
import random
import sys

import numpy as np
import pytest

import oracle
import synth
import integer_image_reductions_amd as iir

pytestmark = pytest.mark.gpu


def _cases(seed: int, n: int):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        w = rng.choice([rng.randint(3, 40), rng.randint(41, 700), rng.randint(700, 1400)])
        h = rng.choice([rng.randint(3, 40), rng.randint(41, 300)])
        out.append(dict(w=w, h=h, bpc=rng.choice([8, 8, 10, 12, 16, 9, 15]), f=rng.randint(1, 7),
                        moments=rng.random() < 0.4, v2=rng.random() < 0.3,
                        mode=rng.choice(["batch", "stream", "split"]),
                        kind=rng.choice(["uniform", "extreme", "impulse", "checker"]),
                        seed=rng.randint(0, 10**6), coalesce=rng.choice([1, 1, 2, 3, 5]),
                        check=rng.random() < 0.3))
    return out


CASES = _cases(20261203, 60)


@pytest.mark.parametrize("c", CASES, ids=[f"r{i}" for i in range(len(CASES))])
def test_random_configuration(c):
    print("[case]", c, flush=True)
    sys.stdout.flush()
    w, h, bpc, f = c["w"], c["h"], c["bpc"], c["f"]
    clip = synth.random_clip(w, h, bpc, f, seed=c["seed"], kind=c["kind"])
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    with iir.Context(w, h, bpc, max_batch=8, moments=c["moments"], motion_v2=c["v2"],
                     coalesce=c["coalesce"], check_range=c["check"]) as ctx:
        if c["mode"] == "batch":
            sums, hm = ctx.run_clip(ref, dist)
        elif c["mode"] == "stream":
            for t in range(f):
                ctx.submit([p[t] for p in ref], [p[t] for p in dist])
            sums, hm = ctx.collect()
        else:
            k = max(1, f // 2)
            ctx.submit_clip(tuple(p[:k] for p in ref), tuple(p[:k] for p in dist))
            if f > k:
                ctx.submit_clip(tuple(p[k:] for p in ref), tuple(p[k:] for p in dist))
            sums, hm = ctx.collect()
    want, want_hm = (oracle.clip_v2 if c["v2"] else oracle.clip)(clip.ref, clip.dist, bpc)
    assert np.array_equal(sums[:, :4], np.asarray(want, np.uint64)), c
    assert list(hm) == list(want_hm), c
    if c["moments"]:
        for t in range(f):
            (r1, r2), (d1, d2) = (oracle.moments(p[0][t], bpc) for p in (clip.ref, clip.dist))
            assert tuple(int(x) for x in sums[t, 4:]) == (r1, d1, r2, d2), (c, t)


def _fast_cases(seed: int, n: int):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        bpc = rng.choice([8, 8, 8, 10, 16])
        moments, v2 = rng.random() < 0.4, rng.random() < 0.25
        # 16-bit motion v2 has only the 12-row tile; 10-bit motion v2 with moments the 12- and 16-row
        ths = [12] if bpc == 16 and v2 else [12, 16] if bpc == 10 and v2 and moments else [12, 16, 20]
        th = rng.choice(ths)
        out.append(dict(w=8 * rng.choice([rng.randint(1, 32), rng.randint(33, 200)]),
                        h=th * rng.randint(1, 12), th=th, bpc=bpc, f=rng.randint(1, 6),
                        moments=moments, v2=v2, mode=rng.choice(["batch", "stream", "split"]),
                        kind=rng.choice(["uniform", "extreme", "impulse", "checker"]),
                        seed=rng.randint(0, 10**6)))
    return out


FAST_CASES = _fast_cases(20261204, 40)


@pytest.mark.parametrize("c", FAST_CASES, ids=[f"f{i}" for i in range(len(FAST_CASES))])
def test_random_fast_path_configuration(c, monkeypatch):
    print("[case]", c, flush=True)
    sys.stdout.flush()
    monkeypatch.setenv("IIR_ROWS_PER_TILE", str(c["th"]))
    w, h, bpc, f = c["w"], c["h"], c["bpc"], c["f"]
    clip = synth.random_clip(w, h, bpc, f, seed=c["seed"], kind=c["kind"])
    ref, dist = iir.upload_planes(clip.ref), iir.upload_planes(clip.dist)
    with iir.Context(w, h, bpc, max_batch=8, moments=c["moments"], motion_v2=c["v2"]) as ctx:
        assert ctx.geometry()["rows_per_tile"] == c["th"]
        if c["mode"] == "batch":
            sums, hm = ctx.run_clip(ref, dist)
        elif c["mode"] == "stream":
            for t in range(f):
                ctx.submit([p[t] for p in ref], [p[t] for p in dist])
            sums, hm = ctx.collect()
        else:
            k = max(1, f // 2)
            ctx.submit_clip(tuple(p[:k] for p in ref), tuple(p[:k] for p in dist))
            if f > k:
                ctx.submit_clip(tuple(p[k:] for p in ref), tuple(p[k:] for p in dist))
            sums, hm = ctx.collect()
    want, want_hm = (oracle.clip_v2 if c["v2"] else oracle.clip)(clip.ref, clip.dist, bpc)
    assert np.array_equal(sums[:, :4], np.asarray(want, np.uint64)), c
    assert list(hm) == list(want_hm), c
    if c["moments"]:
        for t in range(f):
            (r1, r2), (d1, d2) = (oracle.moments(p[0][t], bpc) for p in (clip.ref, clip.dist))
            assert tuple(int(x) for x in sums[t, 4:]) == (r1, d1, r2, d2), (c, t)
