"""Pins that tie the CPU oracle to facts fixed outside its own code.

Each ``pin_*`` function takes a loaded oracle (``oracle.OracleLib``) and raises AssertionError when
the oracle disagrees with a brute-force evaluation, a library routine, a closed form or an
invariant. ``test_oracle_pins.py`` runs them on the real oracle; ``test_oracle_mutants.py`` runs
them on deliberately broken copies and requires every copy to fail at least one pin.

Readings of the pages used here (the pages fix none of the three numerically):
  * taps (3571, 16004, 26386, 16004, 3571), sum 2^16 (sigma = 1 sampled Gaussian);
  * round half up at both shifts (>> bpc after the vertical pass, >> 16 after the horizontal);
  * whole-sample mirror at the edges (numpy 'reflect' == scipy.ndimage 'mirror').
"""
from __future__ import annotations

import math

import numpy as np
import scipy.ndimage as ndi

TAPS = (3571, 16004, 26386, 16004, 3571)
DEPTHS = (8, 10, 12, 16)  # every storage path: uint8, and uint16 at 10, 12 and the full 16 bits
SIZES = [(3, 3), (4, 7), (9, 5), (17, 23), (32, 32), (5, 64), (70, 3)]


def _rng(seed):
    return np.random.default_rng(seed)


def _planes(bpc, seed, sizes=SIZES):
    r = _rng(seed)
    peak = (1 << bpc) - 1
    dt = np.uint8 if bpc == 8 else np.uint16
    out = []
    for h, w in sizes:
        out.append(r.integers(0, peak + 1, size=(h, w)).astype(dt))
        yy, xx = np.mgrid[0:h, 0:w]
        out.append((((yy + xx) % 2) * peak).astype(dt))
        out.append((r.integers(0, 2, size=(h, w)) * peak).astype(dt))
    return out


def brute_force_blur(x: np.ndarray, bpc: int) -> np.ndarray:
    """25 multiply-adds per output: for each of the 5 columns of the output's 5x5 window, its own
    vertical 5-tap sum rounded by the bit depth, then the 5 horizontal taps rounded by 16. The edge
    mirror comes from numpy's whole-sample 'reflect' padding, not from the oracle's index rule."""
    h, w = x.shape
    xp = np.pad(x.astype(np.int64), 2, mode="reflect")
    g = np.array(TAPS, dtype=np.int64)
    out = np.zeros((h, w), dtype=np.int64)
    for l in range(5):
        v = np.zeros((h, w), dtype=np.int64)
        for k in range(5):
            v += g[k] * xp[k:k + h, l:l + w]
        v = (v + (1 << (bpc - 1))) >> bpc
        out += g[l] * v
    return ((out + 32768) >> 16).astype(np.uint16)


def scipy_blur(x: np.ndarray, bpc: int) -> np.ndarray:
    """The same separable filter through scipy.ndimage.correlate1d (mode 'mirror')."""
    g = np.array(TAPS, dtype=np.float64)
    v = ndi.correlate1d(x.astype(np.int64), g, axis=0, mode="mirror")
    v = (v + (1 << (bpc - 1))) >> bpc
    b = ndi.correlate1d(v, g, axis=1, mode="mirror")
    return ((b + 32768) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------------------------
# taps


def pin_taps(o):
    g = [int(v) for v in o.taps()]
    assert g == list(TAPS), g
    assert sum(g) == 1 << 16


# ---------------------------------------------------------------------------------------------
# blur


def pin_blur_brute_force(o):
    for bpc in DEPTHS:
        for i, x in enumerate(_planes(bpc, 11 + bpc)):
            got, want = o.blur(x, bpc), brute_force_blur(x, bpc)
            assert np.array_equal(got, want), (bpc, i, x.shape)


def pin_blur_brute_force_large(o):
    r = _rng(5)
    for (h, w), bpc in (((723, 1283), 8), ((131, 257), 10)):
        x = r.integers(0, 1 << bpc, size=(h, w)).astype(np.uint8 if bpc == 8 else np.uint16)
        assert np.array_equal(o.blur(x, bpc), brute_force_blur(x, bpc)), (h, w, bpc)


def pin_blur_scipy(o):
    for bpc in DEPTHS:
        for i, x in enumerate(_planes(bpc, 23 + bpc)):
            assert np.array_equal(o.blur(x, bpc), scipy_blur(x, bpc)), (bpc, i, x.shape)


def pin_blur_constant(o):
    """A flat plane stays flat, scaled to 16 bits: c * 2^(16 - bpc)."""
    for bpc in DEPTHS:
        for c in (0, 1, 77, (1 << bpc) - 1):
            for h, w in ((3, 3), (6, 16), (11, 4)):
                x = np.full((h, w), c, dtype=np.uint8 if bpc == 8 else np.uint16)
                assert np.all(o.blur(x, bpc) == c << (16 - bpc)), (bpc, c, h, w)


# 5x5 response to one full-scale sample in the middle of a zero plane, hand-derived from the taps:
# vertical 8-bit values (g*255 + 128) >> 8 = 3557, 15941, 26283; each row then (g*V + 32768) >> 16.
# At 10 bits the vertical values are (g*1023 + 512) >> 10 = 3568, 15988, 26360; the vertical pass
# rounds first, so the response is not symmetric under transposition (1437 above, 1436 left).
IMPULSE_8 = [[194, 869, 1432, 869, 194],
             [869, 3893, 6418, 3893, 869],
             [1432, 6418, 10582, 6418, 1432],
             [869, 3893, 6418, 3893, 869],
             [194, 869, 1432, 869, 194]]
IMPULSE_10 = [[194, 871, 1437, 871, 194],
              [871, 3904, 6437, 3904, 871],
              [1436, 6437, 10613, 6437, 1436],
              [871, 3904, 6437, 3904, 871],
              [194, 871, 1437, 871, 194]]


def pin_blur_impulse(o):
    for bpc, resp in ((8, IMPULSE_8), (10, IMPULSE_10)):
        x = np.zeros((9, 11), dtype=np.uint8 if bpc == 8 else np.uint16)
        x[4, 5] = (1 << bpc) - 1
        b = o.blur(x, bpc).astype(np.int64)
        want = np.zeros((9, 11), dtype=np.int64)
        want[2:7, 3:8] = resp
        assert np.array_equal(b, want), (bpc, b)


# A vertical 0 -> full-scale step at column k: every column's vertical value is 0 or 65280 (8-bit,
# (65536*255 + 128) >> 8) or 65472 (10-bit); across the step the blurred row rises through the
# cumulative tap sums 3571, 19575, 45961, 61965 scaled by that value and rounded.
STEP_8 = [0, 3557, 19499, 45781, 61723, 65280]
STEP_10 = [0, 3568, 19556, 45916, 61904, 65472]


def pin_blur_step(o):
    for bpc, prof in ((8, STEP_8), (10, STEP_10)):
        x = np.zeros((7, 16), dtype=np.uint8 if bpc == 8 else np.uint16)
        x[:, 8:] = (1 << bpc) - 1
        b = o.blur(x, bpc)
        for i in range(7):
            assert list(b[i, 5:11]) == prof, (bpc, i, list(b[i]))


def pin_blur_mirror_edges(o):
    """A step placed one column from the left edge: the mirror makes column -1 equal column 1, so
    output column 0 sees (x1, x1... ) = the mirrored neighbours, which differs from clamping."""
    for bpc in DEPTHS:
        peak = (1 << bpc) - 1
        x = np.zeros((5, 8), dtype=np.uint8 if bpc == 8 else np.uint16)
        x[:, 1] = peak  # column 1 bright: mirrored into column -1
        b = o.blur(x, bpc).astype(np.int64)
        vmax = ((65536 * peak) + (1 << (bpc - 1))) >> bpc
        # column 0 sees taps g1 (col -1 -> 1) and g1 (col 1): 2*16004 of vmax
        assert b[2, 0] == (2 * 16004 * vmax + 32768) >> 16, b[2]
        # column 2 sees g1 from column 1 only
        assert b[2, 2] == (16004 * vmax + 32768) >> 16, b[2]
        # the right edge mirrors the same way: flip the plane
        bf = o.blur(np.ascontiguousarray(x[:, ::-1]), bpc).astype(np.int64)
        assert np.array_equal(bf, b[:, ::-1])


def pin_blur_flip(o):
    for bpc in DEPTHS:
        for x in _planes(bpc, 41 + bpc):
            b = o.blur(x, bpc)
            assert np.array_equal(o.blur(np.ascontiguousarray(x[::-1]), bpc), b[::-1])
            assert np.array_equal(o.blur(np.ascontiguousarray(x[:, ::-1]), bpc), b[:, ::-1])


def pin_blur_range_and_linearity(o):
    r = _rng(3)
    for bpc in DEPTHS:
        peak = (1 << bpc) - 1
        dt = np.uint8 if bpc == 8 else np.uint16
        for h, w in ((3, 3), (12, 19), (40, 7)):
            x = r.integers(0, peak // 2, size=(h, w)).astype(dt)
            b = o.blur(x, bpc).astype(np.int64)
            assert b.min() >= 0 and b.max() <= peak << (16 - bpc)
            for c in (1, 5, peak // 2):
                bc = o.blur((x.astype(np.int64) + c).astype(dt), bpc).astype(np.int64)
                assert np.array_equal(bc, b + (c << (16 - bpc))), (bpc, c)


def pin_blur_bit_depth(o):
    """The blur of x * 2^(bpc - 8) at bpc bits equals the 8-bit blur of x: the vertical sum and its
    rounding term both scale by 2^(bpc - 8), so floor((s a + s 128) / (s 256)) = floor((a + 128) /
    256) with s = 2^(bpc - 8); the horizontal pass then sees the same values."""
    for x in _planes(8, 59):
        b8 = o.blur(x, 8)
        for bpc in (9, 10, 12, 16):
            xs = x.astype(np.uint16) << (bpc - 8)
            assert np.array_equal(o.blur(xs, bpc), b8), bpc


def pin_blur_error_bound(o):
    """The integer result is within 1 of the exact real-valued 2-D filter scaled to 16 bits."""
    g = np.array(TAPS, dtype=np.float64) / 65536.0
    for bpc in DEPTHS:
        for x in _planes(bpc, 61 + bpc):
            h, w = x.shape
            xp = np.pad(x.astype(np.float64), 2, mode="reflect")
            exact = np.zeros((h, w))
            for k in range(5):
                for l in range(5):
                    exact += g[k] * g[l] * xp[k:k + h, l:l + w]
            err = np.abs(o.blur(x, bpc) - exact * (1 << (16 - bpc)))
            assert err.max() <= 1.0, (bpc, x.shape, err.max())


def pin_blur_translation(o):
    """Away from the edges a shifted input gives a shifted output."""
    r = _rng(8)
    x = r.integers(0, 256, size=(40, 40)).astype(np.uint8)
    b = o.blur(x, 8)
    bs = o.blur(np.ascontiguousarray(x[3:, 5:]), 8)
    assert np.array_equal(bs[2:-2, 2:-2], b[5:-2, 7:-2])


# ---------------------------------------------------------------------------------------------
# SSE and SAD


def pin_sse_brute_force(o):
    r = _rng(13)
    for bpc in DEPTHS:
        peak = (1 << bpc) - 1
        dt = np.uint8 if bpc == 8 else np.uint16
        for h, w in SIZES + [(1, 1), (1, 9), (8, 1)]:
            a = r.integers(0, peak + 1, size=(h, w)).astype(dt)
            b = r.integers(0, peak + 1, size=(h, w)).astype(dt)
            want = sum((int(p) - int(q)) ** 2 for p, q in zip(a.ravel(), b.ravel()))
            assert o.sse(a, b, bpc) == want
            assert o.sse(b, a, bpc) == want
            assert o.sse(a, a, bpc) == 0


def pin_sse_bit_depth(o):
    """Scaling both planes by 2^(bpc - 8) scales the squared error by 4^(bpc - 8); at 16 bits a
    full-scale difference squares to 65535^2, which needs more than 32 bits once two are added."""
    r = _rng(19)
    a = r.integers(0, 256, size=(9, 14)).astype(np.uint8)
    b = r.integers(0, 256, size=(9, 14)).astype(np.uint8)
    e8 = o.sse(a, b, 8)
    for bpc in (10, 12, 16):
        s = 1 << (bpc - 8)
        assert o.sse(a.astype(np.uint16) * s, b.astype(np.uint16) * s, bpc) == e8 * s * s, bpc
    full = np.full((2, 3), 65535, dtype=np.uint16)
    assert o.sse(full, np.zeros_like(full), 16) == 6 * 65535 ** 2


def pin_sse_constant(o):
    for bpc in DEPTHS:
        dt = np.uint8 if bpc == 8 else np.uint16
        a = np.full((6, 16), 100, dtype=dt)
        b = np.full((6, 16), 103, dtype=dt)
        assert o.sse(a, b, bpc) == 96 * 9
        full = np.full((3, 5), (1 << bpc) - 1, dtype=dt)
        assert o.sse(full, np.zeros_like(full), bpc) == 15 * ((1 << bpc) - 1) ** 2


def pin_sad_brute_force(o):
    r = _rng(17)
    for h, w in SIZES:
        a = r.integers(0, 65536, size=(h, w)).astype(np.uint16)
        b = r.integers(0, 65536, size=(h, w)).astype(np.uint16)
        want = sum(abs(int(p) - int(q)) for p, q in zip(a.ravel(), b.ravel()))
        assert o.sad(a, b) == want
        assert o.sad(b, a) == want
        assert o.sad(a, a) == 0


# ---------------------------------------------------------------------------------------------
# whole clip


def _tiny_clip(bpc, f, h, w, seed):
    r = _rng(seed)
    dt = np.uint8 if bpc == 8 else np.uint16
    hc, wc = (h + 1) // 2, (w + 1) // 2
    mk = lambda *s: r.integers(0, 1 << bpc, size=s).astype(dt)  # noqa: E731
    return ((mk(f, h, w), mk(f, hc, wc), mk(f, hc, wc)), (mk(f, h, w), mk(f, hc, wc), mk(f, hc, wc)))


def pin_clip_composition(o):
    """Per frame: SSE of each plane by brute force, SAD of brute-force blurs of consecutive frames."""
    for bpc, (f, h, w) in ((8, (4, 7, 9)), (10, (3, 5, 6)), (8, (3, 3, 3)), (8, (2, 11, 4)),
                           (12, (3, 6, 5)), (16, (3, 5, 7))):
        ref, dist = _tiny_clip(bpc, f, h, w, 100 + h)
        sums, hm = o.clip(ref, dist, bpc)
        assert list(hm) == [0] + [1] * (f - 1)
        prev = None
        for t in range(f):
            for p in range(3):
                d = ref[p][t].astype(np.int64) - dist[p][t].astype(np.int64)
                assert int(sums[t, 1 + p]) == int((d * d).sum()), (t, p)
            cur = brute_force_blur(ref[0][t], bpc).astype(np.int64)
            want = 0 if prev is None else int(np.abs(cur - prev).sum())
            assert int(sums[t, 0]) == want, (bpc, t)
            prev = cur


def pin_clip_split(o):
    """A clip run in two parts, the second given the first's last blurred plane, matches one run."""
    ref, dist = _tiny_clip(8, 6, 9, 12, 7)
    whole, hm = o.clip(ref, dist, 8)
    a, hma, last = o.clip(tuple(p[:2] for p in ref), tuple(p[:2] for p in dist), 8,
                          want_last_blur=True)
    b, hmb = o.clip(tuple(p[2:] for p in ref), tuple(p[2:] for p in dist), 8, prev_blur=last)
    assert np.array_equal(np.concatenate([a, b]), whole)
    assert list(hma) + list(hmb) == list(hm) == [0, 1, 1, 1, 1, 1]


def pin_clip_constant_motion(o):
    """Constant frames c then c + d: SAD = N |d| 2^(16 - bpc), so motion = |d| (8-bit units)."""
    for bpc in DEPTHS:
        dt = np.uint8 if bpc == 8 else np.uint16
        h, w = 6, 16
        hc, wc = 3, 8
        y = np.stack([np.full((h, w), 100, dt), np.full((h, w), 103, dt), np.full((h, w), 97, dt)])
        c = np.full((3, hc, wc), 50, dt)
        sums, hm = o.clip((y, c, c), (y, c, c), bpc)
        n = h * w
        assert list(sums[:, 0]) == [0, n * 3 << (16 - bpc), n * 6 << (16 - bpc)]
        assert int(sums[:, 1:].sum()) == 0
        s = o.scores(w, h, bpc, sums[2], hm[2])
        assert s["motion"] == 6.0 * (1 << (16 - bpc)) / 256.0


def pin_scores(o):
    """PSNR of a constant difference d is 10 log10(peak^2 / d^2); zero error gives +inf."""
    for bpc in DEPTHS:
        peak = (1 << bpc) - 1
        w, h = 8, 6
        n, nc = 48, 12
        for d in (1, 3, 17):
            s = o.scores(w, h, bpc, [0, n * d * d, nc * d * d, 0], 0)
            want = 10 * math.log10(peak * peak / (d * d))
            assert abs(s["psnr"][0] - want) <= 1e-12 * want
            assert abs(s["psnr"][1] - want) <= 1e-12 * want
            assert s["psnr"][2] == math.inf
            assert s["mse"][0] == d * d and s["mse"][2] == 0.0
            assert s["motion"] == 0.0
        s = o.scores(w, h, bpc, [256 * 48 * 5, 0, 0, 0], 1)
        assert s["motion"] == 5.0
    # odd sizes: chroma planes are ceil(W/2) x ceil(H/2)
    s = o.scores(5, 3, 8, [0, 0, 6 * 4, 0], 0)
    assert s["mse"][1] == 4.0


def pin_rejects_out_of_range(o):
    for bpc in (10, 12):
        x = np.full((4, 4), 1 << bpc, dtype=np.uint16)
        try:
            o.blur(x, bpc)
        except Exception:
            pass
        else:
            raise AssertionError(f"a {bpc}-bit sample of {1 << bpc} was accepted")


# ---------------------------------------------------------------------------------------------
# luma moments, motion2 and clip aggregates (readings: the pages name these outputs only)


def pin_moments_brute_force(o):
    """sum x and sum x^2 against Python integers over random, checkerboard and 0/max planes."""
    for bpc in DEPTHS:
        for i, x in enumerate(_planes(bpc, 41 + bpc)):
            v = [int(a) for a in x.reshape(-1)]
            assert o.moments(x, bpc) == (sum(v), sum(a * a for a in v)), (bpc, i, x.shape)


def pin_moments_closed_form(o):
    """A flat plane of value c: N c and N c^2; a bit-depth step (x4) scales them by 4 and 16."""
    for bpc in DEPTHS:
        for c in (0, 1, 200, (1 << bpc) - 1):
            x = np.full((7, 9), c, dtype=np.uint8 if bpc == 8 else np.uint16)
            assert o.moments(x, bpc) == (63 * c, 63 * c * c), (bpc, c)
    x = _rng(4).integers(0, 256, size=(13, 17)).astype(np.uint8)
    s1, s2 = o.moments(x, 8)
    assert o.moments((x.astype(np.uint16) * 4), 10) == (4 * s1, 16 * s2)
    assert o.moments((x.astype(np.uint16) * 256), 16) == (256 * s1, 65536 * s2)


def pin_motion2_properties(o):
    """Each value is one of its two inputs and no larger than either; the last frame keeps its
    own motion; an increasing clip keeps its motions, a decreasing one takes the next frame's."""
    r = _rng(8)
    for n in (1, 2, 5, 40):
        m = r.random(n) * 10.0
        m2 = o.motion2(m)
        for t in range(n):
            nxt = m[t + 1] if t + 1 < n else m[t]
            assert m2[t] in (m[t], nxt) and m2[t] <= m[t] and m2[t] <= nxt, (n, t)
        assert m2[-1] == m[-1]
    inc = np.arange(1.0, 9.0)
    assert np.array_equal(o.motion2(inc), inc)
    dec = inc[::-1].copy()
    assert np.array_equal(o.motion2(dec)[:-1], dec[1:]) and o.motion2(dec)[-1] == dec[-1]


def pin_aggregate(o):
    """Aggregate PSNR is the PSNR of the clip's mean MSE: equal frames give the frame PSNR, and
    it lies between the per-frame PSNRs; zero error gives +inf; the mean motions average the
    per-frame scores of the per-frame function."""
    w, h, bpc = 6, 4, 8
    sums = [[0, 24, 6, 6]] * 3
    agg = o.aggregate(w, h, bpc, sums, [0, 1, 1])
    frame = o.scores(w, h, bpc, sums[0], 1)
    assert np.allclose(agg["apsnr"], frame["psnr"], rtol=0, atol=1e-12)
    r = _rng(12)
    sums = [[int(r.integers(0, 1 << 20))] + [int(r.integers(1, 5000)) for _ in range(3)]
            for _ in range(7)]
    hm = [0] + [1] * 6
    agg = o.aggregate(w, h, bpc, sums, hm)
    per = [o.scores(w, h, bpc, s, m) for s, m in zip(sums, hm)]
    for c in range(3):
        ps = [p["psnr"][c] for p in per]
        assert min(ps) - 1e-12 <= agg["apsnr"][c] <= max(ps) + 1e-12
        mean_mse = sum(p["mse"][c] for p in per) / len(per)
        assert abs(agg["apsnr"][c] - 10.0 * math.log10(255.0 ** 2 / mean_mse)) < 1e-9
    mot = [p["motion"] for p in per]
    assert abs(agg["mean_motion"] - sum(mot) / 7) < 1e-15
    assert abs(agg["mean_motion2"] - sum(o.motion2(mot)) / 7) < 1e-15
    zero = o.aggregate(w, h, bpc, [[0, 0, 0, 0]] * 2, [0, 1])
    assert all(math.isinf(v) for v in zero["apsnr"])


# ---------------------------------------------------------------------------------------------
# motion v2: the filter of the difference prev - cur (floor shifts)


def brute_force_diff_blur(prev: np.ndarray, cur: np.ndarray, bpc: int) -> np.ndarray:
    """25 multiply-adds per output on D = prev - cur with numpy's floor division (//) for both
    rounded shifts and numpy's 'reflect' padding for the mirror."""
    h, w = prev.shape
    d = np.pad(prev.astype(np.int64) - cur.astype(np.int64), 2, mode="reflect")
    g = np.array(TAPS, dtype=np.int64)
    out = np.zeros((h, w), dtype=np.int64)
    for l in range(5):
        v = np.zeros((h, w), dtype=np.int64)
        for k in range(5):
            v += g[k] * d[k:k + h, l:l + w]
        out += g[l] * ((v + (1 << (bpc - 1))) // (1 << bpc))
    return (out + 32768) // 65536


def scipy_diff_blur(prev: np.ndarray, cur: np.ndarray, bpc: int) -> np.ndarray:
    g = np.array(TAPS, dtype=np.float64)
    d = prev.astype(np.int64) - cur.astype(np.int64)
    v = ndi.correlate1d(d, g, axis=0, mode="mirror").astype(np.int64)
    v = np.floor_divide(v + (1 << (bpc - 1)), 1 << bpc)
    b = ndi.correlate1d(v, g, axis=1, mode="mirror").astype(np.int64)
    return np.floor_divide(b + 32768, 65536)


def _pairs(bpc, seed):
    a, b = _planes(bpc, seed), _planes(bpc, seed + 1)
    return list(zip(a, b))


def pin_diff_blur_brute_force(o):
    for bpc in (8, 10, 12, 15, 16):
        for i, (p, c) in enumerate(_pairs(bpc, 71 + bpc)):
            assert np.array_equal(o.diff_blur(p, c, bpc), brute_force_diff_blur(p, c, bpc)), \
                (bpc, i, p.shape)


def pin_diff_blur_scipy(o):
    for bpc in (8, 10):
        for i, (p, c) in enumerate(_pairs(bpc, 83 + bpc)):
            assert np.array_equal(o.diff_blur(p, c, bpc), scipy_diff_blur(p, c, bpc)), (bpc, i)


def pin_diff_blur_constant(o):
    """Flat frames c + d then c: every output is d 2^(16 - bpc), of either sign."""
    for bpc in (8, 10, 12, 15):
        dt = np.uint8 if bpc == 8 else np.uint16
        for c0, d in ((100, 3), (100, -7), (0, 255), (255, -255)):
            c0, d = c0 << (bpc - 8), d * (1 << (bpc - 8))
            p = np.full((6, 9), c0 + d, dt)
            c = np.full((6, 9), c0, dt)
            assert np.all(o.diff_blur(p, c, bpc) == d * (1 << (16 - bpc))), (bpc, c0, d)
        x = _planes(bpc, 5)[0]
        assert not o.diff_blur(x, x, bpc).any()


def pin_diff_blur_bounds(o):
    """Within 1 of the exact real filter of prev - cur scaled to 16 bits; within 3 of the
    difference of the two blurred frames; swapping the frames negates the result up to 1."""
    g = np.array(TAPS, dtype=np.float64) / 65536.0
    for bpc in (8, 10, 12, 15):
        for p, c in _pairs(bpc, 97 + bpc):
            h, w = p.shape
            f = o.diff_blur(p, c, bpc).astype(np.int64)
            dp = np.pad(p.astype(np.float64) - c.astype(np.float64), 2, mode="reflect")
            exact = np.zeros((h, w))
            for k in range(5):
                for l in range(5):
                    exact += g[k] * g[l] * dp[k:k + h, l:l + w]
            assert np.abs(f - exact * (1 << (16 - bpc))).max() <= 1.0
            blurred = o.blur(p, bpc).astype(np.int64) - o.blur(c, bpc).astype(np.int64)
            assert np.abs(f - blurred).max() <= 3
            assert np.abs(f + o.diff_blur(c, p, bpc).astype(np.int64)).max() <= 1


def pin_diff_blur_depth(o):
    """The filter of 8-bit frames scaled to depth b (x 2^(b - 8)) is the 8-bit filter, exactly: the
    vertical rounding term and shift scale with the samples."""
    for b in (9, 10, 12, 15, 16):
        for i, (p, c) in enumerate(_pairs(8, 113)):
            s = 1 << (b - 8)
            ps, cs = (p.astype(np.uint16) * s), (c.astype(np.uint16) * s)
            assert np.array_equal(o.diff_blur(ps, cs, b), o.diff_blur(p, c, 8)), (b, i)


def pin_clip_v2_composition(o):
    """Per frame: SSE by brute force, SAD2 = sum |F| of the brute-force filter of the previous and
    the current reference luma; a clip split in two with the first part's last luma as prev_luma
    equals the whole clip."""
    for bpc, (f, h, w) in ((8, (4, 7, 9)), (10, (3, 5, 6)), (8, (3, 3, 3)), (12, (3, 6, 5)),
                           (15, (3, 5, 7))):
        ref, dist = _tiny_clip(bpc, f, h, w, 300 + h)
        sums, hm = o.clip_v2(ref, dist, bpc)
        assert list(hm) == [0] + [1] * (f - 1)
        for t in range(f):
            for p in range(3):
                d = ref[p][t].astype(np.int64) - dist[p][t].astype(np.int64)
                assert int(sums[t, 1 + p]) == int((d * d).sum())
            want = 0 if t == 0 else int(np.abs(brute_force_diff_blur(ref[0][t - 1], ref[0][t],
                                                                      bpc)).sum())
            assert int(sums[t, 0]) == want, (bpc, t)
        a, ha = o.clip_v2(tuple(q[:2] for q in ref), tuple(q[:2] for q in dist), bpc)
        b, hb = o.clip_v2(tuple(q[2:] for q in ref), tuple(q[2:] for q in dist), bpc,
                          prev_luma=ref[0][1])
        assert np.array_equal(np.concatenate([a, b]), sums)
        assert list(ha) + list(hb) == [0] + [1] * (f - 1)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
