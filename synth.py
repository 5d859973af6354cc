"""Seeded synthetic 4:2:0 clips that stand in for the video pairs the pages measure.

This module only makes inputs. It holds none of the method's arithmetic (no blur, no SAD, no SSE)
and is shared by the tests, the smoke check and the benchmark, for the GPU path and the oracle
alike. All randomness comes from numpy's PCG64 ``default_rng(seed)``, drawn in a fixed order.

Five named workloads, shaped like the pages' clips (the clips themselves are not available):

  c1  576x324   8-bit, 10 pairs   gradient + uniform noise texture panning 1 px/frame, dist sigma 3
  c2  1920x1080 8-bit, 48 pairs   value-noise texture panning 2 px/frame, dist sigma 5
  c3  3840x2160 8-bit, 50 pairs   value-noise texture, random 0-4 px global motion per frame,
                                  dist = 8x8 block mean + noise sigma 2
  c4  3840x2160 10-bit, 50 pairs  c3's reference times 4, dist = 8x8 block mean + noise sigma 8
  c5  960x544   8-bit, 301 frames breathing sinusoid (amplitude 20, period 40 frames) + noise
                                  sigma 2, dist sigma 4
  c6  3840x2160 16-bit, 50 pairs  not one of the pages' clips: the 16-bit storage path at the 4K
                                  shape; every plane of c4 times 64 plus uniform noise in 0..63

Chroma (not described for the workloads, so fixed here): reference U is the rounded mean of each
2x2 luma block (edge rows/columns replicated for odd sizes), reference V is (peak - U), and the
distorted chroma is the reference chroma put through the same distortion as the luma.
"""
from __future__ import annotations

import dataclasses

import numpy as np


@dataclasses.dataclass
class Clip:
    """A clip of frame pairs: each of ref / dist is (Y, U, V), arrays of shape (F, h, w)."""

    name: str
    width: int
    height: int
    bpc: int
    ref: tuple
    dist: tuple

    @property
    def frames(self) -> int:
        return self.ref[0].shape[0]

    @property
    def dtype(self):
        return self.ref[0].dtype

    def slice(self, a: int, b: int) -> "Clip":
        return Clip(self.name, self.width, self.height, self.bpc,
                    tuple(p[a:b] for p in self.ref), tuple(p[a:b] for p in self.dist))


CONFIGS = {
    "c1": dict(width=576, height=324, bpc=8, frames=10, seed=101),
    "c2": dict(width=1920, height=1080, bpc=8, frames=48, seed=202),
    "c3": dict(width=3840, height=2160, bpc=8, frames=50, seed=303),
    "c4": dict(width=3840, height=2160, bpc=10, frames=50, seed=303, noise_seed=404),
    "c5": dict(width=960, height=544, bpc=8, frames=301, seed=505),
    "c6": dict(width=3840, height=2160, bpc=16, frames=50, seed=303, noise_seed=404, low_seed=606),
}


def _dtype(bpc: int):
    return np.uint8 if bpc == 8 else np.uint16


def _clamp_round(x: np.ndarray, bpc: int) -> np.ndarray:
    return np.clip(np.rint(x), 0, (1 << bpc) - 1).astype(_dtype(bpc))


def chroma_from_luma(y: np.ndarray, bpc: int):
    """(U, V) of one luma frame: rounded 2x2 means, and their complement to the peak."""
    h, w = y.shape
    yy = y.astype(np.int32)
    if h % 2:
        yy = np.concatenate([yy, yy[-1:]], axis=0)
    if w % 2:
        yy = np.concatenate([yy, yy[:, -1:]], axis=1)
    s = yy[0::2, 0::2] + yy[1::2, 0::2] + yy[0::2, 1::2] + yy[1::2, 1::2]
    u = ((s + 2) >> 2).astype(_dtype(bpc))
    v = (((1 << bpc) - 1) - u.astype(np.int32)).astype(_dtype(bpc))
    return u, v


def block_mean(p: np.ndarray, b: int = 8) -> np.ndarray:
    """b x b block means rounded half up; partial blocks at the edges average what they hold."""
    h, w = p.shape
    hb, wb = -(-h // b), -(-w // b)
    acc = np.zeros((hb * b, wb * b), dtype=np.int32)
    acc[:h, :w] = p
    s = acc.reshape(hb, b, wb, b).sum(axis=(1, 3), dtype=np.int32)
    rows = np.minimum(b, h - b * np.arange(hb))
    cols = np.minimum(b, w - b * np.arange(wb))
    n = rows[:, None] * cols[None, :]
    m = ((2 * s + n) // (2 * n)).astype(p.dtype)
    out = np.broadcast_to(m[:, None, :, None], (hb, b, wb, b)).reshape(hb * b, wb * b)
    return out[:h, :w]


def value_noise(rng: np.random.Generator, h: int, w: int, cells=(64, 32, 16),
                weights=(4, 2, 1)) -> np.ndarray:
    """Smoothstep-interpolated lattice noise in [0, 255], octaves summed with the given weights."""
    out = np.zeros((h, w), dtype=np.float32)
    for c, wt in zip(cells, weights):
        lat = rng.uniform(0.0, 255.0, size=(h // c + 2, w // c + 2)).astype(np.float32)
        ys, xs = np.arange(h), np.arange(w)
        iy, ix = ys // c, xs // c
        fy = ((ys % c) / c).astype(np.float32)
        fx = ((xs % c) / c).astype(np.float32)
        sy = (fy * fy * (3 - 2 * fy))[:, None]
        sx = (fx * fx * (3 - 2 * fx))[None, :]
        a = lat[iy][:, ix]
        b = lat[iy][:, ix + 1]
        cc = lat[iy + 1][:, ix]
        d = lat[iy + 1][:, ix + 1]
        out += wt * ((1 - sy) * ((1 - sx) * a + sx * b) + sy * ((1 - sx) * cc + sx * d))
    return out / float(sum(weights))


def _noise(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma)


def _alloc(f, h, w, bpc):
    hc, wc = (h + 1) // 2, (w + 1) // 2
    dt = _dtype(bpc)
    return ([np.empty((f, h, w), dt), np.empty((f, hc, wc), dt), np.empty((f, hc, wc), dt)],
            [np.empty((f, h, w), dt), np.empty((f, hc, wc), dt), np.empty((f, hc, wc), dt)])


def _fill_ref(ref, t, y, bpc):
    ref[0][t] = y
    ref[1][t], ref[2][t] = chroma_from_luma(y, bpc)


def _distort_additive(rng, ref, dist, t, sigma, bpc):
    for p in range(3):
        dist[p][t] = _clamp_round(ref[p][t].astype(np.float32) + _noise(rng, ref[p][t].shape,
                                                                          sigma), bpc)


def _distort_blocky(rng, ref, dist, t, sigma, bpc):
    for p in range(3):
        q = block_mean(ref[p][t]).astype(np.float32)
        dist[p][t] = _clamp_round(q + _noise(rng, q.shape, sigma), bpc)


def _c1(f, seed):
    w, h, bpc = 576, 324, 8
    rng = np.random.default_rng(seed)
    ref, dist = _alloc(f, h, w, bpc)
    wt = w + f
    ys, xs = np.mgrid[0:h, 0:wt]
    tex = np.rint(32 + 192 * (xs + ys / 2) / (w + h)) + rng.integers(-16, 17, size=(h, wt))
    tex = np.clip(tex, 0, 255).astype(np.uint8)
    for t in range(f):
        _fill_ref(ref, t, tex[:, t:t + w], bpc)
        _distort_additive(rng, ref, dist, t, 3.0, bpc)
    return w, h, bpc, ref, dist


def _c2(f, seed):
    w, h, bpc = 1920, 1080, 8
    rng = np.random.default_rng(seed)
    ref, dist = _alloc(f, h, w, bpc)
    tex = _clamp_round(value_noise(rng, h, w + 2 * f), 8)
    for t in range(f):
        _fill_ref(ref, t, tex[:, 2 * t:2 * t + w], bpc)
        _distort_additive(rng, ref, dist, t, 5.0, bpc)
    return w, h, bpc, ref, dist


def _c3_luma(f, seed):
    w, h = 3840, 2160
    rng = np.random.default_rng(seed)
    pad = 4 * f
    tex = _clamp_round(value_noise(rng, h + pad, w + pad), 8)
    steps = rng.integers(0, 5, size=(f, 2))
    off = np.cumsum(steps, axis=0) - steps[0]
    return rng, tex, off


def _c3(f, seed):
    w, h, bpc = 3840, 2160, 8
    rng, tex, off = _c3_luma(f, seed)
    ref, dist = _alloc(f, h, w, bpc)
    for t in range(f):
        dy, dx = off[t]
        _fill_ref(ref, t, tex[dy:dy + h, dx:dx + w], bpc)
        _distort_blocky(rng, ref, dist, t, 2.0, bpc)
    return w, h, bpc, ref, dist


def _c4(f, seed, noise_seed):
    w, h, bpc = 3840, 2160, 10
    _, tex, off = _c3_luma(f, seed)
    rng = np.random.default_rng(noise_seed)
    ref, dist = _alloc(f, h, w, bpc)
    for t in range(f):
        dy, dx = off[t]
        _fill_ref(ref, t, tex[dy:dy + h, dx:dx + w].astype(np.uint16) * 4, bpc)
        _distort_blocky(rng, ref, dist, t, 8.0, bpc)
    return w, h, bpc, ref, dist


def _c5(f, seed):
    w, h, bpc = 960, 544, 8
    rng = np.random.default_rng(seed)
    ref, dist = _alloc(f, h, w, bpc)
    ys, xs = np.mgrid[0:h, 0:w].astype(np.float32)
    pattern = np.sin(2 * np.pi * xs / 64) * np.sin(2 * np.pi * ys / 48)
    for t in range(f):
        amp = 20 * np.sin(2 * np.pi * t / 40)
        y = _clamp_round(128 + amp * pattern + _noise(rng, (h, w), 2.0), 8)
        _fill_ref(ref, t, y, bpc)
        _distort_additive(rng, ref, dist, t, 4.0, bpc)
    return w, h, bpc, ref, dist


def _c6(f, seed, noise_seed, low_seed):
    w, h, _, ref, dist = _c4(f, seed, noise_seed)
    rng = np.random.default_rng(low_seed)
    for planes in (ref, dist):
        for p in planes:
            for t in range(f):
                p[t] = (p[t] << 6) | rng.integers(0, 64, size=p[t].shape, dtype=np.uint16)
    return w, h, 16, ref, dist


def make_clip(name: str, frames: int | None = None) -> Clip:
    """Build a named workload; ``frames`` truncates it (the first frames are the same either way)."""
    cfg = CONFIGS[name]
    f = cfg["frames"] if frames is None else int(frames)
    if not 1 <= f <= cfg["frames"]:
        raise ValueError(f"{name} has {cfg['frames']} frames, asked for {f}")
    if name == "c1":
        w, h, bpc, ref, dist = _c1(f, cfg["seed"])
    elif name == "c2":
        w, h, bpc, ref, dist = _c2(f, cfg["seed"])
    elif name == "c3":
        w, h, bpc, ref, dist = _c3(f, cfg["seed"])
    elif name == "c4":
        w, h, bpc, ref, dist = _c4(f, cfg["seed"], cfg["noise_seed"])
    elif name == "c6":
        w, h, bpc, ref, dist = _c6(f, cfg["seed"], cfg["noise_seed"], cfg["low_seed"])
    else:
        w, h, bpc, ref, dist = _c5(f, cfg["seed"])
    return Clip(name, w, h, bpc, tuple(ref), tuple(dist))


def random_clip(width: int, height: int, bpc: int, frames: int, seed: int,
                kind: str = "uniform") -> Clip:
    """Small clips for sweeps: uniform noise, extreme checkerboards, or sparse impulses."""
    rng = np.random.default_rng(seed)
    peak = (1 << bpc) - 1
    hc, wc = (height + 1) // 2, (width + 1) // 2
    dt = _dtype(bpc)

    def plane(h, w):
        if kind == "uniform":
            return rng.integers(0, peak + 1, size=(h, w)).astype(dt)
        if kind == "checker":
            ph = int(rng.integers(0, 2))
            yy, xx = np.mgrid[0:h, 0:w]
            return (((yy + xx + ph) % 2) * peak).astype(dt)
        if kind == "impulse":
            p = np.zeros((h, w), dtype=dt)
            m = rng.random((h, w)) < 0.05
            p[m] = peak
            return p
        if kind == "extreme":
            return (rng.integers(0, 2, size=(h, w)) * peak).astype(dt)
        raise ValueError(kind)

    ref = [np.stack([plane(height, width) for _ in range(frames)]),
           np.stack([plane(hc, wc) for _ in range(frames)]),
           np.stack([plane(hc, wc) for _ in range(frames)])]
    dist = [np.stack([plane(height, width) for _ in range(frames)]),
            np.stack([plane(hc, wc) for _ in range(frames)]),
            np.stack([plane(hc, wc) for _ in range(frames)])]
    return Clip(f"{kind}{width}x{height}", width, height, bpc, tuple(ref), tuple(dist))


def frame_pair_bytes(width: int, height: int, bpc: int) -> int:
    """Bytes of one reference + distorted 4:2:0 frame pair as stored (1 or 2 bytes per sample)."""
    b = 1 if bpc == 8 else 2
    return 2 * b * (width * height + 2 * ((width + 1) // 2) * ((height + 1) // 2))
