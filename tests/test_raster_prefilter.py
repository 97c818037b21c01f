"""The raster's per-wave box test never drops a Gaussian that the per-pixel
3-sigma test would take (host logic, no GPU).

After staging a batch of Gaussians (the conic scaled to the base-2 power
p2 = log2(e) power), each wave of the raster kernel keeps only those whose
quadratic form q = -p2 can reach 4.5 log2(e) on the box of its pixel centres
(minimum at the mean when the box holds it, else at the clamped vertex of
the parabola on each edge), with a margin of 4e-6 of the box's absolute
terms plus 1.5e-4 for fp32 rounding.  That is an optimisation
only if it keeps every Gaussian some pixel of the wave composites.  This
test evaluates, in fp32 with numpy, the per-pixel power in the kernel's
operation order and the box test in the order of the kernel's code (with and
without the fused multiply-adds a compiler may form), for every entry of the
tile lists of scenes of needle-like and flat splats (2D conic condition up
to 1e8, where fp32 rounding of the power is largest), for both wave shapes
(16 x 4 pixel centres with one pixel per thread, 16 x 8 with two).
"""
import numpy as np
import pytest

import oracle as O
from implicit_attribute_decode_amd import scenes as S

f32 = np.float32
LOG2E = f32(1.44269504088896341)
SCALE_A, SCALE_B = f32(-0.5) * LOG2E, -LOG2E  # staged A and C factor, B factor
P2_MIN = f32(f32(-4.5) * LOG2E)               # 3 sigma in base-2 units


def _fma(a, b, c):
    # a * b is exact in float64 for float32 operands; one rounding to float32
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(f32)


def _scene(seed, frames, thin):
    rng = np.random.default_rng(seed)
    per = 1500
    n = frames * per
    g = S.render_attributes(rng, S.shell_points(rng, n, 3.0), 1e-2, 5e-2)
    kind = rng.integers(0, 4, size=n)
    lo, hi, l0, l1 = thin
    tiny = np.exp(rng.uniform(np.log(lo), np.log(hi), size=(n, 3))).astype(f32)
    long_ = rng.uniform(l0, l1, size=n).astype(f32)
    axis = rng.integers(0, 3, size=n)
    needle = kind <= 1
    g.scales[needle] = tiny[needle]
    g.scales[needle, axis[needle]] = long_[needle]
    flat = kind == 2
    g.scales[flat] = np.repeat(long_[flat, None] * 0.5, 3, axis=1)
    g.scales[flat, axis[flat]] = tiny[flat, 0]
    cams = [S.ring_camera(3 * f, W=256, H=208, fx=200.0, fy=200.0) for f in range(frames)]
    fo = np.arange(frames + 1, dtype=np.int64) * per
    pre = O.preprocess(cams, fo, g.means, g.scales, g.quats)
    return pre, O.bin_and_sort(cams, fo, pre), cams


def _pairs(pre, b, cams, rows, chunk=8192):
    """Per (list entry, wave): whether some pixel passes the per-pixel test,
    and the box test's verdict in both contraction patterns."""
    W = cams[0].W
    tiles_x = (W + 15) // 16
    ntiles = tiles_x * ((cams[0].H + 15) // 16)
    keys, vals = b["keys"], b["vals"]
    waves = 16 // rows
    out = []
    for s in range(0, len(keys), chunk):
        k = keys[s:s + chunk]
        gi = vals[s:s + chunk].astype(np.int64)
        t = (k >> np.uint64(32)).astype(np.int64) % ntiles
        ty, tx = t // tiles_x, t % tiles_x
        u, v = pre["mean2d"][gi, 0], pre["mean2d"][gi, 1]
        A, B, C = (pre["conic"][gi, j] for j in range(3))
        gz, gw, gbx = SCALE_A * A, SCALE_B * B, SCALE_A * C  # the staged A', B', C'
        for wv in range(waves):
            X0 = (tx * 16).astype(f32) + f32(0.5)
            Y0 = (ty * 16 + rows * wv).astype(f32) + f32(0.5)
            fx = X0[:, None] + np.arange(16, dtype=f32)[None, :]
            fy = Y0[:, None] + np.arange(rows, dtype=f32)[None, :]
            dx = (fx - u[:, None]).astype(f32)
            dy = (fy - v[:, None]).astype(f32)
            ta = ((gz[:, None] * dx).astype(f32) * dx).astype(f32)
            tb = (gw[:, None] * dx).astype(f32)
            # power = fma(tb, dy, fma(dy, C' dy, ta)) over the wave's rows x columns
            cdy = (gbx[:, None] * dy).astype(f32)
            inner = _fma(dy[:, :, None], cdy[:, :, None], ta[:, None, :])
            power = _fma(tb[:, None, :], dy[:, :, None], inner)
            passes = (power >= P2_MIN).reshape(len(gi), -1).any(axis=1)
            verdict = [_box(u, v, gz, gw, gbx, X0, X0 + f32(15), Y0, Y0 + f32(rows - 1), fused)
                       for fused in (True, False)]
            out.append((passes, verdict[0], verdict[1]))
    return [np.concatenate(c) for c in zip(*out)]


def _box(u, v, gz, gw, gbx, X0, X1, Y0, Y1, fused):
    """may_reach of the raster kernel, vectorised, in its operation order."""
    x0, x1 = (X0 - u).astype(f32), (X1 - u).astype(f32)
    y0, y1 = (Y0 - v).astype(f32), (Y1 - v).astype(f32)
    inside = (x0 <= 0) & (x1 >= 0) & (y0 <= 0) & (y1 >= 0)
    a, b, c = -gz, -gw, -gbx
    degenerate = ~((a > f32(1e-30)) & (c > f32(1e-30)))
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        ia, ic = (f32(0.5) / a).astype(f32), (f32(0.5) / c).astype(f32)

        def q(dx, dy):
            axx = ((a * dx).astype(f32) * dx).astype(f32)
            if fused:
                t = _fma((c * dy).astype(f32), dy, axx)
                return _fma((b * dx).astype(f32), dy, t)
            cyy = ((c * dy).astype(f32) * dy).astype(f32)
            bxy = ((b * dx).astype(f32) * dy).astype(f32)
            return ((axx + cyy).astype(f32) + bxy).astype(f32)

        def clamp(val, lo, hi):
            return np.minimum(np.maximum(val, lo), hi).astype(f32)

        m = q(x0, clamp(((-b * x0).astype(f32) * ic).astype(f32), y0, y1))
        m = np.minimum(m, q(x1, clamp(((-b * x1).astype(f32) * ic).astype(f32), y0, y1)))
        m = np.minimum(m, q(clamp(((-b * y0).astype(f32) * ia).astype(f32), x0, x1), y0))
        m = np.minimum(m, q(clamp(((-b * y1).astype(f32) * ia).astype(f32), x0, x1), y1))
        xm, ym = np.maximum(np.abs(x0), np.abs(x1)), np.maximum(np.abs(y0), np.abs(y1))
        M = (((a * xm).astype(f32) * xm + (c * ym).astype(f32) * ym).astype(f32)
             + (np.abs(b) * xm).astype(f32) * ym).astype(f32)
        keep = ~(m > (-P2_MIN + (f32(4e-6) * M).astype(f32) + f32(1.5e-4)).astype(f32))
    return inside | degenerate | keep


@pytest.mark.parametrize("thin,seed", [((3e-3, 1e-2, 0.1, 0.5), 41), ((1e-4, 1e-3, 0.2, 1.0), 42),
                                       ((1e-5, 1e-4, 0.5, 1.5), 43)])
def test_box_test_keeps_every_gaussian_a_pixel_takes(thin, seed):
    pre, b, cams = _scene(seed, 2, thin)
    vis = pre["tiles"] > 0
    A, B, C = (pre["conic"][vis, k].astype(np.float64) for k in range(3))
    ev = np.sqrt(((A - C) / 2) ** 2 + B ** 2)
    cond = ((A + C) / 2 + ev) / np.maximum((A + C) / 2 - ev, 1e-300)
    assert cond.max() > 1e4
    for rows in (4, 8):
        passes, keep_fused, keep_plain = _pairs(pre, b, cams, rows)
        for keep in (keep_fused, keep_plain):
            assert not np.any(passes & ~keep), "the box test dropped a Gaussian a pixel takes"
        # and it is not vacuous: most pairs no pixel takes are dropped
        idle = ~passes
        assert idle.sum() > 0.3 * passes.size
        assert (idle & ~keep_fused).sum() > 0.5 * idle.sum()
