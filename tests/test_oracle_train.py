"""Pins of the training-objective oracle (oracle/train.py) against what the
mathematics fixes: SSIM's special cases, a brute-force window sum, finite
differences of the loss, and Adam's closed forms ([SPIN] §3.3 Eq. 12, §4
implementation details; SSIM of Wang et al. 2004; Adam of Kingma & Ba 2015)."""
import math

import numpy as np

from oracle import train as T


def test_window_normalised_symmetric_and_sigma():
    w = T.gaussian_window()
    assert w.shape == (11,)
    assert abs(w.sum() - 1.0) < 1e-15
    assert np.allclose(w, w[::-1], rtol=0, atol=0)
    # ratio of neighbouring taps exp(-((d+1)^2 - d^2) / (2 sigma^2))
    d = np.arange(-5, 5)
    assert np.allclose(w[1:] / w[:-1], np.exp(-((d + 1) ** 2 - d ** 2) / (2 * 1.5 ** 2)), rtol=1e-13)


def test_ssim_of_an_image_with_itself_is_one():
    rng = np.random.default_rng(0)
    x = rng.uniform(0, 1, (2, 3, 17, 23))
    assert np.abs(T.ssim_map(x, x) - 1.0).max() < 1e-12
    out = T.image_loss(x, x)
    assert abs(out["ssim"] - 1.0) < 1e-12 and out["l1"] == 0.0 and abs(out["loss"]) < 1e-12
    # SSIM is maximal at x = y, and L1's subgradient is taken as 0 there
    assert np.abs(out["grad"]).max() < 1e-12


def test_constant_images_closed_form_in_the_interior():
    a, b = 0.3, 0.7
    x = np.full((1, 1, 30, 31), a)
    y = np.full((1, 1, 30, 31), b)
    s = T.ssim_map(x, y)
    want = (2 * a * b + T.SSIM_C1) / (a * a + b * b + T.SSIM_C1)  # variances and covariance vanish
    assert np.abs(s[..., 5:-5, 5:-5] - want).max() < 1e-12
    # at the border the zero taps change the means: not the interior value
    assert abs(s[0, 0, 0, 0] - want) > 1e-3


def test_ssim_map_equals_a_brute_force_window_sum():
    rng = np.random.default_rng(1)
    H, W = 12, 13
    x = rng.uniform(0, 1, (H, W))
    y = rng.uniform(0, 1, (H, W))
    g = T.gaussian_window()
    w2 = np.outer(g, g)
    want = np.zeros((H, W))
    for i in range(H):
        for j in range(W):
            mom = np.zeros(5)
            for di in range(-5, 6):
                for dj in range(-5, 6):
                    ii, jj = i + di, j + dj
                    if 0 <= ii < H and 0 <= jj < W:
                        wt = w2[di + 5, dj + 5]
                        xv, yv = x[ii, jj], y[ii, jj]
                        mom += wt * np.array([xv, yv, xv * xv, yv * yv, xv * yv])
            mx, my, exx, eyy, exy = mom
            sx, sy, sxy = exx - mx * mx, eyy - my * my, exy - mx * my
            want[i, j] = ((2 * mx * my + T.SSIM_C1) * (2 * sxy + T.SSIM_C2)) / (
                (mx * mx + my * my + T.SSIM_C1) * (sx + sy + T.SSIM_C2))
    assert np.abs(T.ssim_map(x, y) - want).max() < 1e-13


def test_loss_gradient_matches_central_differences():
    rng = np.random.default_rng(2)
    x = rng.uniform(0.05, 0.95, (1, 3, 9, 10))
    y = rng.uniform(0.05, 0.95, (1, 3, 9, 10))
    # keep every pixel away from the L1 kink x = y
    y = np.where(np.abs(x - y) < 0.02, y + 0.05, y)
    out = T.image_loss(x, y)
    h = 1e-6
    idx = [(0, c, i, j) for c in range(3) for i in range(9) for j in range(10)]
    num = np.empty(len(idx))
    for k, ix in enumerate(idx):
        xp, xm = x.copy(), x.copy()
        xp[ix] += h
        xm[ix] -= h
        num[k] = (T.image_loss(xp, y)["loss"] - T.image_loss(xm, y)["loss"]) / (2 * h)
    ana = np.array([out["grad"][ix] for ix in idx])
    assert np.abs(ana - num).max() < 1e-8 * max(1.0, np.abs(num).max()) + 1e-9
    # the D-SSIM part alone (lambda = 1) against its own differences
    out1 = T.image_loss(x, y, lam=1.0)
    for ix in idx[::7]:
        xp, xm = x.copy(), x.copy()
        xp[ix] += h
        xm[ix] -= h
        d = (T.image_loss(xp, y, lam=1.0)["loss"] - T.image_loss(xm, y, lam=1.0)["loss"]) / (2 * h)
        assert abs(out1["grad"][ix] - d) < 1e-8


def test_loss_terms_combine_with_lambda_02():
    rng = np.random.default_rng(3)
    x = rng.uniform(0, 1, (1, 3, 16, 16))
    y = rng.uniform(0, 1, (1, 3, 16, 16))
    out = T.image_loss(x, y)
    assert abs(out["l1"] - np.abs(x - y).mean()) < 1e-15
    assert abs(out["loss"] - (0.8 * out["l1"] + 0.2 * (1 - out["ssim"]))) < 1e-15


def test_adam_first_step_is_lr_times_sign():
    """With m = v = 0, bias correction makes the first update lr g / (|g| + eps)."""
    g = np.array([0.5, -2.0, 1e-3, 0.0])
    p0 = np.array([1.0, 1.0, 1.0, 1.0])
    p, m, v = T.adam_step(p0, g, np.zeros(4), np.zeros(4), lr=0.01, beta1=0.9, beta2=0.999, eps=1e-15, step=1)
    assert np.allclose(p, p0 - 0.01 * np.array([1.0, -1.0, 1.0, 0.0]), rtol=0, atol=1e-12)
    assert np.allclose(m, 0.1 * g) and np.allclose(v, 0.001 * g * g)


def test_adam_constant_gradient_moves_lr_per_step():
    """A constant gradient keeps the bias-corrected moments at g and g^2."""
    g = np.array([0.3, -0.7])
    p = np.array([0.0, 0.0])
    m = np.zeros(2)
    v = np.zeros(2)
    for t in range(1, 6):
        p, m, v = T.adam_step(p, g, m, v, lr=1e-3, beta1=0.9, beta2=0.999, eps=0.0, step=t)
    assert np.allclose(p, -5e-3 * np.sign(g), rtol=1e-12, atol=0)


def test_lr_schedule_endpoints():
    base, fin = 8e-3, 1e-7
    assert abs(T.lr_schedule(0, base, 100, 1000) - base / 100) < 1e-18
    assert abs(T.lr_schedule(99, base, 100, 1000) - base) < 1e-18
    assert abs(T.lr_schedule(100, base, 100, 1000) - base) < 1e-18
    assert abs(T.lr_schedule(550, base, 100, 1000) - 0.5 * (base + fin)) < 1e-15
    assert abs(T.lr_schedule(1000, base, 100, 1000) - fin) < 1e-18
    assert abs(T.lr_schedule(5000, base, 100, 1000) - fin) < 1e-18
    assert math.isclose(T.lr_schedule(10, base, 0, 1000), fin + 0.5 * (base - fin) * (1 + math.cos(math.pi * 0.01)))
