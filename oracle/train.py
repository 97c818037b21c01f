"""CPU oracle for the training objective and the optimiser step.  TEST
INFRASTRUCTURE, not the product path: only tests/, the smoke check and the
benchmark's CPU-baseline leg may use it, and it never imports the HIP library
or its Python binding.

Plain numpy in fp64, following the pages' text:

* image loss, [SPIN] §3.3 Eq. 12: L = (1 - lambda) L1 + lambda L_D-SSIM with
  lambda = 0.2 (the value the pages take from 3DGS).  L1 is the mean absolute
  difference; L_D-SSIM = 1 - SSIM.  SSIM is the structural similarity index of
  Wang et al. (2004), which the pages cite for their metric: an 11 x 11
  Gaussian window of standard deviation 1.5, C1 = 0.01^2, C2 = 0.03^2 (pixel
  values in [0, 1]), computed per colour channel, with the window's taps that
  fall outside the image contributing zero, and averaged over every pixel,
  channel and frame.
* the gradient of L with respect to every pixel of the rendered image,
  written out from the SSIM definition (the pins check it against finite
  differences);
* one Adam step (Kingma & Ba, 2015, the optimiser the pages name in §4
  implementation details), with bias correction.
"""
from __future__ import annotations

import math

import numpy as np

SSIM_WINDOW = 11
SSIM_SIGMA = 1.5
SSIM_C1 = 0.01 ** 2
SSIM_C2 = 0.03 ** 2
LAMBDA = 0.2


def gaussian_window(size: int = SSIM_WINDOW, sigma: float = SSIM_SIGMA) -> np.ndarray:
    """1-D Gaussian taps exp(-d^2 / (2 sigma^2)), d = -5..5, normalised to sum 1;
    the 2-D window is their outer product."""
    d = np.arange(size, dtype=np.float64) - (size - 1) / 2.0
    g = np.exp(-(d * d) / (2.0 * sigma * sigma))
    return g / g.sum()


def _blur_axis(a: np.ndarray, w: np.ndarray, axis: int) -> np.ndarray:
    """Window-weighted sum along one axis, taps outside the image zero."""
    r = (len(w) - 1) // 2
    pad = [(0, 0)] * a.ndim
    pad[axis] = (r, r)
    p = np.pad(a, pad)
    out = np.zeros_like(a)
    n = a.shape[axis]
    for k, wk in enumerate(w):
        sl = [slice(None)] * a.ndim
        sl[axis] = slice(k, k + n)
        out += wk * p[tuple(sl)]
    return out


def blur(a: np.ndarray, w: np.ndarray | None = None) -> np.ndarray:
    """The 2-D Gaussian window applied to the last two axes (rows, columns)."""
    w = gaussian_window() if w is None else w
    return _blur_axis(_blur_axis(a, w, a.ndim - 1), w, a.ndim - 2)


def ssim_map(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    """Per-pixel SSIM of images x, y ([..., H, W], fp64): with windowed means
    mu, variances sigma^2 and covariance sigma_xy,
    S = (2 mu_x mu_y + C1)(2 sigma_xy + C2) / ((mu_x^2 + mu_y^2 + C1)(sigma_x^2 + sigma_y^2 + C2))."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    mx, my = blur(x), blur(y)
    sxx = blur(x * x) - mx * mx
    syy = blur(y * y) - my * my
    sxy = blur(x * y) - mx * my
    return ((2 * mx * my + SSIM_C1) * (2 * sxy + SSIM_C2)) / ((mx * mx + my * my + SSIM_C1) * (sxx + syy + SSIM_C2))


def image_loss(image: np.ndarray, target: np.ndarray, lam: float = LAMBDA) -> dict:
    """Eq. 12 on images [F, 3, H, W]: the loss, its two terms and dL/dimage.

    dSSIM/dx(p) = (1/n) sum_q w(q - p) [dS_q/dmu_x + 2 x(p) dS_q/dE[x^2] + y(p) dS_q/dE[xy]]
    with, at every q (A1 = 2 mu_x mu_y + C1, A2 = 2 sigma_xy + C2,
    B1 = mu_x^2 + mu_y^2 + C1, B2 = sigma_x^2 + sigma_y^2 + C2):
      dS/dmu_x   = S (2 mu_y / A1 - 2 mu_y / A2 - 2 mu_x / B1 + 2 mu_x / B2)
      dS/dE[x^2] = -S / B2
      dS/dE[xy]  = 2 S / A2
    (sigma_x^2 = E[x^2] - mu_x^2 and sigma_xy = E[xy] - mu_x mu_y); the window is
    symmetric, so its adjoint is the same zero-padded window sum."""
    x = np.asarray(image, np.float64)
    y = np.asarray(target, np.float64)
    n = x.size
    diff = x - y
    l1 = np.abs(diff).sum() / n
    mx, my = blur(x), blur(y)
    sxx = blur(x * x) - mx * mx
    syy = blur(y * y) - my * my
    sxy = blur(x * y) - mx * my
    a1 = 2 * mx * my + SSIM_C1
    a2 = 2 * sxy + SSIM_C2
    b1 = mx * mx + my * my + SSIM_C1
    b2 = sxx + syy + SSIM_C2
    s = (a1 * a2) / (b1 * b2)
    ssim = s.sum() / n
    d_mx = s * (2 * my / a1 - 2 * my / a2 - 2 * mx / b1 + 2 * mx / b2)
    d_exx = -s / b2
    d_exy = 2 * s / a2
    dssim = (blur(d_mx) + 2 * x * blur(d_exx) + y * blur(d_exy)) / n
    grad = (1.0 - lam) * np.sign(diff) / n - lam * dssim
    return {"loss": (1.0 - lam) * l1 + lam * (1.0 - ssim), "l1": l1, "ssim": ssim, "grad": grad}


def adam_step(p, g, m, v, lr: float, beta1: float, beta2: float, eps: float, step: int):
    """One Adam update (Kingma & Ba, 2015, Algorithm 1) at step t = step >= 1:
    m = b1 m + (1 - b1) g, v = b2 v + (1 - b2) g^2,
    p = p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps).  Returns (p, m, v)."""
    p = np.asarray(p, np.float64)
    g = np.asarray(g, np.float64)
    m = beta1 * np.asarray(m, np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, np.float64) + (1.0 - beta2) * g * g
    mh = m / (1.0 - beta1 ** step)
    vh = v / (1.0 - beta2 ** step)
    return p - lr * mh / (np.sqrt(vh) + eps), m, v


def lr_schedule(step: int, base: float, warmup: int, total: int, final: float = 1e-7) -> float:
    """Linear warm-up over `warmup` steps, then cosine decay from base to final
    at `total` ([SPIN] §4 implementation details; the warm-up length is not
    given there)."""
    if warmup > 0 and step < warmup:
        return base * (step + 1) / warmup
    t = min(max(step - warmup, 0), max(total - warmup, 1)) / max(total - warmup, 1)
    return final + 0.5 * (base - final) * (1.0 + math.cos(math.pi * t))
