"""Coefficients of the fp16 decoder's GELU tail (decode_common.h).

GELU(x) = x Phi(x) = max(x, 0) - |x| Q(|x|), with Q(w) = 1 - Phi(w) the
upper tail of the standard normal distribution.  The kernels evaluate
Q(w) = 2^P(w) for w = min(|x|, W), P a polynomial of degree `DEG` in w fitted
here to log2 Q(w) on [0, W]: one exponential per value, no reciprocal.
log2 Q is smooth on the whole half-line (Q has no real zero), so a low degree
polynomial reaches the fp32 evaluation floor.  The fit is least squares on a
dense grid of Chebyshev nodes, refined by Lawson's iteration towards the
minimax error; it prints the coefficients (lowest order first) and the
largest relative error of Q evaluated as the kernels do (Horner in fp32 with
fused multiply-adds, exp2), on [0, W] and on the range that matters for the
fp16 hidden activations (|x| Q(|x|) above fp16's smallest normal number,
w < 4.3).  Run: python gen_gelu_tail.py
"""
import numpy as np
from scipy.special import log_ndtr

W = 6.0
DEG = 7


def log2_tail(w):
    return log_ndtr(-w) / np.log(2.0)


def fit(deg, w_max, iters=30):
    u = np.cos(np.pi * (np.arange(4000) + 0.5) / 4000)  # Chebyshev nodes on [-1, 1]
    w = 0.5 * w_max * (u + 1.0)
    y = log2_tail(w)
    V = np.vander(w, deg + 1, increasing=True)
    wt = np.ones_like(w)
    for _ in range(iters):  # Lawson: reweight by the error towards equal ripple
        c, *_ = np.linalg.lstsq(V * wt[:, None], y * wt, rcond=None)
        err = np.abs(V @ c - y)
        wt = wt * (err / err.max() + 1e-3)
        wt /= wt.max()
    return c


def fma32(a, b, c):
    # fp32 fused multiply-add: exact product and sum in fp64, one rounding to fp32
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def q_kernel(c32, w):
    acc = np.full(w.shape, c32[-1], np.float32)
    for k in range(len(c32) - 2, -1, -1):
        acc = fma32(acc, w, np.full(w.shape, c32[k], np.float32))
    return np.exp2(acc.astype(np.float64))


if __name__ == "__main__":
    c = fit(DEG, W)
    c32 = c.astype(np.float32)
    w = np.linspace(0.0, W, 600001).astype(np.float32)
    rel = np.abs(q_kernel(c32, w) / np.exp2(log2_tail(w.astype(np.float64))) - 1.0)
    print(f"degree {DEG} on [0, {W}]: max relative error of Q {rel.max():.3e} (w < 4.3: {rel[w < 4.3].max():.3e})")
    print("coefficients, lowest order first:")
    for v in c32:
        print(f"    {float(v):.9e}f,")
