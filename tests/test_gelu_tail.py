"""The fp16 decoder's GELU tail (decode_common.h): Q(w) = 1 - Phi(w) as
2^P(min(w, 6)), P the degree-7 polynomial whose coefficients the header
holds.  Evaluated here as the kernels evaluate it (Horner in fp32 with fused
multiply-adds, then exp2) and compared with scipy's normal tail: the relative
error bounds the header states, and GELU = max(x, 0) - |x| Q against the erf
form within what an fp16 result can resolve."""
import os
import re

import numpy as np
from scipy.special import erf, log_ndtr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _coefficients():
    text = open(os.path.join(ROOT, "implicit_attribute_decode_amd", "csrc", "decode_common.h")).read()
    body = text[text.index("normal_tail(float w)"):text.index("__builtin_amdgcn_exp2f(p);")]
    vals = [float(v) for v in re.findall(r"([-+]?\d\.\d+e[-+]\d+)f", body)]
    assert len(vals) == 8
    return np.float32(vals[::-1])  # lowest order first


def _q(w):
    c = _coefficients()
    v = np.minimum(w.astype(np.float32), np.float32(6.0))
    acc = np.full(v.shape, c[-1], np.float32)
    for k in range(len(c) - 2, -1, -1):
        acc = (acc.astype(np.float64) * v + np.float64(c[k])).astype(np.float32)  # one rounding: a fused multiply-add
    return np.exp2(acc.astype(np.float64))


def test_tail_relative_error_bounds():
    w = np.linspace(0.0, 6.0, 300001).astype(np.float32)
    exact = np.exp(log_ndtr(-w.astype(np.float64)))
    rel = np.abs(_q(w) / exact - 1.0)
    assert rel[w < 4.3].max() <= 3.9e-6, rel[w < 4.3].max()
    assert rel.max() <= 4.6e-6, rel.max()


def test_gelu_against_the_erf_form():
    x = np.linspace(-12.0, 12.0, 480001).astype(np.float32)
    g = np.maximum(x, 0.0) - np.abs(x) * _q(np.abs(x))
    exact = 0.5 * x.astype(np.float64) * (1.0 + erf(x.astype(np.float64) / np.sqrt(2.0)))
    err = np.abs(g - exact)
    # |x| <= 6: fp16 keeps 11 significant bits, and the error stays far below
    # half an fp16 step of the value (or of fp16's smallest normal, 2^-14)
    inner = np.abs(x) <= 6.0
    step = np.maximum(np.abs(exact), 2.0 ** -14) * 2.0 ** -11
    assert (err[inner] <= 0.01 * step[inner]).all(), float((err / step)[inner].max())
    # x < -6: |x| Q(6) instead of |x| Q(|x|) (the clamp), below half of fp16's
    # smallest subnormal step, so the fp16 result is zero as the exact one is
    assert (np.abs(g[x < -6.0]) < 2.0 ** -25).all()
    assert (err[x > 6.0] <= 1e-8 * x[x > 6.0]).all()
