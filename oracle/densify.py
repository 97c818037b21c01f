"""CPU oracle for the refinement of the positions (densify and prune).  TEST
INFRASTRUCTURE, not the product path: only tests/, the smoke check and the
benchmark's CPU-baseline leg may use it, and it never imports the HIP library
or its Python binding.

[SPIN] §3.2 Eq. 6 refines the estimated positions with the rendering loss,
densifying salient points and pruning unnecessary ones, and names no rule of
its own; the rule read here is the adaptive density control of 3D Gaussian
Splatting, applied to the trainable positions (the other attributes come
from the decoder):

* salient: the mean, over the iterations in which the Gaussian received a
  position gradient, of that gradient's norm is at least grad_threshold;
* a salient Gaussian whose largest decoded scale is at most scale_threshold
  is cloned (kept, plus a copy at the same position whose Adam moments start
  at zero);
* a salient Gaussian with a larger scale is split: it is replaced by two
  Gaussians at mu + R(q) (s * n_j), j = 0, 1, with n_j standard normal draws
  the caller passes in (so both sides use the same random numbers), their
  moments zero;
* a Gaussian whose decoded opacity is below min_opacity is pruned (before
  any of the above);
* every other Gaussian is kept with its moments.
The output keeps the input order (a Gaussian's outputs sit where its
predecessors' end).  Time (the fourth coordinate) is carried unchanged.

The decisions compare fp32 values in fp32 (the mean gradient is one fp32
division), exactly as the kernel takes them; the split positions are fp64.
"""
from __future__ import annotations

import numpy as np

KEEP, PRUNE, CLONE, SPLIT = 1, 0, 2, 3


def decide(grad_acc, grad_count, scale_max, opacity, grad_threshold, scale_threshold, min_opacity):
    """Per Gaussian: PRUNE, KEEP, CLONE or SPLIT (fp32 comparisons)."""
    g = np.asarray(grad_acc, np.float32)
    cnt = np.asarray(grad_count, np.int64)
    smax = np.asarray(scale_max, np.float32)
    op = np.asarray(opacity, np.float32)
    mean = np.zeros_like(g)
    seen = cnt > 0
    mean[seen] = (g[seen] / cnt[seen].astype(np.float32)).astype(np.float32)
    salient = seen & (mean >= np.float32(grad_threshold))
    out = np.full(g.shape, KEEP, np.int64)
    out[salient & (smax <= np.float32(scale_threshold))] = CLONE
    out[salient & (smax > np.float32(scale_threshold))] = SPLIT
    out[op < np.float32(min_opacity)] = PRUNE
    return out


def quat_to_matrix(q):
    """Rotation matrix of the quaternion (w, x, y, z), normalised first."""
    q = np.asarray(q, np.float64)
    q = q / np.linalg.norm(q)
    w, x, y, z = q
    return np.array([[1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)],
                      [2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)],
                      [2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)]])


def densify(xyzt, grad_acc, grad_count, scales, quats, opacity, noise, m, v,
            grad_threshold, scale_threshold, min_opacity):
    """Returns (xyzt', m', v', decisions): the refined positions [M, 4] and
    their Adam moments [M, 3] in input order.  noise: [N, 2, 3] normal draws
    for the two children of a split."""
    xyzt = np.asarray(xyzt, np.float64)
    scales = np.asarray(scales, np.float64)
    m = np.asarray(m, np.float64)
    v = np.asarray(v, np.float64)
    noise = np.asarray(noise, np.float64)
    dec = decide(grad_acc, grad_count, np.asarray(scales, np.float32).max(axis=1), opacity,
                 grad_threshold, scale_threshold, min_opacity)
    out_p, out_m, out_v = [], [], []
    zero = np.zeros(3)
    for i, d in enumerate(dec):
        if d == KEEP:
            out_p.append(xyzt[i]); out_m.append(m[i]); out_v.append(v[i])
        elif d == CLONE:
            out_p += [xyzt[i], xyzt[i]]; out_m += [m[i], zero]; out_v += [v[i], zero]
        elif d == SPLIT:
            R = quat_to_matrix(quats[i])
            for j in range(2):
                c = xyzt[i, :3] + R @ (scales[i] * noise[i, j])
                out_p.append(np.array([c[0], c[1], c[2], xyzt[i, 3]]))
                out_m.append(zero); out_v.append(zero)
    if not out_p:
        return np.zeros((0, 4)), np.zeros((0, 3)), np.zeros((0, 3)), dec
    return np.array(out_p), np.array(out_m), np.array(out_v), dec
