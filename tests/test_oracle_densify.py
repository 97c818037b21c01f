"""Pins of the densify / prune oracle (oracle/densify.py) against what the
rule fixes: counts and order, clones as exact copies, split children as
samples of the Gaussian (checked with scipy's rotation and by their spread),
pruning first, and the degenerate cases."""
import numpy as np
from scipy.spatial.transform import Rotation

from oracle import densify as Dn


def _case(n, seed=0):
    rng = np.random.default_rng(seed)
    xyzt = np.concatenate([rng.normal(0, 1, (n, 3)), rng.uniform(0, 1, (n, 1))], 1).astype(np.float32)
    acc = rng.uniform(0, 4e-4, n).astype(np.float32)
    cnt = rng.integers(0, 3, n).astype(np.int32)
    scales = np.exp(rng.uniform(-6, -2, (n, 3))).astype(np.float32)
    quats = rng.normal(0, 1, (n, 4)).astype(np.float32)
    opac = rng.uniform(0, 1, n).astype(np.float32)
    noise = rng.normal(0, 1, (n, 2, 3)).astype(np.float32)
    m = rng.normal(0, 1e-3, (n, 3)).astype(np.float32)
    v = rng.uniform(0, 1e-6, (n, 3)).astype(np.float32)
    return xyzt, acc, cnt, scales, quats, opac, noise, m, v


def test_decisions_and_output_layout():
    xyzt, acc, cnt, scales, quats, opac, noise, m, v = _case(2000)
    P, M, V, dec = Dn.densify(xyzt, acc, cnt, scales, quats, opac, noise, m, v, 1e-4, 0.05, 0.005)
    k = np.choose(dec, [0, 1, 2, 2])
    assert len(P) == k.sum() == len(M) == len(V)
    # every kind occurs in this case
    assert {Dn.PRUNE, Dn.KEEP, Dn.CLONE, Dn.SPLIT} <= set(dec.tolist())
    off = np.concatenate([[0], np.cumsum(k)[:-1]])
    for i in range(len(dec)):
        o = off[i]
        if dec[i] == Dn.KEEP:
            assert np.array_equal(P[o], xyzt[i]) and np.array_equal(M[o], m[i]) and np.array_equal(V[o], v[i])
        elif dec[i] == Dn.CLONE:
            assert np.array_equal(P[o], xyzt[i]) and np.array_equal(P[o + 1], xyzt[i])
            assert np.array_equal(M[o], m[i]) and not M[o + 1].any() and not V[o + 1].any()
        elif dec[i] == Dn.SPLIT:
            assert P[o, 3] == xyzt[i, 3] and P[o + 1, 3] == xyzt[i, 3] and not M[o:o + 2].any()


def test_rule_thresholds_by_hand():
    acc = np.array([3e-4, 3e-4, 3e-4, 1e-4, 3e-4, 0.0], np.float32)
    cnt = np.array([2, 2, 2, 2, 0, 0], np.int32)  # mean 1.5e-4 for the first three, 5e-5, unseen, unseen
    smax = np.array([0.01, 0.2, 0.01, 0.2, 0.2, 0.2], np.float32)
    op = np.array([0.5, 0.5, 0.001, 0.5, 0.5, 0.5], np.float32)
    d = Dn.decide(acc, cnt, smax, op, 1e-4, 0.05, 0.005)
    assert d.tolist() == [Dn.CLONE, Dn.SPLIT, Dn.PRUNE, Dn.KEEP, Dn.KEEP, Dn.KEEP]
    # the threshold itself counts as salient (>=), the scale threshold as small (<=)
    d = Dn.decide(np.float32([2e-4]), [2], np.float32([0.05]), np.float32([0.005]), 1e-4, 0.05, 0.005)
    assert d.tolist() == [Dn.CLONE]


def test_split_children_match_scipy_rotation():
    xyzt, acc, cnt, scales, quats, opac, noise, m, v = _case(300, seed=3)
    P, M, V, dec = Dn.densify(xyzt, acc, cnt, scales, quats, opac, noise, m, v, 0.0, 0.0, 0.0)
    # every seen Gaussian is salient with scale > 0: all of those split
    k = np.choose(dec, [0, 1, 2, 2])
    off = np.concatenate([[0], np.cumsum(k)[:-1]])
    q = quats.astype(np.float64)
    Rs = Rotation.from_quat(np.concatenate([q[:, 1:], q[:, :1]], 1)).as_matrix()  # scipy: (x, y, z, w)
    checked = 0
    for i in np.nonzero(dec == Dn.SPLIT)[0]:
        for j in range(2):
            want = xyzt[i, :3].astype(np.float64) + Rs[i] @ (scales[i].astype(np.float64) * noise[i, j])
            assert np.abs(P[off[i] + j, :3] - want).max() < 1e-12
            checked += 1
    assert checked > 100


def test_split_children_spread_like_the_gaussian():
    """Many children of one Gaussian have the Gaussian's covariance R S^2 R^T."""
    rng = np.random.default_rng(7)
    n = 40000
    q = np.array([0.9, 0.1, -0.3, 0.2], np.float32)
    s = np.array([0.3, 0.05, 0.1], np.float32)
    P, _, _, dec = Dn.densify(np.zeros((n, 4), np.float32), np.ones(n, np.float32), np.ones(n, np.int32),
                              np.tile(s, (n, 1)), np.tile(q, (n, 1)), np.ones(n, np.float32),
                              rng.normal(0, 1, (n, 2, 3)), np.zeros((n, 3)), np.zeros((n, 3)), 0.5, 0.01, 0.0)
    assert (dec == Dn.SPLIT).all() and len(P) == 2 * n
    R = Dn.quat_to_matrix(q)
    cov = R @ np.diag(s.astype(np.float64) ** 2) @ R.T
    emp = np.cov(P[:, :3].T)
    assert np.abs(emp - cov).max() < 0.03 * np.abs(cov).max()
    assert np.abs(P[:, :3].mean(0)).max() < 5e-3


def test_degenerate_cases():
    xyzt, acc, cnt, scales, quats, opac, noise, m, v = _case(50, seed=5)
    # nothing salient, nothing pruned: identity
    P, M, V, dec = Dn.densify(xyzt, acc, cnt, scales, quats, opac, noise, m, v, 1.0, 0.05, 0.0)
    assert np.array_equal(P, xyzt) and np.array_equal(M, m) and np.array_equal(V, v)
    # everything pruned
    P, M, V, dec = Dn.densify(xyzt, acc, cnt, scales, quats, opac, noise, m, v, 1.0, 0.05, 2.0)
    assert P.shape == (0, 4) and (dec == Dn.PRUNE).all()
    # no Gaussians
    e = np.zeros((0,))
    P, M, V, dec = Dn.densify(np.zeros((0, 4)), e, e, np.zeros((0, 3)), np.zeros((0, 4)), e, np.zeros((0, 2, 3)),
                              np.zeros((0, 3)), np.zeros((0, 3)), 1e-4, 0.05, 0.005)
    assert P.shape == (0, 4)
