"""GPU parity of the refinement of the positions (densify / prune, [SPIN]
§3.2 Eq. 6 read as 3DGS's clone / split / prune rule) against
oracle/densify.py, through the C ABI.

The decisions and the order are integer results: equal.  Kept and cloned
rows and every moment are copies: bit-exact.  Split children are computed
in fp32 (quaternion normalisation, rotation, one product and three sums per
coordinate): within 1e-6 (|mu| + sum |R (s * n)|) of the fp64 oracle.  The
accumulated gradient norms are the same fp32 operations on both sides:
bit-exact.
"""
import numpy as np
import pytest
import torch

from oracle import densify as Dn
from implicit_attribute_decode_amd import ia
from implicit_attribute_decode_amd.pipeline import densify_positions

from gpu_util import cuda, host, say

pytestmark = pytest.mark.gpu


def _case(n, seed):
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


def _gpu(xyzt, acc, cnt, scales, quats, opac, noise, m, v, th):
    attrs = {"scales": cuda(scales), "quats": cuda(quats), "opacity": cuda(opac)}
    P, M, V = densify_positions(cuda(xyzt), cuda(acc), cuda(cnt), attrs, cuda(m), cuda(v), cuda(noise), *th)
    torch.cuda.synchronize()
    return host(P), host(M), host(V)


@pytest.mark.parametrize("n,seed", [(1, 1), (4097, 2), (200_003, 3)])
def test_densify_matches_oracle(n, seed):
    case = _case(n, seed)
    th = (1e-4, 0.05, 0.005)
    P, M, V = _gpu(*case, th)
    oP, oM, oV, dec = Dn.densify(*case, *th)
    say(f"n={n}: {len(oP)} rows, kinds {np.bincount(dec, minlength=4).tolist()}")
    assert P.shape == oP.shape
    assert np.array_equal(M, oM.astype(np.float32)) and np.array_equal(V, oV.astype(np.float32))
    k = np.choose(dec, [0, 1, 2, 2])
    off = np.concatenate([[0], np.cumsum(k)[:-1]]).astype(np.int64)
    exact = np.concatenate([off[(dec == Dn.KEEP) | (dec == Dn.CLONE)], off[dec == Dn.CLONE] + 1])
    assert np.array_equal(P[exact], oP[exact].astype(np.float32))
    split = np.nonzero(dec == Dn.SPLIT)[0]
    if len(split):
        rows = np.concatenate([off[split], off[split] + 1])
        xyzt, _, _, scales, _, _, noise, _, _ = case
        src = np.concatenate([split, split])
        j = np.concatenate([np.zeros(len(split), int), np.ones(len(split), int)])
        mag = np.abs(xyzt[src, :3]).max(1) + (np.abs(scales[src]) * np.abs(noise[src, j])).sum(1) * 3
        err = np.abs(P[rows, :3] - oP[rows, :3]).max(1)
        assert np.all(err <= 1e-6 * mag), float((err / mag).max())
        assert np.array_equal(P[rows, 3], oP[rows, 3].astype(np.float32))


def test_densify_degenerate_cases():
    case = list(_case(3000, 9))
    # nothing salient, nothing pruned: identity
    P, M, V = _gpu(*case, (1.0, 0.05, 0.0))
    assert np.array_equal(P, case[0]) and np.array_equal(M, case[7]) and np.array_equal(V, case[8])
    # everything pruned
    P, M, V = _gpu(*case, (1e-4, 0.05, 2.0))
    assert P.shape == (0, 4)
    # no Gaussians
    e = [np.zeros((0,) + a.shape[1:], a.dtype) for a in case]
    P, M, V = _gpu(*e, (1e-4, 0.05, 0.005))
    assert P.shape == (0, 4)


def test_densify_rejects_bad_arguments():
    case = _case(100, 4)
    d = [cuda(a) for a in case]
    out_x = torch.empty((150, 4), device="cuda")  # < 2 N
    out_m = torch.empty((150, 3), device="cuda")
    out_v = torch.empty((150, 3), device="cuda")
    out_n = torch.zeros(1, dtype=torch.int64, device="cuda")
    ws = torch.empty(ia.ia_densify_workspace_size(100), dtype=torch.uint8, device="cuda")
    with pytest.raises(ia.IAError) as e:
        ia.ia_densify(*d, ia.DensifyParams(1e-4, 0.05, 0.005), out_x, out_m, out_v, out_n, ws)
    assert e.value.status == ia.IA_ERR_INVALID_ARG
    out_x = torch.empty((200, 4), device="cuda")
    out_m = torch.empty((200, 3), device="cuda")
    out_v = torch.empty((200, 3), device="cuda")
    with pytest.raises(ia.IAError) as e:
        ia.ia_densify(*d, ia.DensifyParams(-1.0, 0.05, 0.005), out_x, out_m, out_v, out_n, ws)
    assert e.value.status == ia.IA_ERR_INVALID_ARG
    with pytest.raises(ia.IAError) as e:
        ia.ia_densify(*d, ia.DensifyParams(1e-4, 0.05, 0.005), out_x, out_m, out_v, out_n, ws[:0])
    assert e.value.status == ia.IA_ERR_WORKSPACE_TOO_SMALL


def test_accumulate_matches_fp32_formula():
    rng = np.random.default_rng(6)
    n = 100_001
    g = rng.normal(0, 1e-4, (n, 3)).astype(np.float32)
    g[::7] = 0.0
    acc0 = rng.uniform(0, 1e-3, n).astype(np.float32)
    cnt0 = rng.integers(0, 5, n).astype(np.int32)
    A, Cn = cuda(acc0), cuda(cnt0)
    for _ in range(2):
        ia.ia_densify_accumulate(cuda(g), A, Cn)
    torch.cuda.synchronize()
    nrm = np.sqrt((g[:, 0] * g[:, 0] + g[:, 1] * g[:, 1]) + g[:, 2] * g[:, 2]).astype(np.float32)
    want = acc0.copy()
    for _ in range(2):
        want = np.where(nrm > 0, (want + nrm).astype(np.float32), want)
    assert np.array_equal(host(A), want)
    assert np.array_equal(host(Cn), cnt0 + 2 * (nrm > 0))


def test_densify_stress_size_sampled():
    """8M positions (the Stress batch): every decision, the row count and the
    offsets from the oracle's vectorised rule; 3000 sampled Gaussians' rows
    against the oracle one by one."""
    n = 8_000_000
    case = _case(n, 12)
    th = (1e-4, 0.05, 0.005)
    P, M, V = _gpu(*case, th)
    xyzt, acc, cnt, scales, quats, opac, noise, m, v = case
    dec = Dn.decide(acc, cnt, scales.max(axis=1), opac, *th)
    k = np.choose(dec, [0, 1, 2, 2])
    off = np.concatenate([[0], np.cumsum(k)[:-1]])
    assert len(P) == int(k.sum())
    rng = np.random.default_rng(13)
    for i in rng.choice(n, 3000, replace=False):
        oP, oM, oV, d1 = Dn.densify(*[a[i:i + 1] for a in case], *th)
        assert d1[0] == dec[i]
        rows = slice(off[i], off[i] + k[i])
        assert np.array_equal(M[rows], oM.astype(np.float32)) and np.array_equal(V[rows], oV.astype(np.float32))
        if dec[i] == Dn.SPLIT:
            mag = np.abs(xyzt[i, :3]).max() + 3 * (np.abs(scales[i]) * np.abs(noise[i]).max()).sum()
            assert np.abs(P[rows, :3] - oP[:, :3]).max() <= 1e-6 * mag
        else:
            assert np.array_equal(P[rows], oP.astype(np.float32))
