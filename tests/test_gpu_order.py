"""ia_spatial_order: the per-frame Morton order of the positions.

It is a storage layout, not a step of the method, so the checks are what
makes it usable in place of the stored order:
  - perm is a permutation that maps every frame's range onto itself, and the
    reordered positions are exactly the permuted ones;
  - the order is exactly the stable sort by (frame, Morton code of the
    normalised position x~ at 10 bits per axis), the codes recomputed here in
    numpy from the oracle's fp32 normalisation (SPIN-4DGS page, §3.3 Eq. 7);
  - rendering the permuted Gaussians gives the same sorted keys and the same
    image bit for bit (the composite follows depth; Gaussians whose depth
    equals another's in the same frame, whose tie order follows the index,
    are made transparent first), and decoding the permuted positions gives
    the permuted attributes within the fp16 decoder's bar.
"""
import numpy as np
import pytest
import torch

import oracle as O
from implicit_attribute_decode_amd import ia, scenes as S
from implicit_attribute_decode_amd.pipeline import Decoder, Renderer, spatial_order

from gpu_util import cuda, host, say

pytestmark = pytest.mark.gpu


def _morton(q):
    code = np.zeros(q.shape[0], np.uint64)
    for b in range(10):
        for k in range(3):
            code |= ((q[:, k].astype(np.uint64) >> np.uint64(b)) & np.uint64(1)) << np.uint64(3 * b + k)
    return code


def _expected_perm(xyz, fo, hash_cfg):
    xt = O.normalize(hash_cfg, np.ascontiguousarray(xyz, np.float32), 0.0)[:, :3].astype(np.float32)
    q = np.where(xt * np.float32(1024.0) >= 1.0, np.minimum(np.floor(xt * np.float32(1024.0)), 1023), 0)
    code = _morton(q.astype(np.int64))
    perm = np.empty(xyz.shape[0], np.int64)
    for f in range(len(fo) - 1):
        lo, hi = int(fo[f]), int(fo[f + 1])
        perm[lo:hi] = lo + np.argsort(code[lo:hi], kind="stable")
    return perm


def test_sequence_frames_order_and_invariance():
    seq = S.Sequence()
    frames = [0, 1, 37, 149]
    xyzt_h = seq.xyzt(frames)
    fo = np.arange(len(frames) + 1, dtype=np.int64) * seq.per_frame
    x = cuda(xyzt_h)
    perm, xo = spatial_order(x, fo)
    torch.cuda.synchronize()
    p = host(perm).astype(np.int64)
    assert np.array_equal(np.sort(p), np.arange(x.shape[0]))
    for f in range(len(frames)):
        seg = p[fo[f]:fo[f + 1]]
        assert seg.min() == fo[f] and seg.max() == fo[f + 1] - 1
    assert np.array_equal(host(xo), xyzt_h[p])
    want = _expected_perm(xyzt_h[:, :3], fo, S.single_hash())
    assert np.array_equal(p, want)
    # deterministic
    perm2, _ = spatial_order(x, fo)
    assert torch.equal(perm, perm2)

    # The render of the permuted Gaussians: the same sorted keys bit for bit
    # and the same image bit for bit.  Equal depths (a 200k frame has about a
    # thousand exactly equal fp32 depths) composite in index order, which the
    # permutation changes, so Gaussians whose depth is shared within their
    # frame get zero opacity (never composited) before comparing images.
    rng = np.random.default_rng(5)
    g = S.render_attributes(rng, xyzt_h[:, :3].copy(), 1e-3, 5e-2)
    cams = [seq.camera(f) for f in frames]
    pre = O.preprocess(cams, fo, xyzt_h[:, :3].copy(), g.scales, g.quats)
    tied = 0
    for f in range(len(frames)):
        lo, hi = int(fo[f]), int(fo[f + 1])
        d = pre["depth"][lo:hi].view(np.uint32)
        vis = pre["tiles"][lo:hi] > 0
        vals, counts = np.unique(d[vis], return_counts=True)
        shared = np.isin(d, vals[counts > 1]) & vis
        g.opacity[lo:hi][shared] = 0.0
        tied += int(shared.sum())
    attrs = dict(means=x[:, :3], scales=cuda(g.scales), quats=cuda(g.quats), colors=cuda(g.colors),
                 opacity=cuda(g.opacity))
    pt = perm.long()
    attrs_p = dict(means=xo[:, :3], **{k: v[pt].contiguous() for k, v in attrs.items() if k != "means"})
    R = Renderer()
    a = R.render(attrs, fo, cams, 8 * x.shape[0], aux=True)
    img_a = a["image"].clone()
    E = int(a["n_entries"].item())
    keys_a = Renderer.view(a, "sorted_keys", E).clone()
    b = R.render(attrs_p, fo, cams, 8 * x.shape[0], aux=True)
    torch.cuda.synchronize()
    assert int(b["n_entries"].item()) == E
    assert torch.equal(keys_a, Renderer.view(b, "sorted_keys", E))
    assert torch.equal(img_a, b["image"])
    say(f"[order] {tied} Gaussians with a shared depth made transparent; {E} entries")

    # decode of the permuted positions: the permuted attributes
    D = Decoder(S.single_decoder())
    da = D.decode_xyzt(x)
    da = {k: v.clone() for k, v in da.items()}
    db = D.decode_xyzt(xo)
    torch.cuda.synchronize()
    for k in da:
        err = float((da[k][pt] - db[k]).abs().max())
        assert err <= 1e-3, (k, err)
    say(f"[order] {x.shape[0]} positions over {len(frames)} frames: exact Morton order, same image bit for bit")


def test_order_edge_cases():
    """One frame, empty frames, a one-Gaussian frame, non-finite positions
    (cell 0) and argument errors."""
    rng = np.random.default_rng(9)
    pos = rng.normal(0, 3, (5000, 3)).astype(np.float32)
    pos[:7] = np.nan
    pos[7:9] = np.inf
    fo = np.array([0, 0, 1, 1, 4000, 5000], np.int64)
    x = cuda(pos)
    perm, xo = spatial_order(x, fo)
    torch.cuda.synchronize()
    p = host(perm).astype(np.int64)
    assert np.array_equal(p, _expected_perm(pos, fo, S.single_hash()))
    assert np.array_equal(host(xo), pos[p], equal_nan=True)
    with pytest.raises(ia.IAError):
        spatial_order(x, np.array([0, 10, 4999], np.int64))  # last offset must be N
    with pytest.raises(ia.IAError):
        ia.ia_spatial_order(x, fo, perm, x, None)  # pos_out aliases pos (checked before the workspace)
