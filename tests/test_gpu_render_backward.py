"""GPU parity of the render backward (SPIN-4DGS §3.1 Eq. 1-4 differentiated,
with the EWA projection of Eq. 2-3) and of the L1 image loss, against the
oracle's fp64 gradients (which are pinned to central finite differences).

The GPU computes the projection and the compositing in fp32 and sums
per-Gaussian partials with float atomics; the oracle does everything in
fp64.  Gaussians the oracle flags (a discrete decision of theirs, or of a
pixel they composite, lies within fp32 rounding of a threshold) are left
out.  On the others, for each gradient array X:
    |X_gpu - X_oracle| <= 2e-4 |X_oracle| + 2e-5 max|X_oracle|
elementwise, and the median relative difference (over entries above 1 % of
the largest) stays below 1e-5: fp32 rounding of a sum of a few hundred
pixel terms, each recovered through T_i = T_{i+1} / (1 - alpha_i), sits
near 1e-6 relative; a dropped term, wrong sign or transposed operand is
O(1).
"""
import numpy as np
import pytest
import torch

import oracle as O
from implicit_attribute_decode_amd import ia, scenes as S
from implicit_attribute_decode_amd.pipeline import Renderer

from gpu_util import cuda, host, say

pytestmark = pytest.mark.gpu

GROUPS = ("means", "scales", "quats", "opacity", "colors")


def _attrs(g: S.Gaussians):
    return dict(means=cuda(g.means), scales=cuda(g.scales), quats=cuda(g.quats), colors=cuda(g.colors),
                opacity=cuda(g.opacity))


def _compare(tag, grads, ref, rtol=2e-4, atol_frac=2e-5, med_rel=1e-5):
    keep = ~ref["flags"]
    say(f"[{tag}] {int(keep.sum())} of {len(keep)} Gaussians unflagged")
    assert keep.sum() >= 0.5 * len(keep)
    for k in GROUPS:
        a = host(grads[k]).astype(np.float64)[keep]
        b = ref[k][keep]
        scale = np.abs(b).max()
        err = np.abs(a - b)
        lim = rtol * np.abs(b) + atol_frac * scale
        big = np.abs(b) > 1e-2 * scale
        med = float(np.median(err[big] / np.abs(b[big]))) if big.any() else 0.0
        worst = float((err / np.maximum(lim, 1e-300)).max())
        say(f"[{tag}] {k}: max|ref| {scale:.3e} worst err/limit {worst:.3f} median rel {med:.2e}")
        assert worst <= 1.0, (k, worst)
        assert med <= med_rel, (k, med)


def _run(g: S.Gaussians, fo, cams, gimg_fn, tag, cap=None):
    """GPU forward (automatic binning) + backward, and the oracle on the
    same float32 inputs and the same dL/dimage."""
    attrs = _attrs(g)
    R = Renderer()
    cap = cap or 1 << 20
    res = R.render(attrs, fo, cams, cap, aux=True)
    torch.cuda.synchronize()
    assert int(res["overflow"].item()) == 0
    gimg = gimg_fn(res["image"])
    grads = R.backward(attrs, fo, cams, cap, res, gimg)
    torch.cuda.synchronize()
    ref = O.render_grad(cams, fo, g.means.astype(np.float64), g.scales.astype(np.float64),
                        g.quats.astype(np.float64), g.opacity.astype(np.float64), g.colors.astype(np.float64),
                        host(gimg).astype(np.float64))
    # the oracle's fp64 image agrees with the forward before gradients are
    # compared (a pixel where one Gaussian's alpha sits at 1/255 may differ
    # by up to alpha T c < 4e-3)
    d = np.abs(ref["image"] - host(res["image"]))
    assert np.quantile(d, 0.999) <= 1e-4 and d.max() <= 4e-3, (np.quantile(d, 0.999), d.max())
    _compare(tag, grads, ref)
    return grads, ref


def _normal_grad(seed):
    def fn(image):
        gen = torch.Generator(device="cuda").manual_seed(seed)
        return torch.randn(image.shape, generator=gen, device="cuda")
    return fn


def test_l1_loss_value_and_gradient():
    rng = np.random.default_rng(40)
    img = rng.random((3, 3, 37, 53)).astype(np.float32)
    tgt = rng.random(img.shape).astype(np.float32)
    tgt.reshape(-1)[::7] = img.reshape(-1)[::7]  # ties: zero gradient
    loss, grad = Renderer.l1_loss(cuda(img), cuda(tgt))
    torch.cuda.synchronize()
    n = img.size
    want = np.abs(img.astype(np.float64) - tgt.astype(np.float64)).mean()
    assert abs(float(loss.item()) - want) <= 1e-12 * want
    inv = np.float32(1.0) / np.float32(n)
    d = img - tgt
    exp = np.where(d > 0, inv, np.where(d < 0, -inv, np.float32(0.0))).astype(np.float32)
    np.testing.assert_array_equal(host(grad), exp)
    # empty input: loss 0, nothing written
    loss0, _ = Renderer.l1_loss(torch.empty(0, device="cuda"), torch.empty(0, device="cuda"))
    assert float(loss0.item()) == 0.0


def test_backward_64_gaussian_subscene_two_frames():
    """The finite-difference subscene of the oracle's pins, as two 64x48 frames."""
    rng = np.random.default_rng(31)
    half = 32
    means = np.concatenate([
        np.stack([rng.uniform(-0.8, 0.8, half), rng.uniform(-0.8, 0.8, half), rng.uniform(2.2, 3.5, half)], 1),
        S.shell_points(rng, half, 3.0)]).astype(np.float32)
    g = S.render_attributes(rng, means, 0.04, 0.25)
    cams = [S.origin_camera(64, 48, 60.0), S.ring_camera(3, W=64, H=48, fx=40.0, fy=40.0)]
    cams[0].bg = np.float32([0.2, 0.4, 0.6])
    _run(g, np.array([0, half, 64]), cams, _normal_grad(1), "fd subscene")


def test_backward_l1_against_seeded_target():
    """L1 loss against a seeded target image, gradients to every Gaussian."""
    rng = np.random.default_rng(41)
    means = np.concatenate([S.shell_points(rng, 2500, 3.0), S.shell_points(rng, 1500, 2.2)])
    g = S.render_attributes(rng, means, 5e-3, 8e-2)
    cams = [S.ring_camera(k, W=160, H=120, fx=120.0, fy=120.0) for k in (0, 7)]
    fo = np.array([0, 2000, 4000])
    tgt = cuda(np.random.default_rng(42).random((2, 3, 120, 160)).astype(np.float32))

    def l1(image):
        loss, grad = Renderer.l1_loss(image, tgt)
        return grad
    _run(g, fo, cams, l1, "l1")


def test_backward_dense_overlap_and_saturation():
    """Many large, opaque Gaussians: long per-pixel lists, alpha clamped at
    0.99 and early stops (T < 1e-4) on most pixels."""
    rng = np.random.default_rng(43)
    n = 600
    means = np.stack([rng.uniform(-0.6, 0.6, n), rng.uniform(-0.5, 0.5, n), rng.uniform(2.0, 4.0, n)], 1)
    g = S.render_attributes(rng, means.astype(np.float32), 0.05, 0.3)
    g.opacity[:] = rng.uniform(0.6, 1.0, n).astype(np.float32)
    cam = S.origin_camera(96, 80, 70.0)
    _run(g, np.array([0, n]), [cam], _normal_grad(2), "dense")


def test_backward_many_frames_two_pixel_raster():
    """512 frames of 64x64 (8192 tiles): the forward takes its
    two-pixels-per-thread launch shape; the backward reads its n_contrib."""
    rng = np.random.default_rng(44)
    F, per = 512, 48
    means = np.concatenate([
        np.stack([rng.uniform(-0.7, 0.7, per), rng.uniform(-0.7, 0.7, per), rng.uniform(2.0, 3.5, per)], 1)
        for _ in range(F)]).astype(np.float32)
    g = S.render_attributes(rng, means, 0.03, 0.15)
    cams = [S.origin_camera(64, 64, 60.0) for _ in range(F)]
    fo = np.arange(F + 1) * per
    _run(g, fo, cams, _normal_grad(3), "512 frames")


def test_backward_culled_and_empty():
    """Culled Gaussians (behind the camera, NaN) get zero gradients; an empty
    frame in the batch and N = 0 are accepted."""
    rng = np.random.default_rng(45)
    means = np.concatenate([S.shell_points(rng, 300, 3.0), np.float32([[0, 0, -3.0]] * 5)])
    g = S.render_attributes(rng, means, 0.02, 0.1)
    g.means[300] = np.nan
    attrs = _attrs(g)
    cams = [S.origin_camera(64, 64, 60.0)] * 3
    fo = np.array([0, 305, 305, 305])
    R = Renderer()
    res = R.render(attrs, fo, cams, 1 << 16, aux=True)
    gimg = torch.ones_like(res["image"])
    grads = R.backward(attrs, fo, cams, 1 << 16, res, gimg)
    torch.cuda.synchronize()
    for k in GROUPS:
        h = host(grads[k])
        assert np.isfinite(h).all()
        assert np.all(h[300:] == 0), k
    empty = dict(means=torch.empty((0, 3), device="cuda"), scales=torch.empty((0, 3), device="cuda"),
                 quats=torch.empty((0, 4), device="cuda"), colors=torch.empty((0, 3), device="cuda"),
                 opacity=torch.empty((0,), device="cuda"))
    res = R.render(empty, np.array([0, 0]), cams[:1], 16, aux=True)
    grads = R.backward(empty, np.array([0, 0]), cams[:1], 16, res, torch.ones_like(res["image"]))
    torch.cuda.synchronize()
    assert all(grads[k].numel() == 0 for k in GROUPS)


def _sh_attrs(rng, g, scale):
    attrs = _attrs(g)
    attrs.pop("colors")
    sh = (scale * rng.normal(0, 1, (len(g.means), 16, 3))).astype(np.float32)
    attrs["sh"] = cuda(sh)
    return attrs, sh


def test_backward_with_sh_colours_matches_oracle():
    """Render with degree-3 SH colours, backward of a random dL/dimage: the
    oracle differentiates the render with its fp64 SH colours, then chains
    dL/dcolour through the SH colour (sh_colors_grad) to dL/dsh and the view
    direction's share of dL/dmean."""
    rng = np.random.default_rng(47)
    n = 3000
    g = S.render_attributes(rng, S.shell_points(rng, n, 1.0), 0.01, 0.05)
    attrs, sh = _sh_attrs(rng, g, 0.05)  # every channel stays far above the clamp at 0
    fo = np.array([0, n // 2, n])
    cams = [S.ring_camera(0, W=160, H=120, fx=150.0, fy=150.0), S.ring_camera(4, W=160, H=120, fx=150.0, fy=150.0)]
    R = Renderer()
    res = R.render(attrs, fo, cams, 1 << 20, aux=True)
    torch.cuda.synchronize()
    assert int(res["overflow"].item()) == 0
    gimg = _normal_grad(48)(res["image"])
    grads = R.backward(attrs, fo, cams, 1 << 20, res, gimg)
    torch.cuda.synchronize()
    col = O.sh_colors(cams, fo, g.means, sh)
    ref = O.render_grad(cams, fo, g.means.astype(np.float64), g.scales.astype(np.float64),
                        g.quats.astype(np.float64), g.opacity.astype(np.float64), col, host(gimg).astype(np.float64))
    gsh, gdir = O.sh_colors_grad(cams, fo, g.means, sh, ref["colors"])
    ref = dict(ref, means=ref["means"] + gdir)
    _compare("sh", grads, ref)
    keep = ~ref["flags"]
    a = host(grads["sh"]).astype(np.float64).reshape(n, 48)[keep]
    b = gsh.reshape(n, 48)[keep]
    err = np.abs(a - b)
    assert np.all(err <= 2e-4 * np.abs(b) + 2e-5 * np.abs(b).max()), float(err.max())
    assert np.abs(gdir[keep]).max() > 1e-3 * np.abs(ref["means"][keep]).max()  # the direction term matters


def test_backward_sh_clamped_channel_has_no_gradient():
    rng = np.random.default_rng(49)
    n = 500
    g = S.render_attributes(rng, S.shell_points(rng, n, 1.0), 0.01, 0.05)
    attrs, sh = _sh_attrs(rng, g, 0.05)
    sh[:, 0, 1] = -5.0  # green below zero for every Gaussian
    attrs["sh"] = cuda(sh)
    cams = [S.ring_camera(0, W=96, H=64, fx=90.0, fy=90.0)]
    R = Renderer()
    res = R.render(attrs, [0, n], cams, 1 << 18, aux=True)
    grads = R.backward(attrs, [0, n], cams, 1 << 18, res, _normal_grad(50)(res["image"]))
    torch.cuda.synchronize()
    gs = host(grads["sh"])
    assert not gs[:, :, 1].any() and np.abs(gs[:, :, 0]).max() > 0


def test_backward_rejects_missing_sh_buffer():
    rng = np.random.default_rng(46)
    g = S.render_attributes(rng, S.shell_points(rng, 10, 3.0), 0.02, 0.1)
    attrs, _ = _sh_attrs(rng, g, 0.05)
    cam = S.origin_camera(32, 32, 40.0)
    R = Renderer()
    res = R.render(attrs, np.array([0, 10]), [cam], 256, aux=True)
    G = ia.gaussians(means=attrs["means"], scales=attrs["scales"], quats=attrs["quats"], sh=attrs["sh"],
                     opacity=attrs["opacity"], means_stride=3, sh_degree=3)
    out = [torch.empty(sh, device="cuda") for sh in ((10, 3), (10, 3), (10, 4), (10,), (10, 3))]
    GG = ia.GaussianGrads(*[ia._ptr(t) for t in out], None)
    ws = R.workspace(10, 1, 32, 32, 256)
    with pytest.raises(ia.IAError) as e:
        ia.ia_render_backward(G, np.array([0, 10]), [cam], ws, 256, torch.ones_like(res["image"]), res["T_final"],
                              res["n_contrib"], GG)
    assert e.value.status == ia.IA_ERR_INVALID_ARG


def test_backward_sh_with_an_empty_frame():
    """A frame without Gaussians between two with: zero rows stay consistent."""
    rng = np.random.default_rng(51)
    n = 400
    g = S.render_attributes(rng, S.shell_points(rng, n, 1.0), 0.01, 0.05)
    attrs, sh = _sh_attrs(rng, g, 0.05)
    fo = np.array([0, n // 2, n // 2, n])
    cams = [S.ring_camera(k, W=96, H=64, fx=90.0, fy=90.0) for k in (0, 3, 6)]
    R = Renderer()
    res = R.render(attrs, fo, cams, 1 << 18, aux=True)
    gimg = _normal_grad(52)(res["image"])
    grads = R.backward(attrs, fo, cams, 1 << 18, res, gimg)
    torch.cuda.synchronize()
    col = O.sh_colors(cams, fo, g.means, sh)
    ref = O.render_grad(cams, fo, g.means.astype(np.float64), g.scales.astype(np.float64),
                        g.quats.astype(np.float64), g.opacity.astype(np.float64), col, host(gimg).astype(np.float64))
    gsh, gdir = O.sh_colors_grad(cams, fo, g.means, sh, ref["colors"])
    keep = ~ref["flags"]
    a = host(grads["sh"]).astype(np.float64).reshape(n, 48)[keep]
    b = gsh.reshape(n, 48)[keep]
    assert np.all(np.abs(a - b) <= 2e-4 * np.abs(b) + 2e-5 * np.abs(b).max())
