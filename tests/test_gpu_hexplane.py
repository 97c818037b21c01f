"""GPU parity of the HexPlane deformation variant ("4D Gaussian Splatting详解",
§3.1 six planes, §3.2 deformation MLP, §6.1 opacity kept) and of rendering
with degree-3 SH colour, against the oracle.

Tolerance: the deformation MLP runs on fp16 MFMA, so outputs are within 5e-3
absolute of the fp64 oracle (log-scale increments likewise) and within 1e-3
of the oracle's fp16-emulation mode; opacity is copied bit for bit.  The
render of the deformed Gaussians keeps the render bar: projection, keys and
ranges bit-exact, image within 1e-3 on unflagged pixels.
"""
import numpy as np
import pytest
import torch

import oracle as O
from implicit_attribute_decode_amd import scenes as S
from implicit_attribute_decode_amd.pipeline import HexPlane

from gpu_util import check_bins_bitexact, check_image, check_preprocess_bitexact, cuda, gpu_render, host, say

pytestmark = pytest.mark.gpu


def _canon_dev(g):
    return dict(means=cuda(g.means), scales=cuda(g.scales), quats=cuda(g.quats), sh=cuda(g.sh),
                opacity=cuda(g.opacity))


def _check_deform(out, g, hp, t, tag):
    o = O.hexplane_deform(hp, g, t, mode=0)
    e = O.hexplane_deform(hp, g, t, mode=1)
    h = {k: host(v).astype(np.float64) for k, v in out.items()}
    for k in ("means", "sh"):
        err, err_e = np.abs(h[k] - o[k]).max(), np.abs(h[k] - e[k]).max()
        say(f"[{tag}] {k}: {err:.2e} (emu {err_e:.2e})")
        assert err <= 5e-3 and err_e <= 1e-3, k
    err = np.abs(h["quats"] - o["quats"]).max()
    err_e = np.abs(h["quats"] - e["quats"]).max()
    say(f"[{tag}] quats: {err:.2e} (emu {err_e:.2e})")
    assert err <= 5e-3 and err_e <= 1e-3
    dl = np.abs(np.log(h["scales"]) - np.log(o["scales"])).max()
    dle = np.abs(np.log(h["scales"]) - np.log(e["scales"])).max()
    say(f"[{tag}] log-scale: {dl:.2e} (emu {dle:.2e})")
    assert dl <= 5e-3 and dle <= 1e-3
    assert np.array_equal(host(out["opacity"]), g.opacity)


@pytest.mark.parametrize("t", [0.0, 0.37, 75 / 149, 1.0])
def test_deform_matches_oracle(t):
    hp = S.hexplane_params()
    g = S.hexplane_canonical(n_shell=17_000, n_clus=1_001)  # ragged: 20,003 Gaussians
    H = HexPlane(hp)
    out = H.deform(_canon_dev(g), t)
    torch.cuda.synchronize()
    _check_deform(out, g, hp, t, f"t={t:.3f}")


@pytest.mark.parametrize("n", [1, 31, 33, 1000])
def test_deform_ragged_sizes(n):
    hp = S.hexplane_params()
    rng = np.random.default_rng(n)
    g = S.render_attributes(rng, rng.uniform(-4, 4, (n, 3)).astype(np.float32), 1e-3, 5e-2, with_sh=True)
    H = HexPlane(hp)
    out = H.deform(_canon_dev(g), 0.6)
    torch.cuda.synchronize()
    _check_deform(out, g, hp, 0.6, f"n={n}")


def test_full_frame_deform_then_sh_render():
    """300k canonical Gaussians deformed at t = 0.5 and rendered at 1352x1014
    with SH colour; the oracle renders the GPU's deformed attributes."""
    hp = S.hexplane_params()
    g = S.hexplane_canonical()
    H = HexPlane(hp)
    out = H.deform(_canon_dev(g), 0.5)
    torch.cuda.synchronize()
    cam = S.hexplane_camera()
    fo = np.array([0, g.n])
    h = {k: host(v) for k, v in out.items()}
    pre = O.preprocess([cam], fo, h["means"], h["scales"], h["quats"])
    rgb = O.sh_colors([cam], fo, h["means"], h["sh"])
    b = O.bin_and_sort([cam], fo, pre)
    r = O.raster_tiles([cam], b, pre, h["opacity"], rgb)
    gr = gpu_render(out, fo, [cam], b["E"])
    say(f"[hexplane] N={g.n} E={gr['E']}")
    check_preprocess_bitexact(gr, pre)
    vis = pre["tiles"] > 0
    err = np.abs(gr["rgb"][vis].astype(np.float64) - rgb[vis]).max()
    say(f"[hexplane] SH colour max diff {err:.2e}")
    assert err <= 1e-5
    check_bins_bitexact(gr, b)
    say(f"[hexplane] image: {check_image(gr, r)}")
