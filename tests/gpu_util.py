"""Helpers shared by the GPU parity tests (not collected as tests)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle as O
from implicit_attribute_decode_amd.pipeline import Renderer


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def cuda(a, dtype=None):
    t = torch.as_tensor(np.ascontiguousarray(a), device="cuda")
    return t if dtype is None else t.to(dtype)


def host(t):
    return t.detach().cpu().numpy()


def rel_ok(a, b, rtol=1e-5, atol=1e-7):
    """|a - b| <= rtol |b| + atol, elementwise."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.abs(a - b) <= rtol * np.abs(b) + atol


def gpu_render(g: dict, fo, cams, cap: int, renderer: Renderer | None = None, binning: int = 0):
    r = renderer or Renderer()
    res = r.render(g, fo, cams, cap, aux=True, binning=binning)
    torch.cuda.synchronize()
    E = int(res["n_entries"].item())
    n = min(E, cap)
    N = int(np.asarray(fo)[-1])
    out = dict(
        image=host(res["image"]).astype(np.float64), T=host(res["T_final"]).astype(np.float64),
        n_contrib=host(res["n_contrib"]).view(np.uint32), E=E, overflow=int(res["overflow"].item()),
        keys=host(Renderer.view(res, "sorted_keys", n)).view(np.uint64),
        vals=host(Renderer.view(res, "sorted_vals", n)).view(np.uint32),
        ranges=host(Renderer.view(res, "tile_ranges", len(cams) * ((cams[0].W + 15) // 16) * ((cams[0].H + 15) // 16))).view(np.uint32),
    )
    if N > 0:
        pa = host(Renderer.view(res, "proj_a", N))
        pb = host(Renderer.view(res, "proj_b", N))
        pc = host(Renderer.view(res, "proj_c", N))
        out.update(mean2d=pa[:, :2].copy(), conic=np.stack([pa[:, 2], pa[:, 3], pb[:, 0]], 1), opacity=pb[:, 1].copy(),
                   rgb=np.stack([pb[:, 2], pb[:, 3], pc], 1), depth=host(Renderer.view(res, "depth", N)),
                   tiles=host(Renderer.view(res, "tiles_touched", N)).view(np.uint32),
                   tile_rect=host(Renderer.view(res, "tile_rect", N)).view(np.uint16).astype(np.int32))
    return out


def check_preprocess_bitexact(gp: dict, op: dict):
    """GPU projection == oracle projection, bit for bit: the tile counts of
    every Gaussian, the other fields of every visible one (a culled
    Gaussian's projection is not written)."""
    np.testing.assert_array_equal(gp["tiles"], op["tiles"])
    vis = op["tiles"] > 0
    for k in ("mean2d", "conic", "depth"):
        a, b = gp[k][vis], op[k][vis]
        bad = a.view(np.uint32) != b.view(np.uint32)
        assert not bad.any(), (k, int(bad.sum()), a[bad.any(1) if bad.ndim > 1 else bad][:3],
                               b[bad.any(1) if bad.ndim > 1 else bad][:3])
    np.testing.assert_array_equal(gp["tile_rect"][vis], op["tile_rect"][vis])


def check_bins_bitexact(gr: dict, ob: dict):
    assert gr["E"] == ob["E"], (gr["E"], ob["E"])
    np.testing.assert_array_equal(gr["keys"], ob["keys"])
    np.testing.assert_array_equal(gr["vals"], ob["vals"])
    np.testing.assert_array_equal(gr["ranges"].reshape(-1, 2), ob["ranges"])


def check_image(gr: dict, orr: dict, atol=1e-3, max_flag_frac=1e-3):
    """Image within atol on every pixel the oracle did not flag as
    threshold-ambiguous; flagged pixels at most max_flag_frac of all; the
    composited-count and final transmittance agree on the unflagged ones."""
    flags = orr["flags"]
    frac = flags.mean()
    assert frac <= max_flag_frac, f"{frac:.2e} of pixels flagged"
    ok = ~flags
    diff = np.abs(gr["image"] - orr["image"]).max(axis=1)  # over channels -> [F,H,W]
    worst = diff[ok].max() if ok.any() else 0.0
    assert worst <= atol, f"max |image diff| {worst:.3e} on unflagged pixels"
    np.testing.assert_array_equal(gr["n_contrib"][ok], orr["n_contrib"][ok])
    assert np.abs(gr["T"] - orr["T"])[ok].max() <= atol
    return dict(flag_frac=float(frac), max_diff=float(worst))
