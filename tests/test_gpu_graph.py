"""Per-frame decode + render replayed from HIP graphs (pipeline.FrameGraphs).

Four Sequence frames (200k Gaussians each, 640x360, frames 0, 1, 75, 149) are
captured, one graph per frame, after one eager pass.  Checks:
  - every captured node is a kernel node: no memset, memcpy or host nodes
    (the clears are fill kernels and the camera uploads kernel arguments);
  - three replays, with the program's own eager work (decodes and renders of
    other frames through the same objects and workspaces) and synchronisations
    between them, each reproduce the eager pass's attributes and images bit
    for bit (every buffer is poisoned before a replay);
  - a replay of a single frame leaves the other frames' outputs untouched.
"""
import ctypes

import numpy as np
import pytest
import torch

from implicit_attribute_decode_amd import scenes as S
from implicit_attribute_decode_amd.pipeline import Decoder, FrameGraphs, Renderer

from gpu_util import cuda, say

pytestmark = pytest.mark.gpu

KERNEL_NODE = 0  # hipGraphNodeTypeKernel


def _node_types(g) -> list:
    hip = ctypes.CDLL("libamdhip64.so")
    graph = ctypes.c_void_p(g.raw_cuda_graph())
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * n.value)()
    assert hip.hipGraphGetNodes(graph, nodes, ctypes.byref(n)) == 0
    out = []
    for k in range(n.value):
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[k]), ctypes.byref(t)) == 0
        out.append(t.value)
    return out


def _poison(bufs):
    for b in bufs:
        b.fill_(float("nan"))


def test_frame_graphs_replay_bit_exact():
    seq = S.Sequence()
    frames = [0, 1, 75, 149]
    per = seq.per_frame
    F = len(frames)
    xyzt = cuda(seq.xyzt(frames))
    fo = np.arange(F + 1, dtype=np.int64) * per
    cams = [seq.camera(f) for f in frames]
    D = Decoder(S.single_decoder())
    R = Renderer()
    N = F * per
    attrs = dict(scales=torch.empty((N, 3), device="cuda"), quats=torch.empty((N, 4), device="cuda"),
                 colors=torch.empty((N, 3), device="cuda"), opacity=torch.empty((N,), device="cuda"))
    image = torch.empty((F, 3, seq.H, seq.W), device="cuda")
    cap = 8 * per
    G = FrameGraphs(D, R, xyzt, fo, cams, cap, attrs, image)
    ref = {k: v.clone() for k, v in attrs.items()}
    ref_img = image.clone()
    assert torch.isfinite(ref_img).all() and float(ref_img.abs().sum()) > 0

    for f, g in enumerate(G.graphs):
        types = _node_types(g)
        assert types and all(t == KERNEL_NODE for t in types), (f, sorted(set(types)))
        if f == 0:
            say(f"[graph] frame graph: {len(types)} kernel nodes")

    # other frames' positions for the eager work between replays
    other = cuda(seq.xyzt([10, 20]))
    other_cams = [seq.camera(10), seq.camera(20)]
    bufs = [image, *attrs.values()]
    for rep in range(3):
        _poison(bufs)
        G.replay()
        torch.cuda.synchronize()
        assert torch.equal(image, ref_img), rep
        for k in attrs:
            assert torch.equal(attrs[k], ref[k]), (rep, k)
        # eager work through the same decoder, renderer and workspaces
        for j in range(2):
            x = other[j * per:(j + 1) * per]
            a = D.decode_xyzt(x)
            R.render(dict(means=x[:, :3], **a), [0, per], [other_cams[j]], cap)
        torch.cuda.synchronize()

    # one frame alone
    _poison(bufs)
    G.replay([2])
    torch.cuda.synchronize()
    assert torch.equal(image[2], ref_img[2])
    assert torch.isnan(image[0]).all() and torch.isnan(image[3]).all()
    lo, hi = 2 * per, 3 * per
    for k in attrs:
        assert torch.equal(attrs[k][lo:hi], ref[k][lo:hi]), k
        assert torch.isnan(attrs[k][:lo]).all()
    say(f"[graph] {F} frames x {per}: 3 replays bit-identical to the eager pass")
