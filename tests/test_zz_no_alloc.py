"""ia_decode_xyzt_noalloc: the decode with its scratch in the library's static
device array (no allocation, no workspace) against ia_decode_xyzt with a
caller workspace, through the C ABI.  Two calls in a row, the second with a
smaller input, each equal bit for bit to the workspace decode of the same
positions; sizes above the array's capacity are rejected before anything is
enqueued."""
import ctypes as C

import numpy as np
import pytest
import torch

from implicit_attribute_decode_amd import ia, scenes as S
from implicit_attribute_decode_amd.pipeline import Decoder

from gpu_util import cuda, say

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 20 << 20


def _max_n(L: int, F: int) -> int:
    return (SCRATCH_BYTES // (2 * L * F + 16)) & ~255


def _positions(rng, n):
    p = np.concatenate([rng.normal(0.0, 2.0, (n, 3)), rng.uniform(0.0, 1.0, (n, 1))], 1).astype(np.float32)
    p[::5, 3] = np.round(p[::5, 3] * 149.0) / 149.0  # some times on temporal vertices
    return p


@pytest.mark.parametrize("name", ["single", "paper", "tiny"])
def test_noalloc_decode_equals_workspace_decode(name):
    params = {"single": S.single_decoder, "paper": S.paper_decoder, "tiny": S.tiny_decoder}[name]()
    D = Decoder(params)
    L, F = int(params.hash.L), int(params.hash.F)
    big = _max_n(L, F) if params.mlp.f16 else 300_000
    sizes = (big, 70_001)
    rng = np.random.default_rng(91)
    xs = [cuda(_positions(rng, n)) for n in sizes]
    refs = [{k: v.clone() for k, v in D.decode_xyzt(x).items()} for x in xs]
    outs = [D._out(n, None) for n in sizes]
    for o in outs:
        for v in o.values():
            v.fill_(float("nan"))
    torch.cuda.synchronize()
    lib = ia.load()
    stream = torch.cuda.current_stream().cuda_stream
    # two calls in a row, the second smaller, no synchronisation in between
    for x, o, n in zip(xs, outs, sizes):
        g = D._gaussians(o)
        st = lib.ia_decode_xyzt_noalloc(D.handle, C.c_void_p(x.data_ptr()), n, C.byref(g), C.c_void_p(stream))
        assert st == ia.IA_OK, ia.ia_last_error()
    torch.cuda.synchronize()
    for o, r, n in zip(outs, refs, sizes):
        for k in r:
            assert torch.equal(o[k], r[k]), (name, n, k)
    say(f"[noalloc {name}] N = {sizes[0]} then {sizes[1]}: equal to the workspace decode bit for bit")
    if params.mlp.f16:
        n = big + 1
        x = cuda(_positions(rng, n))
        o = D._out(n, None)
        st = lib.ia_decode_xyzt_noalloc(D.handle, C.c_void_p(x.data_ptr()), n, C.byref(D._gaussians(o)),
                                        C.c_void_p(stream))
        assert st == ia.IA_ERR_INVALID_ARG and "exceeds" in ia.ia_last_error()
