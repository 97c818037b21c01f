"""GPU parity of the decode path (SPIN-4DGS §3.3, Eq. 7-11) against the oracle.

Tolerances (fixed by the benchmark spec for this path):
  fp32 decoder : |gpu - oracle| <= 1e-5 |oracle| + 1e-7, every output
  fp16 decoder : <= 5e-3 absolute against the fp64 oracle, every output,
                 and the same bound on the pre-exp log-scale log(s).
The fp16 path is also compared with the oracle's fp16-emulation mode (same
rounding points, fp64 sums) at 1e-3: that leaves only fp32-vs-fp64
accumulation and one-ulp fp16 rounding flips.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
from implicit_attribute_decode_amd import scenes as S
from implicit_attribute_decode_amd.pipeline import Decoder

from gpu_util import cuda, host, rel_ok, say

pytestmark = pytest.mark.gpu

KEYS = ("scales", "quats", "colors", "opacity")


def _gpu_decode(dec, pos, t=None):
    D = Decoder(dec)
    x = cuda(pos)
    out = D.decode(x, t) if pos.shape[1] == 3 else D.decode_xyzt(x)
    torch.cuda.synchronize()
    return {k: host(v).astype(np.float64) for k, v in out.items()}


def _check_f32(g, o):
    """1e-5 relative to each attribute's magnitude: per element for scales,
    colours and opacity; the vector norm for the unit quaternion, whose
    components all carry rounding errors of the size of its norm."""
    for k in ("scales", "colors", "opacity"):
        ok = rel_ok(g[k], o[k], 1e-5, 1e-7)
        assert ok.all(), (k, int((~ok).sum()), np.abs(g[k] - o[k]).max())
    qn = np.linalg.norm(o["quats"], axis=1, keepdims=True)
    dq = np.abs(g["quats"] - o["quats"])
    ok = dq <= 1e-5 * qn + 1e-7
    assert ok.all(), ("quats", int((~ok).sum()), dq.max())
    # the same errors per component, by the component's share of the norm:
    # components of at least a tenth of the norm also meet 1e-5 of their own
    # magnitude; smaller ones are reported
    share = np.abs(o["quats"]) / np.maximum(qn, 1e-30)
    rel = dq / np.maximum(np.abs(o["quats"]), 1e-30)
    figs = []
    for lo, hi in ((0.1, 2.0), (0.01, 0.1), (0.0, 0.01)):
        m = (share >= lo) & (share < hi)
        if m.any():
            figs.append(f"|q_i|/|q| in [{lo}, {hi}): {int(m.sum())} comps, max rel {rel[m].max():.2e}, "
                        f"max err/|q| {(dq / qn)[m].max():.2e}")
    say("[quats per component] " + "; ".join(figs))
    big = share >= 0.1
    assert (rel[big] <= 1e-5).all(), ("quats per component", float(rel[big].max()))


def _check_f16(g, o, emu, tag):
    for k in KEYS:
        err = np.abs(g[k] - o[k]).max()
        err_e = np.abs(g[k] - emu[k]).max()
        say(f"[{tag}] {k}: max|gpu-oracle64| {err:.2e}  max|gpu-oracle16emu| {err_e:.2e}")
        assert err <= 5e-3, (k, err)
        assert err_e <= 1e-3, (k, err_e)
    dl = np.abs(np.log(g["scales"]) - np.minimum(o["raw"][:, 0:3], 20.0)).max()
    say(f"[{tag}] log-scale: max diff {dl:.2e}")
    assert dl <= 5e-3


def _edge_positions(rng, n):
    """Random points plus the edges of Eq. 7-8: the origin, the unit sphere,
    far points, exact time endpoints and out-of-range times."""
    p = np.empty((n, 4), np.float32)
    p[:, :3] = rng.normal(0, 2.0, (n, 3))
    p[:, 3] = rng.random(n)
    d = rng.normal(size=(8, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    special = np.concatenate([np.zeros((1, 3)), d, d * 1e6, d * (1 + 1e-7), [[0.999, 0, 0], [1.0, 0, 0]]])
    k = min(n, len(special))
    p[:k, :3] = special[:k]
    p[:k, 3] = np.resize(np.float32([0.0, 1.0, -0.5, 1.5, 0.5, 0.25, 0.999]), k)
    return p


def test_tiny_fp32_matches_oracle():
    dec = S.tiny_decoder()
    pos = S.tiny_positions()
    g = _gpu_decode(dec, pos, 0.5)
    o = O.decode(dec, pos, 0.5)
    _check_f32(g, o)


@pytest.mark.parametrize("n", [1, 63, 64, 257, 4097, 70001])
def test_tiny_fp32_ragged_sizes_and_edges(n):
    dec = S.tiny_decoder()
    pos = _edge_positions(np.random.default_rng(n), n)
    g = _gpu_decode(dec, pos)
    o = O.decode(dec, pos)
    _check_f32(g, o)


def test_single_fp32_decoder_on_fp16_table():
    """The Single hash (16 hashed levels, fp16 table) with an fp32 32-64-64
    MLP: exercises every hashed level at the fp32 bound."""
    base = S.single_decoder()
    dec = S.DecoderParams(hash=base.hash, mlp=S.MLPConfig(dims=[32, 64, 64, 11], act="gelu", f16=False),
                          tables=base.tables, weights=[w.astype(np.float32) for w in base.weights],
                          biases=base.biases)
    pos, t = S.single_positions(2, n_shell=20_000, n_clus=1_000)
    g = _gpu_decode(dec, pos, t)
    o = O.decode(dec, pos, t)
    _check_f32(g, o)


def test_single_fp16_mfma_full_frame():
    dec = S.single_decoder()
    pos, t = S.single_positions(2)
    g = _gpu_decode(dec, pos, t)
    o = O.decode(dec, pos, t, mode=0)
    e = O.decode(dec, pos, t, mode=1)
    _check_f16(g, o, e, "single")


@pytest.mark.parametrize("n", [1, 15, 64, 1000, 65537])
def test_single_fp16_ragged_xyzt(n):
    dec = S.single_decoder()
    pos = _edge_positions(np.random.default_rng(100 + n), n)
    g = _gpu_decode(dec, pos)
    o = O.decode(dec, pos, mode=0)
    e = O.decode(dec, pos, mode=1)
    _check_f16(g, o, e, f"xyzt n={n}")


def _check_f16_sh(g, o, emu, tag):
    for k in ("scales", "quats", "sh", "opacity"):
        err = np.abs(g[k] - o[k]).max()
        err_e = np.abs(g[k] - emu[k]).max()
        say(f"[{tag}] {k}: max|gpu-oracle64| {err:.2e}  max|gpu-oracle16emu| {err_e:.2e}")
        assert err <= 5e-3, (k, err)
        assert err_e <= 1e-3, (k, err_e)


def test_single_fp16_sh_colour_head_full_frame():
    """The SH colour decoder (56-row head: 48 degree-3 coefficients, no
    activation) on a full Single frame, same bars as the RGB head."""
    dec = S.single_decoder_sh()
    pos, t = S.single_positions(2)
    g = _gpu_decode(dec, pos, t)
    assert "colors" not in g and g["sh"].shape == (pos.shape[0], 16, 3)
    _check_f16_sh(g, O.decode(dec, pos, t, mode=0), O.decode(dec, pos, t, mode=1), "sh head")


@pytest.mark.parametrize("n", [1, 17, 4097])
def test_sh_colour_head_ragged_xyzt(n):
    dec = S.single_decoder_sh()
    pos = _edge_positions(np.random.default_rng(300 + n), n)
    g = _gpu_decode(dec, pos)
    _check_f16_sh(g, O.decode(dec, pos, mode=0), O.decode(dec, pos, mode=1), f"sh xyzt n={n}")


def test_paper_scale_decoder_full_frame():
    """Paper-scale decoder (F = 4, 2^21-entry tables, one 64-64-64 GELU MLP
    per attribute, SH colour) on a full Single frame."""
    dec = S.paper_decoder()
    pos, t = S.single_positions(2)
    g = _gpu_decode(dec, pos, t)
    _check_f16_sh(g, O.decode(dec, pos, t, mode=0), O.decode(dec, pos, t, mode=1), "paper")


@pytest.mark.parametrize("n", [1, 63, 4097, 70001])
def test_paper_scale_decoder_ragged_xyzt(n):
    dec = S.paper_decoder()
    pos = _edge_positions(np.random.default_rng(400 + n), n)
    g = _gpu_decode(dec, pos)
    _check_f16_sh(g, O.decode(dec, pos, mode=0), O.decode(dec, pos, mode=1), f"paper xyzt n={n}")


def test_paper_scale_decoder_2p23_tables():
    """The 2^23-entry variant (1 GiB of fp16 tables, beyond the Infinity Cache)."""
    dec = S.paper_decoder(log2T=23)
    pos = _edge_positions(np.random.default_rng(402), 20000)
    g = _gpu_decode(dec, pos)
    _check_f16_sh(g, O.decode(dec, pos, mode=0), O.decode(dec, pos, mode=1), "paper 2^23")


def test_paper_scale_decoder_rgb_branches():
    dec = S.paper_decoder(sh=False)
    pos = _edge_positions(np.random.default_rng(401), 5000)
    g = _gpu_decode(dec, pos)
    _check_f16(g, O.decode(dec, pos, mode=0), O.decode(dec, pos, mode=1), "paper rgb")


def test_decode_zero_is_noop():
    D = Decoder(S.tiny_decoder())
    out = D.decode(torch.empty((0, 3), device="cuda"), 0.5)
    torch.cuda.synchronize()
    assert out["scales"].shape == (0, 3)


def test_chunked_decode_bitwise_equals_slice_decodes():
    """A decode of more than one chunk (at most 2^22 Gaussians per chunk; the
    MLP of a chunk runs beside the next chunk's gather, and every chunk after
    the first uses the lean gather) gives bit for bit what decoding each
    64-aligned slice on its own gives (one chunk: batched gather, MLP on the
    whole chip).  The MFMA rounding of a Gaussian depends on its index mod 64
    (the matrix column it occupies), so slices start at multiples of 64 and
    the library cuts chunks at multiples of 256."""
    rng = np.random.default_rng(11)
    n = (1 << 22) + 5000
    xyzt = np.concatenate([rng.normal(0.0, 2.0, (n, 3)), rng.uniform(0.0, 1.0, (n, 1))], 1).astype(np.float32)
    xyzt[::7, 3] = np.round(xyzt[::7, 3] * 149.0) / 149.0  # some times on temporal vertices
    D = Decoder(S.single_decoder())
    x0 = cuda(xyzt)
    torch.cuda.synchronize()
    # the positions are produced on the stream right before the call (no host
    # synchronisation): the decode's internal side stream must wait for them
    x = x0 * 1.0
    full = {k: v.clone() for k, v in D.decode_xyzt(x).items()}
    for lo, hi in ((0, 1000), (1 << 21, (1 << 21) + 777), (2_800_000 - 64 * 5, 2_800_000 + 999), (n - 5000 & ~63, n)):
        part = D.decode_xyzt(x[lo:hi].contiguous())
        torch.cuda.synchronize()
        for k in full:
            assert torch.equal(full[k][lo:hi], part[k]), (k, lo, hi)
    say(f"chunked decode of {n} = slice decodes bit for bit")


def test_concurrent_decodes_on_one_handle_match_serial():
    """A decoder handle holds only its parameters (SPIN-4DGS page, §3.3
    Eq. 10-11: decoding is a function of position and time): two host threads
    decode different position sets on one handle at the same time, each on
    its own stream with its own workspace and second stream (both sets span
    two chunks, so each overlaps its MLPs with its gathers).  Every result
    equals, bit for bit, a serial decode of the same set on one stream with no
    second stream."""
    import threading

    from implicit_attribute_decode_amd import ia

    rng = np.random.default_rng(12)
    n = (1 << 22) + 300_000
    D = Decoder(S.single_decoder())
    xs = [cuda(np.concatenate([rng.normal(0.0, 2.0, (n, 3)), rng.uniform(0.0, 1.0, (n, 1))], 1).astype(np.float32))
          for _ in range(2)]
    nbytes = ia.ia_decode_workspace_size(D.handle, n)
    assert nbytes >= 2 * (1 << 22) * (16 * 2 * 2 + 16)  # two slots of a full chunk

    def aligned(nb):
        buf = torch.empty(nb + 256, dtype=torch.uint8, device="cuda")
        off = (-buf.data_ptr()) % 256
        return buf[off:off + nb]

    ref = []
    for x in xs:
        out = D._out(n, None)
        ia.ia_decode_xyzt(D.handle, x, n, D._gaussians(out), aligned(nbytes), None)
        ref.append(out)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    sides = [torch.cuda.Stream() for _ in range(2)]
    wss = [aligned(nbytes) for _ in range(2)]
    for rep in range(3):
        outs = [D._out(n, None) for _ in range(2)]
        for o in outs:
            for v in o.values():
                v.fill_(float("nan"))
        torch.cuda.synchronize()
        barrier = threading.Barrier(2)
        errors = []

        def run(k):
            try:
                barrier.wait()
                ia.ia_decode_xyzt(D.handle, xs[k], n, D._gaussians(outs[k]), wss[k], sides[k], stream=streams[k])
            except Exception as exc:  # reported on the main thread
                errors.append(exc)

        th = [threading.Thread(target=run, args=(k,)) for k in range(2)]
        for t in th:
            t.start()
        for t in th:
            t.join()
        assert not errors, errors
        torch.cuda.synchronize()
        for k in range(2):
            for key in ref[k]:
                assert torch.equal(outs[k][key], ref[k][key]), (rep, k, key)
    say(f"two concurrent decodes of {n} on one handle = serial decodes, bit for bit")


def test_decode_workspace_errors():
    """A missing, misaligned or too small workspace is an argument error,
    returned before anything is enqueued."""
    from implicit_attribute_decode_amd import ia

    D = Decoder(S.single_decoder())
    n = 5000
    x = cuda(np.zeros((n, 4), np.float32))
    out = D._out(n, None)
    need = ia.ia_decode_workspace_size(D.handle, n)
    assert need == (n + 255) // 256 * 256 * (16 * 2 * 2 + 16)
    buf = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
    off = (-buf.data_ptr()) % 256
    with pytest.raises(ia.IAError) as e:
        ia.ia_decode_xyzt(D.handle, x, n, D._gaussians(out), None)
    assert e.value.status == ia.IA_ERR_INVALID_ARG
    with pytest.raises(ia.IAError) as e:
        ia.ia_decode_xyzt(D.handle, x, n, D._gaussians(out), buf[off + 4:off + 4 + need])
    assert e.value.status == ia.IA_ERR_INVALID_ARG
    with pytest.raises(ia.IAError) as e:
        ia.ia_decode_xyzt(D.handle, x, n, D._gaussians(out), buf[off:off + need - 1])
    assert e.value.status == ia.IA_ERR_WORKSPACE_TOO_SMALL
    # an fp32 decoder needs none
    T = Decoder(S.tiny_decoder())
    assert ia.ia_decode_workspace_size(T.handle, n) == 0
    ia.ia_decode_xyzt(T.handle, x, n, T._gaussians(T._out(n, None)), None)
    torch.cuda.synchronize()


def test_sequence_full_size_sampled():
    """All 150 x 200k (x,y,z,t) positions in one launch; 24k sampled rows
    (every frame represented) against the oracle."""
    seq = S.Sequence()
    xyzt = seq.xyzt()
    assert xyzt.shape == (30_000_000, 4)
    dec = S.single_decoder()
    D = Decoder(dec)
    out = D.decode_xyzt(cuda(xyzt))
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    idx = np.sort(np.concatenate([rng.choice(xyzt.shape[0], 20_000, replace=False),
                                  np.arange(150) * seq.per_frame, np.arange(1, 151) * seq.per_frame - 1,
                                  np.arange(xyzt.shape[0] - 3000, xyzt.shape[0])]))
    ti = torch.as_tensor(idx, device="cuda")
    g = {k: host(v.index_select(0, ti)).astype(np.float64) for k, v in out.items()}
    o = O.decode(dec, xyzt[idx], mode=0)
    e = O.decode(dec, xyzt[idx], mode=1)
    _check_f16(g, o, e, "sequence")
    for v in out.values():
        assert torch.isfinite(v).all()
