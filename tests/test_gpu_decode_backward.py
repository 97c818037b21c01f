"""GPU parity of the decode backward (SPIN-4DGS §3.3 Eq. 7-11 differentiated:
hash-table, weight, bias and position gradients) against the oracle's fp64
gradients, which are pinned to central finite differences.

The oracle runs in its fp16-emulating mode with fp32 cell decisions (mode 3):
the same forward function the GPU differentiates, so what is left is fp32
against fp64 arithmetic, float-atomic summation order, and the rare one-ulp
fp16 rounding flip of a hidden activation (2^-11 relative) between the GPU's
fp32 pre-activation and the oracle's fp64 one.  Bounds (written in each
check): a gradient array X of the parameters is compared as
    |X_gpu - X_oracle| <= 1e-3 |X_oracle| + 1e-4 max|X_oracle|,
the position gradient per point as
    |g_gpu - g_oracle| <= 2e-3 |g_oracle| + 1e-4 max|g_oracle| (vector norms).
A flipped fp16 activation errs by 2^-11 of its own term, not of the entry's
sum: where few Gaussians contribute (the per-attribute decoder at n <= 1000)
and their terms cancel, |X_oracle| in the relative part is replaced by the
sum over Gaussians of each Gaussian's |X_oracle| (the oracle run one Gaussian
at a time), which bounds every term.
"""
import numpy as np
import pytest
import torch

import oracle as O
from implicit_attribute_decode_amd import ia, scenes as S
from implicit_attribute_decode_amd.pipeline import Decoder

from gpu_util import cuda, host, say

pytestmark = pytest.mark.gpu

UP = ("scales", "quats", "colors", "opacity")


def _upstream(rng, n):
    return dict(scales=rng.normal(size=(n, 3)), quats=rng.normal(size=(n, 4)), colors=rng.normal(size=(n, 3)),
                opacity=rng.normal(size=n))


def _edge_xyzt(rng, n):
    p = np.empty((n, 4), np.float32)
    p[:, :3] = rng.normal(0, 2.0, (n, 3))
    p[:, 3] = rng.random(n)
    d = rng.normal(size=(8, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    special = np.concatenate([np.zeros((1, 3)), d * 0.5, d * 1e4, d * (1 + 1e-6), [[0.999, 0, 0], [1.0, 0, 0]]])
    k = min(n, len(special))
    p[:k, :3] = special[:k]
    p[:k, 3] = np.resize(np.float32([0.0, 1.0, -0.5, 1.5, 0.5, 0.25, 10 / 149]), k)
    return p


def _close(tag, a, b, rtol, afrac):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = np.abs(b).max()
    lim = rtol * np.abs(b) + afrac * scale
    ratio = float((np.abs(a - b) / np.maximum(lim, 1e-300)).max())
    say(f"[{tag}] max|ref| {scale:.3e} worst err/limit {ratio:.3f}")
    assert ratio <= 1.0, (tag, ratio)


def _gpu_backward(D, pos, up, t=None, grad_means=None, want_pos=True):
    g = {k: cuda(v.astype(np.float32)) for k, v in up.items()}
    out = D.backward(cuda(pos), g, t, None if grad_means is None else cuda(grad_means), want_pos)
    torch.cuda.synchronize()
    return out


def _close_terms(tag, a, b, terms, rtol, afrac):
    """As _close with the relative part taken of `terms` (>= |b|)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = np.abs(b).max()
    lim = rtol * terms + afrac * scale
    ratio = float((np.abs(a - b) / np.maximum(lim, 1e-300)).max())
    say(f"[{tag}] max|ref| {scale:.3e} worst err/limit {ratio:.3f} (term sums)")
    assert ratio <= 1.0, (tag, ratio)


def _term_sums(dec, pos, up):
    """Per parameter entry, the sum over Gaussians of |the oracle's gradient
    of that Gaussian alone|."""
    acc = None
    for g in range(pos.shape[0]):
        r = O.decode_grad(dec, pos[g:g + 1].astype(np.float64), mode=3, grads={k: v[g:g + 1] for k, v in up.items()})
        one = dict(g_tables=np.abs(r["g_tables"]), g_weights=[np.abs(w) for w in r["g_weights"]],
                   g_biases=[np.abs(b) for b in r["g_biases"]])
        if acc is None:
            acc = one
        else:
            acc["g_tables"] += one["g_tables"]
            for l in range(len(acc["g_weights"])):
                acc["g_weights"][l] += one["g_weights"][l]
                acc["g_biases"][l] += one["g_biases"][l]
    return acc


def _compare(tag, dec, out, ref, pos_ref=None, terms=None):
    if terms is None:
        _close(f"{tag} tables", host(out["tables"]).reshape(-1), ref["g_tables"].reshape(-1), 1e-3, 1e-4)
        for l in range(len(ref["g_weights"])):
            _close(f"{tag} W{l}", host(out["weights"][l]), ref["g_weights"][l], 1e-3, 1e-4)
            _close(f"{tag} b{l}", host(out["biases"][l]), ref["g_biases"][l], 1e-3, 1e-4)
    else:
        _close_terms(f"{tag} tables", host(out["tables"]).reshape(-1), ref["g_tables"].reshape(-1),
                     terms["g_tables"].reshape(-1), 1e-3, 1e-4)
        for l in range(len(ref["g_weights"])):
            _close_terms(f"{tag} W{l}", host(out["weights"][l]), ref["g_weights"][l], terms["g_weights"][l],
                         1e-3, 1e-4)
            _close_terms(f"{tag} b{l}", host(out["biases"][l]), ref["g_biases"][l], terms["g_biases"][l],
                         1e-3, 1e-4)
    if out["pos"] is not None:
        g = host(out["pos"]).astype(np.float64)
        o = ref["g_pos"] if pos_ref is None else pos_ref
        err = np.linalg.norm(g - o, axis=1)
        nrm = np.linalg.norm(o, axis=1)
        lim = 2e-3 * nrm + 1e-4 * nrm.max()
        ratio = float((err / lim).max())
        say(f"[{tag} pos] max|ref| {nrm.max():.3e} worst err/limit {ratio:.3f}")
        assert ratio <= 1.0


def test_decode_backward_matches_oracle_xyzt():
    dec = S.single_decoder()
    rng = np.random.default_rng(60)
    n = 20000
    pos = _edge_xyzt(rng, n)
    up = _upstream(rng, n)
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    out = _gpu_backward(Decoder(dec), pos, up)
    _compare("xyzt", dec, out, ref)


def test_decode_backward_sequence_frames_scalar_t():
    """One frame of the sequence at its own time (scalar t, stride 3), a
    temporal vertex (half of the 16 corners have zero weight)."""
    dec = S.single_decoder()
    seq = S.Sequence()
    f = 10
    xyzt = seq.xyzt([f])
    pos = np.ascontiguousarray(xyzt[:30000, :3])
    t = float(xyzt[0, 3])
    rng = np.random.default_rng(61)
    up = _upstream(rng, pos.shape[0])
    ref = O.decode_grad(dec, pos.astype(np.float64), t, mode=3, grads=up)
    out = _gpu_backward(Decoder(dec), pos, up, t=t)
    _compare("scalar t", dec, out, ref)


@pytest.mark.parametrize("n", [1, 17, 1000])
def test_decode_backward_small_and_ragged(n):
    dec = S.single_decoder()
    rng = np.random.default_rng(62 + n)
    pos = _edge_xyzt(rng, n)
    up = _upstream(rng, n)
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    out = _gpu_backward(Decoder(dec), pos, up)
    _compare(f"n={n}", dec, out, ref)


def test_decode_backward_adds_render_position_gradient_and_skips_positions():
    dec = S.single_decoder()
    rng = np.random.default_rng(63)
    n = 5000
    pos = _edge_xyzt(rng, n)
    up = _upstream(rng, n)
    gm = rng.normal(size=(n, 3)).astype(np.float32)
    D = Decoder(dec)
    a = _gpu_backward(D, pos, up, grad_means=gm)
    b = _gpu_backward(D, pos, up, want_pos=False)
    assert b["pos"] is None
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    _compare("with means", dec, a, ref, pos_ref=ref["g_pos"] + gm.astype(np.float64))
    for l in range(3):
        np.testing.assert_array_equal(host(a["weights"][l]), host(b["weights"][l]))  # fixed summation order


def test_decode_backward_two_chunks_is_the_sum_of_its_parts():
    """2^21 + 4097 points (two backward chunks): the parameter gradients are
    sums over points, so the whole equals the sum of the two halves computed
    separately; positions are per point.  A sample of points is checked
    against the oracle one by one."""
    dec = S.single_decoder()
    rng = np.random.default_rng(64)
    n1 = 1 << 21
    n = n1 + 4097
    pos = np.empty((n, 4), np.float32)
    pos[:, :3] = S.shell_points(rng, n, 3.0)
    pos[:, 3] = rng.random(n)
    up = _upstream(rng, n)
    D = Decoder(dec)
    whole = _gpu_backward(D, pos, up)
    p1 = _gpu_backward(D, pos[:n1], {k: v[:n1] for k, v in up.items()})
    p2 = _gpu_backward(D, pos[n1:], {k: v[n1:] for k, v in up.items()})
    for key in ("tables",):
        s = host(p1[key]).astype(np.float64) + host(p2[key])
        _close("chunks tables", host(whole[key]).reshape(-1), s.reshape(-1), 1e-5, 1e-6)
    # sums of 2M terms of random sign in fp32, in two different orders: the
    # cancellation leaves differences near 1e-5 of the largest entry
    for l in range(3):
        _close(f"chunks W{l}", host(whole["weights"][l]), host(p1["weights"][l]).astype(np.float64)
               + host(p2["weights"][l]), 1e-4, 1e-4)
        _close(f"chunks b{l}", host(whole["biases"][l]), host(p1["biases"][l]).astype(np.float64)
               + host(p2["biases"][l]), 1e-4, 1e-4)
    wp = host(whole["pos"])
    np.testing.assert_allclose(wp[:n1], host(p1["pos"]), rtol=1e-5, atol=1e-6 * np.abs(wp).max())
    np.testing.assert_allclose(wp[n1:], host(p2["pos"]), rtol=1e-5, atol=1e-6 * np.abs(wp).max())
    idx = np.sort(np.concatenate([rng.choice(n, 300, replace=False), [0, n1 - 1, n1, n - 1]]))
    ref = O.decode_grad(dec, pos[idx].astype(np.float64), mode=3, grads={k: v[idx] for k, v in up.items()})
    g = wp[idx].astype(np.float64)
    err = np.linalg.norm(g - ref["g_pos"], axis=1)
    nrm = np.linalg.norm(ref["g_pos"], axis=1)
    assert (err <= 2e-3 * nrm + 1e-4 * nrm.max()).all()


def test_decode_backward_sparse_upstream_gradients():
    """Most Gaussians without any upstream gradient (as after a render
    backward where only the front layers composite), some with a single
    non-zero component: the decoder backward works on the compacted list of
    the others and must equal the oracle on the whole set."""
    dec = S.single_decoder()
    rng = np.random.default_rng(66)
    n = 30000
    pos = _edge_xyzt(rng, n)
    up = _upstream(rng, n)
    idle = rng.random(n) < 0.8
    for v in up.values():
        v[idle] = 0.0
    one = np.flatnonzero(~idle)[:500]  # a single non-zero component each
    for k, v in up.items():
        v[one] = 0.0
    for j, i in enumerate(one):
        key = ("scales", "quats", "colors", "opacity")[j % 4]
        if key == "opacity":
            up[key][i] = 1.5
        else:
            up[key][i, j % up[key].shape[1]] = 1.5
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    out = _gpu_backward(Decoder(dec), pos, up)
    _compare("sparse", dec, out, ref)
    assert np.all(host(out["pos"])[idle] == 0.0)


@pytest.mark.parametrize("n", [5000, (1 << 22) + 1000])
def test_kept_features_match_recomputation(n):
    """ia_decode_keep gives the same attributes as ia_decode_xyzt (bit for
    bit) and a backward that reuses the kept encoding gives the same
    gradients as one that recomputes it (weights and biases bit for bit,
    the float-atomic table and position sums to rounding); 2^22 + 1000
    points span two forward chunks and three backward chunks."""
    dec = S.single_decoder()
    rng = np.random.default_rng(65)
    pos = _edge_xyzt(rng, n)
    up = _upstream(rng, n)
    D = Decoder(dec)
    x = cuda(pos)
    plain = D.decode_xyzt(x)
    kept, feats = D.decode_keep(x)
    torch.cuda.synchronize()
    for k in plain:
        assert torch.equal(plain[k], kept[k]), k
    g = {k: cuda(v.astype(np.float32)) for k, v in up.items()}
    a = D.backward(x, g)
    b = D.backward(x, g, features=feats)
    torch.cuda.synchronize()
    for l in range(3):
        assert torch.equal(a["weights"][l], b["weights"][l]) and torch.equal(a["biases"][l], b["biases"][l])
    _close("kept tables", host(b["tables"]).reshape(-1), host(a["tables"]).reshape(-1), 1e-5, 1e-6)
    _close("kept pos", host(b["pos"]), host(a["pos"]), 1e-5, 1e-6)


def test_decode_backward_zero_points_and_errors():
    dec = S.single_decoder()
    D = Decoder(dec)
    out = D.backward(torch.empty((0, 4), device="cuda"), {k: torch.empty(0, device="cuda") for k in UP})
    torch.cuda.synchronize()
    assert float(out["tables"].abs().max()) == 0.0
    assert all(float(w.abs().max()) == 0.0 for w in out["weights"])
    assert all(float(b.abs().max()) == 0.0 for b in out["biases"])
    T = Decoder(S.tiny_decoder())
    with pytest.raises(ia.IAError) as e:
        T.backward(torch.zeros((4, 3), device="cuda"), {k: torch.zeros((4, 4), device="cuda") for k in UP}, 0.5)
    assert e.value.status == ia.IA_ERR_UNSUPPORTED


def test_decode_backward_weight_bias_and_position_gradients_are_deterministic():
    """Weights, biases and positions are summed in fixed orders: repeated
    calls agree bit for bit (the table gradient uses float atomics)."""
    dec = S.single_decoder()
    rng = np.random.default_rng(66)
    n = 300_000  # more than one block per level and several LDS-combining blocks
    pos = _edge_xyzt(rng, n)
    up = _upstream(rng, n)
    D = Decoder(dec)
    a = _gpu_backward(D, pos, up)
    b = _gpu_backward(D, pos, up)
    assert torch.equal(a["pos"], b["pos"])
    for k in range(len(a["weights"])):
        assert torch.equal(a["weights"][k], b["weights"][k]) and torch.equal(a["biases"][k], b["biases"][k])
    # the table gradient adds each entry's contributions with float atomics in
    # whatever order the waves arrive: its last bits may vary between runs,
    # within the rounding of an fp32 sum of that entry's terms
    ta, tb = a["tables"], b["tables"]
    diff = (ta - tb).abs()
    scale = float(ta.abs().max())
    frac = float((diff > 0).float().mean())
    say(f"table gradient run-to-run: max |diff| {float(diff.max()):.2e} of max |g| {scale:.2e}, "
        f"{frac:.2e} of entries differ")
    assert float(diff.max()) <= 1e-5 * scale
    assert bool((diff <= 1e-5 * ta.abs() + 1e-7 * scale).all())


# ---------------------------------------------------------------- SH colour head

def _upstream_sh(rng, n):
    return dict(scales=rng.normal(size=(n, 3)), quats=rng.normal(size=(n, 4)), sh=rng.normal(size=(n, 48)),
                opacity=rng.normal(size=n))


@pytest.mark.parametrize("n", [1, 17, 1000, 20000])
def test_sh_head_backward_matches_oracle(n):
    """The Single decoder with the SH colour head (SPIN-4DGS §3.3: the colour
    decoder regresses the 48 coefficients, whose gradients reach the head
    unchanged), on edge positions and ragged sizes."""
    dec = S.single_decoder_sh()
    rng = np.random.default_rng(70 + n)
    pos = _edge_xyzt(rng, n)
    up = _upstream_sh(rng, n)
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    out = _gpu_backward(Decoder(dec), pos, up)
    _compare(f"sh {n}", dec, out, ref)


def test_sh_head_backward_only_sh_gradients_count():
    """Gaussians whose only non-zero upstream gradient is one SH coefficient
    take part (the active list reads all 48); those with none are skipped
    without changing any gradient.  Three quarters of the Gaussians carry one
    coefficient each, about 300 terms per head row, so that, as in the dense
    cases, a one-ulp fp16 flip of a hidden activation stays inside the
    module's bound."""
    dec = S.single_decoder_sh()
    rng = np.random.default_rng(75)
    n = 20000
    pos = _edge_xyzt(rng, n)
    up = {k: np.zeros_like(v) for k, v in _upstream_sh(rng, n).items()}
    idx = rng.choice(n, size=3 * n // 4, replace=False)
    coef = rng.integers(48, size=idx.size)
    up["sh"][idx, coef] = rng.normal(size=idx.size)
    up["sh"][idx[:5], 47] = 1.0  # the last coefficient too
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    out = _gpu_backward(Decoder(dec), pos, up)
    _compare("sh only", dec, out, ref)
    # Gaussians without any upstream gradient have no position gradient
    rest = np.setdiff1d(np.arange(n), idx)
    assert float(np.abs(host(out["pos"])[rest]).max()) == 0.0


def test_sh_head_backward_is_deterministic():
    dec = S.single_decoder_sh()
    rng = np.random.default_rng(76)
    n = 5000
    pos = _edge_xyzt(rng, n)
    up = _upstream_sh(rng, n)
    D = Decoder(dec)
    a = _gpu_backward(D, pos, up)
    a = {k: ([x.clone() for x in v] if isinstance(v, list) else v.clone()) for k, v in a.items()}
    b = _gpu_backward(D, pos, up)
    for l in range(3):
        assert torch.equal(a["weights"][l], b["weights"][l]) and torch.equal(a["biases"][l], b["biases"][l])
    assert torch.equal(a["pos"], b["pos"])


# ---------------------------------------------------------------- per-attribute decoder

def _upstream_paper(rng, n, sh):
    return _upstream_sh(rng, n) if sh else _upstream(rng, n)


@pytest.mark.parametrize("sh,n", [(True, 1), (True, 17), (True, 1000), (True, 20000), (False, 17), (False, 20000)])
def test_paper_decoder_backward_matches_oracle(sh, n):
    """The per-attribute decoder of SPIN-4DGS §3.3 (one GELU MLP 64 -> 64 ->
    64 -> out per attribute over the F = 4 encoding, hidden width from §4):
    twelve weight and bias gradients, the table gradient (the four branches'
    encoding gradients summed) and the position gradient."""
    dec = S.paper_decoder(log2T=12, sh=sh)
    rng = np.random.default_rng(80 + n + (1000 if sh else 0))
    pos = _edge_xyzt(rng, n)
    up = _upstream_paper(rng, n, sh)
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    out = _gpu_backward(Decoder(dec), pos, up)
    assert len(out["weights"]) == 12
    terms = _term_sums(dec, pos, up) if n <= 1000 else None
    _compare(f"paper {'sh' if sh else 'rgb'} {n}", dec, out, ref, terms=terms)


def test_paper_decoder_backward_one_attribute_at_a_time():
    """Upstream gradients on one attribute only: the other branches' weight
    and bias gradients are exactly zero, and the encoding's gradient is that
    branch's alone (checked against the oracle)."""
    dec = S.paper_decoder(log2T=12, sh=True)
    rng = np.random.default_rng(85)
    n = 8000
    pos = _edge_xyzt(rng, n)
    full = _upstream_sh(rng, n)
    D = Decoder(dec)
    for br, key in enumerate(("scales", "quats", "sh", "opacity")):
        up = {k: (v if k == key else np.zeros_like(v)) for k, v in full.items()}
        ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
        out = _gpu_backward(D, pos, up)
        for k in range(12):
            if k // 3 != br:
                assert float(out["weights"][k].abs().max()) == 0.0 and float(out["biases"][k].abs().max()) == 0.0
        _compare(f"paper only {key}", dec, out, ref)


def test_paper_decoder_backward_chunks_kept_features_and_determinism():
    """2^21 + 4097 points (two backward chunks, the branch gradients reduced
    after each): the parameter gradients equal the sum of the two halves
    computed separately; a backward from the encoding kept by the forward
    equals one that recomputes it (weights and biases bit for bit); repeated
    calls agree bit for bit except for the float-atomic table gradient."""
    dec = S.paper_decoder(log2T=14, sh=True)
    rng = np.random.default_rng(86)
    n1 = 1 << 21
    n = n1 + 4097
    pos = np.empty((n, 4), np.float32)
    pos[:, :3] = S.shell_points(rng, n, 3.0)
    pos[:, 3] = rng.random(n)
    up = _upstream_sh(rng, n)
    D = Decoder(dec)
    whole = _gpu_backward(D, pos, up)
    whole = {k: ([x.clone() for x in v] if isinstance(v, list) else v.clone()) for k, v in whole.items()}
    p1 = _gpu_backward(D, pos[:n1], {k: v[:n1] for k, v in up.items()})
    p1 = {k: ([x.clone() for x in v] if isinstance(v, list) else v.clone()) for k, v in p1.items()}
    p2 = _gpu_backward(D, pos[n1:], {k: v[n1:] for k, v in up.items()})
    s = host(p1["tables"]).astype(np.float64) + host(p2["tables"])
    _close("paper chunks tables", host(whole["tables"]).reshape(-1), s.reshape(-1), 1e-5, 1e-6)
    for l in range(12):
        _close(f"paper chunks W{l}", host(whole["weights"][l]), host(p1["weights"][l]).astype(np.float64)
               + host(p2["weights"][l]), 1e-4, 1e-4)
        _close(f"paper chunks b{l}", host(whole["biases"][l]), host(p1["biases"][l]).astype(np.float64)
               + host(p2["biases"][l]), 1e-4, 1e-4)
    wp = host(whole["pos"])
    np.testing.assert_allclose(wp[:n1], host(p1["pos"]), rtol=1e-5, atol=1e-6 * np.abs(wp).max())
    np.testing.assert_allclose(wp[n1:], host(p2["pos"]), rtol=1e-5, atol=1e-6 * np.abs(wp).max())
    idx = np.sort(np.concatenate([rng.choice(n, 200, replace=False), [0, n1 - 1, n1, n - 1]]))
    ref = O.decode_grad(dec, pos[idx].astype(np.float64), mode=3, grads={k: v[idx] for k, v in up.items()})
    err = np.linalg.norm(wp[idx].astype(np.float64) - ref["g_pos"], axis=1)
    nrm = np.linalg.norm(ref["g_pos"], axis=1)
    assert (err <= 2e-3 * nrm + 1e-4 * nrm.max()).all()
    # kept encoding and repeat
    x = cuda(pos)
    _, feats = D.decode_keep(x)
    g = {k: cuda(v.astype(np.float32)) for k, v in up.items()}
    kept = D.backward(x, g, features=feats)
    torch.cuda.synchronize()
    for l in range(12):
        assert torch.equal(kept["weights"][l], whole["weights"][l]) and torch.equal(kept["biases"][l], whole["biases"][l])
    assert torch.equal(kept["pos"], whole["pos"])
    _close("paper kept tables", host(kept["tables"]).reshape(-1), host(whole["tables"]).reshape(-1), 1e-5, 1e-6)


def test_paper_decoder_backward_zero_points_and_sparse():
    dec = S.paper_decoder(log2T=12, sh=False)
    D = Decoder(dec)
    out = D.backward(torch.empty((0, 4), device="cuda"), {k: torch.empty(0, device="cuda") for k in UP})
    torch.cuda.synchronize()
    assert float(out["tables"].abs().max()) == 0.0
    assert len(out["weights"]) == 12
    assert all(float(w.abs().max()) == 0.0 for w in out["weights"])
    assert all(float(b.abs().max()) == 0.0 for b in out["biases"])
    rng = np.random.default_rng(87)
    n = 20000
    pos = _edge_xyzt(rng, n)
    up = _upstream(rng, n)
    idle = rng.random(n) < 0.8
    for v in up.values():
        v[idle] = 0.0
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    out = _gpu_backward(D, pos, up)
    _compare("paper sparse", dec, out, ref)
    assert np.all(host(out["pos"])[idle] == 0.0)


# Fine-level table gradient through the buckets: above 65,536 Gaussians with a
# gradient per backward chunk, the levels finer than 300 vertices per axis
# write (entry, contribution) records into per-bucket runs that one block per
# bucket sums in LDS; below it they use direct float atomics.  These cases
# cross that threshold and compare with the oracle's fp64 gradients.

def test_bucketed_fine_levels_match_oracle():
    """100,000 points at general times (all 16 corners weighted) and edge
    positions, two features per entry, 2^19-entry tables (256 buckets of
    2,048 entries per level finer than 300 vertices per axis)."""
    dec = S.single_decoder()
    rng = np.random.default_rng(91)
    n = 100_000
    pos = _edge_xyzt(rng, n)
    up = _upstream(rng, n)
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    out = _gpu_backward(Decoder(dec), pos, up)
    _compare("bucketed xyzt", dec, out, ref)


def test_bucketed_fine_levels_paper_decoder_match_oracle():
    """The per-attribute decoder (four features per entry) with 70,000 points
    and 2^17-entry tables (64 buckets per fine level)."""
    dec = S.paper_decoder(log2T=17, sh=False)
    rng = np.random.default_rng(92)
    n = 70_000
    pos = _edge_xyzt(rng, n)
    up = _upstream_paper(rng, n, False)
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    out = _gpu_backward(Decoder(dec), pos, up)
    _compare("bucketed paper", dec, out, ref)


def test_bucket_overflow_goes_to_the_table_directly():
    """80,000 points on six distinct positions: each fine level's records all
    fall into a few buckets, far beyond a bucket's capacity (5/4 of an even
    share), so most of them take the direct-atomic fallback; the gradients
    still match the oracle."""
    dec = S.single_decoder()
    rng = np.random.default_rng(93)
    n = 80_000
    base = _edge_xyzt(rng, 6)
    base[:, 3] = np.float32([0.2, 0.4, 0.6, 0.8, 0.3, 0.7])
    pos = base[rng.integers(0, 6, n)]
    up = _upstream(rng, n)
    ref = O.decode_grad(dec, pos.astype(np.float64), mode=3, grads=up)
    out = _gpu_backward(Decoder(dec), pos, up)
    _compare("bucket overflow", dec, out, ref)
