"""C-ABI checks that need no GPU: libia.so loads, exports every entry point
include/ia.h declares, and rejects invalid arguments on the host before any
HIP call is made."""
import ctypes as C
import os
import re

import pytest

from implicit_attribute_decode_amd import ia

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "ia.h")).read()
    return sorted(set(re.findall(r"^IA_API\s+[\w\s\*]*?\b(ia_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(ia.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ia.load()
    for name in _declared():
        assert hasattr(L, name), name


def _hash(**kw):
    d = dict(L=16, F=2, log2T=19, base_res=16.0, growth=1.5, temporal_res=150, table_dtype=ia.IA_DTYPE_F16,
             t_min=0.0, t_max=1.0)
    d.update(kw)
    return ia.HashDesc(**d)


def _mlp(**kw):
    d = dict(in_dim=32, n_hidden=2, hidden=(C.c_int32 * 4)(64, 64, 0, 0), activation=ia.IA_ACT_GELU,
             dtype=ia.IA_DTYPE_F16)
    d.update(kw)
    return ia.MLPDesc(**d)


def test_decoder_create_accepts_the_supported_shapes():
    h = ia.ia_decoder_create(_hash(), _mlp())
    ia.ia_decoder_destroy(h)
    tiny = ia.HashDesc(4, 2, 12, 8.0, 2.0, 0, ia.IA_DTYPE_F32, 0.0, 1.0)
    h = ia.ia_decoder_create(tiny, ia.MLPDesc(8, 1, (C.c_int32 * 4)(32, 0, 0, 0), ia.IA_ACT_RELU, ia.IA_DTYPE_F32))
    ia.ia_decoder_destroy(h)
    h = ia.ia_decoder_create(_hash(), _mlp(color=ia.IA_COLOR_SH3))
    ia.ia_decoder_destroy(h)
    paper = _hash(F=4, log2T=21)
    for color in (ia.IA_COLOR_RGB, ia.IA_COLOR_SH3):
        h = ia.ia_decoder_create(paper, _mlp(in_dim=64, branches=ia.IA_BRANCHES_PER_ATTRIBUTE, color=color))
        ia.ia_decoder_destroy(h)
    with pytest.raises(ia.IAError) as e:  # the SH head needs the fp16 decoder
        ia.ia_decoder_create(tiny, ia.MLPDesc(8, 1, (C.c_int32 * 4)(32, 0, 0, 0), ia.IA_ACT_RELU, ia.IA_DTYPE_F32,
                                              ia.IA_COLOR_SH3))
    assert e.value.status == ia.IA_ERR_UNSUPPORTED


@pytest.mark.parametrize("hkw,mkw,status", [
    (dict(L=0), {}, ia.IA_ERR_INVALID_ARG),
    (dict(F=3), {}, ia.IA_ERR_UNSUPPORTED),
    (dict(F=4), dict(in_dim=64), ia.IA_ERR_UNSUPPORTED),  # a shared trunk needs F = 2
    (dict(F=4, table_dtype=ia.IA_DTYPE_F32), dict(in_dim=64, branches=1), ia.IA_ERR_UNSUPPORTED),
    ({}, dict(branches=1), ia.IA_ERR_UNSUPPORTED),  # per-attribute branches need F = 4
    ({}, dict(branches=2), ia.IA_ERR_INVALID_ARG),
    ({}, dict(color=5), ia.IA_ERR_INVALID_ARG),
    (dict(log2T=30), {}, ia.IA_ERR_INVALID_ARG),
    (dict(base_res=1.0), {}, ia.IA_ERR_INVALID_ARG),
    (dict(t_max=0.0), {}, ia.IA_ERR_INVALID_ARG),
    (dict(temporal_res=1), {}, ia.IA_ERR_INVALID_ARG),
    ({}, dict(in_dim=31), ia.IA_ERR_INVALID_ARG),
    ({}, dict(n_hidden=3), ia.IA_ERR_UNSUPPORTED),
    ({}, dict(activation=7), ia.IA_ERR_INVALID_ARG),
    ({}, dict(hidden=(C.c_int32 * 4)(128, 64, 0, 0)), ia.IA_ERR_UNSUPPORTED),
    (dict(table_dtype=ia.IA_DTYPE_F32), {}, ia.IA_ERR_UNSUPPORTED),
])
def test_decoder_create_rejects(hkw, mkw, status):
    with pytest.raises(ia.IAError) as e:
        ia.ia_decoder_create(_hash(**hkw), _mlp(**mkw))
    assert e.value.status == status
    assert ia.ia_last_error() != ""


def test_decode_without_params_is_rejected_before_any_gpu_work():
    L = ia.load()
    h = ia.ia_decoder_create(_hash(), _mlp())
    g = ia.Gaussians()
    assert L.ia_decode(h, None, 10, C.c_float(0.5), C.byref(g), None, 0, None, None) == ia.IA_ERR_INVALID_ARG
    assert "not set" in ia.ia_last_error()
    ia.ia_decoder_destroy(h)
    assert L.ia_decode(None, None, 10, C.c_float(0.5), C.byref(g), None, 0, None, None) == ia.IA_ERR_INVALID_ARG


def test_workspace_size_validation_and_growth():
    n = ia.ia_render_workspace_size(200_000, 1, 640, 360, 1_000_000)
    assert n > 24 * 1_000_000
    assert ia.ia_render_workspace_size(200_000, 1, 640, 360, 2_000_000) > n
    assert ia.ia_render_workspace_size(0, 1, 64, 64, 1) > 0
    for args in [(-1, 1, 64, 64, 10), (10, 0, 64, 64, 10), (10, 1, 0, 64, 10), (10, 1, 64, 64, 0),
                 (10, 1, 64, 64, 1 << 32)]:
        with pytest.raises(ia.IAError) as e:
            ia.ia_render_workspace_size(*args)
        assert e.value.status == ia.IA_ERR_INVALID_ARG


def test_render_argument_errors_are_synchronous():
    L = ia.load()
    cam = ia.Camera()
    cam.W, cam.H, cam.fx, cam.fy = 64, 64, 60.0, 60.0
    fo = (C.c_int64 * 2)(0, 0)
    g = ia.Gaussians()
    # null image
    assert L.ia_render(C.byref(g), fo, 1, C.byref(cam), None, 0, 10, None, None, None) == ia.IA_ERR_INVALID_ARG
    # non-monotone frame offsets
    fo2 = (C.c_int64 * 3)(0, 5, 3)
    cams = (ia.Camera * 2)(cam, cam)
    img = C.c_void_p(256)
    assert L.ia_render(C.byref(g), fo2, 2, cams, img, 1 << 20, 10, img, None, None) == ia.IA_ERR_INVALID_ARG
    # mismatched camera sizes
    cam2 = ia.Camera()
    cam2.W, cam2.H = 32, 64
    cams = (ia.Camera * 2)(cam, cam2)
    fo3 = (C.c_int64 * 3)(0, 0, 0)
    assert L.ia_render(C.byref(g), fo3, 2, cams, img, 1 << 20, 10, img, None, None) == ia.IA_ERR_INVALID_ARG
    # workspace too small (fake aligned address: nothing is dereferenced)
    assert L.ia_render(C.byref(g), fo, 1, C.byref(cam), img, 16, 10, img, None, None) == ia.IA_ERR_WORKSPACE_TOO_SMALL
    # unsupported SH degree with Gaussians present
    fo4 = (C.c_int64 * 2)(0, 4)
    g2 = ia.Gaussians(1024, 0, 1024, 1024, 1024, 1024, 1024, 2)
    assert L.ia_render(C.byref(g2), fo4, 1, C.byref(cam), img, 1 << 30, 10, img, None, None) == ia.IA_ERR_UNSUPPORTED


def test_render_binning_mode_is_validated_per_call():
    """An unknown ia_render_aux.binning is an argument error, returned before
    anything is enqueued (fake aligned addresses: nothing is dereferenced)."""
    L = ia.load()
    cam = ia.Camera()
    cam.W, cam.H, cam.fx, cam.fy = 64, 64, 60.0, 60.0
    fo = (C.c_int64 * 2)(0, 0)
    g = ia.Gaussians()
    img = C.c_void_p(256)
    for bad in (-1, 3, 100):
        aux = ia.RenderAux()
        aux.binning = bad
        assert L.ia_render(C.byref(g), fo, 1, C.byref(cam), img, 1 << 30, 10, img, C.byref(aux),
                           None) == ia.IA_ERR_INVALID_ARG
        assert "binning" in ia.ia_last_error()


def test_training_entry_points_validate_before_any_gpu_work():
    """Loss, optimiser and densify argument errors return before anything is
    enqueued (fake aligned addresses: nothing is dereferenced)."""
    L = ia.load()
    p = C.c_void_p(1 << 20)
    # image loss: workspace size, lambda outside [0, 1], too small a workspace, too many frames
    n = ia.ia_image_loss_workspace_size(2, 1080, 1920)
    assert n >= 3 * 2 * 3 * 1080 * 1920 * 4
    with pytest.raises(ia.IAError):
        ia.ia_image_loss_workspace_size(0, 10, 10)
    assert L.ia_image_loss(p, p, 1, 8, 8, C.c_float(1.5), p, 1 << 30, p, p, None) == ia.IA_ERR_INVALID_ARG
    assert L.ia_image_loss(p, p, 1, 8, 8, C.c_float(0.2), p, 16, p, p, None) == ia.IA_ERR_WORKSPACE_TOO_SMALL
    assert L.ia_image_loss(p, p, 30000, 8, 8, C.c_float(0.2), p, 1 << 40, p, p, None) == ia.IA_ERR_INVALID_ARG
    # Adam: step 0, beta1 = 1, negative lr; strided with stride < dim
    f = C.c_float
    assert L.ia_adam_step(p, p, p, p, 10, f(1e-3), f(0.9), f(0.999), f(1e-15), 0, None, None) == ia.IA_ERR_INVALID_ARG
    assert L.ia_adam_step(p, p, p, p, 10, f(1e-3), f(1.0), f(0.999), f(1e-15), 1, None, None) == ia.IA_ERR_INVALID_ARG
    assert L.ia_adam_step(p, p, p, p, 10, f(-1.0), f(0.9), f(0.999), f(1e-15), 1, None, None) == ia.IA_ERR_INVALID_ARG
    assert L.ia_adam_step_strided(p, 3, 4, p, p, p, 10, f(1e-3), f(0.9), f(0.999), f(1e-15), 1,
                                  None) == ia.IA_ERR_INVALID_ARG
    # densify: workspace size, capacity below 2 N, negative threshold, null params
    assert ia.ia_densify_workspace_size(8_000_000) >= 8 * (8_000_000 // 4096)
    prm = ia.DensifyParams(1e-4, 0.05, 0.005)
    args = [p] * 9
    assert L.ia_densify(*args, 100, C.byref(prm), p, p, p, 150, p, p, 1 << 20, None) == ia.IA_ERR_INVALID_ARG
    bad = ia.DensifyParams(-1.0, 0.05, 0.005)
    assert L.ia_densify(*args, 100, C.byref(bad), p, p, p, 200, p, p, 1 << 20, None) == ia.IA_ERR_INVALID_ARG
    assert L.ia_densify(*args, 100, None, p, p, p, 200, p, p, 1 << 20, None) == ia.IA_ERR_INVALID_ARG
    assert L.ia_densify(*args, 100, C.byref(prm), p, p, p, 200, p, p, 0, None) == ia.IA_ERR_WORKSPACE_TOO_SMALL
    # accumulate: negative N
    assert L.ia_densify_accumulate(p, -1, p, p, None) == ia.IA_ERR_INVALID_ARG


def test_lr_schedule_matches_the_oracle_and_validates():
    """ia_lr_at (host-only) against the oracle's warm-up + cosine schedule
    ([SPIN] §4 implementation details): equal within one fp32 ulp of the
    base rate over warm-up, decay and the floor after the last iteration."""
    from oracle import train as T

    for base, warm, total in ((8e-3, 1000, 40000), (3e-5, 2, 10), (1.6e-4, 0, 100)):
        for step in sorted({0, 1, max(warm - 1, 0), warm, warm + 1, (warm + total) // 2, total - 1, total,
                            total + 5}):
            got = ia.ia_lr_at(base, step, warm, total, 1e-7)
            want = T.lr_schedule(step, base, warm, total, 1e-7)
            assert abs(got - want) <= 2.0 ** -23 * base, (base, warm, total, step, got, want)
    assert ia.ia_lr_at(8e-3, 40000, 1000, 40000, 1e-7) == pytest.approx(1e-7, rel=1e-6)
    L = ia.load()
    out = C.c_float()
    for args in ((1e-3, -1, 0, 10), (1e-3, 0, -1, 10), (1e-3, 0, 20, 10), (float("nan"), 0, 0, 10), (-1.0, 0, 0, 10)):
        assert L.ia_lr_at(C.c_float(args[0]), args[1], args[2], args[3], C.c_float(1e-7),
                          C.byref(out)) == ia.IA_ERR_INVALID_ARG
    assert L.ia_lr_at(C.c_float(1e-3), 0, 0, 10, C.c_float(1e-7), None) == ia.IA_ERR_INVALID_ARG


def test_device_memory_is_allocated_only_when_parameters_are_set():
    """Handles own only their parameters: hipMalloc appears only in the
    parameter uploads of the set_params calls; every other entry point takes
    its scratch from a caller workspace."""
    import glob

    allowed = {"upload_param", "ia_decoder_set_params", "ia_hexplane_set_params"}
    defn = re.compile(r"^(?!\s)(?!#)(?!//)[\w:<>\*&, ]*?\b(\w+)\s*\(")
    seen = set()
    for path in sorted(glob.glob(os.path.join(ROOT, "implicit_attribute_decode_amd", "csrc", "*"))):
        if not path.endswith((".hip", ".h", ".cpp", ".c")):
            continue
        fn = None
        for line in open(path).read().splitlines():
            m = defn.match(line)
            if m:
                fn = m.group(1)
            code = line.split("//")[0]
            if re.search(r"\bhipMalloc\w*\s*\(", code):
                assert fn in allowed, (os.path.basename(path), fn, line.strip())
                seen.add(fn)
    assert seen == allowed
