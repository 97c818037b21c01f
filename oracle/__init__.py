"""CPU oracle for decode + render.  TEST INFRASTRUCTURE, not the product path.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It never imports the HIP library or its Python binding; the
two sides share nothing but the seeded inputs they are handed.

Each function wraps one step of oracle.c (plain C, see that file for the
definition and the passage of the pages it follows) and works on numpy arrays.
Configuration objects are duck-typed (attributes L, F, log2T, ... for the
hash; dims, act, f16 for the MLP; R, t, fx, ... for cameras), so this module
does not depend on where the inputs come from.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None


def lib():
    """The compiled oracle.  With ORACLE_SANITIZED=1 in the environment, the
    AddressSanitizer + UndefinedBehaviorSanitizer build (the process must have
    preloaded the sanitizer runtimes, see build.sanitizer_runtimes)."""
    global _lib
    if _lib is None:
        san = os.environ.get("ORACLE_SANITIZED") == "1"
        path = _build.SAN_LIB if san else _build.LIB
        if not os.path.exists(path):
            _build.build(sanitize=san)
        _lib = C.CDLL(path)
        _declare(_lib)
    return _lib


# --------------------------------------------------------------------------
# ctypes structures (mirror oracle.c)
# --------------------------------------------------------------------------


class _Hash(C.Structure):
    _fields_ = [("L", C.c_int), ("F", C.c_int), ("log2T", C.c_int), ("base_res", C.c_double),
                ("growth", C.c_double), ("temporal_res", C.c_int), ("table_f16", C.c_int),
                ("t_min", C.c_float), ("t_max", C.c_float)]


class _MLP(C.Structure):
    _fields_ = [("n_layers", C.c_int), ("dims", C.c_int * 8), ("act", C.c_int), ("w_f16", C.c_int),
                ("branches", C.c_int)]


class _HexPlane(C.Structure):
    _fields_ = [("res_xyz", C.c_int), ("res_t", C.c_int), ("C", C.c_int), ("aabb", C.c_float)]


class _Camera(C.Structure):
    _fields_ = [("R", C.c_float * 9), ("t", C.c_float * 3), ("fx", C.c_float), ("fy", C.c_float),
                ("cx", C.c_float), ("cy", C.c_float), ("near_z", C.c_float), ("W", C.c_int),
                ("H", C.c_int), ("bg", C.c_float * 3)]


P = C.c_void_p


def _declare(L):
    L.orc_num_threads.restype = C.c_int
    L.orc_num_threads.argtypes = []
    L.orc_set_num_threads.restype = None
    L.orc_set_num_threads.argtypes = [C.c_int]
    L.orc_half_to_double.restype = C.c_double
    L.orc_half_to_double.argtypes = [C.c_uint16]
    L.orc_double_to_half.restype = C.c_uint16
    L.orc_double_to_half.argtypes = [C.c_double]
    L.orc_level_res.argtypes = [P, P, P, P]
    L.orc_normalize.argtypes = [P, P, C.c_int, C.c_float, C.c_long, P]
    L.orc_encode.argtypes = [P, P, P, C.c_long, P]
    L.orc_mlp_forward.argtypes = [P, P, P, P, C.c_long, C.c_int, P]
    L.orc_activate.argtypes = [P, C.c_long, P, P, P, P]
    L.orc_activate_sh.argtypes = [P, C.c_long, P, P, P, P]
    L.orc_decode.argtypes = [P, P, P, P, P, P, C.c_int, C.c_float, C.c_long, C.c_int, P, P, P, P, P]
    L.orc_sh_basis.argtypes = [P, C.c_long, P]
    L.orc_hexplane_features.argtypes = [P, P, P, C.c_float, C.c_long, P]
    L.orc_hexplane_deform.argtypes = [P, P, P, P, P, P, P, P, P, C.c_float, C.c_long, C.c_int,
                                      P, P, P, P]
    L.orc_preprocess.argtypes = [P, C.c_int, P, P, P, P, P, P, P, P, P, P]
    L.orc_sh_colors.argtypes = [P, C.c_int, P, P, P, P]
    L.orc_bin.restype = C.c_long
    L.orc_bin.argtypes = [C.c_int, C.c_int, C.c_int, P, P, P, P, C.c_long, P, P, P]
    L.orc_raster_tiles.argtypes = [C.c_int, P, P, P, P, P, P, P, P, P, P, P]
    L.orc_render_grad.argtypes = [P, C.c_int, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
    L.orc_render_grad.restype = None
    L.orc_decode_grad.argtypes = [P, P, P, P, P, P, P, C.c_long, C.c_int, P, P, P, P, P, P, P, P, P, P, P,
                                  P, P, P]
    L.orc_decode_grad.restype = None
    L.orc_raster_brute.argtypes = [P, C.c_long, C.c_long, P, P, P, P, P, P, P, C.c_int, P, C.c_long,
                                   P, P, P, P]


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    """Threads for the oracle's later parallel loops."""
    lib().orc_set_num_threads(int(n))


def _p(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# binary16
# --------------------------------------------------------------------------


def half_to_double(bits: np.ndarray) -> np.ndarray:
    f = lib().orc_half_to_double
    b = np.asarray(bits, np.uint16).ravel()
    return np.array([f(int(x)) for x in b], np.float64).reshape(np.shape(bits))


def double_to_half(x: np.ndarray) -> np.ndarray:
    f = lib().orc_double_to_half
    a = np.asarray(x, np.float64).ravel()
    return np.array([f(float(v)) for v in a], np.uint16).reshape(np.shape(x))


# --------------------------------------------------------------------------
# Decode
# --------------------------------------------------------------------------


def _hash(h) -> _Hash:
    return _Hash(int(h.L), int(h.F), int(h.log2T), float(h.base_res), float(h.growth),
                 int(h.temporal_res), int(bool(h.table_f16)), float(h.t_min), float(h.t_max))


def _mlp(dims, act, f16) -> _MLP:
    m = _MLP()
    m.n_layers = len(dims) - 1
    for i, d in enumerate(dims):
        m.dims[i] = int(d)
    m.act = {"relu": 0, "gelu": 1}[act]
    m.w_f16 = int(bool(f16))
    return m


def level_res(h):
    n = int(h.L)
    rs, rt, dn = (np.zeros(n, np.int32) for _ in range(3))
    hs = _hash(h)
    lib().orc_level_res(C.byref(hs), _p(rs), _p(rt), _p(dn))
    return rs, rt, dn.astype(bool)


def normalize(h, pos: np.ndarray, t: float | None = None) -> np.ndarray:
    """Eq. 7-8 in fp32.  pos is [N,3] (with scalar t) or [N,4] (x,y,z,t)."""
    pos = _c(pos, np.float32)
    n, stride = pos.shape
    out = np.zeros((n, 4), np.float32)
    hs = _hash(h)
    lib().orc_normalize(C.byref(hs), _p(pos), stride, float(t or 0.0), n, _p(out))
    return out


def _tables(h, tables):
    return _c(tables, np.float16 if h.table_f16 else np.float32)


def encode(h, tables: np.ndarray, xt: np.ndarray) -> np.ndarray:
    xt = _c(xt, np.float32)
    tb = _tables(h, tables)
    z = np.zeros((xt.shape[0], int(h.L) * int(h.F)), np.float64)
    hs = _hash(h)
    lib().orc_encode(C.byref(hs), _p(tb), _p(xt), xt.shape[0], _p(z))
    return z


def _layers(weights, biases, f16):
    ws = [_c(w, np.float16 if f16 else np.float32) for w in weights]
    bs = [_c(b, np.float32) for b in biases]
    wp = (C.c_void_p * len(ws))(*[w.ctypes.data for w in ws])
    bp = (C.c_void_p * len(bs))(*[b.ctypes.data for b in bs])
    return ws, bs, wp, bp


def mlp_forward(dims, act, f16, weights, biases, x: np.ndarray, mode: int = 0) -> np.ndarray:
    x = _c(x, np.float64)
    m = _mlp(dims, act, f16)
    keep = _layers(weights, biases, f16)
    out = np.zeros((x.shape[0], dims[-1]), np.float64)
    lib().orc_mlp_forward(C.byref(m), keep[2], keep[3], _p(x), x.shape[0], int(mode), _p(out))
    return out


def activate(raw: np.ndarray) -> dict:
    raw = _c(raw, np.float64)
    n = raw.shape[0]
    s, q, c, o = np.zeros((n, 3)), np.zeros((n, 4)), np.zeros((n, 3)), np.zeros(n)
    lib().orc_activate(_p(raw), n, _p(s), _p(q), _p(c), _p(o))
    return dict(scales=s, quats=q, colors=c, opacity=o)


def activate_sh(raw: np.ndarray) -> dict:
    """Eq. 11 with the SH colour head: raw [N,56] -> scales, quats, sh [N,16,3], opacity."""
    raw = _c(raw, np.float64)
    n = raw.shape[0]
    s, q, sh, o = np.zeros((n, 3)), np.zeros((n, 4)), np.zeros((n, 16, 3)), np.zeros(n)
    lib().orc_activate_sh(_p(raw), n, _p(s), _p(q), _p(sh), _p(o))
    return dict(scales=s, quats=q, sh=sh, opacity=o)


def decode(dec, pos: np.ndarray, t: float | None = None, mode: int = 0) -> dict:
    """Full decode of a DecoderParams-like object.  mode 1 = fp16 emulation.
    A head of 56 outputs is the SH colour decoder (returns sh [N,16,3]
    instead of colors)."""
    h, m = dec.hash, dec.mlp
    if getattr(m, "branches", False):
        # one MLP per attribute (scale, rotation, colour, opacity) on the same z
        z = encode(h, dec.tables, normalize(h, pos, t))
        sh = int(m.dims[-1]) == 56
        outs = (3, 4, 48 if sh else 3, 1)
        nl = len(m.dims) - 1
        raw = np.concatenate([
            mlp_forward(list(m.dims[:-1]) + [o], m.act, m.f16, dec.weights[b * nl:(b + 1) * nl],
                        dec.biases[b * nl:(b + 1) * nl], z, mode) for b, o in enumerate(outs)], axis=1)
        return dict(raw=raw, **(activate_sh(raw) if sh else activate(raw)))
    if int(m.dims[-1]) == 56:
        z = encode(h, dec.tables, normalize(h, pos, t))
        raw = mlp_forward(m.dims, m.act, m.f16, dec.weights, dec.biases, z, mode)
        return dict(raw=raw, **activate_sh(raw))
    pos = _c(pos, np.float32)
    n, stride = pos.shape
    tb = _tables(h, dec.tables)
    mm = _mlp(m.dims, m.act, m.f16)
    keep = _layers(dec.weights, dec.biases, m.f16)
    raw = np.zeros((n, 11))
    s, q, c, o = np.zeros((n, 3)), np.zeros((n, 4)), np.zeros((n, 3)), np.zeros(n)
    hs = _hash(h)
    lib().orc_decode(C.byref(hs), _p(tb), C.byref(mm), keep[2], keep[3], _p(pos), stride,
                     float(t or 0.0), n, int(mode), _p(raw), _p(s), _p(q), _p(c), _p(o))
    return dict(raw=raw, scales=s, quats=q, colors=c, opacity=o)


def decode_grad(dec, pos: np.ndarray, t=None, mode: int = 0, grads: dict | None = None,
                params: dict | None = None) -> dict:
    """fp64 forward (and, with grads, backward) of the decode; see
    orc_decode_grad.  pos: [N,3] with scalar or per-point t, or [N,4].
    Parameters default to the stored values of dec converted exactly to
    float64; params may override tables / weights / biases (float64), e.g.
    for finite differences.  grads: upstream dL/d(scales [N,3], quats [N,4],
    colors [N,3] -- or sh [N,48] for a 56-output SH colour head, which is then
    returned as sh [N,48] --, opacity [N]).  mode bit 0: fp16 rounding of the MLP input
    and hidden activations; bit 1: fp32 normalisation and cell decision.
    Returns raw, scales, quats, colors, opacity, flags, signature and, with
    grads, g_tables [L,T,F], g_weights, g_biases (lists) and g_pos [N,3]."""
    h, m = dec.hash, dec.mlp
    pos = np.asarray(pos, np.float64)
    n = pos.shape[0]
    if pos.shape[1] == 4:
        tp = _c(pos[:, 3], np.float64)
    else:
        tp = _c(np.broadcast_to(np.float64(t or 0.0), (n,)), np.float64)
    xyz = _c(pos[:, :3], np.float64)
    params = params or {}
    tables = _c(params["tables"] if "tables" in params else np.asarray(dec.tables), np.float64)
    ws = [_c(w, np.float64) for w in (params["weights"] if "weights" in params else dec.weights)]
    bs = [_c(b, np.float64) for b in (params["biases"] if "biases" in params else dec.biases)]
    wp = (C.c_void_p * len(ws))(*[w.ctypes.data for w in ws])
    bp = (C.c_void_p * len(bs))(*[b.ctypes.data for b in bs])
    hs = _hash(h)
    mm = _mlp(m.dims, m.act, m.f16)
    mm.branches = int(bool(getattr(m, "branches", False)))
    head = int(m.dims[-1])
    cname, ncol = ("sh", 48) if head == 56 else ("colors", 3)
    out = dict(raw=np.zeros((n, head)), scales=np.zeros((n, 3)), quats=np.zeros((n, 4)), opacity=np.zeros(n),
               flags=np.zeros(n, np.uint8))
    out[cname] = np.zeros((n, ncol))
    sig = C.c_uint64(0)
    gp = [None] * 4
    gw, gb = [], []
    if grads is not None:
        gp = [_c(np.asarray(grads[k], np.float64).reshape(n, -1) if k == cname else grads[k], np.float64)
              for k in ("scales", "quats", cname, "opacity")]
        out["g_tables"] = np.zeros(tables.shape)
        gw = [np.zeros(w.shape) for w in ws]
        gb = [np.zeros(b.shape) for b in bs]
        out["g_pos"] = np.zeros((n, 3))
    gwp = (C.c_void_p * len(ws))(*[w.ctypes.data for w in gw]) if gw else None
    gbp = (C.c_void_p * len(bs))(*[b.ctypes.data for b in gb]) if gb else None
    lib().orc_decode_grad(C.byref(hs), _p(tables), C.byref(mm), wp, bp, _p(xyz), _p(tp), n, int(mode),
                          *[None if g is None else _p(g) for g in gp], _p(out["raw"]), _p(out["scales"]),
                          _p(out["quats"]), _p(out[cname]), _p(out["opacity"]),
                          None if grads is None else _p(out["g_tables"]), gwp, gbp,
                          None if grads is None else _p(out["g_pos"]), _p(out["flags"]), C.byref(sig))
    out["flags"] = out["flags"].astype(bool)
    out["signature"] = int(sig.value)
    if grads is not None:
        out["g_weights"], out["g_biases"] = gw, gb
    return out


def sh_basis(dirs: np.ndarray) -> np.ndarray:
    d = _c(dirs, np.float64)
    Y = np.zeros((d.shape[0], 16))
    lib().orc_sh_basis(_p(d), d.shape[0], _p(Y))
    return Y


# --------------------------------------------------------------------------
# HexPlane
# --------------------------------------------------------------------------


def _hp(hp) -> _HexPlane:
    return _HexPlane(int(hp.res_xyz), int(hp.res_t), int(hp.channels), float(hp.aabb))


def hexplane_features(hp, means: np.ndarray, t: float) -> np.ndarray:
    means = _c(means, np.float32)
    planes = [_c(p, np.float16) for p in hp.planes]
    pp = (C.c_void_p * 6)(*[p.ctypes.data for p in planes])
    feat = np.zeros((means.shape[0], 6 * hp.channels))
    s = _hp(hp)
    lib().orc_hexplane_features(C.byref(s), pp, _p(means), float(t), means.shape[0], _p(feat))
    return feat


def hexplane_deform(hp, g, t: float, mode: int = 0) -> dict:
    n = g.n
    planes = [_c(p, np.float16) for p in hp.planes]
    pp = (C.c_void_p * 6)(*[p.ctypes.data for p in planes])
    dims = [6 * hp.channels, 256, 256, 58]
    mm = _mlp(dims, "relu", True)
    keep = _layers(hp.weights, hp.biases, True)
    means, scales, quats = _c(g.means, np.float32), _c(g.scales, np.float32), _c(g.quats, np.float32)
    sh = _c(g.sh, np.float32)
    om, os_, oq, osh = np.zeros((n, 3)), np.zeros((n, 3)), np.zeros((n, 4)), np.zeros((n, 16, 3))
    s = _hp(hp)
    lib().orc_hexplane_deform(C.byref(s), pp, C.byref(mm), keep[2], keep[3], _p(means), _p(scales),
                              _p(quats), _p(sh), float(t), n, int(mode), _p(om), _p(os_), _p(oq), _p(osh))
    return dict(means=om, scales=os_, quats=oq, sh=osh)


# --------------------------------------------------------------------------
# Render
# --------------------------------------------------------------------------


def cameras(cams) -> C.Array:
    arr = (_Camera * len(cams))()
    for k, c in enumerate(cams):
        arr[k].R[:] = [float(v) for v in np.asarray(c.R, np.float32).ravel()]
        arr[k].t[:] = [float(v) for v in np.asarray(c.t, np.float32).ravel()]
        arr[k].fx, arr[k].fy, arr[k].cx, arr[k].cy = float(c.fx), float(c.fy), float(c.cx), float(c.cy)
        arr[k].near_z = float(c.near)
        arr[k].W, arr[k].H = int(c.W), int(c.H)
        arr[k].bg[:] = [float(v) for v in np.asarray(c.bg, np.float32).ravel()]
    return arr


def preprocess(cams, frame_offsets, means, scales, quats) -> dict:
    fo = _c(frame_offsets, np.int64)
    F = len(cams)
    n = int(fo[-1])
    means, scales, quats = _c(means, np.float32), _c(scales, np.float32), _c(quats, np.float32)
    out = dict(mean2d=np.zeros((n, 2), np.float32), conic=np.zeros((n, 3), np.float32),
               depth=np.zeros(n, np.float32), pix_rect=np.zeros((n, 4), np.int32),
               tile_rect=np.zeros((n, 4), np.int32), tiles=np.zeros(n, np.uint32))
    lib().orc_preprocess(cameras(cams), F, _p(fo), _p(means), _p(scales), _p(quats), _p(out["mean2d"]),
                         _p(out["conic"]), _p(out["depth"]), _p(out["pix_rect"]), _p(out["tile_rect"]),
                         _p(out["tiles"]))
    return out


def sh_colors(cams, frame_offsets, means, sh) -> np.ndarray:
    fo = _c(frame_offsets, np.int64)
    means, sh = _c(means, np.float32), _c(sh, np.float32)
    rgb = np.zeros((means.shape[0], 3))
    lib().orc_sh_colors(cameras(cams), len(cams), _p(fo), _p(means), _p(sh), _p(rgb))
    return rgb


def sh_colors_grad(cams, frame_offsets, means, sh, gcol):
    """Backward of sh_colors for dL/drgb = gcol [N,3]: (dL/dsh [N,16,3],
    dL/dmeans [N,3] through the view direction)."""
    fo = _c(frame_offsets, np.int64)
    means, sh, gcol = _c(means, np.float32), _c(sh, np.float32), _c(gcol, np.float64)
    N = means.shape[0]
    gsh = np.zeros((max(N, 1), 48))
    gm = np.zeros((max(N, 1), 3))
    lib().orc_sh_colors_grad(cameras(cams), len(cams), _p(fo), _p(means), _p(sh), _p(gcol), _p(gsh), _p(gm))
    return gsh[:N].reshape(N, 16, 3), gm[:N]


def bin_and_sort(cams, frame_offsets, pre: dict, cap: int | None = None) -> dict:
    fo = _c(frame_offsets, np.int64)
    F, W, H = len(cams), int(cams[0].W), int(cams[0].H)
    ntiles = ((W + 15) // 16) * ((H + 15) // 16)
    E_total = int(pre["tiles"].astype(np.int64).sum())
    cap = E_total if cap is None else int(cap)
    keys = np.zeros(max(cap, 1), np.uint64)
    vals = np.zeros(max(cap, 1), np.uint32)
    ranges = np.zeros((F * ntiles, 2), np.uint32)
    E = lib().orc_bin(F, W, H, _p(fo), _p(pre["depth"]), _p(pre["tile_rect"]), _p(pre["tiles"]), cap,
                      _p(keys), _p(vals), _p(ranges))
    return dict(E=int(E), keys=keys[:min(E, cap)], vals=vals[:min(E, cap)], ranges=ranges)


def raster_tiles(cams, binned: dict, pre: dict, opacity, colors) -> dict:
    F, W, H = len(cams), int(cams[0].W), int(cams[0].H)
    vals = _c(binned["vals"], np.uint32)
    if vals.size == 0:
        vals = np.zeros(1, np.uint32)
    opacity, colors = _c(opacity, np.float32), _c(colors, np.float64)
    img = np.zeros((F, 3, H, W))
    T = np.zeros((F, H, W))
    nc = np.zeros((F, H, W), np.uint32)
    fl = np.zeros((F, H, W), np.uint8)
    lib().orc_raster_tiles(F, cameras(cams), _p(vals), _p(_c(binned["ranges"], np.uint32)),
                           _p(pre["mean2d"]), _p(pre["conic"]), _p(opacity), _p(colors), _p(img), _p(T),
                           _p(nc), _p(fl))
    return dict(image=img, T=T, n_contrib=nc, flags=fl.astype(bool))


def raster_brute(cam, g0: int, g1: int, pre: dict, opacity, colors, pixels=None,
                 restrict_tiles: bool = True) -> dict:
    """Brute-force composite of one frame (Gaussians [g0, g1)); all pixels, or
    the [n,2] (x, y) list given."""
    opacity, colors = _c(opacity, np.float32), _c(colors, np.float64)
    if pixels is None:
        npx, pix = -1, np.zeros((1, 2), np.int32)
        count = int(cam.W) * int(cam.H)
    else:
        pix = _c(pixels, np.int32)
        npx = count = pix.shape[0]
    rgb = np.zeros((count, 3))
    T = np.zeros(count)
    nc = np.zeros(count, np.uint32)
    fl = np.zeros(count, np.uint8)
    lib().orc_raster_brute(C.byref(cameras([cam])[0]), int(g0), int(g1), _p(pre["mean2d"]), _p(pre["conic"]),
                           _p(opacity), _p(colors), _p(pre["depth"]), _p(pre["tile_rect"]), _p(pre["tiles"]),
                           int(bool(restrict_tiles)), _p(pix), npx, _p(rgb), _p(T), _p(nc), _p(fl))
    return dict(rgb=rgb, T=T, n_contrib=nc, flags=fl.astype(bool))


def render(cams, frame_offsets, means, scales, quats, opacity, colors) -> dict:
    """preprocess -> bin/sort -> tiled raster for a batch of frames."""
    pre = preprocess(cams, frame_offsets, means, scales, quats)
    b = bin_and_sort(cams, frame_offsets, pre)
    r = raster_tiles(cams, b, pre, opacity, colors)
    return dict(pre=pre, bins=b, **r)


def render_grad(cams, frame_offsets, means, scales, quats, opacity, colors, gimg) -> dict:
    """fp64 forward + backward of an image-space gradient gimg = dL/dimage
    [F,3,H,W] (inputs taken as float64): returns image, per-Gaussian gradients (means [N,3], scales
    [N,3], quats [N,4], opacity [N], colors [N,3], proj [N,9] for (u, v, A,
    B, C, o, r, g, b)), flags [N] (near a threshold) and the decision
    signature."""
    fo = _c(frame_offsets, np.int64)
    F = len(cams)
    N = int(fo[-1])
    W, H = int(cams[0].W), int(cams[0].H)
    cam_arr = cameras(cams)
    means, scales, quats = _c(means, np.float64), _c(scales, np.float64), _c(quats, np.float64)
    opacity, colors, gimg = _c(opacity, np.float64), _c(colors, np.float64), _c(gimg, np.float64)
    assert gimg.shape == (F, 3, H, W)
    out = dict(image=np.zeros((F, 3, H, W)), proj=np.zeros((max(N, 1), 9)), means=np.zeros((max(N, 1), 3)),
               scales=np.zeros((max(N, 1), 3)), quats=np.zeros((max(N, 1), 4)), opacity=np.zeros(max(N, 1)),
               colors=np.zeros((max(N, 1), 3)), flags=np.zeros(max(N, 1), np.uint8))
    sig = C.c_uint64(0)
    lib().orc_render_grad(cam_arr, F, _p(fo), _p(means), _p(scales), _p(quats), _p(opacity), _p(colors), _p(gimg),
                          _p(out["image"]), _p(out["proj"]), _p(out["means"]), _p(out["scales"]), _p(out["quats"]),
                          _p(out["opacity"]), _p(out["colors"]), _p(out["flags"]), C.byref(sig))
    for k in ("proj", "means", "scales", "quats", "opacity", "colors", "flags"):
        out[k] = out[k][:N]
    out["flags"] = out["flags"].astype(bool)
    out["signature"] = int(sig.value)
    return out
