"""Seeded synthetic inputs for the decode/render workloads.

This module only draws random numbers and places cameras.  It holds none of
the decode or render arithmetic, so both the HIP path and the CPU oracle can
consume exactly the same inputs.  Everything returned is a plain numpy array
(or a small dataclass of them).

Workloads (sizes follow the sports sequences of the SPIN-4DGS paper,
"Implicit 4D Gaussian Splatting for Fast Motion with Large Inter-Frame
Displacements", §4 "Datasets": 150 frames at 640x360, 27 training views):

* tiny      - 1,000 Gaussians, one t, 4-level fp32 hash, 64x64 image.
* single    - 100k Gaussians per frame, 16-level fp16 hash, 640x360.
* sequence  - 150 frames x 200k Gaussians, 27-camera ring, 640x360.
* hexplane  - 300k canonical Gaussians with degree-3 SH, 1352x1014.
* stress    - 1M Gaussians per frame, 8 frames, 1920x1080.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# --------------------------------------------------------------------------
# Plain parameter containers
# --------------------------------------------------------------------------


@dataclass
class HashConfig:
    L: int
    F: int
    log2T: int
    base_res: float
    growth: float
    temporal_res: int  # 0 = same as the spatial resolution of each level
    table_f16: bool
    t_min: float = 0.0
    t_max: float = 1.0


@dataclass
class MLPConfig:
    dims: list  # [in, hidden..., out]; out = 11 (RGB) or 56 (SH colour), all attributes together
    act: str  # "relu" | "gelu"
    f16: bool
    # False: one trunk and one head block (weights: one matrix per layer);
    # True: one MLP in -> hidden... -> out_a per attribute (scale 3, rotation 4,
    # colour 3 or 48, opacity 1), weights listed branch by branch
    branches: bool = False


@dataclass
class DecoderParams:
    hash: HashConfig
    mlp: MLPConfig
    tables: np.ndarray  # [L, T, F] float16 or float32
    weights: list  # per layer [out, in] float16 or float32
    biases: list  # per layer [out] float32


@dataclass
class Camera:
    R: np.ndarray  # [3,3] world->camera rotation (rows = camera axes)
    t: np.ndarray  # [3] translation, p_cam = R @ p_world + t
    fx: float
    fy: float
    cx: float
    cy: float
    W: int
    H: int
    near: float = 0.2
    bg: np.ndarray = field(default_factory=lambda: np.zeros(3, np.float32))


@dataclass
class Gaussians:
    means: np.ndarray  # [N,3] f32
    scales: np.ndarray  # [N,3] f32 (linear)
    quats: np.ndarray  # [N,4] f32 (w,x,y,z)
    opacity: np.ndarray  # [N] f32
    colors: np.ndarray | None = None  # [N,3] f32
    sh: np.ndarray | None = None  # [N,16,3] f32 (coefficient-major)

    @property
    def n(self) -> int:
        return int(self.means.shape[0])


@dataclass
class HexPlaneParams:
    res_xyz: int  # 64
    res_t: int  # 150
    channels: int  # 32
    planes: list  # 6 x [res_b, res_a, C] float16, order XY XZ YZ XT YT ZT
    weights: list  # [256,192], [256,256], [58,256] float16
    biases: list  # float32
    aabb: float = 3.0


# Opacity-head bias: logit(0.1); rotation-head bias (1,0,0,0) (paper §3.3,
# "Attribute-aware decoder" initialisation paragraphs).
LOGIT_0_1 = math.log(0.1 / 0.9)

# --------------------------------------------------------------------------
# Point sets
# --------------------------------------------------------------------------


def shell_points(rng: np.random.Generator, n: int, radius: float = 3.0) -> np.ndarray:
    v = rng.standard_normal((n, 3))
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    return (v * radius).astype(np.float32)


def ball_offsets(rng: np.random.Generator, n: int, radius: float) -> np.ndarray:
    v = rng.standard_normal((n, 3))
    v /= np.linalg.norm(v, axis=1, keepdims=True)
    r = radius * rng.random(n) ** (1.0 / 3.0)
    return v * r[:, None]


def cluster_centre(j: int, theta_offset: float) -> np.ndarray:
    th = 2.0 * math.pi * j / 3.0 + theta_offset
    return np.array([1.5 * math.cos(th), 0.5 * (j - 1), 1.5 * math.sin(th)])


def random_quats(rng: np.random.Generator, n: int) -> np.ndarray:
    q = rng.standard_normal((n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    return q.astype(np.float32)


# --------------------------------------------------------------------------
# Cameras
# --------------------------------------------------------------------------


def ring_camera(k: int, *, W=640, H=360, fx=500.0, fy=500.0, cx=None, cy=None,
                n_cams=27, radius=4.0) -> Camera:
    """Camera k of a horizontal ring around the origin, looking at the origin.

    OpenCV axes: x right, y down, z forward.  World +y maps to image up.
    """
    a = 2.0 * math.pi * k / n_cams
    C = np.array([radius * math.cos(a), 0.0, radius * math.sin(a)])
    z = -C / np.linalg.norm(C)
    y = np.array([0.0, -1.0, 0.0])
    x = np.cross(y, z)
    R = np.stack([x, y, z]).astype(np.float32)
    t = (-(R.astype(np.float64) @ C)).astype(np.float32)
    return Camera(R=R, t=t, fx=float(fx), fy=float(fy),
                  cx=float(W / 2 if cx is None else cx), cy=float(H / 2 if cy is None else cy),
                  W=int(W), H=int(H))


def origin_camera(W=64, H=64, f=60.0) -> Camera:
    return Camera(R=np.eye(3, dtype=np.float32), t=np.zeros(3, np.float32), fx=f, fy=f,
                  cx=W / 2, cy=H / 2, W=W, H=H)


# --------------------------------------------------------------------------
# Decoder parameters
# --------------------------------------------------------------------------


def _head_bias(scale_bias: float, rows: int = 11) -> np.ndarray:
    """Head-block biases: scale, rotation (w,x,y,z) = (1,0,0,0), colour 0 (RGB
    or SH, no special initialisation), opacity logit(0.1) in the last row."""
    b = np.zeros(rows, np.float32)
    b[0:3] = scale_bias
    b[3] = 1.0
    b[rows - 1] = LOGIT_0_1
    return b


def make_decoder(rng: np.random.Generator, hcfg: HashConfig, mcfg: MLPConfig,
                 scale_bias: float, scale_row_gain: float = 1.0) -> DecoderParams:
    T = 1 << hcfg.log2T
    tdt = np.float16 if hcfg.table_f16 else np.float32
    # U(-1,1) tables: a tiny init would make outputs input-independent.
    tables = rng.uniform(-1.0, 1.0, size=(hcfg.L, T, hcfg.F)).astype(tdt)
    wdt = np.float16 if mcfg.f16 else np.float32
    weights, biases = [], []
    dims = mcfg.dims
    for i in range(len(dims) - 1):
        fan_in, fan_out = dims[i], dims[i + 1]
        w = rng.standard_normal((fan_out, fan_in)) * math.sqrt(1.0 / fan_in)
        b = np.zeros(fan_out, np.float32)
        if i == len(dims) - 2:
            w[0:3] *= scale_row_gain
            b = _head_bias(scale_bias, fan_out)
        weights.append(w.astype(wdt))
        biases.append(b)
    return DecoderParams(hash=hcfg, mlp=mcfg, tables=tables, weights=weights, biases=biases)


BRANCH_OUTS_RGB = (3, 4, 3, 1)
BRANCH_OUTS_SH = (3, 4, 48, 1)


def paper_hash(log2T: int = 21) -> HashConfig:
    """[SPIN] §4 implementation details: 16 levels of 4 features, 2^21 entries
    per level (fp16: 256 MiB; 2^23: 1 GiB); resolutions and time axis as
    single_hash."""
    return HashConfig(L=16, F=4, log2T=log2T, base_res=16, growth=1.5, temporal_res=150, table_f16=True)


def paper_decoder(seed: int = 4, sh: bool = True, log2T: int = 21) -> DecoderParams:
    """Paper-scale decoder: one GELU MLP 64 -> 64 -> 64 -> out per attribute
    ([SPIN] §3.3 Eq. 10, hidden width 64 from §4), reading z of the F = 4
    encoder.  Last-layer biases per §3.3: scale -5, rotation (1,0,0,0),
    opacity logit(0.1), colour 0; the SH rows are scaled by 0.5 as in
    single_decoder_sh."""
    rng = np.random.default_rng([seed, 104])
    h = paper_hash(log2T)
    T = 1 << h.log2T
    tables = np.empty((h.L, T, h.F), np.float16)
    for l in range(h.L):  # level by level (bounded host memory for 2^23)
        tables[l] = rng.uniform(-1.0, 1.0, size=(T, h.F)).astype(np.float16)
    outs = BRANCH_OUTS_SH if sh else BRANCH_OUTS_RGB
    weights, biases = [], []
    for br, out in enumerate(outs):
        for fan_in, fan_out in ((64, 64), (64, 64), (64, out)):
            w = rng.standard_normal((fan_out, fan_in)) * math.sqrt(1.0 / fan_in)
            b = np.zeros(fan_out, np.float32)
            if fan_out == out:
                if br == 0:
                    w *= 2.0
                    b[:] = -5.0
                elif br == 1:
                    b[0] = 1.0
                elif br == 2 and sh:
                    w *= 0.5
                elif br == 3:
                    b[0] = LOGIT_0_1
            weights.append(w.astype(np.float16))
            biases.append(b)
    mcfg = MLPConfig(dims=[64, 64, 64, sum(outs)], act="gelu", f16=True, branches=True)
    return DecoderParams(hash=h, mlp=mcfg, tables=tables, weights=weights, biases=biases)


def tiny_hash() -> HashConfig:
    return HashConfig(L=4, F=2, log2T=12, base_res=8, growth=2.0, temporal_res=0, table_f16=False)


def single_hash() -> HashConfig:
    return HashConfig(L=16, F=2, log2T=19, base_res=16, growth=1.5, temporal_res=150, table_f16=True)


def tiny_decoder(seed: int = 1) -> DecoderParams:
    rng = np.random.default_rng([seed, 101])
    # Scale bias -3 (instead of the paper's -5 init) so that the 64x64 test
    # image has Gaussians a few pixels wide.
    return make_decoder(rng, tiny_hash(), MLPConfig(dims=[8, 32, 11], act="relu", f16=False),
                        scale_bias=-3.0)


def single_decoder_sh(seed: int = 2) -> DecoderParams:
    """The Single decoder with the SH colour head (56 outputs: 48 degree-3
    SH coefficients in place of RGB); the SH rows are scaled by 0.5 so that
    colours stay mostly inside [0, 1]."""
    rng = np.random.default_rng([seed, 103])
    d = make_decoder(rng, single_hash(), MLPConfig(dims=[32, 64, 64, 56], act="gelu", f16=True),
                     scale_bias=0.5 * (math.log(1e-3) + math.log(5e-2)), scale_row_gain=2.0)
    w = d.weights[-1].astype(np.float32)
    w[7:55] *= 0.5
    d.weights[-1] = w.astype(np.float16)
    return d


def single_decoder(seed: int = 2) -> DecoderParams:
    rng = np.random.default_rng([seed, 102])
    # Scale bias = centre of log-uniform [1e-3, 5e-2]; the scale rows get a
    # gain so that the decoded log-scales spread about one unit.
    return make_decoder(rng, single_hash(), MLPConfig(dims=[32, 64, 64, 11], act="gelu", f16=True),
                        scale_bias=0.5 * (math.log(1e-3) + math.log(5e-2)), scale_row_gain=2.0)


# --------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------


def tiny_positions(seed: int = 1) -> np.ndarray:
    rng = np.random.default_rng([seed, 1])
    shell = shell_points(rng, 800, 3.0)
    clus = (np.array([0.0, 0.0, 2.0]) + ball_offsets(rng, 200, 0.2)).astype(np.float32)
    return np.concatenate([shell, clus]).astype(np.float32)


def single_positions(seed: int = 2, t: float | None = None, n_shell=85_000, n_clus=5_000):
    """Positions of one Single frame at time t (drawn U[0,1] when None)."""
    rng = np.random.default_rng([seed, 2])
    if t is None:
        t = float(rng.random())
    shell = shell_points(rng, n_shell, 3.0)
    parts = [shell]
    for j in range(3):
        c = cluster_centre(j, 0.2 * 149.0 * t)
        parts.append((c + ball_offsets(rng, n_clus, 0.2)).astype(np.float32))
    return np.concatenate(parts).astype(np.float32), float(t)


class Sequence:
    """150-frame sequence: fixed shell + 3 rigidly orbiting clusters."""

    def __init__(self, seed: int = 3, frames: int = 150, n_shell: int = 170_000,
                 n_clus: int = 10_000, W=640, H=360, f=500.0, n_cams=27):
        rng = np.random.default_rng([seed, 3])
        self.frames = frames
        self.shell = shell_points(rng, n_shell, 3.0)
        self.offsets = [ball_offsets(rng, n_clus, 0.2) for _ in range(3)]
        self.per_frame = n_shell + 3 * n_clus
        self.W, self.H, self.f, self.n_cams = W, H, f, n_cams

    def t(self, f: int) -> float:
        return f / (self.frames - 1) if self.frames > 1 else 0.0

    def positions(self, f: int) -> np.ndarray:
        parts = [self.shell]
        for j in range(3):
            c = cluster_centre(j, 0.2 * f)  # 0.2 rad x radius 1.5 = 0.3 units per frame
            parts.append((c + self.offsets[j]).astype(np.float32))
        return np.concatenate(parts).astype(np.float32)

    def xyzt(self, frames=None) -> np.ndarray:
        frames = range(self.frames) if frames is None else frames
        out = []
        for f in frames:
            p = self.positions(f)
            out.append(np.concatenate([p, np.full((p.shape[0], 1), self.t(f), np.float32)], 1))
        return np.concatenate(out).astype(np.float32)

    def camera(self, f: int) -> Camera:
        return ring_camera(f % self.n_cams, W=self.W, H=self.H, fx=self.f, fy=self.f,
                           n_cams=self.n_cams)


def render_attributes(rng: np.random.Generator, means: np.ndarray, scale_lo: float, scale_hi: float,
                      with_sh: bool = False) -> Gaussians:
    n = means.shape[0]
    scales = np.exp(rng.uniform(math.log(scale_lo), math.log(scale_hi), size=(n, 3))).astype(np.float32)
    quats = random_quats(rng, n)
    opacity = rng.uniform(0.1, 0.9, size=n).astype(np.float32)
    if with_sh:
        sh = np.empty((n, 16, 3), np.float32)
        sh[:, 0, :] = rng.uniform(-1.0, 1.0, size=(n, 3))
        sh[:, 1:, :] = rng.normal(0.0, 0.2, size=(n, 15, 3))
        return Gaussians(means=means.astype(np.float32), scales=scales, quats=quats, opacity=opacity, sh=sh)
    colors = rng.uniform(0.0, 1.0, size=(n, 3)).astype(np.float32)
    return Gaussians(means=means.astype(np.float32), scales=scales, quats=quats, opacity=opacity, colors=colors)


def single_render_scene(seed: int = 2, n_shell=85_000, n_clus=5_000):
    """Single frame with drawn render attributes (scales log-U[1e-3, 5e-2])."""
    pos, t = single_positions(seed, None, n_shell, n_clus)
    rng = np.random.default_rng([seed, 20])
    return render_attributes(rng, pos, 1e-3, 5e-2), ring_camera(0), t


def hexplane_params(seed: int = 4, res_xyz=64, res_t=150, C=32) -> HexPlaneParams:
    rng = np.random.default_rng([seed, 40])
    planes = []
    for p in range(6):
        rb = res_xyz if p < 3 else res_t
        planes.append(rng.uniform(-0.1, 0.1, size=(rb, res_xyz, C)).astype(np.float16))
    dims = [6 * C, 256, 256, 58]
    weights, biases = [], []
    for i in range(3):
        w = rng.standard_normal((dims[i + 1], dims[i])) * math.sqrt(1.0 / dims[i])
        if i == 2:
            w *= 0.01
        weights.append(w.astype(np.float16))
        biases.append(np.zeros(dims[i + 1], np.float32))
    return HexPlaneParams(res_xyz=res_xyz, res_t=res_t, channels=C, planes=planes,
                          weights=weights, biases=biases)


def hexplane_canonical(seed: int = 4, n_shell=255_000, n_clus=15_000) -> Gaussians:
    rng = np.random.default_rng([seed, 4])
    parts = [shell_points(rng, n_shell, 3.0)]
    for j in range(3):
        parts.append((cluster_centre(j, 0.0) + ball_offsets(rng, n_clus, 0.2)).astype(np.float32))
    means = np.concatenate(parts).astype(np.float32)
    return render_attributes(rng, means, 1e-3, 5e-2, with_sh=True)


def hexplane_camera() -> Camera:
    return ring_camera(0, W=1352, H=1014, fx=1056.25, fy=1056.25, cx=676.0, cy=507.0)


def stress_scene(seed: int = 5, n_per_frame=1_000_000, frames=8, W=1920, H=1080, f=1500.0):
    """Stress batch: per frame a shell + 3 clusters with heavy-overlap attributes."""
    rng = np.random.default_rng([seed, 5])
    n_clus = (n_per_frame * 3) // 20 // 3
    n_shell = n_per_frame - 3 * n_clus
    shell = shell_points(rng, n_shell, 3.0)
    offs = [ball_offsets(rng, n_clus, 0.2) for _ in range(3)]
    means, ts, cams = [], [], []
    for k in range(frames):
        t = k / (frames - 1) if frames > 1 else 0.0
        parts = [shell]
        for j in range(3):
            parts.append((cluster_centre(j, 0.2 * 149.0 * t) + offs[j]).astype(np.float32))
        means.append(np.concatenate(parts))
        ts.append(t)
        cams.append(ring_camera((3 * k) % 27, W=W, H=H, fx=f, fy=f, cx=W / 2, cy=H / 2))
    means = np.concatenate(means).astype(np.float32)
    g = render_attributes(rng, means, 1e-2, 2e-1)
    offsets = np.arange(frames + 1, dtype=np.int64) * n_per_frame
    return g, offsets, cams, ts
