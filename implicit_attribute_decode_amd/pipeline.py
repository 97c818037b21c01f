"""Convenience objects over the C ABI: Decoder, HexPlane, Renderer.

Argument marshalling only (torch tensors in, torch tensors out); the work is
done by libia.so.  Parameter objects are duck-typed like the ones in
scenes.py (DecoderParams, HexPlaneParams, Camera).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import ia


def _dev(a, dtype=None, device="cuda"):
    t = torch.as_tensor(np.ascontiguousarray(a), device=device)
    return t if dtype is None else t.to(dtype)


class _Workspace:
    """A device byte buffer that grows on demand and hands out 256-byte
    aligned views of the requested size (None for zero bytes)."""

    def __init__(self, device):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        if nbytes <= 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes + 256:
            self.buf = None
            self.buf = torch.empty(nbytes + 256, dtype=torch.uint8, device=self.device)
        off = (-self.buf.data_ptr()) % 256
        return self.buf[off:off + nbytes]


class Decoder:
    """Hash encoder + decoder MLP handle (SPIN-4DGS §3.3)."""

    def __init__(self, params, device="cuda"):
        h, m = params.hash, params.mlp
        f16 = bool(m.f16)
        hd = ia.HashDesc(int(h.L), int(h.F), int(h.log2T), float(h.base_res), float(h.growth), int(h.temporal_res),
                         ia.IA_DTYPE_F16 if h.table_f16 else ia.IA_DTYPE_F32, float(h.t_min), float(h.t_max))
        hidden = list(m.dims[1:-1])
        self.sh = int(m.dims[-1]) == 56  # SH colour (48 coefficients)
        branches = bool(getattr(m, "branches", False))
        md = ia.MLPDesc(int(m.dims[0]), len(hidden), (ia.C.c_int32 * 4)(*(hidden + [0] * (4 - len(hidden)))),
                        ia.IA_ACT_GELU if m.act == "gelu" else ia.IA_ACT_RELU,
                        ia.IA_DTYPE_F16 if f16 else ia.IA_DTYPE_F32,
                        ia.IA_COLOR_SH3 if self.sh else ia.IA_COLOR_RGB,
                        ia.IA_BRANCHES_PER_ATTRIBUTE if branches else ia.IA_BRANCHES_SHARED)
        self._destroy = ia.ia_decoder_destroy
        self.handle = ia.ia_decoder_create(hd, md)
        self.device = device
        self._tables = _dev(params.tables, device=device)
        self._W = [_dev(w, device=device) for w in params.weights]
        self._b = [_dev(b, torch.float32, device=device) for b in params.biases]
        ia.ia_decoder_set_params(self.handle, self._tables, self._W, self._b)
        torch.cuda.current_stream().synchronize()
        # this object's scratch (the handle holds only parameters) and a second
        # stream (default priority) for the MLP of one chunk beside the next gather
        self._ws = _Workspace(device)
        self._bwd_ws = _Workspace(device)
        self.side = torch.cuda.Stream(device=device)

    def workspace(self, N: int):
        """Aligned scratch view for a decode of N Gaussians (None if none is needed)."""
        return self._ws.get(ia.ia_decode_workspace_size(self.handle, N))

    def _out(self, N, out):
        if out is None:
            out = dict(scales=torch.empty((N, 3), device=self.device), quats=torch.empty((N, 4), device=self.device),
                       opacity=torch.empty((N,), device=self.device))
            if self.sh:
                out["sh"] = torch.empty((N, 16, 3), device=self.device)
            else:
                out["colors"] = torch.empty((N, 3), device=self.device)
        return out

    def _gaussians(self, out):
        return ia.gaussians(scales=out["scales"], quats=out["quats"], colors=out.get("colors"), sh=out.get("sh"),
                            opacity=out["opacity"], sh_degree=3 if self.sh else -1)

    def decode(self, xyz: torch.Tensor, t: float, out: dict | None = None) -> dict:
        """Decoded attributes: scales, quats, opacity and colors [N,3] (RGB
        head) or sh [N,16,3] (SH head)."""
        N = int(xyz.shape[0])
        out = self._out(N, out)
        ia.ia_decode(self.handle, xyz, N, t, self._gaussians(out), self.workspace(N), self.side)
        return out

    def decode_xyzt(self, xyzt: torch.Tensor, out: dict | None = None) -> dict:
        N = int(xyzt.shape[0])
        out = self._out(N, out)
        ia.ia_decode_xyzt(self.handle, xyzt, N, self._gaussians(out), self.workspace(N), self.side)
        return out

    def decode_keep(self, pos: torch.Tensor, t: float | None = None, out: dict | None = None,
                    features: torch.Tensor | None = None):
        """Decode pos ([N,3] at time t, or [N,4] xyzt) and keep the encoding
        for backward(..., features=...).  Returns (attributes, features)."""
        N, stride = int(pos.shape[0]), int(pos.shape[1])
        out = self._out(N, out)
        nbytes = ia.ia_decode_feature_bytes(self.handle, N)
        if features is None or features.numel() * features.element_size() < nbytes:
            features = torch.empty(max(nbytes, 8) // 8, dtype=torch.int64, device=self.device)
        ia.ia_decode_keep(self.handle, pos, stride, N, float(t or 0.0), self._gaussians(out), features,
                          self.workspace(N), self.side)
        return out, features

    def backward(self, pos: torch.Tensor, grad_attr: dict, t: float | None = None, grad_means=None,
                 want_pos: bool = True, features: torch.Tensor | None = None) -> dict:
        """Gradients of the decode of pos ([N,3] at time t, or [N,4] xyzt)
        for upstream dL/d{scales, quats, colors (RGB) or sh [N,16,3] (SH
        colour), opacity}.  Every fp16 decoder: the shared trunk and the
        per-attribute branches.  Returns tables [L,T,F], weights and biases
        (lists in the order of the parameters, fp32, shaped like them)
        and, with want_pos, pos [N,3] = grad_means + the decoder's share."""
        N = int(pos.shape[0])
        stride = int(pos.shape[1])
        # first: the library says whether this decoder has a backward
        ws = self._bwd_ws.get(ia.ia_decode_backward_workspace_size(self.handle, N))
        out = dict(tables=torch.empty(self._tables.shape, dtype=torch.float32, device=self.device),
                   weights=[torch.empty(w.shape, dtype=torch.float32, device=self.device) for w in self._W],
                   biases=[torch.empty(b.shape, dtype=torch.float32, device=self.device) for b in self._b])
        out["pos"] = torch.empty((N, 3), device=self.device) if want_pos else None
        wp = [ia._ptr(w) for w in out["weights"]] + [None] * (12 - len(out["weights"]))
        bp = [ia._ptr(b) for b in out["biases"]] + [None] * (12 - len(out["biases"]))
        G = ia.DecoderGrads(ia._ptr(out["tables"]), (ia.C.c_void_p * 12)(*wp), (ia.C.c_void_p * 12)(*bp))
        up = ia.gaussians(scales=grad_attr["scales"], quats=grad_attr["quats"], colors=grad_attr.get("colors"),
                          sh=grad_attr.get("sh"), opacity=grad_attr["opacity"])
        ia.ia_decode_backward(self.handle, pos, stride, N, float(t or 0.0), up, grad_means, out["pos"], G, features,
                              ws)
        return out

    def update_params(self):
        """Copy this object's parameter tensors (tables, weights, biases; an
        optimiser updates them in place) into the handle, stream-ordered."""
        ia.ia_decoder_update_params(self.handle, self._tables, self._W, self._b)

    # rows of the shared decoder's head block per attribute (RGB head)
    HEAD_ROWS = {"scale": (0, 3), "rotation": (3, 7), "color": (7, 10), "opacity": (10, 11)}

    def param_groups(self, rates: dict) -> dict:
        """Adam groups of the shared-trunk RGB decoder ([SPIN] §4 implementation
        details: the encoder and each attribute's decoder parameters have their
        own rates).  rates: "encoder", "scale", "rotation", "color", "opacity".
        The hash tables take the encoder rate, the trunk layers (shared by all
        attributes) the largest of the attribute rates, and the head's rows and
        biases of each attribute that attribute's rate.  fp16 tables and
        weights get fp32 master copies with this object's tensors as their fp16
        mirrors; fp32 tensors are updated in place."""
        if self.sh or len(self._W) < 2:
            raise ValueError("parameter groups are defined for the shared-trunk RGB decoder")

        def master(t):
            return (t.float(), t.view(torch.int16)) if t.dtype == torch.float16 else (t, None)

        groups = {}
        p, m = master(self._tables)
        groups["tables"] = {"param": p, "lr": rates["encoder"], "f16": m}
        trunk = max(rates[a] for a in self.HEAD_ROWS)
        for k in range(len(self._W) - 1):
            p, m = master(self._W[k])
            groups[f"w{k}"] = {"param": p, "lr": trunk, "f16": m}
            groups[f"b{k}"] = {"param": self._b[k], "lr": trunk}
        head, m_head = master(self._W[-1])
        for a, (r0, r1) in self.HEAD_ROWS.items():
            groups[f"head_w_{a}"] = {"param": head[r0:r1], "lr": rates[a],
                                     "f16": None if m_head is None else m_head[r0:r1]}
            groups[f"head_b_{a}"] = {"param": self._b[-1][r0:r1], "lr": rates[a]}
        return groups

    def group_grads(self, grads: dict) -> dict:
        """The gradients of backward() keyed like param_groups()."""
        out = {"tables": grads["tables"]}
        for k in range(len(self._W) - 1):
            out[f"w{k}"] = grads["weights"][k]
            out[f"b{k}"] = grads["biases"][k]
        for a, (r0, r1) in self.HEAD_ROWS.items():
            out[f"head_w_{a}"] = grads["weights"][-1][r0:r1]
            out[f"head_b_{a}"] = grads["biases"][-1][r0:r1]
        return out

    def __del__(self):
        # the destroy function is bound at construction: at interpreter exit
        # the module globals may already be gone
        h = getattr(self, "handle", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self.handle = None


class HexPlane:
    """HexPlane deformation handle ("4D Gaussian Splatting详解", §3.1-3.2)."""

    def __init__(self, params, device="cuda"):
        self._destroy = ia.ia_hexplane_destroy
        self.handle = ia.ia_hexplane_create(ia.HexPlaneDesc(int(params.res_xyz), int(params.res_t),
                                                            int(params.channels), float(params.aabb)))
        self.device = device
        self._planes = [_dev(p, device=device) for p in params.planes]
        self._W = [_dev(w, device=device) for w in params.weights]
        self._b = [_dev(b, torch.float32, device=device) for b in params.biases]
        ia.ia_hexplane_set_params(self.handle, self._planes, self._W, self._b)
        torch.cuda.current_stream().synchronize()

    def deform(self, canon: dict, t: float, out: dict | None = None) -> dict:
        N = int(canon["means"].shape[0])
        if out is None:
            out = {k: torch.empty_like(canon[k]) for k in ("means", "scales", "quats", "sh", "opacity")}
        cg = ia.gaussians(means=canon["means"], scales=canon["scales"], quats=canon["quats"], sh=canon["sh"],
                          opacity=canon["opacity"], sh_degree=3)
        og = ia.gaussians(means=out["means"], scales=out["scales"], quats=out["quats"], sh=out["sh"],
                          opacity=out["opacity"], sh_degree=3)
        ia.ia_hexplane_deform(self.handle, cg, N, t, og)
        return out

    def __del__(self):
        # the destroy function is bound at construction: at interpreter exit
        # the module globals may already be gone
        h = getattr(self, "handle", None)
        destroy = getattr(self, "_destroy", None)
        if h is not None and h.value and destroy is not None:
            destroy(h)
            self.handle = None


_VIEW_TYPES = {
    "sorted_keys": (torch.int64, 1), "sorted_vals": (torch.int32, 1), "tile_ranges": (torch.int32, 2),
    "proj_a": (torch.float32, 4), "proj_b": (torch.float32, 4), "proj_c": (torch.float32, 1),
    "depth": (torch.float32, 1), "tiles_touched": (torch.int32, 1), "tile_rect": (torch.int16, 4),
}


class Renderer:
    """Owns a render workspace (a torch uint8 tensor) and calls ia_render."""

    def __init__(self, device="cuda"):
        self.device = device
        self._ws = _Workspace(device)
        self._loss_ws = _Workspace(device)

    def workspace(self, N, frames, W, H, max_entries):
        """Aligned view of this object's render workspace for these sizes."""
        return self._ws.get(ia.ia_render_workspace_size(N, frames, W, H, max_entries))

    def render(self, g: dict, frame_offsets, cams, max_entries: int, aux: bool = False, out: dict | None = None,
               keys: bool = True, binning: int = ia.BINNING_AUTO):
        """g: means [N,k>=3], scales, quats, colors | sh, opacity (cuda tensors).
        Returns image [F,3,H,W] and, with aux, T_final, n_contrib, n_entries,
        overflow and workspace views (ranges, projections and, with keys, the
        sorted keys / values).  binning: ia.BINNING_AUTO, _TILE_SORT or
        _REGIONS (the same lists either way)."""
        fo = np.asarray(frame_offsets, np.int64)
        F, W, H = len(cams), int(cams[0].W), int(cams[0].H)
        N = int(fo[-1])
        ws = self.workspace(N, F, W, H, max_entries)
        out = out or {}
        image = out.get("image")
        if image is None:
            image = torch.empty((F, 3, H, W), device=self.device)
        means = g["means"]
        stride = int(means.stride(0)) if means.dim() == 2 else 3
        sh = g.get("sh")
        G = ia.gaussians(means=means, scales=g["scales"], quats=g["quats"], colors=g.get("colors"), sh=sh,
                         opacity=g["opacity"], means_stride=stride, sh_degree=3 if sh is not None else -1)
        res = {"image": image}
        A = None
        if not aux and binning != ia.BINNING_AUTO:
            A = ia.RenderAux()
            A.binning = int(binning)
        if aux:
            res["T_final"] = torch.empty((F, H, W), device=self.device)
            res["n_contrib"] = torch.empty((F, H, W), dtype=torch.int32, device=self.device)
            res["n_entries"] = torch.zeros(1, dtype=torch.int64, device=self.device)
            res["overflow"] = torch.zeros(1, dtype=torch.int32, device=self.device)
            A = ia.RenderAux(ia._ptr(res["T_final"]), ia._ptr(res["n_contrib"]), ia._ptr(res["n_entries"]),
                             ia._ptr(res["overflow"]))
            A.want_keys = 1 if keys else 0
            A.binning = int(binning)
        ia.ia_render(G, fo, cams, ws, max_entries, image, A)
        if aux:
            base = ws.data_ptr()
            for name, (dt, width) in _VIEW_TYPES.items():
                p = getattr(A, name)
                if p:  # sorted keys / values only when requested
                    res["_view_" + name] = (int(p) - base, dt, width)
            res["_ws"] = ws
        return res

    def backward(self, g: dict, frame_offsets, cams, max_entries: int, res: dict, grad_image):
        """Gradients of the render `res` (made by render(..., aux=True) with
        the same g, frame_offsets, cams, max_entries and this workspace) for
        dL/dimage = grad_image.  Returns dict means, scales, quats, opacity,
        colors and, for SH colours, sh [N,16,3] (cuda float32, packed rows;
        the means include the view direction's share)."""
        fo = np.asarray(frame_offsets, np.int64)
        N = int(fo[-1])
        F, W, H = len(cams), int(cams[0].W), int(cams[0].H)
        ws = self.workspace(N, F, W, H, max_entries)
        means = g["means"]
        stride = int(means.stride(0)) if means.dim() == 2 else 3
        G = ia.gaussians(means=means, scales=g["scales"], quats=g["quats"], colors=g.get("colors"), sh=g.get("sh"),
                         opacity=g["opacity"], means_stride=stride, sh_degree=3 if g.get("sh") is not None else -1)
        out = {k: torch.empty(shape, device=self.device)
               for k, shape in (("means", (N, 3)), ("scales", (N, 3)), ("quats", (N, 4)), ("opacity", (N,)),
                                ("colors", (N, 3)))}
        if g.get("sh") is not None:
            out["sh"] = torch.empty((N, 16, 3), device=self.device)
        GG = ia.GaussianGrads(*[ia._ptr(out.get(k)) for k in ("means", "scales", "quats", "opacity", "colors", "sh")])
        ia.ia_render_backward(G, fo, cams, ws, max_entries, grad_image.contiguous(), res["T_final"],
                              res["n_contrib"], GG)
        return out

    @staticmethod
    def l1_loss(image, target):
        """(loss [1] float64 on the device, dL/dimage)."""
        loss = torch.empty(1, dtype=torch.float64, device=image.device)
        grad = torch.empty_like(image)
        ia.ia_l1_loss(image.contiguous(), target.contiguous(), loss, grad)
        return loss, grad

    def image_loss(self, image, target, lam: float = 0.2):
        """Eq. 12 loss of image against target ([F, 3, H, W] device float):
        (loss [3] float64 on the device = {L, L1, SSIM}, dL/dimage)."""
        F, _, H, W = (int(d) for d in image.shape)
        ws = self._loss_ws.get(ia.ia_image_loss_workspace_size(F, H, W))  # 256-byte aligned
        loss = torch.empty(3, dtype=torch.float64, device=image.device)
        grad = torch.empty_like(image)
        ia.ia_image_loss(image.contiguous(), target.contiguous(), lam, ws, loss, grad)
        return loss, grad

    @staticmethod
    def count_entries(res: dict) -> int:
        return int(res["n_entries"].item())

    @staticmethod
    def view(res: dict, name: str, count: int) -> torch.Tensor:
        """A workspace view of `count` rows (e.g. sorted_keys of n_entries rows)."""
        off, dt, width = res["_view_" + name]
        ws = res["_ws"]
        nbytes = count * width * torch.empty((), dtype=dt).element_size()
        t = ws[off:off + nbytes].view(dt)
        return t.view(count, width) if width > 1 else t



def spatial_order(pos: torch.Tensor, frame_offsets):
    """(perm, reordered positions): every frame's Gaussians along a Morton
    curve of their normalised positions (ia_spatial_order); a one-time
    storage layout for fixed per-frame position sets."""
    fo = np.asarray(frame_offsets, np.int64)
    pos = pos.contiguous()
    N = int(pos.shape[0])
    perm = torch.empty(N, dtype=torch.int32, device=pos.device)
    out = torch.empty_like(pos)
    ws = _Workspace(pos.device).get(ia.ia_spatial_order_workspace_size(N, len(fo) - 1))
    ia.ia_spatial_order(pos, fo, perm, out, ws)
    return perm, out


def lr_at(step: int, base: float, warmup: int, total: int, final: float = 1e-7) -> float:
    """Learning rate at `step` (0-based): linear warm-up over `warmup` steps,
    then cosine decay from base to `final` at `total` ([SPIN] §4
    implementation details); evaluated by ia_lr_at."""
    return ia.ia_lr_at(base, step, warmup, total, final)


class Adam:
    """Adam over named parameter groups, each an fp32 device tensor with its
    own base learning rate ([SPIN] §4 implementation details: per-group rates,
    linear warm-up then cosine decay to 1e-7).  A group may carry an fp16
    mirror (e.g. the decoder's hash table) that every step refreshes, and its
    parameter may be a [rows, dim] view with rows further apart than dim (the
    x, y, z of xyzt positions).  Every update runs in ia_adam_step or
    ia_adam_step_strided."""

    def __init__(self, groups: dict, warmup: int, total: int, beta1: float = 0.9, beta2: float = 0.999,
                 eps: float = 1e-15):
        self.groups = groups  # name -> {"param": fp32 tensor, "lr": base, optional "f16": tensor}
        self.state = {k: (torch.zeros(g["param"].shape, device=g["param"].device),
                          torch.zeros(g["param"].shape, device=g["param"].device)) for k, g in groups.items()}
        self.warmup, self.total = warmup, total
        self.beta1, self.beta2, self.eps = beta1, beta2, eps
        self.t = 0

    def step(self, grads: dict):
        """One update of every group that has a gradient in `grads` (name -> tensor)."""
        self.t += 1
        for name, g in self.groups.items():
            grad = grads.get(name)
            if grad is None:
                continue
            m, v = self.state[name]
            lr = lr_at(self.t - 1, g["lr"], self.warmup, self.total)
            p = g["param"]
            if p.is_contiguous():
                ia.ia_adam_step(p, grad.contiguous(), m, v, lr, self.beta1, self.beta2, self.eps, self.t, g.get("f16"))
            else:
                if g.get("f16") is not None:
                    raise ValueError(f"group {name}: an fp16 mirror needs a contiguous parameter")
                ia.ia_adam_step_strided(p, grad.contiguous(), m, v, lr, self.beta1, self.beta2, self.eps, self.t)


def densify_positions(xyzt, grad_acc, grad_count, attrs: dict, m, v, noise, grad_threshold: float,
                      scale_threshold: float, min_opacity: float):
    """Refine the positions ([SPIN] §3.2 Eq. 6; clone / split / prune, see
    ia_densify) from the decoded attributes `attrs` (scales, quats, opacity).
    Returns (xyzt', m', v') of the rows written; reading their count is the
    one host synchronisation."""
    N = int(xyzt.shape[0])
    dev = xyzt.device
    out_x = torch.empty((2 * N, 4), device=dev)
    out_m = torch.empty((2 * N, 3), device=dev)
    out_v = torch.empty((2 * N, 3), device=dev)
    out_n = torch.zeros(1, dtype=torch.int64, device=dev)
    ws = torch.empty(max(ia.ia_densify_workspace_size(N), 256), dtype=torch.uint8, device=dev)
    p = ia.DensifyParams(grad_threshold, scale_threshold, min_opacity)
    ia.ia_densify(xyzt.contiguous(), grad_acc, grad_count, attrs["scales"], attrs["quats"], attrs["opacity"],
                  noise.contiguous(), m.contiguous(), v.contiguous(), p, out_x, out_m, out_v, out_n, ws)
    n = int(out_n.item())
    return out_x[:n], out_m[:n], out_v[:n]


class PipelinedDecodeRender:
    """Decode + render of a batch of frames whose Gaussians are stored frame
    after frame, in `parts` consecutive groups of frames: the render of group k
    runs on a second stream (default priority) beside the decode of group
    k + 1.  The decode's gather is bound by L2 requests and the raster by VALU
    issue, so the two share the chip well.  Every group has its own render
    workspace; images and decoded attributes land in the caller's tensors.
    Results equal one decode and one render of the whole batch, bit for bit
    when every group starts at a multiple of 64 Gaussians (a decoded value's
    MFMA rounding depends on its index mod 64 within a decode call), else to
    the decoder's tolerance."""

    def __init__(self, decoder: Decoder, xyzt: torch.Tensor, frame_offsets, cams, attrs: dict,
                 image: torch.Tensor, parts: int):
        fo = np.asarray(frame_offsets, np.int64)
        F = len(cams)
        if not 1 <= parts <= F:
            raise ValueError("parts must be in 1..frames")
        self.decoder, self.xyzt = decoder, xyzt
        self.side = torch.cuda.Stream(device=xyzt.device)
        bounds = [(F * k) // parts for k in range(parts + 1)]
        self.groups = []
        for k in range(parts):
            f0, f1 = bounds[k], bounds[k + 1]
            lo, hi = int(fo[f0]), int(fo[f1])
            out = {n: v[lo:hi] for n, v in attrs.items()}
            self.groups.append(dict(lo=lo, hi=hi, fo=fo[f0:f1 + 1] - lo, cams=list(cams[f0:f1]), out=out,
                                    g=dict(means=xyzt[lo:hi, :3], **out), R=Renderer(str(xyzt.device)),
                                    image=image[f0:f1], cap=None))

    def probe(self, slack: float = 1.02) -> int:
        """Decode and render once, counting each group's tile entries (host
        synchronisation); sets the capacities.  Returns the total count."""
        total = 0
        for grp in self.groups:
            self.decoder.decode_xyzt(self.xyzt[grp["lo"]:grp["hi"]], out=grp["out"])
            n = grp["hi"] - grp["lo"]
            res = grp["R"].render(grp["g"], grp["fo"], grp["cams"], 4 * max(n, 1), aux=True,
                                  out={"image": grp["image"]})
            e = Renderer.count_entries(res)
            grp["cap"] = int(e * slack) + 4096
            total += e
        return total

    def __call__(self):
        if any(grp["cap"] is None for grp in self.groups):
            raise RuntimeError("call probe() first")
        main = torch.cuda.current_stream(self.xyzt.device)
        if len(self.groups) == 1:  # nothing to overlap: one decode, one render, one stream
            grp = self.groups[0]
            self.decoder.decode_xyzt(self.xyzt[grp["lo"]:grp["hi"]], out=grp["out"])
            grp["R"].render(grp["g"], grp["fo"], grp["cams"], grp["cap"], out={"image": grp["image"]})
            return
        for grp in self.groups:
            self.decoder.decode_xyzt(self.xyzt[grp["lo"]:grp["hi"]], out=grp["out"])
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                grp["R"].render(grp["g"], grp["fo"], grp["cams"], grp["cap"], out={"image": grp["image"]})
        main.wait_stream(self.side)


class FrameGraphs:
    """Per-frame decode + render replayed from HIP graphs (SPIN-4DGS page §4:
    every frame is decoded from its own position set at its own time and
    rendered on its own).

    Frame f's graph holds its ia_decode_xyzt call (normalisation, hash gather,
    decoder MLP) and its ia_render call (projection, depth sort, key emission,
    tile sort, ranges, raster; the camera and frame offsets travel as kernel
    arguments of upload kernels, clears are fill kernels: no memset or memcpy
    node).  A replay submits the frame's ~45 kernels in one call instead of
    one launch each.  The graphs keep the addresses they were captured with:
    positions, attribute and image buffers, and the decoder's and renderer's
    workspaces must stay allocated and in place while they are used, and the
    decoder's parameters may be updated in place (set_params) but not
    reallocated.

    xyzt: [N, 4] device positions of all frames, frame f at
    frame_offsets[f]:frame_offsets[f+1]; attrs: decoder output buffers [N, ...];
    image: [F, 3, H, W]; max_entries: the tile-entry capacity of one frame."""

    def __init__(self, decoder: "Decoder", renderer: "Renderer", xyzt: torch.Tensor, frame_offsets, cams,
                 max_entries: int, attrs: dict, image: torch.Tensor):
        self.D, self.R = decoder, renderer
        self.xyzt, self.cams, self.cap = xyzt, list(cams), int(max_entries)
        self.fo = np.asarray(frame_offsets, np.int64)
        self.attrs, self.image = attrs, image
        F = len(self.cams)
        # one eager pass: sizes both workspaces (no allocation happens while
        # capturing) and fills the one-time caches of the launch code
        for f in range(F):
            self.frame(f)
        torch.cuda.synchronize()
        self.graphs = []
        pool = None
        for f in range(F):
            g = torch.cuda.CUDAGraph(keep_graph=True)
            with torch.cuda.graph(g, pool=pool):
                self.frame(f)
            g.instantiate()
            pool = g.pool()
            self.graphs.append(g)
        torch.cuda.synchronize()

    def frame(self, f: int):
        """Frame f eagerly: one decode and one single-frame render."""
        lo, hi = int(self.fo[f]), int(self.fo[f + 1])
        x = self.xyzt[lo:hi]
        a = self.D.decode_xyzt(x, out={k: v[lo:hi] for k, v in self.attrs.items()})
        self.R.render(dict(means=x[:, :3], **a), [0, hi - lo], [self.cams[f]], self.cap,
                      out={"image": self.image[f:f + 1]})

    def replay(self, frames=None):
        """Replay the graphs of `frames` (default: all) in order on the current stream."""
        for f in (range(len(self.graphs)) if frames is None else frames):
            self.graphs[f].replay()
