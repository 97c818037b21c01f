"""Benchmark: decode + render of the 150-frame sports-like sequence.

Workload (one "step"): 150 frames x 200k Gaussians = 30M (x, y, z, t)
positions, already resident in HBM: one ia_decode_xyzt call decodes all of
them (16-level 4D hash grid, fp16 MFMA 32-64-64-11 decoder), then one
ia_render call renders the 150 frames at 640x360 from a 27-camera ring
(projection, binning, radix sort, tile raster), both on one stream.  The
level-major hash gather needs the L2 to itself, so decode and render are not
overlapped across streams.  Prints one JSON line.

Also reported: the per-frame mode (150 separate decode + render calls, issued
one by one and replayed from one HIP graph per frame), the
roofline of the dominant kernel (the level-major hash gather) from HIP events
recorded around its launches, and the CPU oracle's rate on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
LEVELS, CORNERS, FEAT_BYTES = 16, 16, 4  # fp16 x 2 features per table entry
# Algorithmic bytes of the hash gather per Gaussian: the 16-byte (x,y,z,t)
# position and 16 levels x 16 corners x 4-byte entries = 1040 B.  Scratch
# traffic of this implementation (the normalised position re-read per level,
# the packed features written) is not counted.
GATHER_BYTES_PER_GAUSSIAN = 16 + LEVELS * CORNERS * FEAT_BYTES
# Whole decode per Gaussian: 16 B position in, 1024 B gathered, 44 B out.
DECODE_BYTES_PER_GAUSSIAN = 16 + LEVELS * CORNERS * FEAT_BYTES + 44
# HBM-side bytes per gather launch of this workload (positions in per-frame Morton order), from two
# rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch, each scaled by what the counter
# reads for a plain device copy of known size).  Per Gaussian the gather's FETCH_SIZE counts 152.49 B and
# its WRITE_SIZE 64.0 B; a 1 GiB copy counts 524,314 KiB of FETCH_SIZE for the 1 GiB it reads (x 2) and
# 1,048,576 KiB of WRITE_SIZE for the 1 GiB it writes (x 1): 2 x 152.49 + 64.0 B per Gaussian, times the
# 3.75M Gaussians of a mean launch.
GATHER_TRAFFIC_BYTES_PER_LAUNCH = (2 * 152.49 + 64.0) * 3_750_000


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(seq, dec, frame: int = 1, one_core_decode: int = 20_000) -> dict:
    """The oracle (plain C, OpenMP, fp64 decode) on the same workload, stage by
    stage, on this host: one whole frame of the sequence (200k Gaussians,
    640x360), median of 5 on all cores; on one core the median of 3, with the
    decode timed on the frame's first `one_core_decode` Gaussians and scaled
    to the frame (it is linear in N).  Value: frames/s on all cores."""
    import oracle as O

    x = seq.xyzt([frame])
    cam = seq.camera(frame)
    fo = np.array([0, x.shape[0]])

    def run(xs, reps, stages=("decode", "preprocess", "bin_sort", "raster"), attrs=None):
        t = {k: [] for k in stages}
        for _ in range(reps):
            t0 = time.perf_counter()
            d = O.decode(dec, xs, mode=0) if "decode" in stages else attrs
            t1 = time.perf_counter()
            if "decode" in stages:
                t["decode"].append(t1 - t0)
            if "preprocess" in stages:
                f = np.array([0, xs.shape[0]])
                pre = O.preprocess([cam], f, xs[:, :3], d["scales"].astype(np.float32),
                                   d["quats"].astype(np.float32))
                t2 = time.perf_counter()
                b = O.bin_and_sort([cam], f, pre)
                t3 = time.perf_counter()
                O.raster_tiles([cam], b, pre, d["opacity"].astype(np.float32), d["colors"])
                t4 = time.perf_counter()
                t["preprocess"].append(t2 - t1)
                t["bin_sort"].append(t3 - t2)
                t["raster"].append(t4 - t3)
        return {k: float(np.median(v)) for k, v in t.items()}, d

    cores = O.num_threads()
    run(x[:2000], 1)  # warm-up (page-in, thread pool)
    all_med, attrs = run(x, 5)
    O.set_num_threads(1)
    try:
        one_dec, _ = run(x[:one_core_decode], 3, stages=("decode",))
        one_rest, _ = run(x, 3, stages=("preprocess", "bin_sort", "raster"), attrs=attrs)
    finally:
        O.set_num_threads(cores)
    one_med = {"decode": one_dec["decode"] * x.shape[0] / one_core_decode, **one_rest}
    all_s, one_s = sum(all_med.values()), sum(one_med.values())
    return {"value": round(1.0 / all_s, 4), "unit": "frames/s", "cores": cores, "kind": "oracle",
            "sample": f"frame {frame} of the 150-frame sequence (200k Gaussians, 640x360): decode (fp64) + "
                      f"preprocess + bin/sort + raster, median of 5 per stage on {cores} cores; one core: "
                      f"median of 3, decode timed on {one_core_decode} Gaussians and scaled to the frame",
            "per_stage_ms": {"all_cores": {k: round(1e3 * v, 2) for k, v in all_med.items()},
                             "one_core": {k: round(1e3 * v, 2) for k, v in one_med.items()}},
            "one_core_value": round(1.0 / one_s, 4)}


HEX_FLOP_PER_GAUSSIAN = 2 * (192 * 256 + 256 * 256 + 256 * 58)  # 259,072
# paper-scale decoder: four 64 -> 64 -> 64 -> out branches, outs 3 + 4 + 48 + 1
PAPER_FLOP_PER_GAUSSIAN = 2 * (4 * (64 * 64 + 64 * 64) + 64 * 56)  # 72,704
MFMA_F16_PEAK_TFLOPS = 2500.0
MLP_FLOP_PER_GAUSSIAN = 2 * (32 * 64 + 64 * 64 + 64 * 11)  # 13,696: the 32-64-64-11 decoder


def secondary(S, Decoder, HexPlane, Renderer, stream, log, only: str | None = None,
              stored_order: bool = False) -> dict:
    """The other workloads of the hot-path table, each timed with HIP events:
    one Single frame, the HexPlane deform + SH render, the Stress batch
    (only: just that one)."""
    import torch

    out = {}
    R = Renderer()
    if only in (None, "single"):
        out["single_frame"] = _single(S, Decoder, R, stream)
    if only in (None, "hexplane"):
        out["hexplane"] = _hexplane(S, HexPlane, R, stream, stored_order)
    if only in (None, "paper"):
        out["paper_scale"] = _paper(S, Decoder, R, stream)
    if only in (None, "stress"):
        out["stress"] = _stress(S, Decoder, Renderer, stream)
    log(f"secondary: {out}")
    return out


def _single(S, Decoder, R, stream) -> dict:
    """Single: one frame, 100k Gaussians, decode + render (RGB head, then the SH colour head)."""
    import torch

    dec = S.single_decoder()
    pos, t = S.single_positions(2)
    x = torch.as_tensor(pos, device="cuda")
    D = Decoder(dec)
    a = D.decode(x, t)
    cam = S.ring_camera(0)
    res = R.render(dict(means=x, **a), [0, x.shape[0]], [cam], 8 * x.shape[0], aux=True)
    cap = R.count_entries(res) + 4096
    ms = timed(lambda: (D.decode(x, t, out=a), R.render(dict(means=x, **a), [0, x.shape[0]], [cam], cap)), 20, stream)
    # the same frame with the SH colour decoder (48 coefficients) and the degree-3 SH render
    Dsh = Decoder(S.single_decoder_sh())
    ash = Dsh.decode(x, t)
    res = R.render(dict(means=x, **ash), [0, x.shape[0]], [cam], 8 * x.shape[0], aux=True)
    cap_sh = R.count_entries(res) + 4096
    ms_sh = timed(lambda: (Dsh.decode(x, t, out=ash), R.render(dict(means=x, **ash), [0, x.shape[0]], [cam], cap_sh)),
                  20, stream)
    return {"gaussians": int(x.shape[0]), "ms": round(ms, 4), "fps": round(1e3 / ms, 1),
            "sh_head_ms": round(ms_sh, 4), "sh_head_fps": round(1e3 / ms_sh, 1)}


def _paper(S, Decoder, R, stream) -> dict:
    """Paper-scale decoder (F = 4, 2^21-entry tables, one GELU MLP per
    attribute, SH colour): one Single frame decoded and rendered with SH, the
    decoder backward of that frame, and the decode alone of 20 sequence
    frames (4M (x,y,z,t) positions), also with 2^23-entry tables."""
    import torch

    D = Decoder(S.paper_decoder())
    pos, t = S.single_positions(2)
    x = torch.as_tensor(pos, device="cuda")
    a = D.decode(x, t)
    cam = S.ring_camera(0)
    res = R.render(dict(means=x, **a), [0, x.shape[0]], [cam], 8 * x.shape[0], aux=True)
    cap = R.count_entries(res) + 4096
    ms = timed(lambda: (D.decode(x, t, out=a), R.render(dict(means=x, **a), [0, x.shape[0]], [cam], cap)), 20, stream)
    # the decoder backward of the frame from the kept encoding, every Gaussian
    # with a seeded N(0, 1) upstream gradient on all 56 outputs
    g = torch.Generator(device="cuda").manual_seed(9)
    nf = int(x.shape[0])
    up = {k: torch.randn(shape, generator=g, device="cuda") for k, shape in
          (("scales", (nf, 3)), ("quats", (nf, 4)), ("sh", (nf, 48)), ("opacity", (nf,)))}
    _, feats = D.decode_keep(x, t)
    D.backward(x, up, t, features=feats)
    ms_b = timed(lambda: D.backward(x, up, t, features=feats), 5, stream)
    kern_b = profiled(lambda: D.backward(x, up, t, features=feats), 1)
    del feats
    seq = S.Sequence()
    xyzt = torch.as_tensor(seq.xyzt(list(range(20))), device="cuda")
    d = D.decode_xyzt(xyzt)
    ms_d = timed(lambda: D.decode_xyzt(xyzt, out=d), 5, stream)
    kern = profiled(lambda: D.decode_xyzt(xyzt, out=d), 1)
    n = int(xyzt.shape[0])
    del D
    # the 2^23-entry tables (1 GiB of fp16)
    D23 = Decoder(S.paper_decoder(log2T=23))
    d23 = D23.decode_xyzt(xyzt)
    ms_23 = timed(lambda: D23.decode_xyzt(xyzt, out=d23), 5, stream)
    kern23 = profiled(lambda: D23.decode_xyzt(xyzt, out=d23), 1)
    return {"single_frame_ms": round(ms, 4), "single_frame_fps": round(1e3 / ms, 1), "decode_gaussians": n,
            "decode_ms": round(ms_d, 4), "decode_gaussians_per_s": round(n / (ms_d / 1e3)), "decode_kernels_ms": kern,
            "decode_2p23_ms": round(ms_23, 4), "decode_2p23_kernels_ms": kern23,
            "mlp_flop_per_gaussian": PAPER_FLOP_PER_GAUSSIAN,
            "decode_backward_frame_ms": round(ms_b, 4), "decode_backward_frame_kernels_ms": kern_b}


def _hexplane(S, HexPlane, R, stream, stored_order: bool = False) -> dict:
    """HexPlane: 300k canonical Gaussians, deform at t = 0.5, SH render at 1352x1014.

    The canonical set is fixed model data; by default it is stored along a
    Morton curve of the positions once (ia_spatial_order, not part of a step),
    so that Gaussians of one wave share plane texels.  The deform of the stored
    order is timed beside it."""
    import torch

    from implicit_attribute_decode_amd.pipeline import spatial_order

    hp = S.hexplane_params()
    cg = S.hexplane_canonical()
    canon = {k: torch.as_tensor(getattr(cg, k), device="cuda") for k in ("means", "scales", "quats", "sh", "opacity")}
    H = HexPlane(hp)
    d = H.deform(canon, 0.5)
    ms_stored = timed(lambda: H.deform(canon, 0.5, out=d), 10, stream)
    order = "stored"
    if not stored_order:
        perm, _ = spatial_order(canon["means"], np.array([0, cg.n], np.int64))
        perm = perm.long()
        canon = {k: v[perm].contiguous() for k, v in canon.items()}
        order = "Morton (ia_spatial_order, once)"
    hcam = S.hexplane_camera()
    res = R.render(d, [0, cg.n], [hcam], 8 * cg.n, aux=True)
    hcap = R.count_entries(res) + 4096
    ms_def = timed(lambda: H.deform(canon, 0.5, out=d), 10, stream)
    hex_kernels = profiled(lambda: H.deform(canon, 0.5, out=d), 3)
    ms_ren = timed(lambda: R.render(d, [0, cg.n], [hcam], hcap), 10, stream)
    # render backward with the SH colours (dL/dsh and the view direction's
    # share of dL/dmean) for a seeded N(0, 1) image gradient
    ra = R.render(d, [0, cg.n], [hcam], hcap, aux=True)
    gimg = torch.randn(ra["image"].shape, generator=torch.Generator(device="cuda").manual_seed(3), device="cuda")
    R.backward(d, [0, cg.n], [hcam], hcap, ra, gimg)
    ms_bwd = timed(lambda: R.backward(d, [0, cg.n], [hcam], hcap, ra, gimg), 5, stream)
    tflops = HEX_FLOP_PER_GAUSSIAN * cg.n / (ms_def / 1e3) / 1e12
    return {"gaussians": cg.n, "order": order, "deform_ms": round(ms_def, 4),
            "deform_stored_order_ms": round(ms_stored, 4), "render_ms": round(ms_ren, 4),
            "render_backward_sh_ms": round(ms_bwd, 4),
            "fps": round(1e3 / (ms_def + ms_ren), 1), "mlp_tflops": round(tflops, 1),
            "mlp_frac_of_fp16_mfma_peak": round(tflops / MFMA_F16_PEAK_TFLOPS, 4), "deform_kernels_ms": hex_kernels}


def _stress(S, Decoder, Renderer, stream) -> dict:
    """Stress: 8 frames x 1M at 1920x1080 (drawn attributes) + decode of the same 8M positions."""
    import torch

    g, fo, cams, ts = S.stress_scene()
    attrs = {k: torch.as_tensor(getattr(g, k), device="cuda") for k in ("means", "scales", "quats", "colors",
                                                                         "opacity")}
    Rs = Renderer()
    res = Rs.render(attrs, fo, cams, 4 * g.n, aux=True)
    E = Renderer.count_entries(res)
    del res
    res = Rs.render(attrs, fo, cams, E + 4096)
    ms_r = timed(lambda: Rs.render(attrs, fo, cams, E + 4096, out=res), 2, stream)
    stress_kernels = profiled(lambda: Rs.render(attrs, fo, cams, E + 4096, out=res), 1)
    xyzt = torch.cat([attrs["means"], torch.as_tensor(np.repeat(np.float32(ts), g.n // len(ts)),
                                                      device="cuda")[:, None]], 1).contiguous()
    D = Decoder(S.single_decoder())
    da = D.decode_xyzt(xyzt)
    ms_d = timed(lambda: D.decode_xyzt(xyzt, out=da), 3, stream)
    # the training step keeps the encoding of the forward decode for the decoder backward
    dk, feats = D.decode_keep(xyzt)
    ms_dk = timed(lambda: D.decode_keep(xyzt, out=dk, features=feats), 3, stream)
    # backward: L1 loss against a seeded U(0,1) target image, render backward
    # (per-Gaussian gradients), decode backward of the same 8M positions fed
    # with those attribute gradients (per-weight, per-table-entry and position
    # gradients)
    gen = torch.Generator(device="cuda").manual_seed(7)
    ra = Rs.render(attrs, fo, cams, E + 4096, aux=True, keys=False)
    target = torch.rand(ra["image"].shape, generator=gen, device="cuda")

    def render_train():
        r = Rs.render(attrs, fo, cams, E + 4096, aux=True, keys=False, out=ra)
        loss, gimg = Renderer.l1_loss(r["image"], target)
        return Rs.backward(attrs, fo, cams, E + 4096, r, gimg)

    ga = render_train()
    ms_rt = timed(render_train, 2, stream)
    bwd_kernels = profiled(render_train, 1)
    ms_db = timed(lambda: D.backward(xyzt, ga, grad_means=ga["means"], features=feats), 2, stream)
    dbwd_kernels = profiled(lambda: D.backward(xyzt, ga, grad_means=ga["means"], features=feats), 1)
    # the same decoder backward with a non-zero gradient on every Gaussian (the L1 step above
    # leaves most of the 8M without one): every corner of every level is a float atomic
    dense = {k: torch.randn(v.shape, generator=gen, device="cuda") * 1e-6 for k, v in dk.items()}
    D.backward(xyzt, dense, features=feats)
    ms_dense = timed(lambda: D.backward(xyzt, dense, features=feats), 1, stream)
    nz = int((ga["opacity"] != 0).sum().item())
    full = _train_full(S, Decoder, Renderer, stream, xyzt, fo, cams, target)
    return {"frames": len(cams), "gaussians": g.n, "tile_entries": E, "render_ms": round(ms_r, 3),
            "render_fps": round(len(cams) / (ms_r / 1e3), 2), "decode_8M_ms": round(ms_d, 3),
            "decode_keep_8M_ms": round(ms_dk, 3), "render_fwd_l1_bwd_ms": round(ms_rt, 3),
            "decode_bwd_8M_ms": round(ms_db, 3), "train_step_ms": round(ms_dk + ms_rt + ms_db, 3),
            "gaussians_with_gradient": nz, "decode_bwd_8M_all_nonzero_ms": round(ms_dense, 3),
            "render_kernels_ms": stress_kernels, "render_train_kernels_ms": bwd_kernels,
            "decode_bwd_kernels_ms": dbwd_kernels, "train_full": full}


# [SPIN] §4 implementation details: encoder and per-attribute decoder rates;
# positions at the 3DGS position rate; 40K iterations
TRAIN_RATES = {"encoder": 8e-3, "color": 1e-3, "scale": 3e-4, "rotation": 3e-5, "opacity": 8e-4}
TRAIN_POSITION_LR = 1.6e-4
TRAIN_ITERS = 40_000
TRAIN_WARMUP = 1_000


def _train_full(S, Decoder, Renderer, stream, xyzt, fo, cams, target) -> dict:
    """One whole training step on the Stress batch, everything the step
    does inside the timed region: decode of the 8M positions (keeping the
    encoding), render of the decoded Gaussians, the Eq. 12 loss (L1 + D-SSIM)
    and its image gradient, render backward, decode backward, the position
    gradients' norms accumulated for densification, Adam over the decoder's
    groups and the positions, and the decoder parameter update.  Then one
    densify / prune of the 8M positions (Eq. 6), timed on its own."""
    import torch

    from implicit_attribute_decode_amd import ia
    from implicit_attribute_decode_amd.pipeline import Adam

    D = Decoder(S.single_decoder())
    xt = xyzt.clone()
    groups = D.param_groups(TRAIN_RATES)
    groups["positions"] = {"param": xt[:, :3], "lr": TRAIN_POSITION_LR}
    opt = Adam(groups, warmup=TRAIN_WARMUP, total=TRAIN_ITERS)
    R = Renderer()
    attrs, feats = D.decode_keep(xt)
    g = dict(attrs, means=xt[:, :3])
    n = int(xt.shape[0])
    E = Renderer.count_entries(R.render(g, fo, cams, 4 * n, aux=True, keys=False))
    cap = E + E // 4 + 4096  # the positions move between steps
    res = R.render(g, fo, cams, cap, aux=True, keys=False)
    acc = torch.zeros(n, device="cuda")
    cnt = torch.zeros(n, dtype=torch.int32, device="cuda")

    def step():
        D.decode_keep(xt, out=attrs, features=feats)
        r = R.render(g, fo, cams, cap, aux=True, keys=False, out=res)
        loss, gimg = R.image_loss(r["image"], target)
        ga = R.backward(g, fo, cams, cap, r, gimg)
        dg = D.backward(xt, ga, grad_means=ga["means"], features=feats)
        grads = D.group_grads(dg)
        grads["positions"] = dg["pos"]
        ia.ia_densify_accumulate(dg["pos"], acc, cnt)
        opt.step(grads)
        D.update_params()
        return loss

    first = step()
    l0 = [float(v) for v in first.cpu()]
    ms = timed(step, 3, stream)
    kernels = profiled(step, 1)
    last = [float(v) for v in step().cpu()]
    overflow = int(res["overflow"].item())
    # one densify / prune of the 8M positions on the gradients accumulated above
    # (3DGS's thresholds: mean gradient 2e-4, scale 1 % of the scene extent, opacity 0.005)
    gen = torch.Generator(device="cuda").manual_seed(11)
    noise = torch.randn((n, 2, 3), generator=gen, device="cuda")
    m_pos, v_pos = opt.state["positions"]
    out_x = torch.empty((2 * n, 4), device="cuda")
    out_m = torch.empty((2 * n, 3), device="cuda")
    out_v = torch.empty((2 * n, 3), device="cuda")
    out_n = torch.zeros(1, dtype=torch.int64, device="cuda")
    dws = torch.empty(ia.ia_densify_workspace_size(n), dtype=torch.uint8, device="cuda")
    prm = ia.DensifyParams(2e-4, 0.01 * 3.0, 0.005)

    def densify():
        ia.ia_densify(xt, acc, cnt, attrs["scales"], attrs["quats"], attrs["opacity"], noise, m_pos, v_pos, prm,
                      out_x, out_m, out_v, out_n, dws)

    densify()
    ms_dn = timed(densify, 3, stream)
    rows = int(out_n.item())
    return {"tile_entries": E, "step_ms": round(ms, 3), "overflow": overflow,
            "densify_ms": round(ms_dn, 3), "densify_rows_out": rows,
            "loss_first": [round(v, 6) for v in l0], "loss_after": [round(v, 6) for v in last],
            "steps_taken": opt.t, "kernels_ms": kernels}


def median_step(fn, n, warm, stream) -> dict:
    """`warm` untimed calls, then `n` calls each bracketed by HIP events on
    the stream: median, min and max milliseconds."""
    import torch

    for _ in range(warm):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for k in range(n):
        fn()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([ev[k].elapsed_time(ev[k + 1]) for k in range(n)])
    return {"steps": n, "warmup": warm, "median_ms": round(float(np.median(ms)), 4),
            "min_ms": round(float(ms.min()), 4), "max_ms": round(float(ms.max()), 4)}


def render_counts(step, xyzt, fo, cams, attrs, E) -> dict:
    """From one render of the step's decoded attributes with T_final and
    n_contrib: visible Gaussians, tile entries and the pixel x Gaussian
    evaluations the compositing rule requires (per pixel, the entries of its
    tile up to the one after which T < 1e-4, else the whole list)."""
    import torch

    from implicit_attribute_decode_amd.pipeline import Renderer

    R = Renderer()
    g = dict(means=xyzt[:, :3], **attrs)
    res = R.render(g, fo, cams, E + E // 50 + 4096, aux=True, keys=False)
    F, W, H = len(cams), cams[0].W, cams[0].H
    tx, ty = (W + 15) // 16, (H + 15) // 16
    rg = Renderer.view(res, "tile_ranges", F * tx * ty).long()
    cnt = (rg[:, 1] - rg[:, 0]).view(F, ty * tx)
    tile = (torch.arange(H, device=xyzt.device)[:, None] // 16) * tx + torch.arange(W, device=xyzt.device)[None, :] // 16
    per_px = cnt[:, tile.view(-1)].view(F, H, W)
    stopped = res["T_final"] < 1e-4
    evals = torch.where(stopped, res["n_contrib"].long(), per_px).sum()
    vis = (Renderer.view(res, "tiles_touched", int(xyzt.shape[0])) > 0).sum()
    out = {"visible": int(vis.item()), "entries": int(res["n_entries"].item()), "evaluations": int(evals.item()),
           "stopped_pixels": int(stopped.sum().item())}
    del res, R
    return out


def fetched_gather_bytes(xyzt, h) -> float:
    """Bytes the hash gather fetches per Gaussian: the 16-byte position and,
    per level, the 8 corners (4 bytes each) of every temporal vertex with a
    non-zero weight (one vertex when t sits exactly on it, else two),
    evaluated with the fp32 operations of the time normalisation and cell
    decision of Eq. 8-9.  (A wave loads a vertex for all its lanes when any
    of them weights it; the Gaussians of a wave share one frame's time.)"""
    import torch

    t = xyzt[:, 3].float()
    tn = ((t - h.t_min) / (h.t_max - h.t_min)).clamp(0.0, 1.0)
    total = torch.zeros_like(t)
    for l in range(h.L):
        res = int(np.floor(h.base_res * h.growth ** l))
        res_t = h.temporal_res if h.temporal_res > 0 else res
        p = tn * float(res_t - 1)
        i = torch.floor(p).clamp(0, res_t - 2)
        f = p - i
        total += 8.0 * torch.where((f == 0.0) | (f == 1.0), 1.0, 2.0)
    return 16.0 + 4.0 * float(total.mean().item())


def general_t_gather(D, xyzt, seq, stream) -> dict:
    """The gather at a general time: the same positions with t moved half a
    frame off the temporal vertices (all 16 corners weighted), decoded as in
    the step; achieved algorithmic bytes against HBM."""
    import torch

    from implicit_attribute_decode_amd import ia

    xg = xyzt.clone()
    half = 0.5 / (seq.frames - 1)
    xg[:, 3] = torch.where(xg[:, 3] + half <= 1.0, xg[:, 3] + half, xg[:, 3] - half)
    out = D.decode_xyzt(xg)
    D.decode_xyzt(xg, out=out)
    torch.cuda.synchronize()
    ia.ia_profile_reset()
    ia.ia_profile_enable(True)
    for _ in range(2):
        D.decode_xyzt(xg, out=out)
    torch.cuda.synchronize()
    prof = ia.ia_profile_report()
    ia.ia_profile_enable(False)
    calls, ms = prof["gather_f16_kernel"]
    n = xyzt.shape[0] * 2 / calls
    got = GATHER_BYTES_PER_GAUSSIAN * n / (ms / calls / 1e3) / 1e9
    del out, xg
    return {"achieved": round(got, 1), "frac": round(got / HBM_PEAK_GBS, 4), "avg_launch_ms": round(ms / calls, 4),
            "positions": "sequence, t + half a frame"}


# per pixel x Gaussian evaluation of the compositing rule: offset, power (five
# products and sums), the 3-sigma and alpha tests, alpha, the colour update and
# the transmittance update; the exponential is not counted
RASTER_FLOP_PER_EVAL = 24
FP32_VALU_PEAK_TFLOPS = 78.6  # non-packed (packed fp32 instructions are not used)


def other_rooflines(ms: dict, N: int, E: int, c: dict) -> dict:
    """The step's other kernels against their own rooflines, from the same
    HIP-event times; algorithmic work per unit as in the design notes."""
    nvis = c["visible"]

    def row(names, work, peak, unit, bound, per):
        t = sum(ms.get(k, 0.0) for k in names)
        if t <= 0:
            return None
        got = work / (t / 1e3)
        return {"kernels": names, "bound": bound, "achieved": round(got, 1), "peak": peak, "unit": unit,
                "frac": round(got / peak, 4), "ms_per_step": round(t, 4), "work_per_unit": per}

    sort = ["sort_upsweep_kernel", "sort_scan_kernel", "sort_downsweep_kernel"]
    emit = ["compact_kernel", "sorted_rects_kernel", "offsets_kernel", "emit_kernel", "scan_reduce_kernel",
            "scan_top_kernel", "scan_down_kernel"]
    out = {
        "raster": row(["raster_kernel"], RASTER_FLOP_PER_EVAL * c["evaluations"] / 1e12, FP32_VALU_PEAK_TFLOPS,
                      "TFLOP/s", "valu", f"{RASTER_FLOP_PER_EVAL} flop per pixel x Gaussian evaluation "
                      f"({c['evaluations']} evaluations, measured)"),
        "preprocess": row(["preprocess_kernel"], (16.0 * N + 92.0 * nvis) / 1e9, HBM_PEAK_GBS, "GB/s", "hbm",
                          "12 B mean in + 4 B tile count out per Gaussian, + 44 B attributes in and 48 B "
                          "projection out per visible Gaussian (culled Gaussians in front of the camera also "
                          "read 28 B of scale and rotation, not counted)"),
        "radix_sort": row(sort, 24.0 * (4 * nvis + 2 * E) / 1e9, HBM_PEAK_GBS, "GB/s", "hbm",
                          f"24 B per item and pass: 4 passes over {nvis} visible Gaussians, 2 over {E} entries"),
        "key_emit": row(emit, (8.0 * N + 12.0 * E) / 1e9, HBM_PEAK_GBS, "GB/s", "hbm",
                        "8 B per Gaussian + 12 B per entry"),
        "ranges": row(["ranges_kernel"], 8.0 * E / 1e9, HBM_PEAK_GBS, "GB/s", "hbm", "8 B per entry"),
        "normalize": row(["normalize_kernel"], 32.0 * N / 1e9, HBM_PEAK_GBS, "GB/s", "hbm",
                         "16 B in + 16 B out per Gaussian"),
        "mlp": row(["mlp_f16_kernel"], MLP_FLOP_PER_GAUSSIAN * N / 1e12, MFMA_F16_PEAK_TFLOPS, "TFLOP/s", "mfma",
                   "13,696 flop per Gaussian (beside the gather, one block per compute unit)"),
    }
    return {k: v for k, v in out.items() if v is not None}


def profiled(fn, reps):
    """Milliseconds per call of each library kernel over `reps` calls of fn
    (HIP events around every launch), largest first."""
    import torch

    from implicit_attribute_decode_amd import ia

    torch.cuda.synchronize()
    ia.ia_profile_reset()
    ia.ia_profile_enable(True)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    prof = ia.ia_profile_report()
    ia.ia_profile_enable(False)
    return {k: round(v[1] / reps, 4) for k, v in sorted(prof.items(), key=lambda kv: -kv[1][1])}


def timed(fn, reps, stream):
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--parts", type=int, default=1,
                    help="groups of frames; each group's render overlaps the next group's decode")
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--frames", type=int, default=150)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the per-frame comparison and the other workloads (Single, HexPlane, Stress)")
    ap.add_argument("--only", choices=("single", "hexplane", "paper", "stress"),
                    help="run just that other workload and print its figures (for profiling)")
    ap.add_argument("--stored-order", action="store_true",
                    help="keep each frame's Gaussians (and the HexPlane canonical set) in their stored order (default: Morton order, "
                         "a one-time ia_spatial_order of the fixed position sets, timed on its own)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy (a reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding is a design, not part of this build", file=sys.stderr)
        sys.exit(2)

    import torch

    from implicit_attribute_decode_amd import ia, scenes as S
    from implicit_attribute_decode_amd.pipeline import (Decoder, FrameGraphs, HexPlane, PipelinedDecodeRender,
                                                        Renderer, spatial_order)

    ia.load()  # fails loudly when the HIP library is missing
    if args.only:
        print(json.dumps(secondary(S, Decoder, HexPlane, Renderer, torch.cuda.current_stream(), log, args.only,
                                   args.stored_order)),
              flush=True)
        return
    dev = "cuda"
    seq = S.Sequence(frames=args.frames)
    F, per = seq.frames, seq.per_frame
    N = F * per
    t0 = time.perf_counter()
    xyzt = torch.as_tensor(seq.xyzt(), device=dev)
    log(f"positions: {N} in {time.perf_counter() - t0:.1f} s")
    dec = S.single_decoder()
    cams = [seq.camera(f) for f in range(F)]
    fo = np.arange(F + 1, dtype=np.int64) * per
    stream = torch.cuda.current_stream()
    layout = {"order": "stored"}
    if not args.stored_order:
        # the per-frame position sets are fixed model data: store each frame's
        # Gaussians along a Morton curve once (not part of a step)
        spatial_order(xyzt, fo)
        order_ms = timed(lambda: spatial_order(xyzt, fo), 3, stream)
        _, xyzt = spatial_order(xyzt, fo)
        layout = {"order": "per-frame Morton (ia_spatial_order, once)", "spatial_order_ms": round(order_ms, 3)}
        log(f"spatial order of {N} positions: {order_ms:.3f} ms")
    attrs = {k: torch.empty((N, w), device=dev) for k, w in (("scales", 3), ("quats", 4), ("colors", 3))}
    attrs["opacity"] = torch.empty((N,), device=dev)
    image = torch.empty((F, 3, seq.H, seq.W), device=dev)

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    D = Decoder(dec)
    # frames in `parts` groups: group k renders on a second stream beside the
    # decode of group k + 1
    step = PipelinedDecodeRender(D, xyzt, fo, cams, attrs, image, args.parts)
    E = step.probe()
    log(f"tile entries: {E}, {args.parts} groups")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms_step = timed(step, args.steps, stream)
    wall = (time.perf_counter() - wall0) / args.steps
    log(f"step: {ms_step:.3f} ms (wall {1e3 * wall:.3f} ms)")
    # the timing protocol of the measurement plan: 10 warm-ups, then the
    # median of 50 steps, each bracketed by HIP events on the stream
    med = median_step(step, 50, 10, stream)
    log(f"median of 50 steps: {med['median_ms']:.3f} ms")

    # per kernel: HIP events around every library launch, on its launch stream
    ia.ia_profile_reset()
    ia.ia_profile_enable(True)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    prof = ia.ia_profile_report()
    ia.ia_profile_enable(False)
    kernels = {k: {"calls_per_step": round(v[0] / 3, 2), "ms_per_step": round(v[1] / 3, 4)}
               for k, v in sorted(prof.items(), key=lambda kv: -kv[1][1])}
    log("per-kernel (ms/step): " + ", ".join(f"{k} {v['ms_per_step']:.3f}" for k, v in kernels.items()))
    per_step_ms = {k: v[1] / 3 for k, v in prof.items()}
    calls, gather_ms = prof["gather_f16_kernel"]
    gather_avg_ms = gather_ms / calls
    gaussians_per_launch = N * 3 / calls
    achieved = GATHER_BYTES_PER_GAUSSIAN * gaussians_per_launch / (gather_avg_ms / 1e3) / 1e9

    # the counts the other rooflines need, from one render of this step's attributes
    counts = render_counts(step, xyzt, fo, cams, attrs, E)
    fetched = fetched_gather_bytes(xyzt, dec.hash)
    general = general_t_gather(D, xyzt, seq, stream)
    kernel_rooflines = other_rooflines(per_step_ms, N, E, counts)
    log(f"rooflines: {kernel_rooflines}")

    extra = {}
    if not args.no_extra:
        # per-frame: 150 x (decode 200k, render 1 frame)
        Rf = Renderer()
        capf = int(E / F * 3) + 4096

        def frame_pass():
            for f in range(F):
                sl = slice(f * per, (f + 1) * per)
                a = D.decode_xyzt(xyzt[sl], out={k: v[sl] for k, v in attrs.items()})
                Rf.render(dict(means=xyzt[sl, :3], **a), [0, per], [cams[f]], capf, out={"image": image[f:f + 1]})

        frame_pass()
        extra["per_frame_mode_fps"] = round(F / (timed(frame_pass, 1, stream) / 1e3), 2)
        log(f"per-frame mode {extra['per_frame_mode_fps']} fps")
        # the same per-frame work replayed from one HIP graph per frame
        FG = FrameGraphs(D, Rf, xyzt, fo, cams, capf, attrs, image)
        ms_graph = timed(FG.replay, 3, stream)
        extra["per_frame_graph_fps"] = round(F / (ms_graph / 1e3), 2)
        one = timed(lambda: FG.replay([0]), 20, stream)
        extra["per_frame_graph_one_frame_ms"] = round(one, 4)
        log(f"per-frame graphs {extra['per_frame_graph_fps']} fps ({one:.4f} ms for one frame)")
        del FG, Rf
        extra["secondary"] = secondary(S, Decoder, HexPlane, Renderer, stream, log, stored_order=args.stored_order)

    fps = F / (ms_step / 1e3)
    result = {
        "metric": "frames/sec and Gaussians/sec (decode+render) at 640×360, 200k Gaussians/frame",
        "value": round(fps, 2),
        "unit": "frames/s",
        "gaussians_per_s": round(N / (ms_step / 1e3), 1),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "median_of_50": med,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 MFMA (decoder MLP) + fp32",
        "data": "synthetic",
        "config": {"workload": f"sequence: {F} frames x {per} Gaussians = {N} (x,y,z,t), 640x360, "
                               "27-camera ring, 16-level fp16 hash (2^19), 32-64-64-11 GELU decoder",
                   "frames": F, "gaussians_per_frame": per, "tile_entries": E, "frame_groups": args.parts,
                   "layout": layout,
                   "kernels": kernels, "kernel_rooflines": kernel_rooflines, "render_counts": counts, **extra},
        "roofline": {"kernel": "gather_f16_kernel", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (round(GATHER_TRAFFIC_BYTES_PER_LAUNCH) if GATHER_TRAFFIC_BYTES_PER_LAUNCH
                                 and F == 150 and per == 200_000 and not args.stored_order else None),
                     "traffic_unit": "bytes/launch", "bytes_per_unit": GATHER_BYTES_PER_GAUSSIAN,
                     "units_per_launch": round(gaussians_per_launch), "avg_launch_ms": round(gather_avg_ms, 4),
                     # the corners the kernel actually fetches (zero-weight corners are skipped)
                     "fetched_bytes_per_unit": round(fetched, 1),
                     "achieved_fetched": round(achieved * fetched / GATHER_BYTES_PER_GAUSSIAN, 1),
                     "frac_fetched": round(achieved * fetched / GATHER_BYTES_PER_GAUSSIAN / HBM_PEAK_GBS, 4),
                     # the same positions half a frame off the temporal vertices: all 16 corners weighted
                     "general_t": general},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(seq, dec)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
