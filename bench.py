"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = one pass of the whole path over one synthetic batch at the
32 760-token video shape (B=1, H=12, d=128, 21 frames of 30x52 latents, bf16,
128x128 tiles): build the window(+-1 frame) + 2 rotating-anchor mask for
rotation r = (layer + step) mod 21 (layer 0), compact it into active-tile
lists, build the forward's work plan from the lists (the mask changes every
step, so the plan is rebuilt every step) and run the fused forward through
it (--planned 0: bsattn_fwd, one workgroup per query-tile pair, no plan).
Inputs are resident in HBM before timing.  SQuad's passes (two key tiles per query
tile, where the per-workgroup set-up of bsattn_fwd dominates) run through
work plans built once; elsewhere both forwards are reported, timed
interleaved call by call.

Printed: ONE JSON line with
  value        active-block TFLOP/s of the whole step (mask + lists + forward),
  ms_per_step  wall time per step,
  roofline     the forward kernel's active TFLOP/s per launch (HIP events on
               the launch stream) against the bf16 dense MFMA peak,
  cpu_baseline the float64 CPU oracle on a bounded row sample,
plus the forward-only time, the same kernel at density 1.0 and the speedup,
a density sweep, the path with LVSA expanded windows on the 84-frame
long-video shape, the static-mask calibration (block energies, selection,
agreement) with the forward on the calibrated mask, SQuad's two-pass
attention against dense attention of the same shape, and spatial
repetition (row cosines, head decision, attention on anchor rows).
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

METRIC = "block-sparse attn fwd TFLOP/s (active blocks) + ms/call at 32760 tokens"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
HEADLINE = 2                # the 32 760-token video workload
TRAFFIC_SUMMARY = "fwd_bf16_t128_d128.video_21x30x52_window_anchor.traffic.txt"
MFMA_SUMMARY = "fwd_bf16_t128_d128.video_21x30x52_window_anchor.mfma.txt"


def active_flops(mask_np: np.ndarray, w) -> float:
    """4*d*rows(i)*cols(j) summed over active tiles, real (unpadded) token
    counts, over every batch entry and head."""
    Hm, Tq, Tk = mask_np.shape
    sizes = np.minimum(w.tile, w.N - np.arange(Tq) * w.tile).astype(np.float64)
    per_slice = np.einsum("hij,i,j->h", mask_np.astype(np.float64), sizes, sizes)
    heads_per_slice = w.H if Hm == 1 else 1
    return float(4.0 * w.d * w.B * heads_per_slice * per_slice.sum())


def forward_fn(bs, torch, q, k, v, o, row_ptr, col_idx, tile, Hm, planned, stream):
    """A callable that runs one forward on fixed lists: through a plan built
    here once (bsattn_fwd_plan; the lists are static) when planned, else
    bsattn_fwd."""
    if not planned or tile != 128 or q.dtype != torch.bfloat16 or q.shape[-1] != 128:
        return lambda: bs.fwd(q, k, v, o, row_ptr, col_idx, tile, mask_heads=Hm, stream=stream)
    B, H, N, _ = q.shape
    plan = torch.empty(bs.fwd_plan_bytes(B, H, N, tile, Hm), dtype=torch.uint8,
                       device=q.device)
    bs.fwd_plan(row_ptr, col_idx, B, H, N, plan, tile, Hm, stream=stream)
    return lambda: bs.fwd_planned(q, k, v, o, row_ptr, col_idx, plan, mask_heads=Hm,
                                  stream=stream)


def settle(torch, fn, ms: float = 50.0, cap: int = 500):
    """Run fn untimed until about `ms` of wall time has passed.  After the
    GPU sits idle (host work between legs), its clock takes several
    milliseconds to come back up: timed calls issued straight away run up to
    15 % slower for the first few."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for n in range(1, cap + 1):
        fn()
        if n % 4 == 0:
            torch.cuda.synchronize()
            if (time.perf_counter() - t0) * 1e3 >= ms:
                break
    torch.cuda.synchronize()


def time_interleaved(torch, stream, fns, calls: int):
    """Median event time (ms) of each callable, the callables run in turn
    call after call, so that all see the same clock (the chip's clock
    drifts by several per cent as a run heats it)."""
    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(calls)] for _ in fns]
    settle(torch, lambda: [f() for f in fns])
    for c in range(calls):
        for f, ev in zip(fns, evs):
            ev[c][0].record(stream)
            f()
            ev[c][1].record(stream)
    torch.cuda.synchronize()
    return [float(np.median([a.elapsed_time(b) for a, b in ev])) for ev in evs]


SWEEP_P = (0.05, 0.1, 0.2, 0.3, 0.5, 0.7, 1.0)


def density_sweep(bs, W, torch, dev, q, k, v, o, calls: int = 5):
    """The forward on the 32 760-token shape with per-head static random
    masks (seed 3, diagonal forced) at several densities: median ms per call
    against active TFLOP, and a least-squares line through them, for
    bsattn_fwd and for the planned forward (a static mask's plan is built
    once, outside the timed calls), the two timed interleaved."""
    base = W.WORKLOADS[3]
    Tn = base.num_tiles
    Hm = base.H
    layout = (base.frames, base.grid_h, base.grid_w, base.tile)
    mask = torch.empty((Hm, Tn, Tn), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(Hm * Tn + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(Hm * Tn * Tn, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    pts = []
    for p in SWEEP_P:
        spec = base.mask
        bs.build_mask(layout, mask, kind=W.MASK_STATIC_RANDOM, window=0,
                      num_anchors=0, rotation=0, seed=spec.seed,
                      thresh24=W.thresh24_for_density(p),
                      force_diagonal=1, mask_heads=Hm)
        bs.compact(mask, row_ptr, col_idx)
        m_np = mask.cpu().numpy()
        flops = active_flops(m_np, base)
        runs = [forward_fn(bs, torch, q, k, v, o, row_ptr, col_idx, base.tile, Hm, pl, stream)
                for pl in (False, True)]
        ms, pms = time_interleaved(torch, stream, runs, calls)
        pts.append({"p": p, "density": round(float(m_np.mean()), 4),
                    "ms": round(ms, 4), "active_tflop": round(flops / 1e12, 4),
                    "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                    "planned_ms": round(pms, 4),
                    "planned_tflops": round(flops / (pms * 1e-3) / 1e12, 1)})

    def fit(key):
        x = np.array([pt["active_tflop"] for pt in pts])
        y = np.array([pt[key] for pt in pts])
        slope, icpt = np.polyfit(x, y, 1)
        r2 = 1.0 - ((y - (slope * x + icpt)) ** 2).sum() / ((y - y.mean()) ** 2).sum()
        return round(float(slope), 4), round(float(icpt), 4), round(float(r2), 5)

    slope, icpt, r2 = fit("ms")
    pslope, picpt, pr2 = fit("planned_ms")
    return {"mask": "static random per head (seed 3, diagonal forced), "
                    "B=1 H=12 N=32760 d=128 tile 128",
            "points": pts,
            "fit_ms_per_active_tflop": slope,
            "fit_intercept_ms": icpt,
            "fit_r2": r2,
            "planned_fit_ms_per_active_tflop": pslope,
            "planned_fit_intercept_ms": picpt,
            "planned_fit_r2": pr2}


def expanded_windows(bs, W, torch, dev, calls: int):
    """The whole path with LVSA expanded windows on the 84-frame long-video
    shape (131 040 tokens, window +-2 grown to a 21-frame budget, 4 rotating
    anchors): `calls` steps at rotations 0, 1, ..., each timed in its three
    parts with events on the launch stream."""
    w = W.EXPANDED
    q, k, v = W.make_qkv(w, device=dev)
    o = torch.empty_like(q)
    Tn = w.num_tiles
    mask = torch.empty((1, Tn, Tn), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(Tn + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(Tn * Tn, dtype=torch.int32, device=dev)
    layout = (w.frames, w.grid_h, w.grid_w, w.tile)
    stream = torch.cuda.current_stream()

    def run(r, ev=None):
        if ev is not None:
            ev[0].record(stream)
        bs.build_mask(layout, mask, stream=stream,
                      **bs.mask_params_of(w.with_rotation(r).mask))
        if ev is not None:
            ev[1].record(stream)
        bs.compact(mask, row_ptr, col_idx, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        bs.fwd(q, k, v, o, row_ptr, col_idx, w.tile, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    flops, dens = [], []
    for r in range(calls):
        run(r)
        m_np = mask.cpu().numpy()
        flops.append(active_flops(m_np, w))
        dens.append(float(m_np.mean()))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
           for _ in range(calls)]
    settle(torch, lambda: run(0))
    for r in range(calls):
        run(r, evs[r])
    torch.cuda.synchronize()
    part = lambda a, b: np.array([e[a].elapsed_time(e[b]) for e in evs])
    fwd_ms, step_ms = part(2, 3), part(0, 3)
    return {"workload": w.name,
            "mask": "window +-2 frames grown to a 21-frame budget + 4 anchors, "
                    "rotation 0.." + str(calls - 1),
            "density_mean": round(float(np.mean(dens)), 4),
            "build_mask_us": round(float(np.median(part(0, 1))) * 1e3, 2),
            "compact_us": round(float(np.median(part(1, 2))) * 1e3, 2),
            "fwd_ms_median": round(float(np.median(fwd_ms)), 4),
            "fwd_tflops": round(float(np.sum(flops) / (fwd_ms.sum() * 1e-3)) / 1e12, 1),
            "step_tflops": round(float(np.sum(flops) / (step_ms.sum() * 1e-3)) / 1e12, 1)}


def d64_leg(bs, W, torch, dev, calls: int):
    """The 32 760-token video shape at head dim 64 and 64 x 64 tiles (24
    heads, window +-1 frame + 2 anchors): `calls` steps at rotations 0, 1,
    ..., each timed in its three parts with events on the launch stream."""
    w = W.VIDEO_D64
    q, k, v = W.make_qkv(w, device=dev)
    o = torch.empty_like(q)
    Tn = w.num_tiles
    mask = torch.empty((1, Tn, Tn), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(Tn + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(Tn * Tn, dtype=torch.int32, device=dev)
    layout = (w.frames, w.grid_h, w.grid_w, w.tile)
    stream = torch.cuda.current_stream()

    def run(r, ev=None):
        if ev is not None:
            ev[0].record(stream)
        bs.build_mask(layout, mask, stream=stream,
                      **bs.mask_params_of(w.with_rotation(r).mask))
        if ev is not None:
            ev[1].record(stream)
        bs.compact(mask, row_ptr, col_idx, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        bs.fwd(q, k, v, o, row_ptr, col_idx, w.tile, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    flops, dens = [], []
    for r in range(calls):
        run(r)
        m_np = mask.cpu().numpy()
        flops.append(active_flops(m_np, w))
        dens.append(float(m_np.mean()))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
           for _ in range(calls)]
    settle(torch, lambda: run(0))
    for r in range(calls):
        run(r, evs[r])
    torch.cuda.synchronize()
    part = lambda a, b: np.array([e[a].elapsed_time(e[b]) for e in evs])
    fwd_ms = part(2, 3)
    tf = float(np.sum(flops) / (fwd_ms.sum() * 1e-3)) / 1e12
    return {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d, "tile": w.tile,
            "mask": "window +-1 frame + 2 anchors, rotation 0.." + str(calls - 1),
            "density_mean": round(float(np.mean(dens)), 4),
            "fwd_ms_median": round(float(np.median(fwd_ms)), 4),
            "fwd_tflops": round(tf, 1),
            "fwd_frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def generic_leg(bs, W, torch, dev, calls: int):
    """The generic forward (the shapes no tuned kernel takes) on the
    32 760-token video shape with the window/anchor mask at rotation 0:
    fp32 I/O at d 128 / tile 128, bf16 at d 128 / tile 64 and at d 64 /
    tile 128 (24 heads); median of `calls` event-timed calls each."""
    stream = torch.cuda.current_stream()
    recs = {}
    for w in W.GENERIC:
        dt, d, tile, H = w.dtype, w.d, w.tile, w.H
        q, k, v = W.make_qkv(w, device=dev)
        o = torch.empty_like(q)
        mask = bs.make_mask(w.frames, w.grid_h, w.grid_w, w.tile, device=dev,
                            **bs.mask_params_of(w.mask))
        row_ptr, col_idx = bs.make_csr(mask)
        flops = active_flops(mask.cpu().numpy(), w)
        run = lambda: bs.fwd(q, k, v, o, row_ptr, col_idx, w.tile, stream=stream)
        settle(torch, run)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(calls)]
        for a, b in evs:
            a.record(stream)
            run()
            b.record(stream)
        torch.cuda.synchronize()
        ms = float(np.median([a.elapsed_time(b) for a, b in evs]))
        tf = flops / (ms * 1e-3) / 1e12
        recs[w.name] = {"H": H, "d": d, "tile": tile,
                        "io": "fp32" if dt == W.DTYPE_F32 else "bf16",
                        "fwd_ms_median": round(ms, 4), "fwd_tflops": round(tf, 1),
                        "fwd_frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        del q, k, v, o
        torch.cuda.empty_cache()
    return recs


def calibration(bs, W, torch, dev, calls: int):
    """Static-mask calibration at the video shape (4 prompts x 12 heads x
    32 760 tokens, frame-local Q/K): block energies, per-prompt selection at
    eps, agreement at rho, each timed with events on the launch stream;
    then the forward on the calibrated mask."""
    w = W.CALIB
    q, k = W.make_qk_frame_local(w, strength=0.7, device=dev)
    T = w.num_tiles
    stream = torch.cuda.current_stream()
    energy = torch.empty((w.B, w.H, T, T), dtype=torch.float32, device=dev)
    ews = torch.empty(bs.block_energy_workspace_bytes(w.B, w.H, w.N, w.tile), dtype=torch.uint8,
                      device=dev)
    sel = torch.empty((w.B, w.H, T, T), dtype=torch.uint8, device=dev)
    mask = torch.empty((w.H, T, T), dtype=torch.uint8, device=dev)

    def run(ev=None):
        if ev is not None:
            ev[0].record(stream)
        bs.block_energy(q, k, energy, w.tile, stream=stream, workspace=ews)
        if ev is not None:
            ev[1].record(stream)
        bs.select_blocks(energy, W.CALIB_EPS, sel, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        bs.aggregate_masks(sel, W.CALIB_RHO, mask, stream=stream)
        if ev is not None:
            ev[3].record(stream)

    settle(torch, run)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(calls)]
    for e in evs:
        run(e)
    torch.cuda.synchronize()
    part = lambda a, b: float(np.median([e[a].elapsed_time(e[b]) for e in evs]))
    e_ms = part(0, 1)
    # algorithmic work: S = Q K^T once over every (query, key) pair (the
    # one-sweep kernel's; the two-sweep one makes the product twice)
    flops = 2.0 * w.N * w.N * w.d * w.B * w.H
    m_np = mask.cpu().numpy()
    # the forward of one prompt on the calibrated (per-head) mask
    v = torch.randn(q[:1].shape, generator=torch.Generator().manual_seed(5)).to(
        torch.bfloat16).to(dev)
    rp, ci = bs.make_csr(mask)
    o = torch.empty_like(v)
    runu = forward_fn(bs, torch, q[:1], k[:1], v, o, rp, ci, w.tile, w.H, False, stream)
    runp = forward_fn(bs, torch, q[:1], k[:1], v, o, rp, ci, w.tile, w.H, True, stream)
    f_ms, fp_ms = time_interleaved(torch, stream, [runu, runp], max(calls, 5))
    from dataclasses import replace
    w1 = replace(w, B=1)
    f_flops = active_flops(m_np, w1)
    return {"workload": w.name,
            "prompts": w.B, "eps": W.CALIB_EPS, "rho": W.CALIB_RHO,
            "energy_ms": round(e_ms, 4),
            "energy_tflops": round(flops / (e_ms * 1e-3) / 1e12, 1),
            "energy_frac_of_peak": round(flops / (e_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "energy_kernel": "one sweep (per-tile row sums in a workspace)",
            "select_us": round(part(1, 2) * 1e3, 1),
            "aggregate_us": round(part(2, 3) * 1e3, 1),
            "calibrated_density": round(float(m_np.mean()), 4),
            "fwd_ms_on_calibrated_mask": round(f_ms, 4),
            "fwd_tflops_on_calibrated_mask": round(f_flops / (f_ms * 1e-3) / 1e12, 1),
            "planned_fwd_ms_on_calibrated_mask": round(fp_ms, 4),
            "planned_fwd_tflops_on_calibrated_mask": round(f_flops / (fp_ms * 1e-3) / 1e12, 1)}


def squad_leg(bs, W, torch, dev, calls: int):
    """SQuad's two-pass attention at 65 536 tokens (w = 256): the local pass
    and the global pass on the grouped view (bsattn_fwd_grouped), each timed
    with events on the launch stream; next to it the same operator through
    explicit reorders of Q, K and the local output and back; then the same
    kernel as dense attention for the comparison the page draws."""
    w = W.SQUAD
    win = W.SQUAD_W
    G = w.N // win
    q, k, v = W.make_qkv(w, device=dev)
    stream = torch.cuda.current_stream()
    layout = (1, 1, w.N, w.tile)
    masks = {}
    for b in (win // w.tile, G // w.tile):
        m = bs.make_mask(*layout, device=dev, kind=W.MASK_BLOCK_DIAGONAL, block_tiles=b)
        masks[b] = bs.make_csr(m)
    o_l, qp, kp, op, og, out = (torch.empty_like(q) for _ in range(6))

    def run(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        rp, ci = masks[win // w.tile]
        bs.fwd(q, k, v, o_l, rp, ci, w.tile, stream=stream)
        mark(1)
        rp, ci = masks[G // w.tile]
        bs.fwd_grouped(q, k, o_l, out, rp, ci, win, stream=stream)
        mark(2)

    def run_reordered(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        rp, ci = masks[win // w.tile]
        bs.fwd(q, k, v, o_l, rp, ci, w.tile, stream=stream)
        mark(1)
        bs.window_reorder(q, qp, win, stream=stream)
        bs.window_reorder(k, kp, win, stream=stream)
        bs.window_reorder(o_l, op, win, stream=stream)
        mark(2)
        rp, ci = masks[G // w.tile]
        bs.fwd(qp, kp, op, og, rp, ci, w.tile, stream=stream)
        mark(3)
        bs.window_reorder(og, out, win, inverse=True, stream=stream)
        mark(4)

    # the same two passes through work plans (built once: the masks are static)
    plans = {}
    for b, view in ((win // w.tile, 0), (G // w.tile, win)):
        rp, ci = masks[b]
        pl = torch.empty(bs.fwd_plan_bytes(w.B, w.H, w.N, w.tile, 1), dtype=torch.uint8,
                         device=dev)
        bs.fwd_plan(rp, ci, w.B, w.H, w.N, pl, w.tile, 1, stream=stream)
        plans[view] = (rp, ci, pl)

    def run_planned(ev=None):
        def mark(i):
            if ev is not None:
                ev[i].record(stream)
        mark(0)
        rp, ci, pl = plans[0]
        bs.fwd_planned(q, k, v, o_l, rp, ci, pl, stream=stream)
        mark(1)
        rp, ci, pl = plans[win]
        bs.fwd_planned(q, k, o_l, out, rp, ci, pl, window=win, stream=stream)
        mark(2)

    settle(torch, lambda: (run(), run_reordered(), run_planned()))
    evp = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(calls)]
    for e in evp:
        run_planned(e)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(calls)]
    evr = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(calls)]
    for e, er in zip(evs, evr):
        run(e)
        run_reordered(er)
    torch.cuda.synchronize()
    part = lambda es, a, b: float(np.median([e[a].elapsed_time(e[b]) for e in es]))
    flops_local = 4.0 * w.d * w.N * win * w.B * w.H
    flops_global = 4.0 * w.d * w.N * G * w.B * w.H
    reorder_bytes = 4 * 2 * w.B * w.H * w.N * w.d * 2   # 4 reorders, read + write
    l_ms, g_ms, total = part(evs, 0, 1), part(evs, 1, 2), part(evs, 0, 2)
    r_ms, rg_ms, i_ms = part(evr, 1, 2), part(evr, 2, 3), part(evr, 3, 4)
    total_r = part(evr, 0, 4)
    # dense attention of the same shape with the same kernel
    dm = bs.make_mask(*layout, device=dev, kind=W.MASK_DENSE)
    drp, dci = bs.make_csr(dm)
    settle(torch, lambda: bs.fwd(q, k, v, og, drp, dci, w.tile))
    de = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(max(1, calls // 2))]
    for a, b in de:
        a.record(stream)
        bs.fwd(q, k, v, og, drp, dci, w.tile, stream=stream)
        b.record(stream)
    torch.cuda.synchronize()
    dense_ms = float(np.median([a.elapsed_time(b) for a, b in de]))
    dense_flops = 4.0 * w.d * w.N * w.N * w.B * w.H
    p_l, p_g, p_t = part(evp, 0, 1), part(evp, 1, 2), part(evp, 0, 2)
    # compulsory HBM bytes of one pass: Q, K and V (the local output in the
    # global pass) read once, O written once.  At w = 256 a pass does 4 d w
    # FLOPs per query row against 8 d bytes: 128 FLOP/B, under the MI355X
    # ridge (2 500 TFLOP/s / 8 TB/s = 312 FLOP/B), so HBM bounds the passes.
    pass_bytes = 4.0 * w.B * w.H * w.N * w.d * 2
    gbs = lambda ms: pass_bytes / (ms * 1e-3) / 1e9
    return {"workload": w.name, "window": win, "groups": G,
            "planned_path": {"ms_total": round(p_t, 4), "local_ms": round(p_l, 4),
                             "local_tflops": round(flops_local / (p_l * 1e-3) / 1e12, 1),
                             "local_hbm_gbs": round(gbs(p_l), 1),
                             "global_grouped_ms": round(p_g, 4),
                             "global_grouped_tflops":
                                 round(flops_global / (p_g * 1e-3) / 1e12, 1),
                             "global_hbm_gbs": round(gbs(p_g), 1),
                             "hbm_frac_of_peak": round(2 * pass_bytes / (p_t * 1e-3) / 1e9
                                                       / PEAK_HBM_GBS, 4),
                             "speedup_vs_dense": round(dense_ms / p_t, 2)},
            "pass_bytes": int(pass_bytes),
            "flop_per_byte": round(flops_local / pass_bytes, 1),
            "ms_total": round(total, 4),
            "local_ms": round(l_ms, 4), "local_tflops": round(flops_local / (l_ms * 1e-3) / 1e12, 1),
            "global_grouped_ms": round(g_ms, 4),
            "global_grouped_tflops": round(flops_global / (g_ms * 1e-3) / 1e12, 1),
            "reordered_path": {"ms_total": round(total_r, 4), "global_ms": round(rg_ms, 4),
                               "reorder_ms": round(r_ms + i_ms, 4),
                               "reorder_gbs": round(reorder_bytes / ((r_ms + i_ms) * 1e-3) / 1e9, 1)},
            "attention_tflop": round((flops_local + flops_global) / 1e12, 4),
            "dense_tflop": round(dense_flops / 1e12, 3),
            "dense_ms": round(dense_ms, 3),
            "speedup_vs_dense": round(dense_ms / total, 2)}


def repetition_leg(bs, W, torch, dev, calls: int):
    """CalibAtt's spatial repetition at the video shape (21 x 30 x 52, 12
    heads; in six of them the rows of a frame repeat, the other six attend
    frame-locally): calibration (row cosines and the head decision at stride
    2, gamma 0.9; block energies, selection and agreement for the block
    lists), then the inference layer itself -- repetitive heads on anchor
    rows copied, the others on their calibrated lists, one forward for all
    heads (gather, forward, broadcast) -- against dense attention of the
    same shape."""
    w = W.WORKLOADS[2]
    stride, gamma = 2, 0.9
    q, k = W.make_qk_row_repetitive(w, rep_heads=6, local_strength=0.7, device=dev)
    v = torch.randn(q.shape, generator=torch.Generator().manual_seed(9)).to(
        torch.bfloat16).to(dev)
    stream = torch.cuda.current_stream()
    cos = torch.empty((w.B, w.H, w.frames, w.grid_h), dtype=torch.float32, device=dev)
    flags = torch.empty(w.H, dtype=torch.uint8, device=dev)
    ws = torch.empty(bs.row_cosines_workspace_bytes(w.B, w.H, w.frames, w.grid_h, w.grid_w,
                                                    stride), dtype=torch.uint8, device=dev)
    settle(torch, lambda: bs.row_cosines(q, k, w.frames, w.grid_h, w.grid_w, stride, cos,
                                         workspace=ws))
    cev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(calls)]
    for ev in cev:
        ev[0].record(stream)
        bs.row_cosines(q, k, w.frames, w.grid_h, w.grid_w, stride, cos, stream=stream,
                       workspace=ws)
        ev[1].record(stream)
        bs.repetitive_heads(cos, stride, gamma, flags, stream=stream)
        ev[2].record(stream)
    torch.cuda.synchronize()
    cos_ms = float(np.median([ev[0].elapsed_time(ev[1]) for ev in cev]))
    heads_ms = float(np.median([ev[1].elapsed_time(ev[2]) for ev in cev]))
    nonanchor = w.grid_h - (-(-w.grid_h // stride))
    # one sweep x two queries x (non-anchor rows x grid_w) x N keys x 2d
    cos_flops = 2 * w.B * w.H * w.frames * nonanchor * w.grid_w * w.N * 2.0 * w.d
    # block lists of every head from this prompt (used by the others)
    cal_mask, _, _ = bs.calibrate(q, k, w.tile, W.CALIB_EPS, W.CALIB_RHO)
    rp, ci, mixed = bs.mixed_layer_csr(flags, cal_mask, w.frames, w.grid_h, w.grid_w, stride,
                                       w.tile)
    torch.cuda.synchronize()
    qb, ob, out = torch.zeros_like(q), torch.empty_like(q), torch.empty_like(q)

    def layer():
        bs.mixed_attention(q, k, v, flags, rp, ci, w.frames, w.grid_h, w.grid_w, stride,
                           w.tile, qbuf=qb, obuf=ob, out=out, stream=stream)

    dm = bs.make_mask(w.frames, w.grid_h, w.grid_w, w.tile, device=dev, kind=W.MASK_DENSE)
    drp, dci = bs.make_csr(dm)
    o = torch.empty_like(q)

    def dense():
        bs.fwd(q, k, v, o, drp, dci, w.tile, stream=stream)

    layer_ms, dense_ms = time_interleaved(torch, stream, [layer, dense], calls)
    c = cos.cpu().numpy()
    fl = flags.cpu().numpy()
    cm = cal_mask.cpu().numpy()
    mm = mixed.cpu().numpy()
    act = active_flops(mm, w)
    return {"workload": w.name + "_calibatt_layer_6_repetitive_heads", "stride": stride,
            "gamma": gamma,
            "row_cosines_ms": round(cos_ms, 3),
            "row_cosines_tflops": round(cos_flops / (cos_ms * 1e-3) / 1e12, 1),
            "heads_ms": round(heads_ms, 4),
            "flags": fl.tolist(),
            "mean_cos_repeating_heads": round(float(c[:, :6, :, 1::2].mean()), 4),
            "mean_cos_other_heads": round(float(c[:, 6:, :, 1::2].mean()), 4),
            "calibrated_density_other_heads":
                round(float(cm[fl == 0].mean()) if (fl == 0).any() else 0.0, 4),
            "layer": "flagged heads: anchor rows (half the rows) copied; others: calibrated "
                     "lists; gather + one forward + broadcast",
            "layer_ms": round(layer_ms, 4),
            "layer_forward_active_tflop": round(act / 1e12, 4),
            "dense_ms": round(dense_ms, 4),
            "speedup_vs_dense": round(dense_ms / layer_ms, 2)}


# Time at half the bf16 dense peak for each workload's active-block work: the
# target each record is read against.
def configs_leg(bs, W, torch, dev, calls: int, planned: bool = True):
    """Every 32 760- and 131 040-token workload on its own: mask build,
    compaction and forward (median of `calls` event-timed calls each, on the
    launch stream), active TFLOP, TFLOP/s and fraction of the bf16 peak, at
    rotation 0; then the LVSA page's linear-cost claim ("Complessita") as
    forward time per active tile-head at 131 040 tokens against 32 760."""
    stream = torch.cuda.current_stream()
    recs = {}
    for key in (2, 3, 4, 5):
        w = W.WORKLOADS[key]
        q, k, v = W.make_qkv(w, device=dev)
        o = torch.empty_like(q)
        Tn = w.num_tiles
        Hm = w.mask.mask_heads
        mask = torch.empty((Hm, Tn, Tn), dtype=torch.uint8, device=dev)
        row_ptr = torch.empty(Hm * Tn + 1, dtype=torch.int32, device=dev)
        col_idx = torch.empty(Hm * Tn * Tn, dtype=torch.int32, device=dev)
        layout = (w.frames, w.grid_h, w.grid_w, w.tile)
        params = bs.mask_params_of(w.mask)

        plan = torch.empty(bs.fwd_plan_bytes(w.B, w.H, w.N, w.tile, Hm), dtype=torch.uint8,
                           device=dev) if planned else None

        def run(ev=None):
            if ev is not None:
                ev[0].record(stream)
            bs.build_mask(layout, mask, stream=stream, **params)
            if ev is not None:
                ev[1].record(stream)
            bs.compact(mask, row_ptr, col_idx, stream=stream)
            if ev is not None:
                ev[2].record(stream)
            if planned:
                bs.fwd_plan(row_ptr, col_idx, w.B, w.H, w.N, plan, w.tile, Hm, stream=stream)
            if ev is not None:
                ev[3].record(stream)
            if planned:
                bs.fwd_planned(q, k, v, o, row_ptr, col_idx, plan, mask_heads=Hm,
                               stream=stream)
            else:
                bs.fwd(q, k, v, o, row_ptr, col_idx, w.tile, mask_heads=Hm, stream=stream)
            if ev is not None:
                ev[4].record(stream)

        run()
        torch.cuda.synchronize()
        m_np = mask.cpu().numpy()
        flops = active_flops(m_np, w)
        tiles = int(m_np.sum()) * (w.H if Hm == 1 else 1) * w.B
        settle(torch, run)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(calls)]
        for e in evs:
            run(e)
        torch.cuda.synchronize()
        part = lambda a, b: float(np.median([e[a].elapsed_time(e[b]) for e in evs]))
        f_ms = part(3, 4)
        # both forwards on the same lists, interleaved
        run_u = forward_fn(bs, torch, q, k, v, o, row_ptr, col_idx, w.tile, Hm, False, stream)
        run_p = forward_fn(bs, torch, q, k, v, o, row_ptr, col_idx, w.tile, Hm, True, stream)
        u_ms, p_ms = time_interleaved(torch, stream, [run_u, run_p], calls)
        tflops = flops / (f_ms * 1e-3) / 1e12
        recs[w.name] = {
            "B": w.B, "H": w.H, "N": w.N, "mask_heads": Hm,
            "density": round(float(m_np.mean()), 4),
            "active_tile_heads": tiles,
            "active_tflop": round(flops / 1e12, 4),
            "build_mask_us": round(part(0, 1) * 1e3, 2),
            "compact_us": round(part(1, 2) * 1e3, 2),
            "plan_us": round(part(2, 3) * 1e3, 2) if planned else None,
            "fwd_ms_median": round(f_ms, 4),
            "fwd_tflops": round(tflops, 1),
            "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
            "ms_at_half_peak": round(flops / (0.5 * PEAK_BF16_TFLOPS * 1e12) * 1e3, 3),
            "us_per_active_tile_head": round(f_ms * 1e3 / tiles, 5),
            "interleaved": {"fwd_ms_median": round(u_ms, 4),
                            "planned_fwd_ms_median": round(p_ms, 4),
                            "fwd_tflops": round(flops / (u_ms * 1e-3) / 1e12, 1),
                            "planned_fwd_tflops": round(flops / (p_ms * 1e-3) / 1e12, 1)},
        }
        del q, k, v, o, mask, row_ptr, col_idx
        torch.cuda.empty_cache()
    short, long_ = recs[W.WORKLOADS[2].name], recs[W.WORKLOADS[4].name]
    recs["linear_cost_check"] = {
        "what": "forward time per active tile-head, 131 040 tokens (+-2 + 4 anchors) "
                "over 32 760 tokens (+-1 + 2 anchors); 1.0 = cost linear in active tiles",
        "ratio": round(long_["us_per_active_tile_head"] / short["us_per_active_tile_head"], 4),
        "tokens_ratio": round(long_["N"] / short["N"], 3),
        "time_ratio": round(long_["fwd_ms_median"] / short["fwd_ms_median"], 3),
    }
    return recs


def cpu_baseline(w, q, k, v, mask_np, tiles: int, workers: int):
    """The oracle as it stands, on `tiles` evenly spaced query tiles (every
    row of them, every head) at rotation 0; TFLOP/s credited like the GPU
    (active blocks only)."""
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    pick = np.linspace(0, w.num_tiles - 1, tiles).round().astype(int)
    rows = np.concatenate([np.arange(i * w.tile, min((i + 1) * w.tile, w.N))
                           for i in pick])
    sizes = np.minimum(w.tile, w.N - np.arange(w.num_tiles) * w.tile)
    flops = 0.0
    for i in pick:
        act = mask_np[0, i].astype(bool)
        flops += 4.0 * w.d * sizes[i] * sizes[act].sum()
    flops *= w.B * w.H
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    t0 = time.perf_counter()
    if threadpool_limits is not None:
        with threadpool_limits(limits=1):
            oracle.block_sparse_attention_rows(qc, kc, vc, mask_np, w.tile, rows,
                                               workers=workers)
    else:
        oracle.block_sparse_attention_rows(qc, kc, vc, mask_np, w.tile, rows,
                                           workers=workers)
    dt = time.perf_counter() - t0
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": workers,
            "threads_used": workers, "kind": "oracle", "cpu_model": cpu_model,
            "blas_threads_per_worker": 1 if threadpool_limits is not None else None,
            "sample": f"{len(rows)} query rows ({tiles} of {w.num_tiles} query "
                      f"tiles) x {w.B * w.H} heads at rotation 0, float64 NumPy, "
                      f"{dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="untimed steps for about this long before the warm-up steps "
                         "(the clock's return after the host-side setup)")
    ap.add_argument("--cpu-tiles", type=int, default=256,
                    help="query tiles in the CPU-oracle sample (0 = skip)")
    ap.add_argument("--dense-calls", type=int, default=5,
                    help="timed calls of the same kernel at density 1.0 "
                         "(0 = skip)")
    ap.add_argument("--mfma-ceiling", type=int, default=1,
                    help="measure the register-only MFMA ceiling (0 = skip)")
    ap.add_argument("--sweep", type=int, default=1,
                    help="density sweep with static masks (0 = skip)")
    ap.add_argument("--expanded", type=int, default=6,
                    help="steps of the expanded-window long-video path "
                         "(0 = skip)")
    ap.add_argument("--d64", type=int, default=6,
                    help="steps of the d 64 / tile 64 video leg (0: skip)")
    ap.add_argument("--generic", type=int, default=5,
                    help="calls per shape of the generic-forward leg (0 = skip)")
    ap.add_argument("--calib", type=int, default=3,
                    help="timed calls of the static-mask calibration leg "
                         "(0 = skip)")
    ap.add_argument("--squad", type=int, default=6,
                    help="timed calls of the SQuad two-pass leg (0 = skip)")
    ap.add_argument("--repetition", type=int, default=5,
                    help="timed calls of the spatial-repetition leg (0 = skip)")
    ap.add_argument("--planned", type=int, default=1,
                    help="headline step: forward through a work plan rebuilt every "
                         "step (bsattn_fwd_plan + bsattn_fwd_planned); 0 = bsattn_fwd")
    ap.add_argument("--other-calls", type=int, default=10,
                    help="timed calls of the other forward (planned or not) on the "
                         "last step's lists (0 = skip)")
    ap.add_argument("--configs", type=int, default=10,
                    help="timed calls per workload of the per-config records "
                         "(0 = skip)")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB "
                         "(byte-counter calibration under a profiler)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the block-sparse path here has no "
              "multi-GPU implementation (heads would shard with no exchange); "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_bsattn_amd as bs
    import workloads as W

    bs.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[HEADLINE]
    q, k, v = W.make_qkv(w, device=dev)
    o = torch.empty_like(q)
    Tn = w.num_tiles
    Hm = w.mask.mask_heads
    mask = torch.empty((Hm, Tn, Tn), dtype=torch.uint8, device=dev)
    row_ptr = torch.empty(Hm * Tn + 1, dtype=torch.int32, device=dev)
    col_idx = torch.empty(Hm * Tn * Tn, dtype=torch.int32, device=dev)
    layout = (w.frames, w.grid_h, w.grid_w, w.tile)
    stream = torch.cuda.current_stream()
    T = w.frames

    # active FLOPs for every rotation the run visits
    flops_by_r = {}
    for r in range(T):
        bs.build_mask(layout, mask, **bs.mask_params_of(w.with_rotation(r).mask))
        flops_by_r[r] = active_flops(mask.cpu().numpy(), w)

    # the planned forward's plan buffer, sized for any list set of this
    # shape (allocated once, outside the timed steps)
    plan = torch.empty(bs.fwd_plan_bytes(w.B, w.H, w.N, w.tile, Hm), dtype=torch.uint8,
                       device=dev) if args.planned else None

    def step(s, ev=None):
        """One pass of the path; ev = 5 events bracketing mask build,
        compaction, the plan (planned forward only) and the forward on the
        launch stream."""
        r = s % T  # (layer + step) mod T with layer 0
        if ev is not None:
            ev[0].record(stream)
        bs.build_mask(layout, mask, stream=stream,
                      **bs.mask_params_of(w.with_rotation(r).mask))
        if ev is not None:
            ev[1].record(stream)
        bs.compact(mask, row_ptr, col_idx, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        if args.planned:
            bs.fwd_plan(row_ptr, col_idx, w.B, w.H, w.N, plan, w.tile, Hm, stream=stream)
        if ev is not None:
            ev[3].record(stream)
        if args.planned:
            bs.fwd_planned(q, k, v, o, row_ptr, col_idx, plan, mask_heads=Hm, stream=stream)
        else:
            bs.fwd(q, k, v, o, row_ptr, col_idx, w.tile, mask_heads=Hm, stream=stream)
        if ev is not None:
            ev[4].record(stream)
        return flops_by_r[r]

    # After the host-side setup above the GPU's clock takes several
    # milliseconds of work to come back up (timed calls issued straight away
    # ran up to 15 % slower for the first few, and the rate still crept up
    # by about 1 % over the next few hundred milliseconds): the step runs
    # untimed for about --settle-ms first, so that the W warm-up steps and the
    # K timed ones start from a running clock whatever W is.
    if args.settle_ms > 0:
        n_settle = iter(range(1 << 30))
        settle(torch, lambda: step(next(n_settle)), ms=args.settle_ms, cap=10000)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)]
              for _ in range(args.steps)]
    total_flops = 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        total_flops += step(args.warmup + s, events[s])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    fwd_ms = np.array([e[3].elapsed_time(e[4]) for e in events])
    mask_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    compact_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    plan_ms = np.array([e[2].elapsed_time(e[3]) for e in events])

    # the other forward on the lists of the last step: without a plan (one
    # workgroup per query-tile pair) or through one (built once here)
    ab = None
    if args.other_calls > 0:
        run_u = forward_fn(bs, torch, q, k, v, o, row_ptr, col_idx, w.tile, Hm, False, stream)
        run_p = forward_fn(bs, torch, q, k, v, o, row_ptr, col_idx, w.tile, Hm, True, stream)
        u_ms, p_ms = time_interleaved(torch, stream, [run_u, run_p], args.other_calls)
        ab = {"lists": "the last step's (rotation %d)" % ((args.warmup + args.steps - 1) % T),
              "fwd_ms_median": round(u_ms, 4), "planned_fwd_ms_median": round(p_ms, 4),
              "planned_speedup": round(u_ms / p_ms, 4)}
    ms_per_step = elapsed * 1e3 / args.steps
    value = total_flops / elapsed / 1e12
    fwd_flops_mean = total_flops / args.steps
    fwd_tflops = fwd_flops_mean / (fwd_ms.mean() * 1e-3) / 1e12

    # achievable matrix-core rate: register-only MFMA stream, best of 3
    ceiling = None
    if args.mfma_ceiling:
        blocks, iters = 1024, 2000
        sink = torch.empty(blocks, dtype=torch.float32, device=dev)
        bs.mfma_ceiling(blocks, iters, sink, stream=stream)
        rates = []
        for _ in range(3):
            a_ev = torch.cuda.Event(enable_timing=True)
            b_ev = torch.cuda.Event(enable_timing=True)
            a_ev.record(stream)
            n = bs.mfma_ceiling(blocks, iters, sink, stream=stream)
            b_ev.record(stream)
            torch.cuda.synchronize()
            rates.append(n / (a_ev.elapsed_time(b_ev) * 1e-3) / 1e12)
        ceiling = max(rates)

    # the same kernel at density 1.0 on the same shape
    dense_ms = dense_flops = None
    if args.dense_calls > 0:
        bs.build_mask(layout, mask, kind=W.MASK_DENSE, mask_heads=Hm)
        bs.compact(mask, row_ptr, col_idx)
        dense_flops = active_flops(mask.cpu().numpy(), w)
        run = forward_fn(bs, torch, q, k, v, o, row_ptr, col_idx, w.tile, Hm,
                         bool(args.planned), stream)
        settle(torch, run)
        dev_ev = [(torch.cuda.Event(enable_timing=True),
                   torch.cuda.Event(enable_timing=True))
                  for _ in range(args.dense_calls)]
        for a, b in dev_ev:
            a.record(stream)
            run()
            b.record(stream)
        torch.cuda.synchronize()
        dense_ms = float(np.median([a.elapsed_time(b) for a, b in dev_ev]))

    sweep = density_sweep(bs, W, torch, dev, q, k, v, o) \
        if args.sweep else None

    expanded = expanded_windows(bs, W, torch, dev, args.expanded) \
        if args.expanded > 0 else None

    d64 = d64_leg(bs, W, torch, dev, args.d64) if args.d64 > 0 else None

    generic = generic_leg(bs, W, torch, dev, args.generic) if args.generic > 0 else None

    calib = calibration(bs, W, torch, dev, args.calib) if args.calib > 0 else None

    squad = squad_leg(bs, W, torch, dev, args.squad) if args.squad > 0 else None

    repetition = repetition_leg(bs, W, torch, dev, args.repetition) \
        if args.repetition > 0 else None

    configs = configs_leg(bs, W, torch, dev, args.configs, bool(args.planned)) \
        if args.configs > 0 else None

    if args.copy_mib > 0:
        src = torch.empty(args.copy_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if args.cpu_tiles > 0:
        bs.build_mask(layout, mask, **bs.mask_params_of(w.with_rotation(0).mask))
        torch.cuda.synchronize()
        # the pool takes every core this process may run on, up to 16 (the
        # host share that goes with one GPU); both counts are reported
        host = len(os.sched_getaffinity(0))
        workers = max(1, min(16, host))
        cpu = cpu_baseline(w, q, k, v, mask.cpu().numpy(), args.cpu_tiles, workers)
        cpu["host_cores_visible"] = host

    # HBM bytes per launch from the committed PMC summary, if it was taken on
    # this kernel source
    from block_sparse_attention_bsattn_amd import rocprof_summary
    src = os.path.join(ROOT, "block_sparse_attention_bsattn_amd", "csrc", "fwd_bf16_t128.hip")
    traffic = rocprof_summary.read_traffic(os.path.join(ROOT, "profiles", TRAFFIC_SUMMARY), src)
    mfma = rocprof_summary.read_mfma(os.path.join(ROOT, "profiles", MFMA_SUMMARY), src)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms_before_warmup": args.settle_ms,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
            "tile": w.tile, "frames": w.frames, "grid": [w.grid_h, w.grid_w],
            "mask": "window +-1 frame + 2 anchors rotating (layer+step) mod 21",
            "step": "build_mask + compact + fwd_plan + fwd_planned" if args.planned
                    else "build_mask + compact + fwd",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(fwd_tflops, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(fwd_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": None if traffic is None else round(traffic["total"]),
            "traffic_unit": "bytes/launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE)",
            "traffic_gbs": None if traffic is None else
            round(traffic["total"] / (float(fwd_ms.mean()) * 1e-3) / 1e9, 1),
            "mfma_busy_rocprof": None if mfma is None else round(mfma["busy"], 4),
            "kernel": "fwd_bf16_t128_d128<false, true>" if args.planned
                      else "fwd_bf16_t128_d128<false, false>",
            "fwd_ms_mean": round(float(fwd_ms.mean()), 4),
            "active_tflop_per_launch": round(fwd_flops_mean / 1e12, 4),
            "mfma_ceiling_measured": None if ceiling is None else round(ceiling, 1),
            "frac_of_measured_ceiling": None if ceiling is None else
            round(fwd_tflops / ceiling, 4),
        },
        "fwd_ms_per_call": round(float(fwd_ms.mean()), 4),
        "fwd_ms_median": round(float(np.median(fwd_ms)), 4),
        "build_mask_us": round(float(np.median(mask_ms)) * 1e3, 2),
        "compact_us": round(float(np.median(compact_ms)) * 1e3, 2),
        "plan_us": round(float(np.median(plan_ms)) * 1e3, 2) if args.planned else None,
        "planned_vs_unplanned_interleaved": ab,
        "density": None if dense_flops is None else round(fwd_flops_mean / dense_flops, 4),
        "dense_fwd_ms": None if dense_ms is None else round(dense_ms, 4),
        "dense_tflops": None if dense_ms is None else
        round(dense_flops / (dense_ms * 1e-3) / 1e12, 3),
        "speedup_vs_density_1": None if dense_ms is None else
        round(dense_ms / float(fwd_ms.mean()), 3),
        "configs": configs,
        "density_sweep": sweep,
        "expanded_windows": expanded,
        "d64_t64": d64,
        "generic_fwd": generic,
        "calibration": calib,
        "squad": squad,
        "repetition": repetition,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
