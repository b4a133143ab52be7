"""The planned forward (bsattn_fwd_plan + bsattn_fwd_planned).

The plan is integer work and is compared bit for bit with what the CSR
fixes: every query-tile pair dealt to exactly one worker, its mode by
bsattn_fwd's rule, for a pair-mode item its merged key-tile list in
ascending order with the right group flags, for a split-mode item each
tile's own list in its group's stream.  The planned forward computes a
pair-mode pair as bsattn_fwd does, and each tile of a split-mode pair as
bsattn_fwd computes a tile in pair mode, so its O and LSE must be bitwise
equal to bsattn_fwd's for pair-mode pairs and to bsattn_fwd's on a CSR whose
pairs hold twin lists for split-mode pairs; at full size it is also
compared with the float64 oracle."""
import numpy as np
import pytest
import torch

import block_sparse_attention_bsattn_amd as bs
import oracle
import workloads as W
from parity_util import (assert_close, check_mask_csr, gpu_mask_csr,
                         oracle_rows_and_lse_tol, to64)

pytestmark = pytest.mark.gpu

PAIR_BITS = 15
TILE_BITS = 13
BAD_TILE = 0x0FFFFFFE


def read_plan(plan, items):
    a = plan.cpu().numpy().view(np.int32)
    h = a[:16]
    W_ = int(h[6])
    sec = {k: int(h[8 + i]) * 4 for i, k in enumerate(
        ("wstep", "witem", "wcnt", "witems", "pinfo", "itmp", "steps"))}
    cap = int(h[15])
    return dict(
        header=h,
        workers=W_,
        wstep=a[sec["wstep"]:sec["wstep"] + 4 * W_].reshape(W_, 4),
        witem=a[sec["witem"]:sec["witem"] + 2 * W_].reshape(W_, 2),
        witems=a[sec["witems"]:sec["witems"] + items],
        itmp=a[sec["itmp"]:sec["itmp"] + 4 * items].reshape(items, 4),
        steps=a[sec["steps"]:sec["steps"] + 2 * cap].reshape(cap, 2),
    )


def _lists(rp, ci, tiles, s, p):
    r0 = s * tiles + 2 * p
    la = ci[rp[r0]:rp[r0 + 1]].tolist()
    lb = ci[rp[r0 + 1]:rp[r0 + 2]].tolist() if 2 * p + 1 < tiles else []
    return la, lb


def expected_items(rp, ci, B, H, N, Hm):
    """Per item (b*H + h) * pairs + p: (split, union steps, list A, list B)
    from the CSR, by the rule bsattn_fwd uses (split mode when 5 I < n0 + n1
    or a list is empty; I common valid tiles, n raw lengths)."""
    tiles = -(-N // 128)
    pairs = (tiles + 1) // 2
    out = {}
    cache = {}
    for s in range(Hm):
        for p in range(pairs):
            la, lb = _lists(rp, ci, tiles, s, p)
            a = {t for t in la if 0 <= t < tiles}
            b = {t for t in lb if 0 <= t < tiles}
            n0, n1 = len(la), len(lb)
            split = n0 == 0 or n1 == 0 or 5 * len(a & b) < n0 + n1
            cache[s, p] = (split, [(t, t in a, t in b) for t in sorted(a | b)],
                           sorted(a), sorted(b))
    for bh in range(B * H):
        s = 0 if Hm == 1 else bh % H
        for p in range(pairs):
            out[bh * pairs + p] = cache[s, p]
    return out, pairs, tiles


def check_plan(plan, rp, ci, B, H, N, Hm):
    """The plan against the CSR, bit for bit; returns (plan fields, number
    of split-mode items)."""
    rp = rp.cpu().numpy()
    ci = ci.cpu().numpy()
    exp, pairs, tiles = expected_items(rp, ci, B, H, N, Hm)
    P = read_plan(plan, len(exp))
    h = P["header"]
    assert (h[0], h[1], h[2], h[3], h[5], h[7]) == (0x42535031, B, H, N, Hm, pairs)
    seen = np.zeros(len(exp), dtype=np.int64)
    pos = 0
    nsplit = 0
    for w in range(P["workers"]):
        first, cnt = P["witem"][w]
        streams = ([], [], [])
        for t in range(cnt):
            iw = int(P["witems"][first + t])
            split = iw < 0
            iw &= 0x7FFFFFFF
            bh, p = iw >> PAIR_BITS, iw & ((1 << PAIR_BITS) - 1)
            i = bh * pairs + p
            seen[i] += 1
            esplit, union, la, lb = exp[i]
            assert split == esplit, f"item {i}: mode"
            if not split:
                streams[0].extend([(t_ | (n0 << 30) | (n1 << 29), iw) for t_, n0, n1 in union]
                                  or [(BAD_TILE, iw)])
                continue
            nsplit += 1
            wd = (bh << TILE_BITS) | (2 * p)
            ga, gb = (2, 1) if (P["itmp"][i][3] >> 30) & 1 else (1, 2)   # orientation
            streams[ga].extend([(t_, wd) for t_ in la] or [(BAD_TILE, wd)])
            if 2 * p + 1 < tiles:
                streams[gb].extend([(t_, wd + 1) for t_ in lb] or [(BAD_TILE, wd + 1)])
        for g in range(3):
            assert P["wstep"][w][g] == pos, f"worker {w}: stream {g} not contiguous"
            got = P["steps"][pos:pos + len(streams[g])]
            assert [tuple(x) for x in got.tolist()] == streams[g], f"worker {w}: stream {g}"
            pos += len(streams[g])
        assert P["wstep"][w][3] == pos
    assert (seen == 1).all(), "every item exactly once"
    return P, nsplit


def _twin_csr(rp, ci, tiles, Hm, keep_even):
    """The CSR with each query-tile pair's two rows both holding one tile's
    list (tile 2p's when keep_even, else tile 2p + 1's)."""
    rp = rp.cpu().numpy()
    ci = ci.cpu().numpy()
    rows, cols = [0], []
    for s in range(Hm):
        for r in range(tiles):
            src = (r & ~1) if keep_even else min(r | 1, tiles - 1)
            r0 = s * tiles + src
            cols += ci[rp[r0]:rp[r0 + 1]].tolist()
            rows.append(len(cols))
    return (torch.tensor(rows, dtype=torch.int32, device="cuda"),
            torch.tensor(cols + [0], dtype=torch.int32, device="cuda"))


def reference_of_plan(q, k, v, rp, ci, Hm, window=0):
    """What the planned forward must give bit for bit: bsattn_fwd's output
    for pair-mode pairs; for split-mode pairs, each tile as bsattn_fwd
    computes a tile in pair mode (its group walking its own list), taken
    from bsattn_fwd on a CSR whose pairs both hold that tile's list.  With
    an odd number of tiles the last one has no partner, so bsattn_fwd can
    compute it in split mode only: its rows are NaN here (not compared; the
    oracle checks them)."""
    B, H, N, _ = q.shape
    tiles = -(-N // 128)

    def run(rp_, ci_):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        if window:
            bs.fwd_grouped(q, k, v, o, rp_, ci_, window, mask_heads=Hm, lse=lse)
        else:
            bs.fwd(q, k, v, o, rp_, ci_, 128, mask_heads=Hm, lse=lse)
        return o, lse

    o, lse = run(rp, ci)
    exp, pairs, _ = expected_items(rp.cpu().numpy(), ci.cpu().numpy(), B, H, N, Hm)
    split_pairs = [(bh, p) for bh in range(B * H) for p in range(pairs)
                   if exp[bh * pairs + p][0]]
    if split_pairs:
        oa, la = run(*_twin_csr(rp, ci, tiles, Hm, True))
        ob, lb = run(*_twin_csr(rp, ci, tiles, Hm, False))
        o = o.view(B * H, N, -1)
        lse = lse.view(B * H, N)
        for src_o, src_l, odd in ((oa, la, 0), (ob, lb, 1)):
            so = src_o.view(B * H, N, -1)
            sl = src_l.view(B * H, N)
            for bh, p in split_pairs:
                t = 2 * p + odd
                if t == tiles - 1 and tiles % 2 == 1:
                    so = so.clone()
                    sl = sl.clone()
                    so[bh, t * 128:N] = float("nan")
                    sl[bh, t * 128:N] = float("nan")
                if t < tiles:
                    r0, r1 = t * 128, min(t * 128 + 128, N)
                    if window:   # rows of position-major tile t in the window-major buffer
                        G = N // window
                        idx = torch.tensor([(pp % G) * window + pp // G for pp in range(r0, r1)],
                                           device=q.device)
                        o[bh, idx] = so[bh, idx]
                        lse[bh, idx] = sl[bh, idx]
                    else:
                        o[bh, r0:r1] = so[bh, r0:r1]
                        lse[bh, r0:r1] = sl[bh, r0:r1]
        o = o.view(q.shape)
        lse = lse.view(q.shape[:3])
    return o, lse, len(split_pairs)


def run_both(q, k, v, rp, ci, Hm, workers=0, window=0):
    B, H, N, _ = q.shape
    plan = bs.make_plan(rp, ci, B, H, N, 128, Hm, workers)
    o_p, l_p = bs.attention_planned(q, k, v, rp, ci, plan, mask_heads=Hm, want_lse=True,
                                    workers=workers, window=window)
    o, lse, _ = reference_of_plan(q, k, v, rp, ci, Hm, window)
    torch.cuda.synchronize()
    return plan, o_p, l_p, o, lse


def assert_bitwise(name, o_p, l_p, o, lse):
    keep = ~torch.isnan(lse)          # rows the reference leaves out (NaN)
    same_o = torch.equal(o_p[keep], o[keep])
    same_l = torch.equal(l_p[keep].view(torch.int32), lse[keep].view(torch.int32))
    if not (same_o and same_l):
        d = (o_p.float() - o.float()).abs().max().item()
        pytest.fail(f"{name}: planned differs from bsattn_fwd (max |dO| {d:.3e}, "
                    f"O equal {same_o}, LSE equal {same_l})")
    print(f"{name}: bitwise equal", flush=True)


def _small(T, gh, gw, H, B, mask, seed):
    return W.small_workload(frames=T, grid_h=gh, grid_w=gw, tile=128, d=128, H=H, B=B,
                            mask=mask, seed=seed, name=f"planned_{T}x{gh}x{gw}")


SMALL = [
    ("window_odd_tiles", _small(7, 9, 13, 2, 1, W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=1,
                                                             num_anchors=2, rotation=3), 1)),
    ("window_b2", _small(5, 8, 16, 3, 2, W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=0,
                                                     num_anchors=1, rotation=1), 2)),
    ("static_perhead", _small(6, 10, 13, 3, 2, W.MaskSpec(
        W.MASK_STATIC_RANDOM, seed=9, thresh24=W.thresh24_for_density(0.4), force_diagonal=1,
        mask_heads=3), 3)),
    ("static_sparse_empty_rows", _small(6, 10, 13, 2, 1, W.MaskSpec(
        W.MASK_STATIC_RANDOM, seed=4, thresh24=W.thresh24_for_density(0.12), force_diagonal=0,
        mask_heads=2), 4)),
    ("dense", _small(4, 8, 9, 2, 1, W.MaskSpec(W.MASK_DENSE), 5)),
    ("expanded", _small(12, 6, 11, 2, 1, W.MaskSpec(W.MASK_WINDOW_ANCHOR_EXPANDED, window=0,
                                                     num_anchors=3, rotation=7, budget=5), 6)),
    ("one_tile", _small(1, 5, 7, 2, 1, W.MaskSpec(W.MASK_DENSE), 7)),
]


@pytest.mark.parametrize("workers", [0, 8, 64])
@pytest.mark.parametrize("name,w", SMALL, ids=[c[0] for c in SMALL])
def test_small_plan_and_bitwise(name, w, workers):
    mask, rp, ci = gpu_mask_csr(w)
    m_ref = check_mask_csr(w, mask, rp, ci)
    q, k, v = W.make_qkv(w, device="cuda")
    Hm = w.mask.mask_heads
    plan, o_p, l_p, o, lse = run_both(q, k, v, rp, ci, Hm, workers)
    _, nsplit = check_plan(plan, rp, ci, w.B, w.H, w.N, Hm)
    print(f"{name}: {nsplit} split-mode pairs", flush=True)
    assert_bitwise(f"{name} workers={workers}", o_p, l_p, o, lse)
    if workers == 0:
        o_ref, l_ref, tol = oracle_rows_and_lse_tol(q, k, v, m_ref, 128, workers=8)
        assert_close(f"{name} planned", to64(o_p), o_ref, to64(l_p), l_ref, tol)


def test_lists_with_out_of_range_entries_and_empty_pairs():
    """Hand-built lists (identical, disjoint, one or both empty, random) with
    key-tile indices outside [0, Tk) mixed in: the plan leaves them out, and
    the planned forward equals bsattn_fwd, which skips them."""
    w = W.small_workload(frames=16, grid_h=8, grid_w=16, tile=128, d=128, H=2)
    Tn = w.num_tiles
    g = np.random.default_rng(77)
    lists = {0: [0, 3, 5, 9, 15], 1: [0, 3, 5, 9, 15], 2: [1, 2, 3, 4, 5, 6, 7, 8],
             3: [1, 2, 3, 4, 5, 6, 7, 8], 4: [0, 2, 4, 6], 5: [1, 3, 7, 11, 13], 6: [],
             7: [6, 7, 8], 8: [1, 2, 3, 4, 5, 9], 9: [2, 3, 4, 5, 9, 10], 10: [], 11: []}
    for i in range(12, 16):
        lists[i] = sorted(g.choice(Tn, size=int(g.integers(1, 9)), replace=False).tolist())
    rows, cols = [0], []
    for r in range(2 * Tn):
        js = list(lists[r % Tn] if r < Tn else lists[(r + 4) % Tn])
        if r % 3 == 0:
            js = js + [Tn]
        if r % 4 == 1:
            js = [-1] + js
        if r % 5 == 2:
            js = js + [1 << 20]
        cols += js
        rows.append(len(cols))
    rp = torch.tensor(rows, dtype=torch.int32, device="cuda")
    ci = torch.tensor(cols + [0], dtype=torch.int32, device="cuda")
    q, k, v = W.make_qkv(w, device="cuda")
    for workers in (0, 8):
        plan, o_p, l_p, o, lse = run_both(q, k, v, rp, ci, 2, workers)
        check_plan(plan, rp, ci, 1, 2, w.N, 2)
        assert_bitwise(f"hand-built lists workers={workers}", o_p, l_p, o, lse)


@pytest.mark.parametrize("N,H,B,seed", [(1300, 5, 1, 1), (32760, 4, 1, 3)])
def test_uneven_per_head_masks(N, H, B, seed):
    g = torch.Generator().manual_seed(seed)
    T = -(-N // 128)
    dens = torch.linspace(0.05, 0.95, H)
    m = (torch.rand(H, T, T, generator=g) < dens[:, None, None]).to(torch.uint8)
    m[0, : max(1, T // 8)] = 1
    m[:, torch.arange(T), torch.arange(T)] = 1
    q, k, v = (torch.randn(B, H, N, 128, generator=g).to(torch.bfloat16).cuda()
               for _ in range(3))
    rp, ci = bs.make_csr(m.cuda())
    plan, o_p, l_p, o, lse = run_both(q, k, v, rp, ci, H)
    check_plan(plan, rp, ci, B, H, N, H)
    assert_bitwise(f"uneven heads N={N}", o_p, l_p, o, lse)


@pytest.mark.parametrize("cfg,rotation,workers", [
    (2, 0, 0), (2, 5, 0), (3, 0, 0), (4, 0, 0), (5, 0, 0), ("expanded", 2, 0),
    # two workers per XCD (each holds about 96 items, too many for the
    # refinement's lists: the deal stands as dealt), six and eight per XCD
    (2, 10, 16), (3, 0, 48), (2, 0, 64)])
def test_full_size_plan_and_bitwise(cfg, rotation, workers):
    """Every full-size workload in the launch configuration the bench
    times (and a few other worker counts): the plan against the CSR, and
    the planned forward bitwise equal to bsattn_fwd."""
    w = (W.EXPANDED if cfg == "expanded" else W.WORKLOADS[cfg]).with_rotation(rotation)
    mask, rp, ci = gpu_mask_csr(w)
    q, k, v = W.make_qkv(w, device="cuda")
    Hm = w.mask.mask_heads
    plan, o_p, l_p, o, lse = run_both(q, k, v, rp, ci, Hm, workers)
    check_plan(plan, rp, ci, w.B, w.H, w.N, Hm)
    assert_bitwise(f"{w.name} r{rotation} workers={workers}", o_p, l_p, o, lse)


@pytest.mark.timeout(900)
def test_full_size_planned_against_the_oracle():
    """The 32 760-token window/anchor workload at rotation 7, planned, on
    every row and head against the float64 oracle."""
    w = W.WORKLOADS[2].with_rotation(7)
    mask, rp, ci = gpu_mask_csr(w)
    m_ref = check_mask_csr(w, mask, rp, ci)
    q, k, v = W.make_qkv(w, device="cuda")
    o, lse = bs.attention_planned(q, k, v, rp, ci, want_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref, tol = oracle_rows_and_lse_tol(q, k, v, m_ref, 128)
    assert_close(f"{w.name} r7 planned (all rows)", to64(o), o_ref, to64(lse), l_ref, tol)


def test_grouped_view_planned_equals_fwd_grouped():
    """SQuad's global pass through a plan on the grouped view: bitwise equal
    to bsattn_fwd_grouped."""
    N, win, H = 16384, 128, 3
    G = N // win
    m = bs.make_mask(1, 1, N, 128, device="cuda", kind=W.MASK_BLOCK_DIAGONAL,
                     block_tiles=G // 128)
    rp, ci = bs.make_csr(m)
    g = torch.Generator().manual_seed(12)
    q, k, v = (torch.randn(1, H, N, 128, generator=g).to(torch.bfloat16).cuda()
               for _ in range(3))
    plan, o_p, l_p, o, lse = run_both(q, k, v, rp, ci, 1, window=win)
    assert_bitwise("grouped view", o_p, l_p, o, lse)


def test_never_read_tiles_are_never_fetched():
    """K/V tiles no query tile reads are NaN; the planned output stays
    finite and bitwise equal to the unpoisoned one."""
    w = W.small_workload(frames=9, grid_h=10, grid_w=26, tile=128, d=128, H=2,
                         mask=W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=0, num_anchors=0))
    Tn = w.num_tiles
    m = np.zeros((1, Tn, Tn), dtype=np.uint8)
    m[0, :, :4] = 1
    rp, ci = bs.make_csr(torch.from_numpy(m).cuda())
    q, k, v = W.make_qkv(w, device="cuda")
    plan = bs.make_plan(rp, ci, 1, 2, w.N)
    o1, l1 = bs.attention_planned(q, k, v, rp, ci, plan, want_lse=True)
    kp, vp = k.clone(), v.clone()
    kp[:, :, 4 * 128:] = float("nan")
    vp[:, :, 4 * 128:] = float("nan")
    o2, l2 = bs.attention_planned(q, kp, vp, rp, ci, plan, want_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o2.float()).all()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def _lumpy_masks(H, T, seed):
    """Per-head masks whose lists are mostly short (12 to 41 tiles) with a
    few long ones (about 8 % of even query tiles get 170 more); each odd
    tile repeats its even neighbour's list plus two tiles, so pairs run in
    pair mode."""
    rng = np.random.default_rng(seed)
    m = np.zeros((H, T, T), dtype=np.uint8)
    for h in range(H):
        for i in range(T):
            if i % 2 == 1:
                m[h, i] = m[h, i - 1]
                m[h, i, rng.choice(T, size=2, replace=False)] = 1
                continue
            n = min(T, 12 + (170 if rng.random() < 0.08 else 0) + int(rng.integers(0, 30)))
            m[h, i, rng.choice(T, size=n, replace=False)] = 1
    return m


def _worker_loads(plan, rp, ci, B, H, N, Hm):
    """Each worker's load by the plan's own cost estimate (pair mode
    5 (union + 1), split mode 4 (n0 + n1) + 5), from its item list."""
    P, _ = check_plan(plan, rp, ci, B, H, N, Hm)
    exp, pairs, tiles = expected_items(rp.cpu().numpy(), ci.cpu().numpy(), B, H, N, Hm)
    load = np.zeros(P["workers"], dtype=np.int64)
    for w in range(P["workers"]):
        first, cnt = P["witem"][w]
        for t in range(cnt):
            iw = int(P["witems"][first + t]) & 0x7FFFFFFF
            bh, p = iw >> PAIR_BITS, iw & ((1 << PAIR_BITS) - 1)
            split, union, la, lb = exp[bh * pairs + p]
            if split:
                sb = max(len(lb), 1) if 2 * p + 1 < tiles else 0
                load[w] += 4 * (max(len(la), 1) + sb) + 5
            else:
                load[w] += 5 * (max(len(union), 1) + 1)
    return load


def test_plan_deals_lumpy_lists_evenly():
    """A few very long items among many short ones: the deal must leave no
    worker far above the mean load.  Dealing one item to every worker in
    each round left the worst worker at about 1.6x the mean here; rounds of
    half the workers, after ranking a whole XCD range, about 1.04x."""
    H, T = 12, 256
    N = T * 128
    m = _lumpy_masks(H, T, 11)
    rp, ci = bs.make_csr(torch.from_numpy(m).cuda())
    plan = bs.make_plan(rp, ci, 1, H, N, 128, H)
    torch.cuda.synchronize()
    load = _worker_loads(plan, rp, ci, 1, H, N, H)
    ratio = float(load.max() / load.mean())
    print(f"lumpy lists: worst worker {ratio:.3f}x the mean load", flush=True)
    assert ratio < 1.15


@pytest.mark.parametrize("rotation", [0, 10])
def test_plan_evens_out_the_window_mask(rotation):
    """The 32 760-token window mask has about six pairs per worker and XCD
    ranges of 190 or 194 of them, so the deal alone leaves two workers of
    an XCD holding seven (about 1.08x the mean load); the refinement after
    it brings the worst worker to within 3 % of the mean."""
    w = W.WORKLOADS[2].with_rotation(rotation)
    mask, rp, ci = gpu_mask_csr(w)
    plan = bs.make_plan(rp, ci, w.B, w.H, w.N, 128, w.mask.mask_heads)
    torch.cuda.synchronize()
    load = _worker_loads(plan, rp, ci, w.B, w.H, w.N, w.mask.mask_heads)
    ratio = float(load.max() / load.mean())
    print(f"window mask r{rotation}: worst worker {ratio:.3f}x the mean load", flush=True)
    assert ratio < 1.03


def test_plan_cuts_xcd_ranges_by_measured_speed():
    """A planned forward leaves each workgroup's run time and load in the
    library's per-GPU table; the next plan weights the eight XCD ranges by
    the speeds measured there (relative to their mean, clamped to
    [0.9, 1.1]) and keeps the weights at byte 64.  Each XCD's share of the
    total estimated cost must follow its weight to within one item's cost."""
    w = W.WORKLOADS[2]
    mask, rp, ci = gpu_mask_csr(w)
    q, k, v = W.make_qkv(w, device="cuda")
    o = torch.empty_like(q)
    plan = bs.make_plan(rp, ci, w.B, w.H, w.N, 128, 1)
    for _ in range(3):
        bs.fwd_planned(q, k, v, o, rp, ci, plan)
    bs.fwd_plan(rp, ci, w.B, w.H, w.N, plan, 128, 1)
    torch.cuda.synchronize()
    wt = plan[64:96].cpu().numpy().view(np.int32).astype(np.float64) / 4096.0
    print("XCD weights:", np.round(wt, 3), flush=True)
    assert ((wt >= 0.9 - 1e-3) & (wt <= 1.1 + 1e-3)).all()
    P, _ = check_plan(plan, rp, ci, w.B, w.H, w.N, 1)
    exp, pairs, tiles = expected_items(rp.cpu().numpy(), ci.cpu().numpy(), w.B, w.H, w.N, 1)
    cost = np.zeros(8)
    biggest = 0
    for wk in range(P["workers"]):
        first, cnt = P["witem"][wk]
        for t in range(cnt):
            iw = int(P["witems"][first + t]) & 0x7FFFFFFF
            bh, p = iw >> PAIR_BITS, iw & ((1 << PAIR_BITS) - 1)
            split, union, la, lb = exp[bh * pairs + p]
            c = (4 * (max(len(la), 1) + (max(len(lb), 1) if 2 * p + 1 < tiles else 0)) + 5
                 if split else 5 * (max(len(union), 1) + 1))
            cost[wk % 8] += c
            biggest = max(biggest, c)
    share, want = cost / cost.sum(), wt / wt.sum()
    print("cost shares:", np.round(share, 4), "weights:", np.round(want, 4), flush=True)
    assert np.abs(share - want).max() <= biggest / cost.sum() + 1e-9


def test_uniform_items_ignore_xcd_weights():
    """With items of one cost (a dense mask: 1 536 pairs of 256 key tiles,
    six per worker) a weighted cut would put a seventh item on some workers
    of a faster XCD; the plan then cuts the ranges evenly whatever the
    weights: 192 pairs per XCD."""
    w = W.WORKLOADS[2]
    m = bs.make_mask(w.frames, w.grid_h, w.grid_w, w.tile, device="cuda", kind=W.MASK_DENSE)
    rp, ci = bs.make_csr(m)
    q, k, v = W.make_qkv(w, device="cuda")
    o = torch.empty_like(q)
    plan = bs.make_plan(rp, ci, w.B, w.H, w.N, 128, 1)
    for _ in range(2):
        bs.fwd_planned(q, k, v, o, rp, ci, plan)
    bs.fwd_plan(rp, ci, w.B, w.H, w.N, plan, 128, 1)
    torch.cuda.synchronize()
    P, _ = check_plan(plan, rp, ci, w.B, w.H, w.N, 1)
    per_xcd = np.zeros(8, dtype=np.int64)
    for wk in range(P["workers"]):
        per_xcd[wk % 8] += P["witem"][wk][1]
    print("weights", plan[64:96].cpu().numpy().view(np.int32) / 4096.0, "pairs per XCD", per_xcd,
          flush=True)
    assert (per_xcd == 192).all()


def test_short_launches_leave_equal_xcd_weights():
    """Speeds measured on short launches (workgroups busy under 400 us on
    average) are not trusted: after a planned forward on a small shape the
    next plan weights every XCD alike."""
    w = W.WORKLOADS[2]
    mask, rp, ci = gpu_mask_csr(w)
    q, k, v = W.make_qkv(w, device="cuda")
    o = torch.empty_like(q)
    plan = bs.make_plan(rp, ci, w.B, w.H, w.N, 128, 1)
    for _ in range(2):
        bs.fwd_planned(q, k, v, o, rp, ci, plan)
    ws = W.small_workload(frames=8, grid_h=8, grid_w=16, tile=128, d=128, H=2)
    _, rps, cis = gpu_mask_csr(ws)
    qs, ks, vs = W.make_qkv(ws, device="cuda")
    plan_s = bs.make_plan(rps, cis, ws.B, ws.H, ws.N, 128, ws.mask.mask_heads)
    bs.fwd_planned(qs, ks, vs, torch.empty_like(qs), rps, cis, plan_s,
                   mask_heads=ws.mask.mask_heads)
    bs.fwd_plan(rp, ci, w.B, w.H, w.N, plan, 128, 1)
    torch.cuda.synchronize()
    wt = plan[64:96].cpu().numpy().view(np.int32)
    assert (wt == 4096).all(), wt


def test_plan_for_other_sizes_writes_nothing():
    w = W.small_workload(frames=4, grid_h=8, grid_w=16, tile=128, d=128, H=2)
    mask, rp, ci = gpu_mask_csr(w)
    q, k, v = W.make_qkv(w, device="cuda")
    plan = bs.make_plan(rp, ci, 1, 3, w.N)        # built for H = 3
    o = torch.full_like(q, 7.0)
    bs.fwd_planned(q, k, v, o, rp, ci, plan)
    torch.cuda.synchronize()
    assert (o == 7.0).all()
