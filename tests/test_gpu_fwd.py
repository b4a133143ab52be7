"""GPU forward against the float64 oracle.

Small workloads are compared on every output element.  The full-size video
workloads run in the launch configuration the benchmark times: the
32 760-token ones are compared on every row and head, the 131 040-token ones
on sampled rows of every query tile (its first and last row plus seeded
random rows, for every head)."""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_bsattn_amd as bs
import oracle
import workloads as W
from parity_util import (assert_close, check_mask_csr, gpu_mask_csr,
                         lse_tolerance, oracle_mask, oracle_rows_and_lse_tol,
                         to64)

pytestmark = pytest.mark.gpu


def run_gpu(w, q=None, k=None, v=None, want_lse=True):
    mask, rp, ci = gpu_mask_csr(w)
    if q is None:
        q, k, v = W.make_qkv(w, device="cuda")
    out = bs.attention(q, k, v, rp, ci, w.tile, mask_heads=w.mask.mask_heads,
                       want_lse=want_lse)
    torch.cuda.synchronize()
    return (q, k, v, mask, rp, ci) + (out if want_lse else (out, None))


def full_parity(w, lse_tol=None):
    q, k, v, mask, rp, ci, o, lse = run_gpu(w)
    m_ref = check_mask_csr(w, mask, rp, ci)
    o_ref, lse_ref = oracle.block_sparse_attention(q.cpu(), k.cpu(), v.cpu(),
                                                   m_ref, w.tile, workers=8)
    if lse_tol is None:
        lse_tol = lse_tolerance(q, k, m_ref, w.tile)
    assert_close(w.name, to64(o), o_ref, to64(lse), lse_ref, lse_tol=lse_tol)
    return o, lse


@pytest.mark.parametrize("r", [0, 1, 2, 3])
def test_tiny_config_every_step(r):
    # fp32 inputs are rounded to bf16 for the matrix products, so the scores
    # (and the log-sum-exp) carry bf16 input rounding: |dS| ~ 2^-8 |q||k|/sqrt(d)
    full_parity(W.WORKLOADS[1].with_rotation(r), lse_tol=2e-2)


SMALL = [
    # name, frames, gh, gw, tile, d, H, B, dtype, mask
    ("ragged_t64_d64", 3, 5, 9, 64, 64, 2, 1, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=1, num_anchors=1, rotation=2)),
    ("ragged_t64_d128", 5, 7, 11, 64, 128, 3, 2, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=0, num_anchors=2, rotation=1)),
    ("ragged_t128_d128", 5, 9, 13, 128, 128, 2, 1, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=1, num_anchors=1, rotation=4)),
    ("ragged_t128_d64", 7, 9, 13, 128, 64, 2, 2, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=1, num_anchors=2, rotation=3)),
    ("static_perhead_t128", 6, 10, 13, 128, 128, 3, 2, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_STATIC_RANDOM, seed=9, thresh24=W.thresh24_for_density(0.4),
                force_diagonal=1, mask_heads=3)),
    ("static_shared_t64", 6, 10, 13, 64, 64, 2, 1, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_STATIC_RANDOM, seed=10, thresh24=W.thresh24_for_density(0.3),
                force_diagonal=1, mask_heads=1)),
    ("dense_f32_t128_d128", 4, 8, 9, 128, 128, 2, 1, W.DTYPE_F32,
     W.MaskSpec(W.MASK_DENSE)),
    ("dense_f32_t64_d128", 4, 8, 9, 64, 128, 1, 1, W.DTYPE_F32,
     W.MaskSpec(W.MASK_DENSE)),
    ("exact_tiles_t128", 4, 8, 16, 128, 128, 2, 1, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=1, num_anchors=1)),
    ("expanded_t64_d64", 9, 4, 5, 64, 64, 2, 1, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_WINDOW_ANCHOR_EXPANDED, window=1, num_anchors=2,
                rotation=5, budget=6)),
    ("expanded_t128_d128", 12, 6, 11, 128, 128, 2, 1, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_WINDOW_ANCHOR_EXPANDED, window=0, num_anchors=3,
                rotation=7, budget=5)),
    ("single_token", 1, 1, 1, 128, 128, 1, 1, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_DENSE)),
    ("one_partial_tile", 1, 5, 7, 64, 64, 2, 1, W.DTYPE_BF16,
     W.MaskSpec(W.MASK_DENSE)),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_full_parity(case):
    name, T, gh, gw, tile, d, H, B, dt, mask = case
    w = W.small_workload(frames=T, grid_h=gh, grid_w=gw, tile=tile, d=d, H=H,
                         B=B, dtype=dt, mask=mask, name=name,
                         seed=zlib.crc32(name.encode()) & 0xFFFF)
    full_parity(w, lse_tol=2e-2 if dt == W.DTYPE_F32 else None)


def test_empty_rows():
    """Rows whose active list is empty give O = 0 and lse = -inf."""
    w = W.small_workload(frames=6, grid_h=10, grid_w=13, tile=64, d=64, H=2,
                         mask=W.MaskSpec(W.MASK_STATIC_RANDOM, seed=4,
                                         thresh24=W.thresh24_for_density(0.15),
                                         force_diagonal=0, mask_heads=2))
    q, k, v, mask, rp, ci, o, lse = run_gpu(w)
    m_ref = check_mask_csr(w, mask, rp, ci)
    assert (m_ref.sum(axis=2) == 0).any(), "case needs an empty row"
    o_ref, lse_ref = oracle.block_sparse_attention(q.cpu(), k.cpu(), v.cpu(),
                                                   m_ref, w.tile)
    assert_close(w.name, to64(o), o_ref, to64(lse), lse_ref,
                 lse_tolerance(q, k, m_ref, w.tile))
    w0 = w.with_mask(thresh24=0)
    q, k, v, mask, rp, ci, o, lse = run_gpu(w0, q, k, v)
    assert int(rp[-1]) == 0
    assert (o == 0).all() and torch.isneginf(lse).all()


def test_scale_argument():
    w = W.small_workload(frames=3, grid_h=8, grid_w=9, tile=64, d=128, H=2)
    mask, rp, ci = gpu_mask_csr(w)
    q, k, v = W.make_qkv(w, device="cuda")
    o = bs.attention(q, k, v, rp, ci, w.tile, scale=0.21)
    torch.cuda.synchronize()
    o_ref, _ = oracle.block_sparse_attention(q.cpu(), k.cpu(), v.cpu(),
                                             oracle_mask(w), w.tile, scale=0.21)
    assert_close("scale=0.21", to64(o), o_ref)


def test_skipped_tiles_are_never_read():
    """K/V tiles that no query tile reads are filled with NaN; the output must
    stay finite and bitwise equal to the unpoisoned run."""
    T, gh, gw, tile = 9, 10, 13, 64
    w = W.small_workload(frames=T, grid_h=gh, grid_w=gw, tile=tile, d=128, H=2,
                         mask=W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=0,
                                         num_anchors=0))
    q, k, v, mask, rp, ci, o, lse = run_gpu(w)
    m_ref = oracle_mask(w)
    # keep only tiles 0..3 active as keys for every query tile
    m_ref[:, :, 4:] = 0
    m_dev = torch.from_numpy(m_ref).cuda()
    rp, ci = bs.make_csr(m_dev)
    o1, lse1 = bs.attention(q, k, v, rp, ci, tile, want_lse=True)
    kp, vp = k.clone(), v.clone()
    kp[:, :, 4 * tile:] = float("nan")
    vp[:, :, 4 * tile:] = float("nan")
    o2, lse2 = bs.attention(q, kp, vp, rp, ci, tile, want_lse=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o2.float()).all()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2)
    o_ref, _ = oracle.block_sparse_attention(q.cpu(), k.cpu(), v.cpu(), m_ref,
                                             tile)
    assert_close("poisoned", to64(o2), o_ref)


def test_constant_and_tile_id_values():
    w = W.small_workload(frames=5, grid_h=9, grid_w=13, tile=128, d=128, H=2,
                         mask=W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=1,
                                         num_anchors=1, rotation=3))
    q, k, _ = W.make_qkv(w, device="cuda")
    v1 = torch.ones_like(q)
    _, _, _, mask, rp, ci, o, _ = run_gpu(w, q, k, v1)
    assert torch.allclose(o.float(), torch.ones_like(o, dtype=torch.float32),
                          atol=1e-2, rtol=0)
    tid = (torch.arange(w.N, device="cuda") // w.tile).to(q.dtype)
    vt = tid[None, None, :, None].expand_as(q).contiguous()
    o = bs.attention(q, k, vt, rp, ci, w.tile)
    torch.cuda.synchronize()
    m = mask.cpu().numpy()[0]
    of = o.float().cpu().numpy()
    for n in range(w.N):
        act = np.nonzero(m[n // w.tile])[0]
        assert act.min() - 0.05 <= of[0, 0, n, 0] <= act.max() + 0.05


def test_deterministic():
    w = W.WORKLOADS[3]
    q, k, v, mask, rp, ci, o1, l1 = run_gpu(w)
    o2, l2 = bs.attention(q, k, v, rp, ci, w.tile, mask_heads=w.mask.mask_heads,
                          want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def sample_rows(w, per_tile, seed=0):
    """`per_tile` rows of every query tile: its first and last row and
    per_tile - 2 further distinct rows drawn at random (all rows of a tile
    shorter than that)."""
    g = np.random.default_rng(seed)
    rows = []
    for i in range(w.num_tiles):
        lo = i * w.tile
        hi = min(lo + w.tile, w.N) - 1
        inner = np.arange(lo + 1, hi)
        k = max(0, min(per_tile - 2, len(inner)))
        pick = g.choice(inner, size=k, replace=False) if k else []
        rows.extend(sorted({lo, hi, *map(int, pick)}))
    return np.array(rows)


# Rows per query tile at the 131 040-token shapes: every query tile (so both
# tiles of every query-tile pair, and both groups of the tuned kernel) is
# checked, with its first and last row.
@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,per_tile,rotation", [(4, 16, 0), (4, 4, 37),
                                                   ("expanded", 8, 0), ("video_d64", 8, 0),
                                                   ("video_d64", 4, 9), ("generic0", 4, 0),
                                                   ("generic1", 4, 3), ("generic2", 4, 6)])
def test_full_size_sampled_rows(cfg, per_tile, rotation):
    """Full-size workloads on the GPU (launch configuration of the
    benchmark): the 131 040-token shapes, the 32 760-token d = 64 / tile 64
    shape and the three 32 760-token shapes of the generic kernel; the
    oracle computes `per_tile` rows of every query tile for every head."""
    generic = {f"generic{i}": g for i, g in enumerate(W.GENERIC)}
    w = ({"expanded": W.EXPANDED, "video_d64": W.VIDEO_D64}.get(cfg) or generic.get(cfg)
         or W.WORKLOADS[cfg])
    w = w.with_rotation(rotation)
    q, k, v, mask, rp, ci, o, lse = run_gpu(w)
    m_ref = check_mask_csr(w, mask, rp, ci)
    rows = sample_rows(w, per_tile, seed=rotation)
    assert len(set((rows // w.tile).tolist())) == w.num_tiles
    o_ref, lse_ref, tol = oracle_rows_and_lse_tol(q, k, v, m_ref, w.tile, rows)
    if w.dtype == W.DTYPE_F32:
        # q and k are rounded to bf16 for the matrix products (fp32 I/O)
        tol = 2e-2
    idx = torch.from_numpy(rows).cuda()
    assert_close(f"{w.name} r{rotation} ({len(rows)} rows: {per_tile} of every "
                 f"query tile, x {w.B * w.H} heads)",
                 to64(o[:, :, idx]), o_ref, to64(lse[:, :, idx]), lse_ref, tol)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cfg,rotation", [(2, 0), (2, 10), (3, 0), (5, 0)])
def test_full_size_every_row(cfg, rotation):
    """The 32 760-token workloads (window/anchor at rotations 0 and 10;
    static per head; dense with 40 heads) compared element by element on
    every output row and head, in the launch configuration the bench
    times."""
    w = W.WORKLOADS[cfg].with_rotation(rotation)
    q, k, v, mask, rp, ci, o, lse = run_gpu(w)
    m_ref = check_mask_csr(w, mask, rp, ci)
    o_ref, lse_ref, tol = oracle_rows_and_lse_tol(q, k, v, m_ref, w.tile)
    print(f"  oracle done for {w.name} r{rotation}", flush=True)
    assert_close(f"{w.name} r{rotation} (all {w.N} rows x {w.B * w.H} heads)", to64(o),
                 o_ref, to64(lse), lse_ref, tol)


def test_tuned_kernel_pair_and_split_lists_and_bad_indices():
    """bf16 / d 128 / tile 128 (the tuned kernel) on hand-built lists whose
    query-tile pairs have identical, disjoint, empty, nearly identical and
    random lists, so both of its per-workgroup modes run in one launch; then
    the same lists with out-of-range key-tile indices mixed in, which must be
    skipped."""
    w = W.small_workload(frames=16, grid_h=8, grid_w=16, tile=128, d=128, H=2)
    Tn = w.num_tiles
    assert Tn == 16
    g = np.random.default_rng(77)
    m = np.zeros((2, Tn, Tn), dtype=np.uint8)
    for h in range(2):
        lists = {
            0: [0, 3, 5, 9, 15], 1: [0, 3, 5, 9, 15],          # identical
            2: [1, 2, 3, 4, 5, 6, 7, 8], 3: [1, 2, 3, 4, 5, 6, 7, 8],
            4: [0, 2, 4, 6], 5: [1, 3, 7, 11, 13],            # disjoint
            6: [], 7: [6, 7, 8],                              # one empty
            8: [1, 2, 3, 4, 5, 9], 9: [2, 3, 4, 5, 9, 10],     # near-identical
            10: [], 11: [],                                   # both empty
        }
        for i in range(12, 16):
            lists[i] = sorted(g.choice(Tn, size=int(g.integers(1, 9)),
                                       replace=False).tolist())
        if h == 1:  # another arrangement for the second head
            lists = {i: lists[(i + 4) % 16] for i in range(16)}
        for i, js in lists.items():
            m[h, i, js] = 1
    q, k, v = W.make_qkv(w, device="cuda")
    rp, ci = bs.make_csr(torch.from_numpy(m).cuda())
    o, lse = bs.attention(q, k, v, rp, ci, w.tile, mask_heads=2, want_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(q.cpu(), k.cpu(), v.cpu(), m,
                                                   w.tile)
    tol = lse_tolerance(q, k, m, w.tile)
    assert_close("pair/split lists", to64(o), o_ref, to64(lse), lse_ref, tol)

    # the same lists with out-of-range entries (-1, Tk, a large index) added
    rows, cols = [0], []
    for r in range(2 * Tn):
        js = np.nonzero(m.reshape(2 * Tn, Tn)[r])[0].tolist()
        if r % 3 == 0:
            js = js + [Tn]
        if r % 4 == 1:
            js = [-1] + js
        if r % 5 == 2:
            js = js + [1 << 20]
        cols += js
        rows.append(len(cols))
    rp2 = torch.tensor(rows, dtype=torch.int32, device="cuda")
    ci2 = torch.tensor(cols + [0], dtype=torch.int32, device="cuda")
    o2, lse2 = bs.attention(q, k, v, rp2, ci2, w.tile, mask_heads=2,
                            want_lse=True)
    torch.cuda.synchronize()
    assert_close("out-of-range entries skipped", to64(o2), o_ref, to64(lse2),
                 lse_ref, tol)


def test_d64_t64_kernel_quad_lists_and_bad_indices():
    """bf16 / d 64 / tile 64 (its tuned kernel: four query tiles walk the
    union of their lists) on hand-built lists: quads with identical,
    disjoint, partly empty, all empty and random lists, and a last quad of
    two tiles; then the same lists with out-of-range key-tile indices mixed
    in, which must be skipped."""
    w = W.small_workload(frames=18, grid_h=8, grid_w=8, tile=64, d=64, H=2)
    Tn = w.num_tiles
    assert Tn == 18
    g = np.random.default_rng(78)
    m = np.zeros((2, Tn, Tn), dtype=np.uint8)
    for h in range(2):
        lists = {
            0: [0, 3, 5, 9, 17], 1: [0, 3, 5, 9, 17], 2: [0, 3, 5, 9, 17],
            3: [0, 3, 5, 9, 17],                                 # identical
            4: [0, 4], 5: [1, 5, 8], 6: [2, 6, 10, 14], 7: [3, 16],  # disjoint
            8: [], 9: [7, 8, 9], 10: [], 11: [1],                # partly empty
            12: [], 13: [], 14: [], 15: [],                      # all empty
        }
        for i in (16, 17):                                        # a quad of two
            lists[i] = sorted(g.choice(Tn, size=int(g.integers(1, 10)),
                                       replace=False).tolist())
        if h == 1:
            lists = {i: lists[(i + 6) % 18] for i in range(18)}
        for i, js in lists.items():
            m[h, i, js] = 1
    q, k, v = W.make_qkv(w, device="cuda")
    rp, ci = bs.make_csr(torch.from_numpy(m).cuda())
    o, lse = bs.attention(q, k, v, rp, ci, w.tile, mask_heads=2, want_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.block_sparse_attention(q.cpu(), k.cpu(), v.cpu(), m, w.tile)
    tol = lse_tolerance(q, k, m, w.tile)
    assert_close("d64 quad lists", to64(o), o_ref, to64(lse), lse_ref, tol)
    rows, cols = [0], []
    for r in range(2 * Tn):
        js = np.nonzero(m.reshape(2 * Tn, Tn)[r])[0].tolist()
        if r % 3 == 0:
            js = js + [Tn]
        if r % 4 == 1:
            js = [-1] + js
        if r % 5 == 2:
            js = js + [1 << 20]
        cols += js
        rows.append(len(cols))
    rp2 = torch.tensor(rows, dtype=torch.int32, device="cuda")
    ci2 = torch.tensor(cols + [0], dtype=torch.int32, device="cuda")
    o2, lse2 = bs.attention(q, k, v, rp2, ci2, w.tile, mask_heads=2, want_lse=True)
    torch.cuda.synchronize()
    assert_close("d64 out-of-range entries skipped", to64(o2), o_ref, to64(lse2), lse_ref,
                 tol)


@pytest.mark.parametrize("mode", ["pair", "split"])
def test_tuned_kernel_never_reads_the_partner_tiles(mode):
    """In a query-tile pair, key tiles that only one tile of the pair reads
    are filled with NaN: the other tile's rows must be bitwise unchanged
    (pair mode skips them, split mode never fetches them for that tile)."""
    w = W.small_workload(frames=4, grid_h=8, grid_w=16, tile=128, d=128, H=1)
    Tn = w.num_tiles
    m = np.zeros((1, Tn, Tn), dtype=np.uint8)
    if mode == "pair":   # nearly identical lists
        m[0, 0, [0, 1, 2, 3]] = 1
        m[0, 1, [0, 1, 3]] = 1
        m[0, 2, [0, 1, 2, 3]] = 1
        m[0, 3, [0, 1, 2, 3]] = 1
        only_a = [2]
    else:                # unrelated lists
        m[0, 0, [0, 2]] = 1
        m[0, 1, [1, 3]] = 1
        m[0, 2, [0, 1, 2, 3]] = 1
        m[0, 3, [0, 1, 2, 3]] = 1
        only_a = [0, 2]
    q, k, v = W.make_qkv(w, device="cuda")
    rp, ci = bs.make_csr(torch.from_numpy(m).cuda())
    o1, l1 = bs.attention(q, k, v, rp, ci, w.tile, want_lse=True)
    kp, vp = k.clone(), v.clone()
    for j in only_a:
        kp[:, :, j * w.tile:(j + 1) * w.tile] = float("nan")
        vp[:, :, j * w.tile:(j + 1) * w.tile] = float("nan")
    o2, l2 = bs.attention(q, kp, vp, rp, ci, w.tile, want_lse=True)
    torch.cuda.synchronize()
    rows_b = slice(w.tile, 2 * w.tile)   # query tile 1
    assert torch.isfinite(o2[:, :, rows_b].float()).all()
    assert torch.equal(o1[:, :, rows_b], o2[:, :, rows_b])
    assert torch.equal(l1[:, :, rows_b], l2[:, :, rows_b])
    o_ref, l_ref = oracle.block_sparse_attention(q.cpu(), k.cpu(), v.cpu(), m,
                                                 w.tile)
    assert_close(f"{mode} mode", to64(o1), o_ref, to64(l1), l_ref,
                 lse_tolerance(q, k, m, w.tile))


@pytest.mark.parametrize("N,H,B,seed", [(1300, 5, 1, 1), (3000, 3, 2, 2), (32760, 4, 1, 3)])
def test_tuned_kernel_uneven_per_head_masks(N, H, B, seed):
    """Per-head masks of very different density (one head near dense, one
    near empty, one with a few long rows): the tuned kernel deals the pairs
    over the XCDs globally; every row must still be computed once.  Grids
    of 30, 72 and 512 pairs (partial last rounds included)."""
    g = torch.Generator().manual_seed(seed)
    T = -(-N // 128)
    dens = torch.linspace(0.05, 0.95, H)
    m = (torch.rand(H, T, T, generator=g) < dens[:, None, None]).to(torch.uint8)
    m[0, : max(1, T // 8)] = 1                          # a few long rows in head 0
    m[:, torch.arange(T), torch.arange(T)] = 1
    q, k, v = (torch.randn(B, H, N, 128, generator=g).to(torch.bfloat16) for _ in range(3))
    rp, ci = bs.make_csr(m.cuda())
    o, lse = bs.attention(q.cuda(), k.cuda(), v.cuda(), rp, ci, 128, mask_heads=H,
                          want_lse=True)
    torch.cuda.synchronize()
    mn = m.numpy()
    if N <= 4096:
        o_ref, lse_ref = oracle.block_sparse_attention(q, k, v, mn, 128)
        assert_close(f"uneven heads N={N}", to64(o), o_ref, to64(lse), lse_ref,
                     lse_tolerance(q, k, mn, 128))
    else:
        rows = np.concatenate([np.arange(t * 128, min((t + 1) * 128, N))[[0, -1]]
                               for t in range(T)])
        o_ref, lse_ref = oracle.block_sparse_attention_rows(q, k, v, mn, 128, rows, workers=16)
        assert_close(f"uneven heads N={N} (first/last row of every tile)",
                     to64(o[:, :, rows]), o_ref, to64(lse[:, :, rows]), lse_ref,
                     lse_tolerance(q, k, mn, 128, rows=rows))
