"""GPU spatial repetition (CalibAtt page, "A. Fase di Calibrazione" step 3
and "B. Fase di Inferenza") against the oracle: row cosines within a
tolerance from fp32 summation, head decisions, gather/broadcast and the
dense-rows mask bit-exact, and attention on anchor rows copied to the rest."""
import numpy as np
import pytest
import torch

import block_sparse_attention_bsattn_amd as bs
import oracle
import workloads as W
from layout_contract import anchor_buffer_rows
from parity_util import assert_close, check_mask_csr, gpu_mask_csr, to64

pytestmark = pytest.mark.gpu

# Each probability carries a few ulp of fp32 rounding (scores, exponent,
# v_exp) and the normalisers and inner products are float sums of per-step
# partials, so the cosine (a ratio of such sums, in [0, 1]) is within about
# 1e-5 of the exact value; 1e-4 leaves a margin.
COS_TOL = 1e-4


def _qk(B, H, T, gh, gw, d, seed, dt=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    shape = (B, H, T * gh * gw, d)
    return (torch.randn(shape, generator=g).to(dt), torch.randn(shape, generator=g).to(dt))


@pytest.mark.parametrize("B,H,T,gh,gw,d,s,dt", [
    (2, 2, 2, 5, 16, 128, 2, torch.bfloat16),
    (1, 1, 2, 7, 52, 128, 3, torch.bfloat16),     # two waves, a ragged one
    (1, 2, 3, 4, 40, 64, 2, torch.float32),      # fp32 inputs, d 64
    (1, 1, 1, 3, 200, 64, 2, torch.bfloat16),    # seven waves
    (1, 1, 2, 4, 8, 128, 1, torch.bfloat16),     # stride 1: all anchors
    (1, 1, 2, 3, 96, 128, 2, torch.bfloat16),    # three waves a row, one idle a group
    (1, 2, 2, 3, 128, 128, 2, torch.bfloat16),   # four waves a row
    (1, 1, 1, 3, 13, 128, 2, torch.bfloat16),    # N = 39: one partial key tile
    (2, 1, 3, 5, 33, 128, 2, torch.bfloat16),    # 31 idle columns in every second wave
    (1, 1, 2, 5, 160, 128, 2, torch.bfloat16),   # grid_w > 128: the generic kernel
    (1, 1, 2, 5, 20, 128, 2, torch.float32),     # fp32 inputs, d 128: the generic kernel
])
@pytest.mark.parametrize("packed", [True, False])
def test_row_cosines(B, H, T, gh, gw, d, s, dt, packed):
    """Both schedules of the tuned kernel (packed columns with a workspace,
    row-aligned without) and the generic kernel against the oracle."""
    q, k = _qk(B, H, T, gh, gw, d, 100 + gh * gw + s, dt)
    cos = torch.empty(B, H, T, gh, dtype=torch.float32, device="cuda")
    bs.row_cosines(q.cuda(), k.cuda(), T, gh, gw, s, cos, packed=packed)
    torch.cuda.synchronize()
    qo, ko = (q, k) if dt == torch.bfloat16 else (q.to(torch.bfloat16), k.to(torch.bfloat16))
    want = oracle.row_cosines(qo, ko, T, gh, gw, s)
    got = cos.cpu().numpy()
    err = float(np.abs(got - want).max())
    print(f"cos B{B} H{H} T{T} {gh}x{gw} d{d} s{s} packed {packed}: max|dcos| {err:.2e}",
          flush=True)
    assert err <= COS_TOL
    anchors = [y for y in range(gh) if s * (y // s) == y]
    assert (got[:, :, :, anchors] == 1.0).all()


@pytest.mark.parametrize("scale", [0.0, 0.25])
def test_row_cosines_rising_scores(scale):
    """Keys ordered so that every query's scores grow with the key index: the
    running max of each query rises at almost every 64-key step, so the
    normalisers and inner products are rescaled many times over the sweep
    (and, at scale 0.25, the softmax is sharp)."""
    B, H, T, gh, gw, d, s = 1, 2, 3, 5, 40, 128, 2
    N = T * gh * gw
    g = torch.Generator().manual_seed(2024)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = torch.randn(B, H, N, d, generator=g) * 0.5 + 2.0 * u
    ramp = torch.linspace(-8.0, 8.0, N).reshape(1, 1, N, 1)
    k = torch.randn(B, H, N, d, generator=g) * 0.5 + ramp * u
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    cos = torch.empty(B, H, T, gh, dtype=torch.float32, device="cuda")
    bs.row_cosines(q.cuda(), k.cuda(), T, gh, gw, s, cos, scale=scale)
    torch.cuda.synchronize()
    want = oracle.row_cosines(q, k, T, gh, gw, s, scale=scale if scale > 0 else None)
    got = cos.cpu().numpy()
    err = float(np.abs(got - want).max())
    print(f"cos rising scores scale {scale}: max|dcos| {err:.2e} "
          f"range [{float(want.min()):.3f}, {float(want.max()):.3f}]", flush=True)
    assert err <= COS_TOL


@pytest.mark.parametrize("jump", [20.0, 60.0, 200.0])
def test_row_cosines_score_jumps(jump):
    """Every query's scores jump by `jump` (log2 units) at one late key tile
    and fall back after it: the running max then grows long after the first
    tile, by less (20: exponentials up to 2^20 against the old max) or more
    (60, 200: the tile is redone against its exact max, and at 200 all
    earlier sums vanish) than the kernel's rescaling limit."""
    B, H, T, gh, gw, d, s = 1, 2, 2, 6, 40, 128, 2
    N = T * gh * gw
    g = torch.Generator().manual_seed(77)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = torch.randn(B, H, N, d, generator=g) * 0.3 + 1.0 * u
    k = torch.randn(B, H, N, d, generator=g) * 0.3
    # scale 1: score ~ 1.0 * c for a key c * u; jump in natural units
    c = jump / 1.4426950408889634
    k[:, :, 5 * 64 + 3:5 * 64 + 40] += c * u
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    cos = torch.empty(B, H, T, gh, dtype=torch.float32, device="cuda")
    bs.row_cosines(q.cuda(), k.cuda(), T, gh, gw, s, cos, scale=1.0)
    torch.cuda.synchronize()
    want = oracle.row_cosines(q, k, T, gh, gw, s, scale=1.0)
    got = cos.cpu().numpy()
    err = float(np.abs(got - want).max())
    print(f"cos score jump {jump}: max|dcos| {err:.2e} "
          f"range [{float(want.min()):.4f}, {float(want.max()):.4f}]", flush=True)
    assert np.isfinite(got).all()
    assert err <= COS_TOL


def test_row_cosines_video_shape_sampled():
    """The benchmark's calibration shape and inputs (21 x 30 x 52, 12 heads,
    stride 2; six heads with repeating rows, six frame-local), sampled: the
    oracle's cosine for three non-anchor rows of every head (first, last
    and one random frame), every anchor row exactly 1, every value
    finite."""
    w = W.WORKLOADS[2]
    s = 2
    q, k = W.make_qk_row_repetitive(w, rep_heads=6, local_strength=0.7)
    qc, kc = q.cuda(), k.cuda()
    rng = np.random.default_rng(5)
    cells = []
    for h in range(w.H):
        for f in (0, w.frames - 1, int(rng.integers(1, w.frames - 1))):
            cells.append((0, h, f, 1 + s * int(rng.integers(0, w.grid_h // s))))
    want = oracle.row_cosines_at(q, k, w.frames, w.grid_h, w.grid_w, s, cells)
    for packed in (True, False):
        cos = torch.empty(w.B, w.H, w.frames, w.grid_h, dtype=torch.float32, device="cuda")
        bs.row_cosines(qc, kc, w.frames, w.grid_h, w.grid_w, s, cos, packed=packed)
        torch.cuda.synchronize()
        got = cos.cpu().numpy()
        assert np.isfinite(got).all()
        assert (got[:, :, :, 0::s] == 1.0).all()
        g = np.array([got[c] for c in cells])
        err = float(np.abs(g - want).max())
        print(f"cos video shape, packed {packed}, {len(cells)} sampled rows: "
              f"max|dcos| {err:.2e}", flush=True)
        assert err <= COS_TOL


def test_row_cosines_of_repeated_rows_are_one():
    B, H, T, gh, gw, d = 1, 2, 2, 6, 24, 128
    q, k = _qk(B, H, T, gh, gw, d, 7)
    q = q.reshape(B, H, T, gh, gw, d)
    q[:, 0, :, 1::2] = q[:, 0, :, 0::2]      # head 0: odd rows repeat their anchors
    q = q.reshape(B, H, T * gh * gw, d)
    cos = torch.empty(B, H, T, gh, dtype=torch.float32, device="cuda")
    bs.row_cosines(q.cuda(), k.cuda(), T, gh, gw, 2, cos)
    flags = torch.empty(H, dtype=torch.uint8, device="cuda")
    bs.repetitive_heads(cos, 2, 0.999, flags)
    torch.cuda.synchronize()
    c = cos.cpu().numpy()
    assert np.abs(c[:, 0] - 1.0).max() < 1e-5
    assert (c[:, 1, :, 1::2] < 0.99).all()
    assert flags.cpu().tolist() == [1, 0]


@pytest.mark.parametrize("B,H,T,gh,s,gamma,seed", [
    (2, 12, 21, 30, 2, 0.9, 1), (1, 3, 4, 7, 3, 0.5, 2), (3, 5, 2, 2, 1, 2.0, 3),
    (1, 40, 8, 9, 4, 0.75, 4),
])
def test_repetitive_heads_bit_exact(B, H, T, gh, s, gamma, seed):
    g = torch.Generator().manual_seed(seed)
    base = torch.rand(1, H, 1, 1, generator=g)
    cos = (base + 0.2 * torch.rand(B, H, T, gh, generator=g)).clamp(max=1.0).float()
    flags = torch.empty(H, dtype=torch.uint8, device="cuda")
    bs.repetitive_heads(cos.cuda(), s, gamma, flags)
    torch.cuda.synchronize()
    assert np.array_equal(flags.cpu().numpy(), oracle.repetitive_heads(cos.numpy(), s, gamma))


@pytest.mark.parametrize("T,gh,gw,d,s,dt", [(2, 5, 3, 128, 2, torch.bfloat16),
                                            (21, 30, 52, 128, 2, torch.bfloat16),
                                            (3, 7, 4, 64, 3, torch.float32),
                                            (1, 4, 8, 8, 5, torch.bfloat16)])
def test_anchor_rows_gather_and_broadcast_bit_exact(T, gh, gw, d, s, dt):
    N = T * gh * gw
    x = torch.randn(2, 3, N, d, generator=torch.Generator().manual_seed(N)).to(dt)
    ga = torch.zeros_like(x).cuda()
    bs.anchor_rows(x.cuda(), ga, T, gh, gw, s)
    bc = torch.empty_like(ga)
    bs.anchor_rows(ga, bc, T, gh, gw, s, broadcast=True)
    torch.cuda.synchronize()
    na = T * oracle.anchor_count(gh, s) * gw
    want_g = oracle.gather_anchor_rows(x.float().numpy(), T, gh, gw, s)
    assert np.array_equal(ga[:, :, :na].cpu().float().numpy(), want_g)
    assert (ga[:, :, na:].cpu() == 0).all()                  # rows >= Na untouched
    want_b = oracle.broadcast_anchor_rows(want_g, T, gh, gw, s)
    assert np.array_equal(bc.cpu().float().numpy(), want_b)


@pytest.mark.parametrize("N,tile,qt", [(300, 64, 2), (1024, 128, 0), (1000, 128, 8)])
def test_dense_rows_masks(N, tile, qt):
    w = W.small_workload(frames=1, grid_h=1, grid_w=N, tile=tile,
                         mask=W.MaskSpec(W.MASK_DENSE_ROWS, query_tiles=qt))
    mask, rp, ci = gpu_mask_csr(w)
    check_mask_csr(w, mask, rp, ci)


@pytest.mark.parametrize("N,tile,qt,bt", [(1024, 128, 3, 2), (2000, 64, 7, 3), (1000, 128, 3, 2),
                                          (640, 64, 0, 1), (640, 64, 10, 1), (32760, 128, 128, 2),
                                          (131040, 128, 342, 2)])
def test_spread_dense_rows_masks(N, tile, qt, bt):
    w = W.small_workload(frames=1, grid_h=1, grid_w=N, tile=tile,
                         mask=W.MaskSpec(W.MASK_DENSE_ROWS_SPREAD, query_tiles=qt,
                                         block_tiles=bt))
    mask, rp, ci = gpu_mask_csr(w)
    check_mask_csr(w, mask, rp, ci)


@pytest.mark.parametrize("T,gh,gw,d,s,br,dt", [(2, 5, 3, 128, 2, 4, torch.bfloat16),
                                               (21, 30, 52, 128, 2, 256, torch.bfloat16),
                                               (3, 7, 4, 64, 3, 5, torch.float32),
                                               (4, 9, 10, 64, 3, 128, torch.bfloat16)])
def test_anchor_rows_spread_bit_exact(T, gh, gw, d, s, br, dt):
    """Gather into blocks of br rows spread over the buffer, and the
    broadcast back from that layout."""
    N = T * gh * gw
    x = torch.randn(2, 3, N, d, generator=torch.Generator().manual_seed(N + br)).to(dt)
    ga = torch.zeros_like(x).cuda()
    bs.anchor_rows(x.cuda(), ga, T, gh, gw, s, block_rows=br)
    bc = torch.empty_like(ga)
    bs.anchor_rows(ga, bc, T, gh, gw, s, broadcast=True, block_rows=br)
    torch.cuda.synchronize()
    na = T * oracle.anchor_count(gh, s) * gw
    rows = anchor_buffer_rows(na, N, br)
    want_g = oracle.gather_anchor_rows(x.float().numpy(), T, gh, gw, s)
    got = ga.cpu().float().numpy()
    assert np.array_equal(got[:, :, rows], want_g)
    rest = np.setdiff1d(np.arange(N), rows)
    assert (got[:, :, rest] == 0).all()                      # other rows untouched
    want_b = oracle.broadcast_anchor_rows(want_g, T, gh, gw, s)
    assert np.array_equal(bc.cpu().float().numpy(), want_b)


@pytest.mark.parametrize("T,gh,gw,d,s,tile,H", [(2, 6, 16, 128, 2, 128, 2),   # packed
                                                (3, 5, 20, 64, 2, 64, 1),
                                                (2, 9, 32, 128, 3, 64, 2),     # spread
                                                (6, 12, 20, 128, 3, 128, 2)])
def test_repeated_attention_full_parity(T, gh, gw, d, s, tile, H):
    N = T * gh * gw
    g = torch.Generator().manual_seed(N + s)
    q, k, v = (torch.randn(1, H, N, d, generator=g).to(torch.bfloat16) for _ in range(3))
    o = bs.repeated_attention(q.cuda(), k.cuda(), v.cuda(), T, gh, gw, s, tile)
    torch.cuda.synchronize()
    want = oracle.repeated_attention(q, k, v, T, gh, gw, s)
    assert_close(f"repeated T{T} {gh}x{gw} s{s} tile{tile}", to64(o), want)


def test_repeated_attention_video_shape():
    """21 x 30 x 52 latents, 12 heads, stride 2: every non-anchor row is a
    bitwise copy of its anchor row; sampled anchor rows match the oracle's
    full attention."""
    w = W.WORKLOADS[2]
    q, k, v = W.make_qkv(w)
    o = bs.repeated_attention(q.cuda(), k.cuda(), v.cuda(), w.frames, w.grid_h, w.grid_w, 2,
                              w.tile)
    torch.cuda.synchronize()
    ov = o.view(w.B, w.H, w.frames, w.grid_h, w.grid_w, w.d)
    assert torch.equal(ov[:, :, :, 1::2], ov[:, :, :, 0:-1:2])
    rows = np.array([f * w.P + y * w.grid_w + x for f in (0, 10, 20) for y in (0, 14, 28)
                     for x in (0, 25, 51)])
    dense = np.ones((1, w.num_tiles, w.num_tiles), dtype=np.uint8)
    want, _ = oracle.block_sparse_attention_rows(q, k, v, dense, w.tile, rows, workers=16)
    assert_close("repeated 21x30x52 anchor rows", to64(o[:, :, rows]), want)


@pytest.mark.parametrize("T,gh,gw,d,s,dt", [(2, 5, 3, 128, 2, torch.bfloat16),
                                            (3, 7, 4, 64, 3, torch.float32)])
def test_anchor_rows_heads_bit_exact(T, gh, gw, d, s, dt):
    """Per-head gather and broadcast: flagged heads as bsattn_anchor_rows
    (spread layout), the others copied row for row."""
    from layout_contract import anchor_buffer_rows
    N = T * gh * gw
    H = 4
    x = torch.randn(2, H, N, d, generator=torch.Generator().manual_seed(N)).to(dt)
    flags = torch.tensor([1, 0, 0, 1], dtype=torch.uint8, device="cuda")
    br = 4
    ga = torch.full_like(x, -7.0).cuda()
    bs.anchor_rows(x.cuda(), ga, T, gh, gw, s, block_rows=br, flags=flags)
    bc = torch.empty_like(ga)
    bs.anchor_rows(ga, bc, T, gh, gw, s, broadcast=True, block_rows=br, flags=flags)
    torch.cuda.synchronize()
    na = T * oracle.anchor_count(gh, s) * gw
    rows = anchor_buffer_rows(na, N, br)
    xf = x.float().numpy()
    got = ga.cpu().float().numpy()
    for h in range(H):
        if flags[h]:
            want = oracle.gather_anchor_rows(xf[:, h], T, gh, gw, s)
            assert np.array_equal(got[:, h][:, rows], want)
            rest = np.setdiff1d(np.arange(N), rows)
            assert (got[:, h][:, rest] == -7.0).all()          # not written
            wb = oracle.broadcast_anchor_rows(want, T, gh, gw, s)
            assert np.array_equal(bc.cpu().float().numpy()[:, h], wb)
        else:
            assert np.array_equal(got[:, h], xf[:, h])
            assert np.array_equal(bc.cpu().float().numpy()[:, h], xf[:, h])


def test_mask_select_bit_exact():
    g = torch.Generator().manual_seed(4)
    H, Tq, Tk = 5, 9, 11
    a = (torch.rand(1, Tq, Tk, generator=g) < 0.5).to(torch.uint8)
    b = (torch.rand(H, Tq, Tk, generator=g) < 0.5).to(torch.uint8)
    f = torch.tensor([0, 1, 1, 0, 1], dtype=torch.uint8)
    out = torch.empty(H, Tq, Tk, dtype=torch.uint8, device="cuda")
    bs.mask_select(f.cuda(), a.cuda(), b.cuda(), out)
    torch.cuda.synchronize()
    want = np.where(f.numpy()[:, None, None] != 0, a.numpy(), b.numpy())
    assert np.array_equal(out.cpu().numpy(), want)


def _mixed_case(T, gh, gw, H, s, flags, p, seed, tile=128):
    N = T * gh * gw
    g = torch.Generator().manual_seed(seed)
    q, k, v = (torch.randn(1, H, N, 128, generator=g).to(torch.bfloat16) for _ in range(3))
    Tn = -(-N // tile)
    cal = oracle.tile_mask_static(H, Tn, Tn, seed, W.thresh24_for_density(p), True)
    f = torch.tensor(flags, dtype=torch.uint8, device="cuda")
    rp, ci, mm = bs.mixed_layer_csr(f, torch.from_numpy(cal).cuda(), T, gh, gw, s, tile)
    o = bs.mixed_attention(q.cuda(), k.cuda(), v.cuda(), f, rp, ci, T, gh, gw, s, tile)
    torch.cuda.synchronize()
    return q, k, v, cal, o, mm


@pytest.mark.parametrize("T,gh,gw,H,s,flags,p", [
    (3, 9, 16, 4, 2, [1, 0, 1, 0], 0.4),
    (2, 12, 20, 3, 3, [0, 1, 1], 0.3),
    (4, 6, 30, 2, 2, [0, 0], 0.5),
    (2, 7, 18, 2, 2, [1, 1], 0.5),
])
def test_mixed_layer_against_the_oracle(T, gh, gw, H, s, flags, p):
    """CalibAtt's inference layer (CalibAtt page, "B. Fase di Inferenza"):
    flagged heads on anchor rows, copied; the others on their block lists;
    one forward for all heads.  Against the oracle's composition, every
    element; the mixed mask bit-exact."""
    from layout_contract import spread_dense_rows_mask
    q, k, v, cal, o, mm = _mixed_case(T, gh, gw, H, s, flags, p, seed=T * gh + H)
    N = T * gh * gw
    na = T * oracle.anchor_count(gh, s) * gw
    rows_mask = spread_dense_rows_mask(1, N, 128, -(-na // 128), 2)
    want_mask = np.where(np.array(flags)[:, None, None] != 0, rows_mask, cal)
    assert np.array_equal(mm.cpu().numpy(), want_mask)
    want = oracle.mixed_heads_attention(q, k, v, flags, cal, 128, T, gh, gw, s)
    assert_close(f"mixed layer {T}x{gh}x{gw} flags {flags}", to64(o), want)


@pytest.mark.timeout(600)
def test_mixed_layer_video_shape():
    """21 x 30 x 52 latents, 12 heads, stride 2, flags on six heads, a
    per-head static mask (p = 0.3) for the others: sampled rows of every
    query tile against the oracle; flagged heads' rows copy their anchors
    bitwise."""
    flags = [1, 0] * 6
    q, k, v, cal, o, _ = _mixed_case(21, 30, 52, 12, 2, flags, 0.3, seed=21)
    N = q.shape[2]
    ov = o.view(1, 12, 21, 30, 52, 128)
    for h in range(0, 12, 2):
        assert torch.equal(ov[:, h, :, 1::2], ov[:, h, :, 0:-1:2])
    rows = np.concatenate([np.arange(t * 128, min(t * 128 + 128, N))[[0, 57, -1]]
                           for t in range(-(-N // 128))])
    want = oracle.mixed_heads_attention_rows(q, k, v, flags, cal, 128, 21, 30, 52, 2, rows,
                                             workers=16)
    assert_close("mixed layer 21x30x52 (3 rows of every tile, 12 heads)",
                 to64(o[:, :, torch.from_numpy(rows).cuda()]), want)
