"""GPU static-mask calibration against the oracle (CalibAtt page,
"A. Fase di Calibrazione"): block energies within a tolerance derived from
the arithmetic, selection and aggregation bit-exact on the same seeded
inputs, and the end-to-end calibrated mask driving the forward."""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_bsattn_amd as bs
import oracle
import workloads as W
from parity_util import assert_close, to64

pytestmark = pytest.mark.gpu

# Energies: every probability carries fp32 rounding from the score sum, the
# exponent arithmetic and v_exp (a few ulp each), and the row's normaliser
# is a float sum of up to 2 * T per-tile partials of 16 terms each per lane
# (relative error below (16 + 2T) * 2^-24, 3e-5 at T = 256, in the worst
# case), so each block sum is within about 1e-4 relative of the exact value.
E_RTOL = 1e-4
E_ATOL = 1e-5


def _gpu_energy(q, k, tile, one_sweep=True):
    B, H, N, d = q.shape
    t = bs.num_tiles(N, tile)
    e = torch.empty((B, H, t, t), dtype=torch.float32, device="cuda")
    bs.block_energy(q, k, e, tile, one_sweep=one_sweep)
    torch.cuda.synchronize()
    return e


def _check_energy(name, got, want, rows_per_tile=None):
    got = got.astype(np.float64)
    err = np.abs(got - want)
    bound = E_RTOL * np.abs(want) + E_ATOL
    worst = float((err / bound).max())
    print(f"{name}: max|dE| {err.max():.3e} worst/bound {worst:.3f}", flush=True)
    assert np.isfinite(got).all(), name
    assert worst <= 1.0, f"{name}: energy error over tolerance ({worst:.2f}x)"


@pytest.mark.parametrize("N,d,tile,dtype,B,H", [
    (700, 128, 128, W.DTYPE_BF16, 2, 2),   # several tiles, ragged tail
    (513, 64, 64, W.DTYPE_BF16, 1, 3),
    (384, 128, 64, W.DTYPE_BF16, 1, 1),    # exact tiles
    (300, 64, 128, W.DTYPE_F32, 2, 1),     # fp32 inputs
    (1, 128, 128, W.DTYPE_BF16, 1, 1),     # one token
    (640, 128, 128, W.DTYPE_BF16, 1, 3),   # odd tile count: the last pair's second tile is absent
    (1100, 128, 128, W.DTYPE_BF16, 2, 1),  # odd and ragged
    (700, 128, 128, W.DTYPE_F32, 1, 1),    # fp32 inputs, d 128: the generic kernel
])
@pytest.mark.parametrize("one_sweep", [True, False])
def test_block_energy_small(N, d, tile, dtype, B, H, one_sweep):
    """Both kernels of the tuned instance (one sweep with a workspace, two
    without) and the generic kernel against the oracle."""
    w = W.small_workload(frames=1, grid_h=1, grid_w=N, tile=tile, d=d, H=H, B=B,
                         dtype=dtype, seed=zlib.crc32(f"{N}{d}{tile}".encode()) & 0xFFFF)
    q, k = W.make_qk_frame_local(w, strength=1.0)
    e = _gpu_energy(q.cuda(), k.cuda(), tile, one_sweep).cpu().numpy()
    # the library rounds fp32 inputs to bf16 for the products (its contract);
    # the oracle gets those rounded values
    qo, ko = (q, k) if dtype == W.DTYPE_BF16 else (q.to(torch.bfloat16), k.to(torch.bfloat16))
    want = oracle.block_energy(qo, ko, tile)
    _check_energy(f"N={N} d={d} tile={tile} one sweep {one_sweep}", e, want)
    rows = np.minimum(tile, N - np.arange(e.shape[-1]) * tile)
    np.testing.assert_allclose(e.sum(-1), np.broadcast_to(rows, e.shape[:-1]), rtol=2e-5)


@pytest.mark.parametrize("one_sweep", [True, False])
@pytest.mark.parametrize("jump", [20.0, 60.0, 200.0])
def test_block_energy_score_jumps(jump, one_sweep):
    """Scores jump by `jump` (log2 units) at a late key tile: the running
    max of the first sweep grows long after the first tile, by less (20) or
    more (60, 200: the tile is redone against its exact max) than the
    rescaling limit; the energy moves onto that tile.  In one sweep the
    redo also rescales the tile sums already in the workspace."""
    B, H, N, d, tile = 1, 2, 1000, 128, 128
    g = torch.Generator().manual_seed(78)
    u = torch.randn(d, generator=g)
    u = u / u.norm()
    q = torch.randn(B, H, N, d, generator=g) * 0.3 + 1.0 * u
    k = torch.randn(B, H, N, d, generator=g) * 0.3
    k[:, :, 5 * 128 + 3:5 * 128 + 40] += (jump / 1.4426950408889634) * u
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    t = bs.num_tiles(N, tile)
    e = torch.empty((B, H, t, t), dtype=torch.float32, device="cuda")
    bs.block_energy(q.cuda(), k.cuda(), e, tile, scale=1.0, one_sweep=one_sweep)
    torch.cuda.synchronize()
    want = oracle.block_energy(q, k, tile, scale=1.0)
    _check_energy(f"score jump {jump} one sweep {one_sweep}", e.cpu().numpy(), want)


def test_block_energy_full_size_sampled_rows():
    """The 32 760-token calibration shape: every row sums to its query rows;
    sampled query tiles (first, last, and spread) against the oracle."""
    w = W.CALIB
    q, k = W.make_qk_frame_local(w, strength=1.0)
    T = w.num_tiles
    rows = np.minimum(w.tile, w.N - np.arange(T) * w.tile)
    pick = [0, 1, 97, 128, 200, T - 1]
    want = oracle.block_energy_rows(q[:2, :3], k[:2, :3], w.tile, pick)
    qc, kc = q.cuda(), k.cuda()
    for one_sweep in (True, False):   # 6144 pairs over 512 persistent workgroups; one each
        e = _gpu_energy(qc, kc, w.tile, one_sweep).cpu().numpy()
        np.testing.assert_allclose(e.sum(-1), np.broadcast_to(rows, e.shape[:-1]),
                                   rtol=E_RTOL)
        _check_energy(f"video shape, one sweep {one_sweep}, 6 query tiles x 2 prompts x "
                      "3 heads", e[:2, :3][:, :, pick], want)


@pytest.mark.parametrize("rows,tk,eps,seed", [
    (300, 256, 0.9, 1), (64, 1024, 0.95, 2), (40, 7, 0.5, 3), (5, 1, 0.9, 4),
    (100, 300, 1.0, 5), (100, 300, 0.0, 6), (100, 300, 1.5, 7), (8, 4096, 0.8, 8),
    (1000, 64, 0.3, 9),
])
def test_select_blocks_bit_exact(rows, tk, eps, seed):
    e = W.make_energies(rows, tk, seed)
    e[0] = 0.0                                   # an all-zero row
    m = torch.empty((rows, tk), dtype=torch.uint8, device="cuda")
    bs.select_blocks(e.cuda(), eps, m)
    torch.cuda.synchronize()
    want = oracle.select_mask(e.numpy(), eps)
    got = m.cpu().numpy()
    assert np.array_equal(got, want), f"{int((got != want).sum())} cells differ"


@pytest.mark.parametrize("P,cells,rho,seed", [
    (4, 12 * 256 * 256, 0.5, 1), (1, 1000, 0.5, 2), (64, 5000, 0.51, 3),
    (3, 777, 0.0, 4), (3, 777, 1.0, 5), (3, 777, 1.5, 6),
])
def test_aggregate_bit_exact(P, cells, rho, seed):
    m = W.make_prompt_masks(P, cells, seed)
    out = torch.empty(cells, dtype=torch.uint8, device="cuda")
    bs.aggregate_masks(m.cuda(), rho, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), oracle.aggregate(m.numpy(), rho))


def _decision_margin(e_row, eps):
    """Relative distance of the selection's stopping decision from the
    threshold (large = no fp32 rounding of the energies can change it)."""
    e = np.sort(np.asarray(e_row, dtype=np.float64))[::-1]
    total = e.sum()
    if total <= 0:
        return np.inf
    cum = np.concatenate([[0.0], np.cumsum(e)])
    return float(np.min(np.abs(cum - eps * total)) / total)


def test_calibration_end_to_end_small():
    """Energies -> per-prompt selection -> agreement -> compact -> forward on
    a small frame-local workload.  The selection is compared with the
    oracle's on every row whose decision is farther from the threshold than
    the energies' error (there the result is unique); the agreement is
    checked as counts; the forward runs on the calibrated mask and matches
    the oracle on the same mask where the two masks agree."""
    w = W.small_workload(frames=10, grid_h=5, grid_w=16, tile=128, d=128, H=2, B=4,
                         seed=4242)
    q, k = W.make_qk_frame_local(w, strength=0.7)
    # V at half scale: the peaked attention of this case sends |O| towards
    # max |V|, and O's bf16 rounding (half an ulp, 2^-7 at |O| in [1, 2))
    # should stay well inside the 1e-2 bar
    v = (0.5 * torch.randn(q.shape, generator=torch.Generator().manual_seed(7))).to(torch.bfloat16)
    eps, rho = 0.9, 0.5
    mask, energy, sel = bs.calibrate(q.cuda(), k.cuda(), w.tile, eps, rho)
    torch.cuda.synchronize()
    E_ref = oracle.block_energy(q, k, w.tile)
    sel_ref = oracle.select_mask(E_ref.astype(np.float32), eps)
    sel_gpu = sel.cpu().numpy()
    unique = np.zeros(E_ref.shape[:-1], dtype=bool)
    for idx in np.ndindex(E_ref.shape[:-1]):
        unique[idx] = _decision_margin(E_ref[idx], eps) > 1e-3
    # this seeded case has every decision at least 1.7e-3 of the row total
    # from the threshold, 17x the energies' tolerance: the selection is unique
    assert unique.all()
    assert np.array_equal(sel_gpu, sel_ref)
    counts = sel_gpu.astype(int).sum(axis=0)
    assert np.array_equal(mask.cpu().numpy(), (counts >= rho * w.B).astype(np.uint8))
    # the frame-local structure shows: fewer than all blocks are kept
    density = float(mask.float().mean())
    print(f"calibrated density {density:.3f}", flush=True)
    assert 0.05 < density < 0.95
    # forward on the calibrated mask (shared by the batch, per head)
    rp, ci = bs.make_csr(mask)
    o, lse = bs.attention(q.cuda(), k.cuda(), v.cuda(), rp, ci, w.tile,
                          mask_heads=w.H, want_lse=True)
    torch.cuda.synchronize()
    m_ref = oracle.aggregate(sel_ref, rho)
    assert np.array_equal(m_ref, mask.cpu().numpy())
    o_ref, lse_ref = oracle.block_sparse_attention(q, k, v, m_ref, w.tile)
    assert_close("calibrated forward", to64(o), o_ref)
