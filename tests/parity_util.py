"""Shared helpers of the GPU parity tests: run the library on a workload and
compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_attention_bsattn_amd as bs
import oracle

# the output bar (bf16 I/O, fp32 accumulation)
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def oracle_mask(w, rotation=None):
    """The expected tile mask of workload w: the oracle's, or for the anchor-
    row layouts (dense-rows kinds, not masks of the method) the library's
    stated layout contract."""
    s = w.mask
    if s.kind in (5, 6):
        from layout_contract import dense_rows_mask, spread_dense_rows_mask
        if s.kind == 5:
            return dense_rows_mask(s.mask_heads, w.N, w.tile, s.query_tiles)
        return spread_dense_rows_mask(s.mask_heads, w.N, w.tile, s.query_tiles,
                                      s.block_tiles)
    return oracle.tile_mask(s.kind, w.frames, w.grid_h, w.grid_w, w.tile,
                            window=s.window, num_anchors=s.num_anchors,
                            rotation=s.rotation if rotation is None else rotation,
                            seed=s.seed, thresh24=s.thresh24,
                            force_diagonal=s.force_diagonal,
                            mask_heads=s.mask_heads, budget=s.budget,
                            block_tiles=s.block_tiles,
                            query_tiles=s.query_tiles)


def gpu_mask_csr(w, device="cuda"):
    mask = bs.make_mask(w.frames, w.grid_h, w.grid_w, w.tile, device=device,
                        **bs.mask_params_of(w.mask))
    row_ptr, col_idx = bs.make_csr(mask)
    return mask, row_ptr, col_idx


def check_mask_csr(w, mask, row_ptr, col_idx):
    """Bit-exact comparison of the GPU mask and CSR with the oracle's (the
    layout contract's for the dense-rows kinds)."""
    m_ref = oracle_mask(w)
    m = mask.cpu().numpy()
    assert m.shape == m_ref.shape
    assert np.array_equal(m, m_ref), f"{w.name}: mask differs in " \
        f"{int((m != m_ref).sum())} cells"
    rp_ref, ci_ref = oracle.tile_csr(m_ref)
    rp = row_ptr.cpu().numpy()
    assert np.array_equal(rp, rp_ref), f"{w.name}: row_ptr differs"
    nnz = int(rp_ref[-1])
    assert np.array_equal(col_idx[:nnz].cpu().numpy(), ci_ref), \
        f"{w.name}: col_idx differs"
    return m_ref


def errors(o_gpu, o_ref):
    d = np.abs(o_gpu.astype(np.float64) - o_ref)
    fro = np.linalg.norm(o_ref.ravel())
    rel = float(np.linalg.norm(d.ravel()) / fro) if fro > 0 else float(d.max())
    return float(d.max()), float(d.mean()), rel


def to64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


# fp32 accumulation, the hardware exponential and reassociation: what the
# log-sum-exp may differ by beyond the input-rounding term below
LSE_BASE = 3e-4


def lse_tolerance(q, k, mask, tile, rows=None, workers=8):
    """Per-row bound on |LSE_gpu - LSE_oracle| for bf16 inputs, [B, H, R].

    The tuned kernel multiplies Q by scale*log2(e) as it loads it and rounds
    the product to bf16, so score j of row n carries
        dx_j = scale * sum_i e_i q_i k_ji,   |e_i| <= 2^-9
    (one bf16 rounding per element of q).  The log-sum-exp moves by the
    attention-weighted mean of these, dLSE = scale * sum_i e_i q_i kbar_i with
    kbar = sum_j p_j k_j, so
        |dLSE| <= 2^-9 * scale * sum_i |q_i| |kbar_i|.
    kbar is the oracle's attention output with V := K.  A missing or extra
    tile moves LSE by about ln(1 +- 1/tiles_in_row), far above this bound
    wherever attention is spread over many keys."""
    N = q.shape[2]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    kbar, _ = oracle.block_sparse_attention_rows(q.cpu(), k.cpu(), k.cpu(), mask,
                                                 tile, rows, workers=workers)
    q64 = q.detach().cpu().to(torch.float64).numpy()[:, :, rows]
    scale = 1.0 / np.sqrt(q.shape[-1])
    return LSE_BASE + 2.0 ** -9 * scale * (np.abs(q64) * np.abs(kbar)).sum(-1)


def oracle_rows_and_lse_tol(q, k, v, mask, tile, rows=None, workers=16):
    """The oracle's O and LSE for the query rows `rows` (all rows if None),
    and the per-row LSE bound of `lse_tolerance`, from one oracle pass: the
    attention weights do not depend on the values, so attending over the
    values [V | K] gives O in the first d columns and kbar in the rest."""
    N, d = q.shape[2], q.shape[3]
    rows = np.arange(N) if rows is None else np.asarray(rows)
    vk = torch.cat([v.cpu(), k.cpu()], dim=-1)
    o2, lse = oracle.block_sparse_attention_rows(q.cpu(), k.cpu(), vk, mask, tile,
                                                 rows, workers=workers)
    q64 = q.detach().cpu().to(torch.float64).numpy()[:, :, rows]
    scale = 1.0 / np.sqrt(d)
    tol = LSE_BASE + 2.0 ** -9 * scale * (np.abs(q64) * np.abs(o2[..., d:])).sum(-1)
    return o2[..., :d], lse, tol


def assert_close(name, o_gpu, o_ref, lse_gpu=None, lse_ref=None,
                 lse_tol=None):
    mx, mean, rel = errors(o_gpu, o_ref)
    msg = f"{name}: max|err| {mx:.3e} mean|err| {mean:.3e} rel-fro {rel:.3e}"
    print(msg, flush=True)
    assert np.isfinite(o_gpu).all(), name + ": non-finite output"
    assert mx <= MAX_ABS and mean <= MEAN_ABS, msg
    if lse_gpu is not None:
        assert lse_tol is not None, name + ": an LSE check needs a tolerance"
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse_gpu), fin), name + ": lse -inf rows"
        assert np.array_equal(lse_gpu[~fin], lse_ref[~fin])
        if fin.any():
            tol = np.broadcast_to(np.asarray(lse_tol, dtype=np.float64),
                                  lse_ref.shape)
            dl = np.abs(lse_gpu - np.where(fin, lse_ref, 0.0))
            worst = float((dl[fin] / tol[fin]).max())
            print(f"{name}: max|dlse| {float(dl[fin].max()):.3e}, "
                  f"worst |dlse|/tol {worst:.3f}", flush=True)
            assert worst <= 1.0, f"{name}: |dlse| over tolerance ({worst:.3f}x)"
