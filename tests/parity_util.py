"""Shared helpers of the GPU parity tests: run the library on a workload and
compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_attention_bsattn_amd as bs
import oracle

# spec gates for the output (bf16 I/O, fp32 accumulation)
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def oracle_mask(w, rotation=None):
    s = w.mask
    return oracle.tile_mask(s.kind, w.frames, w.grid_h, w.grid_w, w.tile,
                            window=s.window, num_anchors=s.num_anchors,
                            rotation=s.rotation if rotation is None else rotation,
                            seed=s.seed, thresh24=s.thresh24,
                            force_diagonal=s.force_diagonal,
                            mask_heads=s.mask_heads, budget=s.budget)


def gpu_mask_csr(w, device="cuda"):
    mask = bs.make_mask(w.frames, w.grid_h, w.grid_w, w.tile, device=device,
                        **bs.mask_params_of(w.mask))
    row_ptr, col_idx = bs.make_csr(mask)
    return mask, row_ptr, col_idx


def check_mask_csr(w, mask, row_ptr, col_idx):
    """Bit-exact comparison of the GPU mask and CSR with the oracle's."""
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


def assert_close(name, o_gpu, o_ref, lse_gpu=None, lse_ref=None,
                 lse_tol=1e-3):
    mx, mean, rel = errors(o_gpu, o_ref)
    msg = f"{name}: max|err| {mx:.3e} mean|err| {mean:.3e} rel-fro {rel:.3e}"
    print(msg, flush=True)
    assert np.isfinite(o_gpu).all(), name + ": non-finite output"
    assert mx <= MAX_ABS and mean <= MEAN_ABS, msg
    if lse_gpu is not None:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse_gpu), fin), name + ": lse -inf rows"
        assert np.array_equal(lse_gpu[~fin], lse_ref[~fin])
        if fin.any():
            dl = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max())
            assert dl <= lse_tol, f"{name}: max|dlse| {dl:.3e}"
