"""bsattn_fwd_noalloc (the forward that allocates nothing: its plan lives in
the library's own device array) against bsattn_fwd, through the C ABI: two
calls in a row, the second on a smaller input, each compared with
bsattn_fwd's output element by element within the output bar (max |err| <=
1e-2, mean |err| <= 1e-3), and bit for bit with bsattn_fwd_planned through
a plan of the caller's (the same kernels); sizes beyond the array are
refused before anything runs."""
import ctypes

import numpy as np
import pytest
import torch

import block_sparse_attention_bsattn_amd as bs
import workloads as W
from parity_util import MAX_ABS, MEAN_ABS, gpu_mask_csr

pytestmark = pytest.mark.gpu


def _noalloc(q, k, v, o, lse, rp, ci, tile, Hm):
    B, H, N, d = q.shape
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    dt = bs.DTYPE_BF16 if q.dtype == torch.bfloat16 else bs.DTYPE_F32
    return bs.lib().bsattn_fwd_noalloc(B, H, N, d, tile, dt, p(q), p(k), p(v), p(o), p(lse),
                                      Hm, p(rp), p(ci), 0.0,
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def _compare(name, w):
    mask, rp, ci = gpu_mask_csr(w)
    q, k, v = W.make_qkv(w, device="cuda")
    Hm = w.mask.mask_heads
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    assert _noalloc(q, k, v, o, lse, rp, ci, w.tile, Hm) == bs.OK, bs.lib().bsattn_last_error()
    o_ref, lse_ref = bs.attention(q, k, v, rp, ci, w.tile, mask_heads=Hm, want_lse=True)
    planned = w.d == 128 and w.tile == 128 and w.dtype == W.DTYPE_BF16
    if planned:
        o_pl, lse_pl = bs.attention_planned(q, k, v, rp, ci, mask_heads=Hm, want_lse=True)
    torch.cuda.synchronize()
    d = (o.double() - o_ref.double()).abs()
    print(f"{name}: max|dO| {d.max().item():.3e} mean {d.mean().item():.3e}", flush=True)
    assert d.max().item() <= MAX_ABS and d.mean().item() <= MEAN_ABS
    fin = torch.isfinite(lse_ref)
    assert torch.equal(torch.isfinite(lse), fin)
    assert (lse[fin] - lse_ref[fin]).abs().max().item() <= 2e-2
    if planned:
        assert torch.equal(o, o_pl)
        assert torch.equal(lse.view(torch.int32), lse_pl.view(torch.int32))
    else:
        assert torch.equal(o, o_ref)


def test_two_calls_in_a_row_the_second_smaller():
    big = W.WORKLOADS[2].with_rotation(4)              # 32 760 tokens, 12 heads
    small = W.small_workload(frames=5, grid_h=9, grid_w=26, tile=128, d=128, H=3, B=2,
                             mask=W.MaskSpec(W.MASK_STATIC_RANDOM, seed=5,
                                             thresh24=W.thresh24_for_density(0.3),
                                             force_diagonal=1, mask_heads=3),
                             name="noalloc_small")
    _compare("noalloc 32 760 tokens", big)
    _compare("noalloc smaller, per-head static", small)


def test_other_shapes_and_sizes_beyond_the_array():
    # d 64: bsattn_fwd's kernels, no scratch
    w = W.small_workload(frames=3, grid_h=5, grid_w=9, tile=64, d=64, H=2)
    _compare("noalloc d64 tile64", w)
    # a plan above the array: refused on the host, nothing enqueued
    p = ctypes.c_void_p(64)
    st = bs.lib().bsattn_fwd_noalloc(4, 40, 131072, 128, 128, bs.DTYPE_BF16, p, p, p, p,
                                    None, 1, p, p, 0.0, None)
    assert st == bs.ERR_INVALID_ARG
    assert b"device scratch" in bs.lib().bsattn_last_error()
