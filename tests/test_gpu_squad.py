"""GPU SQuad two-pass attention (SQuad page, "1. Operatore di Attenzione
SQuad") against the oracle: the block-diagonal masks and the token reorder
bit-exact, the composed operator within the output bar."""
import zlib

import numpy as np
import pytest
import torch

import block_sparse_attention_bsattn_amd as bs
import oracle
import workloads as W
from parity_util import assert_close, check_mask_csr, gpu_mask_csr, to64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("N,tile,b", [(300, 64, 2), (1024, 128, 1), (4096, 64, 8),
                                      (65536, 128, 2), (1000, 128, 3)])
def test_block_diagonal_masks(N, tile, b):
    w = W.small_workload(frames=1, grid_h=1, grid_w=N, tile=tile,
                         mask=W.MaskSpec(W.MASK_BLOCK_DIAGONAL, block_tiles=b))
    mask, rp, ci = gpu_mask_csr(w)
    check_mask_csr(w, mask, rp, ci)


@pytest.mark.parametrize("N,d,w,dt", [(64, 128, 8, torch.bfloat16), (96, 64, 96, torch.float32),
                                      (4096, 128, 64, torch.bfloat16), (30, 8, 1, torch.bfloat16)])
def test_window_reorder_bit_exact(N, d, w, dt):
    g = torch.Generator().manual_seed(N + w)
    x = torch.randn(2, 3, N, d, generator=g).to(dt)
    fwd = torch.empty_like(x.cuda())
    bs.window_reorder(x.cuda(), fwd, w)
    back = torch.empty_like(fwd)
    bs.window_reorder(fwd, back, w, inverse=True)
    torch.cuda.synchronize()
    want = oracle.window_major_to_position_major(x.float().numpy(), w)
    assert np.array_equal(fwd.cpu().float().numpy(), want)
    assert torch.equal(back.cpu(), x)


@pytest.mark.parametrize("N,d,w,tile,H", [(4096, 64, 64, 64, 2), (16384, 128, 128, 128, 2),
                                          (32768, 128, 256, 128, 1), (8192, 128, 128, 64, 1)])
def test_squad_full_parity(N, d, w, tile, H):
    g = torch.Generator().manual_seed(zlib.crc32(f"{N}{w}".encode()) & 0xFFFF)
    q, k, v = (torch.randn(1, H, N, d, generator=g).to(torch.bfloat16) for _ in range(3))
    o = bs.squad(q.cuda(), k.cuda(), v.cuda(), w, tile)
    torch.cuda.synchronize()
    want = oracle.squad_attention(q, k, v, w)
    assert_close(f"squad N={N} w={w} tile={tile}", to64(o), want)


def test_squad_full_size_sampled_rows():
    """65 536 tokens, w = 256: sampled rows against the oracle, for every
    head: six positions (first, last and inside a window) in ten windows
    (first, last and spread), so six global position groups are evaluated."""
    w = W.SQUAD
    q, k, v = W.make_qkv(w)
    o = bs.squad(q.cuda(), k.cuda(), v.cuda(), W.SQUAD_W, w.tile)
    torch.cuda.synchronize()
    G = w.N // W.SQUAD_W
    pos = np.array([0, 1, 77, 128, 200, W.SQUAD_W - 1])
    win = np.array([0, 1, 31, 64, 100, 127, 128, 190, 230, G - 1])
    rows = np.sort((win[:, None] * W.SQUAD_W + pos[None, :]).ravel())
    want = oracle.squad_attention_rows(q, k, v, W.SQUAD_W, rows)
    assert_close(f"squad 65536 ({len(rows)} rows x {w.H} heads)", to64(o[:, :, rows]), want)


def test_squad_rejects_misaligned_windows():
    q = torch.zeros(1, 1, 1000, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        bs.squad(q, q, q, 100, 64)


@pytest.mark.parametrize("N,w,H,B,mask", [(32768, 256, 2, 1, "block"), (16384, 128, 2, 2, "block"),
                                          (16384, 1, 1, 1, "static"),
                                          (32768, 256, 12, 1, "static_h"),
                                          (16384, 64, 3, 2, "static_h"),
                                          (65536, 512, 1, 1, "dense"),
                                          (16384, 128, 3, 1, "empty")])
def test_fwd_grouped_equals_reorder_fwd_reorder(N, w, H, B, mask):
    """bsattn_fwd_grouped gives, bit for bit, what the window reorder of q,
    k and v, bsattn_fwd and the inverse reorder of o and lse give, for
    block-diagonal (SQuad's global pass), static (one mask and one per
    head), dense and empty masks; w = 1 is the identity view."""
    g = torch.Generator().manual_seed(N + w + H + B)
    q, k, v = (torch.randn(B, H, N, 128, generator=g).to(torch.bfloat16).cuda()
               for _ in range(3))
    G = N // w
    T = N // 128
    hm = H if mask == "static_h" else 1
    if mask == "block":
        m = bs.make_mask(1, 1, N, 128, kind=W.MASK_BLOCK_DIAGONAL, block_tiles=G // 128)
    elif mask in ("static", "static_h"):
        m = bs.make_mask(1, 1, N, 128, kind=W.MASK_STATIC_RANDOM, seed=7,
                         thresh24=W.thresh24_for_density(0.2), force_diagonal=1, mask_heads=hm)
    elif mask == "dense":
        m = bs.make_mask(1, 1, N, 128, kind=W.MASK_DENSE)
    else:
        m = torch.zeros(1, T, T, dtype=torch.uint8, device="cuda")
    rp, ci = bs.make_csr(m)
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    bs.fwd_grouped(q, k, v, o, rp, ci, w, mask_heads=hm, lse=lse)
    qp, kp, vp = (torch.empty_like(x) for x in (q, k, v))
    for src, dst in ((q, qp), (k, kp), (v, vp)):
        bs.window_reorder(src, dst, w)
    op = torch.empty_like(q)
    lp = torch.empty_like(lse)
    bs.fwd(qp, kp, vp, op, rp, ci, 128, mask_heads=hm, lse=lp)
    ref = torch.empty_like(op)
    bs.window_reorder(op, ref, w, inverse=True)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    lref = lp.view(B, H, w, G).transpose(2, 3).reshape(B, H, N)   # position-major -> buffer
    assert torch.equal(lse, lref)
    if mask == "empty":
        assert (o == 0).all() and torch.isinf(lse).all()


def test_squad_grouped_equals_reordered_path():
    w = W.SQUAD
    q, k, v = W.make_qkv(w)
    q, k, v = q.cuda(), k.cuda(), v.cuda()
    a = bs.squad(q, k, v, W.SQUAD_W, w.tile, grouped=True)
    b = bs.squad(q, k, v, W.SQUAD_W, w.tile, grouped=False)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
