"""GPU mask builder and compaction against the oracle, bit-exact."""
import numpy as np
import pytest
import torch

import block_sparse_attention_bsattn_amd as bs
import oracle
import workloads as W
from conftest import read_golden
from parity_util import check_mask_csr, gpu_mask_csr

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_configs_every_rotation(cfg):
    w = W.WORKLOADS[cfg]
    for r in w.rotations:
        wr = w.with_rotation(r)
        mask, rp, ci = gpu_mask_csr(wr)
        check_mask_csr(wr, mask, rp, ci)


def test_rotation_reduced_mod_T():
    w = W.WORKLOADS[2]
    for r in (-1, 21, 21 * 5 + 4, -22):
        wr = w.with_rotation(r)
        mask, rp, ci = gpu_mask_csr(wr)
        check_mask_csr(wr, mask, rp, ci)


def test_hand_enumerated_misaligned_layout():
    lines = read_golden("misaligned_window_anchor_mask.txt")
    hdr = lines[0].split()
    kv = dict(zip(hdr[0::2], map(int, hdr[1::2])))
    want = np.array([[int(c) for c in ln] for ln in lines[1:]], dtype=np.uint8)
    mask = bs.make_mask(kv["frames"], kv["grid_h"], kv["grid_w"], kv["tile"],
                        kind=0, window=kv["window"], num_anchors=kv["anchors"],
                        rotation=kv["rotation"])
    assert np.array_equal(mask.cpu().numpy()[0], want)


@pytest.mark.parametrize("T,gh,gw,BT,w,na,r,hm", [
    (5, 1, 3, 2, 1, 2, 3, 1), (7, 1, 5, 4, 0, 2, 6, 2), (9, 3, 3, 5, 2, 3, 7, 1),
    (3, 1, 7, 3, 0, 0, 0, 1), (8, 1, 3, 16, 1, 2, 5, 3), (33, 4, 5, 64, 3, 5, 11, 1),
    (13, 30, 52, 128, 0, 13, 2, 1), (40, 2, 2, 1, 2, 4, 9, 1),
])
def test_window_anchor_odd_layouts(T, gh, gw, BT, w, na, r, hm):
    wl = W.small_workload(frames=T, grid_h=gh, grid_w=gw, tile=BT,
                          mask=W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=w,
                                          num_anchors=na, rotation=r,
                                          mask_heads=hm))
    mask, rp, ci = gpu_mask_csr(wl)
    check_mask_csr(wl, mask, rp, ci)


@pytest.mark.parametrize("hm,seed,p,diag", [(1, 0, 0.5, 0), (3, 12345, 0.1, 1),
                                            (2, 2**64 - 1, 0.9, 1), (4, 7, 0.0, 0),
                                            (1, 7, 1.0, 0)])
def test_static_masks(hm, seed, p, diag):
    wl = W.small_workload(frames=11, grid_h=10, grid_w=13, tile=64,
                          mask=W.MaskSpec(W.MASK_STATIC_RANDOM, seed=seed,
                                          thresh24=W.thresh24_for_density(p),
                                          force_diagonal=diag, mask_heads=hm))
    mask, rp, ci = gpu_mask_csr(wl)
    check_mask_csr(wl, mask, rp, ci)


def test_compact_on_arbitrary_masks():
    """Compaction of masks the builder cannot produce (any nonzero byte is
    active; wide rows spanning several 64-column chunks; empty rows; more
    than 4096 rows; rows of an odd width)."""
    g = torch.Generator().manual_seed(5)
    for rows, tk in [(1, 1), (3, 63), (5, 64), (7, 65), (130, 200), (2, 1024),
                     (1025, 3), (4000, 17), (4096, 16), (256, 256), (4097, 5), (300, 1000),
                     (256, 257)]:
        m = (torch.randint(0, 4, (rows, tk), generator=g) *
             torch.randint(0, 2, (rows, tk), generator=g)).to(torch.uint8)
        m[rows // 2] = 0
        dev = m.cuda().reshape(1, rows, tk)
        rp, ci = bs.make_csr(dev)
        rp_ref, ci_ref = oracle.tile_csr(m.numpy().reshape(1, rows, tk))
        assert np.array_equal(rp.cpu().numpy(), rp_ref)
        assert np.array_equal(ci[:int(rp_ref[-1])].cpu().numpy(), ci_ref)


def test_compact_any_byte_values_and_unaligned_masks():
    """Masks of up to 128 KiB are compacted in one launch that counts the
    cells before each workgroup's rows four bytes at a time: bytes of every
    value (0x80 and above included) must count as active, and a mask that
    starts at an odd address must give the same lists."""
    g = torch.Generator().manual_seed(11)
    for rows, tk, offset in [(100, 100, 0), (256, 256, 0), (512, 256, 0), (33, 31, 1),
                             (256, 256, 3), (17, 7, 2), (513, 255, 1)]:
        vals = torch.randint(0, 256, (rows * tk + offset,), generator=g).to(torch.uint8)
        vals[torch.randint(0, 2, (rows * tk + offset,), generator=g).bool()] = 0
        buf = vals.cuda()
        dev = buf[offset:].reshape(1, rows, tk)
        rp, ci = bs.make_csr(dev)
        m = vals[offset:].numpy().reshape(1, rows, tk)
        rp_ref, ci_ref = oracle.tile_csr(m)
        assert np.array_equal(rp.cpu().numpy(), rp_ref), (rows, tk, offset)
        assert np.array_equal(ci[:int(rp_ref[-1])].cpu().numpy(), ci_ref), (rows, tk, offset)


def test_mask_and_csr_repeatable():
    w = W.WORKLOADS[3]
    m1, rp1, ci1 = gpu_mask_csr(w)
    m2, rp2, ci2 = gpu_mask_csr(w)
    assert torch.equal(m1, m2) and torch.equal(rp1, rp2)
    n = int(rp1[-1])
    assert torch.equal(ci1[:n], ci2[:n])


# ------------------------------------------------ expanded adaptive windows
def test_expanded_hand_enumerated_tile_mask():
    lines = read_golden("expanded_window_tile_mask.txt")
    hdr = lines[0].split()
    kv = dict(zip(hdr[0::2], map(int, hdr[1::2])))
    want = np.array([[int(c) for c in ln] for ln in lines[1:]], dtype=np.uint8)
    mask = bs.make_mask(kv["frames"], kv["grid_h"], kv["grid_w"], kv["tile"],
                        kind=W.MASK_WINDOW_ANCHOR_EXPANDED, window=kv["window"],
                        num_anchors=kv["anchors"], rotation=kv["rotation"],
                        budget=kv["budget"], mask_heads=2)
    m = mask.cpu().numpy()
    assert np.array_equal(m[0], want) and np.array_equal(m[1], want)


def test_expanded_long_video_every_rotation():
    w = W.EXPANDED
    dens = []
    for r in w.rotations:
        wr = w.with_rotation(r)
        mask, rp, ci = gpu_mask_csr(wr)
        m_ref = check_mask_csr(wr, mask, rp, ci)
        dens.append(m_ref.mean())
    # C = 21 of 84 frames, plus the spill of tiles that straddle two frames
    assert 0.25 <= min(dens) and max(dens) <= 0.32, (min(dens), max(dens))


@pytest.mark.parametrize("T,gh,gw,BT,w,na,r,C,hm", [
    (10, 1, 2, 3, 1, 2, 3, 5, 1),      # the hand-enumerated case
    (9, 1, 3, 2, 1, 3, 1, 6, 2),       # anchors in the growth path
    (21, 30, 52, 128, 1, 2, 7, 5, 1),  # headline shape, C = n_a + 2w + 1
    (21, 30, 52, 128, 1, 2, 7, 21, 1),  # C = T: every tile
    (33, 4, 5, 64, 3, 5, 11, 0, 1),    # C = 0: the plain window
    (40, 2, 2, 1, 0, 0, 0, 7, 1),      # no anchors, one token per tile
    (64, 1, 1, 16, 0, 3, 60, 9, 1),    # 16 frames per tile
    (1, 3, 3, 4, 0, 1, 0, 3, 1),       # one frame
    (17, 3, 7, 32, 20, 2, 5, 4, 1),    # window wider than the video
    (50, 2, 3, 8, 2, 50, 3, 10, 1),    # every frame an anchor
])
def test_expanded_odd_layouts(T, gh, gw, BT, w, na, r, C, hm):
    wl = W.small_workload(frames=T, grid_h=gh, grid_w=gw, tile=BT,
                          mask=W.MaskSpec(W.MASK_WINDOW_ANCHOR_EXPANDED,
                                          window=w, num_anchors=na, rotation=r,
                                          budget=C, mask_heads=hm))
    mask, rp, ci = gpu_mask_csr(wl)
    check_mask_csr(wl, mask, rp, ci)
