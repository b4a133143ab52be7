"""The library used from plain C: tests/capi/fwd_driver.c (built by
build(), linked against libbsattn.so and the HIP runtime only, no PyTorch)
runs bsattn_build_mask -> bsattn_compact -> bsattn_fwd on its own stream.
Its mask and lists must equal the oracle's bit for bit and its O and LSE
meet the output bar, for the tuned bf16 d 128 / tile 128 kernel and the
generic fp32 one."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from block_sparse_attention_bsattn_amd import _build
from parity_util import assert_close, lse_tolerance

pytestmark = pytest.mark.gpu

CASES = [
    # name, workload, rotation, LSE tolerance (None: derived from the inputs)
    ("video_4x30x52_bf16_t128", W.small_workload(
        frames=4, grid_h=30, grid_w=52, tile=128, d=128, H=2, B=1, dtype=W.DTYPE_BF16,
        mask=W.MaskSpec(W.MASK_WINDOW_ANCHOR, window=1, num_anchors=2),
        name="capi_video_4x30x52", seed=41), 3, None),
    ("tiny_f32_t64", W.WORKLOADS[1], 2, 2e-2),
]


@pytest.mark.parametrize("name,w,rotation,lse_tol", CASES, ids=[c[0] for c in CASES])
def test_c_program_through_the_abi(tmp_path, name, w, rotation, lse_tol):
    exe = _build.CAPI_EXE
    if not os.path.exists(exe):
        pytest.skip("tests/capi/fwd_driver is not built (build() compiles it)")
    w = w.with_rotation(rotation)
    q, k, v = W.make_qkv(w)
    f32 = w.dtype == W.DTYPE_F32
    hdr = np.array([w.B, w.H, w.N, w.d, w.tile, w.dtype, w.frames, w.grid_h, w.grid_w,
                    w.mask.window, w.mask.num_anchors, rotation], dtype="<i4")
    raw = (lambda t: t.contiguous().numpy().tobytes()) if f32 else \
        (lambda t: t.contiguous().view(torch.int16).numpy().tobytes())
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    inp.write_bytes(hdr.tobytes() + raw(q) + raw(k) + raw(v))
    print(f"case {name}: running {exe}", flush=True)
    r = subprocess.run([exe, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr

    buf = out.read_bytes()
    tq, nnz = np.frombuffer(buf, "<i4", 2)
    pos = 8
    mask = np.frombuffer(buf, np.uint8, tq * tq, pos).reshape(1, tq, tq)
    pos += tq * tq
    row_ptr = np.frombuffer(buf, "<i4", tq + 1, pos)
    pos += 4 * (tq + 1)
    col_idx = np.frombuffer(buf, "<i4", nnz, pos)
    pos += 4 * nnz
    nel = w.B * w.H * w.N * w.d
    if f32:
        o = torch.from_numpy(np.frombuffer(buf, "<f4", nel, pos).copy())
    else:
        o = torch.from_numpy(np.frombuffer(buf, "<i2", nel, pos).copy()).view(torch.bfloat16)
    pos += nel * (4 if f32 else 2)
    lse = np.frombuffer(buf, "<f4", w.B * w.H * w.N, pos)
    assert pos + 4 * w.B * w.H * w.N == len(buf)

    m_ref = oracle.tile_mask(w.mask.kind, w.frames, w.grid_h, w.grid_w, w.tile,
                             window=w.mask.window, num_anchors=w.mask.num_anchors,
                             rotation=rotation, mask_heads=1)
    rp_ref, ci_ref = oracle.tile_csr(m_ref)
    assert np.array_equal(mask, m_ref)
    assert np.array_equal(row_ptr, rp_ref) and np.array_equal(col_idx, ci_ref)
    o_ref, lse_ref = oracle.block_sparse_attention(q, k, v, m_ref, w.tile, workers=8)
    if lse_tol is None:
        lse_tol = lse_tolerance(q, k, m_ref, w.tile)
    o64 = o.reshape(w.B, w.H, w.N, w.d).to(torch.float64).numpy()
    assert_close(name, o64, o_ref, lse.reshape(w.B, w.H, w.N).astype(np.float64), lse_ref,
                 lse_tol=lse_tol)
