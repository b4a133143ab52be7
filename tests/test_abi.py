"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments on the host before touching a GPU (CPU only)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_bsattn_amd as bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(bs.LIB_PATH),
                                reason="libbsattn.so not built")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"BSATTN_API\s+[\w\s\*]+?\b(bsattn_\w+)\s*\(",
                                 text)))


def test_header_lists_the_pipeline():
    syms = declared_symbols()
    for name in ("bsattn_build_mask", "bsattn_compact", "bsattn_fwd"):
        assert name in syms
    assert sorted(bs.EXPORTS) == syms


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(bs.LIB_PATH)
    for name in declared_symbols():
        assert hasattr(L, name), name


def test_version_and_strings():
    assert bs.version() >= 100
    L = bs.lib()
    assert L.bsattn_status_string(0) == b"ok"
    assert L.bsattn_status_string(-1) == b"invalid argument"
    assert L.bsattn_status_string(-2) == b"unsupported configuration"
    assert L.bsattn_status_string(-3) == b"HIP runtime error"
    assert L.bsattn_status_string(7) == b"unknown status"


def test_num_tiles():
    assert bs.num_tiles(32760, 128) == 256
    assert bs.num_tiles(131040, 128) == 1024
    assert bs.num_tiles(256, 64) == 4
    assert bs.num_tiles(0, 64) == 0
    assert bs.num_tiles(1, 128) == 1
    assert bs.num_tiles(10, 0) == -1
    assert bs.num_tiles(-1, 64) == -1


def _fwd(**kw):
    args = dict(B=1, H=2, N=100, d=64, tile=64, dtype=0, q=8, k=8, v=8, o=8,
                lse=None, mask_heads=1, row_ptr=8, col_idx=8, scale=0.0,
                stream=None)
    args.update(kw)
    L = bs.lib()
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.bsattn_fwd(args["B"], args["H"], args["N"], args["d"], args["tile"],
                        args["dtype"], p(args["q"]), p(args["k"]), p(args["v"]),
                        p(args["o"]), p(args["lse"]), args["mask_heads"],
                        p(args["row_ptr"]), p(args["col_idx"]), args["scale"],
                        None)


def test_fwd_rejects_bad_arguments_without_launching():
    assert _fwd(d=96) == bs.ERR_UNSUPPORTED
    assert b"head dim" in bs.lib().bsattn_last_error()
    assert _fwd(tile=32) == bs.ERR_UNSUPPORTED
    assert _fwd(dtype=5) == bs.ERR_UNSUPPORTED
    assert _fwd(N=-1) == bs.ERR_INVALID_ARG
    assert _fwd(mask_heads=3) == bs.ERR_INVALID_ARG
    assert _fwd(q=None) == bs.ERR_INVALID_ARG
    assert _fwd(col_idx=None) == bs.ERR_INVALID_ARG
    assert _fwd(q=9) == bs.ERR_INVALID_ARG       # misaligned
    assert b"aligned" in bs.lib().bsattn_last_error()
    assert _fwd(scale=float("nan")) == bs.ERR_INVALID_ARG
    assert _fwd(H=70000) == bs.ERR_INVALID_ARG
    # empty problems are a successful no-op, even with null pointers
    assert _fwd(N=0, q=None, k=None, v=None, o=None) == bs.OK
    assert _fwd(B=0) == bs.OK
    assert bs.lib().bsattn_last_error() == b""


def _fwd_grouped(**kw):
    args = dict(B=1, H=2, N=32768, d=128, tile=128, dtype=0, q=64, k=64, v=64, o=64,
                lse=None, mask_heads=1, row_ptr=64, col_idx=64, window=256, scale=0.0)
    args.update(kw)
    L = bs.lib()
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.bsattn_fwd_grouped(args["B"], args["H"], args["N"], args["d"], args["tile"],
                                args["dtype"], p(args["q"]), p(args["k"]), p(args["v"]),
                                p(args["o"]), p(args["lse"]), args["mask_heads"],
                                p(args["row_ptr"]), p(args["col_idx"]), args["window"],
                                args["scale"], None)


def test_fwd_grouped_rejects_bad_arguments_without_launching():
    assert _fwd_grouped(d=64) == bs.ERR_UNSUPPORTED
    assert _fwd_grouped(tile=64) == bs.ERR_UNSUPPORTED
    assert _fwd_grouped(dtype=1) == bs.ERR_UNSUPPORTED
    assert _fwd_grouped(window=0) == bs.ERR_INVALID_ARG
    assert _fwd_grouped(N=32760, window=256) == bs.ERR_INVALID_ARG   # not a multiple of w
    assert _fwd_grouped(N=1000, window=10) == bs.ERR_INVALID_ARG     # G = 100
    assert b"multiple of 128" in bs.lib().bsattn_last_error()
    assert _fwd_grouped(q=None) == bs.ERR_INVALID_ARG
    assert _fwd_grouped(mask_heads=3) == bs.ERR_INVALID_ARG
    assert _fwd_grouped(B=0, q=None, k=None, v=None, o=None, row_ptr=None,
                        col_idx=None) == bs.OK


def test_build_mask_rejects_bad_arguments():
    L = bs.lib()
    ok_layout = bs.Layout(4, 8, 8, 64)
    ok_params = bs.MaskParams(0, 1, 1, 0, 0, 0, 0, 1)
    m = ctypes.c_void_p(64)

    def call(layout=ok_layout, params=ok_params, mask=m):
        return L.bsattn_build_mask(None if layout is None else ctypes.byref(layout),
                                   None if params is None else ctypes.byref(params),
                                   mask, None)

    assert call(layout=None) == bs.ERR_INVALID_ARG
    assert call(params=None) == bs.ERR_INVALID_ARG
    assert call(mask=None) == bs.ERR_INVALID_ARG
    assert call(layout=bs.Layout(0, 8, 8, 64)) == bs.ERR_INVALID_ARG
    assert call(layout=bs.Layout(4, 8, 8, 0)) == bs.ERR_INVALID_ARG
    assert call(params=bs.MaskParams(-1, 1, 1, 0, 0, 0, 0, 1)) == bs.ERR_INVALID_ARG
    # expanded windows: negative budget, and the window/anchor checks apply
    assert call(params=bs.MaskParams(3, 1, 1, 0, 0, 0, 0, 1, -1)) == bs.ERR_INVALID_ARG
    assert call(params=bs.MaskParams(3, -1, 1, 0, 0, 0, 0, 1, 5)) == bs.ERR_INVALID_ARG
    assert call(params=bs.MaskParams(3, 1, 5, 0, 0, 0, 0, 1, 5)) == bs.ERR_INVALID_ARG
    # block diagonal: at least one tile per block
    assert call(params=bs.MaskParams(4, 0, 0, 0, 0, 0, 0, 1, 0, 0)) == bs.ERR_INVALID_ARG
    assert call(params=bs.MaskParams(7, 0, 0, 0, 0, 0, 0, 1, 0, 1)) == bs.ERR_INVALID_ARG
    # dense rows: a non-negative tile count
    assert call(params=bs.MaskParams(5, 0, 0, 0, 0, 0, 0, 1, 0, 1, -1)) == bs.ERR_INVALID_ARG
    # spread dense rows: also at least one tile per block, and blocks that fit
    assert call(params=bs.MaskParams(6, 0, 0, 0, 0, 0, 0, 1, 0, 1, -1)) == bs.ERR_INVALID_ARG
    assert call(params=bs.MaskParams(6, 0, 0, 0, 0, 0, 0, 1, 0, 0, 2)) == bs.ERR_INVALID_ARG
    assert call(params=bs.MaskParams(6, 0, 0, 0, 0, 0, 0, 1, 0, 2, 1 << 20)) == \
        bs.ERR_INVALID_ARG
    assert call(params=bs.MaskParams(0, -1, 1, 0, 0, 0, 0, 1)) == bs.ERR_INVALID_ARG
    assert call(params=bs.MaskParams(0, 1, 5, 0, 0, 0, 0, 1)) == bs.ERR_INVALID_ARG
    assert call(params=bs.MaskParams(1, 0, 0, 0, 0, (1 << 24) + 1, 0, 1)) == \
        bs.ERR_INVALID_ARG
    assert call(params=bs.MaskParams(2, 0, 0, 0, 0, 0, 0, 0)) == bs.ERR_INVALID_ARG
    assert call(layout=bs.Layout(1 << 20, 64, 64, 64)) == bs.ERR_INVALID_ARG


def test_compact_rejects_bad_arguments():
    L = bs.lib()
    p = ctypes.c_void_p(64)
    assert L.bsattn_compact(-1, 4, p, p, p, None) == bs.ERR_INVALID_ARG
    assert L.bsattn_compact(4, -1, p, p, p, None) == bs.ERR_INVALID_ARG
    assert L.bsattn_compact(4, 4, p, None, p, None) == bs.ERR_INVALID_ARG
    assert L.bsattn_compact(4, 4, None, p, p, None) == bs.ERR_INVALID_ARG
    assert L.bsattn_compact(1 << 16, 1 << 16, p, p, p, None) == bs.ERR_INVALID_ARG


def test_mfma_ceiling_rejects_bad_arguments():
    L = bs.lib()
    p = ctypes.c_void_p(64)
    assert L.bsattn_mfma_ceiling(0, 10, p, None) == bs.ERR_INVALID_ARG
    assert L.bsattn_mfma_ceiling(4, 0, p, None) == bs.ERR_INVALID_ARG
    assert L.bsattn_mfma_ceiling(4, 10, None, None) == bs.ERR_INVALID_ARG


def test_ctypes_structs_match_the_c_header(tmp_path):
    """The binding's Layout and MaskParams have the C structs' size and field
    offsets (checked by compiling a probe against include/bsattn.h)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    fields = {"bsattn_layout": bs.Layout, "bsattn_mask_params": bs.MaskParams}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "bsattn.h"',
             "int main(void) {"]
    for cname, py in fields.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "probe.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "probe"
    inc = os.path.join(ROOT, "include")
    subprocess.run([cc, "-I", inc, str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True,
                         text=True).stdout.split("\n")
    got = {tuple(ln.split()[:2]): int(ln.split()[2]) for ln in out if ln}
    for cname, py in fields.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)


def test_calibration_calls_reject_bad_arguments():
    L = bs.lib()
    p = ctypes.c_void_p(64)
    E = L.bsattn_block_energy
    n = (None, 0, None)  # no workspace, stream
    assert E(1, 1, 256, 128, 128, 0, p, p, None, 0.0, *n) == bs.ERR_INVALID_ARG
    assert E(1, 1, 256, 96, 128, 0, p, p, p, 0.0, *n) == bs.ERR_UNSUPPORTED
    assert E(1, 1, 256, 128, 32, 0, p, p, p, 0.0, *n) == bs.ERR_UNSUPPORTED
    assert E(1, 1, 256, 128, 128, 7, p, p, p, 0.0, *n) == bs.ERR_UNSUPPORTED
    assert E(-1, 1, 256, 128, 128, 0, p, p, p, 0.0, *n) == bs.ERR_INVALID_ARG
    assert E(1, 1, 256, 128, 128, 0, ctypes.c_void_p(65), p, p, 0.0, *n) == \
        bs.ERR_INVALID_ARG
    assert E(1, 1, 256, 128, 128, 0, p, p, p, float("nan"), *n) == bs.ERR_INVALID_ARG
    assert E(70000, 1, 256, 128, 128, 0, p, p, p, 0.0, *n) == bs.ERR_INVALID_ARG
    assert E(0, 1, 256, 128, 128, 0, None, None, None, 0.0, *n) == bs.OK
    # one-sweep workspace: 1024 * min(512, B * H * ceil(T / 2)) * T bytes at tile 128
    WB = L.bsattn_block_energy_workspace_bytes
    assert WB(1, 1, 256, 128) == 1024 * 1 * 2
    assert WB(4, 12, 32760, 128) == 1024 * 512 * 256
    assert WB(2, 3, 1000, 128) == 1024 * (2 * 3 * 4) * 8
    assert WB(1, 1, 256, 64) == 0 and WB(-1, 1, 256, 128) < 0 and WB(1, 1, 256, 32) < 0
    need = WB(1, 1, 256, 128)
    assert E(1, 1, 256, 128, 128, 0, p, p, p, 0.0, p, need - 1, None) == bs.ERR_INVALID_ARG
    assert E(1, 1, 256, 128, 128, 0, p, p, p, 0.0, ctypes.c_void_p(72), need, None) == \
        bs.ERR_INVALID_ARG                                              # unaligned workspace
    S = L.bsattn_select_blocks
    assert S(-1, 4, p, 0.5, p, None) == bs.ERR_INVALID_ARG
    assert S(4, 4097, p, 0.5, p, None) == bs.ERR_UNSUPPORTED
    assert S(4, 4, None, 0.5, p, None) == bs.ERR_INVALID_ARG
    assert S(4, 4, p, float("inf"), p, None) == bs.ERR_INVALID_ARG
    assert S(0, 4, None, 0.5, None, None) == bs.OK
    A = L.bsattn_aggregate_masks
    assert A(0, 4, p, 0.5, p, None) == bs.ERR_INVALID_ARG
    assert A(2, -1, p, 0.5, p, None) == bs.ERR_INVALID_ARG
    assert A(2, 4, p, float("nan"), p, None) == bs.ERR_INVALID_ARG
    assert A(2, 4, None, 0.5, p, None) == bs.ERR_INVALID_ARG
    assert A(2, 0, None, 0.5, None, None) == bs.OK


def test_window_reorder_rejects_bad_arguments():
    R = bs.lib().bsattn_window_reorder
    p, p2 = ctypes.c_void_p(64), ctypes.c_void_p(128)
    assert R(1, 1, 12, 128, 5, 0, p, p2, 0, None) == bs.ERR_INVALID_ARG    # N % w
    assert R(1, 1, 12, 128, 0, 0, p, p2, 0, None) == bs.ERR_INVALID_ARG    # w < 1
    assert R(1, 1, 12, 128, 4, 0, p, p, 0, None) == bs.ERR_INVALID_ARG     # aliased
    assert R(1, 1, 12, 128, 4, 0, None, p2, 0, None) == bs.ERR_INVALID_ARG
    assert R(1, 1, 12, 4, 4, 0, p, p2, 0, None) == bs.ERR_INVALID_ARG      # 8-byte rows
    assert R(1, 1, 12, 128, 4, 3, p, p2, 0, None) == bs.ERR_UNSUPPORTED
    assert R(1, 1, 12, 128, 4, 0, ctypes.c_void_p(65), p2, 0, None) == bs.ERR_INVALID_ARG
    assert R(0, 1, 12, 128, 4, 0, None, None, 0, None) == bs.OK


def test_repetition_calls_reject_bad_arguments():
    L = bs.lib()
    p, p2 = ctypes.c_void_p(64), ctypes.c_void_p(128)
    C = L.bsattn_row_cosines
    assert C(1, 1, 2, 4, 8, 128, 0, 0, p, p, p, 0.0, None, 0, None) == bs.ERR_INVALID_ARG
    assert C(1, 1, 2, 4, 300, 128, 2, 0, p, p, p, 0.0, None, 0, None) == bs.ERR_UNSUPPORTED
    assert C(1, 1, 2, 4, 8, 96, 2, 0, p, p, p, 0.0, None, 0, None) == bs.ERR_UNSUPPORTED
    assert C(1, 1, 2, 4, 8, 128, 2, 0, p, p, None, 0.0, None, 0, None) == bs.ERR_INVALID_ARG
    assert C(1, 1, 2, 4, 8, 128, 2, 0, p, p, p, float("nan"), None, 0, None) == \
        bs.ERR_INVALID_ARG
    assert C(0, 1, 2, 4, 8, 128, 2, 0, None, None, None, 0.0, None, 0, None) == bs.OK
    # workspace: 12 B per column of the non-anchor rows (2 of 4 at stride 2)
    WB = L.bsattn_row_cosines_workspace_bytes
    assert WB(2, 3, 5, 4, 8, 2) == 12 * 2 * 3 * 5 * 2 * 8
    assert WB(1, 1, 2, 4, 8, 1) == 0
    assert WB(1, 1, 2, 4, 8, 0) < 0 and WB(-1, 1, 2, 4, 8, 2) < 0
    need = WB(1, 1, 2, 4, 8, 2)
    assert C(1, 1, 2, 4, 8, 128, 2, 0, p, p, p, 0.0, p2, need - 1, None) == bs.ERR_INVALID_ARG
    assert C(1, 1, 2, 4, 8, 128, 2, 0, p, p, p, 0.0, ctypes.c_void_p(130), need, None) == \
        bs.ERR_INVALID_ARG                                              # unaligned workspace
    R = L.bsattn_repetitive_heads
    assert R(1, 2, 3, 4, 0, p, 0.9, p, None) == bs.ERR_INVALID_ARG
    assert R(1, 2, 3, 4, 2, None, 0.9, p, None) == bs.ERR_INVALID_ARG
    assert R(1, 2, 3, 4, 2, p, float("inf"), p, None) == bs.ERR_INVALID_ARG
    assert R(1, 0, 3, 4, 2, None, 0.9, None, None) == bs.OK
    A = L.bsattn_anchor_rows
    assert A(1, 1, 2, 4, 8, 128, 2, 0, p, p, 0, 0, None) == bs.ERR_INVALID_ARG     # aliased
    assert A(1, 1, 2, 4, 8, 128, 2, 0, None, p2, 0, 0, None) == bs.ERR_INVALID_ARG
    assert A(1, 1, 2, 0, 8, 128, 2, 0, p, p2, 0, 0, None) == bs.ERR_INVALID_ARG
    assert A(1, 1, 2, 4, 8, 128, 2, 5, p, p2, 0, 0, None) == bs.ERR_UNSUPPORTED
    assert A(1, 1, 2, 4, 8, 4, 2, 0, p, p2, 0, 0, None) == bs.ERR_INVALID_ARG     # 8-byte rows
    assert A(1, 1, 2, 4, 8, 128, 2, 0, p, p2, 0, -1, None) == bs.ERR_INVALID_ARG  # block_rows
    assert A(1, 1, 0, 4, 8, 128, 2, 0, None, None, 0, 0, None) == bs.OK


def _plan_bytes(**kw):
    args = dict(B=1, H=12, N=32760, tile=128, mask_heads=1, nnz=-1, workers=256)
    args.update(kw)
    return bs.lib().bsattn_fwd_plan_bytes(args["B"], args["H"], args["N"], args["tile"],
                                          args["mask_heads"], args["nnz"], args["workers"])


def test_fwd_plan_bytes():
    full = _plan_bytes()
    assert full > 0
    # 8 bytes per step, B * (H / mask_heads) steps per CSR entry
    assert _plan_bytes(nnz=1002) - _plan_bytes(nnz=1000) == 2 * 8 * 12
    assert _plan_bytes(nnz=1002, mask_heads=12) - _plan_bytes(nnz=1000, mask_heads=12) == 16
    assert _plan_bytes(nnz=10**12) == full             # clamped to Hm * Tq * Tk
    assert _plan_bytes(nnz=256 * 256) == full
    # at most ceil(7 Tk / 5) + 2 steps per query-tile pair: 12 heads x 128
    # pairs x 361; the list bound for nnz = 0 is 2 steps per pair
    assert full - _plan_bytes(nnz=0) == 8 * (12 * 128 * 361 - 12 * 2 * 128)
    assert _plan_bytes(nnz=361 * 128 - 256) == full
    assert _plan_bytes(tile=64) == bs.ERR_UNSUPPORTED
    assert _plan_bytes(N=4097 * 128) == bs.ERR_UNSUPPORTED   # Tq > 4096
    assert _plan_bytes(mask_heads=5) == bs.ERR_INVALID_ARG
    assert _plan_bytes(workers=100) == bs.ERR_INVALID_ARG    # not a multiple of 8
    assert _plan_bytes(workers=1024) == bs.ERR_INVALID_ARG
    assert _plan_bytes(B=100, H=1000) == bs.ERR_UNSUPPORTED  # B*H > 65535
    assert _plan_bytes(N=-1) == bs.ERR_INVALID_ARG


def _planned(**kw):
    args = dict(B=1, H=2, N=4096, d=128, tile=128, dtype=0, q=64, k=64, v=64, o=64,
                lse=None, mask_heads=1, row_ptr=64, col_idx=64, plan=64,
                plan_bytes=1 << 30, workers=256, window=0, scale=0.0)
    args.update(kw)
    L = bs.lib()
    p = lambda x: None if x is None else ctypes.c_void_p(x)
    return L.bsattn_fwd_planned(args["B"], args["H"], args["N"], args["d"], args["tile"],
                                args["dtype"], p(args["q"]), p(args["k"]), p(args["v"]),
                                p(args["o"]), p(args["lse"]), args["mask_heads"],
                                p(args["row_ptr"]), p(args["col_idx"]), p(args["plan"]),
                                args["plan_bytes"], args["workers"], args["window"],
                                args["scale"], None)


def test_fwd_planned_and_plan_reject_bad_arguments_without_launching():
    assert _planned(d=64) == bs.ERR_UNSUPPORTED
    assert _planned(tile=64) == bs.ERR_UNSUPPORTED
    assert _planned(dtype=1) == bs.ERR_UNSUPPORTED
    assert _planned(window=-1) == bs.ERR_INVALID_ARG
    assert _planned(window=10) == bs.ERR_INVALID_ARG        # N not w * 128 k
    assert _planned(plan=None) == bs.ERR_INVALID_ARG
    assert _planned(plan=72) == bs.ERR_INVALID_ARG          # unaligned
    assert _planned(plan_bytes=64) == bs.ERR_INVALID_ARG    # below the fixed part
    assert b"plan_bytes" in bs.lib().bsattn_last_error()
    assert _planned(workers=12) == bs.ERR_INVALID_ARG
    assert _planned(mask_heads=3) == bs.ERR_INVALID_ARG
    assert _planned(q=None) == bs.ERR_INVALID_ARG
    assert _planned(B=0, q=None, k=None, v=None, o=None) == bs.OK
    L = bs.lib()
    p = ctypes.c_void_p
    assert L.bsattn_fwd_plan(1, 2, 4096, 128, 1, p(64), p(64), 256, p(64), 64,
                             None) == bs.ERR_INVALID_ARG
    assert L.bsattn_fwd_plan(1, 2, 4096, 128, 1, None, p(64), 256, p(64), 1 << 30,
                             None) == bs.ERR_INVALID_ARG
    assert L.bsattn_fwd_plan(1, 2, 4096, 64, 1, p(64), p(64), 256, p(64), 1 << 30,
                             None) == bs.ERR_UNSUPPORTED
    assert L.bsattn_fwd_plan(0, 2, 4096, 128, 1, None, None, 256, None, 0, None) == bs.OK
