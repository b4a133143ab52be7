"""Python binding of libbsattn (block-sparse video attention for MI355X).

Argument marshalling only: torch tensors supply device memory and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
The calls mirror include/bsattn.h:

    build_mask(layout, params, mask)                    -> bsattn_build_mask
    compact(mask, row_ptr, col_idx)                     -> bsattn_compact
    fwd(q, k, v, o, row_ptr, col_idx, tile, ...)        -> bsattn_fwd
    fwd_grouped(q, k, v, o, row_ptr, col_idx, w, ...)   -> bsattn_fwd_grouped
    fwd_plan_bytes(B, H, N, tile, ...)                  -> bsattn_fwd_plan_bytes
    fwd_plan(row_ptr, col_idx, B, H, N, tile, plan)     -> bsattn_fwd_plan
    fwd_planned(q, k, v, o, row_ptr, col_idx, plan, ..) -> bsattn_fwd_planned
    fwd_noalloc(q, k, v, o, row_ptr, col_idx, tile, ...) -> bsattn_fwd_noalloc
    block_energy(q, k, energy, tile, ...)               -> bsattn_block_energy
    block_energy_workspace_bytes(...)                   -> bsattn_block_energy_workspace_bytes
    select_blocks(energy, eps, mask)                    -> bsattn_select_blocks
    aggregate_masks(masks, rho, out)                    -> bsattn_aggregate_masks
    window_reorder(src, dst, w, inverse)                -> bsattn_window_reorder
    row_cosines(q, k, ..., cos)                         -> bsattn_row_cosines
    row_cosines_workspace_bytes(...)                    -> bsattn_row_cosines_workspace_bytes
    repetitive_heads(cos, stride, gamma, flags)         -> bsattn_repetitive_heads
    anchor_rows(src, dst, ..., broadcast, block_rows)   -> bsattn_anchor_rows
    anchor_rows(..., flags=f)                           -> bsattn_anchor_rows_heads
    mask_select(flags, set_mask, clear_mask, out)       -> bsattn_mask_select

plus small helpers that allocate the outputs with torch (make_mask,
make_csr, make_plan, attention, calibrate, squad, repeated_attention,
mixed_layer_csr, mixed_attention).  There is no fallback: if libbsattn.so is missing or a
call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
# BSATTN_LIB may name another build of the same library (for A/B timing)
LIB_PATH = os.environ.get("BSATTN_LIB") or os.path.join(_PKG, "libbsattn.so")

OK = 0
ERR_INVALID_ARG = -1
ERR_UNSUPPORTED = -2
ERR_HIP = -3

DTYPE_BF16 = 0
DTYPE_F32 = 1

MASK_WINDOW_ANCHOR = 0
MASK_STATIC_RANDOM = 1
MASK_DENSE = 2
MASK_WINDOW_ANCHOR_EXPANDED = 3
MASK_BLOCK_DIAGONAL = 4
MASK_DENSE_ROWS = 5
MASK_DENSE_ROWS_SPREAD = 6

# Every symbol include/bsattn.h exports.
EXPORTS = ("bsattn_version", "bsattn_status_string", "bsattn_last_error",
           "bsattn_num_tiles", "bsattn_build_mask", "bsattn_compact",
           "bsattn_fwd", "bsattn_fwd_grouped", "bsattn_fwd_plan_bytes", "bsattn_fwd_plan",
           "bsattn_fwd_planned", "bsattn_fwd_noalloc", "bsattn_window_reorder",
           "bsattn_row_cosines", "bsattn_row_cosines_workspace_bytes",
           "bsattn_repetitive_heads", "bsattn_anchor_rows", "bsattn_anchor_rows_heads",
           "bsattn_mask_select", "bsattn_block_energy", "bsattn_block_energy_workspace_bytes",
           "bsattn_select_blocks",
           "bsattn_aggregate_masks", "bsattn_mfma_ceiling")


class BsattnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {detail or 'error'} (status {status})")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [("frames", ctypes.c_int32), ("grid_h", ctypes.c_int32),
                ("grid_w", ctypes.c_int32), ("tile", ctypes.c_int32)]


class MaskParams(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("window", ctypes.c_int32),
                ("num_anchors", ctypes.c_int32), ("rotation", ctypes.c_int32),
                ("seed", ctypes.c_uint64), ("thresh24", ctypes.c_uint32),
                ("force_diagonal", ctypes.c_int32),
                ("mask_heads", ctypes.c_int32), ("budget", ctypes.c_int32),
                ("block_tiles", ctypes.c_int32), ("query_tiles", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python __graft_entry__.py build` "
            "(or block_sparse_attention_bsattn_amd/_build.py) first")
    L = ctypes.CDLL(LIB_PATH)
    i32, u8p, i32p, vp = (ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                          ctypes.c_void_p)
    L.bsattn_version.restype = ctypes.c_int
    L.bsattn_version.argtypes = []
    L.bsattn_status_string.restype = ctypes.c_char_p
    L.bsattn_status_string.argtypes = [ctypes.c_int]
    L.bsattn_last_error.restype = ctypes.c_char_p
    L.bsattn_last_error.argtypes = []
    L.bsattn_num_tiles.restype = i32
    L.bsattn_num_tiles.argtypes = [ctypes.c_int64, i32]
    L.bsattn_build_mask.restype = ctypes.c_int
    L.bsattn_build_mask.argtypes = [ctypes.POINTER(Layout),
                                    ctypes.POINTER(MaskParams), u8p, vp]
    L.bsattn_compact.restype = ctypes.c_int
    L.bsattn_compact.argtypes = [i32, i32, u8p, i32p, i32p, vp]
    L.bsattn_fwd.restype = ctypes.c_int
    L.bsattn_fwd.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                             i32, i32p, i32p, ctypes.c_float, vp]
    L.bsattn_fwd_grouped.restype = ctypes.c_int
    L.bsattn_fwd_grouped.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                     i32, i32p, i32p, i32, ctypes.c_float, vp]
    L.bsattn_fwd_plan_bytes.restype = ctypes.c_int64
    L.bsattn_fwd_plan_bytes.argtypes = [i32, i32, i32, i32, i32, ctypes.c_int64, i32]
    L.bsattn_fwd_plan.restype = ctypes.c_int
    L.bsattn_fwd_plan.argtypes = [i32, i32, i32, i32, i32, i32p, i32p, i32, vp,
                                  ctypes.c_int64, vp]
    L.bsattn_fwd_planned.restype = ctypes.c_int
    L.bsattn_fwd_planned.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                     i32, i32p, i32p, vp, ctypes.c_int64, i32, i32,
                                     ctypes.c_float, vp]
    L.bsattn_fwd_noalloc.restype = ctypes.c_int
    L.bsattn_fwd_noalloc.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp,
                                     i32, i32p, i32p, ctypes.c_float, vp]
    L.bsattn_window_reorder.restype = ctypes.c_int
    L.bsattn_window_reorder.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, i32, vp]
    L.bsattn_row_cosines.restype = ctypes.c_int
    L.bsattn_row_cosines.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                     ctypes.c_float, vp, ctypes.c_int64, vp]
    L.bsattn_row_cosines_workspace_bytes.restype = ctypes.c_int64
    L.bsattn_row_cosines_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    L.bsattn_repetitive_heads.restype = ctypes.c_int
    L.bsattn_repetitive_heads.argtypes = [i32, i32, i32, i32, i32, vp, ctypes.c_double, u8p, vp]
    L.bsattn_anchor_rows.restype = ctypes.c_int
    L.bsattn_anchor_rows.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, i32, i32, vp]
    L.bsattn_anchor_rows_heads.restype = ctypes.c_int
    L.bsattn_anchor_rows_heads.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, vp, vp, i32,
                                           i32, u8p, vp]
    L.bsattn_mask_select.restype = ctypes.c_int
    L.bsattn_mask_select.argtypes = [i32, i32, i32, u8p, u8p, i32, u8p, i32, u8p, vp]
    L.bsattn_block_energy.restype = ctypes.c_int
    L.bsattn_block_energy.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp, vp,
                                      ctypes.c_float, vp, ctypes.c_int64, vp]
    L.bsattn_block_energy_workspace_bytes.restype = ctypes.c_int64
    L.bsattn_block_energy_workspace_bytes.argtypes = [i32, i32, i32, i32]
    L.bsattn_select_blocks.restype = ctypes.c_int
    L.bsattn_select_blocks.argtypes = [i32, i32, vp, ctypes.c_double, u8p, vp]
    L.bsattn_aggregate_masks.restype = ctypes.c_int
    L.bsattn_aggregate_masks.argtypes = [i32, ctypes.c_int64, u8p,
                                         ctypes.c_double, u8p, vp]
    L.bsattn_mfma_ceiling.restype = ctypes.c_int64
    L.bsattn_mfma_ceiling.argtypes = [i32, i32, vp, vp]
    _lib = L
    return L


def _check(status: int, where: str):
    if status != OK:
        detail = lib().bsattn_last_error().decode()
        raise BsattnError(status, where, detail)


def _stream(stream):
    """hipStream_t handle: an int, a torch stream, or the current stream."""
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t, name, dtype=None, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must have dtype {dtype}, not {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def version() -> int:
    return lib().bsattn_version()


def num_tiles(tokens: int, tile: int) -> int:
    return lib().bsattn_num_tiles(tokens, tile)


def _params(kind, window=0, num_anchors=0, rotation=0, seed=0, thresh24=0,
            force_diagonal=0, mask_heads=1, budget=0, block_tiles=1,
            query_tiles=0) -> MaskParams:
    return MaskParams(kind, window, num_anchors, rotation,
                      seed & 0xFFFFFFFFFFFFFFFF, thresh24, int(force_diagonal),
                      mask_heads, budget, block_tiles, query_tiles)


def build_mask(layout: Sequence[int], mask, stream=None, **params):
    """bsattn_build_mask into the uint8 tensor `mask` [Hm, Tq, Tk].

    layout = (frames, grid_h, grid_w, tile); params are the fields of
    bsattn_mask_params (kind, window, num_anchors, rotation, seed, thresh24,
    force_diagonal, mask_heads, budget, block_tiles, query_tiles)."""
    import torch
    L = Layout(*[int(x) for x in layout])
    P = _params(**params)
    tiles = num_tiles(L.frames * L.grid_h * L.grid_w, L.tile)
    if tuple(mask.shape) != (P.mask_heads, tiles, tiles):
        raise ValueError(f"mask must have shape {(P.mask_heads, tiles, tiles)}")
    st = lib().bsattn_build_mask(ctypes.byref(L), ctypes.byref(P),
                                 _ptr(mask, "mask", torch.uint8), _stream(stream))
    _check(st, "bsattn_build_mask")
    return mask


def compact(mask, row_ptr, col_idx, stream=None):
    """bsattn_compact of mask [Hm, Tq, Tk] into row_ptr [Hm*Tq+1] and col_idx."""
    import torch
    Hm, Tq, Tk = mask.shape
    rows = Hm * Tq
    if row_ptr.numel() != rows + 1:
        raise ValueError("row_ptr must hold Hm*Tq + 1 entries")
    if col_idx.numel() < rows * Tk:
        raise ValueError("col_idx must hold at least Hm*Tq*Tk entries")
    st = lib().bsattn_compact(rows, Tk, _ptr(mask, "mask", torch.uint8),
                              _ptr(row_ptr, "row_ptr", torch.int32),
                              _ptr(col_idx, "col_idx", torch.int32),
                              _stream(stream))
    _check(st, "bsattn_compact")
    return row_ptr, col_idx


def fwd(q, k, v, o, row_ptr, col_idx, tile: int, mask_heads: int = 1,
        lse=None, scale: float = 0.0, stream=None):
    """bsattn_fwd: o = block-sparse attention of q, k, v ([B, H, N, d])."""
    import torch
    if q.dtype == torch.bfloat16:
        dt = DTYPE_BF16
    elif q.dtype == torch.float32:
        dt = DTYPE_F32
    else:
        raise ValueError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4:
        raise ValueError("q must have shape [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o)):
        if tuple(t.shape) != (B, H, N, d):
            raise ValueError(f"{name} must have the shape of q")
    if lse is not None and tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must have shape [B, H, N]")
    st = lib().bsattn_fwd(B, H, N, d, tile, dt, _ptr(q, "q", q.dtype),
                          _ptr(k, "k", q.dtype), _ptr(v, "v", q.dtype),
                          _ptr(o, "o", q.dtype),
                          _ptr(lse, "lse", torch.float32, allow_none=True),
                          mask_heads, _ptr(row_ptr, "row_ptr", torch.int32),
                          _ptr(col_idx, "col_idx", torch.int32), float(scale),
                          _stream(stream))
    _check(st, "bsattn_fwd")
    return o


def fwd_grouped(q, k, v, o, row_ptr, col_idx, w: int, mask_heads: int = 1,
                lse=None, scale: float = 0.0, stream=None):
    """bsattn_fwd_grouped: the forward over the position-major order of the
    windows of w tokens (bf16, d 128, tile 128), on window-major buffers."""
    import torch
    if q.dtype != torch.bfloat16 or q.dim() != 4:
        raise ValueError("q must be bf16 [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o)):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must have the shape and dtype of q")
    if lse is not None and tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must have shape [B, H, N]")
    st = lib().bsattn_fwd_grouped(B, H, N, d, 128, DTYPE_BF16, _ptr(q, "q", q.dtype),
                                  _ptr(k, "k", q.dtype), _ptr(v, "v", q.dtype),
                                  _ptr(o, "o", q.dtype),
                                  _ptr(lse, "lse", torch.float32, allow_none=True),
                                  mask_heads, _ptr(row_ptr, "row_ptr", torch.int32),
                                  _ptr(col_idx, "col_idx", torch.int32), int(w), float(scale),
                                  _stream(stream))
    _check(st, "bsattn_fwd_grouped")
    return o


def fwd_plan_bytes(B: int, H: int, N: int, tile: int = 128, mask_heads: int = 1,
                   nnz_bound: int = -1, workers: int = 0) -> int:
    """bsattn_fwd_plan_bytes: size of a plan buffer for these sizes."""
    n = lib().bsattn_fwd_plan_bytes(B, H, N, tile, mask_heads, int(nnz_bound), workers)
    if n < 0:
        _check(int(n), "bsattn_fwd_plan_bytes")
    return int(n)


def fwd_plan(row_ptr, col_idx, B: int, H: int, N: int, plan, tile: int = 128,
             mask_heads: int = 1, workers: int = 0, stream=None):
    """bsattn_fwd_plan of a CSR into the uint8 device tensor `plan`."""
    import torch
    st = lib().bsattn_fwd_plan(B, H, N, tile, mask_heads,
                               _ptr(row_ptr, "row_ptr", torch.int32),
                               _ptr(col_idx, "col_idx", torch.int32), workers,
                               _ptr(plan, "plan", torch.uint8), plan.numel(),
                               _stream(stream))
    _check(st, "bsattn_fwd_plan")
    return plan


def make_plan(row_ptr, col_idx, B: int, H: int, N: int, tile: int = 128,
              mask_heads: int = 1, workers: int = 0, nnz_bound: Optional[int] = None,
              stream=None):
    """A plan tensor sized for the CSR (its entry count read from row_ptr
    unless nnz_bound is given) and built by bsattn_fwd_plan."""
    import torch
    if nnz_bound is None:
        nnz_bound = int(row_ptr[-1].item())
    nb = fwd_plan_bytes(B, H, N, tile, mask_heads, nnz_bound, workers)
    plan = torch.empty(nb, dtype=torch.uint8, device=row_ptr.device)
    return fwd_plan(row_ptr, col_idx, B, H, N, plan, tile, mask_heads, workers, stream)


def fwd_planned(q, k, v, o, row_ptr, col_idx, plan, mask_heads: int = 1, lse=None,
                workers: int = 0, window: int = 0, scale: float = 0.0, stream=None):
    """bsattn_fwd_planned: the forward through a plan from fwd_plan (bf16,
    d 128, tile 128; window > 0 for the grouped view)."""
    import torch
    if q.dtype != torch.bfloat16 or q.dim() != 4:
        raise ValueError("q must be bf16 [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o)):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must have the shape and dtype of q")
    if lse is not None and tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must have shape [B, H, N]")
    st = lib().bsattn_fwd_planned(B, H, N, d, 128, DTYPE_BF16, _ptr(q, "q", q.dtype),
                                  _ptr(k, "k", q.dtype), _ptr(v, "v", q.dtype),
                                  _ptr(o, "o", q.dtype),
                                  _ptr(lse, "lse", torch.float32, allow_none=True),
                                  mask_heads, _ptr(row_ptr, "row_ptr", torch.int32),
                                  _ptr(col_idx, "col_idx", torch.int32),
                                  _ptr(plan, "plan", torch.uint8), plan.numel(), workers,
                                  int(window), float(scale), _stream(stream))
    _check(st, "bsattn_fwd_planned")
    return o


def fwd_noalloc(q, k, v, o, row_ptr, col_idx, tile: int, mask_heads: int = 1,
                lse=None, scale: float = 0.0, stream=None):
    """bsattn_fwd_noalloc: bsattn_fwd's result without any allocation (the
    plan lives in the library's own device array)."""
    import torch
    dt = _dtype_code(q)
    if q.dim() != 4:
        raise ValueError("q must have shape [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o)):
        if tuple(t.shape) != (B, H, N, d) or t.dtype != q.dtype:
            raise ValueError(f"{name} must have the shape and dtype of q")
    if lse is not None and tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must have shape [B, H, N]")
    st = lib().bsattn_fwd_noalloc(B, H, N, d, tile, dt, _ptr(q, "q", q.dtype),
                                  _ptr(k, "k", q.dtype), _ptr(v, "v", q.dtype),
                                  _ptr(o, "o", q.dtype),
                                  _ptr(lse, "lse", torch.float32, allow_none=True),
                                  mask_heads, _ptr(row_ptr, "row_ptr", torch.int32),
                                  _ptr(col_idx, "col_idx", torch.int32), float(scale),
                                  _stream(stream))
    _check(st, "bsattn_fwd_noalloc")
    return o


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def window_reorder(src, dst, w: int, inverse: bool = False, stream=None):
    """bsattn_window_reorder of src [B, H, N, d] into dst (window-major ->
    position-major, or back with inverse=True)."""
    if src.dim() != 4 or tuple(dst.shape) != tuple(src.shape) or dst.dtype != src.dtype:
        raise ValueError("src and dst must share shape [B, H, N, d] and dtype")
    B, H, N, d = src.shape
    st = lib().bsattn_window_reorder(B, H, N, d, w, _dtype_code(src),
                                     _ptr(src, "src", src.dtype), _ptr(dst, "dst", src.dtype),
                                     int(bool(inverse)), _stream(stream))
    _check(st, "bsattn_window_reorder")
    return dst


def row_cosines_workspace_bytes(B, H, frames, grid_h, grid_w, stride):
    """bsattn_row_cosines_workspace_bytes."""
    n = lib().bsattn_row_cosines_workspace_bytes(B, H, frames, grid_h, grid_w, stride)
    if n < 0:
        raise ValueError("row_cosines_workspace_bytes: invalid sizes")
    return n


def row_cosines(q, k, frames, grid_h, grid_w, stride, cos, scale=0.0, stream=None,
                workspace=None, packed=True):
    """bsattn_row_cosines into cos [B, H, frames, grid_h] (float32).  With
    packed (the default) a workspace of row_cosines_workspace_bytes bytes is
    passed (`workspace`, a device uint8 tensor, or one allocated here);
    packed=False passes none (the row-aligned schedule)."""
    import torch
    B, H, N, d = q.shape
    if N != frames * grid_h * grid_w or tuple(k.shape) != tuple(q.shape):
        raise ValueError("q, k must be [B, H, frames*grid_h*grid_w, d]")
    if tuple(cos.shape) != (B, H, frames, grid_h):
        raise ValueError("cos must have shape [B, H, frames, grid_h]")
    ws_ptr, ws_bytes = None, 0
    if packed:
        need = row_cosines_workspace_bytes(B, H, frames, grid_h, grid_w, stride)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if workspace is not None:
            ws_ptr, ws_bytes = _ptr(workspace, "workspace", torch.uint8), workspace.numel()
    st = lib().bsattn_row_cosines(B, H, frames, grid_h, grid_w, d, stride, _dtype_code(q),
                                  _ptr(q, "q", q.dtype), _ptr(k, "k", q.dtype),
                                  _ptr(cos, "cos", torch.float32), float(scale),
                                  ws_ptr, ws_bytes, _stream(stream))
    _check(st, "bsattn_row_cosines")
    return cos


def repetitive_heads(cos, stride, gamma, flags, stream=None):
    """bsattn_repetitive_heads: flags [H] (uint8) from cos [B, H, T, grid_h]."""
    import torch
    B, H, T, gh = cos.shape
    if tuple(flags.shape) != (H,):
        raise ValueError("flags must have shape [H]")
    st = lib().bsattn_repetitive_heads(B, H, T, gh, stride, _ptr(cos, "cos", torch.float32),
                                       float(gamma), _ptr(flags, "flags", torch.uint8),
                                       _stream(stream))
    _check(st, "bsattn_repetitive_heads")
    return flags


def anchor_rows(src, dst, frames, grid_h, grid_w, stride, broadcast=False, block_rows=0,
                flags=None, stream=None):
    """bsattn_anchor_rows between [B, H, N, d] buffers (gather, or broadcast
    with broadcast=True); block_rows > 0 spreads the packed anchor rows in
    blocks of that many rows.  With flags (uint8 [H] on the device),
    bsattn_anchor_rows_heads: only the flagged heads are gathered or
    broadcast, the others copied row for row."""
    import torch
    if src.dim() != 4 or tuple(dst.shape) != tuple(src.shape) or dst.dtype != src.dtype:
        raise ValueError("src and dst must share shape [B, H, N, d] and dtype")
    B, H, N, d = src.shape
    if N != frames * grid_h * grid_w:
        raise ValueError("N must equal frames * grid_h * grid_w")
    if flags is None:
        st = lib().bsattn_anchor_rows(B, H, frames, grid_h, grid_w, d, stride, _dtype_code(src),
                                      _ptr(src, "src", src.dtype), _ptr(dst, "dst", src.dtype),
                                      int(bool(broadcast)), int(block_rows), _stream(stream))
        _check(st, "bsattn_anchor_rows")
        return dst
    if tuple(flags.shape) != (H,):
        raise ValueError("flags must have shape [H]")
    st = lib().bsattn_anchor_rows_heads(B, H, frames, grid_h, grid_w, d, stride,
                                        _dtype_code(src), _ptr(src, "src", src.dtype),
                                        _ptr(dst, "dst", src.dtype), int(bool(broadcast)),
                                        int(block_rows), _ptr(flags, "flags", torch.uint8),
                                        _stream(stream))
    _check(st, "bsattn_anchor_rows_heads")
    return dst


def mask_select(flags, set_mask, clear_mask, out, stream=None):
    """bsattn_mask_select: out[h] = set_mask[h or 0] if flags[h] else
    clear_mask[h or 0], masks uint8 [heads, Tq, Tk]."""
    import torch
    H, Tq, Tk = out.shape
    for name, m in (("set_mask", set_mask), ("clear_mask", clear_mask)):
        if m.dim() != 3 or tuple(m.shape[1:]) != (Tq, Tk) or m.shape[0] not in (1, H):
            raise ValueError(f"{name} must have shape [1 or H, Tq, Tk]")
    st = lib().bsattn_mask_select(H, Tq, Tk, _ptr(flags, "flags", torch.uint8),
                                  _ptr(set_mask, "set_mask", torch.uint8), set_mask.shape[0],
                                  _ptr(clear_mask, "clear_mask", torch.uint8),
                                  clear_mask.shape[0], _ptr(out, "out", torch.uint8),
                                  _stream(stream))
    _check(st, "bsattn_mask_select")
    return out


def block_energy_workspace_bytes(B, H, N, tile):
    """bsattn_block_energy_workspace_bytes."""
    n = lib().bsattn_block_energy_workspace_bytes(B, H, N, tile)
    if n < 0:
        raise ValueError("block_energy_workspace_bytes: invalid sizes")
    return n


def block_energy(q, k, energy, tile: int, scale: float = 0.0, stream=None, workspace=None,
                 one_sweep=True):
    """bsattn_block_energy: energy [B, H, T, T] (float32) = block sums of the
    full softmax attention probabilities of q, k ([B, H, N, d]).  With
    one_sweep (the default) a workspace of block_energy_workspace_bytes
    bytes is passed (`workspace`, a device uint8 tensor, or one allocated
    here); one_sweep=False passes none (the two-sweep kernel)."""
    import torch
    if q.dim() != 4 or tuple(k.shape) != tuple(q.shape):
        raise ValueError("q and k must share the shape [B, H, N, d]")
    B, H, N, d = q.shape
    t = num_tiles(N, tile) if N > 0 else 0
    if tuple(energy.shape) != (B, H, t, t):
        raise ValueError(f"energy must have shape {(B, H, t, t)}")
    ws_ptr, ws_bytes = None, 0
    if one_sweep and B * H * N > 0:
        need = block_energy_workspace_bytes(B, H, N, tile)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if workspace is not None:
            ws_ptr, ws_bytes = _ptr(workspace, "workspace", torch.uint8), workspace.numel()
    st = lib().bsattn_block_energy(B, H, N, d, tile, _dtype_code(q),
                                   _ptr(q, "q", q.dtype), _ptr(k, "k", q.dtype),
                                   _ptr(energy, "energy", torch.float32),
                                   float(scale), ws_ptr, ws_bytes, _stream(stream))
    _check(st, "bsattn_block_energy")
    return energy


def select_blocks(energy, eps: float, mask, stream=None):
    """bsattn_select_blocks over the last axis of energy [..., Tk] into the
    uint8 tensor mask of the same shape."""
    import torch
    if tuple(mask.shape) != tuple(energy.shape):
        raise ValueError("mask must have the shape of energy")
    Tk = energy.shape[-1] if energy.dim() else 0
    rows = energy.numel() // Tk if Tk else 0
    st = lib().bsattn_select_blocks(rows, Tk, _ptr(energy, "energy", torch.float32),
                                    float(eps), _ptr(mask, "mask", torch.uint8),
                                    _stream(stream))
    _check(st, "bsattn_select_blocks")
    return mask


def aggregate_masks(masks, rho: float, out, stream=None):
    """bsattn_aggregate_masks: out [...] = 1 where >= rho of the P masks
    [P, ...] select the cell."""
    import torch
    if tuple(out.shape) != tuple(masks.shape[1:]):
        raise ValueError("out must have the shape of one mask")
    st = lib().bsattn_aggregate_masks(masks.shape[0], out.numel(),
                                      _ptr(masks, "masks", torch.uint8), float(rho),
                                      _ptr(out, "out", torch.uint8), _stream(stream))
    _check(st, "bsattn_aggregate_masks")
    return out


def mfma_ceiling(blocks: int, iters: int, sink, stream=None) -> int:
    """bsattn_mfma_ceiling: enqueue the register-only bf16 MFMA
    microbenchmark; sink is a float32 device tensor of >= blocks entries.
    Returns the floating-point operations enqueued."""
    import torch
    if sink.numel() < blocks:
        raise ValueError("sink must hold at least `blocks` floats")
    n = lib().bsattn_mfma_ceiling(blocks, iters,
                                  _ptr(sink, "sink", torch.float32),
                                  _stream(stream))
    if n < 0:
        _check(int(n), "bsattn_mfma_ceiling")
    return int(n)


# ------------------------------------------------------- allocating helpers
def make_mask(frames, grid_h, grid_w, tile, device="cuda", stream=None,
              **params):
    import torch
    hm = params.get("mask_heads", 1)
    t = num_tiles(frames * grid_h * grid_w, tile)
    mask = torch.empty((hm, t, t), dtype=torch.uint8, device=device)
    return build_mask((frames, grid_h, grid_w, tile), mask, stream=stream,
                      **params)


def make_csr(mask, stream=None):
    import torch
    Hm, Tq, Tk = mask.shape
    row_ptr = torch.empty(Hm * Tq + 1, dtype=torch.int32, device=mask.device)
    col_idx = torch.empty(max(Hm * Tq * Tk, 1), dtype=torch.int32,
                          device=mask.device)
    return compact(mask, row_ptr, col_idx, stream=stream)


def attention(q, k, v, row_ptr, col_idx, tile, mask_heads=1, want_lse=False,
              scale=0.0, stream=None):
    import torch
    o = torch.empty_like(q)
    lse = None
    if want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fwd(q, k, v, o, row_ptr, col_idx, tile, mask_heads=mask_heads, lse=lse,
        scale=scale, stream=stream)
    return (o, lse) if want_lse else o


def attention_planned(q, k, v, row_ptr, col_idx, plan=None, mask_heads=1, want_lse=False,
                      workers=0, window=0, scale=0.0, stream=None):
    """As attention(), through a plan (built here from the CSR when None)."""
    import torch
    B, H, N, _ = q.shape
    if plan is None:
        plan = make_plan(row_ptr, col_idx, B, H, N, 128, mask_heads, workers, stream=stream)
    o = torch.empty_like(q)
    lse = None
    if want_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    fwd_planned(q, k, v, o, row_ptr, col_idx, plan, mask_heads=mask_heads, lse=lse,
                workers=workers, window=window, scale=scale, stream=stream)
    return (o, lse) if want_lse else o


def calibrate(q, k, tile, eps, rho, scale=0.0, stream=None, workspace=None):
    """The static mask [H, T, T] (uint8) from the prompts along q's and k's
    batch axis: block energies (one sweep, with `workspace` or one allocated
    here), per-prompt selection at eps, agreement at rho.  Returns (mask,
    energy, per_prompt_masks)."""
    import torch
    B, H, N, d = q.shape
    t = num_tiles(N, tile)
    energy = torch.empty((B, H, t, t), dtype=torch.float32, device=q.device)
    block_energy(q, k, energy, tile, scale=scale, stream=stream, workspace=workspace)
    sel = torch.empty((B, H, t, t), dtype=torch.uint8, device=q.device)
    select_blocks(energy, eps, sel, stream=stream)
    mask = torch.empty((H, t, t), dtype=torch.uint8, device=q.device)
    aggregate_masks(sel, rho, mask, stream=stream)
    return mask, energy, sel


def squad(q, k, v, w: int, tile: int, scale: float = 0.0, stream=None, grouped=None):
    """SQuad's two-pass attention through the library's calls: the local
    pass (block-diagonal mask, w / tile tiles per block) gives O_L; the
    global pass (block-diagonal, G / tile tiles per block, G = N / w) runs
    over the position-major order with O_L as values.  For bf16, d 128 and
    tile 128 the global pass reads and writes the window-major buffers
    through bsattn_fwd_grouped; otherwise (or with grouped=False) Q, K and
    O_L are reordered to position-major and the result back.  Needs w and
    N / w to be multiples of tile."""
    import torch
    B, H, N, d = q.shape
    if w % tile or N % w or (N // w) % tile:
        raise ValueError("w and N / w must be multiples of the tile size")
    G = N // w
    layout = (1, 1, N, tile)

    def pass_(qq, kk, vv, block_tiles):
        mask = make_mask(*layout, device=q.device, stream=stream,
                         kind=MASK_BLOCK_DIAGONAL, block_tiles=block_tiles)
        rp, ci = make_csr(mask, stream=stream)
        o = torch.empty_like(qq)
        fwd(qq, kk, vv, o, rp, ci, tile, scale=scale, stream=stream)
        return o

    o_local = pass_(q, k, v, w // tile)
    if grouped is None:
        grouped = q.dtype == torch.bfloat16 and d == 128 and tile == 128
    if grouped:
        mask = make_mask(*layout, device=q.device, stream=stream,
                         kind=MASK_BLOCK_DIAGONAL, block_tiles=G // tile)
        rp, ci = make_csr(mask, stream=stream)
        out = torch.empty_like(q)
        return fwd_grouped(q, k, o_local, out, rp, ci, w, scale=scale, stream=stream)
    qp, kp, op = torch.empty_like(q), torch.empty_like(k), torch.empty_like(o_local)
    window_reorder(q, qp, w, stream=stream)
    window_reorder(k, kp, w, stream=stream)
    window_reorder(o_local, op, w, stream=stream)
    og = pass_(qp, kp, op, G // tile)
    out = torch.empty_like(q)
    window_reorder(og, out, w, inverse=True, stream=stream)
    return out


def repeated_attention(q, k, v, frames, grid_h, grid_w, stride, tile, scale=0.0,
                       stream=None):
    """Attention of a repetitive head through the library's calls: the
    anchor rows' queries are gathered into blocks of two query tiles spread
    evenly over the sequence, full attention runs for those query tiles only
    (DENSE_ROWS_SPREAD mask), and every row takes its anchor row's output."""
    import torch
    B, H, N, d = q.shape
    na = frames * (-(-grid_h // stride)) * grid_w
    ta = -(-na // tile)
    bt = 2
    block_rows = bt * tile
    qa = torch.zeros_like(q)
    anchor_rows(q, qa, frames, grid_h, grid_w, stride, block_rows=block_rows, stream=stream)
    mask = make_mask(frames, grid_h, grid_w, tile, device=q.device, stream=stream,
                     kind=MASK_DENSE_ROWS_SPREAD, query_tiles=ta, block_tiles=bt)
    rp, ci = make_csr(mask, stream=stream)
    oa = torch.empty_like(q)
    fwd(qa, k, v, oa, rp, ci, tile, scale=scale, stream=stream)
    out = torch.empty_like(q)
    anchor_rows(oa, out, frames, grid_h, grid_w, stride, broadcast=True, block_rows=block_rows,
                stream=stream)
    return out


def mixed_layer_csr(flags, calibrated_mask, frames, grid_h, grid_w, stride, tile,
                    stream=None):
    """The block lists of CalibAtt's mixed inference layer (set up once per
    layer: flags and calibrated masks are static): per head, the spread
    anchor-row mask (DENSE_ROWS_SPREAD, blocks of two query tiles) when the
    head is repetitive, else its calibrated mask [H or 1, Tq, Tk].
    Returns (row_ptr, col_idx, mask) for mask_heads = H."""
    import torch
    H = flags.shape[0]
    na = frames * (-(-grid_h // stride)) * grid_w
    ta = -(-na // tile)
    rows = make_mask(frames, grid_h, grid_w, tile, device=flags.device, stream=stream,
                     kind=MASK_DENSE_ROWS_SPREAD, query_tiles=ta, block_tiles=2)
    out = torch.empty((H,) + tuple(rows.shape[1:]), dtype=torch.uint8, device=flags.device)
    mask_select(flags, rows, calibrated_mask, out, stream=stream)
    rp, ci = make_csr(out, stream=stream)
    return rp, ci, out


def mixed_attention(q, k, v, flags, row_ptr, col_idx, frames, grid_h, grid_w, stride, tile,
                    qbuf=None, obuf=None, out=None, scale=0.0, stream=None):
    """CalibAtt's inference layer with the lists of mixed_layer_csr: the
    repetitive heads' anchor-row queries are gathered into blocks spread over
    their rows (the other heads' queries copied), one forward runs every
    head on its own lists, and the repetitive heads' outputs are broadcast
    from their anchor rows (the other heads' copied).  qbuf, obuf and out
    are optional preallocated [B, H, N, d] buffers."""
    import torch
    block_rows = 2 * tile
    qbuf = torch.zeros_like(q) if qbuf is None else qbuf
    obuf = torch.empty_like(q) if obuf is None else obuf
    out = torch.empty_like(q) if out is None else out
    anchor_rows(q, qbuf, frames, grid_h, grid_w, stride, block_rows=block_rows, flags=flags,
                stream=stream)
    fwd(qbuf, k, v, obuf, row_ptr, col_idx, tile, mask_heads=q.shape[1], scale=scale,
        stream=stream)
    anchor_rows(obuf, out, frames, grid_h, grid_w, stride, broadcast=True,
                block_rows=block_rows, flags=flags, stream=stream)
    return out


def mask_params_of(spec) -> dict:
    """Keyword parameters of build_mask from an object with the fields of
    bsattn_mask_params (e.g. a workload's mask spec)."""
    return dict(kind=spec.kind, window=spec.window,
                num_anchors=spec.num_anchors, rotation=spec.rotation,
                seed=spec.seed, thresh24=spec.thresh24,
                force_diagonal=spec.force_diagonal,
                mask_heads=spec.mask_heads, budget=spec.budget,
                block_tiles=getattr(spec, "block_tiles", 1),
                query_tiles=getattr(spec, "query_tiles", 0))
