"""Seeded synthetic workloads for block-sparse video attention.

This module holds only shapes, mask parameters and seeded random inputs.  It
does none of the method's arithmetic: no masks, no tile lists, no attention.
Both the CPU oracle's tests and the HIP path's tests and benchmark draw their
inputs from here, so the two sides always see identical values.

The shapes follow the video diffusion transformers the pages study (a 21-frame
latent horizon for Wan 2.1, LVSA page, "Meccanismo Core"; 128x128 attention
blocks, CalibAtt page, "A. Fase di Calibrazione").  Real activations and model
weights are not available, so Q, K and V are i.i.d. N(0, 1) draws at those
shapes; VBench-style quality suites are out of scope entirely.

Token order is frame-major: token n = f*P + y*grid_w + x with P = grid_h*grid_w.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import torch

# Mask kinds, numbered as in include/bsattn.h.
MASK_WINDOW_ANCHOR = 0
MASK_STATIC_RANDOM = 1
MASK_DENSE = 2
MASK_WINDOW_ANCHOR_EXPANDED = 3
MASK_BLOCK_DIAGONAL = 4
MASK_DENSE_ROWS = 5
MASK_DENSE_ROWS_SPREAD = 6

DTYPE_BF16 = 0
DTYPE_F32 = 1


def thresh24_for_density(p: float) -> int:
    """24-bit threshold of the static random mask: a tile is drawn active when
    the top 24 bits of its hash are below floor(p * 2**24)."""
    if not (0.0 <= p <= 1.0):
        raise ValueError("density must lie in [0, 1]")
    return min(int(p * (1 << 24)), 1 << 24)


@dataclass(frozen=True)
class MaskSpec:
    kind: int
    window: int = 0          # half-width w, in frames
    num_anchors: int = 0     # n_a global anchor frames
    rotation: int = 0        # r, reduced mod T by the mask builder
    seed: int = 0            # static mode
    thresh24: int = 0        # static mode
    force_diagonal: int = 0  # static mode
    mask_heads: int = 1      # Hm: 1 (shared by all heads) or H
    budget: int = 0          # C, frames per query frame (expanded windows)
    block_tiles: int = 1     # tiles per diagonal block (block-diagonal mode)
    query_tiles: int = 0     # dense query tiles (dense-rows mode)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    frames: int
    grid_h: int
    grid_w: int
    tile: int
    dtype: int
    mask: MaskSpec
    seed: int
    # rotations a run sweeps through (the step index for the tiny case,
    # (layer + step) mod T for the video shapes)
    rotations: tuple = field(default=(0,))

    @property
    def P(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def N(self) -> int:
        return self.frames * self.P

    @property
    def num_tiles(self) -> int:
        return -(-self.N // self.tile)

    def with_rotation(self, r: int) -> "Workload":
        return replace(self, mask=replace(self.mask, rotation=r))

    def with_mask(self, **kw) -> "Workload":
        return replace(self, mask=replace(self.mask, **kw))

    def torch_dtype(self):
        return torch.float32 if self.dtype == DTYPE_F32 else torch.bfloat16


# The five workloads.  Index 1 is the small case the oracle finishes in
# seconds; index 2 is the 32 760-token video shape the headline metric uses.
WORKLOADS = {
    1: Workload("tiny_4x8x8_tile64", B=1, H=2, d=64, frames=4, grid_h=8, grid_w=8,
                tile=64, dtype=DTYPE_F32,
                mask=MaskSpec(MASK_WINDOW_ANCHOR, window=1, num_anchors=1),
                seed=1001, rotations=(0, 1, 2, 3)),
    2: Workload("video_21x30x52_window_anchor", B=1, H=12, d=128, frames=21,
                grid_h=30, grid_w=52, tile=128, dtype=DTYPE_BF16,
                mask=MaskSpec(MASK_WINDOW_ANCHOR, window=1, num_anchors=2),
                seed=1002, rotations=tuple(range(21))),
    3: Workload("video_21x30x52_static_p30", B=1, H=12, d=128, frames=21,
                grid_h=30, grid_w=52, tile=128, dtype=DTYPE_BF16,
                mask=MaskSpec(MASK_STATIC_RANDOM, seed=3,
                              thresh24=thresh24_for_density(0.3),
                              force_diagonal=1, mask_heads=12),
                seed=1003),
    4: Workload("long_84x30x52_window_anchor", B=1, H=12, d=128, frames=84,
                grid_h=30, grid_w=52, tile=128, dtype=DTYPE_BF16,
                mask=MaskSpec(MASK_WINDOW_ANCHOR, window=2, num_anchors=4),
                seed=1004, rotations=tuple(range(84))),
    5: Workload("dense_21x30x52_h40", B=1, H=40, d=128, frames=21, grid_h=30,
                grid_w=52, tile=128, dtype=DTYPE_BF16,
                mask=MaskSpec(MASK_DENSE), seed=1005),
}


# The 32 760-token video shape at head dim 64 and 64 x 64 tiles (24 heads of
# 64: the same width as 12 of 128), window/anchor mask as index 2: the
# measurement and parity case of the d = 64 / tile 64 kernel.
VIDEO_D64 = Workload("video_21x30x52_d64_t64_window_anchor", B=1, H=24, d=64, frames=21,
                     grid_h=30, grid_w=52, tile=64, dtype=DTYPE_BF16,
                     mask=MaskSpec(MASK_WINDOW_ANCHOR, window=1, num_anchors=2),
                     seed=1007, rotations=tuple(range(21)))


# The long-video shape with the LVSA expanded adaptive windows: every query
# frame attends to a budget of C = 21 frames (the 21-frame training horizon),
# made of 4 rotating anchors and a window grown from +/-2 frames.  A parity and
# measurement case of the expanded mask mode, beside the five above.
EXPANDED = Workload("long_84x30x52_expanded_c21", B=1, H=12, d=128, frames=84,
                    grid_h=30, grid_w=52, tile=128, dtype=DTYPE_BF16,
                    mask=MaskSpec(MASK_WINDOW_ANCHOR_EXPANDED, window=2,
                                  num_anchors=4, budget=21),
                    seed=1006, rotations=tuple(range(84)))


# The shapes only the generic forward takes, at the 32 760-token video size
# with the window/anchor mask: fp32 I/O at d 128 / tile 128, bf16 at d 128 /
# tile 64, bf16 at d 64 / tile 128 (24 heads).
GENERIC = tuple(
    replace(WORKLOADS[2], name=f"video_21x30x52_{'f32' if dt == DTYPE_F32 else 'bf16'}_d{d}_t{t}",
            dtype=dt, d=d, tile=t, H=h)
    for dt, d, t, h in ((DTYPE_F32, 128, 128, 12), (DTYPE_BF16, 128, 64, 12),
                        (DTYPE_BF16, 64, 128, 24)))


def make_qkv(w: Workload, seed: Optional[int] = None, device: str = "cpu"):
    """Q, K, V of shape [B, H, N, d] drawn i.i.d. N(0, 1) in float32 from a CPU
    generator (seeded, in the order Q, K, V), then rounded to the workload's
    dtype (round-to-nearest-even for bf16)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    shape = (w.B, w.H, w.N, w.d)
    out = []
    for _ in range(3):
        x = torch.randn(shape, generator=g, dtype=torch.float32)
        out.append(x.to(w.torch_dtype()).to(device))
    return tuple(out)


def make_qk_frame_local(w: Workload, strength: float = 1.0,
                        seed: Optional[int] = None, device: str = "cpu"):
    """Q and K with a shared per-(head, frame) component, so a query scores
    the keys of its own frame higher (attention concentrates locally, the
    structure calibration is meant to find): q_n = a_n + strength * c_f(n),
    k_n = b_n + strength * c_f(n), with a, b, c i.i.d. N(0, 1), the same c for
    every batch entry (prompt) and a, b drawn per batch entry.  Rounded to
    the workload's dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    c = torch.randn((1, w.H, w.frames, w.d), generator=g, dtype=torch.float32)
    cf = c.repeat_interleave(w.P, dim=2)                   # [1, H, N, d]
    q = torch.randn((w.B, w.H, w.N, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.H, w.N, w.d), generator=g, dtype=torch.float32)
    q = q + strength * cf
    k = k + strength * cf
    return (q.to(w.torch_dtype()).to(device), k.to(w.torch_dtype()).to(device))


def make_qk_row_repetitive(w: Workload, rep_heads: int, noise: float = 0.1,
                           seed: Optional[int] = None, device: str = "cpu",
                           local_strength: float = 0.0):
    """Q and K where, in heads 0 .. rep_heads-1, every spatial row of a frame
    repeats one per-frame row of queries plus N(0, noise^2) noise (the rows
    of a frame then attend alike); the other heads are i.i.d. N(0, 1), plus,
    when local_strength > 0, a shared per-(head, frame) component of that
    strength in both Q and K (their attention then concentrates on the
    query's own frame, as make_qk_frame_local).  K is otherwise i.i.d.
    N(0, 1).  Rounded to the workload's dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    q = torch.randn((w.B, w.H, w.N, w.d), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.H, w.N, w.d), generator=g, dtype=torch.float32)
    if rep_heads > 0:
        row = torch.randn((w.B, rep_heads, w.frames, 1, w.grid_w, w.d), generator=g)
        jit = noise * torch.randn((w.B, rep_heads, w.frames, w.grid_h, w.grid_w, w.d),
                                  generator=g)
        q[:, :rep_heads] = (row + jit).reshape(w.B, rep_heads, w.N, w.d)
    if local_strength > 0 and rep_heads < w.H:
        c = torch.randn((1, w.H - rep_heads, w.frames, w.d), generator=g)
        cf = c.repeat_interleave(w.P, dim=2)
        q[:, rep_heads:] += local_strength * cf
        k[:, rep_heads:] += local_strength * cf
    return (q.to(w.torch_dtype()).to(device), k.to(w.torch_dtype()).to(device))


def make_energies(rows: int, tk: int, seed: int, zero_frac: float = 0.1,
                  tie_frac: float = 0.1) -> torch.Tensor:
    """Synthetic float32 block energies [rows, tk] >= 0: heavy-tailed values
    (u^4 for u uniform), a fraction set to exactly 0, and a fraction copied
    from another entry of the same row (exact ties)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    e = torch.rand((rows, tk), generator=g, dtype=torch.float32) ** 4
    z = torch.rand((rows, tk), generator=g) < zero_frac
    e[z] = 0.0
    t = torch.rand((rows, tk), generator=g) < tie_frac
    src = torch.randint(0, tk, (rows, tk), generator=g)
    e = torch.where(t, torch.gather(e, 1, src), e)
    return e


def make_prompt_masks(p: int, cells: int, seed: int, density: float = 0.5):
    """Random uint8 masks [p, cells] (each cell 1 with the given probability)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (torch.rand((p, cells), generator=g) < density).to(torch.uint8)


# The static-mask calibration case at the video shape: four prompts (batch
# entries) with frame-local structure.  rho = 0.5 is the CalibAtt page's
# example; the page gives no number for eps (a per-step schedule, higher
# early in denoising), so 0.9 stands for one step of it.
CALIB = Workload("video_21x30x52_calib_p4", B=4, H=12, d=128, frames=21,
                 grid_h=30, grid_w=52, tile=128, dtype=DTYPE_BF16,
                 mask=MaskSpec(MASK_DENSE), seed=1007)
CALIB_EPS = 0.9
CALIB_RHO = 0.5


# SQuad's two-pass attention at a 65 536-token latent (16 frames of 64x64):
# windows of w = 256 = sqrt(N) consecutive tokens, so both the local pass
# (256 windows) and the global pass (256 position groups of 256 tokens) are
# block-diagonal with 2 x 2-tile blocks.  The mask spec is unused (each pass
# builds its own block-diagonal mask).
SQUAD = Workload("squad_16x64x64_w256", B=1, H=12, d=128, frames=16,
                 grid_h=64, grid_w=64, tile=128, dtype=DTYPE_BF16,
                 mask=MaskSpec(MASK_BLOCK_DIAGONAL, block_tiles=2), seed=1008)
SQUAD_W = 256


def small_workload(frames=3, grid_h=5, grid_w=9, tile=64, d=64, H=2, B=1,
                   dtype=DTYPE_BF16, mask: Optional[MaskSpec] = None,
                   seed=77, name="small") -> Workload:
    """A reduced workload for tests: several tiles and a ragged last tile."""
    if mask is None:
        mask = MaskSpec(MASK_WINDOW_ANCHOR, window=1, num_anchors=1)
    return Workload(name, B=B, H=H, d=d, frames=frames, grid_h=grid_h,
                    grid_w=grid_w, tile=tile, dtype=dtype, mask=mask, seed=seed)
