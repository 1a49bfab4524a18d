"""The five synthetic workloads and their block-mask specifications.

Mask specifications are plain descriptions of a token layout (segments,
anchors, valid length).  What a specification *means* at token level is
defined by the oracle (``oracle/masks.py``) and independently by the C++
block-index builder; this module only records the layout.

Segment kinds (the mask families of the DiT block-sparse article, section 2.1
"local window / block-diagonal / global+local anchors", and its section 3.2
multimodal recipe):

* ``SEG_FULL``     - every token of the segment attends every token of the
  same segment (a per-modality block-diagonal segment).
* ``SEG_BLOCKWIN`` - 1-D local window on base units: tokens i, j of the
  segment are paired iff their unit indices (offset within the segment
  divided by ``unit``) differ by at most ``radius``.
* ``SEG_IMAGE2D``  - a ``grid_h x grid_w`` patch grid in row-major order:
  paired iff the row and the column distance are both at most ``radius``.
* ``SEG_VIDEO3D``  - ``frames`` stacked ``grid_h x grid_w`` grids: inside one
  frame as ``SEG_IMAGE2D``; across frames at distance 1..``t_radius`` paired
  iff both tokens sit in the same spatial unit (offset within the frame
  divided by ``unit``).

Anchors ``[anchor_start, anchor_start + anchor_len)`` are global both ways.
Keys at or beyond ``n_valid`` are padding and are never paired; query rows at
or beyond ``n_valid`` pair with nothing.  The kernel works on the block mask
obtained by rounding this token relation up to (Br, Bc) tiles.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

SEG_FULL = 0
SEG_BLOCKWIN = 1
SEG_IMAGE2D = 2
SEG_VIDEO3D = 3


@dataclass(frozen=True)
class Segment:
    kind: int
    start: int
    length: int
    frames: int = 1
    grid_h: int = 0
    grid_w: int = 0
    radius: int = 0
    t_radius: int = 0
    unit: int = 64


@dataclass(frozen=True)
class MaskSpec:
    n_valid: int
    segments: Tuple[Segment, ...]
    anchor_start: int = 0
    anchor_len: int = 0


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    description: str
    dtype: str                 # "fp32" or "bf16"
    B: int
    Hq: int
    Hkv: int
    N: int                     # tensor length (Nq == Nk), padded
    d: int
    Br: int
    Bc: int
    causal: bool
    lam: float                 # 0 = no dynamic skipping
    mask: Optional[MaskSpec]   # None = dense (or dense causal)
    seed: int
    generator: str             # "iid", "iid_offset", "concentrated", "sink", "sink_last"

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def n_valid(self) -> int:
        return self.mask.n_valid if self.mask is not None else self.N


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    description: str
    B: int
    Hq: int
    Hkv: int
    L: int
    d: int
    Bc: int
    lam: float
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


def _cfg1() -> PrefillWorkload:
    spec = MaskSpec(n_valid=512,
                    segments=(Segment(SEG_BLOCKWIN, 0, 512, unit=64, radius=1),))
    return PrefillWorkload(
        name="cfg1", description="static local-window block mask, fp32, B1 H2 N512 d64, window +-1 block",
        dtype="fp32", B=1, Hq=2, Hkv=2, N=512, d=64, Br=64, Bc=64, causal=False, lam=0.0,
        mask=spec, seed=1, generator="iid")


def dit_image_text_spec(grid: int = 64, text: int = 256, radius: int = 8, anchors: int = 64,
                        unit: int = 64) -> MaskSpec:
    """Image tokens first (row-major grid), then the text segment; the first
    ``anchors`` text tokens are global anchors."""
    n_img = grid * grid
    n = n_img + text
    return MaskSpec(
        n_valid=n,
        segments=(Segment(SEG_IMAGE2D, 0, n_img, grid_h=grid, grid_w=grid, radius=radius, unit=unit),
                  Segment(SEG_FULL, n_img, text)),
        anchor_start=n_img, anchor_len=anchors)


def video_text_spec(frames: int = 16, grid: int = 64, text: int = 320, radius: int = 8,
                    t_radius: int = 2, anchors: int = 64, unit: int = 64) -> MaskSpec:
    n_vid = frames * grid * grid
    n = n_vid + text
    return MaskSpec(
        n_valid=n,
        segments=(Segment(SEG_VIDEO3D, 0, n_vid, frames=frames, grid_h=grid, grid_w=grid,
                          radius=radius, t_radius=t_radius, unit=unit),
                  Segment(SEG_FULL, n_vid, text)),
        anchor_start=n_vid, anchor_len=anchors)


def _cfg2() -> PrefillWorkload:
    return PrefillWorkload(
        name="cfg2", description="multimodal DiT image+text, bf16, B2 H16 N4352 d64, 2-D window +-8, text segment, 64 anchors",
        dtype="bf16", B=2, Hq=16, Hkv=16, N=4352, d=64, Br=128, Bc=64, causal=False, lam=0.0,
        mask=dit_image_text_spec(), seed=2, generator="iid_offset")


def _cfg3() -> PrefillWorkload:
    spec = video_text_spec()
    n_pad = ((spec.n_valid + 127) // 128) * 128
    return PrefillWorkload(
        name="cfg3", description="video DiT, bf16, B1 H24 d128, 16x4096 video + 320 text = 65856 padded to 65920",
        dtype="bf16", B=1, Hq=24, Hkv=24, N=n_pad, d=128, Br=128, Bc=64, causal=False, lam=0.0,
        mask=spec, seed=3, generator="iid")


def _cfg4() -> PrefillWorkload:
    L = 32768
    return PrefillWorkload(
        name="cfg4", description="BLASST dynamic prefill, bf16, causal GQA 32/8, d128, L32768, lambda=40/L",
        dtype="bf16", B=1, Hq=32, Hkv=8, N=L, d=128, Br=128, Bc=64, causal=True, lam=40.0 / L,
        mask=None, seed=4, generator="concentrated")


def _cfg5() -> DecodeWorkload:
    L = 131072
    return DecodeWorkload(
        name="cfg5", description="BLASST dynamic decode, bf16 KV cache [32,131072,8,128], GQA 32/8, lambda=40/L",
        B=32, Hq=32, Hkv=8, L=L, d=128, Bc=64, lam=40.0 / L, seed=5)


def _cfg4_sink() -> PrefillWorkload:
    """The causal GQA 32/8 prefill shape with the "sink" test recipe, whose
    tiles really skip at moderate lambda (the speed-up against sparsity curve)."""
    c = _cfg4()
    return PrefillWorkload(
        name="cfg4_sink", description="causal GQA 32/8, d128, L32768, sink recipe (skips whole tiles at lambda 0.3-0.7)",
        dtype="bf16", B=c.B, Hq=c.Hq, Hkv=c.Hkv, N=c.N, d=c.d, Br=128, Bc=64, causal=True, lam=0.5,
        mask=None, seed=c.seed, generator="sink")


CONFIGS = {"cfg1": _cfg1, "cfg2": _cfg2, "cfg3": _cfg3, "cfg4": _cfg4, "cfg5": _cfg5}
EXTRA = {"cfg4_sink": _cfg4_sink}


def get_config(name: str):
    return CONFIGS[name]() if name in CONFIGS else EXTRA[name]()
