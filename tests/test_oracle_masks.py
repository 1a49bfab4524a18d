"""Pins for the block-mask oracle (CPU only).

* brute force: a pure-Python pair loop written directly from the segment
  definitions, on tiny grids, against the vectorised oracle;
* the article's worked block-grid example (tests/golden);
* block counts of the workload masks, re-derived by hand for cfg1 and by
  a direct count of the band structure for cfg2.
"""

import json
import os

import numpy as np
import pytest

from oracle import masks as M
from workloads import get_config
from workloads.configs import (MaskSpec, Segment, SEG_FULL, SEG_BLOCKWIN, SEG_IMAGE2D, SEG_VIDEO3D,
                               dit_image_text_spec, video_text_spec)

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _brute_related(spec, i, j):
    """One token pair, straight from the definitions (no arrays)."""
    if i >= spec.n_valid or j >= spec.n_valid:
        return False
    a0, a1 = spec.anchor_start, spec.anchor_start + spec.anchor_len
    if a0 <= i < a1 or a0 <= j < a1:
        return True
    for sg in spec.segments:
        if sg.start <= i < sg.start + sg.length and sg.start <= j < sg.start + sg.length:
            oi, oj = i - sg.start, j - sg.start
            if sg.kind == SEG_FULL:
                return True
            if sg.kind == SEG_BLOCKWIN:
                return abs(oi // sg.unit - oj // sg.unit) <= sg.radius
            if sg.kind == SEG_IMAGE2D:
                ri, ci = divmod(oi, sg.grid_w)
                rj, cj = divmod(oj, sg.grid_w)
                return abs(ri - rj) <= sg.radius and abs(ci - cj) <= sg.radius
            if sg.kind == SEG_VIDEO3D:
                fsz = sg.grid_h * sg.grid_w
                fi, pi = divmod(oi, fsz)
                fj, pj = divmod(oj, fsz)
                ri, ci = divmod(pi, sg.grid_w)
                rj, cj = divmod(pj, sg.grid_w)
                if fi == fj:
                    return abs(ri - rj) <= sg.radius and abs(ci - cj) <= sg.radius
                return abs(fi - fj) <= sg.t_radius and pi // sg.unit == pj // sg.unit
    return False


def _brute_tile_mask(spec, n, Br, Bc):
    Tr, Tc = -(-n // Br), -(-n // Bc)
    tm = np.zeros((Tr, Tc), bool)
    for i in range(n):
        for j in range(n):
            if _brute_related(spec, i, j):
                tm[i // Br, j // Bc] = True
    return tm


SMALL_SPECS = {
    "blockwin": MaskSpec(n_valid=180, segments=(Segment(SEG_BLOCKWIN, 0, 180, unit=16, radius=1),)),
    "image_text": dit_image_text_spec(grid=12, text=40, radius=2, anchors=8, unit=12),
    "video_text": video_text_spec(frames=4, grid=8, text=24, radius=1, t_radius=1, anchors=8, unit=8),
    "video_text_pad": MaskSpec(n_valid=4 * 64 + 20, segments=(
        Segment(SEG_VIDEO3D, 0, 4 * 64, frames=4, grid_h=8, grid_w=8, radius=2, t_radius=2, unit=16),
        Segment(SEG_FULL, 256, 20)), anchor_start=256, anchor_len=5),
}


@pytest.mark.parametrize("name", sorted(SMALL_SPECS))
@pytest.mark.parametrize("tiles", [(16, 16), (32, 16), (24, 8)])
def test_tile_mask_equals_brute_force(name, tiles):
    spec = SMALL_SPECS[name]
    n = spec.n_valid + 13                  # padded tensor with a ragged tail
    Br, Bc = tiles
    assert np.array_equal(M.tile_mask(spec, n, n, Br, Bc), _brute_tile_mask(spec, n, Br, Bc))


def test_token_relation_equals_brute_force():
    spec = SMALL_SPECS["video_text_pad"]
    n = spec.n_valid + 9
    rel = M.token_relation(spec, np.arange(n), np.arange(n))
    for i in range(0, n, 3):
        for j in range(n):
            assert rel[i, j] == _brute_related(spec, i, j)


def test_article_block_grid_example():
    g = json.load(open(os.path.join(GOLD, "dit_article_block_grid.json")))
    nb = g["seq_len"] // g["block"]
    assert nb == g["blocks_per_side"]
    assert M.bitmap_bytes(nb, nb) == g["bitmap_bytes"]
    assert M.sparsity(g["kept_blocks"], g["total_blocks"]) == g["sparsity"]


def test_cfg1_counts_by_hand():
    """+-1 block window on 8 blocks: 8 diagonal + 2*7 off-diagonal = 22 (Br=64);
    at Br=128 each of the 4 tiles keeps its 2 blocks plus one neighbour per side: 3+4+4+3 = 14."""
    c = get_config("cfg1")
    assert M.tile_mask(c.mask, 512, 512, 64, 64).sum() == 22
    assert M.tile_mask(c.mask, 512, 512, 128, 64).sum() == 14


def test_cfg2_counts():
    """Image rows (one 64-token block per patch row) see +-8 rows: band of 17
    around each of 64 rows, minus the clipped corners; every image block also
    keeps the anchor block (block 64), the anchor/text tiles keep everything."""
    c = get_config("cfg2")
    tm64 = M.tile_mask(c.mask, c.N, c.N, 64, 64)
    band = sum(min(63, r + 8) - max(0, r - 8) + 1 for r in range(64))
    # image rows: band + anchor block 64; anchor row 64: all 68; text rows 65..67: text blocks 64..67 + all image (anchors? no)
    image_rows = band + 64
    anchor_row = 68
    text_rows = 3 * 4
    assert tm64.sum() == image_rows + anchor_row + text_rows == 1160
    assert M.tile_mask(c.mask, c.N, c.N, 128, 64).sum() == 640


@pytest.mark.slow
def test_cfg3_sampled_tiles():
    c = get_config("cfg3")
    rows = M.tile_mask_rows(c.mask, c.N, c.N, 128, 64, [0, 1, 31, 32, 100, 511, 512, 513, 514])
    # anchor tile 512 (tokens 65536..65663) sees every valid block (1029); pure pad block 1029 never kept
    assert rows[6].sum() == 1029 and not rows[:, 1029].any()
    # last tile: text rows see text blocks 1024..1028 plus anchor rows... and no image (text is not global)
    assert rows[8].sum() == 5
