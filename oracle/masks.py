"""Oracle for the static block mask (test infrastructure only).

Follows the DiT block-sparse article:

* section 2.1: mask families (local window, per-modality block diagonal,
  global + local anchors);
* section 2.3: the mask is a 0/1 matrix over a block grid; sparsity is one
  minus the kept fraction of blocks;
* section 3.1: block boundaries line up with the token layout;
* section 3.2: the multimodal recipe (segments -> per-pair rule -> 0/1 block
  matrix -> sparse index);
* section 5.2: the mask is built with vectorised array operations, and
  padding keys never take part.

Reading (the pages give the families, not a formula): a token relation is
evaluated first (segment rules, anchors, valid length), and a (query tile,
key block) pair at tile sizes (Br, Bc) is kept iff at least one token pair
inside it is related.  The kernel computes every token pair of a kept block
("the block participates in QK^T, softmax and the weighted sum"), so the
token mask that defines the output is the tile mask expanded back to tokens,
intersected with the valid-key range and, when causal, with j <= i.
"""

from __future__ import annotations

import numpy as np

SEG_FULL, SEG_BLOCKWIN, SEG_IMAGE2D, SEG_VIDEO3D = 0, 1, 2, 3


def _segment_of(spec, idx: np.ndarray):
    """Segment number (-1 if none) and offset inside it, per token index."""
    seg = np.full(idx.shape, -1, dtype=np.int64)
    off = np.zeros(idx.shape, dtype=np.int64)
    for s, sg in enumerate(spec.segments):
        inside = (idx >= sg.start) & (idx < sg.start + sg.length)
        seg[inside] = s
        off[inside] = idx[inside] - sg.start
    return seg, off


def _segment_rule(sg, oq: np.ndarray, ok: np.ndarray) -> np.ndarray:
    """Pair rule inside one segment, broadcasting oq [n,1] against ok [1,m]."""
    if sg.kind == SEG_FULL:
        return np.ones(np.broadcast_shapes(oq.shape, ok.shape), dtype=bool)
    if sg.kind == SEG_BLOCKWIN:
        return np.abs(oq // sg.unit - ok // sg.unit) <= sg.radius
    if sg.kind == SEG_IMAGE2D:
        rq, cq = oq // sg.grid_w, oq % sg.grid_w
        rk, ck = ok // sg.grid_w, ok % sg.grid_w
        return (np.abs(rq - rk) <= sg.radius) & (np.abs(cq - ck) <= sg.radius)
    if sg.kind == SEG_VIDEO3D:
        fs = sg.grid_h * sg.grid_w
        fq, pq = oq // fs, oq % fs
        fk, pk = ok // fs, ok % fs
        rq, cq = pq // sg.grid_w, pq % sg.grid_w
        rk, ck = pk // sg.grid_w, pk % sg.grid_w
        same_frame = (fq == fk) & (np.abs(rq - rk) <= sg.radius) & (np.abs(cq - ck) <= sg.radius)
        df = np.abs(fq - fk)
        near_frame = (df >= 1) & (df <= sg.t_radius) & (pq // sg.unit == pk // sg.unit)
        return same_frame | near_frame
    raise ValueError(f"unknown segment kind {sg.kind}")


def token_relation(spec, qi, kj) -> np.ndarray:
    """Boolean [len(qi), len(kj)]: is query token qi related to key token kj.

    Anchors are global both ways; otherwise both tokens must sit in the same
    segment and satisfy its rule; keys >= n_valid and queries >= n_valid are
    never related."""
    qi = np.asarray(qi, dtype=np.int64)
    kj = np.asarray(kj, dtype=np.int64)
    sq, oq = _segment_of(spec, qi)
    sk, ok = _segment_of(spec, kj)
    out = np.zeros((qi.size, kj.size), dtype=bool)
    for s, sg in enumerate(spec.segments):
        rq = np.nonzero(sq == s)[0]
        ck = np.nonzero(sk == s)[0]
        if rq.size == 0 or ck.size == 0:
            continue
        out[np.ix_(rq, ck)] = _segment_rule(sg, oq[rq][:, None], ok[ck][None, :])
    a0, a1 = spec.anchor_start, spec.anchor_start + spec.anchor_len
    anc_q = (qi >= a0) & (qi < a1)
    anc_k = (kj >= a0) & (kj < a1)
    out |= anc_q[:, None] | anc_k[None, :]
    out &= (qi < spec.n_valid)[:, None] & (kj < spec.n_valid)[None, :]
    return out


def tile_mask_rows(spec, n_q: int, n_k: int, Br: int, Bc: int, tiles) -> np.ndarray:
    """Kept key blocks for the listed query tiles: bool [len(tiles), ceil(n_k/Bc)]."""
    Tc = -(-n_k // Bc)
    keys = np.arange(n_k)
    out = np.zeros((len(tiles), Tc), dtype=bool)
    for a, t in enumerate(tiles):
        rows = np.arange(t * Br, min((t + 1) * Br, n_q))
        rel = token_relation(spec, rows, keys)
        pad = np.zeros((rows.size, Tc * Bc), dtype=bool)
        pad[:, :n_k] = rel
        out[a] = pad.reshape(rows.size, Tc, Bc).any(axis=(0, 2))
    return out


def tile_mask(spec, n_q: int, n_k: int, Br: int, Bc: int) -> np.ndarray:
    """The full (Tr, Tc) 0/1 block matrix of the article's section 2.3."""
    Tr = -(-n_q // Br)
    return tile_mask_rows(spec, n_q, n_k, Br, Bc, range(Tr))


def csr_from_tile_mask(tm: np.ndarray):
    """Per-query-tile list of kept key blocks, ascending: (row_ptr, col_idx) int32."""
    counts = tm.sum(axis=1)
    row_ptr = np.zeros(tm.shape[0] + 1, dtype=np.int32)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.nonzero(tm)[1].astype(np.int32)   # row-major order: ascending per row
    return row_ptr, col_idx


def sparsity(n_kept: int, n_total: int) -> float:
    """Article section 2.3: sparsity = 1 - nonzero_blocks / total_blocks."""
    return 1.0 - n_kept / n_total


def bitmap_bytes(n_blocks_q: int, n_blocks_k: int) -> int:
    """Article section 2.3: one bit per block."""
    return (n_blocks_q * n_blocks_k + 7) // 8


def expand_token_mask(tm: np.ndarray, n_q: int, n_k: int, Br: int, Bc: int,
                      n_valid: int, causal: bool) -> np.ndarray:
    """Token mask M[i, j] = tile_mask[i // Br, j // Bc] and j < n_valid and (not causal or j <= i)."""
    i = np.arange(n_q)
    j = np.arange(n_k)
    M = tm[i // Br][:, j // Bc]
    M &= (j < n_valid)[None, :]
    if causal:
        M &= j[None, :] <= i[:, None]
    return M
