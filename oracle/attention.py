"""Oracle for masked, block-sparse and BLASST attention in float64 (test infrastructure only).

Sources (see the package docstring for page titles):

* Attention definition, out = softmax(Q K^T / sqrt(d_k)) V: BLASST notes,
  section 3.1.1.
* Masked entries are absent from the softmax statistics (not filled with a
  large negative value): DiT article, section 5.2.
* Online softmax (running max m, running sum l, rescale by exp(m_old-m_new)):
  attention tutorial, section 4.2; BLASST notes, Algorithm 1.
* Skip rule: after the running-max update, skip the block when its block
  maximum minus the running maximum is below ln(lambda): BLASST notes,
  section 3.1.1 and Algorithm 1; decision shared by the whole tile
  (per-thread predicate, vote, shared flag): BLASST notes, section 4.
* GQA: query head h reads K/V head h // (Hq / Hkv) (consecutive groups, as
  ``repeat_interleave`` on the tutorial's GQA section).

Readings (pages silent or ambiguous):

1. Scores are compared in the scaled domain: S = scale * Q K^T, since the
   softmax being approximated is of the scaled scores and exp(S - m) must be
   its numerator.
2. The vote is tile-uniform: a block is skipped only if every row of the
   tile satisfies the condition; a row with no allowed key in the block
   (block max = -inf) satisfies it.
3. "<" is strict, as printed.  lambda = 0 means ln(lambda) = -inf: never skip.
   lambda must lie in [0, 1).
4. Blocks are visited in ascending key-block order (CSR order for a static
   mask); under a causal mask, blocks lying wholly above the diagonal are
   not visited.
5. Rows with no allowed key at all produce zeros.
6. Decode: the tile is the G query heads that share one K/V head; the
   running maximum runs over the whole key sequence in ascending order, so
   the skip set does not depend on how a kernel splits the sequence.
"""

from __future__ import annotations

import math

import numpy as np


def as_f64(x) -> np.ndarray:
    """Exact upcast of a torch tensor (bf16/fp32) or array to float64 numpy."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """GQA grouping: consecutive groups of Hq/Hkv query heads share a K/V head."""
    return h // (Hq // Hkv)


def log_threshold(lam: float) -> float:
    if not (0.0 <= lam < 1.0):
        raise ValueError("lambda must lie in [0, 1)")
    return -math.inf if lam == 0.0 else math.log(lam)


# ---------------------------------------------------------------------------
# plain definition: masked softmax attention
# ---------------------------------------------------------------------------

def masked_attention(q, k, v, allowed, scale: float, return_probs: bool = False):
    """softmax over the allowed entries of scale * q k^T, times v.

    q [Nq, d], k [Nk, d], v [Nk, dv], allowed bool [Nq, Nk].  Disallowed
    entries are left out of max, exponent and sum; a row with no allowed
    entry returns zeros."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    S = scale * (q @ k.T)
    S = np.where(allowed, S, -np.inf)
    has = allowed.any(axis=1)
    m = np.where(has, S.max(axis=1, initial=-np.inf), 0.0)
    P = np.where(allowed, np.exp(S - m[:, None]), 0.0)
    l = P.sum(axis=1)
    denom = np.where(has, l, 1.0)
    P = P / denom[:, None]
    out = P @ v
    if return_probs:
        return out, P
    return out


# ---------------------------------------------------------------------------
# tiles, visited blocks, allowed entries
# ---------------------------------------------------------------------------

def tile_rows(t: int, Br: int, n_q: int) -> np.ndarray:
    return np.arange(t * Br, min((t + 1) * Br, n_q))


def visited_blocks(t: int, Br: int, Bc: int, n_q: int, n_k: int, causal: bool,
                   row_ptr=None, col_idx=None, order: str = "ascending") -> np.ndarray:
    """Key blocks visited by query tile t: the tile's CSR list (or every block),
    minus blocks wholly above the diagonal when causal, in ascending order
    (Algorithm 1) or descending order (most recent keys first: the block-row
    reordering the BLASST notes study, which finds a running max closer to
    the row's global maximum sooner)."""
    Tc = -(-n_k // Bc)
    if row_ptr is None:
        blocks = np.arange(Tc)
    else:
        blocks = np.asarray(col_idx[row_ptr[t]:row_ptr[t + 1]], dtype=np.int64)
    if causal:
        last_row = min((t + 1) * Br, n_q) - 1
        blocks = blocks[blocks * Bc <= last_row]
    if order == "descending":
        blocks = blocks[::-1].copy()
    elif order != "ascending":
        raise ValueError(order)
    return blocks


def allowed_entries(rows: np.ndarray, keys: np.ndarray, n_valid: int, causal: bool) -> np.ndarray:
    a = np.broadcast_to((keys < n_valid)[None, :], (rows.size, keys.size)).copy()
    if causal:
        a &= keys[None, :] <= rows[:, None]
    return a


def block_keys(j: int, Bc: int, n_k: int) -> np.ndarray:
    return np.arange(j * Bc, min((j + 1) * Bc, n_k))


# ---------------------------------------------------------------------------
# Algorithm 1 (FlashAttention with BLASST), one query tile
# ---------------------------------------------------------------------------

def blasst_tile(qr, k, v, rows, blocks, Bc: int, scale: float, lam: float,
                n_valid: int, causal: bool, force=None):
    """Algorithm 1 of the BLASST notes for one query tile, in float64.

    qr [R, d] are the tile's query rows (token indices ``rows``), k/v the
    K/V head [Nk, d].  ``blocks`` are visited in the given (ascending) order.
    For each block: scores, block row max, running max update, tile-wide
    skip test, then (if kept) exponent, rescaled row sum and rescaled output.

    ``force`` optionally maps a position in ``blocks`` to a forced decision;
    tests use it only for blocks whose margin lies within the accepted band
    around the threshold.

    Returns (out [R, dv], skip bool [nb], margin [nb]) where margin is the
    largest (block max - running max) over rows with a finite block max,
    minus ln(lambda) (-inf if no such row; +inf when lambda = 0)."""
    qr, k, v = as_f64(qr), as_f64(k), as_f64(v)
    lnl = log_threshold(lam)
    R = qr.shape[0]
    n_k = k.shape[0]
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    O = np.zeros((R, v.shape[1]))
    skip = np.zeros(len(blocks), dtype=bool)
    margin = np.full(len(blocks), -np.inf)
    for pos, j in enumerate(blocks):
        keys = block_keys(int(j), Bc, n_k)
        allowed = allowed_entries(rows, keys, n_valid, causal)
        S = np.where(allowed, scale * (qr @ k[keys].T), -np.inf)
        m_blk = S.max(axis=1)                      # local (block) max, -inf if none
        m_new = np.maximum(m, m_blk)               # running max, updated before the test
        finite = np.isfinite(m_blk)
        gap = np.where(finite, m_blk - np.where(finite, m_new, 0.0), -np.inf)
        agree = ~finite | (gap < lnl)
        margin[pos] = (gap[finite].max() - lnl) if finite.any() else -np.inf
        if lam == 0.0:
            margin[pos] = np.inf
        s = bool(agree.all()) and lam > 0.0
        if force is not None and pos in force:
            s = bool(force[pos])
        skip[pos] = s
        if s:
            m = m_new
            continue
        # rows whose running max is still -inf have accumulated nothing
        live = np.isfinite(m_new)
        alpha = np.where(np.isfinite(m) & live, np.exp(np.where(live, m, 0.0) - np.where(live, m_new, 0.0)), 0.0)
        P = np.where(allowed & live[:, None], np.exp(S - np.where(live, m_new, 0.0)[:, None]), 0.0)
        l = alpha * l + P.sum(axis=1)
        O = alpha[:, None] * O + P @ v[keys]
        m = m_new
    out = np.where((l > 0)[:, None], O / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return out, skip, margin


def skip_set_vectorized(qr, k, rows, blocks, Bc: int, scale: float, lam: float,
                        n_valid: int, causal: bool):
    """Closed form of Algorithm 1's skip decisions for 0 < lambda < 1.

    A skipped block has block max < running max for every row, so it never
    moves the running max; the running max before a block is therefore the
    cumulative max of the block maxima.  skip_j <=> for every row,
    bm[r, j] = -inf or bm[r, j] - cummax_{j' <= j} bm[r, j'] < ln(lambda)."""
    qr, k = as_f64(qr), as_f64(k)
    lnl = log_threshold(lam)
    n_k = k.shape[0]
    R = qr.shape[0]
    bm = np.full((R, len(blocks)), -np.inf)
    for pos, j in enumerate(blocks):
        keys = block_keys(int(j), Bc, n_k)
        allowed = allowed_entries(rows, keys, n_valid, causal)
        S = np.where(allowed, scale * (qr @ k[keys].T), -np.inf)
        bm[:, pos] = S.max(axis=1)
    cm = np.maximum.accumulate(bm, axis=1)
    finite = np.isfinite(bm)
    gap = np.where(finite, bm - np.where(np.isfinite(cm), cm, 0.0), -np.inf)
    skip = np.all(~finite | (gap < lnl), axis=0)
    return skip, bm


def skip_set_batched(qr, k, rows, blocks, Bc: int, scale: float, lam: float,
                     n_valid: int, causal: bool):
    """The closed form of ``skip_set_vectorized`` with the scores of all the
    tile's visited blocks taken in one float64 product (torch CPU), for
    full-size checks: the block maxima are the row maxima of each block's
    allowed scores, the running max their cumulative maximum in visiting
    order, and a block is skipped iff every row has no allowed key in it or
    a gap below ln(lambda) (BLASST notes, Algorithm 1 and section 4).
    Returns (skip [nb], margin [nb]) with margin as in ``blasst_tile``."""
    import torch
    lnl = log_threshold(lam)
    n_k = k.shape[0]
    nb = len(blocks)
    if nb == 0:
        return np.zeros(0, bool), np.zeros(0)
    blocks = np.asarray(blocks, dtype=np.int64)
    keys = (blocks[:, None] * Bc + np.arange(Bc)[None, :]).reshape(-1)     # [nb * Bc], padded blocks
    inside = keys < n_k
    kk = torch.as_tensor(k, dtype=torch.float64) if not isinstance(k, torch.Tensor) else k.to(torch.float64)
    qq = torch.as_tensor(qr, dtype=torch.float64) if not isinstance(qr, torch.Tensor) else qr.to(torch.float64)
    S = scale * (qq @ kk[torch.from_numpy(np.where(inside, keys, 0))].T)  # [R, nb * Bc]
    allowed = torch.from_numpy(inside & (keys < n_valid))[None, :].expand(len(rows), -1)
    if causal:
        allowed = allowed & (torch.from_numpy(keys)[None, :] <= torch.from_numpy(np.asarray(rows))[:, None])
    S = torch.where(allowed, S, torch.tensor(-math.inf, dtype=torch.float64))
    bm = S.view(len(rows), nb, Bc).amax(dim=2)                          # [R, nb]
    cm = torch.cummax(bm, dim=1).values
    finite = torch.isfinite(bm)
    gap = torch.where(finite, bm - torch.where(torch.isfinite(cm), cm, torch.zeros_like(cm)),
                      torch.tensor(-math.inf, dtype=torch.float64))
    skip = torch.all(~finite | (gap < lnl), dim=0).numpy() if lam > 0.0 else np.zeros(nb, bool)
    margin = (gap.amax(dim=0) - lnl).numpy() if lam > 0.0 else np.full(nb, np.inf)
    return skip, margin


def row_agreement(qr, k, rows, blocks, Bc: int, scale: float, lam: float, n_valid: int, causal: bool):
    """Per-row form of the BLASST skip condition, for the per-row against
    tile-wide comparison: walk the visited blocks as Algorithm 1 does (running
    max updated with the block maximum before the test) and, for every block,
    count the rows of the tile whose own condition holds (block max - running
    max < ln(lambda), or no allowed key in the block), before the tile-wide
    reduction of BLASST notes section 4.

    Returns (agree [nb] int counts, gap [R, nb]) with gap the row's block max
    minus its running max in natural-log units (-inf where the row has no
    allowed key in the block).  lambda = 0 counts nothing (no test is made)."""
    qr, k = as_f64(qr), as_f64(k)
    lnl = log_threshold(lam)
    n_k = k.shape[0]
    R = qr.shape[0]
    m = np.full(R, -np.inf)
    agree = np.zeros(len(blocks), dtype=np.int64)
    gaps = np.full((R, len(blocks)), -np.inf)
    for pos, j in enumerate(blocks):
        keys = block_keys(int(j), Bc, n_k)
        allowed = allowed_entries(rows, keys, n_valid, causal)
        S = np.where(allowed, scale * (qr @ k[keys].T), -np.inf)
        m_blk = S.max(axis=1)
        m = np.maximum(m, m_blk)
        finite = np.isfinite(m_blk)
        gaps[finite, pos] = m_blk[finite] - m[finite]
        if lam > 0.0:
            agree[pos] = int(np.count_nonzero(~finite | (gaps[:, pos] < lnl)))
    return agree, gaps


def static_tile(qr, k, v, rows, blocks, Bc: int, scale: float, n_valid: int, causal: bool):
    """Block-sparse attention for one tile: plain masked softmax over the keys of
    the tile's visited blocks (two-pass; equal to the online form)."""
    n_k = k.shape[0]
    if len(blocks) == 0:
        return np.zeros((len(rows), v.shape[1]))
    keys = np.concatenate([block_keys(int(j), Bc, n_k) for j in blocks])
    allowed = allowed_entries(rows, keys, n_valid, causal)
    return masked_attention(qr, as_f64(k)[keys], as_f64(v)[keys], allowed, scale)


# ---------------------------------------------------------------------------
# prefill over [B, N, H, d] tensors
# ---------------------------------------------------------------------------

def prefill_tile(q, k, v, b: int, h: int, t: int, *, Br: int, Bc: int, scale: float,
                 causal: bool, lam: float, n_valid: int, row_ptr=None, col_idx=None,
                 force=None, method: str = "loop", order: str = "ascending"):
    """Oracle output of one (batch, query head, query tile) of a prefill call.

    q [B, N, Hq, d], k/v [B, N, Hkv, d] (torch or numpy).  Returns
    (rows, out [R, d], blocks, skip, margin).  ``method`` "loop" runs
    Algorithm 1 literally; "two_pass" (static masks, lambda = 0 only) uses
    the plain masked softmax over the visited blocks."""
    Hq, Hkv = q.shape[2], k.shape[2]
    n_q, n_k = q.shape[1], k.shape[1]
    g = kv_head_of(h, Hq, Hkv)
    rows = tile_rows(t, Br, n_q)
    blocks = visited_blocks(t, Br, Bc, n_q, n_k, causal, row_ptr, col_idx, order)
    qr = as_f64(q[b, rows[0]:rows[-1] + 1, h])
    kk = as_f64(k[b, :, g])
    vv = as_f64(v[b, :, g])
    if method == "two_pass":
        if lam != 0.0:
            raise ValueError("two_pass is the static (lambda = 0) path")
        out = static_tile(qr, kk, vv, rows, blocks, Bc, scale, n_valid, causal)
        return rows, out, blocks, np.zeros(len(blocks), bool), np.full(len(blocks), np.inf)
    out, skip, margin = blasst_tile(qr, kk, vv, rows, blocks, Bc, scale, lam, n_valid, causal, force)
    return rows, out, blocks, skip, margin


# ---------------------------------------------------------------------------
# decode: one new query token per sequence, tile = the G heads of a K/V head
# ---------------------------------------------------------------------------

def decode_group(qg, kg, vg, Bc: int, scale: float, lam: float, method: str = "loop", force=None,
                 order: str = "ascending", split_blocks: int = 0, decisions: str = "group"):
    """Decode oracle for one (sequence, K/V head): qg [G, d] are the G query
    heads sharing the K/V head, kg/vg [L, d] its cache.  The query sits at
    position L-1 and sees keys 0..L-1, visited in blocks of Bc in ascending
    order, or descending (most recent first) with order="descending".

    "loop" runs Algorithm 1 literally; "closed_form" takes the skip set from
    the cumulative-max form (running in the visiting order) and then the
    masked softmax over kept keys.  skip, margin and ``force`` are indexed by
    block number whatever the order.

    ``split_blocks`` > 0 selects the per-split variant (not the pages'
    method; it quantifies what the exact cross-split prefix buys): the
    visiting sequence is cut into runs of split_blocks blocks and the running
    max restarts at -inf at the start of every run.

    ``decisions="head"`` selects the per-head variant (not the pages' method,
    whose tile is the group): every query head takes its own skip decisions,
    as a tile of one row would.  skip and margin are then [G, Tc] and
    ``force`` maps (head, block) pairs."""
    if decisions not in ("group", "head"):
        raise ValueError(decisions)
    qg, kg, vg = as_f64(qg), as_f64(kg), as_f64(vg)
    L = kg.shape[0]
    G = qg.shape[0]
    Tc = -(-L // Bc)
    if order == "ascending":
        blocks = np.arange(Tc)
    elif order == "descending":
        blocks = np.arange(Tc)[::-1].copy()
    else:
        raise ValueError(order)
    rows = np.full(G, L - 1)          # every head's query sits at position L-1
    if method == "loop":
        if split_blocks:
            raise ValueError("the per-split variant has the closed form only")
        if decisions == "head":        # one tile of one row per head
            outs, skips, margins = [], [], []
            for r in range(G):
                fr = None if force is None else {j: v for (h, j), v in force.items() if h == r}
                o, sk, mg = decode_group(qg[r:r + 1], kg, vg, Bc, scale, lam, "loop", fr or None, order)
                outs.append(o[0])
                skips.append(sk)
                margins.append(mg)
            return np.stack(outs), np.stack(skips), np.stack(margins)
        fpos = None if force is None else {int(np.nonzero(blocks == j)[0][0]): v for j, v in force.items()}
        out, skip_v, margin_v = blasst_tile(qg, kg, vg, rows, blocks, Bc, scale, lam, L, False, fpos)
        skip = np.zeros(Tc, dtype=bool)
        margin = np.zeros(Tc)
        skip[blocks], margin[blocks] = skip_v, margin_v
        return out, skip, margin
    if method != "closed_form":
        raise ValueError(method)
    lnl = log_threshold(lam)
    S = scale * (qg @ kg.T)                                   # [G, L]
    pad = np.full((G, Tc * Bc), -np.inf)
    pad[:, :L] = S
    bm = pad.reshape(G, Tc, Bc).max(axis=2)[:, blocks]         # [G, Tc], visiting order
    if split_blocks:
        cm = np.concatenate([np.maximum.accumulate(bm[:, a:a + split_blocks], axis=1)
                             for a in range(0, Tc, split_blocks)], axis=1)
    else:
        cm = np.maximum.accumulate(bm, axis=1)
    gap_v = bm - cm
    gap = np.empty_like(gap_v)
    gap[:, blocks] = gap_v                                     # back to block order
    if decisions == "head":
        if lam == 0.0:
            skip = np.zeros((G, Tc), dtype=bool)
            margin = np.full((G, Tc), np.inf)
        else:
            skip = gap < lnl
            margin = gap - lnl
        if force is not None:
            for (h, j), s in force.items():
                skip[h, j] = bool(s)
        allowed = np.repeat(~skip, Bc, axis=1)[:, :L]
        return masked_attention(qg, kg, vg, allowed, scale), skip, margin
    if lam == 0.0:
        skip = np.zeros(Tc, dtype=bool)
        margin = np.full(Tc, np.inf)
    else:
        skip = np.all(gap < lnl, axis=0)
        margin = gap.max(axis=0) - lnl
    if force is not None:
        for pos, s in force.items():
            skip[pos] = bool(s)
    kept_keys = np.repeat(~skip, Bc)[:L]
    allowed = np.broadcast_to(kept_keys[None, :], (G, L))
    out = masked_attention(qg, kg, vg, allowed, scale)
    return out, skip, margin


def decode_sequence(q, k, v, Bc: int, scale: float, lam: float, method: str = "closed_form",
                    groups=None, order: str = "ascending", split_blocks: int = 0, decisions: str = "group"):
    """Decode oracle for one sequence: q [Hq, d], k/v [L, Hkv, d].
    Returns out [Hq, d] (NaN for heads of groups not computed), skip and
    margin [Hkv, Tc] (per head, decisions="head": [Hq, Tc])."""
    Hq, d = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    Tc = -(-L // Bc)
    nd = Hq if decisions == "head" else Hkv
    per = G if decisions == "head" else 1
    out = np.full((Hq, v.shape[2]), np.nan)
    skip = np.zeros((nd, Tc), dtype=bool)
    margin = np.full((nd, Tc), np.nan)
    for g in (range(Hkv) if groups is None else groups):
        o, s, mg = decode_group(q[g * G:(g + 1) * G], k[:, g], v[:, g], Bc, scale, lam, method, order=order,
                                split_blocks=split_blocks, decisions=decisions)
        out[g * G:(g + 1) * G] = o
        skip[g * per:(g + 1) * per], margin[g * per:(g + 1) * per] = s, mg
    return out, skip, margin


# ---------------------------------------------------------------------------
# split partials and their merge (the online-softmax identity)
# ---------------------------------------------------------------------------

def partial_state(qr, k, v, allowed, scale: float):
    """Unnormalised softmax state of a subset of keys: (m, l, acc) with
    m = max allowed score (-inf if none), l = sum exp(S - m), acc = sum exp(S - m) v."""
    qr, k, v = as_f64(qr), as_f64(k), as_f64(v)
    S = np.where(allowed, scale * (qr @ k.T), -np.inf)
    m = S.max(axis=1, initial=-np.inf)
    safe = np.where(np.isfinite(m), m, 0.0)
    P = np.where(allowed, np.exp(S - safe[:, None]), 0.0)
    return m, P.sum(axis=1), P @ v


def merge_partials(ms, ls, accs):
    """Merge states of disjoint key subsets: M = max m_s; l = sum e^{m_s-M} l_s;
    out = sum e^{m_s-M} acc_s / l (tutorial section 4.2 rescaling rule)."""
    ms = np.asarray(ms)
    M = ms.max(axis=0)
    safeM = np.where(np.isfinite(M), M, 0.0)
    w = np.where(np.isfinite(ms), np.exp(ms - safeM[None]), 0.0)
    l = (w * np.asarray(ls)).sum(axis=0)
    acc = (w[..., None] * np.asarray(accs)).sum(axis=0)
    return np.where((l > 0)[:, None], acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
