"""Helpers for the GPU parity tests: run the oracle on host copies of the very
inputs the GPU consumed and compare element by element.

Tolerances (BLASST workload contract): bf16 outputs max-abs <= 1e-2 and
mean-abs <= 1e-3; fp32 outputs max-abs <= 1e-5; static visited sets
bit-exact; dynamic skip sets identical except blocks whose oracle margin
lies within 1e-3 of the threshold (natural-log units).  Where such an
excused block was decided differently, the oracle output is recomputed with
the GPU's decision for that block only (both decisions are within the
contract, the rest must still match).
"""

from __future__ import annotations

import numpy as np

from oracle import attention as A

BF16_MAX, BF16_MEAN, FP32_MAX = 1e-2, 1e-3, 1e-5
MARGIN = 1e-3


def compare_out(got, ref, fp32: bool, what: str, bf16_mean: float = BF16_MEAN):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if fp32:
        assert err.max() <= FP32_MAX, f"{what}: fp32 max-abs {err.max():.3e}"
    else:
        assert err.max() <= BF16_MAX, f"{what}: bf16 max-abs {err.max():.3e}"
        assert err.mean() <= bf16_mean, f"{what}: bf16 mean-abs {err.mean():.3e}"
    return float(err.max()), float(err.mean())


def check_prefill_tile(q, k, v, out_gpu, state_gpu, counters_gpu, b, h, t, *, Br, Bc, scale, causal, lam,
                       n_valid, row_ptr=None, col_idx=None, fp32=False, rows_limit=None, method="loop",
                       order="ascending", bf16_mean=BF16_MEAN):
    """Oracle for one (b, h, t); compares visited set, skip set, counters and the output rows.

    q/k/v/out_gpu/state_gpu/counters_gpu are host tensors or arrays.  Returns
    (n_visited, n_skipped, n_excused)."""
    Tc = -(-k.shape[1] // Bc)
    rows, ref, blocks, skip, margin = A.prefill_tile(q, k, v, b, h, t, Br=Br, Bc=Bc, scale=scale, causal=causal,
                                                     lam=lam, n_valid=n_valid, row_ptr=row_ptr, col_idx=col_idx,
                                                     method=method, order=order)
    st = np.asarray(state_gpu[b, h, t])
    visited = np.zeros(Tc, bool)
    visited[blocks] = True
    assert np.array_equal(st != 0, visited), f"visited set differs at b{b} h{h} t{t}"
    g_skip = st[blocks] == 2
    excused = np.abs(margin) <= MARGIN
    bad = (g_skip != skip) & ~excused
    assert not bad.any(), f"skip set differs at b{b} h{h} t{t}: blocks {blocks[bad]} margins {margin[bad]}"
    if ((g_skip != skip) & excused).any():
        force = {int(i): bool(g_skip[i]) for i in np.nonzero((g_skip != skip) & excused)[0]}
        qr = A.as_f64(q[b, rows[0]:rows[-1] + 1, h])
        g = A.kv_head_of(h, q.shape[2], k.shape[2])
        ref, _, _ = A.blasst_tile(qr, k[b, :, g], v[b, :, g], rows, blocks, Bc, scale, lam, n_valid, causal, force)
    c = np.asarray(counters_gpu[b, h, t])
    assert c[0] == len(blocks) and c[1] == int(g_skip.sum()), f"counters {c} at b{b} h{h} t{t}"
    got = A.as_f64(out_gpu[b, rows[0]:rows[-1] + 1, h])
    keep = slice(None) if rows_limit is None else (rows < rows_limit)
    compare_out(got[keep], ref[keep], fp32, f"b{b} h{h} t{t}", bf16_mean)
    return len(blocks), int(g_skip.sum()), int(excused.sum())
