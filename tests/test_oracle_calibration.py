"""Pins for the calibration oracle (CPU only): hand-built tables with known
answers, the tie and tolerance readings, the closed-form fit, and a table
measured with the attention oracle on synthetic decode inputs."""

import math

import numpy as np
import pytest

from oracle import attention as A
from oracle import calibration as C
from workloads import gen_decode_sequence
from workloads.configs import DecodeWorkload


def test_exact_inverse_law_is_recovered():
    # sparsity reaches the target exactly at lambda = 3 / L for every length
    a_true = 3.0
    lengths = [1024, 2048, 4096, 8192]
    lambdas = [a_true / L for L in lengths] + [1e-6, 1e-1]
    table = []
    for L in lengths:
        table.append([0.5 if abs(lam - a_true / L) < 1e-15 else 0.9 for lam in lambdas])
    a, pts = C.calibrate(0.5, lengths, lambdas, table, 0.01)
    assert len(pts) == 4
    assert abs(a - a_true) < 1e-12
    assert all(abs(y - a_true * x) < 1e-15 for x, y in pts)


def test_least_squares_through_origin_by_hand():
    # points (1/2, 1), (1/4, 1): a = (0.5 + 0.25) / (0.25 + 0.0625) = 2.4
    lambdas = [1.0, 2.0]
    table = [[0.3, 0.9], [0.3, 0.9]]
    a, pts = C.calibrate(0.3, [2, 4], lambdas, table, 0.05)
    assert pts == [(0.5, 1.0), (0.25, 1.0)]
    assert abs(a - 0.75 / 0.3125) < 1e-15


def test_tolerance_drops_lengths_and_is_strict():
    lambdas = [0.1, 0.2]
    table = [[0.375, 0.875],      # best gap 0.125 (exact) -> dropped at delta 0.125 (strict), kept at 0.13
             [0.4921875, 0.9]]    # best gap 0.0078125 -> kept
    a, pts = C.calibrate(0.5, [100, 200], lambdas, table, 0.125)
    assert pts == [(1 / 200, 0.1)]
    a2, pts2 = C.calibrate(0.5, [100, 200], lambdas, table, 0.13)
    assert len(pts2) == 2
    assert C.calibrate(0.5, [100], [0.1], [[0.0]], 0.1) == (None, [])


def test_ties_keep_the_first_threshold():
    lam, gap = C.best_threshold([0.3, 0.1, 0.2], [0.375, 0.625, 0.625], 0.5)   # three equal gaps of 1/8
    assert lam == 0.3 and gap == 0.125


def _decode_sparsity(L, lam, seed):
    cfg = DecodeWorkload(name="c", description="", B=2, Hq=4, Hkv=1, L=L, d=32, Bc=64, lam=lam, seed=seed)
    skips = []
    for b in range(cfg.B):
        q, k, v = gen_decode_sequence(cfg, b)
        _, skip, _ = A.decode_sequence(q, k, v, 64, cfg.scale, lam, "closed_form")
        skips.append(skip)
    return C.block_sparsity(skips)


def test_measured_table_follows_the_inverse_law():
    """On the synthetic decode recipe, sparsity grows with lambda at every
    length, and a fixed threshold gives a sparsity that changes with length
    (the effect the calibration removes, BLASST notes section 3.2)."""
    lengths = [1024, 2048, 4096]
    lambdas = [c / 1024 for c in (0.5, 1, 2, 4, 8, 16, 32, 64)]
    table = [[_decode_sparsity(L, lam, 5) for lam in lambdas] for L in lengths]
    for row in table:
        assert all(x <= y + 1e-12 for x, y in zip(row, row[1:]))      # monotone in lambda
    a, pts = C.calibrate(0.5, lengths, lambdas, table, 0.2)
    assert a is not None and a > 0
    fixed = [table[k][3] for k in range(len(lengths))]                 # lambda = 4/1024 at every length
    assert max(fixed) - min(fixed) > 0.05
