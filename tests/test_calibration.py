"""The C-ABI calibration fit against the oracle (CPU), and the whole
procedure with sparsities measured by the decode kernel (GPU)."""

import math

import numpy as np
import pytest

import block_sparse_attention_flash_amd as bsa
from oracle import attention as A
from oracle import calibration as OC
from workloads import gen_decode_inputs, gen_decode_sequence
from workloads.configs import DecodeWorkload


def test_fit_equals_oracle_on_random_tables():
    rng = np.random.default_rng(3)
    for trial in range(40):
        K, n = int(rng.integers(1, 7)), int(rng.integers(1, 12))
        lengths = rng.integers(64, 200000, K)
        lambdas = np.sort(rng.uniform(1e-6, 0.5, n))
        table = np.round(rng.uniform(0, 1, (K, n)) * 64) / 64          # ties happen
        target, delta = float(rng.uniform(0, 1)), float(rng.choice([0.01, 0.05, 0.2]))
        a_ref, pts = OC.calibrate(target, lengths, lambdas, table, delta)
        a, npts = bsa.calibrate_fit(target, lengths, lambdas, table, delta)
        assert npts == len(pts)
        if pts:
            assert abs(a - a_ref) <= 1e-12 * abs(a_ref)
        else:
            assert math.isnan(a)


def test_fit_rejects_invalid_input():
    for args in ((1.5, [100], [0.1], [[0.5]], 0.1), (0.5, [0], [0.1], [[0.5]], 0.1),
                 (0.5, [100], [1.0], [[0.5]], 0.1), (0.5, [100], [0.1], [[1.5]], 0.1),
                 (0.5, [100], [0.1], [[0.5]], 0.0)):
        with pytest.raises(bsa.BsattnError):
            bsa.calibrate_fit(*args)


@pytest.mark.gpu
def test_calibration_with_kernel_sparsity_matches_oracle():
    import torch
    lengths = [1024, 2048, 4096]
    lambdas = [c / 1024 for c in (1e-4, 1e-3, 3e-3, 1e-2, 3e-2, 0.05, 0.1, 0.25, 0.5, 1.0)]
    seqs = {}

    def measure(lam, L):
        if L not in seqs:
            cfg = DecodeWorkload(name="c", description="", B=2, Hq=4, Hkv=1, L=L, d=64, Bc=64, lam=lam, seed=5)
            seqs[L] = (cfg, [t.to("cuda") for t in gen_decode_inputs(cfg)])
        cfg, (q, kc, vc) = seqs[L]
        return bsa.decode_sparsity(q, kc, vc, lam=lam, scale=cfg.scale)

    a, n, table = bsa.calibrate(0.5, lengths, lambdas, 0.1, measure)
    # oracle table from the attention oracle's skip sets on the same inputs
    ref = []
    excused_frac = []
    for L in lengths:
        cfg = DecodeWorkload(name="c", description="", B=2, Hq=4, Hkv=1, L=L, d=64, Bc=64, lam=0.0, seed=5)
        row, ex = [], []
        for lam in lambdas:
            skips, near = [], 0
            for b in range(cfg.B):
                q, k, v = gen_decode_sequence(cfg, b)
                _, skip, margin = A.decode_sequence(q, k, v, 64, cfg.scale, lam, "closed_form")
                skips.append(skip)
                near += int(np.count_nonzero(np.abs(margin) <= 1e-3))
            row.append(OC.block_sparsity(skips))
            ex.append(near / sum(s.size for s in skips))
        ref.append(row)
        excused_frac.append(ex)
    assert np.all(np.abs(np.array(table) - np.array(ref)) <= np.array(excused_frac) + 1e-12)
    a_ref, pts = OC.calibrate(0.5, lengths, lambdas, ref, 0.1)
    assert n == len(pts) and n > 0
    assert abs(a - a_ref) <= 1e-9 * abs(a_ref)
