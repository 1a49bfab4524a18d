"""Degenerate sizes on the GPU against the float64 oracle: a single token,
a tile or key block that is mostly padding, exact multiples of the tile
sizes and one past them; prefill (static, causal, BLASST, fp32 path) and
the backward.

Tolerances: as in the targeted tests, except the bf16 prefill mean-abs
bound.  The workloads' 1e-3 assumes output rows that average many keys, so
that their magnitude is well below the inputs'.  Here a row averages at
most 129 keys and as few as one, so its magnitude stays near |V| ~ 1.  P
and the output are each rounded to bf16 (relative 2^-9), which gives an
expected mean error near 2^-10 per element.  The test allows 2^-9 mean, and
keeps the 1e-2 max-abs bound."""

import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_flash_amd as bsa
from workloads import gen_prefill_grad_output, gen_prefill_inputs
from workloads.configs import PrefillWorkload

from _parity import check_prefill_tile
import test_gpu_backward as TB

pytestmark = pytest.mark.gpu
DEV = "cuda"
SIZES = [1, 2, 63, 64, 65, 127, 128, 129]
EDGE_MEAN = 2.0 ** -9


def _say(msg):
    print(f"[gpu-edge] {msg}", file=sys.stderr, flush=True)


def _cfg(N, d, causal, lam, gen, dtype="bf16", seed=0):
    return PrefillWorkload(name="edge", description="", dtype=dtype, B=1, Hq=4, Hkv=2, N=N, d=d, Br=128, Bc=64,
                           causal=causal, lam=lam, mask=None, seed=501 + seed, generator=gen)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", SIZES)
def test_prefill_tiny(N, d):
    """Every tile of every head, dense and causal, lambda 0 and 0.5 (the sink
    recipe, which skips), and a CSR keeping the first key block only."""
    for causal in (False, True):
        for lam, gen in ((0.0, "iid"), (0.5, "sink")):
            for csr_on in (False, True):
                cfg = _cfg(N, d, causal, lam, gen, seed=N + d)
                Tr, Tc = -(-N // 128), -(-N // 64)
                csr = None
                if csr_on:
                    tm = np.zeros((Tr, Tc), bool)
                    tm[:, 0] = True
                    csr = bsa.block_index_from_matrix(tm)
                _say(f"prefill N{N} d{d} causal={causal} lambda={lam} csr={csr_on}")
                q, k, v = gen_prefill_inputs(cfg)
                state = torch.zeros((1, 4, Tr, Tc), dtype=torch.uint8, device=DEV)
                cnt = torch.full((1, 4, Tr, 2), -1, dtype=torch.int32, device=DEV)
                kw = {}
                if csr is not None:
                    kw = dict(row_ptr=torch.from_numpy(csr[0]).to(DEV), col_idx=torch.from_numpy(csr[1]).to(DEV))
                out = bsa.prefill_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=cfg.scale, lam=lam, causal=causal,
                                      tile_counters=cnt, block_state=state, **kw)
                torch.cuda.synchronize()
                out, st, c = out.cpu(), state.cpu().numpy(), cnt.cpu().numpy()
                for h in range(4):
                    for t in range(Tr):
                        check_prefill_tile(q, k, v, out, st, c, 0, h, t, Br=128, Bc=64, scale=cfg.scale,
                                           causal=causal, lam=lam, n_valid=N,
                                           row_ptr=None if csr is None else csr[0],
                                           col_idx=None if csr is None else csr[1], bf16_mean=EDGE_MEAN)


@pytest.mark.parametrize("N", [1, 63, 65, 129])
def test_prefill_tiny_fp32(N):
    cfg = _cfg(N, 64, True, 0.0, "iid", dtype="fp32", seed=N)
    _say(f"prefill fp32 N{N} causal")
    q, k, v = gen_prefill_inputs(cfg)
    Tr, Tc = -(-N // 64), -(-N // 64)
    state = torch.zeros((1, 4, Tr, Tc), dtype=torch.uint8, device=DEV)
    cnt = torch.full((1, 4, Tr, 2), -1, dtype=torch.int32, device=DEV)
    out = bsa.prefill_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=cfg.scale, causal=True, Br=64,
                          tile_counters=cnt, block_state=state)
    torch.cuda.synchronize()
    out, st, c = out.cpu(), state.cpu().numpy(), cnt.cpu().numpy()
    for h in range(4):
        for t in range(Tr):
            check_prefill_tile(q, k, v, out, st, c, 0, h, t, Br=64, Bc=64, scale=cfg.scale, causal=True, lam=0.0,
                               n_valid=N, fp32=True)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 63, 129])
def test_backward_tiny(N, d):
    """Gradients at degenerate sizes, dense causal and a CSR, against the
    oracle with the backward's own tolerance.  Where a row attends a single
    key, P = 1 and dS = dP - Dv cancels to zero exactly, so the reference
    dq and dk are zero.  The error is then set by the cancelling terms,
    whose size is about 1 for these unit-scale inputs (dP and Dv are dot
    products over d scaled by 1/sqrt(d)), not by the zero result: the scale
    is floored at 1."""
    for causal in (False, True):
        cfg = TB._cfg(N=N, d=d, Hq=4, Hkv=2, seed=601 + N, causal=causal)
        _say(f"backward N{N} d{d} causal={causal}")
        q, k, v = gen_prefill_inputs(cfg)
        dout = gen_prefill_grad_output(cfg)
        TB.check_all(cfg, q, k, v, dout, floor=1.0)
        if not causal:
            Tr, Tc = -(-N // 128), -(-N // 64)
            tm = np.ones((Tr, Tc), bool)
            csr = bsa.block_index_from_matrix(tm)
            TB.check_all(cfg, q, k, v, dout, csr, schedule=(1, 1), floor=1.0)
