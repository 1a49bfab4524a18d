"""Seeded random parity sweep on the GPU: prefill (static CSR, causal, BLASST,
block order, cut-tile schedules, valid length), decode (lengths, group sizes,
split counts, order and decision variants) and the backward, over shapes the
targeted tests do not pin down.  Every case is checked element by element
against the float64 oracle with the tolerances of the targeted tests."""

import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_flash_amd as bsa
from workloads import gen_decode_inputs, gen_prefill_grad_output, gen_prefill_inputs
from workloads.configs import DecodeWorkload, PrefillWorkload

from _parity import check_prefill_tile
import test_gpu_backward as TB
import test_gpu_decode as TD

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu-random] {msg}", file=sys.stderr, flush=True)


def _random_tile_mask(g, Tr, Tc):
    tm = g.random((Tr, Tc)) < g.uniform(0.2, 0.8)
    if g.random() < 0.5:
        tm[g.integers(Tr)] = False            # a tile that keeps nothing
    if g.random() < 0.5:
        tm[:, g.integers(Tc)] = False         # a key block nobody keeps
    return tm


@pytest.mark.parametrize("case", range(16))
def test_random_prefill(case):
    g = np.random.default_rng(7000 + case)
    d = int(g.choice([64, 128]))
    Hkv = int(g.choice([1, 2]))
    Hq = Hkv * int(g.choice([1, 2, 4]))
    N = int(g.integers(65, 700))
    causal = bool(g.random() < 0.5)
    lam = 0.0 if g.random() < 0.4 else float(g.choice([0.05, 0.3, 0.6]))
    order = "descending" if g.random() < 0.3 else "ascending"
    gen = str(g.choice(["iid", "sink", "sink_last", "concentrated"]))
    n_valid = N if (causal or g.random() < 0.7) else int(g.integers(N // 2, N + 1))
    Tr, Tc = -(-N // 128), -(-N // 64)
    csr = bsa.block_index_from_matrix(_random_tile_mask(g, Tr, Tc)) if g.random() < 0.6 else None
    max_blocks = int(g.integers(1, 4)) if (csr is not None and g.random() < 0.6) else 0
    cfg = PrefillWorkload(name="rnd", description="", dtype="bf16", B=1 + int(g.random() < 0.3), Hq=Hq, Hkv=Hkv,
                          N=N, d=d, Br=128, Bc=64, causal=causal, lam=lam, mask=None, seed=7000 + case, generator=gen)
    _say(f"case {case}: d{d} Hq{Hq}/Hkv{Hkv} N{N} causal={causal} lambda={lam} {order} {gen} n_valid={n_valid} "
         f"csr={csr is not None} max_blocks={max_blocks}")
    q, k, v = gen_prefill_inputs(cfg)
    kw = dict(scale=cfg.scale, lam=lam, causal=causal, n_valid=n_valid, order=order)
    if csr is not None:
        kw.update(row_ptr=torch.from_numpy(csr[0]).to(DEV), col_idx=torch.from_numpy(csr[1]).to(DEV))
        if max_blocks:
            sched = bsa.build_schedule(csr[0], max_blocks)
            kw.update(schedule=sched, workspace=bsa.prefill_workspace(cfg.B, Hq, d, max(1, sched.n_slots), DEV))
    state = torch.zeros((cfg.B, Hq, Tr, Tc), dtype=torch.uint8, device=DEV)
    cnt = torch.full((cfg.B, Hq, Tr, 2), -1, dtype=torch.int32, device=DEV)
    out = bsa.prefill_fwd(q.to(DEV), k.to(DEV), v.to(DEV), tile_counters=cnt, block_state=state, **kw)
    torch.cuda.synchronize()
    out, st, c = out.cpu(), state.cpu().numpy(), cnt.cpu().numpy()
    tot = [0, 0, 0]
    for b in range(cfg.B):
        for h in range(Hq):
            for t in range(Tr):
                r = check_prefill_tile(q, k, v, out, st, c, b, h, t, Br=128, Bc=64, scale=cfg.scale, causal=causal,
                                       lam=lam, n_valid=n_valid, order=order,
                                       row_ptr=None if csr is None else csr[0],
                                       col_idx=None if csr is None else csr[1])
                tot = [x + y for x, y in zip(tot, r)]
    _say(f"  visited {tot[0]} skipped {tot[1]} excused {tot[2]}")


@pytest.mark.parametrize("case", range(12))
def test_random_decode(case):
    g = np.random.default_rng(8000 + case)
    d = int(g.choice([64, 128]))
    G = int(g.choice([1, 2, 4, 8]))
    Hkv = int(g.choice([1, 2]))
    L = int(g.integers(1, 4000))
    splits = int(g.choice([0, 1, 3, 7]))
    lam = float(g.choice([0.0, 0.01, 0.3]))
    order = "descending" if g.random() < 0.3 else "ascending"
    scope = "split" if g.random() < 0.25 else "sequence"
    decisions = "head" if g.random() < 0.25 else "group"
    cfg = DecodeWorkload(name="rnd", description="", B=2, Hq=G * Hkv, Hkv=Hkv, L=L, d=d, Bc=64, lam=lam,
                         seed=8000 + case)
    _say(f"case {case}: d{d} G{G} Hkv{Hkv} L{L} splits {splits} lambda {lam} {order} {scope} {decisions}")
    q, kc, vc = gen_decode_inputs(cfg)
    out, st, cnt = TD.run_decode(cfg, q.to(DEV), kc.to(DEV), vc.to(DEV), num_splits=splits, lam=lam, order=order,
                                 max_scope=scope, decisions=decisions)
    bps = bsa.decode_split_blocks(cfg.B, cfg.Hq, Hkv, L, d, 64, splits) if scope == "split" else 0
    for b in range(cfg.B):
        TD.check_variant(q[b], kc[b], vc[b], out, st, cnt, b, L, cfg.scale, lam, order, bps, decisions)


@pytest.mark.parametrize("case", range(8))
def test_random_backward(case):
    g = np.random.default_rng(9000 + case)
    d = int(g.choice([64, 128]))
    Hkv = int(g.choice([1, 2]))
    Hq = Hkv * int(g.choice([1, 2, 4]))
    N = int(g.integers(65, 600))
    causal = bool(g.random() < 0.5)
    n_valid = N if (causal or g.random() < 0.6) else int(g.integers(N // 2, N + 1))
    gen = str(g.choice(["iid", "concentrated"]))
    cfg = PrefillWorkload(name="rndb", description="", dtype="bf16", B=1, Hq=Hq, Hkv=Hkv, N=N, d=d, Br=128, Bc=64,
                          causal=causal, lam=0.0, mask=None, seed=9000 + case, generator=gen)
    csr = None
    if g.random() < 0.6:
        csr = bsa.block_index_from_matrix(_random_tile_mask(g, -(-N // 128), -(-N // 64)))
    _say(f"case {case}: d{d} Hq{Hq}/Hkv{Hkv} N{N} causal={causal} n_valid={n_valid} csr={csr is not None} {gen}")
    q, k, v = gen_prefill_inputs(cfg)
    dout = gen_prefill_grad_output(cfg)
    TB.check_all(cfg, q, k, v, dout, csr, n_valid)
