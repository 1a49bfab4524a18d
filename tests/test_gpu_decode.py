"""GPU parity of bsattn_decode_fwd (split kernel + combine, through the C ABI) against the float64 oracle."""

import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_flash_amd as bsa
from oracle import attention as A
from workloads import get_config, gen_decode_inputs, gen_decode_sequence
from workloads.configs import DecodeWorkload

from _parity import MARGIN, compare_out

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu-decode] {msg}", file=sys.stderr, flush=True)


_WS = [None]


def _shared_workspace(nbytes):
    """One zero-filled workspace reused by every decode call of this module, with
    different shapes and split counts: each call must leave its tickets, flags
    and counters at zero for the next."""
    if _WS[0] is None or _WS[0].numel() < nbytes:
        _WS[0] = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=DEV)
    return _WS[0]


def run_decode(cfg, q, kc, vc, *, L=None, num_splits=0, lam=None, order="ascending", max_scope="sequence",
               decisions="group"):
    B, Hq, d = q.shape
    Hkv = kc.shape[2]
    L = kc.shape[1] if L is None else L
    Tc = -(-L // 64)
    ws = _shared_workspace(bsa.decode_workspace_size(B, Hq, Hkv, L, d, 64, num_splits))
    state = torch.zeros((B, Hq if decisions == "head" else Hkv, Tc), dtype=torch.uint8, device=DEV)
    counters = torch.full((B, Hkv, 2), -1, dtype=torch.int32, device=DEV)
    out = bsa.decode_fwd(q, kc, vc, L=L, scale=cfg.scale, lam=cfg.lam if lam is None else lam,
                         num_splits=num_splits, workspace=ws, counters=counters, block_state=state, order=order,
                         max_scope=max_scope, decisions=decisions)
    torch.cuda.synchronize()
    assert bsa.decode_check(ws) == 0, "decode look-back wait timed out"
    return out.cpu(), state.cpu().numpy(), counters.cpu().numpy()


def check_sequence(q, k, v, out, st, cnt, b, L, scale, lam, groups=None, order="ascending"):
    """q [Hq, d], k/v [L, Hkv, d] host copies of sequence b."""
    Hq = q.shape[0]
    Hkv = k.shape[1]
    G = Hq // Hkv
    ref, skip, margin = A.decode_sequence(q, k[:L], v[:L], 64, scale, lam, "closed_form", groups=groups, order=order)
    tot = [0, 0]
    for g in (range(Hkv) if groups is None else groups):
        gs = st[b, g] == 2
        assert np.all(st[b, g] != 0), "every block of the sequence is visited"
        excused = np.abs(margin[g]) <= MARGIN
        bad = (gs != skip[g]) & ~excused
        assert not bad.any(), f"skip set differs b{b} g{g}: {np.nonzero(bad)[0]} margins {margin[g][bad]}"
        r = ref[g * G:(g + 1) * G]
        if ((gs != skip[g]) & excused).any():
            force = {int(i): bool(gs[i]) for i in np.nonzero((gs != skip[g]) & excused)[0]}
            r, _, _ = A.decode_group(q[g * G:(g + 1) * G], k[:L, g], v[:L, g], 64, scale, lam, "closed_form", force,
                                     order=order)
        assert cnt[b, g, 0] == st.shape[2] and cnt[b, g, 1] == int(gs.sum())
        compare_out(A.as_f64(out[b, g * G:(g + 1) * G]), r, False, f"decode b{b} g{g}")
        tot[0] += gs.size
        tot[1] += int(gs.sum())
    return tot


@pytest.mark.parametrize("G,d", [(4, 128), (1, 64), (2, 128), (8, 64), (8, 128)])
def test_decode_small_all_splits(G, d):
    Hkv = 2
    L = 3000                                   # ragged last block
    cfg = DecodeWorkload(name="s", description="", B=2, Hq=G * Hkv, Hkv=Hkv, L=L, d=d, Bc=64, lam=40.0 / L, seed=21)
    _say(f"decode small G{G} d{d} L{L}")
    q, kc, vc = gen_decode_inputs(cfg)
    qd, kd, vd = q.to(DEV), kc.to(DEV), vc.to(DEV)
    states = []
    for S in (0, 1, 3, 7, 47):
        _say(f"  num_splits {S}")
        out, st, cnt = run_decode(cfg, qd, kd, vd, num_splits=S)
        for b in range(cfg.B):
            check_sequence(q[b], kc[b], vc[b], out, st, cnt, b, L, cfg.scale, cfg.lam)
        states.append(st)
    for st in states[1:]:
        assert np.array_equal(st, states[0]), "skip set depends on the split count"


def test_decode_lengths_and_lambda0():
    cfg = DecodeWorkload(name="s", description="", B=3, Hq=8, Hkv=2, L=5000, d=128, Bc=64, lam=0.0, seed=22)
    q, kc, vc = gen_decode_inputs(cfg)
    qd, kd, vd = q.to(DEV), kc.to(DEV), vc.to(DEV)
    for L in (1, 63, 64, 65, 4097, 5000):
        for lam in (0.0, 40.0 / L if L > 40 else 0.5):
            _say(f"decode L{L} (Lmax 5000) lambda {lam}")
            out, st, cnt = run_decode(cfg, qd, kd, vd, L=L, lam=lam)
            for b in range(cfg.B):
                check_sequence(q[b], kc[b], vc[b], out, st, cnt, b, L, cfg.scale, lam)
            if lam == 0.0:
                assert (st == 1).all()


def test_cfg5_full_size_sampled():
    cfg = get_config("cfg5")
    _say("cfg5 bf16 B32 Hq32 Hkv8 L131072 d128 lambda 40/L")
    q, kc, vc = gen_decode_inputs(cfg, device=DEV)
    out, st, cnt = run_decode(cfg, q, kc, vc)
    skipped = int(cnt[..., 1].sum())
    total = int(cnt[..., 0].sum())
    _say(f"  skipped {skipped} of {total} blocks ({100.0 * skipped / total:.1f}%)")
    assert total == 32 * 8 * 2048
    for b in (0, 17, 31):
        _say(f"  oracle on sequence {b}")
        check_sequence(q[b].cpu(), kc[b].cpu(), vc[b].cpu(), out, st, cnt, b, cfg.L, cfg.scale, cfg.lam)


def test_decode_deterministic():
    cfg = DecodeWorkload(name="s", description="", B=4, Hq=32, Hkv=8, L=20000, d=128, Bc=64, lam=40 / 20000, seed=23)
    _say("decode determinism")
    q, kc, vc = (x.to(DEV) for x in gen_decode_inputs(cfg))
    a = run_decode(cfg, q, kc, vc)
    b = run_decode(cfg, q, kc, vc)
    assert torch.equal(a[0], b[0]) and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])


def test_decode_plan_and_graph_replays():
    """A plan gives the eager result; a HIP graph of it (reset + split + combine
    kernels) replays bit-identically, with other GPU work between replays."""
    cfg = DecodeWorkload(name="s", description="", B=2, Hq=8, Hkv=2, L=9000, d=128, Bc=64, lam=40 / 9000, seed=29)
    _say("decode plan + graph")
    q, kc, vc = (x.to(DEV) for x in gen_decode_inputs(cfg))
    ref = bsa.decode_fwd(q, kc, vc, L=cfg.L, scale=cfg.scale, lam=cfg.lam)
    ws = bsa.decode_workspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d, DEV)
    plan = bsa.decode_plan(q, kc, vc, L=cfg.L, scale=cfg.scale, lam=cfg.lam, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(plan(), ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan()
    for r in range(3):
        plan.out.fill_(7.0)
        junk = torch.randn(1 << 20, device=DEV).sum()   # unrelated work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.out, ref), r
        assert bsa.decode_check(ws) == 0
    del junk


@pytest.mark.parametrize("num_splits", [0, 1, 7])
def test_decode_descending_order(num_splits):
    """Most recent blocks first (block-row reordering): skip sets and outputs
    against the oracle in descending order, for several split counts (the
    look-back then runs from the end of the sequence)."""
    L = 5000
    cfg = DecodeWorkload(name="s", description="", B=2, Hq=8, Hkv=2, L=L, d=128, Bc=64, lam=40.0 / L, seed=27)
    _say(f"decode descending order, {num_splits} splits")
    q, kc, vc = gen_decode_inputs(cfg)
    qd, kd, vd = q.to(DEV), kc.to(DEV), vc.to(DEV)
    tot = [0, 0]
    for lam in (0.3, 0.5):       # the sink block is visited last: smaller thresholds skip nothing here
        out, st, cnt = run_decode(cfg, qd, kd, vd, num_splits=num_splits, lam=lam, order="descending")
        for b in range(cfg.B):
            r = check_sequence(q[b], kc[b], vc[b], out, st, cnt, b, L, cfg.scale, lam, order="descending")
            tot = [x + y for x, y in zip(tot, r)]
    asc = run_decode(cfg, qd, kd, vd, num_splits=num_splits, lam=0.3)
    _say(f"  skipped {tot[1]} of {tot[0]} (descending), {int(asc[2][..., 1].sum())} ascending at lambda 0.3")
    assert tot[1] > 0


def check_variant(q, k, v, out, st, cnt, b, L, scale, lam, order, split_blocks, decisions):
    """check_sequence for the variants: per-split running max (split_blocks > 0)
    and per-head decisions (block_state then holds one row per query head)."""
    Hq = q.shape[0]
    Hkv = k.shape[1]
    G = Hq // Hkv
    Tc = -(-L // 64)
    kw = dict(order=order, split_blocks=split_blocks, decisions=decisions)
    ref, skip, margin = A.decode_sequence(q, k[:L], v[:L], 64, scale, lam, "closed_form", **kw)
    per = G if decisions == "head" else 1
    tot = [0, 0, 0]
    for g in range(Hkv):
        rows = slice(g * per, (g + 1) * per)
        gs = st[b, rows] == 2
        assert np.all(st[b, rows] != 0), "every block of the sequence is visited"
        diff = gs != skip[rows]
        excused = np.abs(margin[rows]) <= MARGIN
        bad = diff & ~excused
        assert not bad.any(), f"skip set differs b{b} g{g}: {np.argwhere(bad)} margins {margin[rows][bad]}"
        r = ref[g * G:(g + 1) * G]
        if diff.any():
            if decisions == "head":
                force = {(int(h), int(j)): bool(gs[h, j]) for h, j in np.argwhere(diff)}
            else:
                force = {int(j): bool(gs[0, j]) for j in np.nonzero(diff[0])[0]}
            r, _, _ = A.decode_group(q[g * G:(g + 1) * G], k[:L, g], v[:L, g], 64, scale, lam, "closed_form", force,
                                     **kw)
        v_skipped = int(gs.all(axis=0).sum())         # blocks no head of the group computes
        assert cnt[b, g, 0] == Tc and cnt[b, g, 1] == v_skipped
        compare_out(A.as_f64(out[b, g * G:(g + 1) * G]), r, False, f"decode variant b{b} g{g}")
        tot[0] += gs.size
        tot[1] += int(gs.sum())
        tot[2] += v_skipped
    return tot


VARIANTS = [
    # (max_scope, decisions, order, num_splits, G, d)
    ("split", "group", "ascending", 7, 4, 128),
    ("split", "group", "ascending", 0, 8, 64),
    ("split", "group", "descending", 3, 4, 128),
    ("split", "group", "ascending", 1, 2, 128),
    ("sequence", "head", "ascending", 0, 4, 128),
    ("sequence", "head", "ascending", 7, 8, 64),
    ("sequence", "head", "descending", 5, 4, 128),
    ("split", "head", "ascending", 4, 4, 64),
]


@pytest.mark.parametrize("max_scope,decisions,order,num_splits,G,d", VARIANTS,
                         ids=["-".join(str(x) for x in v) for v in VARIANTS])
def test_decode_variants(max_scope, decisions, order, num_splits, G, d):
    """Per-split running max and per-head decisions against the oracle's
    variants: skip sets (per head where heads decide), the counters (blocks
    whose V load no head needs) and outputs."""
    L = 4100
    Hkv = 2
    cfg = DecodeWorkload(name="s", description="", B=2, Hq=G * Hkv, Hkv=Hkv, L=L, d=d, Bc=64, lam=40.0 / L, seed=31)
    _say(f"decode variant {max_scope}/{decisions}/{order}, splits {num_splits}, G{G} d{d}")
    q, kc, vc = gen_decode_inputs(cfg)
    qd, kd, vd = q.to(DEV), kc.to(DEV), vc.to(DEV)
    bps = bsa.decode_split_blocks(cfg.B, cfg.Hq, Hkv, L, d, 64, num_splits) if max_scope == "split" else 0
    tot = [0, 0, 0]
    lams = (cfg.lam, 0.05, 0.4) + ((0.0,) if decisions == "head" else ())   # lambda 0: the single-pass kernel
    for lam in lams:
        out, st, cnt = run_decode(cfg, qd, kd, vd, num_splits=num_splits, lam=lam, order=order,
                                  max_scope=max_scope, decisions=decisions)
        for b in range(cfg.B):
            r = check_variant(q[b], kc[b], vc[b], out, st, cnt, b, L, cfg.scale, lam, order, bps, decisions)
            tot = [x + y for x, y in zip(tot, r)]
    _say(f"  decisions {tot[0]}, skipped {tot[1]}, V blocks not loaded {tot[2]}")
    assert tot[1] > 0


def test_decode_workspace_any_contents():
    """One workspace, filled with random bytes (header zeroed) and reused by
    calls whose split count, batch and head count grow and shrink: each call
    zeroes the tickets and flags it uses, so stale words of an earlier shape
    (partials now lying where this call's flags are) never count."""
    _say("decode workspace with arbitrary contents, shapes changing between calls")
    cases = [  # (B, Hq, Hkv, L, d, num_splits)
        (2, 8, 2, 3000, 128, 3), (2, 8, 2, 3000, 128, 7), (3, 16, 4, 2500, 64, 47), (2, 8, 2, 3000, 128, 0),
        (1, 4, 1, 6000, 128, 9), (3, 16, 4, 2500, 64, 2)]
    need = max(bsa.decode_workspace_size(B, Hq, Hkv, L, d, 64, S) for B, Hq, Hkv, L, d, S in cases)
    g = torch.Generator(device=DEV)
    g.manual_seed(99)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV, generator=g)
    ws[:256] = 0
    for i, (B, Hq, Hkv, L, d, S) in enumerate(cases):
        cfg = DecodeWorkload(name="ws", description="", B=B, Hq=Hq, Hkv=Hkv, L=L, d=d, Bc=64, lam=40.0 / L,
                             seed=40 + i)
        _say(f"  B{B} Hq{Hq} Hkv{Hkv} L{L} d{d} splits {S} "
             f"({bsa.decode_num_splits(B, Hq, Hkv, L, d, 64, S)} per pair)")
        q, kc, vc = gen_decode_inputs(cfg)
        Tc = -(-L // 64)
        state = torch.zeros((B, Hkv, Tc), dtype=torch.uint8, device=DEV)
        counters = torch.full((B, Hkv, 2), -1, dtype=torch.int32, device=DEV)
        out = bsa.decode_fwd(q.to(DEV), kc.to(DEV), vc.to(DEV), L=L, scale=cfg.scale, lam=cfg.lam, num_splits=S,
                             workspace=ws, counters=counters, block_state=state)
        torch.cuda.synchronize()
        assert bsa.decode_check(ws) == 0, "decode look-back wait timed out or a ticket was out of range"
        out, st, cnt = out.cpu(), state.cpu().numpy(), counters.cpu().numpy()
        for b in range(B):
            check_sequence(q[b], kc[b], vc[b], out, st, cnt, b, L, cfg.scale, cfg.lam)
