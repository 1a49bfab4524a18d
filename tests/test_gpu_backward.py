"""GPU parity of bsattn_prefill_bwd (and the forward's lse output) against the
float64 gradient oracle, through the C ABI.

Tolerance (the pages fix none for gradients; derived from the arithmetic):
the kernels multiply exact bf16 inputs in fp32 but round P and dS to bf16
(relative error <= 2^-9 each) before the dV, dK and dQ products, take
rowsum(dO * O) from the forward's bf16-rounded output, and round the
gradients to bf16 (2^-9 relative).  Each gradient element is a sum of many
such terms with independent roundings, so its error is a few 2^-9 of the
size of its terms; against the scale of the gradient, s = max |reference|
of the tensor, the test asks max-abs <= 2^-6 s and mean-abs <= 2^-9 s.
lse = m + ln(l) comes from the forward, whose row sum l adds the P values
the P.V product uses; at d = 64 those are the bf16-rounded P (relative error
<= 2^-9 per term, so <= 2^-9 on l and on ln l), at d = 128 fp32 P: max-abs
<= 2^-9 + 1e-4.
"""

import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_flash_amd as bsa
from oracle import backward as BW
from oracle import masks as M
from workloads import gen_prefill_grad_output, gen_prefill_inputs, get_config
from workloads.configs import PrefillWorkload, dit_image_text_spec

pytestmark = pytest.mark.gpu
DEV = "cuda"
MAX_REL, MEAN_REL, LSE_ABS = 2.0 ** -6, 2.0 ** -9, 2.0 ** -9 + 1e-4


def _say(msg):
    print(f"[gpu-backward] {msg}", file=sys.stderr, flush=True)


def _cfg(N=300, d=128, Hq=4, Hkv=2, seed=201, generator="iid", causal=False, mask=None):
    return PrefillWorkload(name="bwd", description="", dtype="bf16", B=2, Hq=Hq, Hkv=Hkv, N=N, d=d, Br=128, Bc=64,
                           causal=causal, lam=0.0, mask=mask, seed=seed, generator=generator)


def bwd_schedule(csr, B, Hq, Hkv, d, N, schedule):
    """None; "default" (default_bwd_schedule); or (dq max blocks, dK/dV max
    positions) per item, small bounds forcing many chunks."""
    if schedule is None:
        return None
    colp, rowi = bsa.transpose_block_index(csr[0], csr[1], -(-N // 64))
    if schedule == "default":
        return bsa.default_bwd_schedule(csr[0], colp, rowi, B, Hq, Hkv, d)
    dq_max, kv_max = schedule
    return bsa.BwdSchedule(bsa.build_schedule(csr[0], dq_max), bsa.build_dkdv_schedule(colp, rowi, Hq // Hkv, d, kv_max))


def run_fwd_bwd(cfg, q, k, v, dout, csr=None, n_valid=None, schedule=None):
    """Forward (with lse) then backward on the GPU; host copies of everything."""
    B, N, Hq, d = q.shape
    Tc = -(-N // 64)
    rp = ci = cp = ri = None
    if csr is not None:
        colp, rowi = bsa.transpose_block_index(csr[0], csr[1], Tc)
        rp, ci = torch.from_numpy(csr[0]).to(DEV), torch.from_numpy(csr[1]).to(DEV)
        cp, ri = torch.from_numpy(colp).to(DEV), torch.from_numpy(rowi).to(DEV)
    sched = bwd_schedule(csr, B, Hq, k.shape[2], d, N, schedule)
    if sched is not None:
        _say(f"  schedule: dq {sched.dq.n_items} items / {sched.dq.n_slots} slots, "
             f"dk/dv {sched.kv.n_items} items / {sched.kv.n_slots} slots")
    nv = cfg.n_valid if n_valid is None else n_valid
    lse = torch.full((B, Hq, N), float("nan"), dtype=torch.float32, device=DEV)
    out = bsa.prefill_fwd(q, k, v, scale=cfg.scale, causal=cfg.causal, row_ptr=rp, col_idx=ci, n_valid=nv, lse=lse)
    dq, dk, dv = bsa.prefill_bwd(q, k, v, out, dout, lse, scale=cfg.scale, causal=cfg.causal, row_ptr=rp,
                                 col_idx=ci, col_ptr=cp, row_idx=ri, n_valid=nv, schedule=sched)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu().numpy(), dq.cpu(), dk.cpu(), dv.cpu()


def token_mask(N, csr, n_valid, causal):
    Tr, Tc = -(-N // 128), -(-N // 64)
    tm = np.ones((Tr, Tc), bool)
    if csr is not None:
        tm[:] = False
        for t in range(Tr):
            tm[t, csr[1][csr[0][t]:csr[0][t + 1]]] = True
    return M.expand_token_mask(tm, N, N, 128, 64, n_valid, causal)


def compare_grad(got, ref, what, floor: float = 1e-30):
    """``floor``: the smallest scale s, for gradients that cancel to (near)
    zero, whose rounding error is set by the size of the cancelling terms."""
    got = np.asarray(got.float().numpy(), dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    s = max(float(np.abs(ref).max()), floor)
    err = np.abs(got - ref)
    _say(f"  {what}: scale {s:.3e}, max-abs {err.max():.3e} ({err.max() / s:.2e} s), "
         f"mean-abs {err.mean():.3e} ({err.mean() / s:.2e} s)")
    assert err.max() <= MAX_REL * s, f"{what}: max-abs {err.max():.3e} > {MAX_REL * s:.3e}"
    assert err.mean() <= MEAN_REL * s, f"{what}: mean-abs {err.mean():.3e} > {MEAN_REL * s:.3e}"


def check_all(cfg, q, k, v, dout, csr=None, n_valid=None, schedule=None, floor: float = 1e-30):
    nv = cfg.n_valid if n_valid is None else n_valid
    out, lse, dq, dk, dv = run_fwd_bwd(cfg, q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV), csr, nv, schedule)
    mask = token_mask(cfg.N, csr, nv, cfg.causal)
    rq, rk, rv = BW.prefill_grads(q, k, v, dout, mask, cfg.scale)
    rl = BW.prefill_lse(q, k, mask, cfg.scale)
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin), "lse: rows with and without attended keys differ"
    if fin.any():
        assert np.abs(lse[fin] - rl[fin]).max() <= LSE_ABS, f"lse max-abs {np.abs(lse[fin] - rl[fin]).max():.3e}"
    compare_grad(dq, rq, "dq", floor)
    compare_grad(dk, rk, "dk", floor)
    compare_grad(dv, rv, "dv", floor)
    # structural zeros: keys nobody attends, rows that attend nothing
    dead_k = ~mask.any(axis=0)
    dead_q = ~mask.any(axis=1)
    assert torch.all(dk[:, torch.from_numpy(dead_k)] == 0) and torch.all(dv[:, torch.from_numpy(dead_k)] == 0)
    assert torch.all(dq[:, torch.from_numpy(dead_q)] == 0)


def _random_csr(Tr, Tc, seed):
    """A random tile mask with one empty tile row and one key block no tile keeps."""
    g = np.random.default_rng(seed)
    tm = g.random((Tr, Tc)) < 0.55
    tm[1] = False
    tm[:, 2] = False
    tm[0, 0] = tm[2, 4] = True
    row_ptr = np.concatenate([[0], np.cumsum(tm.sum(axis=1))]).astype(np.int32)
    col_idx = np.concatenate([np.nonzero(r)[0] for r in tm]).astype(np.int32)
    return row_ptr, col_idx


CASES = ["dense", "causal", "csr", "csr_causal_nvalid"]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", CASES)
def test_backward_small(case, d):
    """N = 300 (three query tiles with a ragged last one, five key blocks),
    GQA with two query heads per K/V head."""
    causal = "causal" in case
    n_valid = 280 if "nvalid" in case else 300
    cfg = _cfg(d=d, causal=causal, seed=201 + d)
    _say(f"backward {case} d{d} N300 Hq4 Hkv2 n_valid {n_valid}")
    q, k, v = gen_prefill_inputs(cfg)
    dout = gen_prefill_grad_output(cfg)
    csr = _random_csr(3, 5, 7 + d) if "csr" in case else None
    check_all(cfg, q, k, v, dout, csr, n_valid)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_dit_mask(d):
    """The DiT image+text mask family (2-D window, text segment, anchors) at a
    reduced size, per-head offsets (cfg2's recipe), padding keys past n_valid."""
    spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
    n = spec.n_valid + 13
    cfg = _cfg(N=n, d=d, Hq=4, Hkv=4, generator="iid_offset", seed=211, mask=spec)
    _say(f"backward DiT mask N{n} d{d}")
    q, k, v = gen_prefill_inputs(cfg)
    dout = gen_prefill_grad_output(cfg)
    csr = bsa.build_block_index(spec, n, n, 128, 64)
    check_all(cfg, q, k, v, dout, csr)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("case", ["csr", "csr_causal_nvalid", "dit"])
def test_backward_schedule_forced_chunks(case, d):
    """Schedules with tiny bounds (dQ: 2 blocks per item; dK/dV: 3 (head,
    tile) positions per item), so nearly every tile and key block is cut
    into chunks whose partials the last arriving chunk adds up, and dK/dV
    chunks start mid-way through a head's list (GQA, two query heads per K/V
    head)."""
    causal = "causal" in case
    if case == "dit":
        spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
        n = spec.n_valid + 13
        cfg = _cfg(N=n, d=d, Hq=4, Hkv=2, generator="iid", seed=271, mask=spec)
        csr = bsa.build_block_index(spec, n, n, 128, 64)
        n_valid = None
    else:
        cfg = _cfg(d=d, causal=causal, seed=281 + d)
        csr = _random_csr(3, 5, 17 + d)
        n_valid = 280 if "nvalid" in case else 300
    _say(f"backward with forced chunks: {case} d{d}")
    q, k, v = gen_prefill_inputs(cfg)
    dout = gen_prefill_grad_output(cfg)
    check_all(cfg, q, k, v, dout, csr, n_valid, schedule=(2, 3))


def test_backward_plan_and_graph_replays():
    """The backward with schedules that cut (forced tiny chunks) captured in a
    HIP graph: its arrival counters are cleared by a fill kernel each call,
    so every replay, with other GPU work between replays, equals the eager
    result bit for bit."""
    spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
    n = spec.n_valid + 13
    cfg = _cfg(N=n, d=128, Hq=4, Hkv=2, generator="iid", seed=291, mask=spec)
    _say("backward plan + graph, schedules with cut tiles and key blocks")
    q, k, v = (x.to(DEV) for x in gen_prefill_inputs(cfg))
    dout = gen_prefill_grad_output(cfg).to(DEV)
    csr = bsa.build_block_index(spec, n, n, 128, 64)
    colp, rowi = bsa.transpose_block_index(csr[0], csr[1], -(-n // 64))
    sched = bwd_schedule(csr, 2, 4, 2, 128, n, (2, 3))
    assert sched.dq.n_merges > 0 and sched.kv.n_merges > 0
    rp, ci, cp, ri = (torch.from_numpy(x).to(DEV) for x in (csr[0], csr[1], colp, rowi))
    lse = torch.empty((2, 4, n), dtype=torch.float32, device=DEV)
    out = bsa.prefill_fwd(q, k, v, scale=cfg.scale, row_ptr=rp, col_idx=ci, n_valid=spec.n_valid, lse=lse)
    kw = dict(scale=cfg.scale, row_ptr=rp, col_idx=ci, col_ptr=cp, row_idx=ri, n_valid=spec.n_valid, schedule=sched)
    ref = [x.clone() for x in bsa.prefill_bwd(q, k, v, out, dout, lse, **kw)]
    plan = bsa.prefill_bwd_plan(q, k, v, out, dout, lse, **kw)
    got = plan()
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan()
    for r in range(3):
        for x in plan.out:
            x.fill_(3.0)
        junk = torch.randn(1 << 20, device=DEV).sum()   # unrelated work between replays
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(plan.out, ref):
            assert torch.equal(x, y), r
    del junk


def test_backward_deterministic():
    cfg = _cfg(N=700, d=128, Hq=8, Hkv=2, seed=221, causal=True)
    _say("backward determinism")
    q, k, v = (x.to(DEV) for x in gen_prefill_inputs(cfg))
    dout = gen_prefill_grad_output(cfg).to(DEV)
    a = run_fwd_bwd(cfg, q, k, v, dout)
    b = run_fwd_bwd(cfg, q, k, v, dout)
    for x, y in zip(a[2:], b[2:]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("d", [64, 128])
def test_backward_deterministic_under_full_load(d):
    """The backward at a shape that fills the GPU (causal GQA 32/8, N 4096),
    three runs, bit-identical gradients (see the forward's test of the same
    name)."""
    cfg = PrefillWorkload(name="bwd_det", description="", dtype="bf16", B=1, Hq=32, Hkv=8, N=4096, d=d, Br=128,
                          Bc=64, causal=True, lam=0.0, mask=None, seed=261 + d, generator="iid")
    _say(f"backward determinism under load d{d}")
    q, k, v = (x.to(DEV) for x in gen_prefill_inputs(cfg))
    dout = gen_prefill_grad_output(cfg).to(DEV)
    runs = [run_fwd_bwd(cfg, q, k, v, dout) for _ in range(3)]
    for r in runs[1:]:
        for x, y in zip(r[2:], runs[0][2:]):
            assert torch.equal(x, y)


@pytest.mark.parametrize("schedule", [None, "default"])
def test_backward_cfg2_full_size_sampled(schedule):
    """The DiT image+text workload at full size (B 2, H 16, N 4352, d 64):
    every gradient of two (batch, head) pairs against the oracle run on that
    head alone (dK and dV of a head depend only on that head when Hq = Hkv),
    without and with the default schedule (which cuts the anchor rows and
    the anchor key block)."""
    cfg = get_config("cfg2")
    _say(f"backward cfg2 full size, heads (0, 3) and (1, 12), schedule {schedule}")
    q, k, v = gen_prefill_inputs(cfg)
    dout = gen_prefill_grad_output(cfg)
    csr = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, 128, 64)
    out, lse, dq, dk, dv = run_fwd_bwd(cfg, q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV), csr, schedule=schedule)
    mask = token_mask(cfg.N, csr, cfg.n_valid, False)
    for b, h in ((0, 3), (1, 12)):
        sl = lambda x: x[b:b + 1, :, h:h + 1]
        rq, rk, rv = BW.prefill_grads(sl(q), sl(k), sl(v), sl(dout), mask, cfg.scale)
        compare_grad(sl(dq), rq, f"dq b{b} h{h}")
        compare_grad(sl(dk), rk, f"dk b{b} h{h}")
        compare_grad(sl(dv), rv, f"dv b{b} h{h}")
        rl = BW.prefill_lse(sl(q), sl(k), mask, cfg.scale)[0, 0]
        assert np.abs(lse[b, h] - rl).max() <= LSE_ABS


@pytest.mark.parametrize("d", [64, 128])
def test_backward_causal_gqa_loaded(d):
    """Causal GQA 32/8 at N 3072: enough work-groups to fill the GPU (the dQ
    launch runs 768, the dK/dV launch 384), so the kernels run under the
    contention of a real launch.  Every gradient of K/V head 5 and of its four
    query heads against the oracle (dK and dV of a K/V head sum its query
    heads only)."""
    N, g = 3072, 5
    cfg = PrefillWorkload(name="bwd_loaded", description="", dtype="bf16", B=1, Hq=32, Hkv=8, N=N, d=d, Br=128,
                          Bc=64, causal=True, lam=0.0, mask=None, seed=251 + d, generator="iid")
    _say(f"backward causal GQA 32/8 N{N} d{d}, K/V head {g}")
    q, k, v = gen_prefill_inputs(cfg)
    dout = gen_prefill_grad_output(cfg)
    out, lse, dq, dk, dv = run_fwd_bwd(cfg, q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV))
    mask = token_mask(N, None, N, True)
    heads = list(range(4 * g, 4 * g + 4))
    rk = np.zeros((N, d))
    rv = np.zeros((N, d))
    for h in heads:
        hq, hk, hv = BW.masked_attention_grads(q[0, :, h], k[0, :, g], v[0, :, g], dout[0, :, h], mask, cfg.scale)
        compare_grad(dq[0, :, h], hq, f"dq h{h}")
        rk += hk
        rv += hv
        rl = BW.row_lse(q[0, :, h], k[0, :, g], mask, cfg.scale)
        assert np.abs(lse[0, h] - rl).max() <= LSE_ABS
    compare_grad(dk[0, :, g], rk, f"dk g{g}")
    compare_grad(dv[0, :, g], rv, f"dv g{g}")


def _check_after_skipping_forward(N, Hq, Hkv, d, lam, seed, groups):
    """BLASST forward (causal GQA, the sink recipe so that blocks are
    skipped), then the backward with that forward's block_state: the
    gradients of the K/V heads in ``groups`` and of their query heads are
    those of softmax attention over each tile's kept blocks.  The oracle
    takes its own skip decisions (Algorithm 1); where a decision lies within
    the accepted margin of the threshold it follows the GPU's, as the
    forward tests do.  Returns the number of blocks the forward skipped in
    the checked heads."""
    from oracle import attention as A
    from _parity import MARGIN
    G = Hq // Hkv
    cfg = PrefillWorkload(name="bwd_skip", description="", dtype="bf16", B=1, Hq=Hq, Hkv=Hkv, N=N, d=d, Br=128,
                          Bc=64, causal=True, lam=lam, mask=None, seed=seed, generator="sink")
    q, k, v = gen_prefill_inputs(cfg)
    dout = gen_prefill_grad_output(cfg)
    qd, kd, vd, gd = (x.to(DEV) for x in (q, k, v, dout))
    Tr, Tc = -(-N // 128), -(-N // 64)
    state = torch.zeros((1, Hq, Tr, Tc), dtype=torch.uint8, device=DEV)
    lse = torch.empty((1, Hq, N), dtype=torch.float32, device=DEV)
    out = bsa.prefill_fwd(qd, kd, vd, scale=cfg.scale, lam=lam, causal=True, block_state=state, lse=lse)
    dq, dk, dv = bsa.prefill_bwd(qd, kd, vd, out, gd, lse, scale=cfg.scale, causal=True, block_state=state)
    torch.cuda.synchronize()
    st = state.cpu().numpy()
    dq, dk, dv, lse = dq.cpu(), dk.cpu(), dv.cpu(), lse.cpu().numpy()
    n_skip = 0
    for g in groups:
        rk = np.zeros((N, d))
        rv = np.zeros((N, d))
        for h in range(G * g, G * g + G):
            tm = np.zeros((Tr, Tc), bool)
            for t in range(Tr):
                rows, _, blocks, skip, margin = A.prefill_tile(q, k, v, 0, h, t, Br=128, Bc=64, scale=cfg.scale,
                                                              causal=True, lam=lam, n_valid=N)
                g_skip = st[0, h, t, blocks] == 2
                bad = (g_skip != skip) & ~(np.abs(margin) <= MARGIN)
                assert not bad.any(), f"skip set differs at h{h} t{t}"
                tm[t, blocks[~g_skip]] = True          # oracle decisions, GPU's only inside the margin
                n_skip += int(g_skip.sum())
            mask = M.expand_token_mask(tm, N, N, 128, 64, N, True)
            hq, hk, hv = BW.masked_attention_grads(q[0, :, h], k[0, :, g], v[0, :, g], dout[0, :, h], mask, cfg.scale)
            compare_grad(dq[0, :, h], hq, f"dq h{h}")
            rk += hk
            rv += hv
            rl = BW.row_lse(q[0, :, h], k[0, :, g], mask, cfg.scale)
            assert np.abs(lse[0, h] - rl).max() <= LSE_ABS
        compare_grad(dk[0, :, g], rk, f"dk g{g}")
        compare_grad(dv[0, :, g], rv, f"dv g{g}")
    return n_skip


@pytest.mark.parametrize("d", [64, 128])
def test_backward_after_skipping_forward(d):
    """Causal GQA 8/2 at N 1000, lambda 0.3, every head checked."""
    _say(f"backward after a skipping forward: causal GQA 8/2 N1000 d{d} lambda 0.3")
    n_skip = _check_after_skipping_forward(1000, 8, 2, d, 0.3, 231, groups=(0, 1))
    _say(f"  blocks skipped by the forward: {n_skip}")
    assert n_skip > 0


@pytest.mark.parametrize("d", [64, 128])
def test_backward_after_skipping_forward_loaded(d):
    """Causal GQA 32/8 at N 3072, lambda 0.5: launches that fill the GPU (the
    dQ kernel runs 768 work-groups), so the skip-state reads of both
    backward kernels run under the contention of a real launch.  Every
    gradient of K/V head 3 and of its four query heads."""
    _say(f"backward after a skipping forward: causal GQA 32/8 N3072 d{d} lambda 0.5, K/V head 3")
    n_skip = _check_after_skipping_forward(3072, 32, 8, d, 0.5, 241 + d, groups=(3,))
    _say(f"  blocks skipped by the forward in K/V head 3's query heads: {n_skip}")
    assert n_skip > 0


def test_empty_block_index():
    """A CSR that keeps no block at all (an empty col_idx): the forward writes
    zeros and lse = -inf, the backward zeros everywhere."""
    cfg = _cfg(N=200, d=64, Hq=2, Hkv=1, seed=241)
    _say("empty block index")
    q, k, v = gen_prefill_inputs(cfg)
    dout = gen_prefill_grad_output(cfg)
    csr = (np.zeros(3, np.int32), np.zeros(0, np.int32))
    out, lse, dq, dk, dv = run_fwd_bwd(cfg, q.to(DEV), k.to(DEV), v.to(DEV), dout.to(DEV), csr)
    assert torch.all(out == 0) and np.all(np.isneginf(lse))
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


def test_backward_cfg3_schedule_full_size():
    """The video DiT workload at full size (B 1, H 24, N 65920, d 128) with
    the default schedule: the text query tiles (every key block) and the
    anchor key block (every query tile) are cut into many chunks.  The dQ
    rows of the three text tiles of head 0 against the oracle on those rows
    (a dQ row depends only on its own row); all gradients against the
    unscheduled run, which may differ only in the order of fp32 additions;
    and two scheduled runs bit-identical."""
    cfg = get_config("cfg3")
    _say("backward cfg3 full size, default schedule against none")
    q, k, v = gen_prefill_inputs(cfg)
    dout = gen_prefill_grad_output(cfg)
    csr = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, 128, 64)
    qd, kd, vd, gd = (x.to(DEV) for x in (q, k, v, dout))
    plain = run_fwd_bwd(cfg, qd, kd, vd, gd, csr)
    sched = run_fwd_bwd(cfg, qd, kd, vd, gd, csr, schedule="default")
    again = run_fwd_bwd(cfg, qd, kd, vd, gd, csr, schedule="default")
    for x, y in zip(sched[2:], again[2:]):
        assert torch.equal(x, y)
    for name, x, y in zip(("dq", "dk", "dv"), sched[2:], plain[2:]):
        xf, yf = x.float(), y.float()
        s = float(yf.abs().max())
        err = (xf - yf).abs()
        _say(f"  {name}: scheduled against unscheduled max-abs {float(err.max()):.3e} ({float(err.max()) / s:.2e} s)")
        assert float(err.max()) <= 2.0 ** -6 * s and float(err.mean()) <= 2.0 ** -11 * s
    Tr = cfg.N // 128
    tm = np.zeros((Tr, cfg.N // 64), bool)
    for t in range(Tr):
        tm[t, csr[1][csr[0][t]:csr[0][t + 1]]] = True
    dq = sched[2]
    for t in (Tr - 3, Tr - 2, Tr - 1):
        rows = slice(128 * t, 128 * t + 128)
        allowed = M.expand_token_mask(tm[t:t + 1], 128, cfg.N, 128, 64, cfg.n_valid, False)
        hq, _, _ = BW.masked_attention_grads(q[0, rows, 0], k[0, :, 0], v[0, :, 0], dout[0, rows, 0], allowed,
                                             cfg.scale)
        compare_grad(dq[0, rows, 0], hq, f"dq tile {t} head 0")
