"""GPU parity of bsattn_prefill_fwd (through the C ABI) against the float64 oracle."""

import math
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_flash_amd as bsa
from oracle import attention as A
from oracle import masks as M
from workloads import get_config, gen_prefill_inputs
from workloads.configs import PrefillWorkload, dit_image_text_spec, video_text_spec

from _parity import check_prefill_tile, compare_out

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu-prefill] {msg}", file=sys.stderr, flush=True)


def run_prefill(cfg, q, k, v, *, csr=None, order=None, lam=None, Br=None, schedule=None, workspace=None,
                block_order="ascending"):
    """Launch through the binding; returns host copies of out, block_state, counters."""
    Br = cfg.Br if Br is None else Br
    B, N, Hq, d = q.shape
    Tr, Tc = -(-N // Br), -(-N // cfg.Bc)
    state = torch.zeros((B, Hq, Tr, Tc), dtype=torch.uint8, device=DEV)
    counters = torch.full((B, Hq, Tr, 2), -1, dtype=torch.int32, device=DEV)
    rp = ci = od = None
    if csr is not None:
        rp = torch.from_numpy(csr[0]).to(DEV)
        ci = torch.from_numpy(csr[1]).to(DEV)
    if order is not None:
        od = torch.from_numpy(order).to(DEV)
    out = bsa.prefill_fwd(q, k, v, scale=cfg.scale, lam=cfg.lam if lam is None else lam, causal=cfg.causal,
                          Br=Br, Bc=cfg.Bc, row_ptr=rp, col_idx=ci, tile_order=od, n_valid=cfg.n_valid,
                          tile_counters=counters, block_state=state, schedule=schedule, workspace=workspace,
                          order=block_order)
    torch.cuda.synchronize()
    return out.cpu(), state.cpu().numpy(), counters.cpu().numpy()


def _small(name, **kw):
    base = dict(name=name, description="", dtype="bf16", B=2, Hq=4, Hkv=2, N=300, d=128, Br=128, Bc=64,
                causal=False, lam=0.0, mask=None, seed=101, generator="iid")
    base.update(kw)
    return PrefillWorkload(**base)


# ---------------------------------------------------------------------------- static

def test_cfg1_fp32_full():
    cfg = get_config("cfg1")
    _say("cfg1 fp32 B1 H2 N512 d64 window +-1 block")
    q, k, v = gen_prefill_inputs(cfg)
    csr = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, cfg.Br, cfg.Bc)
    out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr)
    for h in range(cfg.Hq):
        for t in range(cfg.N // cfg.Br):
            check_prefill_tile(q, k, v, out, st, cnt, 0, h, t, Br=64, Bc=64, scale=cfg.scale, causal=False,
                               lam=0.0, n_valid=cfg.N, row_ptr=csr[0], col_idx=csr[1], fp32=True)
    assert (st != 0).sum() == 2 * 22


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_static_small_ragged(d):
    spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
    n = spec.n_valid + 13                                # 309 tokens: 3 tiles, ragged tail, padding keys
    cfg = _small("small", N=n, d=d, Hq=4, Hkv=4, mask=spec, generator="iid_offset")
    _say(f"bf16 static small N{n} d{d}")
    q, k, v = gen_prefill_inputs(cfg)
    csr = bsa.build_block_index(spec, n, n, 128, 64)
    out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr, order=bsa.tile_order_lpt(csr[0]))
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            for t in range(3):
                check_prefill_tile(q, k, v, out, st, cnt, b, h, t, Br=128, Bc=64, scale=cfg.scale, causal=False,
                                   lam=0.0, n_valid=spec.n_valid, row_ptr=csr[0], col_idx=csr[1])


def test_cfg2_full():
    cfg = get_config("cfg2")
    _say("cfg2 bf16 B2 H16 N4352 d64 image+text mask, all heads, all tiles")
    q, k, v = gen_prefill_inputs(cfg)
    csr = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, 128, 64)
    out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr, order=bsa.tile_order_lpt(csr[0]))
    assert (st != 0).sum() == cfg.B * cfg.Hq * 640
    errs = []
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            for t in range(34):
                check_prefill_tile(q, k, v, out, st, cnt, b, h, t, Br=128, Bc=64, scale=cfg.scale, causal=False,
                                   lam=0.0, n_valid=cfg.N, row_ptr=csr[0], col_idx=csr[1], method="two_pass")


def test_cfg3_full_size_sampled():
    cfg = get_config("cfg3")
    _say("cfg3 bf16 B1 H24 N65920 d128 video mask, sampled heads/tiles")
    q, k, v = gen_prefill_inputs(cfg, device=DEV)
    csr = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, 128, 64)
    out, st, cnt = run_prefill(cfg, q, k, v, csr=csr, order=bsa.tile_order_lpt(csr[0]))
    assert int((st != 0).sum()) == cfg.Hq * 13839
    # exact visited set for every head and tile
    rp, ci = csr
    for h in (0, 7, 23):
        for t in range(515):
            vis = np.zeros(1030, bool)
            vis[ci[rp[t]:rp[t + 1]]] = True
            assert np.array_equal(st[0, h, t] != 0, vis)
    # outputs on sampled tiles, including the anchor tile and the padded last tile
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    for h in (0, 23):
        for t in (0, 1, 100, 256, 511, 512, 514):
            check_prefill_tile(qh, kh, vh, out, st, cnt, 0, h, t, Br=128, Bc=64, scale=cfg.scale, causal=False,
                               lam=0.0, n_valid=cfg.mask.n_valid, row_ptr=rp, col_idx=ci, method="two_pass",
                               rows_limit=cfg.mask.n_valid)


# ---------------------------------------------------------------------------- causal / BLASST

@pytest.mark.parametrize("gen,lam", [("concentrated", 0.0), ("concentrated", 0.04), ("sink", 0.3), ("sink", 0.7)])
@pytest.mark.parametrize("d", [64, 128])
def test_causal_gqa_dynamic_small(gen, lam, d):
    cfg = _small("causal", N=1000, d=d, Hq=8, Hkv=2, causal=True, lam=lam, generator=gen, seed=4)
    _say(f"bf16 causal GQA 8/2 N1000 d{d} {gen} lambda {lam}")
    q, k, v = gen_prefill_inputs(cfg)
    out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV))
    tot = [0, 0, 0]
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            for t in range(8):
                r = check_prefill_tile(q, k, v, out, st, cnt, b, h, t, Br=128, Bc=64, scale=cfg.scale, causal=True,
                                       lam=lam, n_valid=cfg.N)
                tot = [x + y for x, y in zip(tot, r)]
    _say(f"  visited {tot[0]} skipped {tot[1]} excused {tot[2]}")
    if gen == "sink" and lam >= 0.3:
        assert tot[1] > 0           # the skip path is exercised


@pytest.mark.parametrize("lam", [0.0, 0.3])
def test_fp32_causal_dynamic_csr(lam):
    spec = video_text_spec(frames=3, grid=8, text=20, radius=1, t_radius=1, anchors=4, unit=8)
    n = spec.n_valid
    cfg = _small("f32", dtype="fp32", N=n, d=64, Hq=4, Hkv=2, causal=True, lam=lam, mask=spec,
                 generator="sink", Br=64)
    _say(f"fp32 causal csr dynamic lambda {lam}")
    q, k, v = gen_prefill_inputs(cfg)
    csr = bsa.build_block_index(spec, n, n, 64, 64)
    out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            for t in range(-(-n // 64)):
                check_prefill_tile(q, k, v, out, st, cnt, b, h, t, Br=64, Bc=64, scale=cfg.scale, causal=True,
                                   lam=lam, n_valid=n, row_ptr=csr[0], col_idx=csr[1], fp32=True)


def test_bf16_causal_with_csr():
    spec = dit_image_text_spec(grid=16, text=64, radius=3, anchors=8, unit=16)
    n = spec.n_valid
    cfg = _small("csr_causal", N=n, d=128, Hq=4, Hkv=1, causal=True, lam=0.5, mask=spec, generator="sink")
    _say("bf16 causal + CSR + dynamic")
    q, k, v = gen_prefill_inputs(cfg)
    csr = bsa.build_block_index(spec, n, n, 128, 64)
    out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr)
    for b in range(cfg.B):
        for h in range(cfg.Hq):
            for t in range(-(-n // 128)):
                check_prefill_tile(q, k, v, out, st, cnt, b, h, t, Br=128, Bc=64, scale=cfg.scale, causal=True,
                                   lam=0.5, n_valid=n, row_ptr=csr[0], col_idx=csr[1])


def test_cfg4_full_size_sampled():
    cfg = get_config("cfg4")
    _say("cfg4 bf16 causal GQA 32/8 L32768 d128 lambda 40/L, sampled heads/tiles")
    q, k, v = gen_prefill_inputs(cfg, device=DEV)
    out, st, cnt = run_prefill(cfg, q, k, v)
    tr = 256
    # visited sets of every head/tile: blocks 0..2t+1
    vis_expected = (np.arange(512)[None, :] <= (2 * np.arange(tr) + 1)[:, None])
    assert np.array_equal(st[0, 0] != 0, vis_expected) and np.array_equal(st[0, 31] != 0, vis_expected)
    c = cnt[0].reshape(-1, 2)
    assert c[:, 0].sum() == 32 * sum(2 * t + 2 for t in range(tr))
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    for h in (0, 31):
        for t in (0, 1, 77, 200, 255):
            check_prefill_tile(qh, kh, vh, out, st, cnt, 0, h, t, Br=128, Bc=64, scale=cfg.scale, causal=True,
                               lam=cfg.lam, n_valid=cfg.N)
    _say(f"  cfg4 skipped {int(c[:, 1].sum())} of {int(c[:, 0].sum())} visited blocks")


def test_deterministic_repeat():
    cfg = _small("det", N=700, d=128, Hq=8, Hkv=2, causal=True, lam=0.5, generator="sink")
    _say("determinism")
    q, k, v = (x.to(DEV) for x in gen_prefill_inputs(cfg))
    o1, s1, c1 = run_prefill(cfg, q, k, v)
    o2, s2, c2 = run_prefill(cfg, q, k, v)
    assert torch.equal(o1, o2) and np.array_equal(s1, s2) and np.array_equal(c1, c2)


@pytest.mark.parametrize("d", [64, 128])
def test_deterministic_under_full_load(d):
    """Timing-dependent faults (a load landing on an operand a queued MFMA
    has not read, a missing wait) show as run-to-run differences: the full
    DiT image+text shape (d 64) and a causal GQA 32/8 shape at N 8192
    (d 128), with and without BLASST, five launches each, bit-identical."""
    if d == 64:
        cfg = get_config("cfg2")
        q, k, v = (x.to(DEV) for x in gen_prefill_inputs(cfg))
        rp, ci = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, 128, 64)
        kw = dict(row_ptr=torch.from_numpy(rp).to(DEV), col_idx=torch.from_numpy(ci).to(DEV))
        causal = False
    else:
        cfg = _small("loaded", N=8192, d=128, Hq=32, Hkv=8, B=1, causal=True, generator="concentrated")
        q, k, v = (x.to(DEV) for x in gen_prefill_inputs(cfg))
        kw = {}
        causal = True
    for lam in (0.0, 0.3):
        _say(f"determinism under load: d{d} lambda {lam}")
        outs = [bsa.prefill_fwd(q, k, v, scale=cfg.scale, causal=causal, lam=lam, **kw) for _ in range(5)]
        torch.cuda.synchronize()
        for o in outs[1:]:
            assert torch.equal(o, outs[0])


def test_strided_views():
    """q/k/v as non-contiguous views of a packed [B, N, 3, H, d] tensor, output into a strided view."""
    B, N, H, d = 1, 260, 2, 64
    g = torch.Generator().manual_seed(3)
    qkv = torch.randn((B, N, 3, H, d), generator=g).to(torch.bfloat16)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    cfg = _small("strided", N=N, d=d, Hq=H, Hkv=H)
    _say("strided views")
    qd = qkv.to(DEV)
    outbig = torch.zeros((B, N, H, 2 * d), dtype=torch.bfloat16, device=DEV)
    out = outbig[..., :d]
    bsa.prefill_fwd(qd[:, :, 0], qd[:, :, 1], qd[:, :, 2], out=out, Br=128, Bc=64)
    torch.cuda.synchronize()
    from oracle import attention as A
    for h in range(H):
        ref = A.masked_attention(q[0, :, h], k[0, :, h], v[0, :, h], np.ones((N, N), bool), 1 / math.sqrt(d))
        compare_out(A.as_f64(out[0, :, h].cpu()), ref, False, f"strided h{h}")
    assert torch.all(outbig[..., d:] == 0)


@pytest.mark.parametrize("max_blocks", [1, 3, 9, 100])
def test_schedule_cut_tiles_small(max_blocks):
    """Tiles cut into chunks (partials + merge) give the same outputs, counters and visited sets."""
    spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
    n = spec.n_valid + 13
    for d in (64, 128):
        cfg = _small("sched", N=n, d=d, Hq=4, Hkv=2, mask=spec, generator="iid_offset")
        cfg = PrefillWorkload(**{**cfg.__dict__, "Hkv": 4})
        _say(f"schedule max_blocks {max_blocks} d{d}")
        q, k, v = gen_prefill_inputs(cfg)
        csr = bsa.build_block_index(spec, n, n, 128, 64)
        sched = bsa.build_schedule(csr[0], max_blocks)
        assert (sched.n_slots > 0) == (int(np.diff(csr[0]).max()) > max_blocks)
        ws = bsa.prefill_workspace(cfg.B, cfg.Hq, d, max(sched.n_slots, 1), DEV)
        out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr, schedule=sched, workspace=ws)
        if sched.n_slots:
            # the arrival counters were left at zero: a second call on the same
            # workspace merges again, in slot order whichever chunk ends last
            assert bool((ws != 0).any())  # partials written
            out2, st2, cnt2 = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr, schedule=sched,
                                          workspace=ws)
            assert torch.equal(out, out2) and np.array_equal(cnt, cnt2) and np.array_equal(st, st2)
        for b in range(cfg.B):
            for h in range(cfg.Hq):
                for t in range(3):
                    check_prefill_tile(q, k, v, out, st, cnt, b, h, t, Br=128, Bc=64, scale=cfg.scale,
                                       causal=False, lam=0.0, n_valid=spec.n_valid, row_ptr=csr[0], col_idx=csr[1])


@pytest.mark.parametrize("max_blocks,order,causal", [(3, "ascending", False), (2, "descending", False),
                                                    (3, "ascending", True), (1, "descending", True)])
def test_schedule_cut_tiles_dynamic(max_blocks, order, causal):
    """lambda > 0 with tiles cut into chunks: the chunk-maximum pass lets each
    chunk start from the running max of the chunks visited before it, so skip
    sets, counters and outputs match the whole-row oracle walk."""
    spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
    n = spec.n_valid
    lam = 0.3
    gen = "sink" if order == "ascending" else "sink_last"  # the dominant block is visited first
    tot = [0, 0, 0]
    for d in (64, 128):
        cfg = _small("sched_dyn", N=n, d=d, Hq=4, Hkv=2, mask=spec, generator=gen, causal=causal, lam=lam)
        _say(f"schedule max_blocks {max_blocks} lambda {lam} {order} causal {causal} d{d}")
        q, k, v = gen_prefill_inputs(cfg)
        csr = bsa.build_block_index(spec, n, n, 128, 64)
        sched = bsa.build_schedule(csr[0], max_blocks)
        assert sched.n_slots > 0
        ws = bsa.prefill_workspace(cfg.B, cfg.Hq, d, sched.n_slots, DEV)
        out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr, schedule=sched, workspace=ws,
                                   block_order=order)
        for b in range(cfg.B):
            for h in range(cfg.Hq):
                for t in range(-(-n // 128)):
                    r = check_prefill_tile(q, k, v, out, st, cnt, b, h, t, Br=128, Bc=64, scale=cfg.scale,
                                           causal=causal, lam=lam, n_valid=n, row_ptr=csr[0], col_idx=csr[1],
                                           order=order)
                    tot = [x + y for x, y in zip(tot, r)]
    _say(f"  visited {tot[0]} skipped {tot[1]} excused {tot[2]}")
    assert tot[1] > 0


def test_cfg3_full_size_schedule():
    cfg = get_config("cfg3")
    _say("cfg3 with the default schedule (anchor tile cut into chunks)")
    q, k, v = gen_prefill_inputs(cfg, device=DEV)
    csr = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, 128, 64)
    sched = bsa.build_schedule(csr[0], bsa.default_max_blocks_per_item(csr[0], cfg.B, cfg.Hq))
    assert sched.n_merges >= 1
    out, st, cnt = run_prefill(cfg, q, k, v, csr=csr, schedule=sched)
    assert int((st != 0).sum()) == cfg.Hq * 13839
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    for h in (0, 23):
        for t in (100, 512, 514):
            check_prefill_tile(qh, kh, vh, out, st, cnt, 0, h, t, Br=128, Bc=64, scale=cfg.scale, causal=False,
                               lam=0.0, n_valid=cfg.mask.n_valid, row_ptr=csr[0], col_idx=csr[1], method="two_pass",
                               rows_limit=cfg.mask.n_valid)


def test_prefill_plan_and_graph_replays():
    """A plan gives the eager result; a HIP graph of a cut-tile schedule (whose
    arrival counters must return to zero) replays bit-identically, with other
    GPU work between replays."""
    spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
    n = spec.n_valid + 13
    cfg = _small("graph", N=n, d=64, Hq=4, Hkv=4, mask=spec, generator="iid_offset")
    _say("prefill plan + graph, schedule with cut tiles")
    q, k, v = (x.to(DEV) for x in gen_prefill_inputs(cfg))
    rp_h, ci_h = bsa.build_block_index(spec, n, n, 128, 64)
    sched = bsa.build_schedule(rp_h, 3).to(DEV)
    assert sched.n_merges > 0
    rp, ci = torch.from_numpy(rp_h).to(DEV), torch.from_numpy(ci_h).to(DEV)
    kw = dict(scale=cfg.scale, row_ptr=rp, col_idx=ci, n_valid=spec.n_valid, schedule=sched)
    ref = bsa.prefill_fwd(q, k, v, **kw)
    plan = bsa.prefill_plan(q, k, v, **kw)
    assert torch.equal(plan(), ref)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        plan()
    for r in range(3):
        plan.out.fill_(3.0)
        junk = torch.randn(1 << 20, device=DEV).sum()   # unrelated work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(plan.out, ref), r
    del junk


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("fp32", 64)])
def test_row_counters_match_oracle(dtype, d):
    """Per-row skip conditions counted by the kernel (before the tile-wide vote)
    equal the oracle's count, except (row, block) pairs whose gap lies within
    the excused band around ln(lambda); with a static CSR and dynamic skipping
    together."""
    spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
    n = spec.n_valid + 13
    for lam, gen, csr_on, causal in ((0.3, "sink", False, True), (0.05, "concentrated", True, False),
                                     (0.6, "sink", True, False)):
        cfg = _small("rows", dtype=dtype, N=n, d=d, Hq=4, Hkv=2, causal=causal, lam=lam, generator=gen, seed=12)
        Br = 128 if dtype == "bf16" else 64
        _say(f"row counters {dtype} d{d} lambda {lam} {gen} csr={csr_on} causal={causal}")
        q, k, v = gen_prefill_inputs(cfg)
        csr = bsa.build_block_index(spec, n, n, Br, 64) if csr_on else None
        Tr = -(-n // Br)
        rc = torch.full((cfg.B, cfg.Hq, Tr), -1, dtype=torch.int32, device=DEV)
        rp = ci = None
        if csr is not None:
            rp, ci = torch.from_numpy(csr[0]).to(DEV), torch.from_numpy(csr[1]).to(DEV)
        bsa.prefill_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=cfg.scale, lam=lam, causal=causal, Br=Br, Bc=64,
                        row_ptr=rp, col_idx=ci, n_valid=spec.n_valid, row_counters=rc)
        torch.cuda.synchronize()
        rc = rc.cpu().numpy()
        total = 0
        for b in range(cfg.B):
            for h in range(cfg.Hq):
                g = A.kv_head_of(h, cfg.Hq, cfg.Hkv)
                for t in range(Tr):
                    rows = A.tile_rows(t, Br, n)
                    blocks = A.visited_blocks(t, Br, 64, n, n, causal, *(csr if csr is not None else (None, None)))
                    qr = A.as_f64(q[b, rows[0]:rows[-1] + 1, h])
                    agree, gaps = A.row_agreement(qr, k[b, :, g], rows, blocks, 64, cfg.scale, lam, spec.n_valid,
                                                  causal)
                    near = int(np.count_nonzero(np.abs(gaps - np.log(lam)) <= 1e-3))
                    assert abs(int(rc[b, h, t]) - int(agree.sum())) <= near, (b, h, t, rc[b, h, t], agree.sum(), near)
                    total += int(agree.sum())
        assert total > 0
    # lambda = 0: no test is made, nothing counted
    rc0 = torch.full((cfg.B, cfg.Hq, Tr), -1, dtype=torch.int32, device=DEV)
    bsa.prefill_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=cfg.scale, lam=0.0, Br=Br, Bc=64, row_ptr=rp,
                    col_idx=ci, n_valid=spec.n_valid, row_counters=rc0)
    torch.cuda.synchronize()
    assert int(rc0.cpu().abs().sum()) == 0


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("fp32", 64)])
def test_descending_block_order(dtype, d):
    """Blocks of each tile visited most recent first: causal dynamic and static
    CSR plus dynamic, skip sets and outputs against the oracle in that order."""
    Br = 128 if dtype == "bf16" else 64
    spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
    n = spec.n_valid
    for lam, causal, csr_on, gen in ((0.3, True, False, "sink"), (0.05, True, True, "concentrated"),
                                     (0.6, False, True, "sink")):
        cfg = _small("desc", dtype=dtype, N=n, d=d, Hq=4, Hkv=2, causal=causal, lam=lam, generator=gen, seed=14)
        _say(f"descending order {dtype} d{d} lambda {lam} causal={causal} csr={csr_on}")
        q, k, v = gen_prefill_inputs(cfg)
        csr = bsa.build_block_index(spec, n, n, Br, 64) if csr_on else None
        out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr, Br=Br, block_order="descending")
        tot = [0, 0, 0]
        for b in range(cfg.B):
            for h in range(cfg.Hq):
                for t in range(-(-n // Br)):
                    r = check_prefill_tile(q, k, v, out, st, cnt, b, h, t, Br=Br, Bc=64, scale=cfg.scale,
                                           causal=causal, lam=lam, n_valid=n, fp32=dtype == "fp32",
                                           row_ptr=None if csr is None else csr[0],
                                           col_idx=None if csr is None else csr[1], order="descending")
                    tot = [x + y for x, y in zip(tot, r)]
        _say(f"  visited {tot[0]} skipped {tot[1]} excused {tot[2]}")


def test_prefill_workspace_any_contents():
    """One prefill workspace, filled with random bytes, reused by cut-tile
    schedules whose slot count grows and shrinks, with and without BLASST:
    each call zeroes its arrival counters before the main launch, so stale
    words of an earlier layout never count as arrivals."""
    spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
    n = spec.n_valid
    csr = bsa.build_block_index(spec, n, n, 128, 64)
    cases = [(3, 0.0, 2), (1, 0.0, 2), (9, 0.3, 1), (1, 0.3, 2), (2, 0.0, 1), (1, 0.0, 2)]  # (max_blocks, lam, B)
    scheds = [bsa.build_schedule(csr[0], mb) for mb, _, _ in cases]
    need = max(bsa.prefill_workspace_size(B, 4, 128, max(sc.n_slots, 1)) for sc, (_, _, B) in zip(scheds, cases))
    g = torch.Generator(device=DEV)
    g.manual_seed(98)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV, generator=g)
    for (mb, lam, B), sched in zip(cases, scheds):
        cfg = _small("ws", N=n, d=128, B=B, Hq=4, Hkv=2, mask=spec, generator="sink", causal=False, lam=lam)
        _say(f"prefill workspace with arbitrary contents: max_blocks {mb} ({sched.n_slots} slots) lambda {lam} B{B}")
        q, k, v = gen_prefill_inputs(cfg)
        out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr, schedule=sched, workspace=ws)
        for b in range(B):
            for h in range(cfg.Hq):
                for t in range(-(-n // 128)):
                    check_prefill_tile(q, k, v, out, st, cnt, b, h, t, Br=128, Bc=64, scale=cfg.scale,
                                       causal=False, lam=lam, n_valid=n, row_ptr=csr[0], col_idx=csr[1])


@pytest.mark.parametrize("d", [64, 128])
def test_row_counters_cut_tiles(d):
    """Per-row skip conditions with a schedule that cuts tiles into chunks:
    every chunk publishes its count and the merging chunk sums them."""
    spec = dit_image_text_spec(grid=16, text=40, radius=2, anchors=8, unit=16)
    n = spec.n_valid
    csr = bsa.build_block_index(spec, n, n, 128, 64)
    for lam, order in ((0.3, "ascending"), (0.6, "descending")):
        cfg = _small("rows_cut", N=n, d=d, Hq=4, Hkv=2, lam=lam, mask=spec,
                     generator="sink" if order == "ascending" else "sink_last", seed=13)
        _say(f"row counters with cut tiles d{d} lambda {lam} {order}")
        q, k, v = gen_prefill_inputs(cfg)
        sched = bsa.build_schedule(csr[0], 2)
        assert sched.n_merges > 0
        Tr = -(-n // 128)
        rc = torch.full((cfg.B, cfg.Hq, Tr), -1, dtype=torch.int32, device=DEV)
        bsa.prefill_fwd(q.to(DEV), k.to(DEV), v.to(DEV), scale=cfg.scale, lam=lam, row_ptr=torch.from_numpy(csr[0]).to(DEV),
                        col_idx=torch.from_numpy(csr[1]).to(DEV), n_valid=n, row_counters=rc, schedule=sched,
                        order=order)
        torch.cuda.synchronize()
        rc = rc.cpu().numpy()
        total = 0
        for b in range(cfg.B):
            for h in range(cfg.Hq):
                g = A.kv_head_of(h, cfg.Hq, cfg.Hkv)
                for t in range(Tr):
                    rows = A.tile_rows(t, 128, n)
                    blocks = A.visited_blocks(t, 128, 64, n, n, False, *csr, order=order)
                    agree, gaps = A.row_agreement(A.as_f64(q[b, rows[0]:rows[-1] + 1, h]), k[b, :, g], rows, blocks,
                                                  64, cfg.scale, lam, n, False)
                    near = int(np.count_nonzero(np.abs(gaps - np.log(lam)) <= 1e-3))
                    assert abs(int(rc[b, h, t]) - int(agree.sum())) <= near, (b, h, t, rc[b, h, t], agree.sum())
                    total += int(agree.sum())
        assert total > 0


@pytest.mark.parametrize("d,Br", [(64, 128), (128, 64), (128, 128)])
def test_fp32_instances(d, Br):
    """The fp32 vector path at every head dim and tile height it accepts:
    static CSR, causal with BLASST, dense with a ragged tail; 1e-5 max-abs."""
    spec = video_text_spec(frames=3, grid=8, text=20, radius=1, t_radius=1, anchors=4, unit=8)
    n = spec.n_valid
    for causal, lam, csr_on, gen in ((False, 0.0, True, "iid"), (True, 0.3, True, "sink"), (True, 0.0, False, "iid"),
                                     (False, 0.5, False, "sink")):
        cfg = _small("f32i", dtype="fp32", N=n, d=d, Hq=4, Hkv=2, causal=causal, lam=lam, mask=spec, generator=gen,
                     Br=Br, seed=15)
        _say(f"fp32 d{d} Br{Br} causal={causal} lambda {lam} csr={csr_on}")
        q, k, v = gen_prefill_inputs(cfg)
        csr = bsa.build_block_index(spec, n, n, Br, 64) if csr_on else None
        out, st, cnt = run_prefill(cfg, q.to(DEV), k.to(DEV), v.to(DEV), csr=csr, Br=Br)
        for b in range(cfg.B):
            for h in range(cfg.Hq):
                for t in range(-(-n // Br)):
                    check_prefill_tile(q, k, v, out, st, cnt, b, h, t, Br=Br, Bc=64, scale=cfg.scale, causal=causal,
                                       lam=lam, n_valid=n, row_ptr=None if csr is None else csr[0],
                                       col_idx=None if csr is None else csr[1], fp32=True)
