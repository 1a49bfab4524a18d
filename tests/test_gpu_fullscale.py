"""Full-launch parity of the BLASST prefill where blocks really are skipped.

The literal workload recipes rarely skip a whole tile (the tile-wide vote of
BLASST notes section 4 binds), so these tests take the full shapes with
inputs that do skip:

* the causal GQA 32/8 prefill shape (B1, L 32768, d 128) with the "sink"
  recipe at lambda 0.5 (about 70 % of visited blocks skipped): skip sets and
  counters of all 32 heads x 256 tiles from one launch of 8192 work-groups,
  outputs on sampled tiles;
* the video DiT shape (B1, H24, N 65920, d 128) with its own inputs, its
  static block mask and the default cut-tile schedule at lambda 0.8, where
  the anchor tile (1029 kept blocks, cut into chunks) skips about half its
  blocks: the chunk-maximum pass and the vote run under a full launch; skip
  sets of every head and tile, outputs of the cut tile and others.

Skip sets are compared with the oracle's closed form (skip_set_batched,
float64), blocks within 1e-3 of the threshold excused.
"""

import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_flash_amd as bsa
from oracle import attention as A
from workloads import get_config, gen_prefill_inputs
from workloads.configs import PrefillWorkload

from _parity import MARGIN, check_prefill_tile

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[gpu-fullscale] {msg}", file=sys.stderr, flush=True)


def _check_skip_sets(q, k, st, cnt, heads, tiles, *, Br, Bc, scale, lam, n_valid, causal, row_ptr=None,
                     col_idx=None):
    """Visited and skip sets of (head, tile) pairs against the oracle; returns (visited, skipped, excused)."""
    B, N, Hq, _ = q.shape
    Hkv = k.shape[2]
    tot = [0, 0, 0]
    for h in heads:
        g = A.kv_head_of(h, Hq, Hkv)
        qq = q[0, :, h].to(torch.float64)
        kk = k[0, :, g].to(torch.float64)
        for t in tiles:
            rows = A.tile_rows(t, Br, N)
            blocks = A.visited_blocks(t, Br, Bc, N, N, causal, row_ptr, col_idx)
            skip, margin = A.skip_set_batched(qq[rows[0]:rows[-1] + 1], kk, rows, blocks, Bc, scale, lam, n_valid,
                                              causal)
            s = st[0, h, t]
            vis = np.zeros(s.shape[0], bool)
            vis[blocks] = True
            assert np.array_equal(s != 0, vis), f"visited set differs h{h} t{t}"
            g_skip = s[blocks] == 2
            excused = np.abs(margin) <= MARGIN
            bad = (g_skip != skip) & ~excused
            assert not bad.any(), f"skip set differs h{h} t{t}: blocks {blocks[bad]} margins {margin[bad]}"
            assert cnt[0, h, t, 0] == len(blocks) and cnt[0, h, t, 1] == int(g_skip.sum()), (h, t, cnt[0, h, t])
            tot[0] += len(blocks)
            tot[1] += int(g_skip.sum())
            tot[2] += int(excused.sum())
    return tot


def _cfg4_sink():
    c = get_config("cfg4")
    return PrefillWorkload(name="cfg4_sink", description="causal GQA 32/8 L32768 d128, sink recipe", dtype="bf16",
                           B=c.B, Hq=c.Hq, Hkv=c.Hkv, N=c.N, d=c.d, Br=128, Bc=64, causal=True, lam=0.5, mask=None,
                           seed=c.seed, generator="sink")


@pytest.fixture(scope="module")
def cfg4_sink_run():
    cfg = _cfg4_sink()
    _say("causal GQA 32/8 L32768 d128 sink recipe, lambda 0.5: one full launch")
    q, k, v = gen_prefill_inputs(cfg, device=DEV)
    Tr, Tc = cfg.N // 128, cfg.N // 64
    st = torch.zeros((1, cfg.Hq, Tr, Tc), dtype=torch.uint8, device=DEV)
    cnt = torch.full((1, cfg.Hq, Tr, 2), -1, dtype=torch.int32, device=DEV)
    out = bsa.prefill_fwd(q, k, v, scale=cfg.scale, lam=cfg.lam, causal=True, tile_counters=cnt, block_state=st)
    torch.cuda.synchronize()
    return cfg, q.cpu(), k.cpu(), v.cpu(), out.cpu(), st.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("heads", [range(0, 8), range(8, 16), range(16, 24), range(24, 32)],
                         ids=["h0-7", "h8-15", "h16-23", "h24-31"])
def test_cfg4_shape_sink_skip_sets_all_tiles(cfg4_sink_run, heads):
    cfg, q, k, v, out, st, cnt = cfg4_sink_run
    _say(f"  skip sets, heads {heads.start}-{heads.stop - 1}, all 256 tiles")
    tot = _check_skip_sets(q, k, st, cnt, heads, range(cfg.N // 128), Br=128, Bc=64, scale=cfg.scale,
                           lam=cfg.lam, n_valid=cfg.N, causal=True)
    _say(f"  visited {tot[0]} skipped {tot[1]} ({100.0 * tot[1] / tot[0]:.1f} %) excused {tot[2]}")
    assert tot[1] >= 0.3 * tot[0]


def test_cfg4_shape_sink_outputs_sampled(cfg4_sink_run):
    cfg, q, k, v, out, st, cnt = cfg4_sink_run
    tot = [0, 0, 0]
    for h in (0, 13, 31):
        for t in (0, 1, 77, 200, 255):
            _say(f"  output h{h} t{t}")
            r = check_prefill_tile(q, k, v, out, st, cnt, 0, h, t, Br=128, Bc=64, scale=cfg.scale, causal=True,
                                   lam=cfg.lam, n_valid=cfg.N)
            tot = [x + y for x, y in zip(tot, r)]
    assert tot[1] > 0


def test_cfg3_schedule_dynamic_full_launch():
    cfg = get_config("cfg3")
    lam = 0.8
    _say(f"video DiT N65920 d128, static mask + default schedule (tile order), lambda {lam}")
    q, k, v = gen_prefill_inputs(cfg, device=DEV)
    rp, ci = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, 128, 64)
    sched = bsa.default_schedule(rp, cfg.B, cfg.Hq, cfg.Hkv, cfg.d)
    assert sched.n_merges >= 1
    Tr, Tc = cfg.N // 128, cfg.N // 64
    st = torch.zeros((1, cfg.Hq, Tr, Tc), dtype=torch.uint8, device=DEV)
    cnt = torch.full((1, cfg.Hq, Tr, 2), -1, dtype=torch.int32, device=DEV)
    rc = torch.full((1, cfg.Hq, Tr), -1, dtype=torch.int32, device=DEV)
    out = bsa.prefill_fwd(q, k, v, scale=cfg.scale, lam=lam, row_ptr=torch.from_numpy(rp).to(DEV),
                          col_idx=torch.from_numpy(ci).to(DEV), n_valid=cfg.mask.n_valid, tile_counters=cnt,
                          block_state=st, row_counters=rc, schedule=sched)
    torch.cuda.synchronize()
    qh, kh, vh, oh = q.cpu(), k.cpu(), v.cpu(), out.cpu()
    st, cnt, rc = st.cpu().numpy(), cnt.cpu().numpy(), rc.cpu().numpy()
    cut = [int(t) for t in sched.merges[:, 0]]
    tot = _check_skip_sets(qh, kh, st, cnt, range(cfg.Hq), range(Tr), Br=128, Bc=64, scale=cfg.scale, lam=lam,
                           n_valid=cfg.mask.n_valid, causal=False, row_ptr=rp, col_idx=ci)
    cut_skipped = int((st[0][:, cut] == 2).sum())
    _say(f"  visited {tot[0]} skipped {tot[1]} (cut tiles {cut}: {cut_skipped}) excused {tot[2]}")
    assert cut_skipped > 0
    # per-row counters of the cut tile (chunks publish theirs, the merge sums them)
    for h in (0, 23):
        for t in cut:
            rows = A.tile_rows(t, 128, cfg.N)
            blocks = A.visited_blocks(t, 128, 64, cfg.N, cfg.N, False, rp, ci)
            agree, gaps = A.row_agreement(A.as_f64(qh[0, rows[0]:rows[-1] + 1, h]), kh[0, :, h], rows, blocks, 64,
                                          cfg.scale, lam, cfg.mask.n_valid, False)
            near = int(np.count_nonzero(np.abs(gaps - np.log(lam)) <= MARGIN))
            assert abs(int(rc[0, h, t]) - int(agree.sum())) <= near, (h, t, rc[0, h, t], agree.sum(), near)
    # outputs: the cut tile and a few others, two heads
    for h in (0, 23):
        for t in cut + [0, 257, 514]:
            _say(f"  output h{h} t{t}")
            check_prefill_tile(qh, kh, vh, oh, st, cnt, 0, h, t, Br=128, Bc=64, scale=cfg.scale, causal=False,
                               lam=lam, n_valid=cfg.mask.n_valid, row_ptr=rp, col_idx=ci,
                               rows_limit=cfg.mask.n_valid)


def test_cfg3_schedule_orders_bit_identical():
    """The launch order of work items changes nothing in the results: the
    video DiT prefill with its schedule longest first and in tile order."""
    cfg = get_config("cfg3")
    _say("video DiT N65920 d128, schedule longest first against tile order, lambda 0")
    q, k, v = gen_prefill_inputs(cfg, device=DEV)
    rp, ci = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, 128, 64)
    mb = bsa.default_max_blocks_per_item(rp, cfg.B, cfg.Hq)
    rp_d, ci_d = torch.from_numpy(rp).to(DEV), torch.from_numpy(ci).to(DEV)
    outs = []
    for order in ("longest_first", "tile"):
        sched = bsa.build_schedule(rp, mb, order=order)
        outs.append(bsa.prefill_fwd(q, k, v, scale=cfg.scale, row_ptr=rp_d, col_idx=ci_d, n_valid=cfg.mask.n_valid,
                                    schedule=sched))
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
