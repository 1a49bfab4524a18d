#!/usr/bin/env python3
"""Benchmark of block-sparse / BLASST attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg2] [--no-also] [--no-cpu-baseline]

One step = one pass of the attention hot path over one batch of the named
synthetic workload, inputs resident in HBM: the prefill kernel for a prefill
workload (the static block index and schedule are built once, on the host,
before timing: a fixed mask is not rebuilt per step), or the decode kernel
(splits and their merge) for the decode workload.  Each step is one C-ABI
call of a prepared plan.

Timing (HIP events on the launch stream): ``ms_per_step`` and ``value`` come
from exactly K back-to-back steps between one event pair; the roofline's
``achieved`` divides by the average duration of a single launch bracketed by
its own events (a second pass of K steps), the figure the profiler's kernel
trace reports.

Prints ONE JSON line.  ``value`` is the dense-equivalent attention TFLOP/s of
the primary workload (the BLASST causal GQA 32/8 prefill at 32K tokens by
default, the largest prefill and the dominant kernel); ``also`` carries the
same measurement for the other full-size workloads (multimodal DiT
image+text and video DiT static masks, BLASST decode in HBM GB/s), each with
its roofline, its share of skipped blocks and its own ``cpu_baseline``: the
float64 oracle timed on the host cores on a bounded sample of that workload
and extrapolated to the whole of it.

Definitions:
* dense-equivalent FLOPs = 4 B Hq d x (allowed query-key pairs of the full
  problem): Nq * n_valid non-causal, N (N + 1) / 2 causal;
* processed FLOPs (MFMA roofline numerator) = 2 Br Bc d per visited block
  (Q K^T) + 2 Br Bc d per computed block (P V), whole blocks;
* decode algorithmic bytes = K of every visited block + V of every computed
  block + q + out (workspace traffic excluded);
* % skipped = skipped / visited blocks (dynamic) or 1 - kept / all tile-blocks
  (static).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dense-equiv attention TFLOP/s (prefill), HBM GB/s (decode), % blocks skipped"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
KERNEL_SOURCES = {
    "prefill_bf16_kernel": "block_sparse_attention_flash_amd/csrc/prefill_bf16.hip",
    "decode_split_kernel": "block_sparse_attention_flash_amd/csrc/decode.hip",
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(kernel: str) -> str:
    with open(os.path.join(ROOT, KERNEL_SOURCES[kernel]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when absent or taken on a different kernel source."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    e = data.get(kernel, {}).get(workload)
    if not e or e.get("source_sha") != source_sha(kernel):
        return None
    return e.get("bytes_per_launch")


def time_launches(fn, steps: int, warmup: int):
    """HIP-event timing on the current stream (the stream the library launches on).

    Pass 1 times exactly ``steps`` back-to-back steps between one pair of
    events (synchronised on both sides): ``ms_per_step`` is that region / steps.
    Pass 2 brackets every launch with its own events; its average is the
    per-launch duration the profiler's kernel trace reports (each event record
    adds a packet between launches, so it reads a few percent above pass 1)."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    region = e0.elapsed_time(e1) / steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return {"ms_per_step": region, "wall_ms_per_step": wall, "per_launch_avg_ms": sum(per) / len(per),
            "per_launch_median_ms": per[len(per) // 2], "per_launch_min_ms": per[0]}


# ---------------------------------------------------------------------------- prefill

def run_prefill_workload(name: str, steps: int, warmup: int, keep_inputs: bool = False, use_schedule: bool = True):
    import torch
    import block_sparse_attention_flash_amd as bsa
    from workloads import get_config, gen_prefill_inputs

    cfg = get_config(name)
    dev = "cuda"
    log(f"{name}: generating inputs ({cfg.description})")
    q, k, v = gen_prefill_inputs(cfg, device=dev)
    Tr, Tc = -(-cfg.N // cfg.Br), -(-cfg.N // cfg.Bc)
    rp = ci = order = sched = ws = None
    build_ms = None
    if cfg.mask is not None:
        t0 = time.perf_counter()
        rp_h, ci_h = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, cfg.Br, cfg.Bc)
        order_h = bsa.tile_order_lpt(rp_h)
        if use_schedule:
            sched = bsa.default_schedule(rp_h, cfg.B, cfg.Hq, cfg.Hkv, cfg.d)
        build_ms = (time.perf_counter() - t0) * 1e3
        rp, ci, order = (torch.from_numpy(x).to(dev) for x in (rp_h, ci_h, order_h))
        if sched is not None:
            sched.to(dev)
            if sched.n_slots:
                ws = bsa.prefill_workspace(cfg.B, cfg.Hq, cfg.d, sched.n_slots, dev)
    out = torch.empty_like(q)
    counters = torch.zeros((cfg.B, cfg.Hq, Tr, 2), dtype=torch.int32, device=dev)

    def plan(cnt=None):
        return bsa.prefill_plan(q, k, v, scale=cfg.scale, lam=cfg.lam, causal=cfg.causal, Br=cfg.Br, Bc=cfg.Bc,
                                row_ptr=rp, col_idx=ci, tile_order=order, n_valid=cfg.n_valid, out=out,
                                tile_counters=cnt, schedule=sched, workspace=ws)

    plan(counters)()                     # untimed: counts visited / skipped blocks
    call = plan()                        # the timed step: one C-ABI call per launch
    torch.cuda.synchronize()
    c = counters.view(-1, 2).sum(0).tolist()
    visited, skipped = int(c[0]), int(c[1])
    log(f"{name}: timing {steps} steps")
    t = time_launches(call, steps, warmup)
    per_block = 2 * cfg.Br * cfg.Bc * cfg.d
    processed = per_block * (visited + (visited - skipped))
    if cfg.causal:
        pairs = cfg.N * (cfg.N + 1) // 2
    else:
        pairs = cfg.N * cfg.n_valid
    dense = 4 * cfg.B * cfg.Hq * cfg.d * pairs
    ms = t["ms_per_step"]
    achieved = processed / (t["per_launch_avg_ms"] * 1e-3) / 1e12
    if cfg.lam > 0:
        pct = 100.0 * skipped / max(1, visited)
    else:
        pct = 100.0 * (1.0 - visited / (cfg.B * cfg.Hq * Tr * Tc))
    res = {
        "workload": name, "description": cfg.description,
        "value": dense / (ms * 1e-3) / 1e12, "unit": "TFLOP/s (dense-equivalent)",
        "ms_per_step": ms, "timing": t,
        "processed_tflops": achieved,
        "processed_tflops_back_to_back": processed / (ms * 1e-3) / 1e12,
        "pct_blocks_skipped": pct,
        "blocks": {"visited": visited, "skipped": skipped, "computed": visited - skipped,
                   "tile_blocks_total": cfg.B * cfg.Hq * Tr * Tc},
        "lambda": cfg.lam, "block_index_build_ms": build_ms,
        "schedule": None if sched is None else {"items": sched.n_items, "cut_tiles": sched.n_merges,
                                                "partial_slots": sched.n_slots},
        "config": {"workload": f"{name}: {cfg.description}", "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "N": cfg.N, "d": cfg.d,
                   "Br": cfg.Br, "Bc": cfg.Bc, "causal": cfg.causal, "lambda": cfg.lam, "dtype": cfg.dtype},
        "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "per_launch_flops": processed,
                     "traffic": traffic_for("prefill_bf16_kernel", name)},
    }
    if keep_inputs:
        res["_inputs"] = (cfg, q, k, v, rp, ci)
    del q, k, v, out
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------- backward

def visited_pairs(cfg, rp_h, ci_h):
    """(query tile, key block) pairs the forward and backward visit, per (batch, head)."""
    Tr, Tc = -(-cfg.N // cfg.Br), -(-cfg.N // cfg.Bc)
    n = 0
    for t in range(Tr):
        blocks = range(Tc) if rp_h is None else ci_h[rp_h[t]:rp_h[t + 1]]
        last = min((t + 1) * cfg.Br, cfg.N) - 1
        n += sum(1 for j in blocks if not cfg.causal or j * cfg.Bc <= last)
    return n


def run_backward_workload(name: str, steps: int, warmup: int, use_schedule: bool = True):
    """The static block-sparse backward (dot, dK/dV, dQ kernels) on a prefill
    workload at lambda = 0, with the forward timed alongside.  Processed
    FLOPs: the dK/dV kernel computes S, dP, dV, dK (4 products) and the dQ
    kernel S, dP, dQ (3) per visited (tile, block) pair of every head, each
    2 Br Bc d; the usual accounting of a backward counts 5 (S and dP once)."""
    import torch
    import block_sparse_attention_flash_amd as bsa
    from workloads import get_config, gen_prefill_inputs, gen_prefill_grad_output

    cfg = get_config(name)
    dev = "cuda"
    log(f"backward {name}: generating inputs ({cfg.description})")
    q, k, v = gen_prefill_inputs(cfg, device=dev)
    dout = gen_prefill_grad_output(cfg, device=dev)
    Tc = -(-cfg.N // cfg.Bc)
    rp = ci = cp = ri = rp_h = ci_h = sched = fsched = fws = None
    if cfg.mask is not None:
        rp_h, ci_h = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, cfg.Br, cfg.Bc)
        cp_h, ri_h = bsa.transpose_block_index(rp_h, ci_h, Tc)
        rp, ci, cp, ri = (torch.from_numpy(x).to(dev) for x in (rp_h, ci_h, cp_h, ri_h))
        if use_schedule:
            sched = bsa.default_bwd_schedule(rp_h, cp_h, ri_h, cfg.B, cfg.Hq, cfg.Hkv, cfg.d).to(dev)
            fsched = bsa.default_schedule(rp_h, cfg.B, cfg.Hq, cfg.Hkv, cfg.d).to(dev)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.N), dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    if fsched is not None and fsched.n_slots:
        fws = bsa.prefill_workspace(cfg.B, cfg.Hq, cfg.d, fsched.n_slots, dev)
    fwd = bsa.prefill_plan(q, k, v, scale=cfg.scale, causal=cfg.causal, row_ptr=rp, col_idx=ci,
                           n_valid=cfg.n_valid, out=out, lse=lse, schedule=fsched, workspace=fws)
    fwd()
    bwd = bsa.prefill_bwd_plan(q, k, v, out, dout, lse, scale=cfg.scale, causal=cfg.causal, row_ptr=rp,
                               col_idx=ci, col_ptr=cp, row_idx=ri, n_valid=cfg.n_valid, schedule=sched)
    torch.cuda.synchronize()
    pairs = visited_pairs(cfg, rp_h, ci_h) * cfg.B * cfg.Hq
    per_gemm = 2 * cfg.Br * cfg.Bc * cfg.d
    log(f"backward {name}: timing {steps} steps")
    tb = time_launches(bwd, steps, warmup)
    tf = time_launches(fwd, steps, warmup)
    ms = tb["ms_per_step"]
    res = {"workload": name, "description": cfg.description, "ms_per_step": ms, "timing": tb,
           "schedule": None if sched is None else {"dq_items": sched.dq.n_items, "dq_slots": sched.dq.n_slots,
                                                   "kv_items": sched.kv.n_items, "kv_slots": sched.kv.n_slots},
           "forward_ms_per_step": tf["ms_per_step"], "backward_over_forward": ms / tf["ms_per_step"],
           "visited_pairs": pairs,
           "processed_tflops": 7 * per_gemm * pairs / (ms * 1e-3) / 1e12,
           "standard_5gemm_tflops": 5 * per_gemm * pairs / (ms * 1e-3) / 1e12,
           "frac_of_bf16_peak_processed": 7 * per_gemm * pairs / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    log(f"backward {name}: {ms:.4f} ms ({res['backward_over_forward']:.2f}x forward), "
        f"{res['processed_tflops']:.0f} processed TFLOP/s, {res['standard_5gemm_tflops']:.0f} standard")
    del q, k, v, dout, out, lse, fwd, bwd
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------- decode

def run_decode_workload(name: str, steps: int, warmup: int, keep_inputs: bool = False):
    import torch
    import block_sparse_attention_flash_amd as bsa
    from workloads import get_config, gen_decode_inputs

    cfg = get_config(name)
    dev = "cuda"
    log(f"{name}: generating inputs ({cfg.description})")
    q, kc, vc = gen_decode_inputs(cfg, device=dev)
    Tc = -(-cfg.L // cfg.Bc)
    ws = bsa.decode_workspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d, dev, cfg.Bc)
    out = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=torch.bfloat16, device=dev)
    counters = torch.zeros((cfg.B, cfg.Hkv, 2), dtype=torch.int32, device=dev)

    def plan(cnt=None):
        return bsa.decode_plan(q, kc, vc, L=cfg.L, scale=cfg.scale, lam=cfg.lam, Bc=cfg.Bc, workspace=ws, out=out,
                               counters=cnt)

    plan(counters)()
    call = plan()
    torch.cuda.synchronize()
    health = bsa.decode_check(ws)
    c = counters.view(-1, 2).sum(0).tolist()
    visited, skipped = int(c[0]), int(c[1])
    log(f"{name}: timing {steps} steps")
    t = time_launches(call, steps, warmup)
    health_after = bsa.decode_check(ws)          # every timed launch's look-back waits ended in time
    blk_bytes = cfg.Bc * cfg.d * 2
    algo = visited * blk_bytes + (visited - skipped) * blk_bytes + 2 * cfg.B * cfg.Hq * cfg.d * 2
    ms = t["ms_per_step"]
    gbs = algo / (ms * 1e-3) / 1e9
    gbs_launch = algo / (t["per_launch_avg_ms"] * 1e-3) / 1e9
    res = {
        "workload": name, "description": cfg.description,
        "value": gbs, "unit": "GB/s (algorithmic HBM bytes)",
        "ms_per_step": ms, "timing": t,
        "pct_blocks_skipped": 100.0 * skipped / max(1, visited),
        "blocks": {"visited": visited, "skipped": skipped, "computed": visited - skipped},
        "lambda": cfg.lam, "num_splits": bsa.decode_num_splits(cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d, cfg.Bc),
        "health": health, "health_after_timing": health_after,
        "config": {"workload": f"{name}: {cfg.description}", "B": cfg.B, "Hq": cfg.Hq, "Hkv": cfg.Hkv, "L": cfg.L, "d": cfg.d,
                   "Bc": cfg.Bc, "lambda": cfg.lam, "dtype": "bf16"},
        "roofline": {"bound": "hbm", "kernel": "decode_split_kernel",
                     "achieved": gbs_launch, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs_launch / PEAK_HBM_GBS,
                     "per_launch_bytes": algo,
                     "traffic": traffic_for("decode_split_kernel", name)},
    }
    if keep_inputs:
        res["_inputs"] = (cfg, q, kc, vc)
    del q, kc, vc, out, ws
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------- lambda sweep

SWEEP_LAMBDAS = {
    "cfg4_sink": [0.0, 0.3, 0.35, 0.4, 0.45, 0.5, 0.6, 0.7],
    "cfg4": [0.0, 40.0 / 32768, 1e-2, 3e-2, 0.1, 0.2, 0.3, 0.5],
    "cfg2": [0.0, 1e-2, 0.05, 0.1, 0.3],
    "cfg3": [0.0, 1e-2, 0.1, 0.3],
    "cfg5": [0.0, 40.0 / 131072, 1e-3, 1e-2, 0.1],
}


def sweep_prefill(name: str, lams, steps: int, warmup: int):
    """BLASST over each workload's visited blocks (the static CSR when the
    workload has a mask: static and dynamic skipping together) at several
    lambda; per lambda the time, the tile skip share, and the share of
    (row, visited block) pairs whose own row condition held."""
    import numpy as np
    import torch
    import block_sparse_attention_flash_amd as bsa
    from workloads import get_config, gen_prefill_inputs

    cfg = get_config(name)
    dev = "cuda"
    log(f"sweep {name}: generating inputs ({cfg.description})")
    q, k, v = gen_prefill_inputs(cfg, device=dev)
    Tr, Tc = -(-cfg.N // cfg.Br), -(-cfg.N // cfg.Bc)
    rows_per_tile = np.minimum(cfg.Br, cfg.N - np.arange(Tr) * cfg.Br)
    rp = ci = order = sched = ws = None
    if cfg.mask is not None:
        rp_h, ci_h = bsa.build_block_index(cfg.mask, cfg.N, cfg.N, cfg.Br, cfg.Bc)
        order_h = bsa.tile_order_lpt(rp_h)
        sched = bsa.default_schedule(rp_h, cfg.B, cfg.Hq, cfg.Hkv, cfg.d).to(dev)
        rp, ci, order = (torch.from_numpy(x).to(dev) for x in (rp_h, ci_h, order_h))
        if sched.n_slots:
            ws = bsa.prefill_workspace(cfg.B, cfg.Hq, cfg.d, sched.n_slots, dev)
    out = torch.empty_like(q)
    res = []
    base_ms = None
    for lam in lams:
        use_sched = sched  # with lambda > 0 a chunk-maximum pass keeps cut tiles exact
        cnt = torch.zeros((cfg.B, cfg.Hq, Tr, 2), dtype=torch.int32, device=dev)
        rowc = torch.zeros((cfg.B, cfg.Hq, Tr), dtype=torch.int32, device=dev)

        def plan(c=None, r=None):
            return bsa.prefill_plan(q, k, v, scale=cfg.scale, lam=lam, causal=cfg.causal, Br=cfg.Br, Bc=cfg.Bc,
                                    row_ptr=rp, col_idx=ci, tile_order=order, n_valid=cfg.n_valid, out=out,
                                    tile_counters=c, row_counters=r, schedule=use_sched, workspace=ws)

        plan(cnt, rowc)()
        torch.cuda.synchronize()
        c = cnt.cpu().numpy().astype(np.int64)
        rc = rowc.cpu().numpy().astype(np.int64)
        t = time_launches(plan(), steps, warmup)
        ms = t["ms_per_step"]
        base_ms = ms if base_ms is None else base_ms
        visited, skipped = int(c[..., 0].sum()), int(c[..., 1].sum())
        pairs = int((c[..., 0] * rows_per_tile).sum())
        pairs_tile = int((c[..., 1] * rows_per_tile).sum())
        per_block = 2 * cfg.Br * cfg.Bc * cfg.d
        pairs_dense = cfg.N * (cfg.N + 1) // 2 if cfg.causal else cfg.N * cfg.n_valid
        res.append({"lambda": lam, "ms": ms, "speedup_vs_lambda0": base_ms / ms,
                    "pct_blocks_skipped": 100.0 * skipped / max(1, visited),
                    "pct_rows_condition_held": 100.0 * int(rc.sum()) / max(1, pairs) if lam > 0 else 0.0,
                    "pct_rows_in_skipped_blocks": 100.0 * pairs_tile / max(1, pairs),
                    "dense_equiv_tflops": 4 * cfg.B * cfg.Hq * cfg.d * pairs_dense / (ms * 1e-3) / 1e12,
                    "processed_tflops": per_block * (2 * visited - skipped) / (t["per_launch_avg_ms"] * 1e-3) / 1e12,
                    "schedule": use_sched is not None})
        log(f"sweep {name} lambda {lam:.3g}: {ms:.4f} ms, skipped {res[-1]['pct_blocks_skipped']:.2f}% of blocks, "
            f"row condition held for {res[-1]['pct_rows_condition_held']:.2f}% of (row, block) pairs")
    del q, k, v, out
    torch.cuda.empty_cache()
    return {"workload": name, "description": cfg.description, "points": res}


def sweep_decode(name: str, lams, steps: int, warmup: int):
    import torch
    import block_sparse_attention_flash_amd as bsa
    from workloads import get_config, gen_decode_inputs

    cfg = get_config(name)
    dev = "cuda"
    log(f"sweep {name}: generating inputs ({cfg.description})")
    q, kc, vc = gen_decode_inputs(cfg, device=dev)
    ws = bsa.decode_workspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d, dev, cfg.Bc)
    out = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=torch.bfloat16, device=dev)
    res = []
    base_ms = None
    for lam in lams:
        cnt = torch.zeros((cfg.B, cfg.Hkv, 2), dtype=torch.int32, device=dev)
        mk = lambda c=None: bsa.decode_plan(q, kc, vc, L=cfg.L, scale=cfg.scale, lam=lam, Bc=cfg.Bc, workspace=ws,
                                            out=out, counters=c)
        mk(cnt)()
        torch.cuda.synchronize()
        c = cnt.view(-1, 2).sum(0).tolist()
        visited, skipped = int(c[0]), int(c[1])
        t = time_launches(mk(), steps, warmup)
        ms = t["ms_per_step"]
        base_ms = ms if base_ms is None else base_ms
        blk = cfg.Bc * cfg.d * 2
        algo = visited * blk + (visited - skipped) * blk + 2 * cfg.B * cfg.Hq * cfg.d * 2
        res.append({"lambda": lam, "ms": ms, "speedup_vs_lambda0": base_ms / ms,
                    "pct_blocks_skipped": 100.0 * skipped / max(1, visited), "algorithmic_GBs": algo / (ms * 1e-3) / 1e9,
                    "health": bsa.decode_check(ws)})
        log(f"sweep {name} lambda {lam:.3g}: {ms:.4f} ms, skipped {res[-1]['pct_blocks_skipped']:.2f}%")
    del q, kc, vc, out, ws
    torch.cuda.empty_cache()
    return {"workload": name, "description": cfg.description, "points": res}


DECODE_VARIANTS = [
    # (order, max_scope, decisions, num_splits): the first is Algorithm 1 as the pages give it
    ("ascending", "sequence", "group", 0),
    ("ascending", "split", "group", 0),
    ("ascending", "split", "group", 256),
    ("ascending", "sequence", "head", 0),
    ("descending", "sequence", "group", 0),
]


def decode_variants(name: str, lams, steps: int, warmup: int):
    """Order and decision variants of the decode on one workload: time, the
    share of V blocks no head loads, and the share of per-head (or per-group)
    decisions that skip."""
    import torch
    import block_sparse_attention_flash_amd as bsa
    from workloads import get_config, gen_decode_inputs

    cfg = get_config(name)
    dev = "cuda"
    log(f"variants {name}: generating inputs ({cfg.description})")
    q, kc, vc = gen_decode_inputs(cfg, device=dev)
    Tc = -(-cfg.L // cfg.Bc)
    out = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=torch.bfloat16, device=dev)
    res = []
    for lam in lams:
        for order, scope, dec, ns in DECODE_VARIANTS:
            ws = bsa.decode_workspace(cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d, dev, cfg.Bc, ns)
            cnt = torch.zeros((cfg.B, cfg.Hkv, 2), dtype=torch.int32, device=dev)
            st = torch.zeros((cfg.B, cfg.Hq if dec == "head" else cfg.Hkv, Tc), dtype=torch.uint8, device=dev)
            mk = lambda c=None, b=None: bsa.decode_plan(q, kc, vc, L=cfg.L, scale=cfg.scale, lam=lam, Bc=cfg.Bc,
                                                        num_splits=ns, workspace=ws, out=out, counters=c,
                                                        block_state=b, order=order, max_scope=scope, decisions=dec)
            mk(cnt, st)()
            torch.cuda.synchronize()
            c = cnt.view(-1, 2).sum(0).tolist()
            dec_skip = float((st == 2).float().mean().item())
            t = time_launches(mk(), steps, warmup)
            bps = bsa.decode_split_blocks(cfg.B, cfg.Hq, cfg.Hkv, cfg.L, cfg.d, cfg.Bc, ns)
            res.append({"lambda": lam, "order": order, "max_scope": scope, "decisions": dec,
                        "blocks_per_split": bps, "ms": t["ms_per_step"],
                        "pct_V_blocks_skipped": 100.0 * c[1] / max(1, c[0]),
                        "pct_decisions_skip": 100.0 * dec_skip, "health": bsa.decode_check(ws)})
            log(f"variants {name} lambda {lam:.3g} {order}/{scope}/{dec} bps {bps}: {t['ms_per_step']:.4f} ms, "
                f"V skipped {res[-1]['pct_V_blocks_skipped']:.2f}%, decisions skip {100 * dec_skip:.2f}%")
            del ws, st
    del q, kc, vc, out
    torch.cuda.empty_cache()
    return {"workload": name, "description": cfg.description, "points": res}


def calibration_demo(target: float = 0.5, delta: float = 0.05):
    """BLASST threshold calibration (notes section 3.2, Algorithm 2) on the
    synthetic decode recipe at several context lengths, and the comparison
    the notes make in their Table 5: sparsity at the calibrated lambda = a / L
    against one fixed lambda (the best one at the middle length)."""
    import numpy as np
    import torch
    import block_sparse_attention_flash_amd as bsa
    from workloads import gen_decode_inputs
    from workloads.configs import DecodeWorkload

    lengths = [4096, 8192, 16384, 32768, 65536]
    lambdas = list(np.geomspace(1e-9, 1e-2, 43))
    cache = {}

    def inputs(L):
        if L not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cfg = DecodeWorkload(name="cal", description="", B=4, Hq=32, Hkv=8, L=L, d=128, Bc=64, lam=40.0 / L,
                                 seed=11)
            cache[L] = (cfg, gen_decode_inputs(cfg, device="cuda"))
        return cache[L]

    def measure(lam, L):
        cfg, (q, kc, vc) = inputs(L)
        return bsa.decode_sparsity(q, kc, vc, lam=lam, scale=cfg.scale)

    log(f"calibration: target sparsity {target}, {len(lengths)} lengths x {len(lambdas)} thresholds")
    a, n, table = bsa.calibrate(target, lengths, lambdas, delta, measure)
    mid = len(lengths) // 2
    row = np.abs(np.array(table[mid]) - target)
    lam_fixed = float(lambdas[int(np.argmin(row))])
    per = []
    for k, L in enumerate(lengths):
        best = int(np.argmin(np.abs(np.array(table[k]) - target)))
        per.append({"L": L, "lambda_best": float(lambdas[best]), "sparsity_at_best": table[k][best],
                    "sparsity_calibrated": measure(a / L, L) if n else None,
                    "sparsity_fixed_lambda": measure(lam_fixed, L)})
        log(f"calibration L {L}: calibrated {per[-1]['sparsity_calibrated']}, fixed {per[-1]['sparsity_fixed_lambda']}")
    cache.clear()
    torch.cuda.empty_cache()
    return {"target": target, "delta": delta, "a": a, "n_points": n, "fixed_lambda": lam_fixed,
            "recipe": "decode, B4 Hq32 Hkv8 d128, same generator as the 131K decode workload", "per_length": per}


# ---------------------------------------------------------------------------- oracle on host cores

def probe_peaks(steps: int = 20, warmup: int = 5):
    """What this GPU reaches on plain library work, beside the published peaks
    the rooflines use: a large bf16 GEMM (hipBLASLt through torch.matmul) for
    the matrix cores, and memory-bound reductions and a copy over a few GB
    for HBM (bytes moved per second; the copy counts its reads and writes)."""
    import torch
    out = {}

    def best_ms(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    for n in (8192, 16384):
        a_ = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        b_ = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        ms = best_ms(lambda: torch.matmul(a_, b_))
        out[f"gemm_bf16_{n}_tflops"] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
        del a_, b_
    torch.cuda.empty_cache()
    nbytes = 8 << 30
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    rows = x.view(-1, 1 << 16)
    ms = best_ms(lambda: rows.sum(dim=1, dtype=torch.float32))
    out["read_sum_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    ms = best_ms(lambda: rows.amax(dim=1))
    out["read_amax_gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    half = x[: x.numel() // 2]
    y = torch.empty_like(half)
    ms = best_ms(lambda: y.copy_(half))
    out["copy_read_plus_write_gbs"] = round(2 * half.numel() * 2 / (ms * 1e-3) / 1e9, 1)
    del x, y, half, rows
    torch.cuda.empty_cache()
    out["published_bf16_tflops"] = PEAK_BF16_TFLOPS
    out["published_hbm_gbs"] = PEAK_HBM_GBS
    return out


def host_info():
    """Host cores available to this process, the BLAS threads the oracle's
    numpy products use, torch's CPU threads, and the CPU model."""
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max((x.get("num_threads", 1) for x in threadpool_info() if x.get("user_api") == "blas"), default=1)
    except Exception:
        blas = None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    import torch
    return {"host_cores_available": cores, "blas_threads": blas, "torch_cpu_threads": torch.get_num_threads(),
            "cpu_model": model}


def cpu_baseline_prefill(res, budget_s: float):
    """Time the float64 oracle (as it stands) on a bounded sample of the same
    workload's (batch, head, tile) items and extrapolate by processed blocks."""
    import numpy as np
    from oracle import attention as A
    cfg, q, k, v, rp, ci = res["_inputs"]
    qh, kh, vh = q.cpu(), k.cpu(), v.cpu()
    rp_h = rp.cpu().numpy() if rp is not None else None
    ci_h = ci.cpu().numpy() if ci is not None else None
    Tr = -(-cfg.N // cfg.Br)
    rng = np.random.default_rng(0)
    items = [(b, h, t) for b in range(cfg.B) for h in range(cfg.Hq) for t in range(Tr)]
    rng.shuffle(items)
    method = "two_pass" if cfg.lam == 0.0 else "loop"
    done_blocks = 0
    n_items = 0
    t0 = time.perf_counter()
    for (b, h, t) in items:
        _, _, blocks, _, _ = A.prefill_tile(qh, kh, vh, b, h, t, Br=cfg.Br, Bc=cfg.Bc, scale=cfg.scale,
                                            causal=cfg.causal, lam=cfg.lam, n_valid=cfg.n_valid,
                                            row_ptr=rp_h, col_idx=ci_h, method=method)
        done_blocks += len(blocks)
        n_items += 1
        if time.perf_counter() - t0 > budget_s:
            break
    el = time.perf_counter() - t0
    est = el * res["blocks"]["visited"] / max(1, done_blocks)
    info = host_info()
    dense = res["value"] * res["ms_per_step"] * 1e-3 * 1e12
    return {"value": dense / est / 1e12, "unit": "TFLOP/s (dense-equivalent)",
            "cores": info["blas_threads"] or info["host_cores_available"], "kind": "oracle",
            "sample": f"{n_items} of {len(items)} (batch, head, tile) items of {res['workload']} in "
                      f"{el:.1f} s, {done_blocks} of {res['blocks']['visited']} visited blocks; full-workload "
                      f"time extrapolated by visited blocks to {est:.1f} s",
            "measured_s": el, "extrapolated_s": est,
            "method": f"oracle.attention.prefill_tile(method={method!r}), float64 numpy", **info}


def cpu_baseline_decode(res, budget_s: float):
    """Time the float64 decode oracle (closed form of Algorithm 1 per sequence
    and K/V head) on whole sequences until the budget is spent, and
    extrapolate by sequences to the batch."""
    from oracle import attention as A
    cfg, q, kc, vc = res["_inputs"]
    n_seq = 0
    t_oracle = 0.0
    t0 = time.perf_counter()
    for b in range(cfg.B):
        qb, kb, vb = q[b].cpu(), kc[b].cpu(), vc[b].cpu()        # one sequence on the host at a time
        t1 = time.perf_counter()
        A.decode_sequence(qb, kb, vb, cfg.Bc, cfg.scale, cfg.lam, "closed_form")
        t_oracle += time.perf_counter() - t1
        n_seq += 1
        del qb, kb, vb
        if time.perf_counter() - t0 > budget_s:
            break
    est = t_oracle * cfg.B / n_seq
    info = host_info()
    algo = res["roofline"]["per_launch_bytes"]
    return {"value": algo / est / 1e9, "unit": "GB/s (algorithmic HBM bytes)",
            "cores": info["blas_threads"] or info["host_cores_available"], "kind": "oracle",
            "sample": f"{n_seq} of {cfg.B} sequences (all {cfg.Hkv} K/V heads each) of {res['workload']}: "
                      f"{t_oracle:.1f} s in the oracle (host copies excluded); batch time extrapolated by "
                      f"sequences to {est:.1f} s",
            "measured_s": t_oracle, "extrapolated_s": est,
            "method": "oracle.attention.decode_sequence(method='closed_form'), float64 numpy", **info}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # an 80 us kernel needs a few hundred launches before the clocks settle
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="cfg4", choices=["cfg2", "cfg3", "cfg4", "cfg5", "cfg4_sink"])
    ap.add_argument("--also", default="cfg2,cfg3,cfg5", help="comma list of further workloads ('' for none)")
    ap.add_argument("--no-also", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-schedule", action="store_true", help="one work-group per tile or key block (no cutting of long ones)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget per workload")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the metric line: a lambda sweep (static + dynamic skipping together) per "
                         "workload, as one JSON line")
    ap.add_argument("--sweep-only", default="", help="with --sweep: comma list of workloads to sweep (no variants "
                                                     "or calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="instead of the metric line: the static block-sparse backward on the prefill workloads")
    ap.add_argument("--variants", action="store_true",
                    help="instead of the metric line: the decode order and decision variants on the decode workload")
    ap.add_argument("--probe-peaks", action="store_true",
                    help="instead of the metric line: what a large library GEMM and memory-bound reductions reach")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy (reference for HBM byte counters)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(json.dumps({"error": "runs on one GPU only: the kernels need no collectives; the path would "
                                   "shard by (batch, head) or by query tiles, one process per GPU",
                          "n_gpus": a.gpus}))
        return 2
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    import block_sparse_attention_flash_amd as bsa
    bsa.library()

    def run(name, keep=False):
        if name == "cfg5":
            return run_decode_workload(name, a.steps, a.warmup, keep_inputs=keep)
        return run_prefill_workload(name, a.steps, a.warmup, keep_inputs=keep, use_schedule=not a.no_schedule)

    def with_baseline(name):
        r = run(name, keep=not a.no_cpu_baseline)
        if "_inputs" in r:
            log(f"{name}: oracle baseline on host cores (~{a.cpu_seconds:.0f} s)")
            r["cpu_baseline"] = (cpu_baseline_decode if name == "cfg5" else cpu_baseline_prefill)(r, a.cpu_seconds)
            r.pop("_inputs")
        torch.cuda.empty_cache()
        return r

    torch.cuda.synchronize()
    if a.sweep:
        rep = []
        for name, lams in SWEEP_LAMBDAS.items():
            if a.sweep_only and name not in a.sweep_only.split(","):
                continue
            fn = sweep_decode if name == "cfg5" else sweep_prefill
            rep.append(fn(name, lams, min(a.steps, 50) if name != "cfg2" else a.steps, min(a.warmup, 20)
                          if name != "cfg2" else a.warmup))
        if a.sweep_only:
            print(json.dumps({"sweep": rep, "steps": a.steps, "device": torch.cuda.get_device_name(0)}))
            return 0
        var = decode_variants("cfg5", [40.0 / 131072, 1e-2, 0.1], min(a.steps, 50), min(a.warmup, 20))
        cal = calibration_demo()
        print(json.dumps({"sweep": rep, "decode_variants": var, "calibration": cal, "steps": a.steps,
                          "device": torch.cuda.get_device_name(0)}))
        return 0
    if a.backward:
        names = [a.workload] + [n for n in (a.also.split(",") if a.also and not a.no_also else []) if n != "cfg5"]
        rep = [run_backward_workload(n, a.steps, a.warmup, use_schedule=not a.no_schedule) for n in names]
        print(json.dumps({"backward": rep, "device": torch.cuda.get_device_name(0)}))
        return 0
    if a.probe_peaks:
        print(json.dumps({"probe_peaks": probe_peaks(), "device": torch.cuda.get_device_name(0)}))
        return 0
    if a.variants:
        var = decode_variants("cfg5", [40.0 / 131072, 1e-2, 0.1], min(a.steps, 50), min(a.warmup, 20))
        print(json.dumps({"decode_variants": var, "device": torch.cuda.get_device_name(0)}))
        return 0
    if a.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 copies of 1 GiB (reads 1 GiB, writes 1 GiB each)")
        del src, dst
        torch.cuda.empty_cache()
    prim = with_baseline(a.workload)
    cpu = prim.pop("cpu_baseline", None)
    also = []
    if not a.no_also and a.also:
        for name in [x for x in a.also.split(",") if x and x != a.workload]:
            also.append(with_baseline(name))
    line = {
        "metric": METRIC, "value": prim["value"], "unit": prim["unit"].split(" ")[0],
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": prim["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded generators shaped like the pages' workloads)",
        "config": prim["config"],
        "pct_blocks_skipped": prim["pct_blocks_skipped"],
        "roofline": prim["roofline"], "cpu_baseline": cpu,
        "primary": {k: v for k, v in prim.items() if k not in ("config", "roofline")},
        "also": also,
        "device": torch.cuda.get_device_name(0),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
