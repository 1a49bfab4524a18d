"""Seeded synthetic inputs.

Layouts follow the flash-attention calling convention used on the attention
tutorial page (``q`` as ``[batch, seq, heads, head_dim]``):

* prefill: Q ``[B, N, Hq, d]``, K and V ``[B, N, Hkv, d]``;
* decode:  q ``[B, Hq, d]`` (one new token per sequence), K/V cache
  ``[B, L, Hkv, d]`` contiguous.

Values are drawn in float32 with ``torch.Generator`` streams keyed by
(workload seed, tensor tag, sequence) and then rounded once to the storage
dtype (round-to-nearest-even for bf16).  The rounded tensors are what both
the GPU path and the oracle consume; the oracle upcasts them exactly to
float64.  Draws made on a CUDA generator differ from CPU draws, so a test
must hand the oracle host copies of the very tensors the GPU used.

Generator readings (the workload text names them, the pages do not):

* ``p(i)``: sinusoidal position code in ``d`` dims, interleaved
  ``p[2k] = sin(i w_k)``, ``p[2k+1] = cos(i w_k)``, ``w_k = 10000^(-2k/d)``,
  divided by ``sqrt(d/2)`` so that ``|p(i)| = 1``.
* "mean-query vector" of a KV head: mean of the float32 query vectors of
  the G query heads sharing that KV head, over every query position
  (prefill) or over the G heads of the single decode step.
* cfg2 offset: one random direction per head, scaled to norm 2, added to
  every Q, K and V row of that head.
* "sink" (test recipe for the skip path): every query gets 4 w and the first
  64 keys get 10 w, w one random unit direction shared by all heads.
* "sink_last": the same with the sink on the last 64 keys (test recipe for
  the recent-first order).
"""

from __future__ import annotations

import numpy as np
import torch

from .configs import DecodeWorkload, PrefillWorkload

_TAG_Q, _TAG_K, _TAG_V, _TAG_OFF, _TAG_DO = 1, 2, 3, 4, 5


def _gen(seed: int, tag: int, sub: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1_000_003 + tag * 7919 + sub)
    return g


def _randn(shape, seed, tag, sub, device) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(seed, tag, sub, device), device=device,
                       dtype=torch.float32)


def sinusoidal_position(positions, d: int) -> torch.Tensor:
    """Unit-norm interleaved sinusoidal code, float32 ``[len(positions), d]``."""
    pos = np.asarray(positions, dtype=np.float64)[:, None]
    k = np.arange(d // 2, dtype=np.float64)[None, :]
    w = 10000.0 ** (-2.0 * k / d)
    out = np.empty((pos.shape[0], d), dtype=np.float64)
    out[:, 0::2] = np.sin(pos * w)
    out[:, 1::2] = np.cos(pos * w)
    out /= np.sqrt(d / 2.0)
    return torch.from_numpy(out.astype(np.float32))


def _store_dtype(cfg) -> torch.dtype:
    return torch.float32 if getattr(cfg, "dtype", "bf16") == "fp32" else torch.bfloat16


def gen_prefill_inputs(cfg: PrefillWorkload, device="cpu", B=None, N=None):
    """Return (q, k, v) for a prefill workload.  ``B``/``N`` override the
    batch and length (used for reduced parity cases with the same recipe)."""
    B = cfg.B if B is None else B
    N = cfg.N if N is None else N
    Hq, Hkv, d = cfg.Hq, cfg.Hkv, cfg.d
    dev = torch.device(device)
    q = _randn((B, N, Hq, d), cfg.seed, _TAG_Q, 0, dev)
    k = _randn((B, N, Hkv, d), cfg.seed, _TAG_K, 0, dev)
    v = _randn((B, N, Hkv, d), cfg.seed, _TAG_V, 0, dev)
    if cfg.generator == "iid_offset":
        # one direction per head, norm 2, shared by Q, K and V rows of that head
        if Hkv != Hq:
            raise ValueError("the per-head offset recipe is defined for Hq == Hkv")
        off = _randn((Hq, d), cfg.seed, _TAG_OFF, 0, dev)
        off = 2.0 * off / off.norm(dim=-1, keepdim=True)
        q += off[None, None]
        k += off[None, None]
        v += off[None, None]
    elif cfg.generator == "concentrated":
        p = sinusoidal_position(range(N), d).to(dev)          # [N, d]
        q += 3.0 * p[None, :, None, :]
        k += 3.0 * p[None, :, None, :]
        G = Hq // Hkv
        # mean query of each KV group over all positions and the group's heads
        mq = q.view(B, N, Hkv, G, d).mean(dim=(1, 3))          # [B, Hkv, d]
        ns = min(64, N)
        k[:, :ns] += 4.0 * mq[:, None, :, :]
    elif cfg.generator in ("sink", "sink_last"):
        # a shared query direction w (norm 4) and a sink of 64 keys along w
        # (norm 10): scores against the sink exceed the others by ~40*scale,
        # so whole key blocks fall below the BLASST threshold
        w = _randn((d,), cfg.seed, _TAG_OFF, 0, dev)
        w = w / w.norm()
        q += 4.0 * w
        ns = min(64, N)
        if cfg.generator == "sink":
            k[:, :ns] += 10.0 * w
        else:  # the mirror: the sink is the last 64 keys (found first when recent blocks go first)
            k[:, N - ns:] += 10.0 * w
    elif cfg.generator != "iid":
        raise ValueError(cfg.generator)
    dt = _store_dtype(cfg)
    return q.to(dt).contiguous(), k.to(dt).contiguous(), v.to(dt).contiguous()


def gen_prefill_grad_output(cfg: PrefillWorkload, device="cpu", B=None, N=None):
    """Gradient of the loss w.r.t. the prefill output, dO [B, N, Hq, d]:
    i.i.d. N(0, 1), rounded to the storage dtype (the backward's input)."""
    B = cfg.B if B is None else B
    N = cfg.N if N is None else N
    g = _randn((B, N, cfg.Hq, cfg.d), cfg.seed, _TAG_DO, 0, torch.device(device))
    return g.to(_store_dtype(cfg)).contiguous()


def gen_decode_sequence(cfg: DecodeWorkload, b: int, device="cpu", L=None):
    """One sequence of the decode workload: (q [Hq, d], k [L, Hkv, d], v [L, Hkv, d]) in bf16.

    The query is the token at position L-1; keys carry the position code of
    their own position, so attention concentrates on recent keys and on the
    first 64 keys (the sink)."""
    L = cfg.L if L is None else L
    Hq, Hkv, d = cfg.Hq, cfg.Hkv, cfg.d
    G = Hq // Hkv
    dev = torch.device(device)
    pq = sinusoidal_position([L - 1], d).to(dev)[0]
    q = _randn((Hq, d), cfg.seed, _TAG_Q, b, dev) + 3.0 * pq[None, :]
    k = _randn((L, Hkv, d), cfg.seed, _TAG_K, b, dev)
    chunk = 1 << 16
    for s in range(0, L, chunk):
        e = min(L, s + chunk)
        k[s:e] += 3.0 * sinusoidal_position(range(s, e), d).to(dev)[:, None, :]
    mq = q.view(Hkv, G, d).mean(dim=1)                          # [Hkv, d]
    ns = min(64, L)
    k[:ns] += 4.0 * mq[None, :, :]
    v = _randn((L, Hkv, d), cfg.seed, _TAG_V, b, dev)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16)


def gen_decode_inputs(cfg: DecodeWorkload, device="cpu", B=None, L=None):
    """Full decode batch: q [B, Hq, d], k_cache/v_cache [B, L, Hkv, d] (bf16, contiguous).

    Sequences are generated one at a time straight into the preallocated
    cache so peak memory stays at one float32 sequence."""
    B = cfg.B if B is None else B
    L = cfg.L if L is None else L
    dev = torch.device(device)
    q = torch.empty((B, cfg.Hq, cfg.d), dtype=torch.bfloat16, device=dev)
    kc = torch.empty((B, L, cfg.Hkv, cfg.d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty((B, L, cfg.Hkv, cfg.d), dtype=torch.bfloat16, device=dev)
    for b in range(B):
        qb, kb, vb = gen_decode_sequence(cfg, b, dev, L=L)
        q[b], kc[b], vc[b] = qb, kb, vb
        del qb, kb, vb
    return q, kc, vc
