"""Oracle for the gradients of static block-sparse attention (test infrastructure only).

The forward is the masked softmax attention of ``oracle.attention`` over the
token mask that a tile mask expands to: tiles of the mask are kept or dropped
whole (DiT article "块稀疏Attention实战", section 2.3), masked entries are absent
from the softmax statistics (section 5.2), keys past the valid length and,
when causal, keys after the query are not attended.  The pages print no
backward pass; the DiT article's training experiments (section 4) take it
for granted.  The gradients here are the chain rule applied to that
definition, written out once (the attention tutorial's section on the
softmax and the usual textbook derivation), in float64:

    S  = scale * Q K^T                       (allowed entries only)
    P  = softmax of S over each row's allowed entries, 0 elsewhere
    O  = P V
    dV = P^T dO
    dP = dO V^T
    dS_ij = P_ij * (dP_ij - sum_k P_ik dP_ik)      (softmax Jacobian)
    dQ = scale * dS K,   dK = scale * dS^T Q

A row with no allowed key has O = 0 and contributes no gradient.  With GQA
(query head h reads K/V head h // (Hq / Hkv)), dK and dV of a K/V head sum
the contributions of its query heads.

``row_lse`` is the natural log of each row's sum of exp(S) over its allowed
entries (-inf for a row with none): the per-row statistic a forward pass
keeps so that a backward pass can rebuild P without a second max pass.
"""

from __future__ import annotations

import numpy as np

from .attention import as_f64


def row_lse(q, k, allowed, scale: float) -> np.ndarray:
    """log(sum_j exp(scale q_i . k_j)) over allowed j, per row; -inf if none."""
    q, k = as_f64(q), as_f64(k)
    S = np.where(allowed, scale * (q @ k.T), -np.inf)
    m = S.max(axis=1, initial=-np.inf)
    safe = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        return np.where(np.isfinite(m), safe + np.log(np.exp(S - safe[:, None]).sum(axis=1)), -np.inf)


def masked_attention_grads(q, k, v, dout, allowed, scale: float):
    """(dq [Nq, d], dk [Nk, d], dv [Nk, dv]) of sum(out * dout) for
    out = masked_attention(q, k, v, allowed, scale), one head."""
    q, k, v, dout = as_f64(q), as_f64(k), as_f64(v), as_f64(dout)
    S = np.where(allowed, scale * (q @ k.T), -np.inf)
    has = allowed.any(axis=1)
    m = np.where(has, S.max(axis=1, initial=-np.inf), 0.0)
    E = np.where(allowed, np.exp(S - m[:, None]), 0.0)
    l = np.where(has, E.sum(axis=1), 1.0)
    P = E / l[:, None]
    dv = P.T @ dout
    dP = dout @ v.T
    dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
    dq = scale * (dS @ k)
    dk = scale * (dS.T @ q)
    return dq, dk, dv


def prefill_grads(q, k, v, dout, token_mask, scale: float):
    """Gradients over [B, N, H, d] tensors: q, dout [B, Nq, Hq, d], k, v
    [B, Nk, Hkv, d], token_mask bool [Nq, Nk] shared by every batch and head.
    Returns dq [B, Nq, Hq, d], dk, dv [B, Nk, Hkv, d] as float64 arrays."""
    q, k, v, dout = as_f64(q), as_f64(k), as_f64(v), as_f64(dout)
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros((B, Nk, Hkv, d))
    dv = np.zeros((B, Nk, Hkv, v.shape[3]))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            gq, gk, gv = masked_attention_grads(q[b, :, h], k[b, :, g], v[b, :, g], dout[b, :, h], token_mask, scale)
            dq[b, :, h] = gq
            dk[b, :, g] += gk
            dv[b, :, g] += gv
    return dq, dk, dv


def prefill_lse(q, k, token_mask, scale: float) -> np.ndarray:
    """row_lse for every (batch, query head): [B, Hq, Nq]."""
    q, k = as_f64(q), as_f64(k)
    B, Nq, Hq, _ = q.shape
    G = Hq // k.shape[2]
    out = np.empty((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            out[b, h] = row_lse(q[b, :, h], k[b, :, h // G], token_mask, scale)
    return out
