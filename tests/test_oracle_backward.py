"""Pins for the float64 backward oracle (CPU only).

Each test ties ``oracle.backward`` to something other than its own formulas:
central finite differences of the forward oracle, a case worked by hand,
torch's float64 autograd through its own attention routine (a library
routine) for the dense special case, identities every softmax gradient obeys
(dK sums to zero over keys, dV sums to the attended rows' dO), and the
structure of a mask (unattended keys and empty rows get no gradient).
"""

import math

import numpy as np
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle import backward as BW
from oracle import masks as M


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _loss(q, k, v, dout, allowed, scale):
    return float((A.masked_attention(q, k, v, allowed, scale) * dout).sum())


def test_finite_differences_with_mask():
    """Central differences of sum(out * dO) against every gradient entry, on
    a mask with an empty row, a fully masked key and a partly masked row."""
    Nq, Nk, d, dv = 5, 7, 3, 2
    q, k, v, dout = _rand((Nq, d), 1), _rand((Nk, d), 2), _rand((Nk, dv), 3), _rand((Nq, dv), 4)
    allowed = _rand((Nq, Nk), 5) > -0.3
    allowed[2] = False            # empty row
    allowed[:, 4] = False         # a key nobody attends
    scale = 0.7
    dq, dk, dvv = BW.masked_attention_grads(q, k, v, dout, allowed, scale)
    h = 1e-6
    for X, G in ((q, dq), (k, dk), (v, dvv)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            old = X[idx]
            X[idx] = old + h
            up = _loss(q, k, v, dout, allowed, scale)
            X[idx] = old - h
            dn = _loss(q, k, v, dout, allowed, scale)
            X[idx] = old
            num[idx] = (up - dn) / (2 * h)
        assert np.max(np.abs(num - G)) < 1e-8
    assert np.all(dq[2] == 0.0)
    assert np.all(dk[4] == 0.0) and np.all(dvv[4] == 0.0)


def test_worked_example():
    """One query, two keys, scale 1, q = 1, k = (0, ln 3), v = (1, 5), dO = 1:
    P = (1/4, 3/4), O = 4, dV = P, dP = v, dS = P * (v - O) = (-3/4, 3/4),
    dq = sum dS k = (3/4) ln 3, dk = dS q."""
    q = np.array([[1.0]])
    k = np.array([[0.0], [math.log(3.0)]])
    v = np.array([[1.0], [5.0]])
    dout = np.array([[1.0]])
    dq, dk, dv = BW.masked_attention_grads(q, k, v, dout, np.ones((1, 2), bool), 1.0)
    assert abs(dq[0, 0] - 0.75 * math.log(3.0)) < 1e-15
    assert np.allclose(dk[:, 0], [-0.75, 0.75], atol=1e-15)
    assert np.allclose(dv[:, 0], [0.25, 0.75], atol=1e-15)
    assert abs(BW.row_lse(q, k, np.ones((1, 2), bool), 1.0)[0] - math.log(4.0)) < 1e-15


def test_dense_equals_torch_autograd():
    """No mask: torch's float64 autograd through its attention routine."""
    Nq, Nk, d = 33, 41, 16
    q, k, v, dout = _rand((Nq, d), 6), _rand((Nk, d), 7), _rand((Nk, d), 8), _rand((Nq, d), 9)
    scale = 1.0 / math.sqrt(d)
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None], scale=scale)[0, 0]
    out.backward(torch.from_numpy(dout))
    dq, dk, dv = BW.masked_attention_grads(q, k, v, dout, np.ones((Nq, Nk), bool), scale)
    assert np.max(np.abs(dq - tq.grad.numpy())) < 1e-12
    assert np.max(np.abs(dk - tk.grad.numpy())) < 1e-12
    assert np.max(np.abs(dv - tv.grad.numpy())) < 1e-12


def test_causal_equals_torch_autograd():
    Nq = Nk = 29
    d = 8
    q, k, v, dout = _rand((Nq, d), 16), _rand((Nk, d), 17), _rand((Nk, d), 18), _rand((Nq, d), 19)
    scale = 0.4
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_(True) for x in (q, k, v))
    out = F.scaled_dot_product_attention(tq[None, None], tk[None, None], tv[None, None], scale=scale,
                                         is_causal=True)[0, 0]
    out.backward(torch.from_numpy(dout))
    causal = np.tril(np.ones((Nq, Nk), bool))
    dq, dk, dv = BW.masked_attention_grads(q, k, v, dout, causal, scale)
    for ours, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(ours - ref.numpy())) < 1e-12


def test_gradient_identities():
    """Softmax rows sum to one, so sum_j dS_ij = 0: dK sums to zero over the
    keys; dV sums to the sum of dO over rows that attend anything."""
    Nq, Nk, d = 20, 30, 6
    q, k, v, dout = _rand((Nq, d), 10), _rand((Nk, d), 11), _rand((Nk, d), 12), _rand((Nq, d), 13)
    allowed = _rand((Nq, Nk), 14) > 0.5
    allowed[7] = False
    dq, dk, dv = BW.masked_attention_grads(q, k, v, dout, allowed, 0.3)
    assert np.max(np.abs(dk.sum(axis=0))) < 1e-12
    has = allowed.any(axis=1)
    assert np.max(np.abs(dv.sum(axis=0) - dout[has].sum(axis=0))) < 1e-12


def test_gqa_sums_query_heads_and_block_mask():
    """Over [B, N, H, d]: a K/V head's gradient is the sum over its query
    heads of the single-head gradient; a block-sparse token mask leaves
    keys of blocks no tile keeps without gradient."""
    B, N, Hq, Hkv, d = 2, 96, 4, 2, 8
    q, dout = _rand((B, N, Hq, d), 20), _rand((B, N, Hq, d), 21)
    k, v = _rand((B, N, Hkv, d), 22), _rand((B, N, Hkv, d), 23)
    tm = np.array([[True, False, False], [True, True, False], [False, False, False]])  # tiles of 32 x 32
    mask = M.expand_token_mask(tm, N, N, 32, 32, N, False)
    dq, dk, dv = BW.prefill_grads(q, k, v, dout, mask, 0.35)
    for b in range(B):
        for g in range(Hkv):
            sk = sum(BW.masked_attention_grads(q[b, :, h], k[b, :, g], v[b, :, g], dout[b, :, h], mask, 0.35)[1]
                     for h in (2 * g, 2 * g + 1))
            assert np.max(np.abs(sk - dk[b, :, g])) < 1e-12
    assert np.all(dk[:, 64:] == 0.0) and np.all(dv[:, 64:] == 0.0)     # key tile 2: no query tile keeps it
    assert np.all(dq[:, 64:] == 0.0)                                    # query tile 2 keeps nothing
    lse = BW.prefill_lse(q, k, mask, 0.35)
    assert np.all(np.isneginf(lse[:, :, 64:]))
    s = 0.35 * q[1, 40, 3] @ k[1, :64, 1].T
    assert abs(lse[1, 3, 40] - np.log(np.exp(s).sum())) < 1e-12
