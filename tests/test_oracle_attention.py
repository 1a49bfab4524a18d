"""Pins for the float64 attention oracle (CPU only).

Each test ties the oracle to something other than itself: torch's float64
scaled_dot_product_attention (a library routine), closed forms computed by
hand, brute force, identities of the online softmax, or the error bound that
follows from the BLASST pruning condition (notes, section 3.1.1).
"""

import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attention as A
from oracle import masks as M
from workloads import get_config, gen_prefill_inputs, gen_decode_sequence
from workloads.configs import DecodeWorkload, PrefillWorkload, MaskSpec, Segment, SEG_BLOCKWIN


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


def _sdpa(q, k, v, **kw):
    """torch fp64 SDPA on [H, N, d] numpy arrays."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None]
    return F.scaled_dot_product_attention(t(q), t(k), t(v), **kw)[0].numpy()


# ---- C-P1: dense special case equals the library routine -------------------

def test_dense_equals_sdpa():
    q, k, v = _rand((40, 16), 0), _rand((56, 16), 1), _rand((56, 8), 2)
    scale = 1 / math.sqrt(16)
    ours = A.masked_attention(q, k, v, np.ones((40, 56), bool), scale)
    ref = _sdpa(q[None], k[None], v[None], scale=scale)[0]
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_causal_equals_sdpa():
    n, d = 70, 32
    q, k, v = _rand((n, d), 3), _rand((n, d), 4), _rand((n, d), 5)
    allowed = np.tril(np.ones((n, n), bool))
    ours = A.masked_attention(q, k, v, allowed, 0.2)
    ref = _sdpa(q[None], k[None], v[None], is_causal=True, scale=0.2)[0]
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_boolean_mask_equals_sdpa():
    n, d = 48, 16
    q, k, v = _rand((n, d), 6), _rand((n, d), 7), _rand((n, d), 8)
    allowed = _rand((n, n), 9) > 0.3
    allowed[np.arange(n), np.arange(n)] = True          # SDPA returns NaN for empty rows
    ours = A.masked_attention(q, k, v, allowed, 0.25)
    ref = _sdpa(q[None], k[None], v[None], attn_mask=torch.from_numpy(allowed)[None], scale=0.25)[0]
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_gqa_mapping_equals_sdpa_enable_gqa():
    """Head h must read K/V head h // (Hq/Hkv): compared with SDPA's own GQA grouping."""
    B, N, Hq, Hkv, d = 1, 64, 8, 2, 16
    q = torch.from_numpy(_rand((B, N, Hq, d), 10))
    k = torch.from_numpy(_rand((B, N, Hkv, d), 11))
    v = torch.from_numpy(_rand((B, N, Hkv, d), 12))
    ref = F.scaled_dot_product_attention(q.transpose(1, 2), k.transpose(1, 2), v.transpose(1, 2),
                                         is_causal=True, enable_gqa=True).transpose(1, 2)
    for h in range(Hq):
        for t in range(2):
            rows, out, blocks, skip, _ = A.prefill_tile(q, k, v, 0, h, t, Br=32, Bc=16,
                                                        scale=1 / 4, causal=True, lam=0.0, n_valid=N)
            assert np.max(np.abs(out - ref[0, rows, h].numpy())) < 1e-12


def test_empty_rows_are_zero():
    q, k, v = _rand((4, 8), 13), _rand((6, 8), 14), _rand((6, 8), 15)
    allowed = np.zeros((4, 6), bool)
    allowed[1, 2] = True
    out = A.masked_attention(q, k, v, allowed, 1.0)
    assert np.all(out[[0, 2, 3]] == 0.0)
    assert np.allclose(out[1], v[2], atol=1e-15)


# ---- C-P2: rows of P sum to one ------------------------------------------

def test_probability_rows_sum_to_one():
    q, k, v = _rand((33, 8), 16, 3.0), _rand((77, 8), 17, 3.0), _rand((77, 8), 18)
    allowed = _rand((33, 77), 19) > -0.5
    _, P = A.masked_attention(q, k, v, allowed, 0.5, return_probs=True)
    has = allowed.any(1)
    assert np.max(np.abs(P[has].sum(1) - 1.0)) < 1e-12
    assert np.all(P[~allowed] == 0.0)


# ---- C-P3: diagonal-only block mask = independent per-block attention --------

def test_diagonal_block_mask_equals_per_block_attention():
    n, d, Bs = 96, 16, 32
    spec = MaskSpec(n_valid=n, segments=(Segment(SEG_BLOCKWIN, 0, n, unit=Bs, radius=0),))
    tm = M.tile_mask(spec, n, n, Bs, Bs)
    assert np.array_equal(tm, np.eye(n // Bs, dtype=bool))
    q, k, v = _rand((1, n, 1, d), 20), _rand((1, n, 1, d), 21), _rand((1, n, 1, d), 22)
    rp, ci = M.csr_from_tile_mask(tm)
    for t in range(n // Bs):
        rows, out, *_ = A.prefill_tile(q, k, v, 0, 0, t, Br=Bs, Bc=Bs, scale=0.25, causal=False,
                                       lam=0.0, n_valid=n, row_ptr=rp, col_idx=ci)
        sl = slice(t * Bs, (t + 1) * Bs)
        ref = _sdpa(q[0, sl, 0][None], k[0, sl, 0][None], v[0, sl, 0][None], scale=0.25)[0]
        assert np.max(np.abs(out - ref)) < 1e-12


# ---- C-P4: Algorithm 1 at lambda = 0 equals the two-pass masked softmax -------

@pytest.mark.parametrize("causal", [False, True])
def test_alg1_lambda0_equals_two_pass(causal):
    N, d, Br, Bc = 200, 16, 64, 32            # ragged tail: 200 = 3*64 + 8
    q, k, v = _rand((1, N, 2, d), 23, 2.0), _rand((1, N, 1, d), 24, 2.0), _rand((1, N, 1, d), 25)
    spec = MaskSpec(n_valid=190, segments=(Segment(SEG_BLOCKWIN, 0, 190, unit=32, radius=2),))
    tm = M.tile_mask(spec, N, N, Br, Bc)
    rp, ci = M.csr_from_tile_mask(tm)
    for h in range(2):
        for t in range(-(-N // Br)):
            kw = dict(Br=Br, Bc=Bc, scale=0.3, causal=causal, lam=0.0, n_valid=190, row_ptr=rp, col_idx=ci)
            _, o1, _, skip, _ = A.prefill_tile(q, k, v, 0, h, t, **kw)
            _, o2, *_ = A.prefill_tile(q, k, v, 0, h, t, method="two_pass", **kw)
            assert not skip.any()
            assert np.max(np.abs(o1 - o2)) < 1e-12
    # and the expanded token mask gives the same output through the plain definition
    Mtok = M.expand_token_mask(tm, N, N, Br, Bc, 190, causal)
    ref = A.masked_attention(q[0, :, 0], k[0, :, 0], v[0, :, 0], Mtok, 0.3)
    for t in range(-(-N // Br)):
        rows, o1, *_ = A.prefill_tile(q, k, v, 0, 0, t, Br=Br, Bc=Bc, scale=0.3, causal=causal,
                                      lam=0.0, n_valid=190, row_ptr=rp, col_idx=ci)
        assert np.max(np.abs(o1 - ref[rows])) < 1e-12


# ---- closed-form worked example of the skip rule ---------------------------

def test_skip_rule_closed_form_example():
    """Keys of block j all equal (a_j, 0); q = (1, 0); scale 1; lambda = e^-2.
    Running max / decision by hand: a = [0, -10, 1, -0.5, -1.01, 3]
      block0 keep (first), block1 -10-0 < -2 skip, block2 keep (max->1),
      block3 -1.5 > -2 keep, block4 -2.01 < -2 skip, block5 keep (max->3).
    Output = sum_kept Bc e^{a_j} v_j / sum_kept Bc e^{a_j}."""
    Bc, lam = 4, math.exp(-2.0)
    a = np.array([0.0, -10.0, 1.0, -0.5, -1.01, 3.0])
    k = np.zeros((len(a) * Bc, 2))
    k[:, 0] = np.repeat(a, Bc)
    vrow = np.arange(len(a), dtype=float) * 10.0 + 1.0
    v = np.repeat(vrow, Bc)[:, None]
    q = np.array([[1.0, 0.0]])
    rows = np.array([len(a) * Bc - 1])
    out, skip, margin = A.blasst_tile(q, k, v, rows, np.arange(len(a)), Bc, 1.0, lam, 10 ** 9, False)
    assert skip.tolist() == [False, True, False, False, True, False]
    kept = ~skip
    w = np.exp(a[kept])
    assert abs(out[0, 0] - (w * vrow[kept]).sum() / w.sum()) < 1e-12
    assert abs(margin[1] - (-10.0 + 2.0)) < 1e-12 and abs(margin[4] - (-2.01 + 2.0)) < 1e-12
    # decode oracle on the same data (G = 1) agrees, both forms
    for meth in ("loop", "closed_form"):
        o2, s2, _ = A.decode_group(q, k, v, Bc, 1.0, lam, meth)
        assert s2.tolist() == skip.tolist()
        assert abs(o2[0, 0] - out[0, 0]) < 1e-12


# ---- C-P5: sequential loop skip set = cumulative-max closed form ------------

def _concentrated_case(L=1024, Hq=4, Hkv=1, d=32):
    cfg = PrefillWorkload(name="t", description="", dtype="bf16", B=1, Hq=Hq, Hkv=Hkv, N=L, d=d,
                          Br=64, Bc=32, causal=True, lam=0.0, mask=None, seed=77, generator="concentrated")
    return cfg, gen_prefill_inputs(cfg)


@pytest.mark.parametrize("lam", [1e-4, 1e-2, 0.1, 0.4, 0.9])
def test_skip_loop_equals_cummax_form(lam):
    cfg, (q, k, v) = _concentrated_case()
    n = cfg.N
    for h in (0, 3):
        for t in (0, 5, 15):
            rows, out, blocks, skip, margin = A.prefill_tile(q, k, v, 0, h, t, Br=64, Bc=32,
                                                             scale=cfg.scale, causal=True, lam=lam, n_valid=n)
            qr = A.as_f64(q[0, rows[0]:rows[-1] + 1, h])
            s2, _ = A.skip_set_vectorized(qr, A.as_f64(k[0, :, 0]), rows, blocks, 32, cfg.scale, lam, n, True)
            assert np.array_equal(skip, s2)


# ---- C-P6: monotone in lambda, first block never skipped --------------------

def _row_agree_brute(qr, k, rows, blocks, Bc, scale, lam, n_valid, causal):
    """Per-row skip condition by plain loops over rows, blocks and keys."""
    cnt = []
    run = [-math.inf] * len(rows)
    for j in blocks:
        c = 0
        for a, r in enumerate(rows):
            best = -math.inf
            for key in range(j * Bc, min((j + 1) * Bc, k.shape[0])):
                if key < n_valid and (not causal or key <= r):
                    best = max(best, scale * float(np.dot(qr[a], k[key])))
            run[a] = max(run[a], best)
            if best == -math.inf or best - run[a] < math.log(lam):
                c += 1
        cnt.append(c)
    return cnt


@pytest.mark.parametrize("lam", [0.05, 0.4, 0.9])
def test_row_agreement_brute_force_and_invariants(lam):
    cfg, (q, k, v) = _concentrated_case(L=160, Hq=2, Hkv=1, d=16)
    for h in range(2):
        for t in range(3):
            rows = A.tile_rows(t, 64, 160)
            blocks = A.visited_blocks(t, 64, 32, 160, 160, True)
            qr = A.as_f64(q[0, rows[0]:rows[-1] + 1, h])
            kk = A.as_f64(k[0, :, 0])
            agree, gaps = A.row_agreement(qr, kk, rows, blocks, 32, 0.25, lam, 160, True)
            assert agree.tolist() == _row_agree_brute(qr, kk, rows, blocks, 32, 0.25, lam, 160, True)
            _, skip, _ = A.blasst_tile(qr, kk, A.as_f64(v[0, :, 0]), rows, blocks, 32, 0.25, lam, 160, True)
            assert all(agree[skip] == len(rows))            # a skipped block: every row agrees
            assert all(agree[~skip] < len(rows))            # a kept block: some row disagrees
            assert agree[0] == np.count_nonzero(~np.isfinite(gaps[:, 0]))   # first block: gap 0 for live rows
    # lambda -> 0+: only rows with no allowed key in the block agree; lambda = 0 counts nothing
    agree, gaps = A.row_agreement(qr, kk, rows, blocks, 32, 0.25, 1e-300, 160, True)
    assert agree.tolist() == np.count_nonzero(~np.isfinite(gaps), axis=0).tolist()
    assert A.row_agreement(qr, kk, rows, blocks, 32, 0.25, 0.0, 160, True)[0].sum() == 0


def _block_const_keys(a, Bc=4):
    """Keys whose scores against q = (1, 0) equal a[j] on every key of block j."""
    k = np.zeros((len(a) * Bc, 2))
    k[:, 0] = np.repeat(np.asarray(a, dtype=float), Bc)
    v = np.repeat(np.arange(len(a), dtype=float) * 10.0 + 1.0, Bc)[:, None]
    return np.array([[1.0, 0.0]]), k, v


def test_descending_order_worked_example():
    # block maxima 5, 0, 3, -2, 4, 1 and ln(lambda) = -2 (scale 1):
    # ascending running max 5 everywhere -> gaps 0 -5 -2 -7 -1 -4 -> skip {1, 3, 5};
    # descending visits 1, 4, -2, 3, 0, 5 with running max 1 4 4 4 4 5 -> gaps (by block)
    # 0 -4 -1 -6 0 0 -> skip {1, 3}
    a = [5.0, 0.0, 3.0, -2.0, 4.0, 1.0]
    q, k, v = _block_const_keys(a)
    lam = math.exp(-2.0)
    for meth in ("loop", "closed_form"):
        _, s_up, _ = A.decode_group(q, k, v, 4, 1.0, lam, meth)
        _, s_dn, _ = A.decode_group(q, k, v, 4, 1.0, lam, meth, order="descending")
        assert np.nonzero(s_up)[0].tolist() == [1, 3, 5], meth
        assert np.nonzero(s_dn)[0].tolist() == [1, 3], meth


def test_descending_order_mirror_symmetry_and_forms():
    """Reversing the key blocks and visiting in descending order is ascending
    order on the original blocks: the skip sets mirror.  The literal loop and
    the closed form agree in descending order; at lambda = 0 the order does
    not change the output."""
    cfg = DecodeWorkload(name="o", description="", B=1, Hq=4, Hkv=1, L=64 * 24, d=32, Bc=64, lam=0.0, seed=31)
    q, k, v = gen_decode_sequence(cfg, 0)
    q, k, v = A.as_f64(q), A.as_f64(k)[:, 0], A.as_f64(v)[:, 0]
    L, Bc = k.shape[0], 64
    perm = np.concatenate([np.arange(j * Bc, (j + 1) * Bc) for j in range(L // Bc)[::-1]])
    for lam in (1e-3, 0.02, 0.2):
        _, s_up, _ = A.decode_group(q, k, v, Bc, cfg.scale, lam, "closed_form")
        _, s_mir, _ = A.decode_group(q, k[perm], v[perm], Bc, cfg.scale, lam, "closed_form", order="descending")
        assert np.array_equal(s_mir[::-1], s_up)
        o_l, s_l, _ = A.decode_group(q, k, v, Bc, cfg.scale, lam, "loop", order="descending")
        o_c, s_c, _ = A.decode_group(q, k, v, Bc, cfg.scale, lam, "closed_form", order="descending")
        assert np.array_equal(s_l, s_c) and np.max(np.abs(o_l - o_c)) < 1e-12
    o_up, _, _ = A.decode_group(q, k, v, Bc, cfg.scale, 0.0, "loop")
    o_dn, _, _ = A.decode_group(q, k, v, Bc, cfg.scale, 0.0, "loop", order="descending")
    assert np.max(np.abs(o_up - o_dn)) < 1e-12
    # prefill tile, causal: descending visits the diagonal block first
    pc, (qq, kk, vv) = _concentrated_case(L=256, Hq=2, Hkv=1, d=16)
    blocks_dn = A.visited_blocks(3, 64, 32, 256, 256, True, order="descending")
    assert blocks_dn.tolist() == list(range(7, -1, -1))
    for lam in (0.05, 0.3):
        _, _, b_dn, s_dn, _ = A.prefill_tile(qq, kk, vv, 0, 0, 3, Br=64, Bc=32, scale=0.25, causal=True, lam=lam,
                                             n_valid=256, order="descending")
        rows = A.tile_rows(3, 64, 256)
        sv, _ = A.skip_set_vectorized(A.as_f64(qq[0, rows[0]:rows[-1] + 1, 0]), A.as_f64(kk[0, :, 0]), rows, b_dn,
                                      32, 0.25, lam, 256, True)
        assert np.array_equal(s_dn, sv)


def test_per_split_reset_variant():
    """The per-split variant restarts the running max at every split: worked
    example by hand, equal to the exact rule when one split holds all blocks,
    and equal to running each split as its own sequence."""
    a = [5.0, 0.0, 3.0, -2.0, 4.0, 1.0]
    q, k, v = _block_const_keys(a)
    lam = math.exp(-2.0)
    # splits of 2 blocks: (5, 0) (3, -2) (4, 1) -> gaps 0 -5 | 0 -5 | 0 -3 -> skip {1, 3, 5}
    _, s2, _ = A.decode_group(q, k, v, 4, 1.0, lam, "closed_form", split_blocks=2)
    assert np.nonzero(s2)[0].tolist() == [1, 3, 5]
    # splits of 3 blocks: (5, 0, 3) (-2, 4, 1) -> gaps 0 -5 -2 | 0 0 -3 -> skip {1, 5}
    _, s3, _ = A.decode_group(q, k, v, 4, 1.0, lam, "closed_form", split_blocks=3)
    assert np.nonzero(s3)[0].tolist() == [1, 5]
    cfg = DecodeWorkload(name="o", description="", B=1, Hq=4, Hkv=1, L=64 * 20, d=32, Bc=64, lam=0.0, seed=33)
    qq, kk, vv = gen_decode_sequence(cfg, 0)
    qq, kk, vv = A.as_f64(qq), A.as_f64(kk)[:, 0], A.as_f64(vv)[:, 0]
    for lam in (1e-3, 0.05):
        _, exact, _ = A.decode_group(qq, kk, vv, 64, cfg.scale, lam, "closed_form")
        _, whole, _ = A.decode_group(qq, kk, vv, 64, cfg.scale, lam, "closed_form", split_blocks=20)
        assert np.array_equal(exact, whole)
        _, per, _ = A.decode_group(qq, kk, vv, 64, cfg.scale, lam, "closed_form", split_blocks=8)
        parts = [A.decode_group(qq, kk[a * 64:(a + 8) * 64], vv[a * 64:(a + 8) * 64], 64, cfg.scale, lam,
                                "closed_form")[1] for a in (0, 8, 16)]
        assert np.array_equal(per, np.concatenate(parts))


def test_per_head_decision_variant():
    """Per-head decisions: the loop (a tile of one row per head) equals the
    closed form; the group's skip set is the intersection of the heads' skip
    sets (same running max per row, the vote only ANDs); with one head per
    group the two variants coincide; a hand-built case where heads differ."""
    cfg = DecodeWorkload(name="o", description="", B=1, Hq=8, Hkv=2, L=64 * 9 + 17, d=32, Bc=64, lam=0.0, seed=41)
    q, k, v = gen_decode_sequence(cfg, 0)
    for lam in (1e-3, 0.02, 0.2):
        for order in ("ascending", "descending"):
            o1, s1, m1 = A.decode_sequence(q, k, v, 64, cfg.scale, lam, "loop", order=order, decisions="head")
            o2, s2, m2 = A.decode_sequence(q, k, v, 64, cfg.scale, lam, "closed_form", order=order,
                                           decisions="head")
            assert s1.shape == (8, 10)
            assert np.array_equal(s1, s2)
            assert np.allclose(m1, m2, atol=1e-12) and np.allclose(o1, o2, atol=1e-12)
            _, sg, _ = A.decode_sequence(q, k, v, 64, cfg.scale, lam, "closed_form", order=order)
            assert np.array_equal(sg, s2.reshape(2, 4, 10).all(axis=1))
    # G = 1: a head is its group
    q1, k1, v1 = q[:2], k, v
    og, sg, _ = A.decode_sequence(q1, k1, v1, 64, cfg.scale, 0.05, "closed_form")
    oh, sh, _ = A.decode_sequence(q1, k1, v1, 64, cfg.scale, 0.05, "closed_form", decisions="head")
    assert np.array_equal(sg, sh) and np.allclose(og, oh, atol=1e-14)
    # two heads, keys with block-constant scores: head 0 sees (5, 0, 3), head 1 sees (0, 5, 3);
    # at ln(lambda) = -2 head 0 skips block 1 only, head 1 skips nothing, the group skips nothing
    qh = np.zeros((2, 2))
    qh[0, 0] = qh[1, 1] = 1.0
    kh = np.zeros((12, 2))
    for j, (a0, a1) in enumerate([(5.0, 0.0), (0.0, 5.0), (3.0, 3.0)]):
        kh[4 * j:4 * j + 4] = (a0, a1)
    vh = np.arange(24, dtype=np.float64).reshape(12, 2)
    lam = math.exp(-2.0)
    oh, sh, mh = A.decode_group(qh, kh, vh, 4, 1.0, lam, "closed_form", decisions="head")
    assert sh.tolist() == [[False, True, False], [False, False, False]]
    assert np.allclose(mh, [[2.0, -3.0, 0.0], [2.0, 2.0, 0.0]])
    _, sgrp, _ = A.decode_group(qh, kh, vh, 4, 1.0, lam, "closed_form")
    assert sgrp.tolist() == [False, False, False]
    # head 0 attends to blocks 0 and 2 only: weights e^5 (4 keys) and e^3 (4 keys)
    w0, w2 = math.exp(5.0), math.exp(3.0)
    want0 = (w0 * vh[0:4].sum(0) + w2 * vh[8:12].sum(0)) / (4 * w0 + 4 * w2)
    assert np.allclose(oh[0], want0, atol=1e-12)


def test_skip_monotone_and_first_block_kept():
    cfg, (q, k, v) = _concentrated_case()
    prev = None
    for lam in (0.0, 1e-6, 1e-3, 0.05, 0.3, 0.7, 0.99):
        sets = []
        for t in (3, 9, 15):
            _, _, blocks, skip, _ = A.prefill_tile(q, k, v, 0, 1, t, Br=64, Bc=32, scale=cfg.scale,
                                                   causal=True, lam=lam, n_valid=cfg.N)
            assert not skip[0]
            sets.append(skip)
        cur = np.concatenate(sets)
        if prev is not None:
            assert np.all(cur >= prev)          # skip(l1) subset of skip(l2) for l1 < l2
        prev = cur
    assert prev.any()                           # lambda close to 1 does skip something


# ---- C-P7: the error bound implied by the pruning condition ------------------

@pytest.mark.parametrize("lam", [1e-3, 0.05, 0.3])
def test_dynamic_error_within_page_bound(lam):
    """Skipped entries satisfy S - M < ln(lambda) with M the row's global max,
    so their weights e^{S-M} are each below lambda.  With eps the exact sum of
    skipped weights and Z >= 1 the dense denominator,
    |O_dyn - O_dense| <= 2 eps max|V| / Z per row and component."""
    cfg, (q, k, v) = _concentrated_case()
    n = cfg.N
    vv = A.as_f64(v[0, :, 0])
    for t in (4, 12, 15):
        rows, out, blocks, skip, _ = A.prefill_tile(q, k, v, 0, 2, t, Br=64, Bc=32, scale=cfg.scale,
                                                    causal=True, lam=lam, n_valid=n)
        qr = A.as_f64(q[0, rows[0]:rows[-1] + 1, 2])
        keys = np.arange(n)
        allowed = keys[None, :] <= rows[:, None]
        dense = A.masked_attention(qr, A.as_f64(k[0, :, 0]), vv, allowed, cfg.scale)
        S = np.where(allowed, cfg.scale * qr @ A.as_f64(k[0, :, 0]).T, -np.inf)
        Mx = S.max(1)
        W = np.exp(S - Mx[:, None])
        skipped_keys = np.zeros(n, bool)
        for j in blocks[skip]:
            skipped_keys[j * 32:(j + 1) * 32] = True
        eps = (W * skipped_keys[None, :]).sum(1)
        Z = W.sum(1)
        assert np.all(W[:, skipped_keys] < lam + 1e-15)
        bound = 2 * eps * np.abs(vv).max() / Z
        err = np.abs(out - dense).max(1)
        assert np.all(err <= bound + 1e-12)


# ---- C-P8: decode equals prefill at one query row -----------------------------

def test_decode_equals_prefill_single_row():
    cfg = DecodeWorkload(name="t", description="", B=1, Hq=4, Hkv=4, L=700, d=32, Bc=64, lam=0.02, seed=9)
    q, k, v = gen_decode_sequence(cfg, 0, L=cfg.L)
    for g in range(4):
        od, sd, _ = A.decode_group(q[g:g + 1], k[:, g], v[:, g], 64, cfg.scale, cfg.lam, "loop")
        rows = np.array([cfg.L - 1])
        op, sp, _ = A.blasst_tile(A.as_f64(q[g:g + 1]), k[:, g], v[:, g], rows, np.arange(11), 64,
                                  cfg.scale, cfg.lam, cfg.L, True)
        assert np.array_equal(sd, sp)
        assert np.max(np.abs(od - op)) < 1e-12


def test_decode_loop_equals_closed_form():
    cfg = DecodeWorkload(name="t", description="", B=1, Hq=8, Hkv=2, L=2000, d=64, Bc=64, lam=40 / 2000, seed=11)
    q, k, v = gen_decode_sequence(cfg, 0)
    o1, s1, m1 = A.decode_sequence(q, k, v, 64, cfg.scale, cfg.lam, "loop")
    o2, s2, m2 = A.decode_sequence(q, k, v, 64, cfg.scale, cfg.lam, "closed_form")
    assert np.array_equal(s1, s2)
    assert s1.any()
    assert np.max(np.abs(o1 - o2)) < 1e-12
    assert np.max(np.abs(m1 - m2)) < 1e-9


# ---- C-P9: merging split partials reproduces the unsplit result ---------------

def test_split_merge_identity():
    L, d = 1000, 16
    q, k, v = _rand((3, d), 30, 2.0), _rand((L, d), 31, 2.0), _rand((L, d), 32)
    kept = _rand((L,), 33) > -0.8
    full = A.masked_attention(q, k, v, np.broadcast_to(kept, (3, L)), 0.3)
    for cuts in ([0, 1000], [0, 10, 1000], [0, 128, 256, 640, 999, 1000], list(range(0, 1001, 64)) + [1000]):
        cuts = sorted(set(cuts))
        parts = [A.partial_state(q, k[a:b], v[a:b], np.broadcast_to(kept[a:b], (3, b - a)), 0.3)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        merged = A.merge_partials([p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts])
        assert np.max(np.abs(merged - full)) < 1e-12


def test_lambda_range_rejected():
    for bad in (-0.1, 1.0, 2.0):
        with pytest.raises(ValueError):
            A.log_threshold(bad)


# ---- the batched closed form equals the per-block loop and Algorithm 1 ------

@pytest.mark.parametrize("causal,n_valid,order", [(False, 300, "ascending"), (True, 300, "ascending"),
                                                  (False, 270, "descending"), (True, 300, "descending")])
def test_skip_set_batched_equals_loop(causal, n_valid, order):
    """skip_set_batched (one product per tile, torch float64) takes the same
    decisions as skip_set_vectorized and the literal Algorithm 1 loop, and its
    margins equal blasst_tile's, on a ragged last block, padding keys, causal
    diagonal tiles, a CSR list and both visiting orders."""
    n, d, Br, Bc = 300, 32, 128, 64
    g = np.random.default_rng(77)
    q = g.standard_normal((n, d))
    k = g.standard_normal((n, d))
    v = g.standard_normal((n, d))
    w = g.standard_normal(d)
    w /= np.linalg.norm(w)
    q += 4.0 * w                                      # a sink: later blocks fall below the threshold
    k[:64] += 12.0 * w
    row_ptr = np.array([0, 3, 4, 9])
    col_idx = np.array([0, 2, 4, 1, 0, 1, 2, 3, 4])
    n_skipped = 0
    for lam in (0.05, 0.3, 0.0):
        for t in range(3):
            for csr in (False, True):
                rows = A.tile_rows(t, Br, n)
                blocks = A.visited_blocks(t, Br, Bc, n, n, causal, *((row_ptr, col_idx) if csr else (None, None)),
                                          order=order)
                qr = q[rows[0]:rows[-1] + 1]
                sk, mg = A.skip_set_batched(qr, k, rows, blocks, Bc, 0.1, lam, n_valid, causal)
                _, sk1, mg1 = A.blasst_tile(qr, k, v, rows, blocks, Bc, 0.1, lam, n_valid, causal)
                assert np.array_equal(sk, sk1)
                assert np.allclose(mg, mg1, rtol=0, atol=1e-12) or np.array_equal(mg, mg1)
                n_skipped += int(sk.sum())
                if lam > 0.0:
                    sk2, _ = A.skip_set_vectorized(qr, k, rows, blocks, Bc, 0.1, lam, n_valid, causal)
                    assert np.array_equal(sk, sk2)
    assert n_skipped > 0 or order == "descending"    # the sink comes first only in ascending order
