"""The C++ block-index builder against the oracle's block mask (host code, CPU only)."""

import numpy as np
import pytest

import block_sparse_attention_flash_amd as bsa
from oracle import masks as M
from workloads import get_config
from workloads.configs import MaskSpec, Segment, SEG_FULL, SEG_BLOCKWIN, SEG_IMAGE2D, SEG_VIDEO3D, \
    dit_image_text_spec, video_text_spec

from test_oracle_masks import SMALL_SPECS


def _csr_equal(spec, n, Br, Bc):
    rp, ci = bsa.build_block_index(spec, n, n, Br, Bc)
    tm = M.tile_mask(spec, n, n, Br, Bc)
    orp, oci = M.csr_from_tile_mask(tm)
    assert np.array_equal(rp, orp)
    assert np.array_equal(ci, oci)
    bsa.validate_block_index(rp, ci, -(-n // Bc))
    return rp, ci


@pytest.mark.parametrize("name", sorted(SMALL_SPECS))
@pytest.mark.parametrize("tiles", [(16, 16), (32, 16), (24, 8), (128, 64), (7, 5)])
def test_small_specs(name, tiles):
    spec = SMALL_SPECS[name]
    _csr_equal(spec, spec.n_valid + 13, *tiles)


def test_cfg1_and_cfg2_full():
    c1 = get_config("cfg1")
    _csr_equal(c1.mask, c1.N, 64, 64)
    c2 = get_config("cfg2")
    rp, ci = _csr_equal(c2.mask, c2.N, 128, 64)
    assert rp[-1] == 640
    rp64, _ = _csr_equal(c2.mask, c2.N, 64, 64)
    assert rp64[-1] == 1160


def test_cfg3_sampled_tiles_and_counts():
    c3 = get_config("cfg3")
    rp, ci = bsa.build_block_index(c3.mask, c3.N, c3.N, 128, 64)
    assert rp[-1] == 13839                   # kept tile-blocks; 97.4% sparse of 515 x 1030
    Tr, Tc = 515, 1030
    assert rp.size == Tr + 1
    bsa.validate_block_index(rp, ci, Tc)
    rng = np.random.default_rng(0)
    tiles = sorted(set([0, 1, 31, 32, 33, 255, 511, 512, 513, 514] + list(rng.integers(0, Tr, 12))))
    ref = M.tile_mask_rows(c3.mask, c3.N, c3.N, 128, 64, tiles)
    for a, t in enumerate(tiles):
        assert np.array_equal(ci[rp[t]:rp[t + 1]], np.nonzero(ref[a])[0]), t
    assert rp[513] - rp[512] == 1029         # the anchor tile sees every valid block
    assert not (ci == 1029).any()            # the all-padding key block is never kept


def test_random_specs_against_oracle():
    rng = np.random.default_rng(5)
    for trial in range(25):
        W = int(rng.integers(3, 9))
        H = int(rng.integers(2, 6))
        F = int(rng.integers(1, 4))
        text = int(rng.integers(1, 30))
        nv = F * H * W + text
        segs = (Segment(SEG_VIDEO3D, 0, F * H * W, frames=F, grid_h=H, grid_w=W, radius=int(rng.integers(0, 3)),
                        t_radius=int(rng.integers(0, 3)), unit=int(rng.integers(1, W * H + 1))),
                Segment(SEG_FULL, F * H * W, text))
        na = int(rng.integers(0, 4))
        spec = MaskSpec(n_valid=nv, segments=segs, anchor_start=F * H * W, anchor_len=min(na, text))
        n = nv + int(rng.integers(0, 20))
        Br, Bc = int(rng.integers(1, 20)), int(rng.integers(1, 20))
        _csr_equal(spec, n, Br, Bc)


def test_capacity_and_spec_errors():
    c1 = get_config("cfg1")
    lib = bsa.library()
    import ctypes as C
    from block_sparse_attention_flash_amd import _abi
    cs, keep = bsa._c_spec(c1.mask)
    rp = np.zeros(9, np.int32)
    ci = np.zeros(4, np.int32)
    nnz = C.c_int64(0)
    st = lib.bsattn_build_block_index(C.byref(cs), 512, 512, 64, 64, rp.ctypes.data, ci.ctypes.data, 4, C.byref(nnz))
    assert st == _abi.BSATTN_ERR_CAPACITY and nnz.value == 22
    bad = [
        MaskSpec(n_valid=600, segments=c1.mask.segments),                                  # n_valid > n_k
        MaskSpec(n_valid=512, segments=(Segment(SEG_FULL, 0, 300), Segment(SEG_FULL, 200, 100))),  # overlap
        MaskSpec(n_valid=512, segments=(Segment(SEG_IMAGE2D, 0, 100, grid_h=8, grid_w=8),)),       # 100 != 64
        MaskSpec(n_valid=512, segments=(Segment(9, 0, 10),)),                              # unknown kind
        MaskSpec(n_valid=512, segments=(Segment(SEG_BLOCKWIN, 0, 10, unit=0),)),           # unit 0
        MaskSpec(n_valid=512, segments=(), anchor_start=500, anchor_len=20),               # anchors past n_valid
    ]
    for spec in bad:
        with pytest.raises(bsa.BsattnError) as e:
            bsa.build_block_index(spec, 512, 512, 64, 64)
        assert e.value.status == _abi.BSATTN_ERR_INVALID_ARG


def test_validate_rejects_malformed_csr():
    ok_rp = np.array([0, 2, 3], np.int32)
    ok_ci = np.array([0, 3, 1], np.int32)
    bsa.validate_block_index(ok_rp, ok_ci, 4)
    cases = [
        (np.array([1, 2, 3], np.int32), ok_ci),        # row_ptr[0] != 0
        (np.array([0, 2, 1], np.int32), ok_ci),        # decreasing
        (ok_rp, np.array([0, 4, 1], np.int32)),        # out of range
        (ok_rp, np.array([3, 0, 1], np.int32)),        # not ascending
        (ok_rp, np.array([0, 0, 1], np.int32)),        # duplicate
    ]
    for rp, ci in cases:
        with pytest.raises(bsa.BsattnError):
            bsa.validate_block_index(rp, ci, 4)


def test_tile_order_lpt():
    rp = np.array([0, 2, 7, 8, 13, 13], np.int32)   # counts 2, 5, 1, 5, 0
    assert bsa.tile_order_lpt(rp).tolist() == [1, 3, 0, 2, 4]


def test_schedule_covers_every_entry_once():
    c3 = get_config("cfg3")
    rp, ci = bsa.build_block_index(c3.mask, c3.N, c3.N, 128, 64)
    for mx in (1, 7, 64, 5000):
        sc = bsa.build_schedule(rp, mx)
        seen = np.zeros(rp[-1], np.int32)
        tiles_direct = set()
        lens = []
        assert sc.items.shape[1] == 5
        for t, a, b, slot, m in sc.items:
            assert rp[t] <= a <= b <= rp[t + 1]
            assert b - a <= mx
            seen[a:b] += 1
            lens.append(b - a)
            assert (slot < 0) == (m < 0)
            if slot < 0:
                tiles_direct.add(int(t))
            else:                                                  # the item's merge owns its slot
                mt, s0, n = sc.merges[m]
                assert mt == t and s0 <= slot < s0 + n
        assert (seen == 1).all()
        assert lens == sorted(lens, reverse=True)                  # longest first
        cut = {int(t) for t, s0, n in sc.merges}
        assert cut.isdisjoint(tiles_direct) and len(cut | tiles_direct) == 515
        slots = sorted(int(s) for s in sc.items[:, 3] if s >= 0)
        assert slots == list(range(sc.n_slots))
        for t, s0, n in sc.merges:                                 # slots of a cut tile are consecutive
            assert sorted(int(s) for tt, a, b, s, m in sc.items if tt == t) == list(range(s0, s0 + n))
    assert bsa.build_schedule(rp, 5000).n_slots == 0


def test_schedule_tile_order():
    c3 = get_config("cfg3")
    rp, _ = bsa.build_block_index(c3.mask, c3.N, c3.N, 128, 64)
    lpt = bsa.build_schedule(rp, 64)
    tile = bsa.build_schedule(rp, 64, order="tile")
    assert tile.n_slots == lpt.n_slots and np.array_equal(tile.merges, lpt.merges)
    # the same items, each with its fields
    key = lambda a: sorted(map(tuple, a.tolist()))
    assert key(tile.items) == key(lpt.items)
    chunk = tile.items[:, 3] >= 0
    k = int(chunk.sum())
    assert k > 0 and chunk[:k].all() and not chunk[k:].any()            # chunks first
    assert np.array_equal(tile.items[:k], lpt.items[lpt.items[:, 3] >= 0])  # in their longest-first order
    assert (np.diff(tile.items[k:, 0]) > 0).all()                        # whole tiles ascending
    with pytest.raises(ValueError):
        bsa.build_schedule(rp, 64, order="random")
    bad = np.array([[0, 0, 1, 0, -1]], np.int32)                         # a slot without a merge
    assert bsa.library().bsattn_schedule_tile_order(bad.ctypes.data, 1) != 0


def test_prefill_group_major():
    c2, c3 = get_config("cfg2"), get_config("cfg3")
    rp2, _ = bsa.build_block_index(c2.mask, c2.N, c2.N, 128, 64)
    rp3, _ = bsa.build_block_index(c3.mask, c3.N, c3.N, 128, 64)
    s2 = bsa.default_schedule(rp2, c2.B, c2.Hq, c2.Hkv, c2.d)
    s3 = bsa.default_schedule(rp3, c3.B, c3.Hq, c3.Hkv, c3.d)
    # multimodal DiT image+text: too few work-groups per XCD, rank by rank, longest first
    assert not bsa.prefill_group_major(c2.B, c2.Hq, c2.Hkv, c2.d, s2.n_items)
    lens = (s2.items[:, 2] - s2.items[:, 1]).tolist()
    assert lens == sorted(lens, reverse=True)
    # video DiT: many waves of work-groups per XCD, group by group, tile order
    assert bsa.prefill_group_major(c3.B, c3.Hq, c3.Hkv, c3.d, s3.n_items)
    k = int((s3.items[:, 3] >= 0).sum())
    assert (np.diff(s3.items[k:, 0]) > 0).all()
    # groups that do not divide into the 8 XCDs, and the threshold: 4 waves of 2 or 3 resident work-groups
    assert not bsa.prefill_group_major(1, 12, 12, 128, 10000)
    assert bsa.prefill_group_major(1, 8, 8, 128, 256) and not bsa.prefill_group_major(1, 8, 8, 128, 255)
    assert bsa.prefill_group_major(1, 8, 8, 64, 384) and not bsa.prefill_group_major(1, 8, 8, 64, 383)
    with pytest.raises(ValueError):
        bsa.prefill_group_major(1, 8, 3, 128, 10)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("G", [1, 3])
def test_dkdv_schedule_covers_every_position_once(d, G):
    c3 = get_config("cfg3")
    rp, ci = bsa.build_block_index(c3.mask, c3.N, c3.N, 128, 64)
    Tc = c3.N // 64
    cp, ri = bsa.transpose_block_index(rp, ci, Tc)
    NB = 1 if d == 64 else 2
    for mx in (7, 100, 1 << 30):
        sc = bsa.build_dkdv_schedule(cp, ri, G, d, mx)
        assert sc.items.shape[1] == 8
        lens = (sc.items[:, 2] - sc.items[:, 1]).tolist()
        assert lens == sorted(lens, reverse=True)                      # longest first
        by_group = {}
        for it in sc.items.tolist():
            by_group.setdefault(it[0], []).append(it)
        assert sorted(by_group) == list(range(-(-Tc // NB)))           # every group has an item
        slots = []
        for m, its in by_group.items():
            lists = [ri[cp[j]:cp[j + 1]].tolist() for j in range(NB * m, min(NB * m + NB, Tc))]
            uni = sorted(set().union(*map(set, lists)))
            P = G * len(uni)
            its.sort(key=lambda x: x[1])
            assert its[0][1] == 0 and its[-1][2] == P                  # the positions, partitioned
            assert all(a[2] == b[1] for a, b in zip(its, its[1:]))
            assert all(x[2] - x[1] <= mx for x in its)
            if len(its) == 1 and its[0][6] < 0:
                continue
            for m_, p0, p1, hc, i0, i1, slot, mrg in its:                # chunks: the cursor at p0
                t0 = uni[p0 % len(uni)]
                assert hc == p0 // len(uni)
                assert i0 == sum(1 for t in lists[0] if t < t0)
                assert i1 == (sum(1 for t in lists[1] if t < t0) if len(lists) > 1 else 0)
                mt, s0, n = sc.merges[mrg]
                assert mt == m and s0 <= slot < s0 + n and n == len(its)
                slots.append(slot)
        assert sorted(slots) == list(range(sc.n_slots))
    assert bsa.build_dkdv_schedule(cp, ri, G, d, 1 << 30).n_slots == 0


def test_dkdv_schedule_validation():
    cp = np.array([0, 2, 3], np.int32)
    with pytest.raises(bsa.BsattnError):
        bsa.build_dkdv_schedule(cp, np.array([1, 0, 0], np.int32), 1, 128, 4)   # list not ascending
    with pytest.raises(bsa.BsattnError):
        bsa.build_dkdv_schedule(np.array([0, 2, 1], np.int32), np.array([0, 1], np.int32), 1, 128, 4)
    with pytest.raises(bsa.BsattnError):
        bsa.build_dkdv_schedule(cp, np.array([0, 1, 0], np.int32), 1, 96, 4)    # head dim
    with pytest.raises(bsa.BsattnError):
        bsa.build_dkdv_schedule(cp, np.array([0, 1, 0], np.int32), 1, 64, 0)    # max positions < 1
    sc = bsa.build_dkdv_schedule(np.array([0, 0, 0], np.int32), np.zeros(0, np.int32), 2, 64, 4)
    assert sc.items.tolist() == [[0, 0, 0, 0, 0, 0, -1, -1], [1, 0, 0, 0, 0, 0, -1, -1]]  # empty blocks: zeros


def test_schedule_validation():
    import ctypes as C
    from block_sparse_attention_flash_amd import _abi
    from test_abi import _good_prefill
    with pytest.raises(bsa.BsattnError):
        bsa.build_schedule(np.array([0, 3, 1], np.int32), 4)          # decreasing row_ptr
    with pytest.raises(bsa.BsattnError):
        bsa.build_schedule(np.array([0, 3], np.int32), 0)             # max_blocks < 1
    lib = bsa.library()
    a = _good_prefill()
    a.sched_items, a.n_items = 0x20000, 4
    st = lib.bsattn_prefill_fwd(C.byref(a), None)
    assert st == _abi.BSATTN_ERR_INVALID_ARG                         # schedule without CSR
    a.row_ptr = a.col_idx = 0x30000
    a.sched_merges, a.n_merges, a.n_slots = 0x40000, 1, 2
    a.lam = 0.1                                                    # cut tiles + BLASST: accepted,
    assert lib.bsattn_prefill_fwd(C.byref(a), None) == _abi.BSATTN_ERR_INVALID_ARG   # needs its workspace
    a.workspace, a.workspace_bytes = 0x50000, 16
    assert lib.bsattn_prefill_fwd(C.byref(a), None) == _abi.BSATTN_ERR_CAPACITY
    a.lam = 0.0
    assert lib.bsattn_prefill_fwd(C.byref(a), None) == _abi.BSATTN_ERR_CAPACITY
    a.n_merges = 0
    assert lib.bsattn_prefill_fwd(C.byref(a), None) == _abi.BSATTN_ERR_INVALID_ARG   # inconsistent counts
    assert bsa.prefill_workspace_size(2, 16, 64, 3) >= 3 * 2 * 16 * (128 * 66 * 4 + 3 * 4)
    a.n_merges, a.n_slots = 4, 2                                   # more merges than slots
    assert lib.bsattn_prefill_fwd(C.byref(a), None) == _abi.BSATTN_ERR_INVALID_ARG


def test_transpose_block_index():
    """CSC of a CSR: every (tile, block) pair exactly once, tiles ascending per
    block; empty tiles and never-kept blocks; malformed CSRs are refused."""
    g = np.random.default_rng(5)
    for Tr, Tc in ((1, 1), (3, 5), (34, 68), (7, 2)):
        tm = g.random((Tr, Tc)) < 0.4
        tm[0] = False
        row_ptr = np.concatenate([[0], np.cumsum(tm.sum(axis=1))]).astype(np.int32)
        col_idx = np.concatenate([np.nonzero(r)[0] for r in tm] + [np.zeros(0, int)]).astype(np.int32)
        col_ptr, row_idx = bsa.transpose_block_index(row_ptr, col_idx, Tc)
        assert col_ptr[0] == 0 and col_ptr[-1] == tm.sum()
        for j in range(Tc):
            assert row_idx[col_ptr[j]:col_ptr[j + 1]].tolist() == np.nonzero(tm[:, j])[0].tolist()
    with pytest.raises(bsa.BsattnError):
        bsa.transpose_block_index(np.array([0, 2], np.int32), np.array([1, 0], np.int32), 4)   # not ascending
    with pytest.raises(bsa.BsattnError):
        bsa.transpose_block_index(np.array([0, 1], np.int32), np.array([4], np.int32), 4)      # out of range


def test_block_index_from_matrix_bitmap_coo():
    """The block-mask forms of the DiT article (0/1 matrix, one-bit-per-block
    bitmap, COO pairs) give the oracle's CSR of the same matrix; the bitmap
    has the article's size; bad input is refused."""
    g = np.random.default_rng(9)
    for Tr, Tc in ((1, 1), (3, 5), (34, 68), (9, 2)):
        tm = g.random((Tr, Tc)) < 0.3
        tm[0] = False
        ref = M.csr_from_tile_mask(tm)
        got = bsa.block_index_from_matrix(tm)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
        bits = np.packbits(tm.reshape(-1), bitorder="little")
        assert bits.size == M.bitmap_bytes(Tr, Tc)
        got = bsa.block_index_from_bitmap(bits, Tr, Tc)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
        r, c = np.nonzero(tm)
        perm = g.permutation(r.size)
        r2, c2 = np.concatenate([r[perm], r[:3]]), np.concatenate([c[perm], c[:3]])   # shuffled, duplicates
        got = bsa.block_index_from_coo(r2, c2, Tr, Tc)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
        bsa.validate_block_index(got[0], got[1], Tc)
    with pytest.raises(bsa.BsattnError):
        bsa.block_index_from_coo(np.array([0, 3]), np.array([0, 0]), 3, 4)      # row out of range
    with pytest.raises(bsa.BsattnError):
        bsa.block_index_from_coo(np.array([0]), np.array([-1]), 3, 4)            # col out of range
    with pytest.raises(bsa.BsattnError):
        bsa.block_index_from_bitmap(np.zeros(1, np.uint8), 3, 4)                # 8 bits < 12 blocks
