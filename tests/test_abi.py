"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/bsattn.h, and rejects invalid arguments on the host
(validation returns before any HIP call)."""

import ctypes as C
import os
import re

import pytest

import block_sparse_attention_flash_amd as bsa
from block_sparse_attention_flash_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "bsattn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsattn_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = bsa.library()
    names = _declared_functions()
    assert len(names) >= 10
    assert set(names) == set(_abi.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.bsattn_version() == 0x000100


def test_status_strings():
    lib = bsa.library()
    assert lib.bsattn_status_string(0) == b"BSATTN_OK"
    assert lib.bsattn_status_string(3) == b"BSATTN_ERR_CAPACITY"
    assert lib.bsattn_status_string(99) == b"BSATTN_ERR_UNKNOWN"


# ---- prefill validation ---------------------------------------------------------

FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def _good_prefill():
    a = _abi.PrefillArgs()
    a.dtype = _abi.BSATTN_BF16
    a.q = a.k = a.v = a.out = FAKE
    a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.d = 1, 4, 2, 256, 256, 128
    for f in ("q_stride", "k_stride", "v_stride", "o_stride"):
        getattr(a, f)[:] = [256 * 4 * 128, 4 * 128, 128]
    a.scale, a.lam, a.causal, a.Br, a.Bc = 0.088, 0.0, 0, 128, 64
    return a


BAD_PREFILL = [
    ("dtype", lambda a: setattr(a, "dtype", 7), _abi.BSATTN_ERR_UNSUPPORTED),
    ("null q", lambda a: setattr(a, "q", None), _abi.BSATTN_ERR_INVALID_ARG),
    ("misaligned k", lambda a: setattr(a, "k", FAKE + 2), _abi.BSATTN_ERR_UNSUPPORTED),
    ("B = 0", lambda a: setattr(a, "B", 0), _abi.BSATTN_ERR_INVALID_ARG),
    ("Hq % Hkv", lambda a: setattr(a, "Hkv", 3), _abi.BSATTN_ERR_INVALID_ARG),
    ("d = 96", lambda a: setattr(a, "d", 96), _abi.BSATTN_ERR_UNSUPPORTED),
    ("token stride not x8", lambda a: a.q_stride.__setitem__(1, 4 * 128 + 4), _abi.BSATTN_ERR_UNSUPPORTED),
    ("negative stride", lambda a: a.v_stride.__setitem__(0, -8), _abi.BSATTN_ERR_INVALID_ARG),
    ("row_ptr without col_idx", lambda a: setattr(a, "row_ptr", FAKE), _abi.BSATTN_ERR_INVALID_ARG),
    ("scale 0", lambda a: setattr(a, "scale", 0.0), _abi.BSATTN_ERR_INVALID_ARG),
    ("scale nan", lambda a: setattr(a, "scale", float("nan")), _abi.BSATTN_ERR_INVALID_ARG),
    ("lambda 1", lambda a: setattr(a, "lam", 1.0), _abi.BSATTN_ERR_INVALID_ARG),
    ("lambda < 0", lambda a: setattr(a, "lam", -0.5), _abi.BSATTN_ERR_INVALID_ARG),
    ("causal Nq != Nk", lambda a: (setattr(a, "causal", 1), setattr(a, "Nk", 128)), _abi.BSATTN_ERR_INVALID_ARG),
    ("n_valid > Nk", lambda a: setattr(a, "n_valid", 257), _abi.BSATTN_ERR_INVALID_ARG),
    ("Bc 32", lambda a: setattr(a, "Bc", 32), _abi.BSATTN_ERR_UNSUPPORTED),
    ("bf16 Br 64", lambda a: setattr(a, "Br", 64), _abi.BSATTN_ERR_UNSUPPORTED),
    ("K extent past 32-bit offsets", lambda a: (setattr(a, "Nk", 1 << 21), setattr(a, "Nq", 1 << 21),
                                                 a.k_stride.__setitem__(1, 1024)), _abi.BSATTN_ERR_UNSUPPORTED),
]


def _good_bwd():
    a = _abi.BwdArgs()
    a.dtype = _abi.BSATTN_BF16
    a.q = a.k = a.v = a.out = a.dout = a.dq = a.dk = a.dv = FAKE
    a.lse = FAKE
    a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.d = 2, 8, 2, 256, 256, 128
    for fld, h in (("q_stride", 8), ("k_stride", 2), ("v_stride", 2), ("o_stride", 8), ("do_stride", 8),
                   ("dq_stride", 8), ("dk_stride", 2), ("dv_stride", 2)):
        getattr(a, fld)[:] = [256 * h * 128, h * 128, 128]
    a.scale, a.Br, a.Bc = 0.088, 128, 64
    a.workspace = 0x100000
    a.workspace_bytes = bsa.prefill_bwd_workspace_size(2, 8, 2, 256, 128)
    return a


BAD_BWD = [
    ("fp32", lambda a: setattr(a, "dtype", _abi.BSATTN_FP32), _abi.BSATTN_ERR_UNSUPPORTED),
    ("null dout", lambda a: setattr(a, "dout", None), _abi.BSATTN_ERR_INVALID_ARG),
    ("misaligned dk", lambda a: setattr(a, "dk", FAKE + 8), _abi.BSATTN_ERR_UNSUPPORTED),
    ("null lse", lambda a: setattr(a, "lse", None), _abi.BSATTN_ERR_INVALID_ARG),
    ("Hq % Hkv", lambda a: setattr(a, "Hkv", 3), _abi.BSATTN_ERR_INVALID_ARG),
    ("d = 96", lambda a: setattr(a, "d", 96), _abi.BSATTN_ERR_UNSUPPORTED),
    ("dq stride not x8", lambda a: a.dq_stride.__setitem__(1, 8 * 128 + 4), _abi.BSATTN_ERR_UNSUPPORTED),
    ("CSR without CSC", lambda a: (setattr(a, "row_ptr", FAKE), setattr(a, "col_idx", FAKE)),
     _abi.BSATTN_ERR_INVALID_ARG),
    ("causal Nq != Nk", lambda a: (setattr(a, "causal", 1), setattr(a, "Nk", 128)), _abi.BSATTN_ERR_INVALID_ARG),
    ("n_valid > Nk", lambda a: setattr(a, "n_valid", 257), _abi.BSATTN_ERR_INVALID_ARG),
    ("Br 64", lambda a: setattr(a, "Br", 64), _abi.BSATTN_ERR_UNSUPPORTED),
    ("workspace small", lambda a: setattr(a, "workspace_bytes", 64), _abi.BSATTN_ERR_CAPACITY),
    ("workspace misaligned", lambda a: setattr(a, "workspace", 0x100010), _abi.BSATTN_ERR_INVALID_ARG),
    ("dq schedule without CSR", lambda a: (setattr(a, "dq_items", FAKE), setattr(a, "dq_n_items", 4)),
     _abi.BSATTN_ERR_INVALID_ARG),
    ("kv schedule without CSC", lambda a: (setattr(a, "kv_items", FAKE), setattr(a, "kv_n_items", 4)),
     _abi.BSATTN_ERR_INVALID_ARG),
    ("dq slots without items", lambda a: setattr(a, "dq_n_slots", 2), _abi.BSATTN_ERR_INVALID_ARG),
    ("kv merges without merge array", lambda a: (_with_index(a), setattr(a, "kv_items", FAKE),
                                                 setattr(a, "kv_n_items", 3), setattr(a, "kv_n_merges", 1),
                                                 setattr(a, "kv_n_slots", 2)), _abi.BSATTN_ERR_INVALID_ARG),
    ("dq slots beyond workspace", lambda a: (_with_index(a), setattr(a, "dq_items", FAKE), setattr(a, "dq_n_items", 3),
                                             setattr(a, "dq_merges", FAKE), setattr(a, "dq_n_merges", 1),
                                             setattr(a, "dq_n_slots", 2)), _abi.BSATTN_ERR_CAPACITY),
]


def _with_index(a):
    a.row_ptr = a.col_idx = a.col_ptr = a.row_idx = FAKE


def test_backward_workspace_covers_schedule_slots():
    base = bsa.prefill_bwd_workspace_size(2, 8, 2, 256, 128)
    assert base >= 2 * 8 * 256 * 4
    # dQ partials: 128 rows x d floats per slot, batch and head; dK/dV: 2 blocks x 64 keys x d x 2 at d = 128
    assert bsa.prefill_bwd_workspace_size(2, 8, 2, 256, 128, dq_n_slots=3) >= base + 3 * 2 * 8 * 128 * 128 * 4
    assert bsa.prefill_bwd_workspace_size(2, 8, 2, 256, 128, kv_n_slots=5) >= base + 5 * 2 * 2 * 2 * 64 * 128 * 2 * 4
    assert bsa.prefill_bwd_workspace_size(2, 8, 2, 256, 64, kv_n_slots=5) >= 5 * 2 * 2 * 1 * 64 * 64 * 2 * 4
    assert bsa.prefill_bwd_workspace_size(2, 8, 2, 256, 96) == 0
    assert bsa.prefill_bwd_workspace_size(2, 8, 2, 256, 128, dq_n_slots=-1) == 0


@pytest.mark.parametrize("name,mutate,status", BAD_BWD, ids=[b[0] for b in BAD_BWD])
def test_backward_rejects(name, mutate, status):
    a = _good_bwd()
    mutate(a)
    st = bsa.library().bsattn_prefill_bwd(C.byref(a), None)
    assert st == status, (name, bsa.library().bsattn_last_error())


@pytest.mark.parametrize("name,mutate,status", BAD_PREFILL, ids=[b[0] for b in BAD_PREFILL])
def test_prefill_rejects(name, mutate, status):
    a = _good_prefill()
    mutate(a)
    st = bsa.library().bsattn_prefill_fwd(C.byref(a), None)
    assert st == status, (name, bsa.library().bsattn_last_error())
    assert bsa.library().bsattn_last_error()


def test_prefill_null_args():
    assert bsa.library().bsattn_prefill_fwd(None, None) == _abi.BSATTN_ERR_INVALID_ARG


# ---- decode validation ----------------------------------------------------------

def _good_decode():
    a = _abi.DecodeArgs()
    a.q = a.k_cache = a.v_cache = a.out = FAKE
    a.B, a.Hq, a.Hkv, a.L, a.Lmax, a.d = 2, 8, 2, 1000, 1024, 128
    a.q_stride[:] = [8 * 128, 128]
    a.kv_stride[:] = [1024 * 2 * 128, 2 * 128, 128]
    a.o_stride[:] = [8 * 128, 128]
    a.scale, a.lam, a.Bc, a.num_splits = 0.088, 0.01, 64, 0
    a.workspace = 0x100000
    a.workspace_bytes = bsa.decode_workspace_size(2, 8, 2, 1000, 128)
    return a


BAD_DECODE = [
    ("null workspace", lambda a: setattr(a, "workspace", None), _abi.BSATTN_ERR_INVALID_ARG),
    ("workspace misaligned", lambda a: setattr(a, "workspace", 0x100010), _abi.BSATTN_ERR_INVALID_ARG),
    ("workspace small", lambda a: setattr(a, "workspace_bytes", 64), _abi.BSATTN_ERR_CAPACITY),
    ("L > Lmax", lambda a: setattr(a, "L", 2000), _abi.BSATTN_ERR_INVALID_ARG),
    ("L = 0", lambda a: setattr(a, "L", 0), _abi.BSATTN_ERR_INVALID_ARG),
    ("G = 16", lambda a: (setattr(a, "Hq", 32), setattr(a, "Hkv", 2)), _abi.BSATTN_ERR_UNSUPPORTED),
    ("G = 3", lambda a: (setattr(a, "Hq", 6), setattr(a, "Hkv", 2)), _abi.BSATTN_ERR_UNSUPPORTED),
    ("lambda 1", lambda a: setattr(a, "lam", 1.5), _abi.BSATTN_ERR_INVALID_ARG),
    ("d 80", lambda a: setattr(a, "d", 80), _abi.BSATTN_ERR_UNSUPPORTED),
    ("Bc 128", lambda a: setattr(a, "Bc", 128), _abi.BSATTN_ERR_UNSUPPORTED),
    ("kv stride", lambda a: a.kv_stride.__setitem__(1, 2 * 128 + 1), _abi.BSATTN_ERR_UNSUPPORTED),
    ("negative splits", lambda a: setattr(a, "num_splits", -1), _abi.BSATTN_ERR_INVALID_ARG),
    ("block order 2", lambda a: setattr(a, "block_order", 2), _abi.BSATTN_ERR_INVALID_ARG),
    ("max scope 2", lambda a: setattr(a, "max_scope", 2), _abi.BSATTN_ERR_INVALID_ARG),
    ("decisions -1", lambda a: setattr(a, "decisions", -1), _abi.BSATTN_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("name,mutate,status", BAD_DECODE, ids=[b[0] for b in BAD_DECODE])
def test_decode_rejects(name, mutate, status):
    a = _good_decode()
    mutate(a)
    st = bsa.library().bsattn_decode_fwd(C.byref(a), None)
    assert st == status, (name, bsa.library().bsattn_last_error())


def test_decode_split_policy():
    # automatic: splits of at most 56 blocks (7/8 of the 64-block cap), enough work-groups for the chip
    S = bsa.decode_num_splits(32, 32, 8, 131072, 128)
    assert S == 37                                                    # ceil(2048 / 56)
    assert bsa.decode_num_splits(1, 32, 8, 131072, 128) == 256      # 8 blocks per split: 2048 work-groups
    assert bsa.decode_num_splits(1, 4, 1, 4096, 128) >= 2
    # an explicit count is honoured up to 64 blocks per split (one 64-bit skip mask)
    assert bsa.decode_num_splits(1, 4, 1, 64 * 64, 128, num_splits=4) == 4
    assert bsa.decode_num_splits(1, 4, 1, 64 * 64, 128, num_splits=1) == 1
    assert bsa.decode_num_splits(1, 4, 1, 128 * 64, 128, num_splits=1) == 2
    # blocks per split: S = ceil(Tc / n)
    assert bsa.decode_split_blocks(32, 32, 8, 131072, 128) == 56
    assert bsa.decode_split_blocks(1, 4, 1, 64 * 10, 128, num_splits=3) == 4
    assert bsa.decode_split_blocks(1, 4, 1, 128 * 64, 128, num_splits=1) == 64
    assert bsa.decode_split_blocks(1, 4, 3, 64, 128) == 0                        # Hq % Hkv != 0
    assert bsa.decode_workspace_size(32, 32, 8, 131072, 128) > 32 * 8 * 32 * 4 * 128 * 4   # partial O of every split
    assert bsa.decode_workspace_size(0, 1, 1, 1, 64) == 0


def test_decode_noalloc_rejects_on_the_host():
    """bsattn_decode_fwd_noalloc refuses a workspace argument and a call whose
    workspace would exceed its fixed scratch, before anything is enqueued."""
    lib = bsa.library()
    a = _good_decode()
    assert lib.bsattn_decode_fwd_noalloc(C.byref(a), None) == _abi.BSATTN_ERR_INVALID_ARG   # workspace given
    a.workspace, a.workspace_bytes = None, 0
    a.B, a.Hq, a.Hkv, a.L, a.Lmax = 64, 32, 8, 131072, 131072                               # ~40 MiB of workspace
    assert bsa.decode_workspace_size(64, 32, 8, 131072, 128) > 32 << 20
    assert lib.bsattn_decode_fwd_noalloc(C.byref(a), None) == _abi.BSATTN_ERR_CAPACITY
    assert b"scratch" in lib.bsattn_last_error()
    a.lam = 2.0                                                                             # ordinary validation
    assert lib.bsattn_decode_fwd_noalloc(C.byref(a), None) == _abi.BSATTN_ERR_INVALID_ARG
    assert lib.bsattn_decode_fwd_noalloc(None, None) == _abi.BSATTN_ERR_INVALID_ARG
