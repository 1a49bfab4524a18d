"""Block-sparse and BLASST flash attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libbsattn.so`` (``include/bsattn.h``).
It only marshals arguments: torch tensors supply device pointers, strides and
the current HIP stream; every step of the computation runs in the library's
HIP kernels (or, for the block index, its host C++ builder).  If the library
is missing the binding raises; there is no fallback implementation.

Entry points (same names as the C ABI, minus the ``bsattn_`` prefix):

* ``build_block_index(spec, n_q, n_k, Br, Bc)`` -> (row_ptr, col_idx) int32 numpy
* ``validate_block_index(row_ptr, col_idx, Tc)``
* ``block_index_from_matrix(m)``, ``block_index_from_bitmap(bits, Tr, Tc)``,
  ``block_index_from_coo(rows, cols, Tr, Tc)`` -> (row_ptr, col_idx)
* ``tile_order_lpt(row_ptr)`` -> int32 numpy launch order
* ``build_schedule(row_ptr, max_blocks_per_item, order="longest_first")`` -> Schedule
  (host arrays, counts); ``order="tile"`` applies ``bsattn_schedule_tile_order``;
  ``prefill_group_major(B, Hq, Hkv, d, n_units)``; ``default_schedule(row_ptr, B, Hq, Hkv, d)``
  (chunk bound and order chosen for the launch)
* ``prefill_workspace_size(B, Hq, d, n_slots)``, ``prefill_workspace(...)`` (zero-filled)
* ``prefill_fwd(q, k, v, ...)`` -> out tensor (async on the current stream)
* ``prefill_bwd(q, k, v, out, dout, lse, ...)`` -> (dq, dk, dv) for a static mask;
  ``transpose_block_index(row_ptr, col_idx, Tc)`` -> (col_ptr, row_idx),
  ``prefill_bwd_workspace_size(B, Hq, Hkv, Nq, d, dq_n_slots=0, kv_n_slots=0)``,
  ``build_dkdv_schedule(col_ptr, row_idx, G, d, max_positions_per_item)``, ``BwdSchedule``,
  ``default_bwd_schedule(row_ptr, col_ptr, row_idx, B, Hq, Hkv, d)``
* ``decode_fwd(q, k_cache, v_cache, ...)`` -> out tensor (``noalloc=True``:
  ``bsattn_decode_fwd_noalloc``, the library's fixed scratch instead of a workspace)
* ``calibrate_fit(...)``, ``calibrate(target, lengths, lambdas, delta, measure)``,
  ``decode_sparsity(...)``: threshold calibration lambda = a / L
* ``prefill_plan(...)``, ``decode_plan(...)`` -> Plan: the same calls marshalled
  once; ``plan(stream=None)`` enqueues with a single C-ABI call
* ``decode_workspace_size(...)``, ``decode_workspace(...)`` (zero-filled), ``decode_num_splits(...)``, ``decode_split_blocks(...)``,
  ``decode_check(workspace)`` (reads and clears the health word)
"""

from __future__ import annotations

import ctypes as C
import math
from typing import Optional

import numpy as np

from . import _abi

__all__ = [
    "BsattnError", "library", "build_block_index", "validate_block_index", "tile_order_lpt",
    "block_index_from_matrix", "block_index_from_bitmap", "block_index_from_coo",
    "Schedule", "build_schedule", "default_max_blocks_per_item", "default_schedule", "prefill_group_major", "prefill_workspace_size", "prefill_workspace",
    "prefill_fwd", "prefill_plan", "prefill_bwd", "prefill_bwd_plan", "prefill_bwd_workspace_size", "transpose_block_index",
    "build_dkdv_schedule", "BwdSchedule", "default_bwd_schedule",
    "decode_fwd", "decode_plan", "Plan", "decode_workspace_size", "decode_workspace", "decode_num_splits",
    "decode_split_blocks", "decode_check",
    "calibrate_fit", "calibrate", "decode_sparsity",
]


class BsattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


_LIB: Optional[C.CDLL] = None


def library() -> C.CDLL:
    """The loaded libbsattn (raises if it has not been built).

    The library shares the HIP runtime of the host process.  Its code objects
    register with that runtime when it is loaded, so torch's HIP context is
    brought up first when a GPU is present (loading it before the runtime has
    enumerated devices leaves the library's launches without a device)."""
    global _LIB
    if _LIB is None:
        try:
            import torch
            if torch.cuda.is_available():
                torch.cuda.init()
        except ImportError:  # pragma: no cover - C-only callers manage HIP themselves
            pass
        _LIB = _abi.load()
    return _LIB


def _status_name(st: int) -> str:
    try:
        return library().bsattn_status_string(st).decode()
    except Exception:  # pragma: no cover
        return f"status {st}"


def _check(st: int):
    if st != _abi.BSATTN_OK:
        raise BsattnError(st, library().bsattn_last_error().decode())


# ---------------------------------------------------------------------------
# block index (host)
# ---------------------------------------------------------------------------

def _c_spec(spec):
    segs = list(spec.segments)
    arr = (_abi.Segment * max(1, len(segs)))()
    for i, s in enumerate(segs):
        arr[i] = _abi.Segment(int(s.kind), int(s.start), int(getattr(s, "length", getattr(s, "len", 0))),
                              int(s.frames), int(s.grid_h), int(s.grid_w), int(s.radius), int(s.t_radius),
                              int(s.unit))
    cs = _abi.MaskSpec(int(spec.n_valid), len(segs), C.cast(arr, C.POINTER(_abi.Segment)),
                       int(spec.anchor_start), int(spec.anchor_len))
    return cs, arr


def build_block_index(spec, n_q: int, n_k: int, Br: int, Bc: int):
    """Per-query-tile CSR of kept key blocks for a mask specification.

    ``spec`` is any object with ``n_valid``, ``segments`` (objects with kind,
    start, length, frames, grid_h, grid_w, radius, t_radius, unit),
    ``anchor_start`` and ``anchor_len``."""
    lib = library()
    cs, keep = _c_spec(spec)
    Tr = -(-n_q // Br)
    row_ptr = np.zeros(Tr + 1, dtype=np.int32)
    nnz = C.c_int64(0)
    _check(lib.bsattn_build_block_index(C.byref(cs), n_q, n_k, Br, Bc, row_ptr.ctypes.data, None, 0, C.byref(nnz)))
    col_idx = np.zeros(max(1, nnz.value), dtype=np.int32)
    _check(lib.bsattn_build_block_index(C.byref(cs), n_q, n_k, Br, Bc, row_ptr.ctypes.data, col_idx.ctypes.data,
                                        col_idx.size, C.byref(nnz)))
    del keep
    return row_ptr, col_idx[:nnz.value].copy()


def validate_block_index(row_ptr, col_idx, Tc: int):
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    _check(library().bsattn_validate_block_index(row_ptr.ctypes.data, col_idx.ctypes.data if col_idx.size else None,
                                                 row_ptr.size - 1, Tc))


def _csr_two_call(fn, head_args, Tr: int):
    row_ptr = np.zeros(Tr + 1, np.int32)
    nnz = C.c_int64(0)
    _check(fn(*head_args, row_ptr.ctypes.data, None, 0, C.byref(nnz)))
    col_idx = np.zeros(max(1, nnz.value), np.int32)
    _check(fn(*head_args, row_ptr.ctypes.data, col_idx.ctypes.data, col_idx.size, C.byref(nnz)))
    return row_ptr, col_idx[:nnz.value].copy()


def block_index_from_matrix(m):
    """CSR of a 0/1 block matrix (host array [Tr, Tc], nonzero = kept)."""
    m = np.ascontiguousarray(m, dtype=np.uint8)
    Tr, Tc = m.shape
    return _csr_two_call(library().bsattn_block_index_from_matrix, (m.ctypes.data, Tr, Tc), Tr)


def block_index_from_bitmap(bits, Tr: int, Tc: int):
    """CSR of a block bitmap: bit t * Tc + j (LSB first) set = kept."""
    bits = np.ascontiguousarray(bits, dtype=np.uint8)
    if bits.size * 8 < Tr * Tc:
        raise BsattnError(_abi.BSATTN_ERR_INVALID_ARG, "bitmap shorter than Tr * Tc bits")
    return _csr_two_call(library().bsattn_block_index_from_bitmap, (bits.ctypes.data, Tr, Tc), Tr)


def block_index_from_coo(rows, cols, Tr: int, Tc: int):
    """CSR of COO (row, col) pairs of kept blocks (any order, duplicates allowed)."""
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    cols = np.ascontiguousarray(cols, dtype=np.int32)
    if rows.shape != cols.shape:
        raise BsattnError(_abi.BSATTN_ERR_INVALID_ARG, "rows and cols differ in length")
    return _csr_two_call(library().bsattn_block_index_from_coo,
                         (rows.ctypes.data, cols.ctypes.data, rows.size, Tr, Tc), Tr)


def transpose_block_index(row_ptr, col_idx, Tc: int):
    """CSR (tiles -> key blocks) to CSC (key blocks -> tiles), host int32 arrays."""
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    col_idx = np.ascontiguousarray(col_idx, dtype=np.int32)
    Tr = row_ptr.size - 1
    col_ptr = np.zeros(Tc + 1, np.int32)
    row_idx = np.zeros(max(1, int(row_ptr[-1])), np.int32)
    _check(library().bsattn_transpose_block_index(row_ptr.ctypes.data, col_idx.ctypes.data, Tr, int(Tc),
                                                  col_ptr.ctypes.data, row_idx.ctypes.data))
    return col_ptr, row_idx[:int(row_ptr[-1])].copy()


def tile_order_lpt(row_ptr):
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    order = np.zeros(row_ptr.size - 1, dtype=np.int32)
    _check(library().bsattn_tile_order_lpt(row_ptr.ctypes.data, row_ptr.size - 1, order.ctypes.data))
    return order


class Schedule:
    """Host arrays of bsattn_build_schedule plus their device copies (``to``)."""

    def __init__(self, items, merges, n_slots):
        self.items, self.merges, self.n_slots = items, merges, int(n_slots)
        self.d_items = self.d_merges = None

    @property
    def n_items(self) -> int:
        return self.items.shape[0]

    @property
    def n_merges(self) -> int:
        return self.merges.shape[0]

    def to(self, device):
        torch = _torch()
        self.d_items = torch.from_numpy(self.items.reshape(-1)).to(device)
        self.d_merges = torch.from_numpy(self.merges.reshape(-1)).to(device) if self.n_merges else None
        return self


def default_max_blocks_per_item(row_ptr, B: int, Hq: int, slots: int = 512) -> int:
    """Chunk bound: half the mean work per concurrent work-group slot, at least 16 blocks."""
    total = int(row_ptr[-1]) * B * Hq
    return max(16, -(-total // (2 * slots)))


def build_schedule(row_ptr, max_blocks_per_item: int, order: str = "longest_first") -> Schedule:
    """``order``: "longest_first" (the builder's order) or "tile" (cut chunks
    first, then whole tiles by index: ``bsattn_schedule_tile_order``)."""
    if order not in ("longest_first", "tile"):
        raise ValueError(f"order must be 'longest_first' or 'tile', not {order!r}")
    row_ptr = np.ascontiguousarray(row_ptr, dtype=np.int32)
    Tr = row_ptr.size - 1
    ni, nm, ns = C.c_int32(0), C.c_int32(0), C.c_int32(0)
    lib = library()
    _check(lib.bsattn_build_schedule(row_ptr.ctypes.data, Tr, int(max_blocks_per_item), None, 0, None, 0,
                                     C.byref(ni), C.byref(nm), C.byref(ns)))
    items = np.zeros((ni.value, 5), np.int32)
    merges = np.zeros((max(1, nm.value), 3), np.int32)
    _check(lib.bsattn_build_schedule(row_ptr.ctypes.data, Tr, int(max_blocks_per_item), items.ctypes.data,
                                     ni.value, merges.ctypes.data, merges.shape[0], C.byref(ni), C.byref(nm),
                                     C.byref(ns)))
    if order == "tile":
        _check(lib.bsattn_schedule_tile_order(items.ctypes.data, ni.value))
    return Schedule(items, merges[:nm.value].copy(), ns.value)


def prefill_group_major(B: int, Hq: int, Hkv: int, d: int, n_units: int) -> bool:
    """True when a bf16 prefill launch walks each (batch, K/V head) group's
    work items consecutively (``bsattn_prefill_group_major``)."""
    r = int(library().bsattn_prefill_group_major(B, Hq, Hkv, d, n_units))
    if r < 0:
        raise ValueError(f"invalid prefill shape B={B} Hq={Hq} Hkv={Hkv} d={d} n_units={n_units}")
    return r == 1


def default_schedule(row_ptr, B: int, Hq: int, Hkv: int, d: int) -> Schedule:
    """Schedule with ``default_max_blocks_per_item``, in tile order when the
    launch walks groups one at a time (neighbouring tiles then share K/V
    blocks in L2), longest first otherwise (the shorter tail)."""
    s = build_schedule(row_ptr, default_max_blocks_per_item(row_ptr, B, Hq))
    if prefill_group_major(B, Hq, Hkv, d, s.n_items):
        _check(library().bsattn_schedule_tile_order(s.items.ctypes.data, s.n_items))
    return s


def prefill_workspace_size(B: int, Hq: int, d: int, n_slots: int) -> int:
    return int(library().bsattn_prefill_workspace_size(B, Hq, d, n_slots))


def prefill_workspace(B: int, Hq: int, d: int, n_slots: int, device):
    """A prefill workspace (zero-filled; every call zeroes the words it counts
    with, so calls of any shape can reuse it on one stream)."""
    return _torch().zeros(prefill_workspace_size(B, Hq, d, n_slots), dtype=_torch().uint8, device=device)


# ---------------------------------------------------------------------------
# device entry points
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream_handle(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _order_code(order: str) -> int:
    if order not in ("ascending", "descending"):
        raise BsattnError(_abi.BSATTN_ERR_INVALID_ARG, f"order must be 'ascending' or 'descending', not {order!r}")
    return 1 if order == "descending" else 0


def _choice_code(name: str, value: str, choices) -> int:
    if value not in choices:
        raise BsattnError(_abi.BSATTN_ERR_INVALID_ARG, f"{name} must be one of {choices}, not {value!r}")
    return choices.index(value)


def _ptr(t) -> Optional[int]:
    return None if t is None else int(t.data_ptr())


def _index_tensor(t):
    """A block-index array for the C ABI: an empty one (a CSR that keeps no
    block) has no data pointer, so it is replaced by a one-element array the
    kernels never read (row_ptr says there is nothing to read)."""
    if t is None or t.numel() > 0:
        return t
    return _torch().zeros(1, dtype=t.dtype, device=t.device)


class Plan:
    """A marshalled call: the C argument struct is built once; each call of the
    plan enqueues the operation on a stream (default: torch's current stream)
    with one C-ABI call.  The plan keeps a reference to every tensor it points
    at; the caller must not resize or reallocate them while the plan is used."""

    def __init__(self, fn, args, out, keep):
        self._fn, self._args, self.out, self._keep = fn, args, out, keep
        self._ref = C.byref(args)

    def __call__(self, stream=None):
        _check(self._fn(self._ref, C.c_void_p(_stream_handle(stream))))
        return self.out


def prefill_plan(q, k, v, *, scale: Optional[float] = None, lam: float = 0.0, causal: bool = False,
                 Br: int = 128, Bc: int = 64, row_ptr=None, col_idx=None, tile_order=None, n_valid: int = 0,
                 out=None, tile_counters=None, block_state=None, row_counters=None,
                 schedule: Optional[Schedule] = None, workspace=None, order: str = "ascending",
                 lse=None) -> Plan:
    """Marshal a prefill (arguments as ``prefill_fwd``) into a reusable Plan."""
    torch = _torch()
    if q.dtype == torch.bfloat16:
        dt = _abi.BSATTN_BF16
    elif q.dtype == torch.float32:
        dt = _abi.BSATTN_FP32
    else:
        raise BsattnError(_abi.BSATTN_ERR_UNSUPPORTED, f"dtype {q.dtype} not supported")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise BsattnError(_abi.BSATTN_ERR_INVALID_ARG, "q, k, v must share a dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dim() != 4 or t.stride(3) != 1:
            raise BsattnError(_abi.BSATTN_ERR_INVALID_ARG, f"{name} must be [B, N, H, d] with d contiguous")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    a = _abi.PrefillArgs()
    a.dtype = dt
    a.q, a.k, a.v, a.out = _ptr(q), _ptr(k), _ptr(v), _ptr(out)
    a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.d = B, Hq, Hkv, Nq, Nk, d
    for fld, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out)):
        getattr(a, fld)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    col_idx = _index_tensor(col_idx)
    a.row_ptr, a.col_idx, a.tile_order = _ptr(row_ptr), _ptr(col_idx), _ptr(tile_order)
    a.n_valid = int(n_valid)
    a.scale = float(scale if scale is not None else 1.0 / math.sqrt(d))
    a.lam = float(lam)
    a.causal = 1 if causal else 0
    a.Br, a.Bc = int(Br), int(Bc)
    a.tile_counters, a.block_state = _ptr(tile_counters), _ptr(block_state)
    a.row_counters = _ptr(row_counters)
    a.block_order = _order_code(order)
    a.lse = _ptr(lse)
    if schedule is not None:
        if schedule.d_items is None:
            schedule.to(q.device)
        a.sched_items, a.n_items = _ptr(schedule.d_items), schedule.n_items
        a.sched_merges, a.n_merges, a.n_slots = _ptr(schedule.d_merges), schedule.n_merges, schedule.n_slots
        if schedule.n_slots > 0:
            if workspace is None:
                workspace = prefill_workspace(B, Hq, d, schedule.n_slots, q.device)
            a.workspace = _ptr(workspace)
            a.workspace_bytes = int(workspace.numel() * workspace.element_size())
    keep = (q, k, v, row_ptr, col_idx, tile_order, tile_counters, block_state, row_counters, schedule, workspace,
            lse)
    return Plan(library().bsattn_prefill_fwd, a, out, keep)


def prefill_fwd(q, k, v, *, scale: Optional[float] = None, lam: float = 0.0, causal: bool = False,
                Br: int = 128, Bc: int = 64, row_ptr=None, col_idx=None, tile_order=None, n_valid: int = 0,
                out=None, tile_counters=None, block_state=None, row_counters=None,
                schedule: Optional[Schedule] = None, workspace=None, order: str = "ascending", lse=None,
                stream=None):
    """Block-sparse / BLASST attention forward, q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] (last dim contiguous).

    ``row_ptr``/``col_idx``/``tile_order`` are int32 device tensors (or None);
    ``tile_counters`` int32 [B, Hq, Tr, 2] and ``block_state`` uint8
    [B, Hq, Tr, Tc] are optional device outputs, as is ``row_counters`` int32
    [B, Hq, Tr] (per-row skip conditions that held, for lambda > 0).
    ``order`` "descending" visits each tile's blocks most recent first (the
    BLASST notes' block-row reordering).  ``schedule`` (from
    ``build_schedule``, device copies made with ``.to``) cuts long tiles;
    its partials go to ``workspace`` (a uint8 device tensor from
    ``prefill_workspace``, allocated here if None).  ``lse`` float32
    [B, Hq, Nq] optionally receives each row's natural-log sum of exp of
    its attended scores (input of ``prefill_bwd``).  Returns ``out``."""
    return prefill_plan(q, k, v, scale=scale, lam=lam, causal=causal, Br=Br, Bc=Bc, row_ptr=row_ptr,
                        col_idx=col_idx, tile_order=tile_order, n_valid=n_valid, out=out,
                        tile_counters=tile_counters, block_state=block_state, row_counters=row_counters,
                        schedule=schedule, order=order,
                        workspace=workspace, lse=lse)(stream)


def prefill_bwd_workspace_size(B: int, Hq: int, Hkv: int, Nq: int, d: int, dq_n_slots: int = 0,
                               kv_n_slots: int = 0) -> int:
    return int(library().bsattn_prefill_bwd_workspace_size(B, Hq, Hkv, Nq, d, dq_n_slots, kv_n_slots))


class KvSchedule:
    """Host arrays of bsattn_build_dkdv_schedule plus their device copies (``to``)."""

    def __init__(self, items, merges, n_slots):
        self.items, self.merges, self.n_slots = items, merges, int(n_slots)
        self.d_items = self.d_merges = None

    @property
    def n_items(self) -> int:
        return self.items.shape[0]

    @property
    def n_merges(self) -> int:
        return self.merges.shape[0]

    def to(self, device):
        torch = _torch()
        self.d_items = torch.from_numpy(self.items.reshape(-1)).to(device)
        self.d_merges = torch.from_numpy(self.merges.reshape(-1)).to(device) if self.n_merges else None
        return self


def build_dkdv_schedule(col_ptr, row_idx, G: int, d: int, max_positions_per_item: int) -> KvSchedule:
    col_ptr = np.ascontiguousarray(col_ptr, dtype=np.int32)
    row_idx = np.ascontiguousarray(row_idx, dtype=np.int32)
    if row_idx.size == 0:
        row_idx = np.zeros(1, np.int32)
    Tc = col_ptr.size - 1
    ni, nm, ns = C.c_int32(0), C.c_int32(0), C.c_int32(0)
    lib = library()
    args = (col_ptr.ctypes.data, row_idx.ctypes.data, Tc, int(G), int(d), int(max_positions_per_item))
    _check(lib.bsattn_build_dkdv_schedule(*args, None, 0, None, 0, C.byref(ni), C.byref(nm), C.byref(ns)))
    items = np.zeros((ni.value, 8), np.int32)
    merges = np.zeros((max(1, nm.value), 3), np.int32)
    _check(lib.bsattn_build_dkdv_schedule(*args, items.ctypes.data, ni.value, merges.ctypes.data, merges.shape[0],
                                          C.byref(ni), C.byref(nm), C.byref(ns)))
    return KvSchedule(items, merges[:nm.value].copy(), ns.value)


class BwdSchedule:
    """The backward's two schedules: ``dq`` (a Schedule over the CSR) and
    ``kv`` (a KvSchedule over the CSC); either may be None."""

    def __init__(self, dq=None, kv=None):
        self.dq, self.kv = dq, kv

    def to(self, device):
        for s in (self.dq, self.kv):
            if s is not None and s.d_items is None:
                s.to(device)
        return self


def default_bwd_schedule(row_ptr, col_ptr, row_idx, B: int, Hq: int, Hkv: int, d: int,
                         slots: int = 512) -> BwdSchedule:
    """Chunk bounds of half the mean work per concurrent work-group slot: dQ
    as the forward's ``default_max_blocks_per_item``; dK/dV over the (head,
    tile) positions of every group of key blocks."""
    row_ptr = np.asarray(row_ptr, dtype=np.int32)
    dq = build_schedule(row_ptr, default_max_blocks_per_item(row_ptr, B, Hq, slots))
    G = Hq // Hkv
    probe = build_dkdv_schedule(col_ptr, row_idx, G, d, 1 << 30)   # one item per group: their sizes
    total = int((probe.items[:, 2] - probe.items[:, 1]).sum()) * B * Hkv
    kv = build_dkdv_schedule(col_ptr, row_idx, G, d, max(8, -(-total // (2 * slots))))
    return BwdSchedule(dq, kv)


def prefill_bwd_plan(q, k, v, out, dout, lse, *, scale: Optional[float] = None, causal: bool = False,
                     row_ptr=None, col_idx=None, col_ptr=None, row_idx=None, n_valid: int = 0,
                     dq=None, dk=None, dv=None, workspace=None, block_state=None,
                     schedule: Optional[BwdSchedule] = None) -> Plan:
    """Marshal a backward (arguments as ``prefill_bwd``) into a reusable Plan
    whose call returns (dq, dk, dv)."""
    torch = _torch()
    if q.dtype != torch.bfloat16:
        raise BsattnError(_abi.BSATTN_ERR_UNSUPPORTED, "the backward is implemented for bf16")
    B, Nq, Hq, d = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    sq = schedule.dq if schedule is not None else None
    sk = schedule.kv if schedule is not None else None
    if schedule is not None:
        schedule.to(q.device)
    if workspace is None:
        workspace = torch.empty(prefill_bwd_workspace_size(B, Hq, Hkv, Nq, d, sq.n_slots if sq else 0,
                                                           sk.n_slots if sk else 0),
                                dtype=torch.uint8, device=q.device)
    a = _abi.BwdArgs()
    a.dtype = _abi.BSATTN_BF16
    a.q, a.k, a.v, a.out, a.dout = _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout)
    a.lse, a.dq, a.dk, a.dv = _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv)
    a.B, a.Hq, a.Hkv, a.Nq, a.Nk, a.d = B, Hq, Hkv, Nq, Nk, d
    for fld, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("o_stride", out), ("do_stride", dout),
                   ("dq_stride", dq), ("dk_stride", dk), ("dv_stride", dv)):
        if t.dim() != 4 or t.stride(3) != 1:
            raise BsattnError(_abi.BSATTN_ERR_INVALID_ARG, f"{fld[:-7]} must be [B, N, H, d] with d contiguous")
        getattr(a, fld)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    col_idx, row_idx = _index_tensor(col_idx), _index_tensor(row_idx)
    a.row_ptr, a.col_idx, a.col_ptr, a.row_idx = _ptr(row_ptr), _ptr(col_idx), _ptr(col_ptr), _ptr(row_idx)
    a.n_valid = int(n_valid)
    a.scale = float(scale if scale is not None else 1.0 / math.sqrt(d))
    a.causal = 1 if causal else 0
    a.Br, a.Bc = 128, 64
    a.workspace = _ptr(workspace)
    a.workspace_bytes = int(workspace.numel() * workspace.element_size())
    a.block_state = _ptr(block_state)
    if sq is not None:
        a.dq_items, a.dq_n_items = _ptr(sq.d_items), sq.n_items
        a.dq_merges, a.dq_n_merges, a.dq_n_slots = _ptr(sq.d_merges), sq.n_merges, sq.n_slots
    if sk is not None:
        a.kv_items, a.kv_n_items = _ptr(sk.d_items), sk.n_items
        a.kv_merges, a.kv_n_merges, a.kv_n_slots = _ptr(sk.d_merges), sk.n_merges, sk.n_slots
    keep = (q, k, v, out, dout, lse, row_ptr, col_idx, col_ptr, row_idx, workspace, block_state, schedule)
    return Plan(library().bsattn_prefill_bwd, a, (dq, dk, dv), keep)


def prefill_bwd(q, k, v, out, dout, lse, *, scale: Optional[float] = None, causal: bool = False,
                row_ptr=None, col_idx=None, col_ptr=None, row_idx=None, n_valid: int = 0,
                dq=None, dk=None, dv=None, workspace=None, block_state=None, schedule=None, stream=None):
    """Gradients of the block-sparse forward for the loss
    sum(out * dout): q, out, dout [B, Nq, Hq, d], k, v [B, Nk, Hkv, d] bf16,
    ``lse`` float32 [B, Hq, Nq] from ``prefill_fwd(..., lse=)``.  The mask
    arguments are the forward's; with a CSR, ``col_ptr``/``row_idx`` are the
    device copies of ``transpose_block_index``.  ``workspace`` (uint8, at
    least ``prefill_bwd_workspace_size`` bytes) is allocated here if None.
    After a forward with lambda > 0, pass its ``block_state`` (uint8
    [B, Hq, Tr, Tc]): the blocks it skipped get no gradient.  ``schedule``
    (a BwdSchedule, e.g. ``default_bwd_schedule``) cuts long tiles and key
    blocks into chunks.  Returns (dq, dk, dv)."""
    return prefill_bwd_plan(q, k, v, out, dout, lse, scale=scale, causal=causal, row_ptr=row_ptr,
                            col_idx=col_idx, col_ptr=col_ptr, row_idx=row_idx, n_valid=n_valid, dq=dq, dk=dk,
                            dv=dv, workspace=workspace, block_state=block_state, schedule=schedule)(stream)


def decode_workspace_size(B: int, Hq: int, Hkv: int, L: int, d: int, Bc: int = 64, num_splits: int = 0) -> int:
    return int(library().bsattn_decode_workspace_size(B, Hq, Hkv, L, d, Bc, num_splits))


def decode_workspace(B: int, Hq: int, Hkv: int, L: int, d: int, device, Bc: int = 64, num_splits: int = 0):
    """A zero-filled decode workspace (the header's health word must start at
    zero; every call zeroes its tickets and flags, so calls of any shape can
    reuse it on one stream)."""
    torch = _torch()
    return torch.zeros(decode_workspace_size(B, Hq, Hkv, L, d, Bc, num_splits), dtype=torch.uint8, device=device)


def decode_num_splits(B: int, Hq: int, Hkv: int, L: int, d: int, Bc: int = 64, num_splits: int = 0) -> int:
    return int(library().bsattn_decode_num_splits(B, Hq, Hkv, L, d, Bc, num_splits))


def decode_split_blocks(B: int, Hq: int, Hkv: int, L: int, d: int, Bc: int = 64, num_splits: int = 0) -> int:
    """Key blocks per split (visiting positions [s n, (s + 1) n) form split s)."""
    return int(library().bsattn_decode_split_blocks(B, Hq, Hkv, L, d, Bc, num_splits))


def decode_plan(q, k_cache, v_cache, *, L: Optional[int] = None, scale: Optional[float] = None, lam: float = 0.0,
                Bc: int = 64, num_splits: int = 0, workspace=None, out=None, counters=None,
                block_state=None, order: str = "ascending", max_scope: str = "sequence",
                decisions: str = "group", noalloc: bool = False) -> Plan:
    """Marshal a decode (arguments as ``decode_fwd``) into a reusable Plan.
    ``noalloc=True`` marshals ``bsattn_decode_fwd_noalloc`` instead: no
    workspace (the library's fixed per-device scratch holds it; ``out`` must
    then be given for a call that may allocate nothing at all)."""
    torch = _torch()
    B, Hq, d = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    L = Lmax if L is None else int(L)
    if k_cache.stride() != v_cache.stride():
        raise BsattnError(_abi.BSATTN_ERR_INVALID_ARG, "k_cache and v_cache must share strides")
    if q.stride(2) != 1 or k_cache.stride(3) != 1:
        raise BsattnError(_abi.BSATTN_ERR_INVALID_ARG, "head dim must be contiguous")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=q.dtype, device=q.device)
    if noalloc and workspace is not None:
        raise BsattnError(_abi.BSATTN_ERR_INVALID_ARG, "the no-allocation decode takes no workspace")
    if workspace is None and not noalloc:
        workspace = decode_workspace(B, Hq, Hkv, L, d, q.device, Bc, num_splits)
    a = _abi.DecodeArgs()
    a.q, a.k_cache, a.v_cache, a.out = _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out)
    a.B, a.Hq, a.Hkv, a.L, a.Lmax, a.d = B, Hq, Hkv, L, Lmax, d
    a.q_stride[:] = [q.stride(0), q.stride(1)]
    a.kv_stride[:] = [k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)]
    a.o_stride[:] = [out.stride(0), out.stride(1)]
    a.scale = float(scale if scale is not None else 1.0 / math.sqrt(d))
    a.lam = float(lam)
    a.Bc = int(Bc)
    a.num_splits = int(num_splits)
    a.workspace = _ptr(workspace)
    a.workspace_bytes = 0 if workspace is None else int(workspace.numel() * workspace.element_size())
    a.counters, a.block_state = _ptr(counters), _ptr(block_state)
    a.block_order = _order_code(order)
    a.max_scope = _choice_code("max_scope", max_scope, ("sequence", "split"))
    a.decisions = _choice_code("decisions", decisions, ("group", "head"))
    keep = (q, k_cache, v_cache, workspace, counters, block_state)
    fn = library().bsattn_decode_fwd_noalloc if noalloc else library().bsattn_decode_fwd
    return Plan(fn, a, out, keep)


def decode_fwd(q, k_cache, v_cache, *, L: Optional[int] = None, scale: Optional[float] = None, lam: float = 0.0,
               Bc: int = 64, num_splits: int = 0, workspace=None, out=None, counters=None, block_state=None,
               order: str = "ascending", max_scope: str = "sequence", decisions: str = "group", noalloc: bool = False,
               stream=None):
    """BLASST decode: q [B, Hq, d] (token at position L-1), caches [B, Lmax, Hkv, d] bf16.

    ``workspace`` is a uint8 device tensor of at least
    ``decode_workspace_size`` bytes from ``decode_workspace`` (allocated here if None).
    ``max_scope="split"`` restarts the running max at every split and
    ``decisions="head"`` lets every query head decide for itself (variants;
    ``block_state`` is then [B, Hq, Tc]).  ``noalloc=True`` calls
    ``bsattn_decode_fwd_noalloc`` (no workspace; the library's per-device
    scratch, up to 32 MiB of workspace)."""
    return decode_plan(q, k_cache, v_cache, L=L, scale=scale, lam=lam, Bc=Bc, num_splits=num_splits,
                       workspace=workspace, out=out, counters=counters, block_state=block_state,
                       order=order, max_scope=max_scope, decisions=decisions, noalloc=noalloc)(stream)


def calibrate_fit(target: float, lengths, lambdas, sparsity, delta: float):
    """Algorithm 2's selection and fit on a measured table (C ABI):
    sparsity[k][i] measured at lengths[k] with lambdas[i].  Returns (a, n_points)."""
    lengths = np.ascontiguousarray(lengths, dtype=np.int32)
    lambdas = np.ascontiguousarray(lambdas, dtype=np.float64)
    table = np.ascontiguousarray(sparsity, dtype=np.float64).reshape(lengths.size, lambdas.size)
    a, n = C.c_double(0.0), C.c_int32(0)
    _check(library().bsattn_calibrate_threshold(float(target), lengths.ctypes.data, lengths.size, lambdas.ctypes.data,
                                                lambdas.size, table.ctypes.data, float(delta), C.byref(a),
                                                C.byref(n)))
    return float(a.value), int(n.value)


def calibrate(target: float, lengths, lambdas, delta: float, measure):
    """BLASST threshold calibration (notes section 3.2, Algorithm 2).

    ``measure(lam, L)`` returns the sparsity measured at context length L with
    threshold lam (for instance ``decode_sparsity`` on a sample of sequences
    of that length).  Returns (a, n_points, table): lambda(L) = a / L."""
    table = [[float(measure(lam, L)) for lam in lambdas] for L in lengths]
    a, n = calibrate_fit(target, lengths, lambdas, table, delta)
    return a, n, table


def decode_sparsity(q, k_cache, v_cache, *, lam: float, L: Optional[int] = None, scale: Optional[float] = None,
                    Bc: int = 64, order: str = "ascending") -> float:
    """Fraction of visited key blocks the decode kernel skips at threshold lam
    (synchronous: reads the kernel's skip counters back)."""
    torch = _torch()
    B, Hkv = q.shape[0], k_cache.shape[2]
    cnt = torch.zeros((B, Hkv, 2), dtype=torch.int32, device=q.device)
    decode_fwd(q, k_cache, v_cache, L=L, scale=scale, lam=lam, Bc=Bc, counters=cnt, order=order)
    c = cnt.view(-1, 2).sum(0).tolist()
    return c[1] / c[0] if c[0] else 0.0


def decode_check(workspace) -> int:
    """Health word of the last decode on this workspace (synchronous read and
    clear): 0 = fine.  ``None`` reads the no-allocation decode's scratch on
    the current device."""
    h = C.c_int32(0)
    _check(library().bsattn_decode_check(C.c_void_p(_ptr(workspace)), C.byref(h)))
    return int(h.value)
