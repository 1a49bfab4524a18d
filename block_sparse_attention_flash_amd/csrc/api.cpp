// C-ABI entry points of libbsattn: argument validation, error reporting and
// dispatch to the HIP kernels.  Nothing here allocates device memory or
// synchronises a stream (bsattn_decode_check aside, which is a documented
// synchronous read of one workspace word).

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"

namespace bsattn {

static thread_local char g_err[512] = {0};

bsattn_status fail(bsattn_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = 0; }

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static bsattn_status check_strides(const char* name, const int64_t* s, int n, int64_t vec) {
  for (int i = 0; i < n; ++i) {
    if (s[i] < 0) return fail(BSATTN_ERR_INVALID_ARG, "%s stride %d is negative", name, i);
    if (s[i] % vec != 0)
      return fail(BSATTN_ERR_UNSUPPORTED, "%s stride %d (%lld) must be a multiple of %lld elements", name, i,
                  (long long)s[i], (long long)vec);
  }
  return BSATTN_OK;
}

static bsattn_status hip_status(int e, const char* what) {
  if (e == 0) return BSATTN_OK;
  return fail(BSATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(static_cast<hipError_t>(e)));
}

// ---------------------------------------------------------------------------
// decode split policy and workspace layout
// ---------------------------------------------------------------------------

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

DecodeWorkspace decode_workspace_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t S) {
  DecodeWorkspace w{};
  const size_t units = (size_t)B * Hkv * S;
  const int32_t G = Hq / Hkv;
  size_t off = 0;
  w.header = off; off = align256(off + 16 * sizeof(int32_t));
  w.tickets = off; off = align256(off + (size_t)B * Hkv * sizeof(int32_t));
  w.flags = off;  off = align256(off + units * sizeof(int32_t));
  w.agg = off;    off = align256(off + units * 16 * sizeof(float));
  w.incl = off;   off = align256(off + units * 16 * sizeof(float));
  w.stats = off;  off = align256(off + units * G * 2 * sizeof(float));
  w.acc = off;    off = align256(off + units * G * (size_t)d * sizeof(float));
  w.counts = off; off = align256(off + units * sizeof(int32_t));
  w.total = off;
  return w;
}

PrefillWorkspace prefill_workspace_layout(int32_t B, int32_t Hq, int32_t d, int32_t n_slots) {
  PrefillWorkspace w{};
  const size_t units = (size_t)n_slots * B * Hq;
  size_t off = 0;
  w.o = off;   off = align256(off + units * 128 * (size_t)d * sizeof(float));
  w.ml = off;  off = align256(off + units * 128 * 2 * sizeof(float));
  w.cnt = off; off = align256(off + units * 4 * sizeof(int32_t));  // {visited, skipped, rows agreeing, -}
  w.arrive = off; off = align256(off + units * sizeof(int32_t));  // n_merges <= n_slots
  w.pre = off; off = align256(off + units * 128 * kPreSplit * sizeof(float));
  w.total = off;
  return w;
}

BwdWorkspace bwd_workspace_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t Nq, int32_t d, int32_t dq_n_slots,
                                  int32_t kv_n_slots) {
  BwdWorkspace w{};
  const int32_t NB = d == 64 ? kDkdvBlocks64 : kDkdvBlocks128;
  size_t off = 0;
  w.dvec = off;      off = align256(off + (size_t)B * Hq * Nq * sizeof(float));
  w.dq_part = off;   off = align256(off + (size_t)dq_n_slots * B * Hq * 128 * d * sizeof(float));
  w.dq_arrive = off; off = align256(off + (size_t)dq_n_slots * B * Hq * sizeof(int32_t));  // n_merges <= n_slots
  w.kv_part = off;   off = align256(off + (size_t)kv_n_slots * B * Hkv * NB * 64 * 2 * d * sizeof(float));
  w.kv_arrive = off; off = align256(off + (size_t)kv_n_slots * B * Hkv * sizeof(int32_t));
  w.total = off;
  return w;
}

// Largest split (in Bc-blocks): the kernel's skip mask is one 64-bit word.
static int32_t max_blocks_per_split(int32_t G) {
  (void)G;
  return 64;
}

int32_t decode_choose_splits(int32_t B, int32_t Hkv, int32_t Tc, int32_t G, int32_t requested,
                             int32_t* blocks_per_split) {
  const int32_t cap = max_blocks_per_split(G);
  int32_t bps;
  if (requested > 0) {
    int32_t S = requested < Tc ? requested : Tc;
    bps = (Tc + S - 1) / S;
  } else {
    // aim for at least ~2048 split work-groups (8 per CU on 256 CUs), splits of 2..7/8 of the
    // cap blocks (longer splits stream K longer between the latency-bound look-back and V
    // phases; on the 131K-key, 8-head decode, splits of exactly 64 blocks measured about 2 %
    // slower than any length from 54 to 61, so the automatic length stops at 56)
    const int32_t auto_cap = cap - cap / 8;
    int64_t want = ((int64_t)Tc * B * Hkv + 2047) / 2048;
    bps = (int32_t)(want < 2 ? 2 : (want > auto_cap ? auto_cap : want));
  }
  if (bps > cap) bps = cap;
  if (bps < 1) bps = 1;
  *blocks_per_split = bps;
  return (Tc + bps - 1) / bps;
}

bool prefill_group_major(int B, int Hq, int Hkv, int d, int64_t units) {
  // groups divide into the 8 XCDs, and one XCD (32 CUs) has at least four
  // waves of resident work-groups
  if (((int64_t)B * Hkv) % 8 != 0) return false;
  const int64_t grid = (int64_t)B * Hq * units;
  return grid / 8 >= 4 * 32 * (d == 64 ? kPrefillWgPerCu64 : kPrefillWgPerCu128);
}

}  // namespace bsattn

using namespace bsattn;

extern "C" {

const char* bsattn_status_string(int status) {
  switch (status) {
    case BSATTN_OK: return "BSATTN_OK";
    case BSATTN_ERR_INVALID_ARG: return "BSATTN_ERR_INVALID_ARG";
    case BSATTN_ERR_UNSUPPORTED: return "BSATTN_ERR_UNSUPPORTED";
    case BSATTN_ERR_CAPACITY: return "BSATTN_ERR_CAPACITY";
    case BSATTN_ERR_HIP: return "BSATTN_ERR_HIP";
    default: return "BSATTN_ERR_UNKNOWN";
  }
}

const char* bsattn_last_error(void) { return g_err; }

int bsattn_version(void) { return 0x000100; }

bsattn_status bsattn_prefill_fwd(const bsattn_prefill_args* a, void* stream) {
  clear_error();
  if (!a) return fail(BSATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != BSATTN_BF16 && a->dtype != BSATTN_FP32)
    return fail(BSATTN_ERR_UNSUPPORTED, "dtype %d not supported", a->dtype);
  if (!a->q || !a->k || !a->v || !a->out) return fail(BSATTN_ERR_INVALID_ARG, "q, k, v, out must be non-NULL");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out))
    return fail(BSATTN_ERR_UNSUPPORTED, "q, k, v, out must be 16-byte aligned");
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Nq < 1 || a->Nk < 1)
    return fail(BSATTN_ERR_INVALID_ARG, "B, Hq, Hkv, Nq, Nk must be >= 1");
  if (a->Hq % a->Hkv != 0) return fail(BSATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", a->Hq, a->Hkv);
  if (a->d != 64 && a->d != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head dim %d not supported (64, 128)", a->d);
  const int64_t vec = a->dtype == BSATTN_BF16 ? 8 : 4;
  bsattn_status st;
  if ((st = check_strides("q", a->q_stride, 3, vec)) != BSATTN_OK) return st;
  if ((st = check_strides("k", a->k_stride, 3, vec)) != BSATTN_OK) return st;
  if ((st = check_strides("v", a->v_stride, 3, vec)) != BSATTN_OK) return st;
  if ((st = check_strides("out", a->o_stride, 3, vec)) != BSATTN_OK) return st;
  if ((a->row_ptr == nullptr) != (a->col_idx == nullptr))
    return fail(BSATTN_ERR_INVALID_ARG, "row_ptr and col_idx must both be set or both be NULL");
  if (!(a->scale > 0.0f) || !std::isfinite(a->scale)) return fail(BSATTN_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!(a->lambda >= 0.0f && a->lambda < 1.0f)) return fail(BSATTN_ERR_INVALID_ARG, "lambda must lie in [0, 1)");
  if (a->causal && a->Nq != a->Nk) return fail(BSATTN_ERR_INVALID_ARG, "causal attention requires Nq == Nk");
  if (a->n_valid < 0 || a->n_valid > a->Nk) return fail(BSATTN_ERR_INVALID_ARG, "n_valid must lie in [0, Nk]");
  if (a->Bc != 64) return fail(BSATTN_ERR_UNSUPPORTED, "Bc must be 64");
  if (a->dtype == BSATTN_BF16 && a->Br != 128) return fail(BSATTN_ERR_UNSUPPORTED, "bf16 path needs Br = 128");
  if (a->dtype == BSATTN_FP32 && a->Br != 64 && a->Br != 128)
    return fail(BSATTN_ERR_UNSUPPORTED, "fp32 path needs Br in {64, 128}");
  if (a->dtype == BSATTN_BF16) {
    // the bf16 kernel addresses one head's K/V rows with 32-bit byte offsets
    const int64_t lim = 0xffffffffLL;
    if (((int64_t)a->Nk + 64) * a->k_stride[1] * 2 > lim || ((int64_t)a->Nk + 64) * a->v_stride[1] * 2 > lim)
      return fail(BSATTN_ERR_UNSUPPORTED, "bf16 path: (Nk + 64) * token stride must stay below 4 GiB per head");
  }
  PrefillParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.out = a->out;
  p.B = a->B; p.Hq = a->Hq; p.Hkv = a->Hkv; p.Nq = a->Nq; p.Nk = a->Nk; p.d = a->d;
  p.qs_b = a->q_stride[0]; p.qs_t = a->q_stride[1]; p.qs_h = a->q_stride[2];
  p.ks_b = a->k_stride[0]; p.ks_t = a->k_stride[1]; p.ks_h = a->k_stride[2];
  p.vs_b = a->v_stride[0]; p.vs_t = a->v_stride[1]; p.vs_h = a->v_stride[2];
  p.os_b = a->o_stride[0]; p.os_t = a->o_stride[1]; p.os_h = a->o_stride[2];
  p.row_ptr = a->row_ptr; p.col_idx = a->col_idx; p.tile_order = a->tile_order;
  p.n_valid = a->n_valid == 0 ? a->Nk : a->n_valid;
  p.scale = a->scale; p.lambda = a->lambda; p.causal = a->causal ? 1 : 0;
  p.Br = a->Br; p.Bc = a->Bc;
  p.Tr = (a->Nq + a->Br - 1) / a->Br;
  p.Tc = (a->Nk + a->Bc - 1) / a->Bc;
  p.tile_counters = a->tile_counters; p.block_state = a->block_state;
  p.row_counters = a->row_counters;
  p.lse = a->lse;
  if (a->block_order != 0 && a->block_order != 1) return fail(BSATTN_ERR_INVALID_ARG, "block_order must be 0 or 1");
  p.block_order = a->block_order;
  if (a->sched_items) {
    if (a->dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "schedules are implemented for the bf16 path");
    if (!a->row_ptr) return fail(BSATTN_ERR_INVALID_ARG, "a schedule needs the CSR (row_ptr, col_idx)");
    if (a->n_items < 1) return fail(BSATTN_ERR_INVALID_ARG, "n_items must be >= 1");
    if (a->n_slots < 0 || a->n_merges < 0 || (a->n_merges > 0) != (a->n_slots > 0) || (a->n_merges > 0 && !a->sched_merges) ||
        a->n_merges > a->n_slots)
      return fail(BSATTN_ERR_INVALID_ARG, "inconsistent schedule counts (n_merges, n_slots, sched_merges)");
    if (a->n_slots > 0) {
      const PrefillWorkspace w = prefill_workspace_layout(a->B, a->Hq, a->d, a->n_slots);
      if (!a->workspace || (reinterpret_cast<uintptr_t>(a->workspace) & 255u))
        return fail(BSATTN_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
      if (a->workspace_bytes < w.total)
        return fail(BSATTN_ERR_CAPACITY, "workspace_bytes %zu < required %zu", a->workspace_bytes, w.total);
      char* ws = static_cast<char*>(a->workspace);
      p.part_o = reinterpret_cast<float*>(ws + w.o);
      p.part_ml = reinterpret_cast<float*>(ws + w.ml);
      p.part_cnt = reinterpret_cast<int32_t*>(ws + w.cnt);
      p.arrive = reinterpret_cast<int32_t*>(ws + w.arrive);
      p.part_pre = reinterpret_cast<float*>(ws + w.pre);
    }
    p.sched_items = a->sched_items; p.n_items = a->n_items;
    p.sched_merges = a->sched_merges; p.n_merges = a->n_merges; p.n_slots = a->n_slots;
  }
  const int64_t units = p.sched_items ? p.n_items : p.Tr;
  if ((int64_t)p.B * p.Hq * units > 0x7fffffffLL) return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
  int e = a->dtype == BSATTN_BF16 ? launch_prefill_bf16(p, stream) : launch_prefill_f32(p, stream);
  return hip_status(e, "prefill launch");
}

size_t bsattn_prefill_bwd_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t Nq, int32_t d,
                                         int32_t dq_n_slots, int32_t kv_n_slots) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || (d != 64 && d != 128) || dq_n_slots < 0 || kv_n_slots < 0) return 0;
  return bwd_workspace_layout(B, Hq, Hkv, Nq, d, dq_n_slots, kv_n_slots).total;
}

bsattn_status bsattn_prefill_bwd(const bsattn_prefill_bwd_args* a, void* stream) {
  clear_error();
  if (!a) return fail(BSATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->dtype != BSATTN_BF16) return fail(BSATTN_ERR_UNSUPPORTED, "the backward is implemented for bf16");
  const void* ptrs[] = {a->q, a->k, a->v, a->out, a->dout, a->dq, a->dk, a->dv};
  for (const void* x : ptrs) {
    if (!x) return fail(BSATTN_ERR_INVALID_ARG, "q, k, v, out, dout, dq, dk, dv must be non-NULL");
    if (!aligned16(x)) return fail(BSATTN_ERR_UNSUPPORTED, "q, k, v, out, dout, dq, dk, dv must be 16-byte aligned");
  }
  if (!a->lse || (reinterpret_cast<uintptr_t>(a->lse) & 3u)) return fail(BSATTN_ERR_INVALID_ARG, "lse must be a non-NULL float array");
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->Nq < 1 || a->Nk < 1)
    return fail(BSATTN_ERR_INVALID_ARG, "B, Hq, Hkv, Nq, Nk must be >= 1");
  if (a->Hq % a->Hkv != 0) return fail(BSATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", a->Hq, a->Hkv);
  if (a->d != 64 && a->d != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head dim %d not supported (64, 128)", a->d);
  bsattn_status st;
  const struct { const char* n; const int64_t* s; } strides[] = {
      {"q", a->q_stride},   {"k", a->k_stride},   {"v", a->v_stride},   {"out", a->o_stride},
      {"dout", a->do_stride}, {"dq", a->dq_stride}, {"dk", a->dk_stride}, {"dv", a->dv_stride}};
  for (const auto& x : strides)
    if ((st = check_strides(x.n, x.s, 3, 8)) != BSATTN_OK) return st;
  if ((a->row_ptr == nullptr) != (a->col_idx == nullptr) || (a->row_ptr == nullptr) != (a->col_ptr == nullptr) ||
      (a->row_ptr == nullptr) != (a->row_idx == nullptr))
    return fail(BSATTN_ERR_INVALID_ARG, "row_ptr, col_idx, col_ptr, row_idx must all be set or all be NULL");
  if (!(a->scale > 0.0f) || !std::isfinite(a->scale)) return fail(BSATTN_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (a->causal && a->Nq != a->Nk) return fail(BSATTN_ERR_INVALID_ARG, "causal attention requires Nq == Nk");
  if (a->n_valid < 0 || a->n_valid > a->Nk) return fail(BSATTN_ERR_INVALID_ARG, "n_valid must lie in [0, Nk]");
  if (a->Br != 128 || a->Bc != 64) return fail(BSATTN_ERR_UNSUPPORTED, "the backward needs Br = 128, Bc = 64");
  if (!a->workspace || (reinterpret_cast<uintptr_t>(a->workspace) & 255u))
    return fail(BSATTN_ERR_INVALID_ARG, "workspace must be non-NULL and 256-byte aligned");
  // schedules: both need the block index; counts consistent with their arrays
  if (a->dq_items) {
    if (!a->row_ptr) return fail(BSATTN_ERR_INVALID_ARG, "a dQ schedule needs the CSR");
    if (a->dq_n_items < 1 || a->dq_n_merges < 0 || a->dq_n_slots < a->dq_n_merges || (a->dq_n_merges > 0) != (a->dq_merges != nullptr) ||
        (a->dq_n_slots > 0) != (a->dq_n_merges > 0))
      return fail(BSATTN_ERR_INVALID_ARG, "dQ schedule counts inconsistent (items %d, merges %d, slots %d)",
                  a->dq_n_items, a->dq_n_merges, a->dq_n_slots);
  } else if (a->dq_n_items || a->dq_n_merges || a->dq_n_slots || a->dq_merges) {
    return fail(BSATTN_ERR_INVALID_ARG, "dQ schedule counts or merges without items");
  }
  if (a->kv_items) {
    if (!a->col_ptr) return fail(BSATTN_ERR_INVALID_ARG, "a dK/dV schedule needs the CSC");
    if (a->kv_n_items < 1 || a->kv_n_merges < 0 || a->kv_n_slots < a->kv_n_merges || (a->kv_n_merges > 0) != (a->kv_merges != nullptr) ||
        (a->kv_n_slots > 0) != (a->kv_n_merges > 0))
      return fail(BSATTN_ERR_INVALID_ARG, "dK/dV schedule counts inconsistent (items %d, merges %d, slots %d)",
                  a->kv_n_items, a->kv_n_merges, a->kv_n_slots);
  } else if (a->kv_n_items || a->kv_n_merges || a->kv_n_slots || a->kv_merges) {
    return fail(BSATTN_ERR_INVALID_ARG, "dK/dV schedule counts or merges without items");
  }
  const int32_t dq_slots = a->dq_items ? a->dq_n_slots : 0, kv_slots = a->kv_items ? a->kv_n_slots : 0;
  const BwdWorkspace w = bwd_workspace_layout(a->B, a->Hq, a->Hkv, a->Nq, a->d, dq_slots, kv_slots);
  if (a->workspace_bytes < w.total)
    return fail(BSATTN_ERR_CAPACITY, "workspace_bytes %zu < required %zu", a->workspace_bytes, w.total);
  BwdParams p{};
  p.q = a->q; p.k = a->k; p.v = a->v; p.out = a->out; p.dout = a->dout; p.lse = a->lse;
  p.dq = a->dq; p.dk = a->dk; p.dv = a->dv;
  char* ws = static_cast<char*>(a->workspace);
  p.dvec = reinterpret_cast<float*>(ws + w.dvec);
  if (a->dq_items) {
    p.dq_items = a->dq_items; p.dq_n_items = a->dq_n_items;
    p.dq_merges = a->dq_merges; p.dq_n_merges = a->dq_n_merges;
    p.dq_part = reinterpret_cast<float*>(ws + w.dq_part);
    p.dq_arrive = reinterpret_cast<int32_t*>(ws + w.dq_arrive);
  }
  if (a->kv_items) {
    p.kv_items = a->kv_items; p.kv_n_items = a->kv_n_items;
    p.kv_merges = a->kv_merges; p.kv_n_merges = a->kv_n_merges;
    p.kv_part = reinterpret_cast<float*>(ws + w.kv_part);
    p.kv_arrive = reinterpret_cast<int32_t*>(ws + w.kv_arrive);
  }
  p.B = a->B; p.Hq = a->Hq; p.Hkv = a->Hkv; p.Nq = a->Nq; p.Nk = a->Nk; p.d = a->d;
  p.qs_b = a->q_stride[0]; p.qs_t = a->q_stride[1]; p.qs_h = a->q_stride[2];
  p.ks_b = a->k_stride[0]; p.ks_t = a->k_stride[1]; p.ks_h = a->k_stride[2];
  p.vs_b = a->v_stride[0]; p.vs_t = a->v_stride[1]; p.vs_h = a->v_stride[2];
  p.os_b = a->o_stride[0]; p.os_t = a->o_stride[1]; p.os_h = a->o_stride[2];
  p.dos_b = a->do_stride[0]; p.dos_t = a->do_stride[1]; p.dos_h = a->do_stride[2];
  p.dqs_b = a->dq_stride[0]; p.dqs_t = a->dq_stride[1]; p.dqs_h = a->dq_stride[2];
  p.dks_b = a->dk_stride[0]; p.dks_t = a->dk_stride[1]; p.dks_h = a->dk_stride[2];
  p.dvs_b = a->dv_stride[0]; p.dvs_t = a->dv_stride[1]; p.dvs_h = a->dv_stride[2];
  p.row_ptr = a->row_ptr; p.col_idx = a->col_idx; p.col_ptr = a->col_ptr; p.row_idx = a->row_idx;
  p.n_valid = a->n_valid == 0 ? a->Nk : a->n_valid;
  p.scale = a->scale;
  p.causal = a->causal ? 1 : 0;
  p.Tr = (a->Nq + 127) / 128;
  p.Tc = (a->Nk + 63) / 64;
  p.block_state = a->block_state;
  if ((int64_t)p.B * p.Hq * std::max(p.Tr, p.dq_n_items) > 0x7fffffffLL ||
      (int64_t)p.B * p.Hkv * std::max(p.Tc, p.kv_n_items) > 0x7fffffffLL || (int64_t)p.B * p.Hq * p.Nq > 0x7fffffffLL)
    return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
  return hip_status(launch_prefill_bwd(p, stream), "prefill backward launch");
}

int32_t bsattn_prefill_group_major(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t n_units) {
  if (B < 1 || Hq < 1 || Hkv < 1 || n_units < 1 || Hq % Hkv || (d != 64 && d != 128)) return -1;
  return prefill_group_major(B, Hq, Hkv, d, n_units) ? 1 : 0;
}

size_t bsattn_prefill_workspace_size(int32_t B, int32_t Hq, int32_t d, int32_t n_slots) {
  if (B < 1 || Hq < 1 || d < 1 || n_slots < 0) return 0;
  return prefill_workspace_layout(B, Hq, d, n_slots).total;
}

size_t bsattn_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t L, int32_t d, int32_t Bc,
                                    int32_t num_splits) {
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || d < 1 || Bc < 1 || Hq % Hkv) return 0;
  int32_t bps;
  int32_t Tc = (L + Bc - 1) / Bc;
  int32_t S = decode_choose_splits(B, Hkv, Tc, Hq / Hkv, num_splits, &bps);
  return decode_workspace_layout(B, Hq, Hkv, d, S).total;
}

int32_t bsattn_decode_num_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t L, int32_t d, int32_t Bc,
                                 int32_t num_splits) {
  (void)d;
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || Bc < 1 || Hq % Hkv) return 0;
  int32_t bps;
  return decode_choose_splits(B, Hkv, (L + Bc - 1) / Bc, Hq / Hkv, num_splits, &bps);
}

int32_t bsattn_decode_split_blocks(int32_t B, int32_t Hq, int32_t Hkv, int32_t L, int32_t d, int32_t Bc,
                                   int32_t num_splits) {
  (void)d;
  if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || Bc < 1 || Hq % Hkv) return 0;
  int32_t bps;
  decode_choose_splits(B, Hkv, (L + Bc - 1) / Bc, Hq / Hkv, num_splits, &bps);
  return bps;
}

// Validation and parameters shared by the decode entry points (the
// workspace itself is checked by each caller).
static bsattn_status decode_prepare(const bsattn_decode_args* a, DecodeParams& p, DecodeWorkspace& w) {
  if (!a->q || !a->k_cache || !a->v_cache || !a->out)
    return fail(BSATTN_ERR_INVALID_ARG, "q, k_cache, v_cache, out must be non-NULL");
  if (!aligned16(a->q) || !aligned16(a->k_cache) || !aligned16(a->v_cache) || !aligned16(a->out))
    return fail(BSATTN_ERR_UNSUPPORTED, "q, k_cache, v_cache, out must be 16-byte aligned");
  if (a->B < 1 || a->Hq < 1 || a->Hkv < 1 || a->L < 1 || a->Lmax < a->L)
    return fail(BSATTN_ERR_INVALID_ARG, "need B, Hq, Hkv >= 1 and 1 <= L <= Lmax");
  if (a->Hq % a->Hkv != 0) return fail(BSATTN_ERR_INVALID_ARG, "Hq (%d) must be a multiple of Hkv (%d)", a->Hq, a->Hkv);
  const int32_t G = a->Hq / a->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(BSATTN_ERR_UNSUPPORTED, "Hq/Hkv = %d not supported (1, 2, 4, 8)", G);
  if (a->d != 64 && a->d != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head dim %d not supported (64, 128)", a->d);
  if (a->Bc != 64) return fail(BSATTN_ERR_UNSUPPORTED, "Bc must be 64");
  if (!(a->scale > 0.0f) || !std::isfinite(a->scale)) return fail(BSATTN_ERR_INVALID_ARG, "scale must be finite and > 0");
  if (!(a->lambda >= 0.0f && a->lambda < 1.0f)) return fail(BSATTN_ERR_INVALID_ARG, "lambda must lie in [0, 1)");
  if (a->num_splits < 0) return fail(BSATTN_ERR_INVALID_ARG, "num_splits must be >= 0");
  bsattn_status st;
  if ((st = check_strides("q", a->q_stride, 2, 8)) != BSATTN_OK) return st;
  if ((st = check_strides("kv", a->kv_stride, 3, 8)) != BSATTN_OK) return st;
  if ((st = check_strides("out", a->o_stride, 2, 8)) != BSATTN_OK) return st;
  p = DecodeParams{};
  p.q = a->q; p.k = a->k_cache; p.v = a->v_cache; p.out = a->out;
  p.B = a->B; p.Hq = a->Hq; p.Hkv = a->Hkv; p.L = a->L; p.d = a->d; p.G = G;
  p.qs_b = a->q_stride[0]; p.qs_h = a->q_stride[1];
  p.ks_b = a->kv_stride[0]; p.ks_t = a->kv_stride[1]; p.ks_h = a->kv_stride[2];
  p.os_b = a->o_stride[0]; p.os_h = a->o_stride[1];
  p.scale = a->scale; p.lambda = a->lambda; p.Bc = a->Bc;
  p.Tc = (a->L + a->Bc - 1) / a->Bc;
  p.num_splits = decode_choose_splits(a->B, a->Hkv, p.Tc, G, a->num_splits, &p.blocks_per_split);
  if (a->block_order != 0 && a->block_order != 1) return fail(BSATTN_ERR_INVALID_ARG, "block_order must be 0 or 1");
  w = decode_workspace_layout(a->B, a->Hq, a->Hkv, a->d, p.num_splits);
  if ((int64_t)a->B * a->Hkv * p.num_splits > 0x7fffffffLL) return fail(BSATTN_ERR_UNSUPPORTED, "grid too large");
  p.counters = a->counters; p.block_state = a->block_state;
  p.block_order = a->block_order;
  if (a->max_scope != 0 && a->max_scope != 1) return fail(BSATTN_ERR_INVALID_ARG, "max_scope must be 0 or 1");
  if (a->decisions != 0 && a->decisions != 1) return fail(BSATTN_ERR_INVALID_ARG, "decisions must be 0 or 1");
  p.split_reset = a->max_scope;
  p.per_head = a->decisions;
  return BSATTN_OK;
}

bsattn_status bsattn_decode_fwd(const bsattn_decode_args* a, void* stream) {
  clear_error();
  if (!a) return fail(BSATTN_ERR_INVALID_ARG, "args is NULL");
  if (!a->workspace) return fail(BSATTN_ERR_INVALID_ARG, "workspace must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(a->workspace) & 255u) != 0)
    return fail(BSATTN_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  DecodeParams p;
  DecodeWorkspace w;
  bsattn_status st = decode_prepare(a, p, w);
  if (st != BSATTN_OK) return st;
  if (a->workspace_bytes < w.total)
    return fail(BSATTN_ERR_CAPACITY, "workspace_bytes %zu < required %zu", a->workspace_bytes, w.total);
  p.workspace = a->workspace;
  return hip_status(launch_decode(p, stream), "decode launch");
}

bsattn_status bsattn_decode_fwd_noalloc(const bsattn_decode_args* a, void* stream) {
  clear_error();
  if (!a) return fail(BSATTN_ERR_INVALID_ARG, "args is NULL");
  if (a->workspace || a->workspace_bytes)
    return fail(BSATTN_ERR_INVALID_ARG, "the no-allocation decode takes no workspace (workspace must be NULL, "
                                        "workspace_bytes 0)");
  DecodeParams p;
  DecodeWorkspace w;
  bsattn_status st = decode_prepare(a, p, w);
  if (st != BSATTN_OK) return st;
  if (w.total > kNoAllocScratchBytes)
    return fail(BSATTN_ERR_CAPACITY, "this decode needs %zu bytes of scratch; the no-allocation call has %zu "
                "(fewer splits, sequences or heads per call fit)", w.total, kNoAllocScratchBytes);
  void* ptr = nullptr;
  const int e = noalloc_scratch(&ptr);
  if (e != 0) return hip_status(e, "no-allocation scratch lookup");
  p.workspace = ptr;
  return hip_status(launch_decode(p, stream), "decode launch");
}

bsattn_status bsattn_decode_check(void* workspace, int32_t* health_out) {
  clear_error();
  if (!health_out) return fail(BSATTN_ERR_INVALID_ARG, "health_out must be non-NULL");
  if (!workspace) {  // the no-allocation decode's scratch on the current device
    const int e = noalloc_scratch(&workspace);
    if (e != 0) return hip_status(e, "no-allocation scratch lookup");
  }
  int32_t h = 0;
  char* word = static_cast<char*>(workspace) + sizeof(int32_t);
  hipError_t e = hipMemcpy(&h, word, sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "hipMemcpy: %s", hipGetErrorString(e));
  if (h != 0) {
    const int32_t zero = 0;
    e = hipMemcpy(word, &zero, sizeof(int32_t), hipMemcpyHostToDevice);
    if (e != hipSuccess) return fail(BSATTN_ERR_HIP, "hipMemcpy: %s", hipGetErrorString(e));
  }
  *health_out = h;
  return BSATTN_OK;
}

}  // extern "C"
