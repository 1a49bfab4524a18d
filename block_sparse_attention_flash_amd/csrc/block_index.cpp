// Host-side block-index builder: mask specification -> per-query-tile CSR.
//
// DiT block-sparse article, section 2.1 (local window, per-modality block
// diagonal, global + local anchors), section 2.3 (0/1 matrix over a block
// grid stored as a sparse index) and section 3.2 (segments -> per-pair rule
// -> block matrix).  Section 5.2 warns against per-element loops; this
// builder never enumerates token pairs.  It splits each query tile into
// runs of query tokens that share a segment, a frame and a patch row, turns
// each run into the exact union of the key-token intervals its tokens may
// attend, and marks the key blocks those intervals touch.  Cost is
// O(tiles * (runs * window rows + Tc / 64)), i.e. microseconds to a few
// milliseconds for a 66K-token video sequence.

#include <algorithm>
#include <iterator>
#include <cstdint>
#include <cstring>
#include <vector>

#include "internal.h"

namespace bsattn {
namespace {

struct BlockSet {
  std::vector<uint64_t> words;
  int32_t Bc = 1;
  int32_t Tc = 0;
  void reset(int32_t tc, int32_t bc) {
    Tc = tc;
    Bc = bc;
    words.assign((tc + 63) / 64, 0ull);
  }
  // mark every block touched by key tokens [lo, hi)
  void mark_tokens(int64_t lo, int64_t hi) {
    if (lo >= hi) return;
    int64_t b0 = lo / Bc, b1 = (hi - 1) / Bc;
    if (b1 >= Tc) b1 = Tc - 1;
    for (int64_t b = b0; b <= b1;) {
      int64_t w = b >> 6, bit = b & 63;
      int64_t span = std::min<int64_t>(64 - bit, b1 - b + 1);
      uint64_t m = (span == 64) ? ~0ull : (((1ull << span) - 1ull) << bit);
      words[w] |= m;
      b += span;
    }
  }
};

int64_t clampi(int64_t x, int64_t lo, int64_t hi) { return x < lo ? lo : (x > hi ? hi : x); }

// Key intervals for query tokens [a, b) of one segment (a, b absolute; the
// run never crosses a frame or a patch row for the grid kinds).
void mark_run(const bsattn_segment& s, int64_t a, int64_t b, BlockSet& set) {
  const int64_t st = s.start, len = s.len;
  switch (s.kind) {
    case BSATTN_SEG_FULL:
      set.mark_tokens(st, st + len);
      return;
    case BSATTN_SEG_BLOCKWIN: {
      int64_t u0 = (a - st) / s.unit, u1 = (b - 1 - st) / s.unit;
      int64_t nu = (len + s.unit - 1) / s.unit;
      int64_t lo = clampi(u0 - s.radius, 0, nu - 1), hi = clampi(u1 + s.radius, 0, nu - 1);
      set.mark_tokens(st + lo * s.unit, std::min<int64_t>(st + (hi + 1) * s.unit, st + len));
      return;
    }
    case BSATTN_SEG_IMAGE2D:
    case BSATTN_SEG_VIDEO3D: {
      const int64_t W = s.grid_w, H = s.grid_h, fs = W * H;
      int64_t off_a = a - st, off_b = b - 1 - st;
      int64_t f = off_a / fs;
      int64_t pa = off_a % fs, pb = off_b % fs;  // same frame and same row by construction
      int64_t r = pa / W, c0 = pa % W, c1 = pb % W;
      // same-frame 2-D window: rows r-R..r+R, columns c0-R..c1+R
      int64_t rlo = clampi(r - s.radius, 0, H - 1), rhi = clampi(r + s.radius, 0, H - 1);
      int64_t clo = clampi(c0 - s.radius, 0, W - 1), chi = clampi(c1 + s.radius, 0, W - 1);
      int64_t fbase = st + f * fs;
      if (clo == 0 && chi == W - 1) {
        set.mark_tokens(fbase + rlo * W, fbase + (rhi + 1) * W);
      } else {
        for (int64_t rr = rlo; rr <= rhi; ++rr) set.mark_tokens(fbase + rr * W + clo, fbase + rr * W + chi + 1);
      }
      if (s.kind == BSATTN_SEG_VIDEO3D && s.t_radius > 0) {
        // neighbouring frames: the spatial units covered by the run
        int64_t ulo = pa / s.unit, uhi = pb / s.unit;
        int64_t klo = ulo * s.unit, khi = std::min<int64_t>((uhi + 1) * s.unit, fs);
        for (int64_t df = -s.t_radius; df <= s.t_radius; ++df) {
          int64_t ff = f + df;
          if (df == 0 || ff < 0 || ff >= s.frames) continue;
          set.mark_tokens(st + ff * fs + klo, st + ff * fs + khi);
        }
      }
      return;
    }
    default:
      return;
  }
}

// Split [a, b) (inside segment s) into runs on which mark_run's assumptions hold.
void mark_segment_part(const bsattn_segment& s, int64_t a, int64_t b, BlockSet& set) {
  if (s.kind == BSATTN_SEG_FULL) {
    mark_run(s, a, b, set);
    return;
  }
  if (s.kind == BSATTN_SEG_BLOCKWIN) {
    mark_run(s, a, b, set);
    return;
  }
  const int64_t W = s.grid_w;
  for (int64_t x = a; x < b;) {
    int64_t off = x - s.start;
    int64_t row_end = s.start + (off / W + 1) * W;  // next patch row (also a frame boundary)
    int64_t y = std::min<int64_t>(b, row_end);
    mark_run(s, x, y, set);
    x = y;
  }
}

}  // namespace

bsattn_status validate_spec(const bsattn_mask_spec* spec, int32_t n_k) {
  if (!spec) return fail(BSATTN_ERR_INVALID_ARG, "spec is NULL");
  if (spec->n_valid < 0 || spec->n_valid > n_k)
    return fail(BSATTN_ERR_INVALID_ARG, "n_valid must lie in [0, n_k]");
  if (spec->n_segments < 0 || (spec->n_segments > 0 && !spec->segments))
    return fail(BSATTN_ERR_INVALID_ARG, "segments pointer is NULL");
  if (spec->anchor_len < 0 || spec->anchor_start < 0 ||
      (spec->anchor_len > 0 && (int64_t)spec->anchor_start + spec->anchor_len > spec->n_valid))
    return fail(BSATTN_ERR_INVALID_ARG, "anchors must lie inside [0, n_valid)");
  std::vector<std::pair<int64_t, int64_t>> spans;
  for (int32_t i = 0; i < spec->n_segments; ++i) {
    const bsattn_segment& s = spec->segments[i];
    if (s.start < 0 || s.len <= 0 || (int64_t)s.start + s.len > spec->n_valid)
      return fail(BSATTN_ERR_INVALID_ARG, "segment %d must lie inside [0, n_valid) and be non-empty", i);
    if (s.radius < 0 || s.t_radius < 0) return fail(BSATTN_ERR_INVALID_ARG, "segment %d: negative radius", i);
    switch (s.kind) {
      case BSATTN_SEG_FULL:
        break;
      case BSATTN_SEG_BLOCKWIN:
        if (s.unit <= 0) return fail(BSATTN_ERR_INVALID_ARG, "segment %d: unit must be positive", i);
        break;
      case BSATTN_SEG_IMAGE2D:
        if (s.grid_h <= 0 || s.grid_w <= 0 || (int64_t)s.grid_h * s.grid_w != s.len)
          return fail(BSATTN_ERR_INVALID_ARG, "segment %d: len must equal grid_h * grid_w", i);
        break;
      case BSATTN_SEG_VIDEO3D:
        if (s.frames <= 0 || s.grid_h <= 0 || s.grid_w <= 0 || s.unit <= 0 ||
            (int64_t)s.frames * s.grid_h * s.grid_w != s.len)
          return fail(BSATTN_ERR_INVALID_ARG, "segment %d: len must equal frames * grid_h * grid_w, unit > 0", i);
        break;
      default:
        return fail(BSATTN_ERR_INVALID_ARG, "segment %d: unknown kind %d", i, s.kind);
    }
    spans.push_back({s.start, (int64_t)s.start + s.len});
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second) return fail(BSATTN_ERR_INVALID_ARG, "segments overlap");
  return BSATTN_OK;
}

bsattn_status build_block_index(const bsattn_mask_spec* spec, int32_t n_q, int32_t n_k, int32_t Br,
                                int32_t Bc, std::vector<int32_t>& row_ptr, std::vector<int32_t>& col_idx) {
  if (n_q < 1 || n_k < 1) return fail(BSATTN_ERR_INVALID_ARG, "n_q and n_k must be >= 1");
  if (Br < 1 || Br > 4096 || Bc < 1 || Bc > 4096) return fail(BSATTN_ERR_INVALID_ARG, "Br, Bc must lie in [1, 4096]");
  bsattn_status st = validate_spec(spec, n_k);
  if (st != BSATTN_OK) return st;
  const int32_t Tr = (n_q + Br - 1) / Br, Tc = (n_k + Bc - 1) / Bc;
  const int64_t nv = spec->n_valid;
  const int64_t a0 = spec->anchor_start, a1 = (int64_t)spec->anchor_start + spec->anchor_len;
  row_ptr.assign(Tr + 1, 0);
  col_idx.clear();
  BlockSet set;
  for (int32_t t = 0; t < Tr; ++t) {
    set.reset(Tc, Bc);
    int64_t r0 = (int64_t)t * Br, r1 = std::min<int64_t>((int64_t)(t + 1) * Br, n_q);
    r1 = std::min<int64_t>(r1, nv);  // padding queries pair with nothing
    if (r0 < r1) {
      if (spec->anchor_len > 0) {
        if (r0 < a1 && a0 < r1) set.mark_tokens(0, nv);  // an anchor query sees every valid key
        set.mark_tokens(a0, a1);                         // every valid query sees the anchors
      }
      for (int32_t i = 0; i < spec->n_segments; ++i) {
        const bsattn_segment& s = spec->segments[i];
        int64_t a = std::max<int64_t>(r0, s.start), b = std::min<int64_t>(r1, (int64_t)s.start + s.len);
        if (a < b) mark_segment_part(s, a, b, set);
      }
    }
    for (int32_t w = 0; w < (int32_t)set.words.size(); ++w) {
      uint64_t x = set.words[w];
      while (x) {
        int bit = __builtin_ctzll(x);
        col_idx.push_back(w * 64 + bit);
        x &= x - 1;
      }
    }
    row_ptr[t + 1] = (int32_t)col_idx.size();
  }
  return BSATTN_OK;
}

}  // namespace bsattn

namespace {

// CSR of a kept-block predicate, tile-major and ascending within a tile.
template <class Kept>
bsattn_status csr_of(Kept kept, int32_t Tr, int32_t Tc, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                     int64_t* nnz_out) {
  using namespace bsattn;
  if (!row_ptr || !nnz_out || Tr < 1 || Tc < 1) return fail(BSATTN_ERR_INVALID_ARG, "row_ptr / nnz_out NULL or Tr, Tc < 1");
  int64_t nnz = 0;
  row_ptr[0] = 0;
  for (int32_t t = 0; t < Tr; ++t) {
    for (int32_t j = 0; j < Tc; ++j) {
      if (!kept(t, j)) continue;
      if (col_idx) {
        if (nnz >= col_capacity) return fail(BSATTN_ERR_CAPACITY, "col_idx capacity %lld too small", (long long)col_capacity);
        col_idx[nnz] = j;
      }
      ++nnz;
    }
    if (nnz > 0x7fffffffLL) return fail(BSATTN_ERR_CAPACITY, "more than 2^31 - 1 kept blocks");
    row_ptr[t + 1] = (int32_t)nnz;
  }
  *nnz_out = nnz;
  return BSATTN_OK;
}

}  // namespace

extern "C" {

bsattn_status bsattn_build_block_index(const bsattn_mask_spec* spec, int32_t n_q, int32_t n_k, int32_t Br,
                                       int32_t Bc, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                       int64_t* nnz_out) {
  using namespace bsattn;
  clear_error();
  if (!row_ptr || !nnz_out) return fail(BSATTN_ERR_INVALID_ARG, "row_ptr and nnz_out must be non-NULL");
  std::vector<int32_t> rp, ci;
  bsattn_status st;
  try {
    st = build_block_index(spec, n_q, n_k, Br, Bc, rp, ci);
  } catch (...) {
    return fail(BSATTN_ERR_INVALID_ARG, "block index build failed (out of host memory)");
  }
  if (st != BSATTN_OK) return st;
  *nnz_out = (int64_t)ci.size();
  std::memcpy(row_ptr, rp.data(), rp.size() * sizeof(int32_t));
  if (!col_idx) return BSATTN_OK;
  if (col_capacity < (int64_t)ci.size())
    return fail(BSATTN_ERR_CAPACITY, "col_capacity %lld < nnz %lld", (long long)col_capacity, (long long)ci.size());
  if (!ci.empty()) std::memcpy(col_idx, ci.data(), ci.size() * sizeof(int32_t));
  return BSATTN_OK;
}

bsattn_status bsattn_validate_block_index(const int32_t* row_ptr, const int32_t* col_idx, int32_t Tr, int32_t Tc) {
  using namespace bsattn;
  clear_error();
  if (!row_ptr || Tr < 1 || Tc < 1) return fail(BSATTN_ERR_INVALID_ARG, "row_ptr NULL or Tr/Tc < 1");
  if (row_ptr[0] != 0) return fail(BSATTN_ERR_INVALID_ARG, "row_ptr[0] must be 0");
  for (int32_t t = 0; t < Tr; ++t) {
    if (row_ptr[t + 1] < row_ptr[t]) return fail(BSATTN_ERR_INVALID_ARG, "row_ptr decreases at tile %d", t);
    if (row_ptr[t + 1] - row_ptr[t] > Tc) return fail(BSATTN_ERR_INVALID_ARG, "tile %d lists more than Tc blocks", t);
  }
  if (row_ptr[Tr] > 0 && !col_idx) return fail(BSATTN_ERR_INVALID_ARG, "col_idx NULL with nnz > 0");
  for (int32_t t = 0; t < Tr; ++t) {
    for (int32_t e = row_ptr[t]; e < row_ptr[t + 1]; ++e) {
      int32_t c = col_idx[e];
      if (c < 0 || c >= Tc) return fail(BSATTN_ERR_INVALID_ARG, "col_idx[%d] = %d outside [0, %d)", e, c, Tc);
      if (e > row_ptr[t] && c <= col_idx[e - 1])
        return fail(BSATTN_ERR_INVALID_ARG, "col_idx not strictly ascending in tile %d", t);
    }
  }
  return BSATTN_OK;
}

bsattn_status bsattn_block_index_from_matrix(const uint8_t* m, int32_t Tr, int32_t Tc, int32_t* row_ptr,
                                             int32_t* col_idx, int64_t col_capacity, int64_t* nnz_out) {
  using namespace bsattn;
  clear_error();
  if (!m) return fail(BSATTN_ERR_INVALID_ARG, "block matrix is NULL");
  return csr_of([&](int32_t t, int32_t j) { return m[(int64_t)t * Tc + j] != 0; }, Tr, Tc, row_ptr, col_idx,
                col_capacity, nnz_out);
}

bsattn_status bsattn_block_index_from_bitmap(const uint8_t* bits, int32_t Tr, int32_t Tc, int32_t* row_ptr,
                                             int32_t* col_idx, int64_t col_capacity, int64_t* nnz_out) {
  using namespace bsattn;
  clear_error();
  if (!bits) return fail(BSATTN_ERR_INVALID_ARG, "bitmap is NULL");
  return csr_of(
      [&](int32_t t, int32_t j) {
        const int64_t k = (int64_t)t * Tc + j;
        return ((bits[k >> 3] >> (k & 7)) & 1) != 0;
      },
      Tr, Tc, row_ptr, col_idx, col_capacity, nnz_out);
}

bsattn_status bsattn_block_index_from_coo(const int32_t* rows, const int32_t* cols, int64_t n, int32_t Tr,
                                          int32_t Tc, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                          int64_t* nnz_out) {
  using namespace bsattn;
  clear_error();
  if (n < 0 || (n > 0 && (!rows || !cols))) return fail(BSATTN_ERR_INVALID_ARG, "rows / cols NULL or n < 0");
  if (Tr < 1 || Tc < 1) return fail(BSATTN_ERR_INVALID_ARG, "Tr, Tc must be >= 1");
  std::vector<uint8_t> m((size_t)Tr * Tc, 0);
  for (int64_t x = 0; x < n; ++x) {
    if (rows[x] < 0 || rows[x] >= Tr || cols[x] < 0 || cols[x] >= Tc)
      return fail(BSATTN_ERR_INVALID_ARG, "pair %lld = (%d, %d) outside [0, %d) x [0, %d)", (long long)x, rows[x],
                  cols[x], Tr, Tc);
    m[(size_t)rows[x] * Tc + cols[x]] = 1;
  }
  return csr_of([&](int32_t t, int32_t j) { return m[(size_t)t * Tc + j] != 0; }, Tr, Tc, row_ptr, col_idx,
                col_capacity, nnz_out);
}

bsattn_status bsattn_transpose_block_index(const int32_t* row_ptr, const int32_t* col_idx, int32_t Tr, int32_t Tc,
                                           int32_t* col_ptr, int32_t* row_idx) {
  using namespace bsattn;
  clear_error();
  if (!col_ptr || (!row_idx && row_ptr && row_ptr[Tr] > 0))
    return fail(BSATTN_ERR_INVALID_ARG, "col_ptr / row_idx NULL");
  const bsattn_status st = bsattn_validate_block_index(row_ptr, col_idx, Tr, Tc);
  if (st != BSATTN_OK) return st;
  // counting sort by key block; walking the tiles in ascending order keeps
  // every key block's tile list ascending
  for (int32_t c = 0; c <= Tc; ++c) col_ptr[c] = 0;
  for (int32_t e = 0; e < row_ptr[Tr]; ++e) ++col_ptr[col_idx[e] + 1];
  for (int32_t c = 0; c < Tc; ++c) col_ptr[c + 1] += col_ptr[c];
  std::vector<int32_t> fill(col_ptr, col_ptr + Tc);
  for (int32_t t = 0; t < Tr; ++t)
    for (int32_t e = row_ptr[t]; e < row_ptr[t + 1]; ++e) row_idx[fill[col_idx[e]]++] = t;
  return BSATTN_OK;
}

bsattn_status bsattn_build_schedule(const int32_t* row_ptr, int32_t Tr, int32_t max_blocks, int32_t* items,
                                    int32_t items_capacity, int32_t* merges, int32_t merges_capacity, int32_t* n_items,
                                    int32_t* n_merges, int32_t* n_slots) {
  using namespace bsattn;
  clear_error();
  if (!row_ptr || Tr < 1 || !n_items || !n_merges || !n_slots)
    return fail(BSATTN_ERR_INVALID_ARG, "row_ptr / counts NULL or Tr < 1");
  if (max_blocks < 1) return fail(BSATTN_ERR_INVALID_ARG, "max_blocks_per_item must be >= 1");
  struct Item { int32_t tile, first, end, slot, merge; };
  std::vector<Item> it;
  std::vector<int32_t> mg;
  int32_t slots = 0;
  for (int32_t t = 0; t < Tr; ++t) {
    const int32_t b = row_ptr[t], e = row_ptr[t + 1];
    if (e < b) return fail(BSATTN_ERR_INVALID_ARG, "row_ptr decreases at tile %d", t);
    const int32_t n = e - b;
    if (n <= max_blocks) {
      it.push_back({t, b, e, -1, -1});
      continue;
    }
    const int32_t k = (n + max_blocks - 1) / max_blocks;  // chunks of near-equal size
    const int32_t m = (int32_t)(mg.size() / 3);
    mg.insert(mg.end(), {t, slots, k});
    for (int32_t c = 0; c < k; ++c) {
      const int32_t cb = b + (int32_t)((int64_t)n * c / k), ce = b + (int32_t)((int64_t)n * (c + 1) / k);
      it.push_back({t, cb, ce, slots + c, m});
    }
    slots += k;
  }
  std::stable_sort(it.begin(), it.end(), [](const Item& x, const Item& y) { return (x.end - x.first) > (y.end - y.first); });
  *n_items = (int32_t)it.size();
  *n_merges = (int32_t)(mg.size() / 3);
  *n_slots = slots;
  if (!items) return BSATTN_OK;
  if (items_capacity < *n_items || (*n_merges > 0 && (!merges || merges_capacity < *n_merges)))
    return fail(BSATTN_ERR_CAPACITY, "schedule needs %d items and %d merges", *n_items, *n_merges);
  for (size_t i = 0; i < it.size(); ++i) {
    int32_t* o = items + 5 * i;
    o[0] = it[i].tile;
    o[1] = it[i].first;
    o[2] = it[i].end;
    o[3] = it[i].slot;
    o[4] = it[i].merge;
  }
  if (!mg.empty()) std::memcpy(merges, mg.data(), mg.size() * sizeof(int32_t));
  return BSATTN_OK;
}

bsattn_status bsattn_schedule_tile_order(int32_t* items, int32_t n_items) {
  using namespace bsattn;
  clear_error();
  if (n_items < 0 || (n_items > 0 && !items)) return fail(BSATTN_ERR_INVALID_ARG, "items NULL or n_items < 0");
  struct Item { int32_t f[5]; };
  std::vector<Item> it(n_items);
  std::memcpy(it.data(), items, (size_t)n_items * sizeof(Item));
  for (const Item& x : it)
    if ((x.f[3] < 0) != (x.f[4] < 0)) return fail(BSATTN_ERR_INVALID_ARG, "item with slot %d but merge %d", x.f[3], x.f[4]);
  // chunks of cut tiles first, in their present order; then whole tiles by index
  std::stable_sort(it.begin(), it.end(), [](const Item& x, const Item& y) {
    const bool cx = x.f[3] >= 0, cy = y.f[3] >= 0;
    if (cx != cy) return cx;
    return !cx && x.f[0] < y.f[0];
  });
  std::memcpy(items, it.data(), (size_t)n_items * sizeof(Item));
  return BSATTN_OK;
}

bsattn_status bsattn_build_dkdv_schedule(const int32_t* col_ptr, const int32_t* row_idx, int32_t Tc, int32_t G,
                                         int32_t d, int32_t max_positions_per_item, int32_t* items,
                                         int32_t items_capacity, int32_t* merges, int32_t merges_capacity,
                                         int32_t* n_items, int32_t* n_merges, int32_t* n_slots) {
  using namespace bsattn;
  clear_error();
  if (!col_ptr || !row_idx || Tc < 1 || G < 1 || !n_items || !n_merges || !n_slots)
    return fail(BSATTN_ERR_INVALID_ARG, "col_ptr / row_idx / counts NULL, Tc < 1 or G < 1");
  if (d != 64 && d != 128) return fail(BSATTN_ERR_UNSUPPORTED, "head dim %d not supported (64, 128)", d);
  if (max_positions_per_item < 1) return fail(BSATTN_ERR_INVALID_ARG, "max_positions_per_item must be >= 1");
  const int32_t NB = d == 64 ? kDkdvBlocks64 : kDkdvBlocks128;
  for (int32_t j = 0; j < Tc; ++j) {
    if (col_ptr[j + 1] < col_ptr[j]) return fail(BSATTN_ERR_INVALID_ARG, "col_ptr decreases at block %d", j);
    for (int32_t e = col_ptr[j] + 1; e < col_ptr[j + 1]; ++e)
      if (row_idx[e] <= row_idx[e - 1]) return fail(BSATTN_ERR_INVALID_ARG, "row_idx not ascending for block %d", j);
  }
  struct Item { int32_t f[kKvItemInts]; };
  std::vector<Item> it;
  std::vector<int32_t> mg;
  int32_t slots = 0;
  std::vector<int32_t> uni;
  for (int32_t m = 0; m * NB < Tc; ++m) {
    // the tiles of the group: the union of its blocks' ascending lists
    const int32_t j0 = NB * m, nb = std::min(NB, Tc - j0);
    const int32_t* l0 = row_idx + col_ptr[j0];
    const int32_t n0 = col_ptr[j0 + 1] - col_ptr[j0];
    const int32_t* l1 = nb > 1 ? row_idx + col_ptr[j0 + 1] : nullptr;
    const int32_t n1 = nb > 1 ? col_ptr[j0 + 2] - col_ptr[j0 + 1] : 0;
    uni.clear();
    std::set_union(l0, l0 + n0, l1, l1 + n1, std::back_inserter(uni));
    const int64_t U = (int64_t)uni.size(), P = (int64_t)G * U;
    if (P <= max_positions_per_item) {
      it.push_back({{m, 0, (int32_t)P, 0, 0, 0, -1, -1}});
      continue;
    }
    const int32_t k = (int32_t)((P + max_positions_per_item - 1) / max_positions_per_item);
    const int32_t mi = (int32_t)(mg.size() / 3);
    mg.insert(mg.end(), {m, slots, k});
    for (int32_t c = 0; c < k; ++c) {
      const int64_t p0 = P * c / k, p1 = P * (c + 1) / k;
      const int32_t t0 = uni[p0 % U];
      const int32_t i0 = (int32_t)(std::lower_bound(l0, l0 + n0, t0) - l0);
      const int32_t i1 = l1 ? (int32_t)(std::lower_bound(l1, l1 + n1, t0) - l1) : 0;
      it.push_back({{m, (int32_t)p0, (int32_t)p1, (int32_t)(p0 / U), i0, i1, slots + c, mi}});
    }
    slots += k;
  }
  std::stable_sort(it.begin(), it.end(),
                   [](const Item& x, const Item& y) { return (x.f[2] - x.f[1]) > (y.f[2] - y.f[1]); });
  *n_items = (int32_t)it.size();
  *n_merges = (int32_t)(mg.size() / 3);
  *n_slots = slots;
  if (!items) return BSATTN_OK;
  if (items_capacity < *n_items || (*n_merges > 0 && (!merges || merges_capacity < *n_merges)))
    return fail(BSATTN_ERR_CAPACITY, "schedule needs %d items and %d merges", *n_items, *n_merges);
  std::memcpy(items, it.data(), it.size() * sizeof(Item));
  if (!mg.empty()) std::memcpy(merges, mg.data(), mg.size() * sizeof(int32_t));
  return BSATTN_OK;
}

bsattn_status bsattn_tile_order_lpt(const int32_t* row_ptr, int32_t Tr, int32_t* order) {
  using namespace bsattn;
  clear_error();
  if (!row_ptr || !order || Tr < 1) return fail(BSATTN_ERR_INVALID_ARG, "row_ptr/order NULL or Tr < 1");
  std::vector<int32_t> idx(Tr);
  for (int32_t t = 0; t < Tr; ++t) idx[t] = t;
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t x, int32_t y) {
    return (row_ptr[x + 1] - row_ptr[x]) > (row_ptr[y + 1] - row_ptr[y]);
  });
  std::memcpy(order, idx.data(), Tr * sizeof(int32_t));
  return BSATTN_OK;
}

}  // extern "C"
