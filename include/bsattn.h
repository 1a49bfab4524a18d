/*
 * bsattn.h - block-sparse and BLASST attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libbsattn.so.  Every function has C linkage, throws nothing, and
 * reports errors through its return status plus a thread-local message
 * (bsattn_last_error).  The library never allocates, frees or copies device
 * memory and never synchronises: compute entry points validate their
 * arguments on the host, then enqueue kernels on the caller's stream and
 * return.  All buffers are owned by the caller and must stay valid and
 * unmodified until the enqueued work has finished.
 *
 * Operation (the attention operator of the BLASST paper notes, section
 * 3.1.1):  out = softmax(scale * Q K^T) V, computed FlashAttention-style
 * (online softmax, attention tutorial section 4.2) over tiles of Br query
 * rows and blocks of Bc keys, where whole key blocks are skipped in two ways:
 *
 *   static  - a per-query-tile list of kept key blocks (CSR), built from a
 *             mask specification (DiT block-sparse article, sections 2.1,
 *             2.3 and 3.2; the kernel checks the list before loading K/V,
 *             section 3.3);
 *   dynamic - BLASST (paper notes, section 3.1 and Algorithm 1): after the
 *             running row max is updated with a block's row max, the block
 *             is skipped (no exponent, no row-sum update, no P.V product)
 *             when block max - running max < ln(lambda) holds for every row
 *             of the tile (tile-wide vote, notes section 4).  The decode
 *             path also skips the V-block load (notes, section 4.2).
 *
 * Semantics fixed where the pages are open:
 *   - scores are compared in the scaled domain (S = scale * Q K^T);
 *   - "<" is strict; lambda = 0 disables skipping; lambda must be in [0, 1);
 *   - key blocks are visited in ascending order (CSR order);
 *   - a row with no allowed key in a block satisfies the skip condition;
 *   - a query row with no allowed key at all produces zeros;
 *   - GQA: query head h reads K/V head h / (Hq / Hkv);
 *   - decode: the vote is taken by the G = Hq/Hkv query heads that share a
 *     K/V head, and the running max spans the whole sequence, so the skip
 *     set does not depend on num_splits.
 */
#ifndef BSATTN_H
#define BSATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------------ */
/* status                                                                     */
/* ------------------------------------------------------------------------ */

typedef enum {
  BSATTN_OK = 0,
  BSATTN_ERR_INVALID_ARG = 1, /* null pointer, bad size, lambda out of range, malformed CSR */
  BSATTN_ERR_UNSUPPORTED = 2, /* valid request the library does not implement (dtype, d, tile) */
  BSATTN_ERR_CAPACITY = 3,    /* caller buffer too small (col_idx capacity, workspace) */
  BSATTN_ERR_HIP = 4          /* a HIP call or kernel launch failed */
} bsattn_status;

typedef enum { BSATTN_BF16 = 0, BSATTN_FP32 = 1 } bsattn_dtype;

/* Static string for a status code. */
const char* bsattn_status_string(int status);
/* Message of the last failing call on this thread ("" if none). */
const char* bsattn_last_error(void);
/* Library version, e.g. 0x000100 for 0.1.0. */
int bsattn_version(void);

/* ------------------------------------------------------------------------ */
/* mask specification and block index (host only)                             */
/* DiT block-sparse article: section 2.1 (mask families), 2.3 (block grid,   */
/* sparse index), 3.1 (block boundaries aligned with the token layout), 3.2  */
/* (multimodal recipe: segments -> per-pair rule -> 0/1 block matrix).       */
/* ------------------------------------------------------------------------ */

enum {
  BSATTN_SEG_FULL = 0,     /* every token of the segment pairs with every other (block diagonal) */
  BSATTN_SEG_BLOCKWIN = 1, /* |(i-start)/unit - (j-start)/unit| <= radius (1-D local window)       */
  BSATTN_SEG_IMAGE2D = 2,  /* grid_h x grid_w row-major patches: |drow| <= radius && |dcol| <= radius */
  BSATTN_SEG_VIDEO3D = 3   /* frames x grid_h x grid_w: same frame as IMAGE2D; frames 1..t_radius
                              apart pair iff both tokens lie in the same spatial unit
                              ((offset within frame) / unit equal)                                  */
};

typedef struct {
  int32_t kind;   /* BSATTN_SEG_* */
  int32_t start;  /* first token of the segment */
  int32_t len;    /* number of tokens (frames*grid_h*grid_w for VIDEO3D, grid_h*grid_w for IMAGE2D) */
  int32_t frames, grid_h, grid_w;
  int32_t radius;   /* spatial / 1-D window radius (patches, or units for BLOCKWIN) */
  int32_t t_radius; /* temporal radius in frames (VIDEO3D) */
  int32_t unit;     /* unit size in tokens (BLOCKWIN window unit, VIDEO3D spatial unit) */
} bsattn_segment;

typedef struct {
  int32_t n_valid;                 /* tokens >= n_valid are padding: never keys, pair with nothing */
  int32_t n_segments;              /* segments must not overlap */
  const bsattn_segment* segments;  /* host memory */
  int32_t anchor_start, anchor_len;/* global anchor tokens: pair with every valid token both ways */
} bsattn_mask_spec;

/*
 * Build the per-query-tile CSR of kept key blocks.  Token pair (i, j) is
 * related by the spec's rules; tile t (query rows [t*Br, (t+1)*Br)) keeps
 * key block c (keys [c*Bc, (c+1)*Bc)) iff at least one related pair lies
 * in it.  Output (host buffers):
 *   row_ptr[Tr + 1], Tr = ceil(n_q / Br): row_ptr[0] = 0, nondecreasing;
 *   col_idx[nnz]: ascending within each tile.
 * Two-call pattern: pass col_idx = NULL to get *nnz_out only.  If
 * col_capacity < nnz, returns BSATTN_ERR_CAPACITY with *nnz_out set.
 * Requirements: 1 <= Br, Bc <= 4096; n_q, n_k >= 1; 0 <= n_valid <= n_k; segments
 * inside [0, n_valid), non-overlapping and consistent with their grid sizes;
 * anchors inside [0, n_valid).  Violations return BSATTN_ERR_INVALID_ARG.
 */
bsattn_status bsattn_build_block_index(const bsattn_mask_spec* spec, int32_t n_q, int32_t n_k,
                                       int32_t Br, int32_t Bc, int32_t* row_ptr, int32_t* col_idx,
                                       int64_t col_capacity, int64_t* nnz_out);

/* The same CSR from the block-mask forms the DiT article's mask flow produces
 * (section 2.3: a 0/1 matrix over (query block, key block), stored as a
 * bitmap of one bit per block or as COO pairs; section 3.2):
 *   _from_matrix  uint8 [Tr][Tc] row-major, nonzero = kept
 *   _from_bitmap  bit (t * Tc + j) of the byte string, least significant bit
 *                 first, set = kept ((Tr * Tc + 7) / 8 bytes)
 *   _from_coo     n (row, col) pairs of kept blocks, any order, duplicates
 *                 allowed; a pair outside [0, Tr) x [0, Tc) is INVALID_ARG
 * Host buffers, two-call pattern as bsattn_build_block_index (col_idx NULL
 * returns the count in *nnz_out; BSATTN_ERR_CAPACITY if col_capacity is
 * short).  Tiles list their blocks in ascending order. */
bsattn_status bsattn_block_index_from_matrix(const uint8_t* m, int32_t Tr, int32_t Tc, int32_t* row_ptr,
                                             int32_t* col_idx, int64_t col_capacity, int64_t* nnz_out);
bsattn_status bsattn_block_index_from_bitmap(const uint8_t* bits, int32_t Tr, int32_t Tc, int32_t* row_ptr,
                                             int32_t* col_idx, int64_t col_capacity, int64_t* nnz_out);
bsattn_status bsattn_block_index_from_coo(const int32_t* rows, const int32_t* cols, int64_t n, int32_t Tr,
                                          int32_t Tc, int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                          int64_t* nnz_out);

/* Check a host CSR: row_ptr[0] == 0, nondecreasing, row_ptr[Tr] = nnz,
 * col_idx strictly ascending within each tile and inside [0, Tc). */
bsattn_status bsattn_validate_block_index(const int32_t* row_ptr, const int32_t* col_idx,
                                          int32_t Tr, int32_t Tc);

/* Transpose of a host CSR (tiles -> key blocks) into its CSC (key blocks ->
 * tiles): col_ptr [Tc + 1], row_idx [nnz], each key block's tiles in
 * ascending order.  The backward pass walks it to find the query tiles that
 * attended a key block.  Validates the CSR first (errors as
 * bsattn_validate_block_index).  Host buffers. */
bsattn_status bsattn_transpose_block_index(const int32_t* row_ptr, const int32_t* col_idx, int32_t Tr, int32_t Tc,
                                           int32_t* col_ptr, int32_t* row_idx);

/* Longest-first launch order for the tiles of a CSR (DiT article section 5.3
 * point 3: uneven rows unbalance the GPU): order[k] is the tile launched
 * k-th; ties keep ascending tile index.  Host buffers. */
bsattn_status bsattn_tile_order_lpt(const int32_t* row_ptr, int32_t Tr, int32_t* order);

/*
 * Work schedule for a static CSR (same load-imbalance concern): tiles with
 * more than max_blocks_per_item kept blocks are cut into near-equal chunks of
 * consecutive CSR entries, each chunk a separate work-group writing a partial
 * (running max, row sum, unnormalised output) to the prefill workspace; the
 * last chunk of a cut tile to finish combines the partials with the online-
 * softmax rescaling rule (attention tutorial section 4.2), in slot order, and
 * writes the output.  With lambda > 0 the skip decisions depend on the
 * running max of every block visited before (BLASST notes Algorithm 1): a
 * first pass over the chunks of cut tiles writes each chunk's per-row block
 * maximum, and every chunk then starts from the maximum of the chunks
 * visited before it, so the decisions equal those of a whole-row walk.
 *   items  [n_items][5]  {tile, first CSR entry, end CSR entry, slot, merge};
 *                        slot = merge = -1 means the item writes the output
 *                        directly, else merge indexes `merges`; items are
 *                        ordered longest first
 *   merges [n_merges][3] {tile, first slot, number of slots}; the slots of a
 *                        cut tile are consecutive, and chunk c of k covers
 *                        the tile's CSR entries [f + n c / k, f + n (c + 1) / k)
 *                        (f its first entry, n its count; integer division):
 *                        the chunk-maximum pass (lambda > 0) takes the
 *                        ranges from this rule, so a hand-made schedule must
 *                        cut the same way
 * Two-call pattern: items == NULL returns the counts only.  Host buffers.
 * max_blocks_per_item >= 1.  Returns BSATTN_ERR_CAPACITY if a buffer is short.
 */
bsattn_status bsattn_build_schedule(const int32_t* row_ptr, int32_t Tr, int32_t max_blocks_per_item,
                                    int32_t* items, int32_t items_capacity, int32_t* merges,
                                    int32_t merges_capacity, int32_t* n_items, int32_t* n_merges,
                                    int32_t* n_slots);

/*
 * Locality order for a schedule (DiT article section 5.3: memory throughput).
 * Reorders the items of bsattn_build_schedule in place: the chunks of cut
 * tiles first, in their present order (longest first), then the whole tiles
 * by ascending tile index, so that work-groups started together hold
 * neighbouring tiles, whose key blocks overlap, in one L2.  Merges and slots
 * are unchanged (items keep their fields).  Pays off when a launch walks each
 * (batch, K/V head) group's items consecutively, see
 * bsattn_prefill_group_major; otherwise longest first gives the shorter tail.
 * Host buffer [n_items][5].  INVALID_ARG if an item has a slot but no merge
 * or the reverse.
 */
bsattn_status bsattn_schedule_tile_order(int32_t* items, int32_t n_items);

/*
 * Work order of a bf16 prefill launch with n_units work items per (batch,
 * query head): tiles (Tr), or the n_items of a schedule.  Returns 1 when each
 * XCD walks one (batch, K/V head) group's items consecutively (group-major:
 * B * Hkv divisible by 8 and enough work-groups for four waves per XCD), 0
 * when the launch takes items rank by rank across groups, -1 for an invalid
 * shape (any size < 1, Hq % Hkv != 0, d not 64 or 128).  The launch itself
 * uses this rule.
 */
int32_t bsattn_prefill_group_major(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t n_units);

/* ------------------------------------------------------------------------ */
/* prefill                                                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
  int32_t dtype;          /* BSATTN_BF16 (MFMA path) or BSATTN_FP32 (vector path) for q, k, v, out */
  const void* q;          /* device [B, Nq, Hq, d] (strides below), d contiguous */
  const void* k;          /* device [B, Nk, Hkv, d] */
  const void* v;          /* device [B, Nk, Hkv, d] */
  void* out;              /* device [B, Nq, Hq, d], written for every row < Nq */
  int32_t B, Hq, Hkv, Nq, Nk, d; /* d in {64, 128}; Hq % Hkv == 0 */
  int64_t q_stride[3];    /* element strides for batch, token, head */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  const int32_t* row_ptr; /* device CSR at (Br, Bc), [Tr + 1]; NULL = every block */
  const int32_t* col_idx; /* device [nnz], ascending per tile */
  const int32_t* tile_order; /* optional device [Tr] launch order (a permutation); NULL = default
                                (longest-first for causal, ascending otherwise) */
  int32_t n_valid;        /* keys >= n_valid are never attended; 0 means Nk */
  float scale;            /* score scale, e.g. 1/sqrt(d); > 0 */
  float lambda;           /* 0 = static only; 0 < lambda < 1 = BLASST skipping; else INVALID_ARG */
  int32_t causal;         /* key j attends query i iff j <= i; requires Nq == Nk */
  int32_t Br, Bc;         /* bf16: Br = 128, Bc = 64.  fp32: Br in {64, 128}, Bc = 64 */
  int32_t* tile_counters; /* optional device [B, Hq, Tr, 2] int32: {visited, skipped} blocks */
  uint8_t* block_state;   /* optional device [B, Hq, Tr, Tc]: the kernel writes 1 (computed) or
                             2 (skipped) for visited blocks; the caller zero-fills it first */
  int32_t* row_counters;  /* optional device [B, Hq, Tr] int32: for lambda > 0, the number of
                             (query row < Nq, visited block) pairs whose own row condition
                             holds (block max - running max < ln lambda, or no allowed key),
                             before the tile-wide vote (BLASST notes sections 3.1.1 and 4);
                             0 for lambda = 0.  Compare with skipped x rows for the cost of
                             tile-wide decisions */
  int32_t block_order;    /* 0: visited blocks in ascending order (Algorithm 1); 1: descending,
                             most recent keys first (the block-row reordering the BLASST notes
                             study).  The order changes which blocks lambda > 0 skips */
  const int32_t* sched_items;  /* optional device copy of bsattn_build_schedule's items (needs the CSR);
                                  NULL = one work-group per tile (tile_order applies) */
  int32_t n_items;
  const int32_t* sched_merges; /* device copy of the schedule's merges (NULL if n_merges == 0) */
  int32_t n_merges;
  int32_t n_slots;             /* partial slots of the schedule (cut tiles) */
  void* workspace;             /* device, >= bsattn_prefill_workspace_size(B, Hq, d, n_slots) bytes,
                                  256-byte aligned; unused when n_slots == 0.  Holds the
                                  partials and one arrival counter per (merge, batch, head).
                                  No initial contents are needed, and calls of any shape may
                                  share it: a launch ahead of the main kernel zeroes the
                                  call's arrival counters (the chunk-maximum pass when
                                  lambda > 0, else a small clear kernel).  Calls that share a
                                  workspace must not overlap (same stream, or ordered by
                                  events). */
  size_t workspace_bytes;
  float* lse;             /* optional device [B, Hq, Nq] float32: each row's natural-log sum of
                             exp(scale q.k) over the keys it attended (-inf for a row with none),
                             the statistic the backward pass (bsattn_prefill_bwd) rebuilds P from */
} bsattn_prefill_args;

/* Workspace bytes for a prefill whose schedule has n_slots partial slots. */
size_t bsattn_prefill_workspace_size(int32_t B, int32_t Hq, int32_t d, int32_t n_slots);

/* Enqueue the prefill on `stream` (a hipStream_t; NULL = default stream).
 * Validation: pointers non-null and 16-byte aligned, token/head strides
 * multiples of 8 (bf16) or 4 (fp32) elements, d contiguous; CSR pointers
 * both set or both NULL (the CSR itself is not read on the host: call
 * bsattn_validate_block_index on the host copy); bf16: (Nk + 64) x K/V
 * token stride x 2 bytes below 4 GiB (32-bit offsets within one head,
 * else BSATTN_ERR_UNSUPPORTED).  Returns BSATTN_ERR_HIP if the launch fails. */
bsattn_status bsattn_prefill_fwd(const bsattn_prefill_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* prefill backward (static block mask)                                       */
/* ------------------------------------------------------------------------ */

/*
 * Gradients of the block-sparse attention computed by bsattn_prefill_fwd
 * (lambda = 0, or lambda > 0 with that call's block_state passed in, which
 * drops the blocks it skipped): for the loss sum(out * dout),
 *   dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dout,
 *   P = the forward's softmax over each row's attended keys (rebuilt from
 *       q, k and the forward's lse), dP = dout V^T,
 *   dS = P * (dP - rowsum(dout * out))
 * over the same token mask as the forward: blocks of the tile's CSR list (or
 * every block), keys < n_valid, and key <= query when causal (blocks wholly
 * above the diagonal are not visited).  With GQA, dk and dv of a K/V head
 * sum its query heads.  The pages give no backward; this is the chain rule
 * applied to the forward's definition (the DiT article trains with the
 * block-sparse forward, section 4).  Every element of dq, dk, dv (rows < Nq,
 * keys < Nk) is written; keys or rows that attend nothing get zeros.
 *
 * Launches on `stream`: rowsum(dout * out) into the workspace, dk/dv (one
 * work-group per batch, K/V head and group of adjacent 64-key blocks - one
 * block at d = 64, two at d = 128 - walking the CSC over the group's query
 * heads), dq (one work-group per batch, head and 128-row tile, walking the
 * CSR).  Optional schedules cut long work items (DiT article section 5.3:
 * uneven rows unbalance the GPU): dq_items from bsattn_build_schedule on the
 * CSR, kv_items from bsattn_build_dkdv_schedule on the CSC.  A chunk writes
 * fp32 partial sums to the workspace; the last chunk of an item to arrive
 * adds them in slot order and writes the gradient, so the results stay
 * deterministic (they differ from an uncut run only in the order of fp32
 * additions).  The rowsum launch also zeroes the arrival counters that a
 * cutting schedule counts with.  No float atomics.
 */
typedef struct {
  int32_t dtype;          /* BSATTN_BF16 */
  const void* q;          /* device [B, Nq, Hq, d] bf16, as given to the forward */
  const void* k;          /* device [B, Nk, Hkv, d] */
  const void* v;          /* device [B, Nk, Hkv, d] */
  const void* out;        /* device [B, Nq, Hq, d]: the forward's output */
  const void* dout;       /* device [B, Nq, Hq, d]: gradient of the loss w.r.t. out */
  const float* lse;       /* device [B, Hq, Nq]: the forward's lse output */
  void* dq;               /* device [B, Nq, Hq, d] bf16 output */
  void* dk;               /* device [B, Nk, Hkv, d] bf16 output */
  void* dv;               /* device [B, Nk, Hkv, d] bf16 output */
  int32_t B, Hq, Hkv, Nq, Nk, d; /* d in {64, 128}; Hq % Hkv == 0 */
  int64_t q_stride[3];    /* element strides for batch, token, head (d contiguous), per tensor */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  int64_t do_stride[3];
  int64_t dq_stride[3];
  int64_t dk_stride[3];
  int64_t dv_stride[3];
  const int32_t* row_ptr; /* device CSR at (128, 64) as in the forward, or NULL (every block) */
  const int32_t* col_idx;
  const int32_t* col_ptr; /* device transpose of that CSR (bsattn_transpose_block_index),
                             required with it, NULL without */
  const int32_t* row_idx;
  int32_t n_valid;        /* as in the forward; 0 means Nk */
  float scale;            /* as in the forward */
  int32_t causal;         /* as in the forward; requires Nq == Nk */
  int32_t Br, Bc;         /* 128, 64 */
  void* workspace;        /* device, >= bsattn_prefill_bwd_workspace_size(B, Hq, Nq) bytes,
                             256-byte aligned; no initial contents needed */
  size_t workspace_bytes;
  const uint8_t* block_state; /* optional device [B, Hq, Tr, Tc]: the block_state a forward with
                             lambda > 0 wrote; blocks it skipped (2) get no gradient, so the
                             gradients are those of the function that forward computed (softmax
                             over its kept blocks; BLASST notes, training with the skipping
                             forward).  Read through the scalar cache in aligned 4-byte words,
                             so the up to 3 bytes beside the array in its first and last words
                             are read and ignored (never past a page the array touches).
                             NULL = every visited block */
  const int32_t* dq_items;  /* optional device copy of bsattn_build_schedule's items for the CSR
                               (needs it); NULL = one dq work-group per tile, and the four dq_
                               counts / merges below must be 0 / NULL */
  int32_t dq_n_items;
  const int32_t* dq_merges; /* device copy of that schedule's merges (NULL if dq_n_merges == 0) */
  int32_t dq_n_merges;
  int32_t dq_n_slots;
  const int32_t* kv_items;  /* optional device copy of bsattn_build_dkdv_schedule's items for the
                               CSC (needs it, with the same d); NULL = one dk/dv work-group per
                               group of key blocks, and the kv_ counts / merges must be 0 / NULL */
  int32_t kv_n_items;
  const int32_t* kv_merges; /* device copy of its merges (NULL if kv_n_merges == 0) */
  int32_t kv_n_merges;
  int32_t kv_n_slots;
} bsattn_prefill_bwd_args;

/* Workspace bytes of a backward call: one float per query row and head,
 * plus the partial sums and arrival counters of the schedules' slots
 * (dq_n_slots, kv_n_slots: 0 without a schedule).  0 for an invalid shape.
 * Calls may share a workspace (no initial contents are needed; the counters
 * are cleared by the call) if they do not overlap. */
size_t bsattn_prefill_bwd_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t Nq, int32_t d,
                                         int32_t dq_n_slots, int32_t kv_n_slots);

/*
 * Schedule of the backward dK/dV kernel over the CSC (col_ptr [Tc + 1],
 * row_idx: ascending query tiles per key block, bsattn_transpose_block_index)
 * for G query heads per K/V head and head dim d (which fixes the key blocks
 * per work-group: 1 at d = 64, 2 at d = 128).  A group of blocks visits, for
 * each query head, every tile of the union of its blocks' lists: G * |union|
 * positions.  A group with more than max_positions_per_item positions is cut
 * into near-equal chunks of consecutive positions.
 *   items  [n_items][8]  {group, first position, end position, head of the
 *                        first position, list positions (block 0, block 1)
 *                        of its tile, slot, merge}; slot = merge = -1: the
 *                        item writes dk/dv directly; longest first
 *   merges [n_merges][3] {group, first slot, number of slots}
 * Every group gets an item (one with no position writes zeros).  Two-call
 * pattern as bsattn_build_schedule.  Host buffers.  INVALID_ARG if col_ptr
 * decreases or a list is not strictly ascending.
 */
bsattn_status bsattn_build_dkdv_schedule(const int32_t* col_ptr, const int32_t* row_idx, int32_t Tc, int32_t G,
                                         int32_t d, int32_t max_positions_per_item, int32_t* items,
                                         int32_t items_capacity, int32_t* merges, int32_t merges_capacity,
                                         int32_t* n_items, int32_t* n_merges, int32_t* n_slots);

/* Enqueue the backward on `stream`.  Validation as for the forward (pointers
 * non-null and 16-byte aligned, strides multiples of 8 elements, d
 * contiguous), plus: CSR and CSC both given or both NULL, lse non-NULL.
 * The CSR and CSC contents are not read on the host.  BSATTN_ERR_HIP if a
 * launch fails. */
bsattn_status bsattn_prefill_bwd(const bsattn_prefill_bwd_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* decode (one new query token per sequence, split-KV + combine)              */
/* BLASST notes section 4.2: the decode kernel is memory bound; a skipped     */
/* block costs the K load and the score, never the V load nor the P.V work.  */
/* ------------------------------------------------------------------------ */

typedef struct {
  const void* q;          /* device bf16 [B, Hq, d]; query of the token at position L-1 */
  const void* k_cache;    /* device bf16 [B, Lmax, Hkv, d] */
  const void* v_cache;    /* device bf16 [B, Lmax, Hkv, d] */
  void* out;              /* device bf16 [B, Hq, d] */
  int32_t B, Hq, Hkv, L, Lmax, d; /* 1 <= L <= Lmax; d in {64, 128}; G = Hq/Hkv in {1, 2, 4, 8} */
  int64_t q_stride[2];    /* batch, head (elements) */
  int64_t kv_stride[3];   /* batch, token, head (elements), shared by k_cache and v_cache */
  int64_t o_stride[2];    /* batch, head */
  float scale;
  float lambda;           /* [0, 1) */
  int32_t Bc;             /* 64 */
  int32_t num_splits;     /* splits per (sequence, K/V head); 0 = automatic.  Never changes results
                             beyond float rounding order; never changes the skip set (except under
                             max_scope = 1, below) */
  void* workspace;        /* device, >= bsattn_decode_workspace_size(...) bytes, 256-byte aligned.
                             Its first 256 bytes are a header holding the health word (read by
                             bsattn_decode_check): zero them once before the first use (a zero
                             fill of the whole buffer does).  The rest needs no initial contents,
                             and calls of any shape may share the workspace: with lambda > 0 a
                             small kernel launched ahead of the split kernel zeroes the call's
                             split tickets and look-back flags.  Calls that share a workspace
                             must not overlap (same stream, or ordered by events). */
  size_t workspace_bytes;
  int32_t* counters;      /* optional device [B, Hkv, 2] int32: {visited, skipped} blocks, where a
                             skipped block is one whose V block no head of the group loads */
  uint8_t* block_state;   /* optional device [B, Hkv, Tc]: 1 computed, 2 skipped; with
                             decisions = 1 it is [B, Hq, Tc], the decision of each query head */
  int32_t block_order;    /* 0: ascending key blocks (Algorithm 1); 1: descending, most recent
                             keys first (block-row reordering, BLASST notes) */
  int32_t max_scope;      /* 0: the running max of the skip test spans the whole sequence in
                             visiting order (Algorithm 1, exact whatever the split count);
                             1: variant, the running max restarts at the first block of every
                             split, so the skip set depends on num_splits */
  int32_t decisions;      /* 0: one skip decision per group of G query heads sharing the K/V head
                             (the tile of Algorithm 1), which lets a skipped V block go unloaded;
                             1: variant, every query head decides for itself; a V block is then
                             loaded when any head of the group keeps it */
} bsattn_decode_args;

/* Workspace bytes for a decode call with these sizes (num_splits as in the args). */
size_t bsattn_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t L, int32_t d,
                                    int32_t Bc, int32_t num_splits);

/* Splits per (sequence, K/V head) a call with these sizes would use. */
int32_t bsattn_decode_num_splits(int32_t B, int32_t Hq, int32_t Hkv, int32_t L, int32_t d,
                                 int32_t Bc, int32_t num_splits);

/* Key blocks per split of such a call: split s holds visiting positions
 * [s * n, (s + 1) * n) of the block sequence (the last split may be shorter).
 * Needed to state the skip set under max_scope = 1.  0 for invalid sizes. */
int32_t bsattn_decode_split_blocks(int32_t B, int32_t Hq, int32_t Hkv, int32_t L, int32_t d,
                                   int32_t Bc, int32_t num_splits);

/* Enqueue the decode on `stream`: with lambda > 0 the clear of the call's
 * tickets and flags, the split kernel (BLASST skipping with the exact running
 * max), then the combine kernel (merge of the splits, attention tutorial
 * section 4.2); with lambda = 0 a single-pass split kernel and the combine. */
bsattn_status bsattn_decode_fwd(const bsattn_decode_args* args, void* stream);

/* Read and clear the decode workspace health word after the stream has
 * finished (host call, synchronous copies): 0 = fine, else a kernel-side wait
 * timed out (bit 0) or a split ticket fell out of range (bit 1) in a call
 * since the previous check, and that call's output is not valid.
 * workspace = NULL reads the scratch of bsattn_decode_fwd_noalloc on the
 * current device. */
bsattn_status bsattn_decode_check(void* workspace, int32_t* health_out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as bsattn_decode_fwd, but the workspace is a fixed scratch array of
 * 32 MiB that the library's code object holds on each GPU it runs on, from
 * the first call on that device (current device; the stream must belong to
 * it) until the process ends.  args->workspace must be NULL and
 * args->workspace_bytes 0 (else BSATTN_ERR_INVALID_ARG).  A call whose
 * workspace (bsattn_decode_workspace_size) exceeds 32 MiB returns
 * BSATTN_ERR_CAPACITY before enqueueing anything; for scale, 32 sequences x
 * 8 K/V heads x 131072 keys at d = 128 with automatic splits need about
 * 20 MiB.  No device memory is allocated or freed by the call.  Every call on
 * one GPU shares that GPU's scratch, and each call clears the tickets and
 * flags it uses: calls that overlap on one GPU (different streams without
 * ordering, several host threads) race and give undefined results.  Its
 * health word is read with bsattn_decode_check(NULL, ...). */
bsattn_status bsattn_decode_fwd_noalloc(const bsattn_decode_args* args, void* stream);

/* ------------------------------------------------------------------------ */
/* threshold calibration (host only)                                          */
/* ------------------------------------------------------------------------ */

/* BLASST notes section 3.2 and Algorithm 2: the best threshold follows
 * lambda = a / L.  For each context length lengths[k], the threshold of
 * lambdas[] whose measured sparsity sparsity[k * n_lambdas + i] (fraction of
 * visited blocks skipped, measured by the caller with the attention calls
 * above) lies closest to `target` is kept when that distance is strictly
 * below `delta` (the first of equal distances wins); *a_out is the slope of
 * the least-squares line through the origin on the kept (1 / L, lambda)
 * points and *n_points_out their number (0 leaves *a_out = NaN).
 * Host buffers; target in [0, 1], delta > 0, lambdas in (0, 1), lengths >= 1,
 * sparsities in [0, 1], else BSATTN_ERR_INVALID_ARG. */
bsattn_status bsattn_calibrate_threshold(double target, const int32_t* lengths, int32_t n_lengths,
                                         const double* lambdas, int32_t n_lambdas, const double* sparsity,
                                         double delta, double* a_out, int32_t* n_points_out);

#ifdef __cplusplus
}
#endif

#endif /* BSATTN_H */
