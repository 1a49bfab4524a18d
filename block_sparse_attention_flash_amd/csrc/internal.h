// Internal declarations shared by the host-side translation units of libbsattn.
#pragma once

#include <cstdint>
#include <vector>

#include "../../include/bsattn.h"

namespace bsattn {

// thread-local error message (api.cpp)
bsattn_status fail(bsattn_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

bsattn_status validate_spec(const bsattn_mask_spec* spec, int32_t n_k);
bsattn_status build_block_index(const bsattn_mask_spec* spec, int32_t n_q, int32_t n_k, int32_t Br, int32_t Bc,
                                std::vector<int32_t>& row_ptr, std::vector<int32_t>& col_idx);

// Validated, normalised launch parameters.  Strides are in elements.
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int32_t B, Hq, Hkv, Nq, Nk, d;
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_t, os_h;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* tile_order;
  int32_t n_valid;
  float scale;
  float lambda;
  int32_t causal;
  int32_t Br, Bc;
  int32_t Tr, Tc;
  int32_t* tile_counters;
  uint8_t* block_state;
  int32_t* row_counters;
  int32_t block_order;
  const int32_t* sched_items;   // [n_items][5] or NULL
  int32_t n_items;
  const int32_t* sched_merges;  // [n_merges][3]
  int32_t n_merges;
  int32_t n_slots;
  float* part_o;                // [n_slots][B][Hq][128 * d], in accumulator order (see the kernel)
  float* part_ml;               // [n_slots][B][Hq][128][2]  (reference max in raw score units, row sum)
  int32_t* part_cnt;            // [n_slots][B][Hq][4] {visited, skipped, rows agreeing, unused}
  int32_t* arrive;              // [n_merges][B][Hq] chunk arrival counters (zero between calls)
  float* part_pre;              // [n_slots][B][Hq][kPreSplit][128] lambda > 0: per-row max of each share of a chunk
  int32_t rank_major;           // bf16 kernel: XCD work order (set by its launcher)
  float* lse;                   // optional [B][Hq][Nq] natural-log row sums of exp
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dvec;                  // [B][Hq][Nq] rowsum(dout * out)
  int32_t B, Hq, Hkv, Nq, Nk, d;
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_t, os_h;
  int64_t dos_b, dos_t, dos_h;
  int64_t dqs_b, dqs_t, dqs_h;
  int64_t dks_b, dks_t, dks_h;
  int64_t dvs_b, dvs_t, dvs_h;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const int32_t* col_ptr;
  const int32_t* row_idx;
  int32_t n_valid;
  float scale;
  int32_t causal;
  int32_t Tr, Tc;
  const uint8_t* block_state;   // optional [B][Hq][Tr][Tc] of a skipping forward: 2 = no gradient
  const int32_t* dq_items;      // [dq_n_items][5] schedule of the dQ kernel over the CSR, or NULL
  int32_t dq_n_items;
  const int32_t* dq_merges;     // [dq_n_merges][3]
  int32_t dq_n_merges;
  float* dq_part;               // [dq_n_slots][B][Hq][128 * d] partial dQ^T in accumulator order
  int32_t* dq_arrive;           // [dq_n_merges][B][Hq] chunk arrival counters
  const int32_t* kv_items;      // [kv_n_items][kKvItemInts] schedule of the dK/dV kernel over the CSC, or NULL
  int32_t kv_n_items;
  const int32_t* kv_merges;     // [kv_n_merges][3]
  int32_t kv_n_merges;
  float* kv_part;               // [kv_n_slots][B][Hkv][blocks per group * 2 * 2 * d * 64] partial dK, dV
  int32_t* kv_arrive;           // [kv_n_merges][B][Hkv]
};

int launch_prefill_bwd(const BwdParams& p, void* stream);

// Work-groups per chunk of a cut tile in the chunk-maximum pass (each takes
// an equal share of the chunk's blocks and keeps its own row maxima).
constexpr int kPreSplit = 8;

struct PrefillWorkspace {
  size_t o, ml, cnt, arrive, pre, total;
};
PrefillWorkspace prefill_workspace_layout(int32_t B, int32_t Hq, int32_t d, int32_t n_slots);

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  int32_t B, Hq, Hkv, L, d, G;
  int64_t qs_b, qs_h;
  int64_t ks_b, ks_t, ks_h;  // shared by k and v
  int64_t os_b, os_h;
  float scale;
  float lambda;
  int32_t Bc;
  int32_t Tc;
  int32_t num_splits;      // per (sequence, kv head)
  int32_t blocks_per_split;
  void* workspace;
  int32_t* counters;
  uint8_t* block_state;
  int32_t block_order;
  int32_t split_reset;     // running max restarts per split (variant)
  int32_t per_head;        // skip decisions per query head (variant)
};

// Decode workspace layout (all offsets 256-byte aligned), see decode.hip.
struct DecodeWorkspace {
  size_t header;    // [1]: health word (sticky until bsattn_decode_check reads it)
  size_t tickets;   // int32 [B*Hkv]: split tickets per (sequence, kv head)
  size_t flags;     // int32 [B*Hkv*S]
  size_t agg;       // float [B*Hkv*S*16]  split aggregate max per row
  size_t incl;      // float [B*Hkv*S*16]  inclusive prefix max per row
  size_t stats;     // float [B*Hkv*S*G*2] partial (m, l)
  size_t acc;       // float [B*Hkv*S*G*d] partial unnormalised output
  size_t counts;    // int32 [B*Hkv*S] skipped blocks per split
  size_t total;
};
DecodeWorkspace decode_workspace_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t d, int32_t S);
int32_t decode_choose_splits(int32_t B, int32_t Hkv, int32_t Tc, int32_t G, int32_t requested,
                             int32_t* blocks_per_split);

// Fixed device scratch of the no-allocation decode (decode.hip): its size,
// and its address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
int noalloc_scratch(void** ptr);

// Kernel launchers (HIP translation units).  Return hipError_t as int.
int launch_prefill_bf16(const PrefillParams& p, void* stream);
// Key blocks per work-group of the backward dK/dV kernel (they share each
// query stage's loads): one at d = 64, two at d = 128.
constexpr int kDkdvBlocks64 = 1;
constexpr int kDkdvBlocks128 = 2;
// Ints per item of a dK/dV schedule: {key-block group, first position, end
// position, head of the first position, list positions of both blocks at
// the first position, slot, merge}.
constexpr int kKvItemInts = 8;

struct BwdWorkspace {
  size_t dvec, dq_part, dq_arrive, kv_part, kv_arrive, total;
};
BwdWorkspace bwd_workspace_layout(int32_t B, int32_t Hq, int32_t Hkv, int32_t Nq, int32_t d, int32_t dq_n_slots,
                                  int32_t kv_n_slots);

// Resident work-groups per CU of the bf16 prefill kernel (its launch bounds).
constexpr int kPrefillWgPerCu64 = 3;
constexpr int kPrefillWgPerCu128 = 2;
// Work order of a bf16 prefill launch over `units` work items per head (tiles,
// or schedule items): true = group-major (each XCD walks one (batch, K/V
// head) group's items consecutively), false = rank-major.
bool prefill_group_major(int B, int Hq, int Hkv, int d, int64_t units);
int launch_prefill_f32(const PrefillParams& p, void* stream);
int launch_decode(const DecodeParams& p, void* stream);

}  // namespace bsattn
