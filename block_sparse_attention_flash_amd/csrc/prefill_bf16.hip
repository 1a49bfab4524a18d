// bf16 prefill on CDNA4 matrix cores: block-sparse / BLASST flash attention.
//
// One work-group (4 waves, 256 threads) owns a tile of Br = 128 query rows
// of one (batch, query head); wave w owns rows 32w..32w+31.  The tile walks
// its visited key blocks (Bc = 64) in ascending order: the CSR list of a
// static block mask (DiT article section 3.3: the list is consulted before
// any K/V load) or every block up to the diagonal.  Per block:
//
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, K from LDS, Q held in registers
//   block row max, running max (BLASST notes Algorithm 1, lines 5-6)
//   [lambda > 0] tile-wide vote: block max - running max < ln(lambda) in
//                every row (notes section 3.1.1; per-lane predicate, wave
//                ballot, one LDS word per wave, as in notes section 4)
//   if kept:     P = 2^(S*scale*log2e - m),  l += rowsum(P),
//                O^T += V^T P^T  (V read transposed from LDS with
//                ds_read_b64_tr_b16: at d = 128 one key step at a time,
//                the first under the QK^T products, each later one under
//                the previous step's products; at d = 64 without the vote,
//                all four steps at once under the QK^T products)
//
// Layout choice: computing S^T (keys x rows) puts one query row per lane
// (row = lane % 32, split over lanes l and l+32), so the row max, the row
// sum and the rescale factor are per-lane values, and the S^T accumulator
// is already the B operand of the O^T MFMA after a bf16 pack - no LDS
// round trip for P.  O^T keeps the row in the lane as well, so rescaling O
// is a per-lane multiply.
//
// The running max is rescaled lazily: the reference max used in the
// exponent moves only when a row's max grows by more than 2^8, which keeps
// P <= 256 (exact in the bf16/fp32 ranges) and removes most O rescales.
// The skip test always uses the true running max.
//
// K/V blocks stream global -> LDS directly (buffer_load_dwordx4 ... lds,
// range-checked at the last key) into a two-stage ring, swizzled so that the
// K-fragment reads and the V transpose reads are bank-conflict free; block
// j+1 streams in during all of block j's work, and its block index is read
// two blocks ahead.  One barrier per block; the vote needs no second one
// (a wave waits for the others' words only when its own rows all agree).
// Several work-groups share a CU, so one group's exponentials overlap
// another's MFMAs.
//
// Long static tiles can be cut into chunks by a host schedule; a chunk
// publishes its (reference max, row sum, unnormalised O) and the last chunk
// of the tile to finish combines them in slot order (online-softmax
// rescaling, attention tutorial 4.2), in the same launch.  As in the BLASST notes
// section 4.1, the prefill still streams V for blocks it skips: prefill is
// compute bound and the load is issued one block ahead, before the skip
// decision is known.

#include "device_common.h"
#include "internal.h"

namespace bsattn {
namespace {

constexpr int BR = 128;
constexpr int BC = 64;
constexpr int NT = 256;
constexpr float kTau = 8.0f;  // lazy-rescale threshold, log2 units

typedef __attribute__((address_space(3))) void lds_void;

// 64 x D bf16 tile in LDS as 16-byte chunks, chunk c of row r stored at
// r*CH + (c ^ xor(r)).  K tiles are read 16 rows x 1 chunk at a time (MFMA A
// operand), V tiles 4 rows x 4 chunks (transpose reads): each gets its own
// swizzle so that either access pattern touches 64 distinct banks.
template <int D>
struct Tile {
  static constexpr int CH = D / 8;
  __device__ static __forceinline__ int kxor(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
  __device__ static __forceinline__ int vxor(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }
  __device__ static __forceinline__ int kpos(int r, int c) { return (r * CH + (c ^ kxor(r))) * 8; }
  __device__ static __forceinline__ int vpos(int r, int c) { return (r * CH + (c ^ vxor(r))) * 8; }
};

// K/V ring in LDS: two stages (block j+1 streams in during all of block j's
// work).  The loop also runs three (block j+2 requested while j is used); at
// d = 64 that measured no faster (0.0648 against 0.0639 ms on the DiT
// image+text workload), and at d = 128 it would not fit two work-groups per CU.
template <int D>
constexpr int kStages = 2;

template <int D>
struct Smem {
  __bf16 k[kStages<D>][BC * D];
  __bf16 v[kStages<D>][BC * D];
  int vote[2][4];  // [0][w]: wave w's vote word on the current block; also scratch after the loop
};

// Fourth word of a raw buffer descriptor on gfx9-family parts (32-bit data
// format, no swizzle; range checking against num_records).
constexpr int kBufferWord3 = 0x00020000;

// Global -> LDS loads of one 64-key tile (K or V) through a buffer
// descriptor whose range ends at the last key: rows of keys >= Nk read as
// zeros (hardware range check), which the score mask and P = 0 make
// harmless.  Lane (wave, lane) of instruction i moves one 16-byte chunk; its
// byte offset inside a tile is fixed, the tile's start is a scalar offset.
template <int D, bool IS_V>
struct TileSrc {
  static constexpr int NI = D / 32;  // instructions per wave per tile
  uint32_t voff[NI];                 // byte offset of (row, chunk) from the tile's first key
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ __forceinline__ void init(const __bf16* head, int64_t stride_t, int Nk, int wave, int lane) {
    constexpr int CH = D / 8;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int slot = (4 * i + wave) * 64 + lane;
      const int r = slot / CH, cp = slot % CH;
      const int c = cp ^ (IS_V ? Tile<D>::vxor(r) : Tile<D>::kxor(r));
      voff[i] = (uint32_t)(((int64_t)r * stride_t + c * 8) * 2);
    }
    const uint32_t extent = (uint32_t)(((int64_t)(Nk - 1) * stride_t + D) * 2);
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(head), (short)0, (int)extent, kBufferWord3);
  }
  __device__ __forceinline__ void issue(__bf16* tile, int64_t stride_t, int j, int wave) const {
    const uint32_t soff = (uint32_t)((int64_t)j * BC * stride_t * 2);
#pragma unroll
    for (int i = 0; i < NI; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + (4 * i + wave) * 64 * 8), 16, voff[i], soff,
                                               0, 0);
  }
};

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(ptr);
}

// The V fragments of one 16-key step of O^T += V^T P^T: for each of the NTD
// 32-wide d tiles, two ds_read_b64_tr_b16 (keys r and r + 8), issued together
// and waited for inside the same asm block.  base[n] is this lane's byte
// address for d tile n at key step 0; step kk adds 32 kk D bytes, the upper
// 8 keys 16 D bytes.  (The intrinsic form makes the compiler wait for every
// pending global->LDS load first: it cannot tell the V stage from the stage
// being filled.)  The loads return into their registers after the block has
// issued them, which the compiler does not see, while MFMAs issued just
// before may not have read their operands yet: those operands (`busy`, the
// previous step's fragments and P) are inputs of the block, so its outputs
// (early-clobber) are never placed on top of them.
template <int D, int KK>
__device__ __forceinline__ void read_v_step(bf16x8 (&vf)[D / 32], const uint32_t (&base)[D / 32],
                                            const bf16x8 (&busy)[D / 32], const bf16x8& busy_p) {
  constexpr int O0 = 32 * KK * D, O1 = 32 * KK * D + 16 * D;
  i16x4 x[2 * (D / 32)];
  if constexpr (D == 64) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%c6\n"
        "ds_read_b64_tr_b16 %1, %4 offset:%c7\n"
        "ds_read_b64_tr_b16 %2, %5 offset:%c6\n"
        "ds_read_b64_tr_b16 %3, %5 offset:%c7\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
        : "v"(base[0]), "v"(base[1]), "i"(O0), "i"(O1), "v"(busy[0]), "v"(busy[1]), "v"(busy_p)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%c12\n"
        "ds_read_b64_tr_b16 %1, %8 offset:%c13\n"
        "ds_read_b64_tr_b16 %2, %9 offset:%c12\n"
        "ds_read_b64_tr_b16 %3, %9 offset:%c13\n"
        "ds_read_b64_tr_b16 %4, %10 offset:%c12\n"
        "ds_read_b64_tr_b16 %5, %10 offset:%c13\n"
        "ds_read_b64_tr_b16 %6, %11 offset:%c12\n"
        "ds_read_b64_tr_b16 %7, %11 offset:%c13\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
        : "v"(base[0]), "v"(base[1]), "v"(base[2]), "v"(base[3]), "i"(O0), "i"(O1), "v"(busy[0]), "v"(busy[1]),
          "v"(busy[2]), "v"(busy[3]), "v"(busy_p)
        : "memory");
  }
#pragma unroll
  for (int n = 0; n < D / 32; ++n) vf[n] = join_bf16x4(x[2 * n], x[2 * n + 1]);
}

// d = 64: all four key steps' V fragments in one block of reads, issued
// while the QK^T products run (busy: the K fragments those products read).
__device__ __forceinline__ void read_v_all64(bf16x8 (&vf)[4][2], const uint32_t (&base)[2], const bf16x8 (&busy)[4]) {
  i16x4 x[16];
  asm volatile(
        "ds_read_b64_tr_b16 %0, %16 offset:0\n"
        "ds_read_b64_tr_b16 %1, %16 offset:1024\n"
        "ds_read_b64_tr_b16 %2, %17 offset:0\n"
        "ds_read_b64_tr_b16 %3, %17 offset:1024\n"
        "ds_read_b64_tr_b16 %4, %16 offset:2048\n"
        "ds_read_b64_tr_b16 %5, %16 offset:3072\n"
        "ds_read_b64_tr_b16 %6, %17 offset:2048\n"
        "ds_read_b64_tr_b16 %7, %17 offset:3072\n"
        "ds_read_b64_tr_b16 %8, %16 offset:4096\n"
        "ds_read_b64_tr_b16 %9, %16 offset:5120\n"
        "ds_read_b64_tr_b16 %10, %17 offset:4096\n"
        "ds_read_b64_tr_b16 %11, %17 offset:5120\n"
        "ds_read_b64_tr_b16 %12, %16 offset:6144\n"
        "ds_read_b64_tr_b16 %13, %16 offset:7168\n"
        "ds_read_b64_tr_b16 %14, %17 offset:6144\n"
        "ds_read_b64_tr_b16 %15, %17 offset:7168\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]), "=&v"(x[12]), "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15])
        : "v"(base[0]), "v"(base[1]), "v"(busy[0]), "v"(busy[1]), "v"(busy[2]), "v"(busy[3])
        : "memory");
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int n = 0; n < 2; ++n) vf[kk][n] = join_bf16x4(x[4 * kk + 2 * n], x[4 * kk + 2 * n + 1]);
}

// Partials combined per round trip by the last chunk of a cut tile.
template <int D>
constexpr int kMergeBatch = D == 64 ? 3 : 2;

template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Work-group barrier without the memory fence of __syncthreads (whose
// vmcnt(0) would also wait for the K/V blocks still streaming in).  Every
// wait it relies on is explicit: the block's own loads (vmcnt), and the LDS
// reads of the previous block, which each wave waits for before using them.
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Work-groups per CU the register budget is cut for: three at d = 64 (at most
// 168 VGPRs), two at d = 128 (at most 256).
template <int D>
constexpr int kMinBlocksPerCu = D == 64 ? kPrefillWgPerCu64 : kPrefillWgPerCu128;

// MAXONLY (with DYN): the pass that runs before a skipping launch whose
// schedule cuts tiles.  Each chunk of a cut tile writes, per query row, the
// maximum score over its blocks (no exponentials, no V); the main pass then
// starts a chunk's running max at the maximum of the chunks visited before
// it, which is the running max Algorithm 1 reaches there, so cut tiles take
// exactly the skip decisions of a whole-row walk.
template <int D, bool CAUSAL, bool DYN, bool MAXONLY>
__global__ __launch_bounds__(NT, kMinBlocksPerCu<D>) void prefill_bf16_kernel(const PrefillParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass needs only the launch stub
  constexpr int KS = D / 16;  // k-steps of the S MFMA
  constexpr int NTD = D / 32; // 32-wide d tiles of the O MFMA
  static_assert(NTD * 16 * NT == BR * D, "one partial = the accumulators of all threads");
  __shared__ Smem<D> sm;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: LDS addresses stay scalar
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- work item.  Work-group i runs on XCD i % 8.  When the (batch, kv
  //      head) groups divide into 8, group bg lives on XCD bg % 8, so its K/V
  //      stays in one L2, and the G query heads of a group are adjacent.  An
  //      XCD takes its work either rank-major (item ranks are longest first,
  //      so every group's long items start before any short one: the better
  //      tail when the XCD has few waves of work) or group-major (consecutive
  //      tiles of one group share K/V blocks in L2: better over many waves).
  const int units = p.sched_items ? p.n_items : p.Tr;
  const int G = p.Hq / p.Hkv;
  const int NBG = p.B * p.Hkv;
  int hh, rank = 0, bg, sub = 0;
  if (MAXONLY) {
    // grid: (slot, batch, head, kPreSplit sub-ranges), sub-range fastest
    int64_t k = blockIdx.x;
    sub = (int)(k % kPreSplit);
    k /= kPreSplit;
    const int h0 = (int)(k % p.Hq);
    k /= p.Hq;
    hh = h0 % G;
    bg = (int)(k % p.B) * p.Hkv + h0 / G;
    rank = (int)(k / p.B);  // the slot
  } else if ((NBG & 7) == 0) {
    const int per = NBG >> 3;
    int64_t k = blockIdx.x >> 3;
    hh = (int)(k % G);
    k /= G;
    if (p.rank_major) {
      bg = (int)(k % per) * 8 + (int)(blockIdx.x & 7);
      rank = (int)(k / per);
    } else {
      rank = (int)(k % units);
      bg = (int)(k / units) * 8 + (int)(blockIdx.x & 7);
    }
  } else {
    int64_t k = blockIdx.x;
    hh = (int)(k % G);
    k /= G;
    bg = (int)(k % NBG);
    rank = (int)(k / NBG);
  }
  const int g = bg % p.Hkv;
  const int b = bg / p.Hkv;
  const int h = g * G + hh;
  int t, e0, e1, slot = -1, mrg = -1;
  if (MAXONLY) {
    // chunk `slot` of a cut tile: its merge (slots are numbered merge by
    // merge, so the merge is the last one starting at or below the slot),
    // and its block range, cut exactly as the schedule builder cuts it
    slot = rank;
    int lo = 0, hi_m = p.n_merges;
    while (hi_m - lo > 1) {
      const int mid = (lo + hi_m) >> 1;
      if (p.sched_merges[3 * mid + 1] <= slot) lo = mid; else hi_m = mid;
    }
    mrg = lo;
    t = p.sched_merges[3 * mrg];
    const int c = slot - p.sched_merges[3 * mrg + 1], ns = p.sched_merges[3 * mrg + 2];
    const int rb = p.row_ptr[t], n = p.row_ptr[t + 1] - rb;
    e0 = rb + (int)((int64_t)n * c / ns);
    e1 = rb + (int)((int64_t)n * (c + 1) / ns);
  } else if (p.sched_items) {
    const int32_t* item = p.sched_items + 5 * rank;
    t = item[0];
    e0 = item[1];
    e1 = item[2];
    slot = item[3];
    mrg = item[4];
  } else {
    t = p.tile_order ? p.tile_order[rank] : (CAUSAL ? p.Tr - 1 - rank : rank);
    // a branch, not two selects: the compiler turns a select between a CSR
    // entry and p.Tc into one load through a select of the two addresses,
    // which needs a private copy of p.Tc and a flat load
    e0 = 0;
    e1 = p.Tc;
    if (p.row_ptr) {
      e0 = p.row_ptr[t];
      e1 = p.row_ptr[t + 1];
    }
  }
  // the work item is wave-uniform: keep it (and all block-index arithmetic
  // derived from it) in scalar registers
  t = __builtin_amdgcn_readfirstlane(t);
  e0 = __builtin_amdgcn_readfirstlane(e0);
  e1 = __builtin_amdgcn_readfirstlane(e1);
  slot = __builtin_amdgcn_readfirstlane(slot);
  mrg = __builtin_amdgcn_readfirstlane(mrg);
  if constexpr (MAXONLY) {
    const int s0 = p.sched_merges[3 * mrg + 1], ns = p.sched_merges[3 * mrg + 2];
    // this launch runs before the main one: it zeroes the merge's arrival
    // counter (the workspace may hold anything there, see the launcher)
    if (slot == s0 && sub == 0 && tid == 0) p.arrive[((int64_t)mrg * p.B + b) * p.Hq + h] = 0;
    // the chunk visited last (ascending: the highest slot; descending: the
    // lowest) has no later chunk that reads its maxima
    if (slot == (p.block_order ? s0 : s0 + ns - 1)) return;
  }

  const __bf16* qbase = static_cast<const __bf16*>(p.q) + (int64_t)b * p.qs_b + (int64_t)h * p.qs_h;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + (int64_t)b * p.vs_b + (int64_t)g * p.vs_h;

  const int row = t * BR + wave * 32 + l32;  // this lane's query row
  const bool row_ok = row < p.Nq;

  // Q fragment (B operand of S^T = K Q^T): lane holds Q[row][16 ks + 8 hi + 0..7]
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (row_ok)
      qf[ks] = *reinterpret_cast<const bf16x8*>(qbase + (int64_t)row * p.qs_t + 16 * ks + 8 * hi);
    else
      qf[ks] = bf16x8{};
  }

  // visited blocks: entries [e0, e1) of the CSR list (or blocks e0..e1-1),
  // minus blocks wholly above the diagonal
  const int last_row = min(t * BR + BR, p.Nq) - 1;
  const int32_t* cols = p.row_ptr ? p.col_idx + e0 : nullptr;
  int nblk = e1 - e0;
  if (CAUSAL) {
    if (cols) {  // ascending list: keep entries with j*BC <= last_row
      int lo = 0, hi2 = nblk;
      while (lo < hi2) {
        const int mid = (lo + hi2) >> 1;
        if (cols[mid] * BC <= last_row) lo = mid + 1; else hi2 = mid;
      }
      nblk = lo;
    } else {
      nblk = max(0, min(nblk, last_row / BC + 1 - e0));
    }
  }
  // MAXONLY: this work-group's share of the chunk, visiting positions
  // [first, first + nblk) (order does not matter for a maximum)
  int first = 0;
  if (MAXONLY) {
    first = (int)((int64_t)nblk * sub / kPreSplit);
    nblk = (int)((int64_t)nblk * (sub + 1) / kPreSplit) - first;
  }
  nblk = __builtin_amdgcn_readfirstlane(nblk);
  first = __builtin_amdgcn_readfirstlane(first);

  const float c2 = p.scale * kLog2e;                    // raw score -> log2 units
  const float log2_lambda = DYN ? log2f(p.lambda) : kNegInf;
  float m_run = kNegInf;   // true running max (raw score units)
  if (DYN && !MAXONLY && slot >= 0) {
    // a chunk of a cut tile starts from the maxima of the chunks visited
    // before it (ascending: lower slots; descending: higher slots)
    const int s0 = p.sched_merges[3 * mrg + 1];
    const int ns = p.sched_merges[3 * mrg + 2];
    const int lo = p.block_order ? slot + 1 : s0, hi_s = p.block_order ? s0 + ns : slot;
    for (int sl = lo; sl < hi_s; ++sl)
#pragma unroll
      for (int q = 0; q < kPreSplit; ++q)
        m_run = fmaxf(m_run, p.part_pre[((((int64_t)sl * p.B + b) * p.Hq + h) * kPreSplit + q) * BR + wave * 32 + l32]);
  }
  float m_chunk = kNegInf;  // MAXONLY: this row's maximum over the chunk
  float m_ref = kNegInf;   // reference max used in the exponent (raw units)
  // Row sums.  At d = 64 the vector ALUs are the busier unit, so the sums run
  // on the matrix core: an all-ones A operand makes every element of lacc in
  // lane l the sum of P over the keys of query row l % 32 (the same bf16 P the
  // numerator uses); only element 0 is read and rescaled.  At d = 128 the
  // matrix core is the busier one and the sums stay on the vector ALUs.
  constexpr bool kSumOnMfma = D == 64;
  // d = 64 without the vote: all of a block's V fragments fit beside the
  // scores, so they are read once, under the QK^T products
  constexpr bool kVAll = D == 64 && !DYN;
  f32x16 lacc = f32x16{};
  float l4[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // vector-ALU form: this lane's half, four partial sums
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
  f32x16 oacc[NTD];
#pragma unroll
  for (int n = 0; n < NTD; ++n) oacc[n] = f32x16{};
  int skipped = 0;
  int rows_agree = 0;  // row conditions that held (this wave's rows), for row_counters
  if (DYN && !MAXONLY && tid < 4) {  // vote words: no block yet (the first block barrier orders this)
    sm.vote[0][tid] = -1;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }

  constexpr int ST = kStages<D>;
  constexpr int DMA_PER_BLOCK = 2 * (D / 32);  // K and V loads of one block, per wave
  // CSR entries through the scalar cache (wave-uniform, read-only here), so
  // they never share the vector-memory counter with the K/V loads
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const const_i32_ptr ccols = cols ? (const_i32_ptr)(cols) : nullptr;
  // visiting position i -> key block: ascending, or descending (most recent keys first)
  const bool desc = !MAXONLY && p.block_order != 0;
  auto blk = [&](int i) __attribute__((always_inline)) {
    const int e = desc ? nblk - 1 - i : first + i;
    return i < nblk ? (ccols ? ccols[e] : e0 + e) : 0;
  };
  TileSrc<D, false> ksrc;
  TileSrc<D, true> vsrc;
  ksrc.init(kbase, p.ks_t, p.Nk, wave, lane);
  vsrc.init(vbase, p.vs_t, p.Nk, wave, lane);
  auto fetch = [&](int i, int jj) __attribute__((always_inline)) {
    const int stg = i % ST;
    ksrc.issue(sm.k[stg], p.ks_t, jj, wave);
    if constexpr (!MAXONLY) vsrc.issue(sm.v[stg], p.vs_t, jj, wave);
  };
  // block indices of blocks it .. it+3; the farthest is read a full iteration
  // (two at two stages) before its loads are issued
  int q0 = blk(0), q1 = blk(1), q2 = blk(2), q3 = ST == 3 ? blk(3) : 0;
  if (nblk > 0) fetch(0, q0);
  if (ST == 3 && nblk > 1) fetch(1, q1);

  const int g16 = lane >> 4, j16 = lane & 15;
  const int vr0 = 4 * (g16 >> 1) + (j16 >> 2);
  const int vcs = 2 * (g16 & 1) + ((j16 & 3) >> 1);
  const int vhalf = 4 * (j16 & 1);

  for (int it = 0; it < nblk; ++it) {
    const int stg = it % ST;
    const int j = q0;
    // block it has landed once at most the next block's loads are in flight
    // (block-state stores, when requested, also count: then wait for all)
    if (ST == 3 && it + 1 < nblk && !p.block_state) wait_vmem_le<(ST == 3 ? DMA_PER_BLOCK : 0)>();
    else wait_vmem_le<0>();
    block_barrier();  // block it visible; every wave is done with block it-1's stage
    // lgkmcnt(0): the block index read at the end of the last iteration has
    // long arrived; saying so (through the builtin the compiler tracks) keeps
    // its scalar load from coarsening the K-fragment waits below
    __builtin_amdgcn_s_waitcnt(0xC07F);
    // The next stage's loads: here in the static kernels; with the vote,
    // after it (below), so that their LDS writes land under the
    // exponentials and P.V instead of under the QK^T reads and the vote's
    // polls (measured: the causal GQA 32K launch 1-1.7 % faster, its sink
    // recipe 1.5-2.5 %; the same placement 0.5 % slower on the static video
    // mask).
    const int jf = ST == 3 ? q2 : q1;
    if (!DYN && it + ST - 1 < nblk) fetch(it + ST - 1, jf);
    q0 = q1;
    q1 = q2;
    if constexpr (ST == 3) q2 = q3;
    const __bf16* ktile = sm.k[stg];
    const __bf16* vtile = sm.v[stg];

    // ---- S^T = K Q^T : two 32-key tiles; K-fragment reads run four MFMAs ahead
    f32x16 sacc[2] = {f32x16{}, f32x16{}};
    uint32_t vb[NTD];
#pragma unroll
    for (int n = 0; n < NTD; ++n) vb[n] = lds_addr(vtile + Tile<D>::vpos(vr0, 4 * n + vcs) + vhalf);
    bf16x8 vall[4][2];
    bf16x8 va[NTD];
    {
      constexpr int NS = 2 * KS;
      auto kread = [&](int st) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8*>(ktile + Tile<D>::kpos(32 * (st & 1) + l32, 2 * (st >> 1) + hi));
      };
      bf16x8 kfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kfr[i] = kread(i);
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        sacc[st & 1] = mfma32(kfr[st & 3], qf[st >> 1], sacc[st & 1]);
        if (st + 4 < NS) kfr[st & 3] = kread(st + 4);
        __builtin_amdgcn_sched_barrier(0);
      }
      // the block's V fragments, under these products.  A wave issues a
      // product only when the matrix pipe takes it, so the products that may
      // not yet have read their operands when these loads land are the last
      // few QK^T ones (the previous block's P.V products were issued before
      // all of them): the K fragments of the last four are busy inputs, Q and
      // the scores stay live.
      if constexpr (kVAll) read_v_all64(vall, vb, kfr);
      // d = 128: the first key step's V fragments (same rule)
      if constexpr (D == 128 && !MAXONLY) read_v_step<D, 0>(va, vb, kfr, kfr[3]);
    }

    // ---- masks: causal diagonal, invalid keys, rows past Nq
    const bool need_mask = (j * BC + BC > p.n_valid) || (CAUSAL && j * BC + BC - 1 > t * BR);
    if (need_mask || !row_ok) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          const int key = j * BC + 32 * mt + 8 * (a >> 2) + 4 * hi + (a & 3);
          const bool ok = row_ok && key < p.n_valid && (!CAUSAL || key <= row);
          if (!ok) sacc[mt][a] = kNegInf;
        }
      }
    }

    // ---- block row max and running max
    float mb0 = kNegInf, mb1 = kNegInf;  // two independent chains
#pragma unroll
    for (int a = 0; a < 16; ++a) {
      mb0 = fmaxf(mb0, sacc[0][a]);
      mb1 = fmaxf(mb1, sacc[1][a]);
    }
    const float mb = wave_max_xor32(fmaxf(mb0, mb1));
    if constexpr (MAXONLY) {
      if (it + ST - 1 < nblk) fetch(it + ST - 1, jf);
      m_chunk = fmaxf(m_chunk, mb);
      if constexpr (ST == 3) q3 = blk(it + 4);
      else q2 = blk(it + 3);
      continue;
    }
    const float m_new = fmaxf(m_run, mb);

    bool skip = false;
    if (DYN) {
      const bool agree = (mb == kNegInf) || ((mb - m_new) * c2 < log2_lambda);
      const bool wave_all = __all(agree);
      // lanes l and l + 32 hold the same row: count the wave's 32 rows once
      if (p.row_counters) rows_agree += __popcll(__ballot(agree && row_ok) & 0xffffffffull);
      // one word per wave: 2 it + (every row of the wave agrees).  A wave
      // with a disagreeing row knows the block is kept and goes on; a wave
      // whose rows all agree waits for the other waves' words on this block.
      // Every wave writes its word before it can wait, and no wave passes
      // the next block's barrier before all have finished this one (so a
      // word is never overwritten while it is awaited): every wait ends.
      if (lane == 0) sm.vote[0][wave] = 2 * it + (wave_all ? 1 : 0);
      if (wave_all) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's word is in LDS
        const uint32_t yes = 2u * it + 1u;
        const uint32_t vote_addr = lds_addr(sm.vote[0]);
        for (;;) {
          // an LDS read, waited for in place: a volatile read through a
          // generic pointer becomes a flat load, whose vmcnt wait would also
          // drain the next block's K/V loads
          u32x4 w;
          asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(w) : "v"(vote_addr) : "memory");
          if (w[0] == yes - 1 || w[1] == yes - 1 || w[2] == yes - 1 || w[3] == yes - 1) break;  // kept
          if (w[0] == yes && w[1] == yes && w[2] == yes && w[3] == yes) {
            skip = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
    }
    if (DYN && it + ST - 1 < nblk) fetch(it + ST - 1, jf);
    if (p.block_state && tid == 0)
      p.block_state[(((int64_t)b * p.Hq + h) * p.Tr + t) * p.Tc + j] = skip ? 2 : 1;
    m_run = m_new;

    if (!skip) {
      // ---- lazy rescale of the reference max
      const bool need = (m_new != kNegInf) && (m_ref == kNegInf || (m_new - m_ref) * c2 > kTau);
      if (__any(need)) {
        const float alpha = need ? ((m_ref == kNegInf) ? 0.0f : fast_exp2((m_ref - m_new) * c2)) : 1.0f;
        if (need) m_ref = m_new;
        if constexpr (kSumOnMfma) {
          lacc[0] *= alpha;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) l4[i] *= alpha;
        }
#pragma unroll
        for (int n = 0; n < NTD; ++n)
#pragma unroll
          for (int a = 0; a < 16; ++a) oacc[n][a] *= alpha;
      }
      const float mref2 = (m_ref == kNegInf) ? 0.0f : m_ref * c2;
      // ---- P = 2^(S*c2 - m_ref*c2), row sums, pack to bf16 B-operand fragments
      bf16x8 pf[4];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          float pv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            pv[i] = fast_exp2(fmaf(sacc[mt][8 * hf + i], c2, -mref2));
            if constexpr (!kSumOnMfma) l4[i & 3] += pv[i];
          }
          pf[2 * mt + hf] = to_bf16x8(pv);
        }
      }
      // ---- O^T += V^T P^T : 4 key steps of 16 x NTD d tiles
      if constexpr (kVAll) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
          for (int n = 0; n < NTD; ++n) oacc[n] = mfma32(vall[kk][n], pf[kk], oacc[n]);
          lacc = mfma32(ones, pf[kk], lacc);
        }
      } else {
        // two fragment sets in turn: a step's loads never land on the operands
        // of the previous step's products.  At d = 128 the first step's set
        // was read under the QK^T products; at d = 64 it is read here, when no
        // product is in flight (the block row max waited for the last QK^T
        // product, and the matrix pipe runs a wave's products in order).
        bf16x8 vb2[NTD];
        if constexpr (D == 64) {
          const bf16x8 live[NTD] = {pf[2], pf[3]};
          read_v_step<D, 0>(va, vb, live, pf[1]);
        }
#pragma unroll
        for (int n = 0; n < NTD; ++n) oacc[n] = mfma32(va[n], pf[0], oacc[n]);
        if constexpr (kSumOnMfma) lacc = mfma32(ones, pf[0], lacc);
        read_v_step<D, 1>(vb2, vb, va, pf[0]);
#pragma unroll
        for (int n = 0; n < NTD; ++n) oacc[n] = mfma32(vb2[n], pf[1], oacc[n]);
        if constexpr (kSumOnMfma) lacc = mfma32(ones, pf[1], lacc);
        read_v_step<D, 2>(va, vb, vb2, pf[1]);
#pragma unroll
        for (int n = 0; n < NTD; ++n) oacc[n] = mfma32(va[n], pf[2], oacc[n]);
        if constexpr (kSumOnMfma) lacc = mfma32(ones, pf[2], lacc);
        read_v_step<D, 3>(vb2, vb, va, pf[2]);
#pragma unroll
        for (int n = 0; n < NTD; ++n) oacc[n] = mfma32(vb2[n], pf[3], oacc[n]);
        if constexpr (kSumOnMfma) lacc = mfma32(ones, pf[3], lacc);
      }
    } else {
      ++skipped;
    }
    // the farthest block index, read through the scalar cache after this
    // block's LDS traffic (its wait then costs nothing where it is used)
    if constexpr (ST == 3) q3 = blk(it + 4);
    else q2 = blk(it + 3);
  }
  if constexpr (MAXONLY) {
    if (hi == 0) p.part_pre[((((int64_t)slot * p.B + b) * p.Hq + h) * kPreSplit + sub) * BR + wave * 32 + l32] = m_chunk;
    return;
  }
  float l_tot;
  if constexpr (kSumOnMfma) {
    l_tot = lacc[0];
  } else {
    const float l_part = (l4[0] + l4[1]) + (l4[2] + l4[3]);
    l_tot = l_part + __shfl_xor(l_part, 32);
  }
  int vis_tot = nblk, skip_tot = skipped;
  int rows_tot = 0;  // row_counters: the work item's four waves (LDS words; the vote words are free now)
  if (p.row_counters) {
    __syncthreads();
    if (lane == 0) sm.vote[1][wave] = rows_agree;
    __syncthreads();
    rows_tot = sm.vote[1][0] + sm.vote[1][1] + sm.vote[1][2] + sm.vote[1][3];
  }

  if (slot >= 0) {
    // ---- chunk of a cut tile: publish the partial (unnormalised O relative
    //      to m_ref, plus m_ref and l), then take an arrival ticket; the last
    //      chunk to arrive combines all partials of the tile and stores O.
    const int s0 = p.sched_merges[3 * mrg + 1];
    const int ns = p.sched_merges[3 * mrg + 2];
    const int lrow = wave * 32 + l32;
    auto unit = [&](int sl) __attribute__((always_inline)) { return ((int64_t)sl * p.B + b) * p.Hq + h; };
    // partials are kept in accumulator order, element (16 n + a) of thread
    // tid at [16 n + a][tid]: each store / load instruction of a wave covers
    // 256 contiguous bytes
    {
      float* po = p.part_o + unit(slot) * BR * D + tid;
#pragma unroll
      for (int n = 0; n < NTD; ++n)
#pragma unroll
        for (int a = 0; a < 16; ++a) store_coherent(po + (16 * n + a) * NT, oacc[n][a]);
      if (hi == 0) {
        store_coherent(p.part_ml + (unit(slot) * BR + lrow) * 2 + 0, m_ref);
        store_coherent(p.part_ml + (unit(slot) * BR + lrow) * 2 + 1, l_tot);
      }
      if (tid == 0) {
        store_coherent(p.part_cnt + unit(slot) * 4 + 0, nblk);
        store_coherent(p.part_cnt + unit(slot) * 4 + 1, skipped);
        store_coherent(p.part_cnt + unit(slot) * 4 + 2, rows_tot);
      }
    }
    wait_stores_done();
    __syncthreads();  // every wave's partial has completed
    int32_t* arrive = p.arrive + ((int64_t)mrg * p.B + b) * p.Hq + h;
    if (tid == 0) sm.vote[0][0] = atomicAdd(arrive, 1);
    __syncthreads();
    if (sm.vote[0][0] != ns - 1) return;  // a later chunk merges
    if (tid == 0) store_coherent(arrive, 0);  // leave the counter at zero for the next call

    // ---- merge, in slot order, with the online rescaling rule:
    //      M' = max(M, m_s), a = 2^((M - M') c2), w = 2^((m_s - M') c2),
    //      O = a O + w O_s, l = a l + w l_s.  kMergeBatch slots per round
    //      trip (the own partial is read back like the others).
    constexpr int NB = kMergeBatch<D>;
    float M = kNegInf, l = 0.0f;
#pragma unroll
    for (int n = 0; n < NTD; ++n) oacc[n] = f32x16{};
    for (int base = s0; base < s0 + ns; base += NB) {
      float ms[NB], ls[NB];
      f32x16 os[NB][NTD];
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int sl = min(base + u, s0 + ns - 1);  // past the end: a valid slot, ignored below
        const float* ml = p.part_ml + (unit(sl) * BR + lrow) * 2;
        ms[u] = load_coherent(ml);
        ls[u] = load_coherent(ml + 1);
        const float* po = p.part_o + unit(sl) * BR * D + tid;
#pragma unroll
        for (int n = 0; n < NTD; ++n)
#pragma unroll
          for (int a = 0; a < 16; ++a) os[u][n][a] = load_coherent(po + (16 * n + a) * NT);
      }
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        if (base + u >= s0 + ns || ms[u] == kNegInf) continue;
        const float Mn = fmaxf(M, ms[u]);
        const float al = M == kNegInf ? 0.0f : fast_exp2((M - Mn) * c2);
        const float w = fast_exp2((ms[u] - Mn) * c2);
        M = Mn;
        l = fmaf(w, ls[u], l * al);
#pragma unroll
        for (int n = 0; n < NTD; ++n)
#pragma unroll
          for (int a = 0; a < 16; ++a) oacc[n][a] = fmaf(w, os[u][n][a], oacc[n][a] * al);
      }
    }
    l_tot = l;
    m_ref = M;
    if ((p.tile_counters || p.row_counters) && tid == 0) {
      vis_tot = skip_tot = 0;
      int rows_own = rows_tot;
      rows_tot = 0;
      for (int sl = s0; sl < s0 + ns; ++sl) {
        vis_tot += sl == slot ? nblk : load_coherent(p.part_cnt + unit(sl) * 4);
        skip_tot += sl == slot ? skipped : load_coherent(p.part_cnt + unit(sl) * 4 + 1);
        rows_tot += sl == slot ? rows_own : load_coherent(p.part_cnt + unit(sl) * 4 + 2);
      }
    }
  }

  // ---- epilogue: O / l, bf16 store
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (row_ok) {
    __bf16* obase =
        static_cast<__bf16*>(p.out) + (int64_t)b * p.os_b + (int64_t)row * p.os_t + (int64_t)h * p.os_h;
#pragma unroll
    for (int n = 0; n < NTD; ++n) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dcol = 32 * n + 8 * q4 + 4 * hi;
        f32x4 v4 = {oacc[n][4 * q4 + 0] * inv, oacc[n][4 * q4 + 1] * inv, oacc[n][4 * q4 + 2] * inv,
                    oacc[n][4 * q4 + 3] * inv};
        *reinterpret_cast<bf16x4*>(obase + dcol) = __builtin_convertvector(v4, bf16x4);
      }
    }
  }
  if (p.lse && row_ok && hi == 0)  // ln(sum exp(scale s)) = m scale + ln(l), l relative to m_ref
    p.lse[((int64_t)b * p.Hq + h) * p.Nq + row] = l_tot > 0.0f ? fmaf(m_ref, p.scale, logf(l_tot)) : kNegInf;
  if (p.tile_counters && tid == 0) {
    int32_t* tc = p.tile_counters + 2 * ((((int64_t)b * p.Hq + h) * p.Tr) + t);
    tc[0] = vis_tot;
    tc[1] = skip_tot;
  }
  if (p.row_counters && tid == 0) p.row_counters[((int64_t)b * p.Hq + h) * p.Tr + t] = rows_tot;
#endif
}

// Zero n words (the arrival counters of a call whose schedule cuts tiles).
__global__ __launch_bounds__(NT) void clear_words_kernel(int32_t* w, int n) {
  for (int i = blockIdx.x * NT + threadIdx.x; i < n; i += gridDim.x * NT) w[i] = 0;
}

template <int D, bool CAUSAL, bool DYN>
hipError_t launch(const PrefillParams& p0, hipStream_t s) {
  PrefillParams p = p0;
  const int64_t units = p.sched_items ? p.n_items : p.Tr;
  const int64_t grid = (int64_t)p.B * p.Hq * units;
  p.rank_major = prefill_group_major(p.B, p.Hq, p.Hkv, D, units) ? 0 : 1;
  // Cut tiles: the arrival counters sit at offsets that depend on the call's
  // shape (n_slots), so a workspace reused with another shape may hold any
  // bytes there.  A launch before the main one zeroes them: the chunk-maximum
  // pass when lambda > 0 (kPreSplit work-groups per chunk and head), else a
  // small clear kernel.
  if (DYN && p.n_slots > 0) {
    const int64_t pre_grid = (int64_t)p.n_slots * p.B * p.Hq * kPreSplit;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, true, true>), dim3((unsigned)pre_grid), dim3(NT), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (p.n_slots > 0) {
    const int n = p.n_merges * p.B * p.Hq;
    hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)min(64, (n + NT - 1) / NT)), dim3(NT), 0, s, p.arrive, n);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, DYN, false>), dim3((unsigned)grid), dim3(NT), 0, s, p);
  return hipGetLastError();
}

template <int D>
hipError_t dispatch_d(const PrefillParams& p, hipStream_t s) {
  const bool dyn = p.lambda > 0.0f;
  if (p.causal) return dyn ? launch<D, true, true>(p, s) : launch<D, true, false>(p, s);
  return dyn ? launch<D, false, true>(p, s) : launch<D, false, false>(p, s);
}

}  // namespace

int launch_prefill_bf16(const PrefillParams& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return p.d == 64 ? dispatch_d<64>(p, s) : dispatch_d<128>(p, s);
}

}  // namespace bsattn
