// BLASST decode: split-KV attention of one new query token per sequence
// against a bf16 KV cache, then a combine kernel.
//
// BLASST notes section 4.2: decode is memory bound, so a skipped block must
// save the V-block load (and the P.V work); only the K block and its scores
// are paid for.  The skip rule is Algorithm 1's, with the tile being the G
// query heads that share one K/V head (notes section 4: the decision is
// shared by the tile), and the running max spanning the whole sequence in
// ascending block order.  A per-split running max would make the skip set
// depend on the split count; instead each split learns the exact maximum of
// all earlier blocks through a single-pass decoupled look-back (Merrill and
// Garland, "Single-pass Parallel Prefix Scan with Decoupled Look-back",
// 2016), applied to the max operator:
//
//   phase 1  stream the split's K blocks (each wave its own blocks, the next
//            block prefetched into registers), scores q.K^T (G rows x 64 keys
//            per block) with the 16x16x32 bf16 MFMA, block row maxima only
//   publish  the split aggregate (max over its blocks), look back over earlier
//            splits for their inclusive prefix, publish the inclusive prefix
//   phase 2  running max within the split seeded with the exclusive prefix,
//            tile-wide skip decision per block (strict <, as printed)
//   phase 3  kept blocks only: their scores (kept in LDS since phase 1 where
//            that costs no occupancy, else recomputed bit for bit from a K
//            reload: same MFMA on the same data) and V,
//            P = 2^(s - m_ref), O_partial = P V on the vector ALUs (G <= 8
//            rows), write the partial (m_ref, l, O) of the split.  Where the
//            registers do not already hold a CU to two work-groups, the
//            scores stay out of LDS: the work-group stays small, so enough of
//            them share a CU to keep HBM busy while some sit in phases 2-3.
//   combine  merge the splits of each (sequence, head): online-softmax
//            rescaling (attention tutorial section 4.2)
//
// The tickets and look-back flags of a call are cleared by a small kernel
// launched just before the split kernel, on the same stream.  Their offsets
// depend on the call's shape (the split count S), so a workspace reused with
// another shape may hold any bytes there (an earlier call's partials); the
// clear makes every word the split kernel waits on or counts with start at
// zero whatever the workspace held.  Only the health word in the fixed
// header must be zero before the first call.
//
// Forward progress: a work-group takes its (sequence, K/V head) from its index
// and its split number from an atomic ticket of that pair, so a split only
// ever waits for splits that already hold a ticket, i.e. are resident or
// finished.  One counter per pair keeps the ticket atomics from serialising on
// a single address.  Every wait is also bounded; a timed-out wait sets the
// workspace health word instead of hanging.

#include <mutex>

#include "device_common.h"
#include "internal.h"

namespace bsattn {

// ---------------------------------------------------------------------------
// Scratch of bsattn_decode_fwd_noalloc: the decode workspace (health header,
// tickets, flags, split aggregates, partials) in a fixed device array of the
// library's code object, for callers that cannot allocate device memory.
// Each GPU the library runs on holds its own copy for the life of the
// process.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is taken once per device with
// hipGetSymbolAddress (that device current) and only that address is used.
// The array starts zeroed (the health word must), and every call clears the
// tickets and flags it uses; calls on one GPU share it and must not overlap.
// ---------------------------------------------------------------------------

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

namespace {

constexpr int NT = 256;
constexpr int BC = 64;
constexpr int kSpinLimit = 1 << 20;  // ~1 s; a normal wait is well under 1 ms

// Look-back words are written and read with the device-coherent helpers of
// device_common.h; the flag is stored only after the value stores completed.
__device__ __forceinline__ void publish_flag(int* flag, int v) {
  wait_stores_done();
  __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait for a look-back flag.  Bounded: gives up after kSpinLimit polls, or at
// once when another work-group has already given up (health word set).
__device__ __forceinline__ int spin_flag(const int* flag, int* health) {
  for (int n = 0; n < kSpinLimit; ++n) {
    const int f = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (f != 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      return f;
    }
    if (__hip_atomic_load(health, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return 0;
    __builtin_amdgcn_s_sleep(2);
  }
  atomicOr(health, 1);
  return 0;
}

// Phase 1 keeps every block's scores in LDS for phase 3 (no K reload for kept
// blocks) where that costs no occupancy: at d = 128 the registers already
// limit a CU to two work-groups (G <= 4; 64 KB more LDS still fits two) or to
// one (G = 8; 128 KB more still fits).
template <int D, int G>
constexpr bool kKeepScores = D == 128;
template <int G>
constexpr int kScoreRows = G <= 4 ? 4 : 8;  // rows 4 q16 + i of lanes q16 < kScoreRows / 4

template <int D, int G>
struct DecSmem {
  float sc[kKeepScores<D, G> ? 64 : 1][64][kScoreRows<G>];  // scores [block][key][row]
  float bm[64][G];              // block row maxima (log2 units)
  float m_ref[G];
  float lsum[4][G];
  float pre[G];
  uint64_t rskip[G];            // per-head variant: blocks each head skips (else 0)
  float pbuf[4][G][64];         // per-wave P of the kept block in flight
  int kept[64];
  int nkept;
  int ticket;
  float obuf[4][G][D];
};

template <int D>
__device__ __forceinline__ void load_k_block(bf16x8 (&kf)[4][D / 32], const __bf16* kbase, int64_t ks_t, int j, int L,
                                             int r16, int q16) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    const int key = min(j * BC + 16 * kt + r16, L - 1);  // past L: any valid key, masked below
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      kf[kt][ks] = *reinterpret_cast<const bf16x8*>(kbase + (int64_t)key * ks_t + 32 * ks + 8 * q16);
  }
}

// scores (log2 units) of one block: acc[kt][i] = row 4*q16+i, key 16*kt + r16
template <int D>
__device__ __forceinline__ void block_scores(f32x4 (&acc)[4], const bf16x8 (&kf)[4][D / 32], const bf16x8 (&qa)[D / 32],
                                             float c2, int j, int L, int r16) {
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
    f32x4 a = f32x4{};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) a = mfma16(qa[ks], kf[kt][ks], a);
    const bool ok = j * BC + 16 * kt + r16 < L;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[kt][i] = ok ? a[i] * c2 : kNegInf;
  }
}

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Zero the tickets [B*Hkv] and look-back flags [B*Hkv*S] of this call.
__global__ __launch_bounds__(NT) void decode_clear_kernel(int* tickets, int n_tickets, int* flags, int n_flags) {
  const int stride = gridDim.x * NT;
  for (int i = blockIdx.x * NT + threadIdx.x; i < n_tickets; i += stride) tickets[i] = 0;
  for (int i = blockIdx.x * NT + threadIdx.x; i < n_flags; i += stride) flags[i] = 0;
}

template <int D, int G>
__global__ __launch_bounds__(NT) void decode_split_kernel(const DecodeParams p, DecodeWorkspace wl) {
  __shared__ DecSmem<D, G> sm;
  constexpr int KS = D / 32;   // k-steps of the 16x16x32 MFMA
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  char* ws = static_cast<char*>(p.workspace);
  int* header = reinterpret_cast<int*>(ws + wl.header);
  int* flags = reinterpret_cast<int*>(ws + wl.flags);
  float* aggv = reinterpret_cast<float*>(ws + wl.agg);
  float* inclv = reinterpret_cast<float*>(ws + wl.incl);
  float* stats = reinterpret_cast<float*>(ws + wl.stats);
  float* accw = reinterpret_cast<float*>(ws + wl.acc);
  int* counts = reinterpret_cast<int*>(ws + wl.counts);

  const int S = p.num_splits;
  // pair-major: the S work-groups of one (sequence, K/V head) are consecutive,
  // so a pair's last splits (where recent keys usually keep blocks, making
  // phase 3 long) finish while later pairs still stream K, not all at the end
  const int pair = blockIdx.x / S;
  int* tickets = reinterpret_cast<int*>(ws + wl.tickets);
  if (tid == 0) sm.ticket = atomicAdd(&tickets[pair], 1);
  __syncthreads();
  const int s = sm.ticket;
  if (s < 0 || s >= S) {  // cannot happen after the clear kernel; never index past the workspace
    if (tid == 0) atomicOr(&header[1], 2);
    return;
  }
  const int b = pair / p.Hkv, g = pair % p.Hkv;
  const int unit = pair * S + s;
  // split s in visiting order: ascending, its blocks are [s bps, (s+1) bps);
  // descending (most recent keys first), split 0 holds the last blocks
  const int desc = p.block_order;
  const int blk0 = desc ? max(0, p.Tc - (s + 1) * p.blocks_per_split) : s * p.blocks_per_split;
  const int nb = desc ? p.Tc - s * p.blocks_per_split - blk0 : min(p.blocks_per_split, p.Tc - blk0);
  const float c2 = p.scale * kLog2e;

  const __bf16* qbase = static_cast<const __bf16*>(p.q) + (int64_t)b * p.qs_b;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;

  // A operand = q rows (row = lane%16 < G, zero otherwise), B operand = K keys.
  const int r16 = lane & 15, q16 = lane >> 4;
  bf16x8 qa[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if (r16 < G)
      qa[ks] = *reinterpret_cast<const bf16x8*>(qbase + (int64_t)(g * G + r16) * p.qs_h + 32 * ks + 8 * q16);
    else
      qa[ks] = bf16x8{};
  }

  // ---- phase 1: block maxima, K streamed with one block of register prefetch
  if (wave < nb) {
    bf16x8 kcur[4][KS], knxt[4][KS];
    load_k_block<D>(kcur, kbase, p.ks_t, blk0 + wave, p.L, r16, q16);
    for (int lb = wave; lb < nb; lb += 4) {
      if (lb + 4 < nb) load_k_block<D>(knxt, kbase, p.ks_t, blk0 + lb + 4, p.L, r16, q16);
      f32x4 acc[4];
      block_scores<D>(acc, kcur, qa, c2, blk0 + lb, p.L, r16);
      if constexpr (kKeepScores<D, G>) {
        if (q16 < kScoreRows<G> / 4)  // rows 4 q16 .. 4 q16 + 3 of key 16 kt + r16
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) *reinterpret_cast<f32x4*>(&sm.sc[lb][16 * kt + r16][4 * q16]) = acc[kt];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = fmaxf(fmaxf(acc[0][i], acc[1][i]), fmaxf(acc[2][i], acc[3][i]));
        x = fmaxf(x, __shfl_xor(x, 1));
        x = fmaxf(x, __shfl_xor(x, 2));
        x = fmaxf(x, __shfl_xor(x, 4));
        x = fmaxf(x, __shfl_xor(x, 8));
        const int row = 4 * q16 + i;
        if (r16 == 0 && row < G) sm.bm[lb][row] = x;
      }
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kcur[kt][ks] = knxt[kt][ks];
    }
  }
  __syncthreads();

  // ---- publish aggregate, look back, publish inclusive prefix ----------------
  // (per-split variant: no prefix, the running max starts afresh in the split)
  if (tid == 0 && p.split_reset) {
#pragma unroll
    for (int r = 0; r < G; ++r) sm.pre[r] = kNegInf;
  } else if (tid == 0) {
    float agg[G];
#pragma unroll
    for (int r = 0; r < G; ++r) {
      float x = kNegInf;
      for (int lb = 0; lb < nb; ++lb) x = fmaxf(x, sm.bm[lb][r]);
      agg[r] = x;
      store_coherent(&aggv[unit * 16 + r], x);
    }
    publish_flag(&flags[unit], 1);
    float pre[G];
#pragma unroll
    for (int r = 0; r < G; ++r) pre[r] = kNegInf;
    for (int q = s - 1; q >= 0; --q) {
      const int u = pair * S + q;
      const int f = spin_flag(&flags[u], &header[1]);
      if (f == 0) break;  // timed out: health word set, result invalid
      const float* src = (f == 2) ? inclv : aggv;
#pragma unroll
      for (int r = 0; r < G; ++r) pre[r] = fmaxf(pre[r], load_coherent(src + u * 16 + r));
      if (f == 2) break;
    }
#pragma unroll
    for (int r = 0; r < G; ++r) {
      store_coherent(&inclv[unit * 16 + r], fmaxf(pre[r], agg[r]));
      sm.pre[r] = pre[r];
    }
    publish_flag(&flags[unit], 2);
  }
  __syncthreads();

  // ---- phase 2: skip decisions (wave 0; lane r < G runs row r) --------------
  if (wave == 0) {
    const bool dyn = p.lambda > 0.0f;
    const float log2_lambda = dyn ? log2f(p.lambda) : kNegInf;
    uint64_t agree = ~0ull;
    if (lane < G) {
      float cm = sm.pre[lane];
      agree = 0ull;
      for (int v = 0; v < nb; ++v) {  // the running max in visiting order
        const int lb = desc ? nb - 1 - v : v;
        const float x = sm.bm[lb][lane];
        cm = fmaxf(cm, x);
        if (x == kNegInf || x - cm < log2_lambda) agree |= (1ull << lb);
      }
    }
    const uint64_t valid = nb == 64 ? ~0ull : ((1ull << nb) - 1ull);
    const uint64_t own = dyn ? (agree & valid) : 0ull;  // this row's own test (lanes >= G: all)
    // all rows must agree
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t other = ((uint64_t)__shfl_xor((unsigned)(agree >> 32), o) << 32) |
                             (uint64_t)(unsigned)__shfl_xor((unsigned)agree, o);
      agree &= other;
    }
    const uint64_t skipm = dyn ? (agree & valid) : 0ull;  // no head computes these
    const uint64_t keepm = valid & ~skipm;
    if (lane < G) {
      // a row's reference max spans the blocks the row itself computes
      const uint64_t rowkeep = valid & ~(p.per_head ? own : skipm);
      float mr = kNegInf;
      for (int lb = 0; lb < nb; ++lb)
        if ((rowkeep >> lb) & 1ull) mr = fmaxf(mr, sm.bm[lb][lane]);
      sm.m_ref[lane] = mr;
      sm.rskip[lane] = p.per_head ? own : 0ull;
    }
    if (lane == 0) {
      int n = 0;
      for (int lb = 0; lb < nb; ++lb)
        if ((keepm >> lb) & 1ull) sm.kept[n++] = lb;
      sm.nkept = n;
      counts[unit] = __popcll(skipm);
    }
    if (p.block_state && p.per_head) {  // [B, Hq, Tc]: each head's own decisions
      lds_fence();                       // sm.rskip written above by this wave
      for (int x = lane; x < G * nb; x += 64) {
        const int r = x / nb, lb = x % nb;
        p.block_state[((int64_t)b * p.Hq + g * G + r) * p.Tc + blk0 + lb] = ((sm.rskip[r] >> lb) & 1ull) ? 2 : 1;
      }
    } else if (p.block_state) {
      for (int lb = lane; lb < nb; lb += 64)
        p.block_state[((int64_t)b * p.Hkv + g) * p.Tc + blk0 + lb] = ((skipm >> lb) & 1ull) ? 2 : 1;
    }
  }
  __syncthreads();
  const int nkept = sm.nkept;

  // ---- phase 3: kept blocks, one per wave at a time --------------------------
  constexpr int DCH = D / 8;        // 16-byte chunks per key row
  constexpr int KPS = 64 / DCH;     // keys per load step across the wave
  constexpr int STEPS = BC / KPS;
  const int dch = lane % DCH, kg = lane / DCH;
  float acc[G][8];
#pragma unroll
  for (int r = 0; r < G; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
  float lpart[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // rows 4*q16+i, keys of this lane
  float mref_l[4];
  uint64_t rskip_l[4];  // per-head variant: a row's skipped blocks get P = 2^(s - inf) = 0
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * q16 + i;
    mref_l[i] = row < G ? sm.m_ref[row] : 0.0f;
    rskip_l[i] = row < G ? sm.rskip[row] : 0ull;
  }
  for (int k = wave; k < nkept; k += 4) {
    const int lb = sm.kept[k];
    const int j = blk0 + lb;
    float mb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mb[i] = ((rskip_l[i] >> lb) & 1ull) ? kPosInf : mref_l[i];
    bf16x8 kf[4][KS];
    if constexpr (!kKeepScores<D, G>) load_k_block<D>(kf, kbase, p.ks_t, j, p.L, r16, q16);
    u32x4 vv[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int key = j * BC + st * KPS + kg;
      vv[st] = key < p.L ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * p.ks_t + 8 * dch)
                         : u32x4{0, 0, 0, 0};
    }
    f32x4 sc[4];
    if constexpr (kKeepScores<D, G>) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)  // lanes past the stored rows hold no row (row >= G): any stored value
        sc[kt] = *reinterpret_cast<const f32x4*>(&sm.sc[lb][16 * kt + r16][4 * (q16 % (kScoreRows<G> / 4))]);
    } else {
      block_scores<D>(sc, kf, qa, c2, j, p.L, r16);
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * q16 + i;
        if (row < G) {
          const float e = fast_exp2(sc[kt][i] - mb[i]);  // 2^-inf = 0 for keys >= L
          lpart[i] += e;
          sm.pbuf[wave][row][16 * kt + r16] = e;
        }
      }
    lds_fence();
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int kl = st * KPS + kg;
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_bits_to_float(vv[st][e] & 0xffffu);
        vf[2 * e + 1] = bf16_bits_to_float(vv[st][e] >> 16);
      }
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const float pr = sm.pbuf[wave][r][kl];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pr, vf[e], acc[r][e]);
      }
    }
    lds_fence();
  }
  // row sums: lanes of a 16-lane group hold different keys of the same rows
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = lpart[i];
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    const int row = 4 * q16 + i;
    if (r16 == 0 && row < G) sm.lsum[wave][row] = x;
  }
  // reduce over the key groups of the wave (lanes sharing dch)
#pragma unroll
  for (int r = 0; r < G; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      for (int o = DCH; o < 64; o <<= 1) acc[r][e] += __shfl_xor(acc[r][e], o);
  if (kg == 0) {
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.obuf[wave][r][8 * dch + e] = acc[r][e];
  }
  __syncthreads();
  for (int x = tid; x < G * D; x += NT) {
    const int r = x / D, c = x % D;
    const float o = sm.obuf[0][r][c] + sm.obuf[1][r][c] + sm.obuf[2][r][c] + sm.obuf[3][r][c];
    accw[((int64_t)unit * G + r) * D + c] = o;
  }
  if (tid < G) {
    stats[((int64_t)unit * G + tid) * 2 + 0] = sm.m_ref[tid];
    stats[((int64_t)unit * G + tid) * 2 + 1] = sm.lsum[0][tid] + sm.lsum[1][tid] + sm.lsum[2][tid] + sm.lsum[3][tid];
  }
}

// lambda = 0: nothing is decided, so a split needs neither the block maxima
// pass nor the look-back.  One pass: each wave streams K and V of its blocks
// together, keeps an online softmax per row (running max, rescale; attention
// tutorial section 4.2), and the four waves merge in LDS into the split's
// partial, in the layout the combine kernel reads.
template <int D, int G>
struct DenseSmem {
  float pbuf[4][G][64];  // per-wave P of the block in flight
  float alpha[4][G];     // per-wave rescale of the current block
  float wm[4][G];        // per-wave final running max (log2 units)
  float wl[4][G];        // per-wave row sums
  float obuf[4][G][D];
};

template <int D, int G>
__global__ __launch_bounds__(NT) void decode_dense_kernel(const DecodeParams p, DecodeWorkspace wl) {
  __shared__ DenseSmem<D, G> sm;
  constexpr int KS = D / 32;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  char* ws = static_cast<char*>(p.workspace);
  float* stats = reinterpret_cast<float*>(ws + wl.stats);
  float* accw = reinterpret_cast<float*>(ws + wl.acc);
  int* counts = reinterpret_cast<int*>(ws + wl.counts);
  const int S = p.num_splits;
  const int pair = blockIdx.x / S, s = blockIdx.x % S;
  const int b = pair / p.Hkv, g = pair % p.Hkv;
  const int unit = pair * S + s;
  const int blk0 = s * p.blocks_per_split;
  const int nb = min(p.blocks_per_split, p.Tc - blk0);
  const float c2 = p.scale * kLog2e;
  const __bf16* qbase = static_cast<const __bf16*>(p.q) + (int64_t)b * p.qs_b;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;

  const int r16 = lane & 15, q16 = lane >> 4;
  bf16x8 qa[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qa[ks] = r16 < G ? *reinterpret_cast<const bf16x8*>(qbase + (int64_t)(g * G + r16) * p.qs_h + 32 * ks + 8 * q16)
                     : bf16x8{};

  constexpr int DCH = D / 8;     // 16-byte chunks per key row
  constexpr int KPS = 64 / DCH;  // keys per load step across the wave
  constexpr int STEPS = BC / KPS;
  const int dch = lane % DCH, kg = lane / DCH;
  float acc[G][8];
#pragma unroll
  for (int r = 0; r < G; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
  float lpart[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // rows 4*q16+i, keys of this lane
  float mrun[4] = {kNegInf, kNegInf, kNegInf, kNegInf};

  for (int lb = wave; lb < nb; lb += 4) {
    const int j = blk0 + lb;
    bf16x8 kf[4][KS];
    load_k_block<D>(kf, kbase, p.ks_t, j, p.L, r16, q16);
    u32x4 vv[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int key = j * BC + st * KPS + kg;
      vv[st] = key < p.L ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * p.ks_t + 8 * dch) : u32x4{0, 0, 0, 0};
    }
    f32x4 sc[4];
    block_scores<D>(sc, kf, qa, c2, j, p.L, r16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = fmaxf(fmaxf(sc[0][i], sc[1][i]), fmaxf(sc[2][i], sc[3][i]));
      x = fmaxf(x, __shfl_xor(x, 1));
      x = fmaxf(x, __shfl_xor(x, 2));
      x = fmaxf(x, __shfl_xor(x, 4));
      x = fmaxf(x, __shfl_xor(x, 8));
      const float m_new = fmaxf(mrun[i], x);
      const float alpha = mrun[i] == kNegInf ? 0.0f : fast_exp2(mrun[i] - m_new);
      const float mref = m_new == kNegInf ? 0.0f : m_new;
      mrun[i] = m_new;
      lpart[i] *= alpha;
      const int row = 4 * q16 + i;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const float e = fast_exp2(sc[kt][i] - mref);  // 2^-inf = 0 past L
        lpart[i] += e;
        if (row < G) sm.pbuf[wave][row][16 * kt + r16] = e;
      }
      if (r16 == 0 && row < G) sm.alpha[wave][row] = alpha;
    }
    lds_fence();
#pragma unroll
    for (int r = 0; r < G; ++r) {
      const float a = sm.alpha[wave][r];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[r][e] *= a;
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int kl = st * KPS + kg;
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_bits_to_float(vv[st][e] & 0xffffu);
        vf[2 * e + 1] = bf16_bits_to_float(vv[st][e] >> 16);
      }
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const float pr = sm.pbuf[wave][r][kl];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pr, vf[e], acc[r][e]);
      }
    }
    lds_fence();
  }
  // per-wave row stats and outputs to LDS
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float x = lpart[i];
    x += __shfl_xor(x, 1);
    x += __shfl_xor(x, 2);
    x += __shfl_xor(x, 4);
    x += __shfl_xor(x, 8);
    const int row = 4 * q16 + i;
    if (r16 == 0 && row < G) {
      sm.wl[wave][row] = x;
      sm.wm[wave][row] = mrun[i];
    }
  }
#pragma unroll
  for (int r = 0; r < G; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      for (int o = DCH; o < 64; o <<= 1) acc[r][e] += __shfl_xor(acc[r][e], o);
  if (kg == 0) {
#pragma unroll
    for (int r = 0; r < G; ++r)
#pragma unroll
      for (int e = 0; e < 8; ++e) sm.obuf[wave][r][8 * dch + e] = acc[r][e];
  }
  __syncthreads();
  // merge the waves: M = max m_w, O = sum 2^(m_w - M) O_w, l = sum 2^(m_w - M) l_w
  for (int x = tid; x < G * D; x += NT) {
    const int r = x / D, c = x % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.wm[w][r]);
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (sm.wm[w][r] != kNegInf) o = fmaf(fast_exp2(sm.wm[w][r] - M), sm.obuf[w][r][c], o);
    accw[((int64_t)unit * G + r) * D + c] = o;
  }
  if (tid < G) {
    float M = kNegInf, l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.wm[w][tid]);
#pragma unroll
    for (int w = 0; w < 4; ++w)
      if (sm.wm[w][tid] != kNegInf) l = fmaf(fast_exp2(sm.wm[w][tid] - M), sm.wl[w][tid], l);
    stats[((int64_t)unit * G + tid) * 2 + 0] = M;
    stats[((int64_t)unit * G + tid) * 2 + 1] = l;
  }
  if (tid == 0) counts[unit] = 0;
  if (p.block_state && p.per_head) {  // [B, Hq, Tc]: every head of the group computes every block
    for (int x = tid; x < G * nb; x += NT)
      p.block_state[((int64_t)b * p.Hq + g * G + x / nb) * p.Tc + blk0 + x % nb] = 1;
  } else if (p.block_state) {
    for (int lb = tid; lb < nb; lb += NT) p.block_state[((int64_t)b * p.Hkv + g) * p.Tc + blk0 + lb] = 1;
  }
}

// Merge the S split partials of one (sequence, query head); write bf16 output
// and the per-(sequence, K/V head) counters.  256 threads: NT/D groups of D
// threads walk disjoint split subsets, then the groups are summed.
template <int D>
__global__ __launch_bounds__(NT) void decode_combine_kernel(const DecodeParams p, DecodeWorkspace wl) {
  constexpr int NGRP = NT / D;
  __shared__ float red_m[NT];
  __shared__ float red_l[NGRP];
  __shared__ float red_o[NGRP][D];
  char* ws = static_cast<char*>(p.workspace);
  const float* stats = reinterpret_cast<const float*>(ws + wl.stats);
  const float* accw = reinterpret_cast<const float*>(ws + wl.acc);
  const int* counts = reinterpret_cast<const int*>(ws + wl.counts);
  const int bh = blockIdx.x;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int g = h / p.G, r = h % p.G;
  const int S = p.num_splits;
  const int pair = b * p.Hkv + g;
  const int tid = threadIdx.x, grp = tid / D, c = tid % D;
  auto ustat = [&](int s) { return ((int64_t)(pair * S + s) * p.G + r); };
  float m = kNegInf;
  for (int s = tid; s < S; s += NT) m = fmaxf(m, stats[ustat(s) * 2]);
  red_m[tid] = m;
  __syncthreads();
  for (int o = NT / 2; o > 0; o >>= 1) {
    if (tid < o) red_m[tid] = fmaxf(red_m[tid], red_m[tid + o]);
    __syncthreads();
  }
  const float M = red_m[0];
  float l = 0.0f, o = 0.0f;
  if (M != kNegInf) {
#pragma unroll 4
    for (int s = grp; s < S; s += NGRP) {
      const float ms = stats[ustat(s) * 2];
      const float w = ms == kNegInf ? 0.0f : fast_exp2(ms - M);
      l += w * stats[ustat(s) * 2 + 1];
      o += w * accw[ustat(s) * D + c];
    }
  }
  red_o[grp][c] = o;
  if (c == 0) red_l[grp] = l;
  __syncthreads();
  if (grp == 0) {
    float lt = 0.0f, ot = 0.0f;
#pragma unroll
    for (int q = 0; q < NGRP; ++q) {
      lt += red_l[q];
      ot += red_o[q][c];
    }
    const float res = lt > 0.0f ? ot / lt : 0.0f;
    __bf16* out = static_cast<__bf16*>(p.out) + (int64_t)b * p.os_b + (int64_t)h * p.os_h;
    out[c] = (__bf16)res;
  }
  if (p.counters && r == 0 && tid == 0) {
    int sk = 0;
    for (int s = 0; s < S; ++s) sk += counts[pair * S + s];
    p.counters[2 * pair + 0] = p.Tc;
    p.counters[2 * pair + 1] = sk;
  }
}

template <int D, int G>
hipError_t launch_g(const DecodeParams& p, hipStream_t s) {
  const DecodeWorkspace wl = decode_workspace_layout(p.B, p.Hq, p.Hkv, p.d, p.num_splits);
  const int units = p.B * p.Hkv * p.num_splits;
  if (p.lambda > 0.0f) {
    char* ws = static_cast<char*>(p.workspace);
    const int n_tickets = p.B * p.Hkv;
    const int clear_grid = min(64, (units + NT - 1) / NT);
    hipLaunchKernelGGL(decode_clear_kernel, dim3(clear_grid), dim3(NT), 0, s, reinterpret_cast<int*>(ws + wl.tickets),
                       n_tickets, reinterpret_cast<int*>(ws + wl.flags), units);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_split_kernel<D, G>), dim3(units), dim3(NT), 0, s, p, wl);
  } else
    hipLaunchKernelGGL((decode_dense_kernel<D, G>), dim3(units), dim3(NT), 0, s, p, wl);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(p.B * p.Hq), dim3(NT), 0, s, p, wl);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t s) {
  switch (p.G) {
    case 1: return launch_g<D, 1>(p, s);
    case 2: return launch_g<D, 2>(p, s);
    case 4: return launch_g<D, 4>(p, s);
    default: return launch_g<D, 8>(p, s);
  }
}

}  // namespace

int launch_decode(const DecodeParams& p, void* stream) {
  if (p.blocks_per_split > 64) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return p.d == 64 ? launch_d<64>(p, s) : launch_d<128>(p, s);
}

}  // namespace bsattn
