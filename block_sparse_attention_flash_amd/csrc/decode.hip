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
//   phase 1  stream the split's K blocks, scores q.K^T (G rows x 64 keys per
//            block) with the 16x16x32 bf16 MFMA, keep all scores of the split
//            in LDS, block row maxima
//   publish  the split aggregate (max over its blocks), look back over earlier
//            splits for their inclusive prefix, publish the inclusive prefix
//   phase 2  running max within the split seeded with the exclusive prefix,
//            tile-wide skip decision per block (strict <, as printed)
//   phase 3  P = 2^(s - m_ref) for kept blocks, V loads only for kept blocks,
//            O_partial = P V on the vector ALUs (G <= 8 rows), write the
//            partial (m_ref, l, O) of the split
//   combine  merge the splits of each (sequence, head): online-softmax
//            rescaling (attention tutorial section 4.2)
//
// Forward progress: split work items are handed out through an atomic ticket
// in (split, sequence, head) order, so a split only ever waits for splits that
// already hold a ticket, i.e. are resident or finished.  Every wait is also
// bounded; a timed-out wait sets the workspace health word instead of hanging.

#include "device_common.h"
#include "internal.h"

namespace bsattn {
namespace {

constexpr int NT = 256;
constexpr int BC = 64;
constexpr int kMaxScores = 8192;  // floats of LDS score storage per split
constexpr int kSpinLimit = 1 << 20;  // ~1 s; a normal wait is well under 1 ms

template <int D, int G>
struct DecSmem {
  float score[kMaxScores];      // [G][bps * 64], log2 units
  float bm[64][G];              // block row maxima
  float m_ref[G];
  float lsum[4][G];
  float pre[G];
  int kept[64];
  int nkept;
  int ticket;
  float obuf[4][G][D];
};

// Wait for a look-back flag.  Bounded: gives up after kSpinLimit polls, or at
// once when another work-group has already given up (health word set).
__device__ __forceinline__ int spin_acquire(const int* flag, int* health) {
  for (int n = 0; n < kSpinLimit; ++n) {
    const int f = __hip_atomic_load(flag, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
    if (f != 0) return f;
    if (__hip_atomic_load(health, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return 0;
    __builtin_amdgcn_s_sleep(2);
  }
  atomicOr(health, 1);
  return 0;
}

__device__ __forceinline__ float load_agent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
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

  if (tid == 0) sm.ticket = atomicAdd(&header[0], 1);
  __syncthreads();
  const int S = p.num_splits;
  const int pairs = p.B * p.Hkv;
  const int ticket = sm.ticket;
  const int s = ticket / pairs;
  const int pair = ticket % pairs;
  const int b = pair / p.Hkv, g = pair % p.Hkv;
  const int unit = pair * S + s;
  const int blk0 = s * p.blocks_per_split;
  const int nb = min(p.blocks_per_split, p.Tc - blk0);
  const int span = p.blocks_per_split * BC;  // score row pitch
  const float c2 = p.scale * kLog2e;

  const __bf16* qbase = static_cast<const __bf16*>(p.q) + (int64_t)b * p.qs_b;
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;

  // ---- phase 1: scores and block maxima --------------------------------------
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
  for (int lb = wave; lb < nb; lb += 4) {
    const int j = blk0 + lb;
    bf16x8 kf[4][KS];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key = j * BC + 16 * kt + r16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (key < p.L)
          kf[kt][ks] = *reinterpret_cast<const bf16x8*>(kbase + (int64_t)key * p.ks_t + 32 * ks + 8 * q16);
        else
          kf[kt][ks] = bf16x8{};
      }
    }
    float bmax[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 acc = f32x4{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) acc = mfma16(qa[ks], kf[kt][ks], acc);
      const int key = j * BC + 16 * kt + r16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * q16 + i;
        const float sc = key < p.L ? acc[i] * c2 : kNegInf;
        if (row < G) sm.score[row * span + lb * BC + 16 * kt + r16] = sc;
        bmax[i] = fmaxf(bmax[i], sc);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float x = bmax[i];
      x = fmaxf(x, __shfl_xor(x, 1));
      x = fmaxf(x, __shfl_xor(x, 2));
      x = fmaxf(x, __shfl_xor(x, 4));
      x = fmaxf(x, __shfl_xor(x, 8));
      const int row = 4 * q16 + i;
      if (r16 == 0 && row < G) sm.bm[lb][row] = x;
    }
  }
  __syncthreads();

  // ---- publish aggregate, look back, publish inclusive prefix ----------------
  if (tid == 0) {
    float agg[G];
#pragma unroll
    for (int r = 0; r < G; ++r) {
      float x = kNegInf;
      for (int lb = 0; lb < nb; ++lb) x = fmaxf(x, sm.bm[lb][r]);
      agg[r] = x;
      aggv[unit * 16 + r] = x;
    }
    __hip_atomic_store(&flags[unit], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    float pre[G];
#pragma unroll
    for (int r = 0; r < G; ++r) pre[r] = kNegInf;
    for (int q = s - 1; q >= 0; --q) {
      const int u = pair * S + q;
      const int f = spin_acquire(&flags[u], &header[1]);
      if (f == 0) break;  // timed out: health word set, result invalid
      const float* src = (f == 2) ? inclv : aggv;
#pragma unroll
      for (int r = 0; r < G; ++r) pre[r] = fmaxf(pre[r], load_agent(src + u * 16 + r));
      if (f == 2) break;
    }
#pragma unroll
    for (int r = 0; r < G; ++r) {
      inclv[unit * 16 + r] = fmaxf(pre[r], agg[r]);
      sm.pre[r] = pre[r];
    }
    __hip_atomic_store(&flags[unit], 2, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
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
      for (int lb = 0; lb < nb; ++lb) {
        const float x = sm.bm[lb][lane];
        cm = fmaxf(cm, x);
        if (x == kNegInf || x - cm < log2_lambda) agree |= (1ull << lb);
      }
    }
    // all rows must agree
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t other = ((uint64_t)__shfl_xor((unsigned)(agree >> 32), o) << 32) |
                             (uint64_t)(unsigned)__shfl_xor((unsigned)agree, o);
      agree &= other;
    }
    const uint64_t valid = nb == 64 ? ~0ull : ((1ull << nb) - 1ull);
    const uint64_t skipm = dyn ? (agree & valid) : 0ull;
    const uint64_t keepm = valid & ~skipm;
    if (lane < G) {
      float mr = kNegInf;
      for (int lb = 0; lb < nb; ++lb)
        if ((keepm >> lb) & 1ull) mr = fmaxf(mr, sm.bm[lb][lane]);
      sm.m_ref[lane] = mr;
    }
    if (lane == 0) {
      int n = 0;
      for (int lb = 0; lb < nb; ++lb)
        if ((keepm >> lb) & 1ull) sm.kept[n++] = lb;
      sm.nkept = n;
      counts[unit] = __popcll(skipm);
    }
    if (p.block_state)
      for (int lb = lane; lb < nb; lb += 64)
        p.block_state[((int64_t)b * p.Hkv + g) * p.Tc + blk0 + lb] = ((skipm >> lb) & 1ull) ? 2 : 1;
  }
  __syncthreads();
  const int nkept = sm.nkept;

  // ---- phase 3a: P = 2^(s - m_ref) in place for kept blocks, row sums --------
  {
    const int key = tid & 63;
    float lacc[(G + 3) / 4];
#pragma unroll
    for (int x = 0; x < (G + 3) / 4; ++x) lacc[x] = 0.0f;
    for (int k = 0; k < nkept; ++k) {
      const int lb = sm.kept[k];
#pragma unroll
      for (int x = 0; x < (G + 3) / 4; ++x) {
        const int r = wave + 4 * x;
        if (r < G) {
          float* sp = &sm.score[r * span + lb * BC + key];
          const float e = fast_exp2(*sp - sm.m_ref[r]);  // 2^-inf = 0 for keys >= L
          *sp = e;
          lacc[x] += e;
        }
      }
    }
#pragma unroll
    for (int x = 0; x < (G + 3) / 4; ++x) {
      float v = lacc[x];
      for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
      const int r = wave + 4 * x;
      if (lane == 0 && r < G) sm.lsum[0][r] = v;
    }
  }
  __syncthreads();

  // ---- phase 3b: O_partial = P V over kept blocks (vector ALUs) --------------
  constexpr int DCH = D / 8;        // 16-byte chunks per key row
  constexpr int KPS = 64 / DCH;     // keys per load step across the wave
  constexpr int STEPS = BC / KPS;
  const int dch = lane % DCH, kg = lane / DCH;
  float acc[G][8];
#pragma unroll
  for (int r = 0; r < G; ++r)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[r][e] = 0.0f;
  for (int k = wave; k < nkept; k += 4) {
    const int lb = sm.kept[k];
    const int j = blk0 + lb;
    u32x4 vv[STEPS];
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int key = j * BC + st * KPS + kg;
      vv[st] = key < p.L ? *reinterpret_cast<const u32x4*>(vbase + (int64_t)key * p.ks_t + 8 * dch)
                         : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
      const int kl = lb * BC + st * KPS + kg;
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16_bits_to_float(vv[st][e] & 0xffffu);
        vf[2 * e + 1] = bf16_bits_to_float(vv[st][e] >> 16);
      }
#pragma unroll
      for (int r = 0; r < G; ++r) {
        const float pr = sm.score[r * span + kl];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[r][e] = fmaf(pr, vf[e], acc[r][e]);
      }
    }
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
    stats[((int64_t)unit * G + tid) * 2 + 1] = sm.lsum[0][tid];
  }
}

// Merge the S split partials of one (sequence, query head); write bf16 output
// and the per-(sequence, K/V head) counters.
template <int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(const DecodeParams p, DecodeWorkspace wl) {
  const char* ws = static_cast<const char*>(p.workspace);
  const float* stats = reinterpret_cast<const float*>(ws + wl.stats);
  const float* accw = reinterpret_cast<const float*>(ws + wl.acc);
  const int* counts = reinterpret_cast<const int*>(ws + wl.counts);
  const int bh = blockIdx.x;
  const int b = bh / p.Hq, h = bh % p.Hq;
  const int g = h / p.G, r = h % p.G;
  const int S = p.num_splits;
  const int pair = b * p.Hkv + g;
  const int c = threadIdx.x;
  float M = kNegInf;
  for (int s = 0; s < S; ++s) M = fmaxf(M, stats[((int64_t)(pair * S + s) * p.G + r) * 2]);
  float l = 0.0f, o = 0.0f;
  if (M != kNegInf) {
    for (int s = 0; s < S; ++s) {
      const int64_t u = (int64_t)(pair * S + s) * p.G + r;
      const float ms = stats[u * 2];
      if (ms == kNegInf) continue;
      const float w = fast_exp2(ms - M);
      l += w * stats[u * 2 + 1];
      o += w * accw[u * D + c];
    }
  }
  const float res = l > 0.0f ? o / l : 0.0f;
  __bf16* out = static_cast<__bf16*>(p.out) + (int64_t)b * p.os_b + (int64_t)h * p.os_h;
  out[c] = (__bf16)res;
  if (p.counters && r == 0 && c == 0) {
    int sk = 0;
    for (int s = 0; s < S; ++s) sk += counts[pair * S + s];
    p.counters[2 * pair + 0] = p.Tc;
    p.counters[2 * pair + 1] = sk;
  }
}

// Clear the ticket, the health word and the look-back flags (a fill kernel,
// so the sequence stays valid inside captured graphs).
__global__ void decode_reset_kernel(int* header, int* flags, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 16) header[i] = 0;
  if (i < n) flags[i] = 0;
}

template <int D, int G>
hipError_t launch_g(const DecodeParams& p, hipStream_t s) {
  const DecodeWorkspace wl = decode_workspace_layout(p.B, p.Hq, p.Hkv, p.d, p.num_splits);
  char* ws = static_cast<char*>(p.workspace);
  const int units = p.B * p.Hkv * p.num_splits;
  const int rb = (units > 16 ? units : 16) + 255;
  hipLaunchKernelGGL(decode_reset_kernel, dim3(rb / 256), dim3(256), 0, s, reinterpret_cast<int*>(ws + wl.header),
                     reinterpret_cast<int*>(ws + wl.flags), units);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_split_kernel<D, G>), dim3(units), dim3(NT), 0, s, p, wl);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(p.B * p.Hq), dim3(D), 0, s, p, wl);
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
  if (p.blocks_per_split * BC * p.G > kMaxScores || p.blocks_per_split > 64) return (int)hipErrorInvalidValue;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return p.d == 64 ? launch_d<64>(p, s) : launch_d<128>(p, s);
}

}  // namespace bsattn
