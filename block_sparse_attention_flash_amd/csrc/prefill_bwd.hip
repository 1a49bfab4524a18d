// bf16 backward of static block-sparse attention on CDNA4 matrix cores.
//
// For the loss sum(out * dout) of the forward out = softmax(scale Q K^T) V
// over the block mask (tiles of 128 query rows x blocks of 64 keys, plus the
// token-level valid-length and causal limits), with P rebuilt from the
// forward's per-row log-sum-exp:
//
//   dot   Dv[i] = sum_c dout[i][c] out[i][c]            (one float per row)
//   dkdv  per (batch, K/V head, key block j): walk the query tiles whose CSR
//         list holds j (the transposed index), for every query head of the
//         group, and accumulate in registers
//            S  = Q K_j^T,  P = 2^(S c2 - lse log2e)    (masked entries 0)
//            dP = dO V_j^T, dS = P (dP - Dv)
//            dV_j^T += dO^T P,   dK_j^T += Q^T dS
//   dq    per (batch, head, query tile): walk the tile's CSR list
//            S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - Dv)
//            dQ^T += K^T dS^T
//
// Every product is a v_mfma_f32_32x32x16_bf16.  An accumulator in layout
// D[m][n] (lane n % 32, rows 8(a/4) + 4(l/32) + a%4 in element a) is the B
// operand of a product that contracts over m, after a bf16 pack: the
// contraction index runs through the same permutation in both operands, and
// the other operand is read with ds_read_b64_tr_b16 in that order.  So P and
// dS never leave registers.  Each kernel owns its outputs: no atomics, and
// the results do not depend on scheduling.
//
// The pages print no backward pass; the gradients are the chain rule on the
// forward's definition (the DiT article trains with the block-sparse
// forward, section 4; its section 3.3 check of the block list before any
// load applies to both walks here).

#include "device_common.h"
#include "internal.h"

namespace bsattn {
namespace {

constexpr int BR = 128;
constexpr int BC = 64;
constexpr int NT = 256;

// R x D bf16 tile in LDS read both row-wise (16-byte chunks: MFMA operand
// rows) and transposed (ds_read_b64_tr_b16 over 4 rows x 4 chunks per
// instruction).  Chunk c of row r sits at r * CH + (c ^ swz(r)), swz a
// bijection of r % 16 (d = 128) or of (r / 2) % 8 (d = 64, two rows per
// 256-byte bank line) chosen so that both patterns touch every bank once:
//   row reads: 16 consecutive rows, one chunk each -> 16 (8 per row parity
//              at d = 64) different chunk positions;
//   transposed reads: 4 consecutive rows, 4 chunks of one 64-byte group each
//              -> the rows land in 4 different 64-byte groups (bits 2-3 of
//              swz; at d = 64 rows r and r + 2 differ in bit 2, rows r and
//              r + 1 already sit in different halves of the line).
template <int D>
struct BTile {
  static constexpr int CH = D / 8;
  __device__ static __forceinline__ int swz(int r) {
    return D == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
  __device__ static __forceinline__ int pos(int r, int c) { return (r * CH + (c ^ swz(r))) * 8; }
};

// A R x D global tile staged through registers: load() issues the global
// reads of rows [0, nrows) (rows >= nrows read as zeros) one tile ahead,
// store() writes them to LDS once the tile there is no longer read.
template <int D, int R>
struct Staged {
  static constexpr int CH = D / 8;
  static constexpr int PER = R * CH / NT;
  bf16x8 v[PER];
  __device__ __forceinline__ void load(const __bf16* src, int64_t stride, int nrows, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int x = i * NT + tid;
      const int r = x / CH, c = x % CH;
      v[i] = r < nrows ? *reinterpret_cast<const bf16x8*>(src + (int64_t)r * stride + 8 * c) : bf16x8{};
    }
  }
  __device__ __forceinline__ void store(__bf16* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int x = i * NT + tid;
      const int r = x / CH, c = x % CH;
      *reinterpret_cast<bf16x8*>(tile + BTile<D>::pos(r, c)) = v[i];
    }
  }
};

// Row fragment: X[r][16 ks + 8 hi + 0..7] (A operand rows, or B operand columns).
template <int D>
__device__ __forceinline__ bf16x8 read_row(const __bf16* tile, int r, int ks, int hi) {
  return *reinterpret_cast<const bf16x8*>(tile + BTile<D>::pos(r, 2 * ks + hi));
}

// Transposed fragment (A operand X^T[m = d][k]): lane l gets, in slot i,
// X[r0 + 8 (i/4) + 4 (l/32) + i%4][32 n + l%32], the row order of the
// accumulator layout above.
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const __bf16* tile, int r0, int n, int lane) {
  const int g16 = lane >> 4, j16 = lane & 15;
  const int r = r0 + 4 * (g16 >> 1) + (j16 >> 2);
  const int c = 4 * n + 2 * (g16 & 1) + ((j16 & 3) >> 1);
  const int half = 4 * (j16 & 1);
  return join_bf16x4(lds_read_tr16(tile + BTile<D>::pos(r, c) + half),
                     lds_read_tr16(tile + BTile<D>::pos(r + 8, c) + half));
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr_b(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(ptr);
}

// Dv = rowsum(dout * out), fp32, one row per D/8 lanes.
template <int D>
__global__ __launch_bounds__(NT) void bwd_dot_kernel(const BwdParams p) {
  constexpr int LPR = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * NT + threadIdx.x;
  const int64_t rid = gid / LPR;  // (b, h, i) with i fastest
  const int c = (int)(gid % LPR);
  const int64_t total = (int64_t)p.B * p.Hq * p.Nq;
  float acc = 0.0f;
  if (rid < total) {
    const int i = (int)(rid % p.Nq);
    const int bh = (int)(rid / p.Nq);
    const int h = bh % p.Hq, b = bh / p.Hq;
    const bf16x8 o = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.out) + (int64_t)b * p.os_b +
                                                     (int64_t)i * p.os_t + (int64_t)h * p.os_h + 8 * c);
    const bf16x8 g = *reinterpret_cast<const bf16x8*>(static_cast<const __bf16*>(p.dout) + (int64_t)b * p.dos_b +
                                                     (int64_t)i * p.dos_t + (int64_t)h * p.dos_h + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int o = 1; o < LPR; o <<= 1) acc += __shfl_xor(acc, o);
  if (rid < total && c == 0) p.dvec[rid] = acc;
}

// Store 4 consecutive d values (accumulator elements 4q..4q+3 of tile n) as bf16.
__device__ __forceinline__ void store4(__bf16* dst, const f32x16& acc, int q4, float s) {
  f32x4 v4 = {acc[4 * q4 + 0] * s, acc[4 * q4 + 1] * s, acc[4 * q4 + 2] * s, acc[4 * q4 + 3] * s};
  *reinterpret_cast<bf16x4*>(dst) = __builtin_convertvector(v4, bf16x4);
}

// Fourth word of a raw buffer descriptor on gfx9-family parts (32-bit data
// format, no swizzle; range checking against num_records).
constexpr int kBufferWord3 = 0x00020000;

typedef __attribute__((address_space(3))) void lds_void;

// Global -> LDS DMA of a 64 x D tile (buffer_load_dwordx4 ... lds).  The
// descriptor's range ends at the tensor's last row of this (batch, head), so
// rows past it read as zeros.  Instruction i of wave w lands lane l's 16 bytes
// at LDS chunk slot (4 i + w) 64 + l; the lane fetches the global chunk whose
// swizzled position is that slot (BTile::pos is a bijection on every row).
template <int D>
__device__ __forceinline__ void dma_tile64(__bf16* tile, const __bf16* head, int rows_total, int64_t stride_t,
                                           int row0, int wave, int lane) {
  constexpr int CH = D / 8;
  constexpr int NI = 64 * CH / NT;
  const uint32_t extent = (uint32_t)(((int64_t)(rows_total - 1) * stride_t + D) * 2);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(head), (short)0, (int)extent, kBufferWord3);
  const uint32_t soff = (uint32_t)((int64_t)row0 * stride_t * 2);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot = (4 * i + wave) * 64 + lane;
    const int r = slot / CH, cp = slot % CH;
    const int c = cp ^ BTile<D>::swz(r);
    const uint32_t voff = (uint32_t)(((int64_t)r * stride_t + 8 * c) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + (4 * i + wave) * 64 * 8), 16, voff, soff, 0, 0);
  }
}

template <int D>
struct DkdvSmem {
  __bf16 k[BC * D];   // the block's keys
  __bf16 v[BC * D];
  __bf16 q[64 * D];   // 64 query rows of the current tile (one stage)
  __bf16 g[64 * D];   // their dout
  float lse2[64];     // lse in log2 units
  float dv[64];
};

// Work-groups per CU the dK/dV kernel is cut for: K and V stay in LDS and
// query rows stream in 64-row stages, so two groups fit at d = 128 (64.5 KB
// of LDS, at most 256 registers each) and three at d = 64.
template <int D>
constexpr int kDkdvBlocksPerCu = D == 64 ? 3 : 2;

// One work-group per (batch, K/V head, key block).  Wave w: keys 32 (w & 1)
// .. +31 of the block (kh), rows 32 (w >> 1) .. +31 of each 64-row stage (qh).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, kDkdvBlocksPerCu<D>) void bwd_dkdv_kernel(const BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KS = D / 16;
  constexpr int NTD = D / 32;
  __shared__ DkdvSmem<D> sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int kh = wave & 1, qh = wave >> 1;
  // work order: key block major, ascending (under a causal mask the first
  // blocks have the most query tiles: longest first); the (batch, K/V head)
  // index runs fastest, so with B Hkv a multiple of 8 a group stays on one
  // XCD (work-group i runs on XCD i % 8) and its Q / dO tiles in one L2
  const int NBG = p.B * p.Hkv;
  const int j = blockIdx.x / NBG;
  const int bg = blockIdx.x % NBG;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int G = p.Hq / p.Hkv;
  const float c2 = p.scale * kLog2e;

  const int key = j * BC + 32 * kh + l32;  // this lane's key (column of S)
  const bool key_ok = key < p.n_valid;
  dma_tile64<D>(sm.k, static_cast<const __bf16*>(p.k) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h, p.Nk, p.ks_t,
                j * BC, wave, lane);
  dma_tile64<D>(sm.v, static_cast<const __bf16*>(p.v) + (int64_t)b * p.vs_b + (int64_t)g * p.vs_h, p.Nk, p.vs_t,
                j * BC, wave, lane);

  f32x16 dk[NTD], dv[NTD];
#pragma unroll
  for (int n = 0; n < NTD; ++n) {
    dk[n] = f32x16{};
    dv[n] = f32x16{};
  }

  // query tiles that attend block j: the transposed CSR, or every tile (from
  // the diagonal on when causal)
  int e0, e1;
  if (p.col_ptr) {
    e0 = p.col_ptr[j];
    e1 = p.col_ptr[j + 1];
  } else {
    e0 = CAUSAL ? (j * BC) / BR : 0;
    e1 = p.Tr;
  }
  e0 = __builtin_amdgcn_readfirstlane(e0);
  e1 = __builtin_amdgcn_readfirstlane(e1);
  const int ntile = e1 - e0;

  // work: (query head, tile, 64-row half) in order; halves past the last row
  // or (causal) wholly above the block's first key are not visited
  for (int it = 0; it < 2 * G * ntile; ++it) {
    const int hf = it & 1;
    const int e = e0 + (it >> 1) % ntile;
    const int h = g * G + (it >> 1) / ntile;
    const int t = __builtin_amdgcn_readfirstlane(p.row_idx ? p.row_idx[e] : e);
    const int row0 = t * BR + 64 * hf;
    if (row0 >= p.Nq || (CAUSAL && row0 + 63 < j * BC)) continue;
    if (p.block_state && p.block_state[(((int64_t)b * p.Hq + h) * p.Tr + t) * p.Tc + j] == 2) continue;
    const int nrows = min(64, p.Nq - row0);
    __syncthreads();  // every wave is done reading the previous stage
    dma_tile64<D>(sm.q, static_cast<const __bf16*>(p.q) + (int64_t)b * p.qs_b + (int64_t)h * p.qs_h, p.Nq, p.qs_t,
                  row0, wave, lane);
    dma_tile64<D>(sm.g, static_cast<const __bf16*>(p.dout) + (int64_t)b * p.dos_b + (int64_t)h * p.dos_h, p.Nq,
                  p.dos_t, row0, wave, lane);
    if (tid < 64) {
      const int64_t ri = ((int64_t)b * p.Hq + h) * p.Nq + row0 + tid;
      sm.lse2[tid] = tid < nrows ? p.lse[ri] * kLog2e : 0.0f;
      sm.dv[tid] = tid < nrows ? p.dvec[ri] : 0.0f;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's DMA has landed
    __syncthreads();                                   // and every other wave's

    const int r0 = 32 * qh;  // first stage row of this wave's chunk
    // S = Q K^T and dP = dO V^T, the fragments of one k-step at a time (the
    // scheduling barriers keep the compiler from hoisting every LDS read,
    // which would not fit two work-groups' registers)
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma32(read_row<D>(sm.q, r0 + l32, ks, hi), read_row<D>(sm.k, 32 * kh + l32, ks, hi), s);   // S[q][key]
      dp = mfma32(read_row<D>(sm.g, r0 + l32, ks, hi), read_row<D>(sm.v, 32 * kh + l32, ks, hi), dp);  // dP[q][key]
      if (ks % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float pv[8], dsv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int a = 8 * kk + i;
        const int rl = r0 + 8 * (a >> 2) + 4 * hi + (a & 3);
        const bool ok = key_ok && rl < nrows && (!CAUSAL || key <= row0 + rl);
        pv[i] = ok ? fast_exp2(fmaf(s[a], c2, -sm.lse2[rl])) : 0.0f;
        dsv[i] = pv[i] * (dp[a] - sm.dv[rl]);
      }
      const bf16x8 pb = to_bf16x8(pv);
      const bf16x8 db = to_bf16x8(dsv);
#pragma unroll
      for (int n = 0; n < NTD; ++n) {
        dv[n] = mfma32(read_tr<D>(sm.g, r0 + 16 * kk, n, lane), pb, dv[n]);  // dV^T += dO^T P
        dk[n] = mfma32(read_tr<D>(sm.q, r0 + 16 * kk, n, lane), db, dk[n]);  // dK^T += Q^T dS
        if (n % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // the two row halves of each key half: waves with qh = 1 hand their sums to
  // the waves with qh = 0 through LDS (the Q / dO area is free now)
  __syncthreads();
  static_assert(sizeof(float) * 2 * 2 * NTD * 16 * 64 <= sizeof(__bf16) * 4 * 64 * D, "reduction fits in k, v, q, g");
  float* red = reinterpret_cast<float*>(&sm) + kh * (2 * NTD * 16 * 64);
  if (qh == 1) {
#pragma unroll
    for (int n = 0; n < NTD; ++n)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        red[(n * 16 + a) * 64 + lane] = dk[n][a];
        red[((NTD + n) * 16 + a) * 64 + lane] = dv[n][a];
      }
  }
  __syncthreads();
  if (qh == 0 && key < p.Nk) {
    __bf16* dkp = static_cast<__bf16*>(p.dk) + (int64_t)b * p.dks_b + (int64_t)key * p.dks_t + (int64_t)g * p.dks_h;
    __bf16* dvp = static_cast<__bf16*>(p.dv) + (int64_t)b * p.dvs_b + (int64_t)key * p.dvs_t + (int64_t)g * p.dvs_h;
#pragma unroll
    for (int n = 0; n < NTD; ++n) {
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        dk[n][a] += red[(n * 16 + a) * 64 + lane];
        dv[n][a] += red[((NTD + n) * 16 + a) * 64 + lane];
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dcol = 32 * n + 8 * q4 + 4 * hi;
        store4(dkp + dcol, dk[n], q4, p.scale);
        store4(dvp + dcol, dv[n], q4, 1.0f);
      }
    }
  }
#endif
}

// ---- dK/dV at d = 128: key-block pairs, double-buffered query stages --------
//
// The kernel above keeps one 64-row query stage in LDS and waits for each
// stage's load before computing on it: at d = 128 two work-groups fill a
// CU's LDS, so the load latency of every stage is exposed to the MFMAs of
// only one other work-group.  Here one work-group of eight waves takes two
// adjacent key blocks (2m, 2m + 1), so their K/V (64 KB) and two 64-row
// query stages (64 KB) fit one CU: the next stage streams in while the
// current one is computed, behind a single barrier per stage.  Waves 4 kb ..
// 4 kb + 3 work on block 2m + kb exactly as the four waves above do; the
// stages visited are those of either block (the union of the two tiles'
// lists, or the shared causal range), and a block's waves sit out stages that
// do not touch it.  The Q / dO stages' transposed reads are inline asm that
// waits inside the block: the intrinsic would make the compiler wait for
// the next stage's load first (it cannot tell the stages apart).

constexpr int NT2 = 512;

template <int D>
struct Dkdv2Smem {
  __bf16 k[2][BC * D];  // keys of blocks 2m, 2m + 1
  __bf16 v[2][BC * D];
  __bf16 q[2][64 * D];  // double-buffered 64-row query stages
  __bf16 g[2][64 * D];  // their dout
  float lse[2][64];     // per stage: lse (natural log) and Dv of its rows
  float dvec[2][64];
};

// 64 x D tile, global -> LDS, by all eight waves (rows past rows_total: zeros).
template <int D>
__device__ __forceinline__ void dma_tile64_w8(__bf16* tile, const __bf16* head, int rows_total, int64_t stride_t,
                                              int row0, int wave, int lane) {
  constexpr int CH = D / 8;
  constexpr int NI = 64 * CH / NT2;
  const uint32_t extent = (uint32_t)(((int64_t)(rows_total - 1) * stride_t + D) * 2);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(head), (short)0, (int)extent, kBufferWord3);
  const uint32_t soff = (uint32_t)((int64_t)row0 * stride_t * 2);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot = (8 * i + wave) * 64 + lane;
    const int r = slot / CH, cp = slot % CH;
    const int c = cp ^ BTile<D>::swz(r);
    const uint32_t voff = (uint32_t)(((int64_t)r * stride_t + 8 * c) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + (8 * i + wave) * 64 * 8), 16, voff, soff, 0, 0);
  }
}

// 64 consecutive floats of a row vector (rows row0 .. row0 + 63 of a [.., N]
// float array, zeros past n_total), global -> LDS by one wave.
__device__ __forceinline__ void dma_row64(float* dst, const float* src_row, int n_total, int row0, int lane) {
  const uint32_t extent = (uint32_t)n_total * 4;
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(src_row), (short)0, (int)extent, kBufferWord3);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 4, (uint32_t)lane * 4, (uint32_t)row0 * 4, 0, 0);
}

// The four d-tiles' transposed fragments of one 16-row step (read_tr for
// n = 0..3), issued together and waited for inside the asm block.  The
// loads return into their registers some cycles after the block issues
// them, which the compiler does not see: `busy` (the operands of the MFMAs
// issued just before, which may not have read them yet) are inputs of the
// block, so its outputs (early-clobber) are never placed on top of them.
__device__ __forceinline__ void read_tr_x4(bf16x8 (&out)[4], const __bf16* tile, int r0, int lane,
                                           const bf16x8 (&busy)[4], const bf16x8& busy_b) {
  const int g16 = lane >> 4, j16 = lane & 15;
  const int r = r0 + 4 * (g16 >> 1) + (j16 >> 2);
  const int half = 4 * (j16 & 1);
  uint32_t a[8];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int c = 4 * n + 2 * (g16 & 1) + ((j16 & 3) >> 1);
    a[2 * n] = lds_addr_b(tile + BTile<128>::pos(r, c) + half);
    a[2 * n + 1] = lds_addr_b(tile + BTile<128>::pos(r + 8, c) + half);
  }
  i16x4 x[8];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n"
      "ds_read_b64_tr_b16 %1, %9\n"
      "ds_read_b64_tr_b16 %2, %10\n"
      "ds_read_b64_tr_b16 %3, %11\n"
      "ds_read_b64_tr_b16 %4, %12\n"
      "ds_read_b64_tr_b16 %5, %13\n"
      "ds_read_b64_tr_b16 %6, %14\n"
      "ds_read_b64_tr_b16 %7, %15\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]), "v"(busy[0]),
        "v"(busy[1]), "v"(busy[2]), "v"(busy[3]), "v"(busy_b)
      : "memory");
#pragma unroll
  for (int n = 0; n < 4; ++n) out[n] = join_bf16x4(x[2 * n], x[2 * n + 1]);
}

template <bool CAUSAL>
__global__ __launch_bounds__(NT2, 1) void bwd_dkdv_pair_kernel(const BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int D = 128;
  constexpr int KS = D / 16;
  constexpr int NTD = D / 32;
  __shared__ Dkdv2Smem<D> sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int kb = wave >> 2, kh = wave & 1, qh = (wave >> 1) & 1;
  // work order as above: key-block pairs ascending, (batch, K/V head) fastest
  const int NBG = p.B * p.Hkv;
  const int m = blockIdx.x / NBG;
  const int bg = blockIdx.x % NBG;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int G = p.Hq / p.Hkv;
  const float c2 = p.scale * kLog2e;
  const int j0 = 2 * m;
  const bool has1 = j0 + 1 < p.Tc;
  const int jw = j0 + kb;  // this wave's block

  const int key = jw * BC + 32 * kh + l32;
  const bool key_ok = key < p.n_valid;
  const __bf16* kh_base = static_cast<const __bf16*>(p.k) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;
  const __bf16* vh_base = static_cast<const __bf16*>(p.v) + (int64_t)b * p.vs_b + (int64_t)g * p.vs_h;
  dma_tile64_w8<D>(sm.k[0], kh_base, p.Nk, p.ks_t, j0 * BC, wave, lane);
  dma_tile64_w8<D>(sm.v[0], vh_base, p.Nk, p.vs_t, j0 * BC, wave, lane);
  if (has1) {
    dma_tile64_w8<D>(sm.k[1], kh_base, p.Nk, p.ks_t, (j0 + 1) * BC, wave, lane);
    dma_tile64_w8<D>(sm.v[1], vh_base, p.Nk, p.vs_t, (j0 + 1) * BC, wave, lane);
  }

  // the stages: for each query head of the group, the tiles holding either
  // block (merge of the two transposed lists, or the causal / dense range
  // shared by the pair), two 64-row halves each; a stage is kept when it
  // touches a block (not past the last row, not wholly above the block's
  // first key, not a block the forward skipped for that head and tile)
  // the transposed index through the scalar cache (wave-uniform, read-only)
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const const_i32_ptr rowi = p.row_idx ? (const_i32_ptr)p.row_idx : nullptr;
  int b0 = 0, n0 = 0, b1 = 0, n1 = 0, tlo = 0;
  if (p.col_ptr) {
    b0 = p.col_ptr[j0];
    n0 = p.col_ptr[j0 + 1] - b0;
    if (has1) {
      b1 = p.col_ptr[j0 + 1];
      n1 = p.col_ptr[j0 + 2] - b1;
    }
  } else {
    tlo = CAUSAL ? (j0 * BC) / BR : 0;  // both blocks of the pair start at this tile
  }
  b0 = __builtin_amdgcn_readfirstlane(b0);
  n0 = __builtin_amdgcn_readfirstlane(n0);
  b1 = __builtin_amdgcn_readfirstlane(b1);
  n1 = __builtin_amdgcn_readfirstlane(n1);
  // cursor: head index hc, list positions (i0, i1) or tile tc, half hf
  struct Cur {
    int hc, i0, i1, tc, hf;
  };
  auto touches = [&](int h, int t, int hf, int jb) __attribute__((always_inline)) {
    const int row0 = t * BR + 64 * hf;
    if (jb >= p.Tc || row0 >= p.Nq) return false;
    if (CAUSAL && row0 + 63 < jb * BC) return false;
    if (p.block_state && p.block_state[(((int64_t)b * p.Hq + h) * p.Tr + t) * p.Tc + jb] == 2) return false;
    return true;
  };
  // tile at the cursor and which blocks' lists hold it (-1: head exhausted)
  auto tile_at = [&](const Cur& c, bool& in0, bool& in1) __attribute__((always_inline)) {
    if (p.col_ptr) {
      const int t0 = c.i0 < n0 ? rowi[b0 + c.i0] : INT32_MAX;
      const int t1 = c.i1 < n1 ? rowi[b1 + c.i1] : INT32_MAX;
      const int t = min(t0, t1);
      in0 = t0 == t;
      in1 = t1 == t;
      return t == INT32_MAX ? -1 : t;
    }
    in0 = true;
    in1 = has1;
    return c.tc < p.Tr ? c.tc : -1;
  };
  auto step = [&](Cur& c) __attribute__((always_inline)) {  // to the next (tile, half) position
    bool in0, in1;
    if (c.hf == 0) {
      c.hf = 1;
      return;
    }
    c.hf = 0;
    if (p.col_ptr) {
      tile_at(c, in0, in1);
      c.i0 += in0 ? 1 : 0;
      c.i1 += in1 ? 1 : 0;
    } else {
      ++c.tc;
    }
  };
  // advance c to the first kept stage at or after it; false when none is left
  auto settle = [&](Cur& c, int& t, int& need) __attribute__((always_inline)) {
    for (;;) {
      if (c.hc >= G) return false;
      bool in0, in1;
      t = tile_at(c, in0, in1);
      if (t < 0) {  // next head
        c = Cur{c.hc + 1, 0, 0, tlo, 0};
        continue;
      }
      const int h = g * G + c.hc;
      need = (in0 && touches(h, t, c.hf, j0) ? 1 : 0) | (in1 && touches(h, t, c.hf, j0 + 1) ? 2 : 0);
      if (need) return true;
      step(c);
    }
  };
  auto fetch = [&](int buf, int h, int t, int hf) __attribute__((always_inline)) {
    const int row0 = t * BR + 64 * hf;
    dma_tile64_w8<D>(sm.q[buf], static_cast<const __bf16*>(p.q) + (int64_t)b * p.qs_b + (int64_t)h * p.qs_h, p.Nq,
                     p.qs_t, row0, wave, lane);
    dma_tile64_w8<D>(sm.g[buf], static_cast<const __bf16*>(p.dout) + (int64_t)b * p.dos_b + (int64_t)h * p.dos_h,
                     p.Nq, p.dos_t, row0, wave, lane);
    const int64_t rb = ((int64_t)b * p.Hq + h) * p.Nq;
    if (wave == 0) dma_row64(sm.lse[buf], p.lse + rb, p.Nq, row0, lane);
    if (wave == 1) dma_row64(sm.dvec[buf], p.dvec + rb, p.Nq, row0, lane);
  };

  f32x16 dk[NTD], dv[NTD];
#pragma unroll
  for (int n = 0; n < NTD; ++n) {
    dk[n] = f32x16{};
    dv[n] = f32x16{};
  }

  Cur cur{0, 0, 0, tlo, 0};
  int t_cur = 0, need_cur = 0;
  bool have = settle(cur, t_cur, need_cur);
  if (have) fetch(0, g * G + cur.hc, t_cur, cur.hf);
  for (int st = 0; have; ++st) {
    const int buf = st & 1;
    // this stage (and, the first time, K and V) has landed in every wave, and
    // every wave is done with the previous stage, whose buffers are next
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const int h = g * G + cur.hc, t = t_cur, hf = cur.hf, need = need_cur;
    Cur nxt = cur;
    step(nxt);
    int t_nxt = 0, need_nxt = 0;
    const bool have_nxt = settle(nxt, t_nxt, need_nxt);
    if (have_nxt) fetch(buf ^ 1, g * G + nxt.hc, t_nxt, nxt.hf);

    if ((need >> kb) & 1) {
      const int row0 = t * BR + 64 * hf;
      const int nrows = min(64, p.Nq - row0);
      const int r0 = 32 * qh;
      const __bf16* sq = sm.q[buf];
      const __bf16* sg = sm.g[buf];
      f32x16 s = f32x16{}, dp = f32x16{};
      bf16x8 frg[4], frq[4], dbp = bf16x8{};
#pragma unroll
      for (int n = 0; n < 4; ++n) frq[n] = bf16x8{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(read_row<D>(sq, r0 + l32, ks, hi), read_row<D>(sm.k[kb], 32 * kh + l32, ks, hi), s);
        dp = mfma32(read_row<D>(sg, r0 + l32, ks, hi), read_row<D>(sm.v[kb], 32 * kh + l32, ks, hi), dp);
        if (ks % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float pv[8], dsv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int a = 8 * kk + i;
          const int rl = r0 + 8 * (a >> 2) + 4 * hi + (a & 3);
          const bool ok = key_ok && rl < nrows && (!CAUSAL || key <= row0 + rl);
          pv[i] = ok ? fast_exp2(fmaf(s[a], c2, -sm.lse[buf][rl] * kLog2e)) : 0.0f;
          dsv[i] = pv[i] * (dp[a] - sm.dvec[buf][rl]);
        }
        const bf16x8 pb = to_bf16x8(pv);
        const bf16x8 db = to_bf16x8(dsv);
        // (the first read follows the dK products of the previous step; the
        // S and dP products before the first step have been waited for)
        read_tr_x4(frg, sg, r0 + 16 * kk, lane, frq, dbp);
#pragma unroll
        for (int n = 0; n < NTD; ++n) dv[n] = mfma32(frg[n], pb, dv[n]);  // dV^T += dO^T P
        read_tr_x4(frq, sq, r0 + 16 * kk, lane, frg, pb);
#pragma unroll
        for (int n = 0; n < NTD; ++n) dk[n] = mfma32(frq[n], db, dk[n]);  // dK^T += Q^T dS
        dbp = db;
      }
    }
    cur = nxt;
    t_cur = t_nxt;
    need_cur = need_nxt;
    have = have_nxt;
  }

  // each block's row halves: waves with qh = 1 hand their sums to the waves
  // with qh = 0 through LDS (free once every wave is past its last stage)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  static_assert(sizeof(float) * 4 * 2 * NTD * 16 * 64 <= sizeof(Dkdv2Smem<D>), "reduction fits in the tiles");
  float* red = reinterpret_cast<float*>(&sm) + (2 * kb + kh) * (2 * NTD * 16 * 64);
  if (qh == 1) {
#pragma unroll
    for (int n = 0; n < NTD; ++n)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        red[(n * 16 + a) * 64 + lane] = dk[n][a];
        red[((NTD + n) * 16 + a) * 64 + lane] = dv[n][a];
      }
  }
  __syncthreads();
  if (qh == 0 && jw < p.Tc && key < p.Nk) {
    __bf16* dkp = static_cast<__bf16*>(p.dk) + (int64_t)b * p.dks_b + (int64_t)key * p.dks_t + (int64_t)g * p.dks_h;
    __bf16* dvp = static_cast<__bf16*>(p.dv) + (int64_t)b * p.dvs_b + (int64_t)key * p.dvs_t + (int64_t)g * p.dvs_h;
#pragma unroll
    for (int n = 0; n < NTD; ++n) {
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        dk[n][a] += red[(n * 16 + a) * 64 + lane];
        dv[n][a] += red[((NTD + n) * 16 + a) * 64 + lane];
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int dcol = 32 * n + 8 * q4 + 4 * hi;
        store4(dkp + dcol, dk[n], q4, p.scale);
        store4(dvp + dcol, dv[n], q4, 1.0f);
      }
    }
  }
#endif
}

template <int D>
struct DqSmem {
  __bf16 k[BC * D];
  __bf16 v[BC * D];
};

// One work-group per (batch, query head, query tile); wave w owns rows
// 32 w .. 32 w + 31 of the tile, one row per lane (split over l and l + 32).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void bwd_dq_kernel(const BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KS = D / 16;
  constexpr int NTD = D / 32;
  __shared__ DqSmem<D> sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  // work order: tile major (under a causal mask the last tiles, the longest,
  // first), then the group's query heads, the (batch, K/V head) index
  // fastest: with B Hkv a multiple of 8 a group stays on one XCD
  const int G = p.Hq / p.Hkv;
  const int NBG = p.B * p.Hkv;
  const int bg = blockIdx.x % NBG;
  const int hh = (blockIdx.x / NBG) % G;
  const int rank = blockIdx.x / (NBG * G);
  const int t = CAUSAL ? p.Tr - 1 - rank : rank;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int h = g * G + hh;
  const float c2 = p.scale * kLog2e;

  const int row = t * BR + wave * 32 + l32;
  const bool row_ok = row < p.Nq;
  const __bf16* qrow = static_cast<const __bf16*>(p.q) + (int64_t)b * p.qs_b + (int64_t)row * p.qs_t + (int64_t)h * p.qs_h;
  const __bf16* grow =
      static_cast<const __bf16*>(p.dout) + (int64_t)b * p.dos_b + (int64_t)row * p.dos_t + (int64_t)h * p.dos_h;
  bf16x8 qf[KS], gf[KS];  // B operands: X[row][16 ks + 8 hi + 0..7]
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * hi) : bf16x8{};
    gf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(grow + 16 * ks + 8 * hi) : bf16x8{};
  }
  const int64_t ri = ((int64_t)b * p.Hq + h) * p.Nq + row;
  const float lse2 = row_ok ? p.lse[ri] * kLog2e : 0.0f;
  const float dvr = row_ok ? p.dvec[ri] : 0.0f;

  // visited blocks: the tile's CSR list (or every block), minus blocks wholly
  // above the diagonal, exactly as the forward visits them
  const int last_row = min(t * BR + BR, p.Nq) - 1;
  int e0 = p.row_ptr ? p.row_ptr[t] : 0;
  int e1 = p.row_ptr ? p.row_ptr[t + 1] : p.Tc;
  if (CAUSAL) {
    if (p.row_ptr) {
      while (e1 > e0 && p.col_idx[e1 - 1] * BC > last_row) --e1;
    } else {
      e1 = min(e1, last_row / BC + 1);
    }
  }
  e0 = __builtin_amdgcn_readfirstlane(e0);
  e1 = __builtin_amdgcn_readfirstlane(e1);

  const __bf16* kbase = static_cast<const __bf16*>(p.k) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + (int64_t)b * p.vs_b + (int64_t)g * p.vs_h;
  f32x16 dq[NTD];
#pragma unroll
  for (int n = 0; n < NTD; ++n) dq[n] = f32x16{};

  // the next block's K and V are read into registers while this one computes
  Staged<D, BC> nk, nv;
  auto fetch = [&](int e) __attribute__((always_inline)) {
    const int j = __builtin_amdgcn_readfirstlane(p.row_ptr ? p.col_idx[e] : e);
    const int nkeys = min(BC, p.Nk - j * BC);
    nk.load(kbase + (int64_t)(j * BC) * p.ks_t, p.ks_t, nkeys, tid);
    nv.load(vbase + (int64_t)(j * BC) * p.vs_t, p.vs_t, nkeys, tid);
  };
  if (e0 < e1) fetch(e0);
  const uint8_t* skipped = p.block_state ? p.block_state + (((int64_t)b * p.Hq + h) * p.Tr + t) * p.Tc : nullptr;
  for (int e = e0; e < e1; ++e) {
    const int j = __builtin_amdgcn_readfirstlane(p.row_ptr ? p.col_idx[e] : e);
    __syncthreads();  // every wave is done reading the previous block
    nk.store(sm.k, tid);
    nv.store(sm.v, tid);
    __syncthreads();
    if (e + 1 < e1) fetch(e + 1);
    if (skipped && skipped[j] == 2) continue;  // the forward skipped it: no gradient (uniform branch)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {  // 32-key halves of the block
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(read_row<D>(sm.k, 32 * mt + l32, ks, hi), qf[ks], s);   // S^T[key][q]
        dp = mfma32(read_row<D>(sm.v, 32 * mt + l32, ks, hi), gf[ks], dp);  // dP^T[key][q]
      }
      float dsv[16];
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int key = j * BC + 32 * mt + 8 * (a >> 2) + 4 * hi + (a & 3);
        const bool ok = row_ok && key < p.n_valid && (!CAUSAL || key <= row);
        const float pr = ok ? fast_exp2(fmaf(s[a], c2, -lse2)) : 0.0f;
        dsv[a] = pr * (dp[a] - dvr);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 db = to_bf16x8(dsv + 8 * kk);
#pragma unroll
        for (int n = 0; n < NTD; ++n) dq[n] = mfma32(read_tr<D>(sm.k, 32 * mt + 16 * kk, n, lane), db, dq[n]);
      }
    }
  }

  if (row_ok) {
    __bf16* dqp = static_cast<__bf16*>(p.dq) + (int64_t)b * p.dqs_b + (int64_t)row * p.dqs_t + (int64_t)h * p.dqs_h;
#pragma unroll
    for (int n = 0; n < NTD; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) store4(dqp + 32 * n + 8 * q4 + 4 * hi, dq[n], q4, p.scale);
  }
#endif
}

// dQ at d = 128 with the key blocks streamed global -> LDS by DMA into two
// stages (the kernel above reads the next block into registers and copies
// it to LDS between two barriers): block e + 1 lands while block e is
// computed, behind one barrier per block.  The transposed reads are asm
// blocks under the same rule as in the dK/dV pair kernel.
template <bool CAUSAL>
__global__ __launch_bounds__(NT, 2) void bwd_dq_db_kernel(const BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int D = 128;
  constexpr int KS = D / 16;
  constexpr int NTD = D / 32;
  __shared__ __bf16 smk[2][BC * D];
  __shared__ __bf16 smv[2][BC * D];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  // work order as above
  const int G = p.Hq / p.Hkv;
  const int NBG = p.B * p.Hkv;
  const int bg = blockIdx.x % NBG;
  const int hh = (blockIdx.x / NBG) % G;
  const int rank = blockIdx.x / (NBG * G);
  const int t = CAUSAL ? p.Tr - 1 - rank : rank;
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int h = g * G + hh;
  const float c2 = p.scale * kLog2e;

  const int row = t * BR + wave * 32 + l32;
  const bool row_ok = row < p.Nq;
  const __bf16* qrow = static_cast<const __bf16*>(p.q) + (int64_t)b * p.qs_b + (int64_t)row * p.qs_t + (int64_t)h * p.qs_h;
  const __bf16* grow =
      static_cast<const __bf16*>(p.dout) + (int64_t)b * p.dos_b + (int64_t)row * p.dos_t + (int64_t)h * p.dos_h;
  bf16x8 qf[KS], gf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * hi) : bf16x8{};
    gf[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(grow + 16 * ks + 8 * hi) : bf16x8{};
  }
  const int64_t ri = ((int64_t)b * p.Hq + h) * p.Nq + row;
  const float lse2 = row_ok ? p.lse[ri] * kLog2e : 0.0f;
  const float dvr = row_ok ? p.dvec[ri] : 0.0f;

  const int last_row = min(t * BR + BR, p.Nq) - 1;
  int e0 = p.row_ptr ? p.row_ptr[t] : 0;
  int e1 = p.row_ptr ? p.row_ptr[t + 1] : p.Tc;
  if (CAUSAL) {
    if (p.row_ptr) {
      while (e1 > e0 && p.col_idx[e1 - 1] * BC > last_row) --e1;
    } else {
      e1 = min(e1, last_row / BC + 1);
    }
  }
  e0 = __builtin_amdgcn_readfirstlane(e0);
  e1 = __builtin_amdgcn_readfirstlane(e1);

  // block indices through the scalar cache, one iteration ahead
  typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
  const const_i32_ptr cols = p.col_idx ? (const_i32_ptr)p.col_idx : nullptr;
  auto blk = [&](int e) __attribute__((always_inline)) { return e < e1 ? (cols ? cols[e] : e) : 0; };
  const __bf16* kbase = static_cast<const __bf16*>(p.k) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + (int64_t)b * p.vs_b + (int64_t)g * p.vs_h;
  auto fetch = [&](int buf, int j) __attribute__((always_inline)) {
    dma_tile64<D>(smk[buf], kbase, p.Nk, p.ks_t, j * BC, wave, lane);
    dma_tile64<D>(smv[buf], vbase, p.Nk, p.vs_t, j * BC, wave, lane);
  };
  f32x16 dq[NTD];
#pragma unroll
  for (int n = 0; n < NTD; ++n) dq[n] = f32x16{};

  const uint8_t* skipped = p.block_state ? p.block_state + (((int64_t)b * p.Hq + h) * p.Tr + t) * p.Tc : nullptr;
  int j = blk(e0), jn = blk(e0 + 1);
  if (e0 < e1) fetch(0, j);
  bf16x8 fa[4], fb[4], dbp = bf16x8{};
#pragma unroll
  for (int n = 0; n < 4; ++n) fb[n] = bf16x8{};
  for (int e = e0; e < e1; ++e) {
    const int buf = (e - e0) & 1;
    // block e has landed in every wave, and every wave is done with block e - 1
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (e + 1 < e1) fetch(buf ^ 1, jn);
    const int jc = j;
    j = jn;
    jn = blk(e + 2);
    if (skipped && skipped[jc] == 2) continue;  // the forward skipped it: no gradient (uniform branch)
    const __bf16* sk = smk[buf];
    const __bf16* sv = smv[buf];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {  // 32-key halves of the block
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(read_row<D>(sk, 32 * mt + l32, ks, hi), qf[ks], s);   // S^T[key][q]
        dp = mfma32(read_row<D>(sv, 32 * mt + l32, ks, hi), gf[ks], dp);  // dP^T[key][q]
      }
      float dsv[16];
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        const int key = jc * BC + 32 * mt + 8 * (a >> 2) + 4 * hi + (a & 3);
        const bool ok = row_ok && key < p.n_valid && (!CAUSAL || key <= row);
        const float pr = ok ? fast_exp2(fmaf(s[a], c2, -lse2)) : 0.0f;
        dsv[a] = pr * (dp[a] - dvr);
      }
      const bf16x8 d0 = to_bf16x8(dsv), d1 = to_bf16x8(dsv + 8);
      read_tr_x4(fa, sk, 32 * mt, lane, fb, dbp);
#pragma unroll
      for (int n = 0; n < NTD; ++n) dq[n] = mfma32(fa[n], d0, dq[n]);
      read_tr_x4(fb, sk, 32 * mt + 16, lane, fa, d0);
#pragma unroll
      for (int n = 0; n < NTD; ++n) dq[n] = mfma32(fb[n], d1, dq[n]);
      dbp = d1;
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (row_ok) {
    __bf16* dqp = static_cast<__bf16*>(p.dq) + (int64_t)b * p.dqs_b + (int64_t)row * p.dqs_t + (int64_t)h * p.dqs_h;
#pragma unroll
    for (int n = 0; n < NTD; ++n)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) store4(dqp + 32 * n + 8 * q4 + 4 * hi, dq[n], q4, p.scale);
  }
#endif
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.Hq * p.Nq;
  const int64_t dot_blocks = (rows * (D / 8) + NT - 1) / NT;
  hipLaunchKernelGGL((bwd_dot_kernel<D>), dim3((unsigned)dot_blocks), dim3(NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D == 128)
    hipLaunchKernelGGL((bwd_dkdv_pair_kernel<CAUSAL>), dim3((unsigned)((int64_t)p.B * p.Hkv * ((p.Tc + 1) / 2))),
                       dim3(NT2), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)p.B * p.Hkv * p.Tc)), dim3(NT), 0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if constexpr (D == 128)
    hipLaunchKernelGGL((bwd_dq_db_kernel<CAUSAL>), dim3((unsigned)((int64_t)p.B * p.Hq * p.Tr)), dim3(NT), 0, s, p);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)p.B * p.Hq * p.Tr)), dim3(NT), 0, s, p);
  return hipGetLastError();
}

}  // namespace

int launch_prefill_bwd(const BwdParams& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.d == 64) return p.causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
  return p.causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
}

}  // namespace bsattn
