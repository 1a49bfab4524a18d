// bf16 backward of static block-sparse attention on CDNA4 matrix cores.
//
// For the loss sum(out * dout) of the forward out = softmax(scale Q K^T) V
// over the block mask (tiles of 128 query rows x blocks of 64 keys, plus the
// token-level valid-length and causal limits), with P rebuilt from the
// forward's per-row log-sum-exp:
//
//   dot   Dv[i] = sum_c dout[i][c] out[i][c]            (one float per row;
//         the same launch zeroes the schedules' arrival counters)
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
// Optional schedules cut the longest walks (a tile whose list holds every
// key block, a key block every tile attends) into chunks of the list, or of
// the (query head, tile) positions of a key-block group: a chunk writes its
// fp32 accumulators to a workspace slot and the last chunk to arrive adds
// the slots in slot order (DiT article section 5.3: uneven rows unbalance
// the GPU).  The sums stay deterministic.
//
// The pages print no backward pass; the gradients are the chain rule on the
// forward's definition (the DiT article trains with the block-sparse
// forward, section 4; its section 3.3 check of the block list before any
// load applies to both walks here).

#include <cstddef>

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

// Row fragment: X[r][16 ks + 8 hi + 0..7] (A operand rows, or B operand columns).
template <int D>
__device__ __forceinline__ bf16x8 read_row(const __bf16* tile, int r, int ks, int hi) {
  return *reinterpret_cast<const bf16x8*>(tile + BTile<D>::pos(r, 2 * ks + hi));
}

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr_b(const void* ptr) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)(ptr);
}

// Byte i of a block-state array, at a wave-uniform index, through the scalar
// cache: the aligned word that holds it is read (a word never straddles a
// page, so this stays inside the array's page) and the byte taken out.  A
// vector byte load would be waited for with vmcnt, which also waits for
// the next stage's loads in flight.
__device__ __forceinline__ int state_byte(const uint8_t* base, int64_t i) {
  typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
  const uintptr_t a = reinterpret_cast<uintptr_t>(base) + (uintptr_t)i;
  const uint32_t w = *reinterpret_cast<const_u32_ptr>(a & ~(uintptr_t)3);
  return (int)((w >> (8 * (a & 3))) & 0xffu);
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
  // the schedules' arrival counters sit at offsets that depend on the call's
  // shape, so a shared workspace may hold any bytes there: zero them here,
  // ahead of the kernels that count with them
  const int64_t nthreads = (int64_t)gridDim.x * NT;
  if (p.dq_arrive) {
    const int64_t n = (int64_t)p.dq_n_merges * p.B * p.Hq;
    for (int64_t i = gid; i < n; i += nthreads) p.dq_arrive[i] = 0;
  }
  if (p.kv_arrive) {
    const int64_t n = (int64_t)p.kv_n_merges * p.B * p.Hkv;
    for (int64_t i = gid; i < n; i += nthreads) p.kv_arrive[i] = 0;
  }
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

// ---- dK/dV: double-buffered query stages ------------------------------------
//
// One work-group per (batch, K/V head, group of NB adjacent key blocks).  K
// and V of its blocks stay in LDS; the query rows of every tile that attends
// one of them stream in 64-row stages (Q, dO, and the rows' lse and Dv),
// double-buffered: the next stage lands while the current one is computed,
// behind a single barrier per stage.  Waves 4 kb .. 4 kb + 3 work on block
// NB m + kb: wave bits (kh, qh) pick keys 32 kh .. +31 of the block and rows
// 32 qh .. +31 of the stage.  The stages visited are those of any of the
// blocks (the union of their tiles' lists, or the shared causal range), and
// a block's waves sit out stages that do not touch it.
//
// At d = 128, NB = 2: two blocks share each stage's loads, one work-group of
// eight waves per CU (129 KB of LDS).  At d = 64, NB = 1: three four-wave
// work-groups per CU (49 KB each); pairs there (one or two eight-wave groups
// per CU) measured slower on the multimodal DiT shape, which has few key
// blocks per head.  The stages' transposed reads are inline asm that waits
// inside the block: the intrinsic would make the compiler wait for the next
// stage's load first (it cannot tell the stages apart).

template <int D>
constexpr int kDkdvBlocks = D == 64 ? kDkdvBlocks64 : kDkdvBlocks128;
template <int D>
constexpr int kDkdvGroupsPerCu = D == 64 ? 3 : 1;

template <int D, int NB>
struct DkdvSmem {
  __bf16 k[NB][BC * D];  // keys of blocks NB m .. NB m + NB - 1
  __bf16 v[NB][BC * D];
  __bf16 q[2][64 * D];  // double-buffered 64-row query stages
  __bf16 g[2][64 * D];  // their dout
  alignas(16) float lse[2][64];  // per stage: lse (natural log) and Dv of its rows
  alignas(16) float dvec[2][64];
  int ticket;           // a chunk's arrival ticket (after the reduction, which overlays the tiles)
};

// 64 x D tile, global -> LDS, by all NW waves of the work-group (rows past
// rows_total: zeros); the layout of dma_tile64 for any wave count.
template <int D, int NW>
__device__ __forceinline__ void dma_tile64_wn(__bf16* tile, const __bf16* head, int rows_total, int64_t stride_t,
                                              int row0, int wave, int lane) {
  constexpr int CH = D / 8;
  constexpr int NI = 64 * CH / (64 * NW);
  const uint32_t extent = (uint32_t)(((int64_t)(rows_total - 1) * stride_t + D) * 2);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(head), (short)0, (int)extent, kBufferWord3);
  const uint32_t soff = (uint32_t)((int64_t)row0 * stride_t * 2);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int slot = (NW * i + wave) * 64 + lane;
    const int r = slot / CH, cp = slot % CH;
    const int c = cp ^ BTile<D>::swz(r);
    const uint32_t voff = (uint32_t)(((int64_t)r * stride_t + 8 * c) * 2);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + (NW * i + wave) * 64 * 8), 16, voff, soff, 0, 0);
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

// Transposed fragments (A operands X^T[m = d][k]) of one 16-row step at row
// r0, for the D / 32 d-tiles n: lane l gets, in slot i of out[n],
// X[r0 + 8 (i/4) + 4 (l/32) + i%4][32 n + l%32], the row order of the
// accumulator layout above.  The loads are issued together and waited for
// inside the asm block.
// The loads return into their registers some cycles after the block issues
// them, which the compiler does not see: `busy` (the operands of the MFMAs
// issued just before) are inputs of the block, and its outputs are
// early-clobber, so no output is placed on an input.
template <int D>
__device__ __forceinline__ void read_tr_xn(bf16x8 (&out)[D / 32], const __bf16* tile, int r0, int lane,
                                           const bf16x8 (&busy)[D / 32], const bf16x8& busy_b) {
  constexpr int NN = D / 32;
  const int g16 = lane >> 4, j16 = lane & 15;
  const int r = r0 + 4 * (g16 >> 1) + (j16 >> 2);
  const int half = 4 * (j16 & 1);
  uint32_t a[2 * NN];
#pragma unroll
  for (int n = 0; n < NN; ++n) {
    const int c = 4 * n + 2 * (g16 & 1) + ((j16 & 3) >> 1);
    a[2 * n] = lds_addr_b(tile + BTile<D>::pos(r, c) + half);
    a[2 * n + 1] = lds_addr_b(tile + BTile<D>::pos(r + 8, c) + half);
  }
  i16x4 x[2 * NN];
  if constexpr (D == 128) {
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
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n"
        "ds_read_b64_tr_b16 %1, %5\n"
        "ds_read_b64_tr_b16 %2, %6\n"
        "ds_read_b64_tr_b16 %3, %7\n"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(busy[0]), "v"(busy[1]), "v"(busy_b)
        : "memory");
  }
#pragma unroll
  for (int n = 0; n < NN; ++n) out[n] = join_bf16x4(x[2 * n], x[2 * n + 1]);
}

// launch bound: waves per SIMD (a work-group puts NB waves on each SIMD)
template <int D, bool CAUSAL>
__global__ __launch_bounds__(256 * kDkdvBlocks<D>, kDkdvBlocks<D> * kDkdvGroupsPerCu<D>) void bwd_dkdv_kernel(
    const BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NB = kDkdvBlocks<D>;
  constexpr int NW = 4 * NB;
  constexpr int KS = D / 16;
  constexpr int NTD = D / 32;
  __shared__ DkdvSmem<D, NB> sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int kb = wave >> 2, kh = wave & 1, qh = (wave >> 1) & 1;
  // work order: key-block groups ascending (under a causal mask the first
  // blocks have the most query tiles: longest first), or the schedule's
  // items (longest first); the (batch, K/V head) index runs fastest, so with
  // B Hkv a multiple of 8 a group stays on one XCD (work-group i runs on XCD
  // i % 8) and its Q / dO tiles in one L2
  const int NBG = p.B * p.Hkv;
  const int rank = blockIdx.x / NBG;
  const int bg = blockIdx.x % NBG;
  // the item: a group's (query head, tile) positions [pos_begin, pos_end)
  // in head-major order, starting at head hc0 with list positions (i00, i10)
  int m = rank, pos_begin = 0, pos_end = INT32_MAX, hc0 = 0, i00 = 0, i10 = 0, slot = -1, mrg = -1;
  if (p.kv_items) {
    const int32_t* item = p.kv_items + kKvItemInts * rank;
    m = item[0];
    pos_begin = item[1];
    pos_end = item[2];
    hc0 = item[3];
    i00 = item[4];
    i10 = item[5];
    slot = item[6];
    mrg = item[7];
  }
  m = __builtin_amdgcn_readfirstlane(m);
  pos_begin = __builtin_amdgcn_readfirstlane(pos_begin);
  pos_end = __builtin_amdgcn_readfirstlane(pos_end);
  hc0 = __builtin_amdgcn_readfirstlane(hc0);
  i00 = __builtin_amdgcn_readfirstlane(i00);
  i10 = __builtin_amdgcn_readfirstlane(i10);
  slot = __builtin_amdgcn_readfirstlane(slot);
  mrg = __builtin_amdgcn_readfirstlane(mrg);
  const int g = bg % p.Hkv, b = bg / p.Hkv;
  const int G = p.Hq / p.Hkv;
  const float c2 = p.scale * kLog2e;
  const int j0 = NB * m;
  const bool has1 = NB == 2 && j0 + 1 < p.Tc;
  const int jw = j0 + kb;  // this wave's block

  const int key = jw * BC + 32 * kh + l32;
  const bool key_ok = key < p.n_valid;
  const __bf16* kh_base = static_cast<const __bf16*>(p.k) + (int64_t)b * p.ks_b + (int64_t)g * p.ks_h;
  const __bf16* vh_base = static_cast<const __bf16*>(p.v) + (int64_t)b * p.vs_b + (int64_t)g * p.vs_h;
  dma_tile64_wn<D, NW>(sm.k[0], kh_base, p.Nk, p.ks_t, j0 * BC, wave, lane);
  dma_tile64_wn<D, NW>(sm.v[0], vh_base, p.Nk, p.vs_t, j0 * BC, wave, lane);
  if constexpr (NB == 2) {
    if (has1) {
      dma_tile64_wn<D, NW>(sm.k[1], kh_base, p.Nk, p.ks_t, (j0 + 1) * BC, wave, lane);
      dma_tile64_wn<D, NW>(sm.v[1], vh_base, p.Nk, p.vs_t, (j0 + 1) * BC, wave, lane);
    }
  }

  // the stages: for each query head of the group, the tiles holding either
  // block (merge of the two transposed lists, or the causal / dense range
  // shared by the group), two 64-row halves each; a stage is kept when it
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
    tlo = CAUSAL ? (j0 * BC) / BR : 0;  // every block of the group starts at this tile
  }
  b0 = __builtin_amdgcn_readfirstlane(b0);
  n0 = __builtin_amdgcn_readfirstlane(n0);
  b1 = __builtin_amdgcn_readfirstlane(b1);
  n1 = __builtin_amdgcn_readfirstlane(n1);
  // cursor: head index hc, list positions (i0, i1) or tile tc, half hf, and
  // the position (head, tile) index
  struct Cur {
    int hc, i0, i1, tc, hf, pos;
  };
  auto touches = [&](int h, int t, int hf, int jb) __attribute__((always_inline)) {
    const int row0 = t * BR + 64 * hf;
    if (jb >= p.Tc || row0 >= p.Nq) return false;
    if (CAUSAL && row0 + 63 < jb * BC) return false;
    if (p.block_state && state_byte(p.block_state, (((int64_t)b * p.Hq + h) * p.Tr + t) * p.Tc + jb) == 2) return false;
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
    ++c.pos;
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
      if (c.hc >= G || c.pos >= pos_end) return false;
      bool in0, in1;
      t = tile_at(c, in0, in1);
      if (t < 0) {  // next head (a head's positions end with its last tile)
        c = Cur{c.hc + 1, 0, 0, tlo, 0, c.pos};
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
    dma_tile64_wn<D, NW>(sm.q[buf], static_cast<const __bf16*>(p.q) + (int64_t)b * p.qs_b + (int64_t)h * p.qs_h,
                         p.Nq, p.qs_t, row0, wave, lane);
    dma_tile64_wn<D, NW>(sm.g[buf], static_cast<const __bf16*>(p.dout) + (int64_t)b * p.dos_b + (int64_t)h * p.dos_h,
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

  Cur cur{hc0, i00, i10, tlo, 0, pos_begin};
  int t_cur = 0, need_cur = 0;
  bool have = settle(cur, t_cur, need_cur);
  if (have) fetch(0, g * G + cur.hc, t_cur, cur.hf);
  for (int st = 0; have; ++st) {
    const int buf = st & 1;
    // this stage (and, the first time, K and V) has landed in every wave, and
    // every wave is done with the previous stage, whose buffers are next
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    const int t = t_cur, hf = cur.hf, need = need_cur;
    Cur nxt = cur;
    step(nxt);
    int t_nxt = 0, need_nxt = 0;
    const bool have_nxt = settle(nxt, t_nxt, need_nxt);
    // the next stage's loads: after this stage's S and dP products, so that
    // their LDS writes do not land under those products' fragment reads (at
    // once in waves whose block sits this stage out; every wave loads its
    // share of the stage)
    const bool mine = (need >> kb) & 1;
    if (!mine && have_nxt) fetch(buf ^ 1, g * G + nxt.hc, t_nxt, nxt.hf);

    if (mine) {
      const int row0 = t * BR + 64 * hf;
      const int nrows = min(64, p.Nq - row0);
      const int r0 = 32 * qh;
      const __bf16* sq = sm.q[buf];
      const __bf16* sg = sm.g[buf];
      const __bf16* skb = sm.k[kb];
      const __bf16* svb = sm.v[kb];
      f32x16 s = f32x16{}, dp = f32x16{};
      bf16x8 frg[NTD], frq[NTD], dbp = bf16x8{};
#pragma unroll
      for (int n = 0; n < NTD; ++n) frq[n] = bf16x8{};
      // S = Q K^T and dP = dO V^T: each pair of fragments is read for the
      // next key step as soon as the product that used it has issued, so the
      // read runs under the other chain's product
      bf16x8 fq = read_row<D>(sq, r0 + l32, 0, hi), fk = read_row<D>(skb, 32 * kh + l32, 0, hi);
      bf16x8 fg = read_row<D>(sg, r0 + l32, 0, hi), fv = read_row<D>(svb, 32 * kh + l32, 0, hi);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = mfma32(fq, fk, s);
        if (ks + 1 < KS) {
          fq = read_row<D>(sq, r0 + l32, ks + 1, hi);
          fk = read_row<D>(skb, 32 * kh + l32, ks + 1, hi);
        }
        dp = mfma32(fg, fv, dp);
        if (ks + 1 < KS) {
          fg = read_row<D>(sg, r0 + l32, ks + 1, hi);
          fv = read_row<D>(svb, 32 * kh + l32, ks + 1, hi);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (have_nxt) fetch(buf ^ 1, g * G + nxt.hc, t_nxt, nxt.hf);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // P and dS of this lane's 8 (row, key) pairs of the key step, rows
        // r0 + 16 kk + 8 q + 4 hi + (0..3), q = 0, 1; masked pairs take 0 by a
        // select (no branch).  The rows' lse and Dv come in four-row reads
        // issued and waited for in one asm block: read plainly, they made the
        // compiler wait first for the next stage's global->LDS loads (it
        // cannot tell the stage read from the stage being filled).  The S and
        // dP accumulators stay live, so no output lands on an in-flight
        // product's accumulator.
        f32x4 l4[2], d4[2];
        asm volatile(
            "ds_read_b128 %0, %4\n"
            "ds_read_b128 %1, %4 offset:32\n"
            "ds_read_b128 %2, %5\n"
            "ds_read_b128 %3, %5 offset:32\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(l4[0]), "=&v"(l4[1]), "=&v"(d4[0]), "=&v"(d4[1])
            : "v"(lds_addr_b(sm.lse[buf] + r0 + 16 * kk + 4 * hi)), "v"(lds_addr_b(sm.dvec[buf] + r0 + 16 * kk + 4 * hi))
            : "memory");
        float pv[8], dsv[8];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int rb = r0 + 16 * kk + 8 * q + 4 * hi;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 4 * q + u, a = 8 * kk + i, rl = rb + u;
            const bool ok = key_ok && rl < nrows && (!CAUSAL || key <= row0 + rl);
            const float e = fast_exp2(fmaf(s[a], c2, -l4[q][u] * kLog2e));
            pv[i] = ok ? e : 0.0f;
            dsv[i] = pv[i] * (dp[a] - d4[q][u]);
          }
        }
        const bf16x8 pb = to_bf16x8(pv);
        const bf16x8 db = to_bf16x8(dsv);
        // (key step 1: the operands of key step 0's dK products; key step 0:
        // nothing, the S and dP products having been waited for)
        read_tr_xn<D>(frg, sg, r0 + 16 * kk, lane, frq, dbp);
#pragma unroll
        for (int n = 0; n < NTD; ++n) dv[n] = mfma32(frg[n], pb, dv[n]);  // dV^T += dO^T P
        __builtin_amdgcn_sched_barrier(0);  // the dV products issue before the Q^T reads
        read_tr_xn<D>(frq, sq, r0 + 16 * kk, lane, frg, pb);
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
  using Sm = DkdvSmem<D, NB>;
  static_assert(sizeof(float) * 2 * NB * 2 * NTD * 16 * 64 <= offsetof(Sm, ticket),
                "reduction fits in the tiles, clear of the ticket");
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
  if (qh == 0) {
#pragma unroll
    for (int n = 0; n < NTD; ++n)
#pragma unroll
      for (int a = 0; a < 16; ++a) {
        dk[n][a] += red[(n * 16 + a) * 64 + lane];
        dv[n][a] += red[((NTD + n) * 16 + a) * 64 + lane];
      }
  }
  if (slot >= 0) {
    // ---- chunk of a cut group: the waves holding the sums (qh = 0) publish
    //      them, the work-group takes an arrival ticket, and the last chunk
    //      to arrive adds every partial of the group in slot order (its own
    //      read back like the others)
    constexpr int PER = NB * 2 * 2 * NTD * 16 * 64;  // floats per (slot, batch, K/V head)
    const int s0 = p.kv_merges[3 * mrg + 1];
    const int ns = p.kv_merges[3 * mrg + 2];
    auto part = [&](int sl) __attribute__((always_inline)) {
      return p.kv_part + (((int64_t)sl * p.B + b) * p.Hkv + g) * PER + (2 * kb + kh) * (2 * NTD * 16 * 64) + lane;
    };
    if (qh == 0) {
      float* pp = part(slot);
#pragma unroll
      for (int n = 0; n < NTD; ++n)
#pragma unroll
        for (int a = 0; a < 16; ++a) {
          store_coherent(pp + (n * 16 + a) * 64, dk[n][a]);
          store_coherent(pp + ((NTD + n) * 16 + a) * 64, dv[n][a]);
        }
    }
    wait_stores_done();
    __syncthreads();  // every wave's partial has completed
    if (tid == 0) sm.ticket = atomicAdd(p.kv_arrive + ((int64_t)mrg * p.B + b) * p.Hkv + g, 1);
    __syncthreads();
    if (sm.ticket != ns - 1) return;  // a later chunk adds them up
    if (qh == 0) {
#pragma unroll
      for (int n = 0; n < NTD; ++n) {
        dk[n] = f32x16{};
        dv[n] = f32x16{};
      }
      for (int sl = s0; sl < s0 + ns; ++sl) {
        const float* pp = part(sl);
#pragma unroll
        for (int n = 0; n < NTD; ++n) {
          // a d tile's 32 values loaded together, then added (added as each
          // arrived, the loads went out one at a time)
          float tk[16], tv[16];
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            tk[a] = load_coherent(pp + (n * 16 + a) * 64);
            tv[a] = load_coherent(pp + ((NTD + n) * 16 + a) * 64);
          }
#pragma unroll
          for (int a = 0; a < 16; ++a) {
            dk[n][a] += tk[a];
            dv[n][a] += tv[a];
          }
        }
      }
    }
  }
  if (qh == 0 && jw < p.Tc && key < p.Nk) {
    __bf16* dkp = static_cast<__bf16*>(p.dk) + (int64_t)b * p.dks_b + (int64_t)key * p.dks_t + (int64_t)g * p.dks_h;
    __bf16* dvp = static_cast<__bf16*>(p.dv) + (int64_t)b * p.dvs_b + (int64_t)key * p.dvs_t + (int64_t)g * p.dvs_h;
#pragma unroll
    for (int n = 0; n < NTD; ++n) {
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

// dQ: one work-group per (batch, query head, query tile or chunk of its CSR
// list); wave w owns rows 32 w .. 32 w + 31 of the tile, one row per lane
// (split over l and l + 32).  Per visited key block
//   S^T = K Q^T, dP^T = V dO^T, dS^T = P^T (dP^T - Dv), dQ^T += K^T dS^T
// with Q and dO in registers and the key blocks streamed global -> LDS by
// DMA into two stages: block e + 1 lands while block e is computed, behind
// one barrier per block.  (At d = 64 a form that staged the next block
// through registers measured 3 % faster without a schedule on the
// multimodal DiT shape; one kernel serves both head dims.)  The transposed
// reads are asm blocks under the same rule as in the dK/dV kernel.
template <int D>
constexpr int kDqBlocksPerCu = D == 64 ? 3 : 2;

// the dQ kernel's LDS: two stages of one key block's K and V, and a chunk's
// arrival ticket.  One structure: with K and V as two separate arrays the
// compiler waited for the next block's global->LDS loads before the first
// read of the current block (it could not tell the two stages of an array
// apart), which took the prefetch off the loop.
template <int D>
struct DqSmem {
  __bf16 k[2][BC * D];
  __bf16 v[2][BC * D];
  int ticket;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT, kDqBlocksPerCu<D>) void bwd_dq_db_kernel(const BwdParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KS = D / 16;
  constexpr int NTD = D / 32;
  __shared__ DqSmem<D> sm;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  // work order: rank major (tiles, or the schedule's items, longest first;
  // under a causal mask without a schedule the last tiles, the longest,
  // first), then the group's query heads, the (batch, K/V head) index
  // fastest: with B Hkv a multiple of 8 a group stays on one XCD
  const int G = p.Hq / p.Hkv;
  const int NBG = p.B * p.Hkv;
  const int bg = blockIdx.x % NBG;
  const int hh = (blockIdx.x / NBG) % G;
  const int rank = blockIdx.x / (NBG * G);
  int t, e0, e1, slot = -1, mrg = -1;
  if (p.dq_items) {  // a work item of the schedule: a tile, or a chunk of its CSR list
    const int32_t* item = p.dq_items + 5 * rank;
    t = item[0];
    e0 = item[1];
    e1 = item[2];
    slot = item[3];
    mrg = item[4];
  } else {
    t = CAUSAL ? p.Tr - 1 - rank : rank;
    e0 = 0;
    e1 = p.Tc;
    if (p.row_ptr) {
      e0 = p.row_ptr[t];
      e1 = p.row_ptr[t + 1];
    }
  }
  t = __builtin_amdgcn_readfirstlane(t);
  slot = __builtin_amdgcn_readfirstlane(slot);
  mrg = __builtin_amdgcn_readfirstlane(mrg);
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

  // visited blocks: the item's CSR range (or every block), minus blocks
  // wholly above the diagonal, exactly as the forward visits them
  const int last_row = min(t * BR + BR, p.Nq) - 1;
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
    dma_tile64<D>(sm.k[buf], kbase, p.Nk, p.ks_t, j * BC, wave, lane);
    dma_tile64<D>(sm.v[buf], vbase, p.Nk, p.vs_t, j * BC, wave, lane);
  };
  f32x16 dq[NTD];
#pragma unroll
  for (int n = 0; n < NTD; ++n) dq[n] = f32x16{};

  const uint8_t* skipped = p.block_state ? p.block_state + (((int64_t)b * p.Hq + h) * p.Tr + t) * p.Tc : nullptr;
  int j = blk(e0), jn = blk(e0 + 1);
  if (e0 < e1) fetch(0, j);
  for (int e = e0; e < e1; ++e) {
    const int buf = (e - e0) & 1;
    // block e has landed in every wave, and every wave is done with block e - 1
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (e + 1 < e1) fetch(buf ^ 1, jn);
    const int jc = j;
    j = jn;
    jn = blk(e + 2);
    if (skipped && state_byte(skipped, jc) == 2) continue;  // the forward skipped it: no gradient
    const __bf16* sk = sm.k[buf];
    const __bf16* sv = sm.v[buf];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {  // 32-key halves of the block
      f32x16 s = f32x16{}, dp = f32x16{};
      // S^T[key][q] and dP^T[key][q], alternating; each K or V fragment is
      // read RA products ahead, into the register its product RA back used
      constexpr int NP = 2 * KS, RA = 2;
      auto frag = [&](int i) __attribute__((always_inline)) {
        return read_row<D>((i & 1) ? sv : sk, 32 * mt + l32, i >> 1, hi);
      };
      bf16x8 ring[RA];
#pragma unroll
      for (int i = 0; i < RA; ++i) ring[i] = frag(i);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        if (i & 1) dp = mfma32(ring[i % RA], gf[i >> 1], dp);
        else s = mfma32(ring[i % RA], qf[i >> 1], s);
        if (i + RA < NP) ring[i % RA] = frag(i + RA);
        __builtin_amdgcn_sched_barrier(0);
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
      // No product is in flight at this read: d0 comes from the results of
      // the last S and dP products, and a wave's products finish in the
      // order they were issued.  d0 fills the busy list so that the read
      // stays after that computation.
      bf16x8 dep[NTD];
#pragma unroll
      for (int n = 0; n < NTD; ++n) dep[n] = d0;
      bf16x8 fa[NTD], fb[NTD];
      read_tr_xn<D>(fa, sk, 32 * mt, lane, dep, d0);
#pragma unroll
      for (int n = 0; n < NTD; ++n) dq[n] = mfma32(fa[n], d0, dq[n]);
      __builtin_amdgcn_sched_barrier(0);
      read_tr_xn<D>(fb, sk, 32 * mt + 16, lane, fa, d0);
#pragma unroll
      for (int n = 0; n < NTD; ++n) dq[n] = mfma32(fb[n], d1, dq[n]);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (slot >= 0) {
    // ---- chunk of a cut tile: publish the partial dQ^T (accumulator order,
    //      element 16 n + a of thread tid at [16 n + a][tid]), take an
    //      arrival ticket; the last chunk to arrive adds every partial of the
    //      tile in slot order (its own read back like the others)
    const int s0 = p.dq_merges[3 * mrg + 1];
    const int ns = p.dq_merges[3 * mrg + 2];
    auto part = [&](int sl) __attribute__((always_inline)) {
      return p.dq_part + (((int64_t)sl * p.B + b) * p.Hq + h) * BR * D + tid;
    };
    {
      float* po = part(slot);
#pragma unroll
      for (int n = 0; n < NTD; ++n)
#pragma unroll
        for (int a = 0; a < 16; ++a) store_coherent(po + (16 * n + a) * NT, dq[n][a]);
    }
    wait_stores_done();
    __syncthreads();  // every wave's partial has completed
    if (tid == 0) sm.ticket = atomicAdd(p.dq_arrive + ((int64_t)mrg * p.B + b) * p.Hq + h, 1);
    __syncthreads();
    if (sm.ticket != ns - 1) return;  // a later chunk adds them up
#pragma unroll
    for (int n = 0; n < NTD; ++n) dq[n] = f32x16{};
    for (int sl = s0; sl < s0 + ns; ++sl) {
      const float* po = part(sl);
#pragma unroll
      for (int n = 0; n < NTD; ++n) {
        float t[16];  // loaded together, then added
#pragma unroll
        for (int a = 0; a < 16; ++a) t[a] = load_coherent(po + (16 * n + a) * NT);
#pragma unroll
        for (int a = 0; a < 16; ++a) dq[n][a] += t[a];
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

// Zero n words (the chunk arrival counters of the schedules).
template <int D, bool CAUSAL>
hipError_t launch(const BwdParams& p, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.Hq * p.Nq;
  const int64_t dot_blocks = (rows * (D / 8) + NT - 1) / NT;
  hipLaunchKernelGGL((bwd_dot_kernel<D>), dim3((unsigned)dot_blocks), dim3(NT), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int NB = kDkdvBlocks<D>;
  const int64_t kv_units = p.kv_items ? p.kv_n_items : (p.Tc + NB - 1) / NB;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)p.B * p.Hkv * kv_units)), dim3(256 * NB),
                     0, s, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t dq_units = p.dq_items ? p.dq_n_items : p.Tr;
  hipLaunchKernelGGL((bwd_dq_db_kernel<D, CAUSAL>), dim3((unsigned)((int64_t)p.B * p.Hq * dq_units)), dim3(NT), 0, s,
                     p);
  return hipGetLastError();
}

}  // namespace

int launch_prefill_bwd(const BwdParams& p, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p.d == 64) return p.causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
  return p.causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
}

}  // namespace bsattn
