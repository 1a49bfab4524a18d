// Device helpers for the gfx950 (CDNA4) kernels of libbsattn.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace bsattn {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef float f32x8 __attribute__((__vector_size__(8 * sizeof(float))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kPosInf = __builtin_huge_valf();

// v_exp_f32: 2^x (flushes results below the float range to 0; 2^-inf = 0).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 32x32x16 bf16 MFMA.  Lane l holds A[m = l%32][k = 8*(l/32) + i] and
// B[k = 8*(l/32) + i][n = l%32], i = 0..7; accumulator element a of lane l is
// D[m = 8*(a/4) + 4*(l/32) + a%4][n = l%32].  (Checked on the device.)
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA.  Lane l holds A[m = l%16][k = 8*(l/16) + i] and
// B[k = 8*(l/16) + i][n = l%16]; accumulator element a of lane l is
// D[m = 4*(l/16) + a][n = l%16].  (Checked on the device.)
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16 (issued from inline asm by the kernels): within each
// group of 16 lanes, lane j receives, in slot s (0..3), the 16-bit element
// j%4 of the 8 bytes addressed by lane 4*s + j/4 of the same group.
// (Checked on the device.)  Two such reads, of keys r and r + 8, joined
// below, give one 8-element MFMA operand.
__device__ __forceinline__ bf16x8 join_bf16x4(i16x4 lo, i16x4 hi) {
  union {
    i16x4 h[2];
    bf16x8 v;
  } u;
  u.h[0] = lo;
  u.h[1] = hi;
  return u.v;
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float* x) {
  f32x8 v = {x[0], x[1], x[2], x[3], x[4], x[5], x[6], x[7]};
  return __builtin_convertvector(v, bf16x8);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// Data handed between work-groups of one launch (which may sit on different
// XCDs, each with its own L2) goes through device-coherent relaxed atomics:
// no L2 write-back / invalidate, which an acquire-release pair would cost.
// Protocol: the writer stores its values with store_coherent, waits until
// they completed (wait_stores_done: on gfx9 vmcnt also counts stores), then
// signals with an atomic; a reader that has seen the signal reads the values
// with load_coherent.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<unsigned*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent(int32_t* p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_coherent(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const unsigned*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}

__device__ __forceinline__ int32_t load_coherent(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void wait_stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// max(x of lane l, x of lane l ^ 32) in registers: v_permlane32_swap with the
// same value in both operands returns, in every lane l, x of lane l % 32
// (first result) and x of lane l % 32 + 32 (second).  (Checked on the device.)
__device__ __forceinline__ float wave_max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

}  // namespace bsattn
