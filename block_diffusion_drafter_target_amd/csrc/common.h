// Device-side helpers shared by the gfx950 kernels: bf16 bit handling, the
// 16x16x32 bf16 MFMA, wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfl {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// Native vectors (not HIP's struct uint4/uint2): copies stay in registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf2f(bf16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

// Two fp32 -> packed bf16 pair (lo in the low half), round to nearest even, by
// gfx950's packed conversion instruction.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t{lo, hi}), bf2_t));
}

// 2^x by the hardware exponential (no denormal range fix-up: results below
// 2^-126 may flush to zero, which the softmax weights tolerate).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).
// Operand layout: lane l supplies row (A) / column (B) l%16 and the eight
// k-elements 8*(l/16) .. 8*(l/16)+7. Result: lane l holds column l%16, rows
// 4*(l/16) .. 4*(l/16)+3. Any permutation of k applied to both operands leaves
// the product unchanged.
__device__ __forceinline__ f32x4_t mfma16x16x32(u32x4 a, u32x4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Sum over a 256-thread workgroup; every thread gets the result.
__device__ __forceinline__ float block_sum_256(float v, float* smem4) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) smem4[wave] = v;
  __syncthreads();
  return smem4[0] + smem4[1] + smem4[2] + smem4[3];
}

// Monotone map of fp32 to uint32 (larger float -> larger key), finite inputs.
__device__ __forceinline__ uint32_t orderable(float v) {
  uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit argmax key: the maximum key is the largest value and, among equal
// values, the lowest index.
__device__ __forceinline__ unsigned long long argmax_key(float v, int idx) {
  return ((unsigned long long)orderable(v) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)idx);
}

// --- direct global -> LDS loads (global_load_lds_dwordx4) -------------------
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with vmcnt(N) only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0) only.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier for LDS data published by direct loads. The barrier
// intrinsic alone does not order memory accesses in the compiler, so LDS
// reads could be hoisted above it; the empty asm with a memory clobber keeps
// every memory access on its side, and the scheduling barriers keep the
// machine scheduler from moving instructions across. No s_waitcnt comes with
// it: each wave waits for its own direct loads (vmcnt) before calling it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace dfl
