// mfma_util.h -- device helpers shared by the gfx950 matrix-core kernels:
// operand types, the 32x32x16 MFMA wrappers, buffer resources, explicit
// vector-memory waits and cross-lane reductions.
//
// MFMA 32x32x16 lane layout (checked on the device): A[m][k] comes from lane
// m + 32*(k/8), element k%8; B[k][n] from lane n + 32*(k/8), element k%8;
// C[m][n] lands in lane n + 32*((m/4)%2), register 4*(m/8) + m%4.
#pragma once

#include <hip/hip_ext.h>

#include "mha_internal.h"

namespace mha {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr uint32_t kBufferWord3 = 0x00020000u;  // raw buffer, 32-bit data format (gfx9)
constexpr float kLog2e = 1.4426950408889634f;

#define MHA_LDS(p) ((__attribute__((address_space(3))) void*)(p))

// kGuard: the largest partial softmax sum a query may reach before its
// reference maximum is raised -- far inside the range of the P type.
struct BF16 {
  static constexpr float kGuard = 18446744073709551616.0f;  // 2^64
  __device__ static f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack(float x, float y) {  // round to nearest even
    bf16x2_t r = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static float to_float(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
  __device__ static float sum2(uint32_t packed, float acc) {  // acc + lo + hi of a packed pair
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, packed), bf16x2_t{(__bf16)1.0f, (__bf16)1.0f},
                                           acc, false);
  }
};

struct F16 {
  static constexpr float kGuard = 32768.0f;  // 2^15
  __device__ static f32x16_t mma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static uint32_t pack(float x, float y) {
    f16x2_t r = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static float to_float(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
  __device__ static float sum2(uint32_t packed, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, packed), f16x2_t{(_Float16)1.0f, (_Float16)1.0f}, acc,
                                  false);
  }
};

// Buffer resource over `bytes` bytes from `base` (clamped to the 32-bit range
// check); loads at or beyond `bytes` return zeros and touch no memory.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, (int)kBufferWord3);
}

// s_waitcnt with the vector-memory count set to N and the other counters left
// unconstrained (gfx9 encoding: vmcnt in bits 3:0 and 15:14).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt out of range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Barrier without the memory fence of __syncthreads (whose release semantics
// would wait for every load in flight, including later pipeline stages); the
// empty asm statements keep the compiler from moving LDS accesses across it.
__device__ inline void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ inline float lanes_max(float x) {  // max over lanes l and l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float lanes_sum(float x) {  // sum over lanes l and l^32
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float wave_max(float x) {  // max over the 64 lanes
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ inline float wave_sum(float x) {  // sum over the 64 lanes
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Swizzle of 16-byte chunks within 128-byte LDS rows for MFMA operand reads
// (16 bytes per lane from 32 consecutive rows): chunk c of row r sits in slot
// c ^ operand_swizzle(r), which spreads the 32 rows over all banks.
__device__ inline int operand_swizzle(int row) { return (row & 7) ^ ((row >> 3) & 1); }

}  // namespace
}  // namespace mha
