// Device-side types and helpers shared by the MoE kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_ffn.h"
#include "plan.h"

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint16_t bf16_t;  // storage type of bfloat16 data

constexpr int kWave = 64;
constexpr int kRouterThreads = 256;

// Element-type traits: how a 16-byte chunk of K is fed to 16x16 MFMA.
// bf16: one chunk = 8 elements = one v_mfma_f32_16x16x32_bf16 k-group.
// f32:  one chunk = 4 elements = four v_mfma_f32_16x16x4_f32, element i of the
//       chunk feeding the i-th instruction.  A and B use the same mapping, so
//       every k is paired with itself exactly once.
// Two floats rounded to nearest-even bf16 in one conversion (lo in the low
// half); the same rounding as a scalar conversion of each.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;  // elements per 16-byte chunk
  __device__ static inline float to_f32(bf16_t v) {
    return __uint_as_float(static_cast<uint32_t>(v) << 16);
  }
  __device__ static inline bf16_t from_f32(float f) {
    __bf16 b = static_cast<__bf16>(f);  // round to nearest even
    return __builtin_bit_cast(bf16_t, b);
  }
  __device__ static inline f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  __device__ static inline float to_f32(float v) { return v; }
  __device__ static inline float from_f32(float f) { return f; }
  __device__ static inline f32x4 mfma16(uint4 a, uint4 b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

__device__ inline float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// ---- buffer loads and the waits around them (gfx950)
typedef __attribute__((address_space(3))) void lds_void;
constexpr int kBufferCfg = 0x00020000;  // raw buffer, 32-bit data format

// A raw buffer resource of `bytes` bytes from `base`: loads past the range
// return zeros.  Resources must sit in scalar registers, so every field is
// made provably wave-uniform; otherwise each load is wrapped in a per-lane
// loop.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)n, kBufferCfg);
}

// Wait until at most N of this wave's vector-memory operations (loads, LDS
// DMA loads) are outstanding; the LDS and export counters are left alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// All of this wave's LDS operations done, then the workgroup barrier.  No
// memory fence: unlike __syncthreads it does not wait for global stores, and
// LDS DMA completion is waited for explicitly with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ inline uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ inline void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

}  // namespace moe
