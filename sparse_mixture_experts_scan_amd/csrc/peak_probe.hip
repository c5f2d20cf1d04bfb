// Microbenchmarks of what one MI355X reaches on the two resources that bound
// the MoE layer: HBM streaming (the decode shapes read every touched expert's
// weights once) and bf16 MFMA issue (the prefill shapes).  They give measured
// ceilings to set beside the datasheet peaks; they are not part of the layer.
//
//  - read:  every lane streams 16-byte loads over a buffer far larger than
//           the 256 MB last-level cache, four loads in flight per lane, and
//           folds them into one word per block (so nothing is optimised away).
//  - copy:  the same loads, each stored to a second buffer.
//  - mfma:  each wave issues v_mfma_f32_32x32x16_bf16 back to back on eight
//           independent accumulators with operands held in registers, two
//           waves per SIMD (the occupancy of the tiled GEMMs).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src,
                                                        size_t n16, uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[kThreads];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] ^= red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

constexpr int kMfmaWaves = 8;   // two per SIMD
constexpr int kMfmaAcc = 8;     // independent accumulators per wave

__global__ __launch_bounds__(64 * kMfmaWaves) void mfma_kernel(int iters, float* __restrict__ sink) {
  const uint32_t lane = threadIdx.x;
  // operands that differ per lane and per accumulator (bf16 values in [1, 2))
  uint4 a[kMfmaAcc], b;
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j) {
    const uint32_t v = 0x3f803f80u | ((lane * 2654435761u + j * 40503u) & 0x007f007fu);
    a[j] = make_uint4(v, v ^ 0x00150015u, v ^ 0x002a002au, v ^ 0x00330033u);
  }
  {
    const uint32_t v = 0x3f803f80u | ((lane * 40503u) & 0x007f007fu);
    b = make_uint4(v, v ^ 0x00110011u, v ^ 0x00220022u, v ^ 0x00440044u);
  }
  f32x16 acc[kMfmaAcc];
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaAcc; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[j]),
                                                       __builtin_bit_cast(bf16x8, b), acc[j],
                                                       0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kMfmaAcc; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  if (lane % 64 == 0) sink[blockIdx.x * kMfmaWaves + threadIdx.x / 64] = s;
}

int launch_status() {
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // namespace

extern "C" {

int moe_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!src || !sink || bytes % 16 || blocks < 1 || reinterpret_cast<uintptr_t>(src) % 16) return 1;
  read_kernel<<<blocks, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const u32x4*>(src), bytes / 16, sink);
  return launch_status();
}

int moe_probe_copy(const void* src, void* dst, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || bytes % 16 || blocks < 1 || reinterpret_cast<uintptr_t>(src) % 16 ||
      reinterpret_cast<uintptr_t>(dst) % 16)
    return 1;
  copy_kernel<<<blocks, kThreads, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst), bytes / 16);
  return launch_status();
}

int moe_probe_mfma(float* sink, int blocks, int iters, void* stream) {
  if (!sink || blocks < 1 || iters < 1) return 1;
  mfma_kernel<<<blocks, 64 * kMfmaWaves, 0, reinterpret_cast<hipStream_t>(stream)>>>(iters, sink);
  return launch_status();
}

double moe_probe_mfma_flops(int blocks, int iters) {
  // 2 * 32 * 32 * 16 flops per MFMA
  return 2.0 * 32 * 32 * 16 * (double)kMfmaAcc * iters * kMfmaWaves * blocks;
}

}  // extern "C"
