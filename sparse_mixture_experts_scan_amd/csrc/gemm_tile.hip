// Grouped expert GEMMs, LDS-tiled form (many token rows per expert), bf16.
//
// "Mistral/Mixtralのアーキテクチャ", section "各エキスパートの構造":
//   E_i(x) = W2 (SiLU(W1 x) * W3 x).
// Gate/up: H[r][f] = SiLU(sum_c W_gate[e][f][c] Xs[r][c]) * sum_c W_up[e][f][c] Xs[r][c]
// Down:    Y[r][o] = sum_f W_down[e][o][f] H[r][f]   (fp32 out)
//
// Tile: 256 weight rows x 256 token rows per workgroup of 8 waves (two per
// SIMD, so one wave's MFMAs cover the other's LDS and barrier stalls), each
// wave 128 weight rows x 64 token rows in eight 32x32 fp32 accumulators fed
// by v_mfma_f32_32x32x16_bf16 (A = weight rows, B = token rows, both
// K-contiguous).  For gate/up the 256 weight rows are 128 gate rows and the
// same 128 up rows, and each wave holds gate and up accumulators of the same
// features, so SiLU(gate) * up is applied in registers and only H is stored.
//
// K is staged 64 at a time through a ring of LDS stage buffers filled by
// gfx950 buffer loads straight to LDS (no VGPR staging): each lane fetches the
// 16 bytes that belong at its slot of the XOR-swizzled layout, the next stage
// is issued right after the barrier that opens the current one, and each
// wave waits for its own loads before that barrier.  LDS rows are 128 bytes;
// chunk c of row r sits at c ^ ((r ^ r >> 3) & 7), so the 32 rows an MFMA
// fragment reads fall in distinct banks (no bank conflicts measured).
//
// Token rows past the expert's count lie outside the token operand's buffer
// range, so the hardware loads zeros; 32-row token fragments entirely past it
// skip their MFMAs.  Work-group ids are remapped so that the tiles an XCD
// runs together share weight and token panels in its L2.

#include <algorithm>
#include <cmath>

#include "common.h"
#include "launch.h"

namespace moe {

#ifndef MOE_TILE_WAVES
#define MOE_TILE_WAVES 8
#endif
constexpr int kTileWaves = MOE_TILE_WAVES;          // 4 (1 per SIMD) or 8 (2 per SIMD)
constexpr int kTileThreads = 64 * kTileWaves;
constexpr int kWaveTok = 256 / (kTileWaves / 2);    // token rows per wave (128 or 64)
constexpr int kBFrags = kWaveTok / 32;              // 32-row token fragments per wave
constexpr int kTileBT = kTileTokens;  // token rows per tile (= padding unit)
constexpr int kTileRows = 256;        // weight rows per tile
#ifndef MOE_TILE_BK
#define MOE_TILE_BK 64
#endif
#ifndef MOE_TILE_NS
#define MOE_TILE_NS 2
#endif
constexpr int kTileBK = MOE_TILE_BK;  // K per LDS stage
constexpr int kTileNS = MOE_TILE_NS;  // LDS ring depth (stages)
constexpr int kXcds = 8;
#ifndef MOE_TILE_PERSISTENT
#define MOE_TILE_PERSISTENT 0
#endif
#ifndef MOE_TILE_FEAT_GROUP
#define MOE_TILE_FEAT_GROUP 4
#endif
constexpr int kFeatGroup = MOE_TILE_FEAT_GROUP;  // feature tiles per XCD-local group

constexpr int kRowBytes = kTileBK * 2;              // LDS bytes per tile row
constexpr int kChunks = kRowBytes / 16;             // 16-byte chunks per row
constexpr int kOperBytes = 256 * kRowBytes;         // one operand tile in LDS
constexpr int kStageBytes = 2 * kOperBytes;         // A + B
constexpr int kDmaPerWave = 256 * kChunks / 64 / kTileWaves;  // 1 KiB DMA loads per wave per operand
constexpr int kKSteps = kTileBK / 16;               // 32x32x16 MFMA k-steps per stage
static_assert(kTileBK == 32 || kTileBK == 64, "stage K must be 32 or 64");
static_assert(kTileNS >= 2 && kTileNS <= 4, "ring depth 2..4");
static_assert(kTileNS * kStageBytes <= 160 * 1024, "LDS ring exceeds 160 KiB");

// XOR swizzle of the 16-byte chunks of LDS row r: the 32 rows an MFMA fragment
// reads (and the rows a DMA fills) fall in distinct banks.
__device__ inline int swz_key(int r) {
  return kChunks == 8 ? ((r ^ (r >> 3)) & 7) : (((r >> 1) ^ (r >> 3)) & 3);
}
__device__ inline int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ swz_key(row)) << 4);
}

__device__ inline f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

typedef __attribute__((address_space(3))) void lds_void;
constexpr int kBufferCfg = 0x00020000;  // raw buffer, 32-bit data format

// Buffer resources must live in scalar registers: the fields are made provably
// wave-uniform, otherwise each load is wrapped in a per-lane loop.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)n, kBufferCfg);
}

// Wait until at most N of this wave's vector-memory operations (here: LDS DMA
// loads) are outstanding; lgkm/exp counters untouched.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// All of this wave's LDS reads done, then the workgroup barrier.  No memory
// fence: LDS DMA completion is waited for explicitly with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct TileCtx {
  __amdgpu_buffer_rsrc_t rA, rB;   // this wave's A resource (gate or up half), B
  uint32_t voffA[kDmaPerWave], voffB[kDmaPerWave];
  int dma_base;                    // this wave's first DMA slot (1 KiB units)
  uint32_t k_byte0;                // byte offset of this part's first K column
  int arow[4];
  int brow;                        // first token row of this wave inside the tile
};

// Issue stage ks's DMA loads into stage buffer `buf`: each lane fetches the
// global 16 bytes that belong at LDS slot (dma_base + j) * 64 + lane.
__device__ __forceinline__ void tile_issue(const TileCtx& c, char* buf, int ks) {
  const uint32_t so = c.k_byte0 + (uint32_t)ks * kTileBK * 2;
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        c.rA, (lds_void*)(buf + (c.dma_base + j) * 1024), 16, c.voffA[j], so, 0, 0);
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        c.rB, (lds_void*)(buf + kOperBytes + (c.dma_base + j) * 1024), 16, c.voffB[j], so, 0, 0);
}

template <int NBV>
__device__ __forceinline__ void tile_frags(const TileCtx& c, const char* buf, int kk, int lane,
                                           uint4 (&af)[4], uint4 (&bf)[kBFrags]) {
  const char* A = buf;
  const char* B = buf + kOperBytes;
  const int r32 = lane & 31, chunk = kk * 2 + (lane >> 5);
#pragma unroll
  for (int a = 0; a < 4; ++a) af[a] = *reinterpret_cast<const uint4*>(A + swz(c.arow[a] + r32, chunk));
#pragma unroll
  for (int b = 0; b < NBV; ++b)
    bf[b] = *reinterpret_cast<const uint4*>(B + swz(c.brow + b * 32 + r32, chunk));
}

// Scheduling masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

#ifndef MOE_TILE_PRELOAD
#define MOE_TILE_PRELOAD 0
#endif

template <int NBV>
__device__ __forceinline__ void tile_compute(const TileCtx& c, const char* buf, int lane,
                                             f32x16 (&acc)[4][kBFrags]) {
#if MOE_TILE_PRELOAD
  // all of the stage's fragments first (LDS returns in order, so each
  // k-step's MFMAs wait only for their own reads), then the MFMAs
  uint4 fa[kKSteps][4], fb[kKSteps][kBFrags];
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) tile_frags<NBV>(c, buf, kk, lane, fa[kk], fb[kk]);
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk)
#pragma unroll
    for (int b = 0; b < NBV; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a][b] = mfma32(fa[kk][a], fb[kk][b], acc[a][b]);
  return;
#endif
  uint4 af[4], bf[kBFrags], na[4], nb[kBFrags];
  tile_frags<NBV>(c, buf, 0, lane, af, bf);
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) {
    if (kk + 1 < kKSteps) tile_frags<NBV>(c, buf, kk + 1, lane, na, nb);
#if MOE_TILE_SCHED
    __builtin_amdgcn_sched_barrier(0);
#endif
#pragma unroll
    for (int b = 0; b < NBV; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a][b] = mfma32(af[a], bf[b], acc[a][b]);
#ifndef MOE_TILE_SCHED
#define MOE_TILE_SCHED 0
#endif
#if MOE_TILE_SCHED
    // hard grouping: the next k-step's reads were issued before this
    // k-step's MFMAs and both fragment sets stay live
    __builtin_amdgcn_sched_barrier(0);
    if (false) {
#else
    // order: the next k-step's fragment reads one per MFMA, then the rest
    // of the MFMAs, so the reads overlap this k-step's matrix work
    if (kk + 1 < kKSteps) {
#endif
      constexpr int nr = 4 + NBV, nm = 4 * NBV;
      constexpr int pairs = nr < nm ? nr : nm;
#pragma unroll
      for (int i = 0; i < pairs; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      if (nm > pairs) __builtin_amdgcn_sched_group_barrier(kSchedMfma, nm - pairs, 0);
      if (nr > pairs) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, nr - pairs, 0);
    }
    if (kk + 1 < kKSteps) {
#pragma unroll
      for (int a = 0; a < 4; ++a) af[a] = na[a];
#pragma unroll
      for (int b = 0; b < kBFrags; ++b) bf[b] = nb[b];
    }
  }
}

// Wait for stage ks's loads: the loads of the n_after stages issued after it
// may stay in flight.
__device__ __forceinline__ void wait_stage(int n_after) {
  constexpr int per_stage = 2 * kDmaPerWave;
  if (n_after >= 2) wait_vmcnt<2 * per_stage>();
  else if (n_after == 1) wait_vmcnt<per_stage>();
  else wait_vmcnt<0>();
}

// Main loop over K.  Ring of kTileNS stage buffers: stage ks lives in buffer
// ks % NS; after the barrier that opens stage ks (all waves have finished
// stage ks - 1), the loads of stage ks + NS - 1 are issued into the buffer
// stage ks - 1 used, so loads run NS - 1 stages ahead of the MFMAs.
// nk is a multiple of kTileNS (checked on the host), so every pass of the
// outer loop runs all kTileNS stages: no early exit inside the unrolled body.
template <int NBV>
__device__ __forceinline__ void tile_main_loop(const TileCtx& c, char* const (&bufs)[kTileNS],
                                               int nk, int lane, f32x16 (&acc)[4][kBFrags]) {
#pragma unroll
  for (int s = 0; s < kTileNS - 1; ++s) tile_issue(c, bufs[s], s);
  for (int ks0 = 0; ks0 < nk; ks0 += kTileNS) {
    const bool last = ks0 + kTileNS >= nk;
#pragma unroll
    for (int u = 0; u < kTileNS; ++u) {
      const int ks = ks0 + u;
      // stages issued after ks: NS - 2 in steady state; in the last pass the
      // loads stop at stage nk - 1 (issued at u = 0)
      wait_stage(last ? min(kTileNS - 2, kTileNS - 1 - u) : kTileNS - 2);
      lds_barrier();
      // keep the DMA issue right after the barrier: the scheduler would
      // otherwise sink it behind the MFMAs and shrink the prefetch distance
      __builtin_amdgcn_sched_barrier(0);
      if (!last || u == 0) tile_issue(c, bufs[(u + kTileNS - 1) % kTileNS], ks + kTileNS - 1);
      __builtin_amdgcn_sched_barrier(0);
      tile_compute<NBV>(c, bufs[u], lane, acc);
    }
  }
}

#ifdef MOE_TILE_WPE
#define MOE_TILE_WPE_ATTR __attribute__((amdgpu_waves_per_eu(MOE_TILE_WPE, MOE_TILE_WPE)))
#else
#define MOE_TILE_WPE_ATTR
#endif

template <bool GATEUP>
__global__ __launch_bounds__(kTileThreads, 1) MOE_TILE_WPE_ATTR void tile_gemm_kernel(
    const bf16_t* __restrict__ act, const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ num_tiles,
    const int32_t* __restrict__ tile_expert, int N, int K, int n_ft, int n_tt, int per_xcd,
    int parts, size_t part_stride) {
  // one __shared__ array per ring stage, so that the compiler can tell which
  // DMA each LDS read depends on
  __shared__ __attribute__((aligned(1024))) char st0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) char st1[kStageBytes];
#if MOE_TILE_NS > 2
  __shared__ __attribute__((aligned(1024))) char st2[kStageBytes];
#endif
#if MOE_TILE_NS > 3
  __shared__ __attribute__((aligned(1024))) char st3[kStageBytes];
#endif
  char* const bufs[kTileNS] = {st0, st1
#if MOE_TILE_NS > 2
                               , st2
#endif
#if MOE_TILE_NS > 3
                               , st3
#endif
  };
  constexpr int FB = GATEUP ? kTileRows / 2 : kTileRows;  // output features per tile

  // ---- tile id: XCD-contiguous remap, then groups of kFeatGroup feature tiles
#if MOE_TILE_PERSISTENT
  // persistent: workgroup j of XCD x walks positions j, j + W, ... of that
  // XCD's contiguous range, W = workgroups per XCD, so the W tiles an XCD runs
  // together are W consecutive positions (shared panels) and stay in step
  const int xcd = blockIdx.x % kXcds;
  const int wg_per_xcd = gridDim.x / kXcds;
  for (int pos = blockIdx.x / kXcds; pos < per_xcd; pos += wg_per_xcd) {
  int Lp = xcd * per_xcd + pos;
  if (Lp >= parts * n_ft * n_tt) break;
#else
  do {                                      // one tile; `continue` leaves
  const int L = blockIdx.x;
  int Lp = (L % kXcds) * per_xcd + L / kXcds;
  if (Lp >= parts * n_ft * n_tt) return;
#endif
  const int part = Lp / (n_ft * n_tt);      // K-split part (slowest)
  Lp -= part * n_ft * n_tt;
  const int grp = Lp / (kFeatGroup * n_tt);
  const int rem = Lp - grp * kFeatGroup * n_tt;
  const int gsize = min(kFeatGroup, n_ft - grp * kFeatGroup);
  const int tt = rem / gsize;
  const int ft = grp * kFeatGroup + rem % gsize;
  if (tt >= *num_tiles) continue;          // past the token tiles in use
  const int e = tile_expert[tt];
  const int row0 = tt * kTileBT;
  const int valid_end = offsets[e] + counts[e];
  const int f0 = ft * FB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wf = wave & 1, wt = wave >> 1;   // weight half, token slice

  // ---- DMA assignment: wave w fills LDS slots [w * kDmaPerWave, +kDmaPerWave)
  // of each operand (1 KiB each); slot q's lane i holds LDS chunk position
  // p = q * 64 + i = row * kChunks + swizzled chunk.
  TileCtx c;
  c.dma_base = wave * kDmaPerWave;
  const int Kp = K / parts;                 // K columns of this part
  c.k_byte0 = (uint32_t)(part * Kp) * 2;
  const uint32_t row_bytes = (uint32_t)K * 2;
#pragma unroll
  for (int j = 0; j < kDmaPerWave; ++j) {
    const int p = (c.dma_base + j) * 64 + lane;
    const int r = p / kChunks, cs = p % kChunks;
    const int cg = cs ^ swz_key(r);                         // global chunk stored there
    const int ra = GATEUP ? (r & (kTileRows / 2 - 1)) : r;  // row inside A's resource
    c.voffA[j] = (uint32_t)ra * row_bytes + cg * 16;
    c.voffB[j] = (uint32_t)r * row_bytes + cg * 16;
  }
  if constexpr (GATEUP) {
    // the first half of the waves fills A rows 0..127 (gate), the second
    // half rows 128..255 (up)
    const bf16_t* Wsrc = (wave < kTileWaves / 2 ? W0 : W1) + ((size_t)e * N + f0) * K;
    c.rA = make_rsrc(Wsrc, 128 * row_bytes);
  } else {
    c.rA = make_rsrc(W0 + ((size_t)e * N + f0) * K, 256 * row_bytes);
  }
  // token rows past the expert's count fall outside the resource: read as 0
  const int nvalid = max(0, min(kTileBT, valid_end - row0));
  c.rB = make_rsrc(act + (size_t)row0 * K, (uint32_t)nvalid * row_bytes);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    if constexpr (GATEUP) c.arow[a] = (a < 2 ? 0 : 128) + wf * 64 + (a & 1) * 32;
    else c.arow[a] = wf * 128 + a * 32;
  }
  c.brow = wt * kWaveTok;
  const int nbv = max(0, min(kBFrags, (valid_end - (row0 + wt * kWaveTok) + 31) / 32));

  f32x16 acc[4][kBFrags];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < kBFrags; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.f;

  // wave-uniform choice; every variant runs the same loads and barriers
  const int nk = Kp / kTileBK;
  switch (nbv) {
#if MOE_TILE_WAVES == 4
    case 4: tile_main_loop<4>(c, bufs, nk, lane, acc); break;
    case 3: tile_main_loop<3>(c, bufs, nk, lane, acc); break;
#endif
    case 2: tile_main_loop<2>(c, bufs, nk, lane, acc); break;
    case 1: tile_main_loop<1>(c, bufs, nk, lane, acc); break;
    default: tile_main_loop<0>(c, bufs, nk, lane, acc); break;
  }

  // ---- epilogue.  D of a 32x32 MFMA: lane holds column n = lane % 32 and rows
  // 8 * (j / 4) + 4 * (lane / 32) + j % 4, j = 0..15: four consecutive
  // features.  Skipped fragments hold zeros (padding rows).
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int b = 0; b < kBFrags; ++b) {
    const size_t row = (size_t)(row0 + wt * kWaveTok + b * 32 + r32);
    if constexpr (GATEUP) {
      bf16_t* h = reinterpret_cast<bf16_t*>(outp) + row * N;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int feat = f0 + wf * 64 + a * 32 + jj * 8 + half * 4;
          uint32_t p[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float g0 = acc[a][b][jj * 4 + 2 * q], u0 = acc[a + 2][b][jj * 4 + 2 * q];
            const float g1 = acc[a][b][jj * 4 + 2 * q + 1], u1 = acc[a + 2][b][jj * 4 + 2 * q + 1];
            p[q] = (uint32_t)Elem<bf16_t>::from_f32(silu_f32(g0) * u0) |
                   ((uint32_t)Elem<bf16_t>::from_f32(silu_f32(g1) * u1) << 16);
          }
          *reinterpret_cast<uint2*>(h + feat) = make_uint2(p[0], p[1]);
        }
    } else {
      float* y = reinterpret_cast<float*>(outp) + part * part_stride + row * N;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int feat = f0 + wf * 128 + a * 32 + jj * 8 + half * 4;
          *reinterpret_cast<float4*>(y + feat) =
              make_float4(acc[a][b][jj * 4], acc[a][b][jj * 4 + 1], acc[a][b][jj * 4 + 2],
                          acc[a][b][jj * 4 + 3]);
        }
    }
  }
#if MOE_TILE_PERSISTENT
  }  // tile loop
#else
  } while (0);
#endif
}

template <bool GATEUP>
static void tile_launch(const Dims& D, const void* act, const void* W0, const void* W1,
                        void* out, const int32_t* counts, const int32_t* offsets,
                        const int32_t* num_tiles, const int32_t* tile_expert, hipStream_t s) {
  const int N = GATEUP ? D.f : D.d;
  const int K = GATEUP ? D.d : D.f;
  const int FB = GATEUP ? kTileRows / 2 : kTileRows;
  const int n_ft = N / FB;
  const int n_tt = D.max_tiles;
  const int parts = GATEUP ? 1 : D.down_splits;
  const int total = parts * n_ft * n_tt;
  const int per_xcd = (total + kXcds - 1) / kXcds;
#if MOE_TILE_PERSISTENT
  // one workgroup per CU (the LDS ring allows one), at most one per position
  static int n_cu = 0;
  if (n_cu == 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      n_cu = 256;
  }
  const int wg_per_xcd = std::max(1, std::min(per_xcd, n_cu / kXcds));
  const int grid = wg_per_xcd * kXcds;
#else
  const int grid = per_xcd * kXcds;
#endif
  tile_gemm_kernel<GATEUP><<<grid, kTileThreads, 0, s>>>(
      (const bf16_t*)act, (const bf16_t*)W0, (const bf16_t*)W1, out, counts, offsets, num_tiles,
      tile_expert, N, K, n_ft, n_tt, per_xcd, parts, (size_t)D.max_rows * N);
}

bool tile_shape_ok(const Dims& D) {
  // buffer offsets are 32-bit: 256 rows of either K must stay below 2 GiB
  const int64_t kmax = D.d > D.f ? D.d : D.f;
  return D.bf16 && D.BT == kTileBT && D.f % (kTileRows / 2) == 0 && D.d % kTileRows == 0 &&
         D.d % (kTileBK * kTileNS) == 0 && D.f % (kTileBK * kTileNS) == 0 &&
         kTileRows * kmax * 2 < (int64_t(1) << 31);
}

// K-splits of the down GEMM: the expected tile count (ceil(rows / BT) plus
// about half a tile of padding per expert) is spread over the CUs; a split
// that fills the last round of workgroups markedly better is taken.
int tile_down_splits(const Dims& D) {
  constexpr int kCus = 256;
  const int n_ft = D.d / kTileRows;
  const double tiles = n_ft * ((double)D.T * D.k / kTileBT + D.E * 0.5);
  auto fill = [&](int sp) {
    const double t = tiles * sp;
    return t / (std::ceil(t / kCus) * kCus);
  };
  const bool can2 = D.f % (2 * kTileBK * kTileNS) == 0;
  return (can2 && fill(1) < 0.9 && fill(2) > fill(1) + 0.05) ? 2 : 1;
}

void launch_gateup_tile(const Dims& D, const void* xs, const void* Wg, const void* Wu, void* h,
                        const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                        const int32_t* tile_expert, hipStream_t s) {
  tile_launch<true>(D, xs, Wg, Wu, h, counts, offsets, num_tiles, tile_expert, s);
}

void launch_down_tile(const Dims& D, const void* h, const void* Wd, float* y,
                      const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                      const int32_t* tile_expert, hipStream_t s) {
  tile_launch<false>(D, h, Wd, nullptr, y, counts, offsets, num_tiles, tile_expert, s);
}

}  // namespace moe
