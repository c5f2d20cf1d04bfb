// Grouped expert GEMMs, weight-streaming form (few token rows per expert).
//
// "Mistral/Mixtralのアーキテクチャ", section "各エキスパートの構造":
//   E_i(x) = W2 (SiLU(W1 x) * W3 x), W1, W3: d_ff x d_model, W2: d_model x d_ff.
// Gate/up: H[r][f] = SiLU(sum_c W_gate[e][f][c] Xs[r][c]) * sum_c W_up[e][f][c] Xs[r][c]
// Down:    Y[r][o] = sum_f W_down[e][o][f] H[r][f]   (fp32 out)
// for every permuted row r of expert e's segment.
//
// Shape of the work: with a handful of rows per expert the weights are read
// exactly once and nothing is reused.  Two kernels.  bf16 with K a multiple
// of 128 (stream_dma_kernel, further down) stages each wave's weight runs
// through LDS so that every load instruction fetches whole 256-byte pieces of
// rows.  Otherwise (fp32, or K = 64 mod 128) stream_gemm_kernel goes
// straight from HBM to registers: the MFMA A operand is 16 weight rows
// (output features), the B operand 16 token rows, both K-contiguous, 16 bytes
// per lane per raw buffer load (scalar resource, loop-invariant lane offsets,
// the K advance in the scalar offset).  A workgroup owns FT output features
// of one token tile; its 4 waves split K in interleaved runs of k-steps and
// keep the next batch of loads in flight while the current batch's MFMAs
// run.  The partial sums are added in fixed wave order through LDS
// (deterministic), then the epilogue (SiLU(gate)*up, or plain fp32) is
// applied and stored.
//
// Token rows past the expert's count (segment padding) read as zero, so the
// padding rows of H are exactly zero and every row stored is in bounds.
// The bf16 gate/up kernel can also take Xs[r] = x[row_token[r]] straight
// from x (the tokens read in place), which spares the scatter's copy.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kStreamThreads = 256;
// cache policy of the LDS-staged kernel's weight DMA (gfx950 bits: 1 sc0,
// 2 nt, 16 sc1), measured on MI355X at the Mixtral decode shape:
// non-temporal for the down GEMM (0.164 -> 0.150 ms); for gate/up on the up
// matrix only (0.329 -> 0.319 ms; on the gate matrix only 0.322, on both
// 0.338)
#ifndef MOE_WSTREAM_CPOL_GU
#define MOE_WSTREAM_CPOL_GU 0     // gate matrix (W1)
#endif
#ifndef MOE_WSTREAM_CPOL_GU1
#define MOE_WSTREAM_CPOL_GU1 2    // up matrix (W3)
#endif
#ifndef MOE_WSTREAM_CPOL_DN
#define MOE_WSTREAM_CPOL_DN 2
#endif
#ifndef MOE_STREAM_U
#define MOE_STREAM_U 8       // k-steps per run (per batch of loads)
#endif
#ifndef MOE_STREAM_FT_GU
#define MOE_STREAM_FT_GU 16
#endif
#ifndef MOE_STREAM_FT_DN
#define MOE_STREAM_FT_DN 32
#endif
// down GEMM output features per block of the LDS-staged kernel: 16 rows
// (4 KiB runs, four blocks per CU) balance the CUs better than 32 (3% on
// the Mixtral-shaped decode step) at the same bytes in flight per CU
#ifndef MOE_STREAM_DMA_FT_DN
#define MOE_STREAM_DMA_FT_DN 16
#endif


__device__ __forceinline__ uint4 sload(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// One batch = a run of U consecutive k-steps (16 bytes per lane each) of one
// wave; run r belongs to wave r % 4, so the 4 waves' runs interleave along K.
template <typename T, int BT, int FT, bool GATEUP, int U>
struct StreamBatch {
  static constexpr int VEC = Elem<T>::kVec;
  static constexpr int KSTEP = 4 * VEC;   // K covered by one 16-byte k-group set
  static constexpr int NF = FT / 16;      // 16-row weight fragments
  static constexpr int NT = BT / 16;      // 16-row token fragments
  static constexpr int NW = GATEUP ? 2 : 1;
  uint4 wv[NW][NF][U], av[NT][U];

  template <bool FULL>
  __device__ __forceinline__ void load(const __amdgpu_buffer_rsrc_t (&rw)[NW],
                                       __amdgpu_buffer_rsrc_t ra, const uint32_t (&wo)[NF],
                                       const uint32_t (&ao)[NT], int run, int valid) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (FULL || u < valid) {
        const uint32_t so = (uint32_t)(run * U + u) * KSTEP * sizeof(T);
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int f = 0; f < NF; ++f) wv[w][f][u] = sload(rw[w], wo[f], so);
#pragma unroll
        for (int n = 0; n < NT; ++n) av[n][u] = sload(ra, ao[n], so);
      }
    }
  }
  // the first batch: weights as soon as the expert is known, tokens once
  // their row range is
  __device__ __forceinline__ void load_w(const __amdgpu_buffer_rsrc_t (&rw)[NW],
                                         const uint32_t (&wo)[NF], int run) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t so = (uint32_t)(run * U + u) * KSTEP * sizeof(T);
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int f = 0; f < NF; ++f) wv[w][f][u] = sload(rw[w], wo[f], so);
    }
  }
  __device__ __forceinline__ void load_x(__amdgpu_buffer_rsrc_t ra, const uint32_t (&ao)[NT],
                                         int run) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t so = (uint32_t)(run * U + u) * KSTEP * sizeof(T);
#pragma unroll
      for (int n = 0; n < NT; ++n) av[n][u] = sload(ra, ao[n], so);
    }
  }
  template <bool FULL>
  __device__ __forceinline__ void compute(f32x4 (&acc)[NW][NF][NT], int valid) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (FULL || u < valid) {
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int n = 0; n < NT; ++n)
              acc[w][f][n] = Elem<T>::mfma16(wv[w][f][u], av[n][u], acc[w][f][n]);
      }
    }
  }
};

template <typename T, int BT, int FT, bool GATEUP, int U>
__global__ __launch_bounds__(kStreamThreads) void stream_gemm_kernel(
    const T* __restrict__ act, const T* __restrict__ W0, const T* __restrict__ W1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ num_tiles,
    const int32_t* __restrict__ tile_expert, int N, int K) {
  using SB = StreamBatch<T, BT, FT, GATEUP, U>;
  constexpr int NF = SB::NF, NT = SB::NT, NW = SB::NW, KSTEP = SB::KSTEP;
  constexpr int NWAVE = kStreamThreads / kWave;
  __shared__ f32x4 red[NWAVE - 1][NW * NF * NT][kWave];

  // Tiles past those in use have expert -1.  One dependent lookup (the
  // expert) stands between the launch and the first weight loads; the token
  // row range (offsets, counts) is needed only for the token loads.
  const int tile = blockIdx.y;
  const int e = tile_expert[tile];
  if (e < 0) return;
  const int row0 = tile * BT;
  const int f0 = blockIdx.x * FT;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  const int lr = lane & 15, kg = lane >> 4;

  const uint32_t row_bytes = (uint32_t)K * sizeof(T);
  __amdgpu_buffer_rsrc_t rw[NW];
  rw[0] = buffer_rsrc(W0 + ((size_t)e * N + f0) * K, FT * row_bytes);
  if constexpr (GATEUP) rw[1] = buffer_rsrc(W1 + ((size_t)e * N + f0) * K, FT * row_bytes);
  uint32_t wo[NF], ao[NT];
#pragma unroll
  for (int f = 0; f < NF; ++f) wo[f] = (uint32_t)(f * 16 + lr) * row_bytes + kg * 16;
#pragma unroll
  for (int n = 0; n < NT; ++n) ao[n] = (uint32_t)(n * 16 + lr) * row_bytes + kg * 16;

  f32x4 acc[NW][NF][NT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[w][f][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Full runs r < nruns; this wave owns runs wave, wave + 4, ...  Software
  // pipeline: run b + 1's loads are issued before run b's MFMAs.
  const int nks = K / KSTEP;
  const int nruns = nks / U, rem = nks % U;
  const int nb = nruns > wave ? (nruns - wave + NWAVE - 1) / NWAVE : 0;
  SB A, B;
  if (nb > 0) A.load_w(rw, wo, wave);
  // token rows past the expert's count fall outside the resource: read as 0
  const int valid_end = offsets[e] + counts[e];
  const int nvalid = max(0, min(BT, valid_end - row0));
  const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(act + (size_t)row0 * K, (uint32_t)nvalid * row_bytes);
  if (nb > 0) A.load_x(ra, ao, wave);
  for (int b = 0; b < nb; b += 2) {
    if (b + 1 < nb) B.template load<true>(rw, ra, wo, ao, wave + (b + 1) * NWAVE, U);
    A.template compute<true>(acc, U);
    if (b + 1 >= nb) break;
    if (b + 2 < nb) A.template load<true>(rw, ra, wo, ao, wave + (b + 2) * NWAVE, U);
    B.template compute<true>(acc, U);
  }
  if (rem > 0 && wave == nruns % NWAVE) {  // the one partial run
    A.template load<false>(rw, ra, wo, ao, nruns, rem);
    A.template compute<false>(acc, rem);
  }

  // cross-wave reduction in fixed order 0,1,2,3
  if (wave > 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int n = 0; n < NT; ++n) red[wave - 1][(w * NF + f) * NT + n][lane] = acc[w][f][n];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          f32x4 a = acc[w][f][n];
#pragma unroll
          for (int q = 0; q < NWAVE - 1; ++q) a += red[q][(w * NF + f) * NT + n][lane];
          acc[w][f][n] = a;
        }
    // D[m][n]: lane holds features f0 + f*16 + 4*kg + i (i = 0..3) of token row
    // row0 + n*16 + lr
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const size_t r = (size_t)(row0 + n * 16 + lr);
        const int col = f0 + f * 16 + 4 * kg;
        if constexpr (GATEUP) {
          T* h = reinterpret_cast<T*>(outp) + r * N + col;
          const f32x4 g = acc[0][f][n], u = acc[1][f][n];
#pragma unroll
          for (int i = 0; i < 4; ++i) h[i] = Elem<T>::from_f32(silu_f32(g[i]) * u[i]);
        } else {
          float* y = reinterpret_cast<float*>(outp) + r * N + col;
          *reinterpret_cast<float4*>(y) =
              make_float4(acc[0][f][n][0], acc[0][f][n][1], acc[0][f][n][2], acc[0][f][n][3]);
        }
      }
  }
}

// ---------------------------------------------------------------------------
// bf16 form with the weights staged through LDS.  A wave's run is 128 k (256
// bytes of each of the block's weight rows: 32 for gate/up, 16 gate + 16 up,
// and 16 for down); it is fetched by LDS DMA loads of 4 rows x 256 bytes
// each -- whole 256-byte pieces of a row per
// load, which the memory system serves markedly faster than the 16 rows x 64
// bytes of an MFMA-layout load -- into a per-wave slot where 16-byte chunk c
// of row r sits at c ^ (r % 16); the MFMA fragments are then read from LDS
// without bank conflicts.  Two slots (separate arrays, so that the compiler
// can tell which DMA each read waits for) alternate: run i + 1 is in flight
// while run i's MFMAs run.  Every step issues its loads unconditionally (past
// the wave's last run with offsets beyond the buffer ranges, which load
// zeros and move no bytes), so the waits before the reads never depend on a
// branch.  Token rows as in the register form.
// ---------------------------------------------------------------------------
template <int BT, int FT, bool GATEUP>
__device__ __forceinline__ void stream_dma_body(
    const bf16_t* __restrict__ act, const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_expert, int N, int K,
    const int32_t* __restrict__ row_token, int nT) {
  constexpr int NW = GATEUP ? 2 : 1, NF = FT / 16, NT = BT / 16;
  constexpr int NROW = NW * FT;                   // weight rows of the block
  constexpr int kRunK = 128, kRunBytes = kRunK * 2;
  constexpr int kSlot = NROW * kRunBytes;         // one wave's slot (8 KiB)
  constexpr int kDma = kSlot / 1024;              // DMA loads per run
  constexpr int NWAVE = kStreamThreads / kWave;
  static_assert(NROW % 16 == 0 && FT % 4 == 0 && kDma * 4 == NROW, "block shape");
  __shared__ __attribute__((aligned(1024))) char sl0[NWAVE * kSlot];
  __shared__ __attribute__((aligned(1024))) char sl1[NWAVE * kSlot];
  __shared__ f32x4 red[NWAVE - 1][NW * NF * NT][kWave];

  const int tile = blockIdx.y;
  const int row0 = tile * BT;
  const int lane = threadIdx.x & (kWave - 1);
  const int lr = lane & 15, kg = lane >> 4;
  // tokens in place: the token of each of this lane's rows (the load does
  // not wait on the expert lookup)
  int tok[NT];
  if (row_token != nullptr) {
#pragma unroll
    for (int n = 0; n < NT; ++n) tok[n] = row_token[row0 + n * 16 + lr];
  }
  const int e = tile_expert[tile];
  if (e < 0) return;
  const int f0 = blockIdx.x * FT;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  const uint32_t row_bytes = (uint32_t)K * 2;
  __amdgpu_buffer_rsrc_t rw[NW];
  rw[0] = buffer_rsrc(W0 + ((size_t)e * N + f0) * K, FT * row_bytes);
  if constexpr (GATEUP) rw[1] = buffer_rsrc(W1 + ((size_t)e * N + f0) * K, FT * row_bytes);
  // DMA load j: block rows 4 j .. 4 j + 3; lane i fills row 4 j + i / 16,
  // stored chunk i % 16 = global chunk (i % 16) ^ (row % 16)
  uint32_t dvo[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int rr = 4 * j + lane / 16;
    dvo[j] = (uint32_t)(rr % FT) * row_bytes + (uint32_t)(((lane & 15) ^ (rr & 15)) * 16);
  }
  // fragment (w, f) at k-step ks: row w * FT + f * 16 + lr, chunk ks * 4 + kg
  uint32_t fro[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    fro[ks] = (uint32_t)wave * kSlot + (uint32_t)lr * kRunBytes + (uint32_t)(((ks * 4 + kg) ^ lr) * 16);

  f32x4 acc[NW][NF][NT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[w][f][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nrun = K / kRunK;
  const int nb = nrun > wave ? (nrun - wave + NWAVE - 1) / NWAVE : 0;
  const int valid_end = offsets[e] + counts[e];
  const int nvalid = max(0, min(BT, valid_end - row0));
  // token rows past the expert's count load as zeros: outside the gathered
  // rows' range, or (in place) at an offset past the end of x
  uint32_t ao[NT];
  __amdgpu_buffer_rsrc_t ra;
  if (row_token != nullptr) {
    ra = buffer_rsrc(act, (uint32_t)nT * row_bytes);
#pragma unroll
    for (int n = 0; n < NT; ++n)
      ao[n] = (n * 16 + lr < nvalid && tok[n] >= 0) ? (uint32_t)tok[n] * row_bytes + kg * 16
                                                     : 0x80000000u;
  } else {
    ra = buffer_rsrc(act + (size_t)row0 * K, (uint32_t)nvalid * row_bytes);
#pragma unroll
    for (int n = 0; n < NT; ++n) ao[n] = (uint32_t)(n * 16 + lr) * row_bytes + kg * 16;
  }

  uint4 t0[NT][4], t1[NT][4];
  // Run i of this wave (clamped to its last run).  A run past the wave's
  // last (the steady state issues one, so that every wait counts the same
  // loads; nothing reads its slot) takes offsets past the buffer ranges: it
  // loads zeros and moves no bytes.
  auto issue = [&](char* slot, uint4 (&tk)[NT][4], int i) {
    const bool past = i >= nb;
    const int run = wave + NWAVE * min(i, nb - 1);
    const uint32_t so = (uint32_t)run * kRunBytes;
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
      lds_void* dst = (lds_void*)(slot + wave * kSlot + j * 1024);
      const uint32_t vo = past ? 0x80000000u : dvo[j];
      if (!GATEUP)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw[0], dst, 16, vo, so, 0,
                                                 MOE_WSTREAM_CPOL_DN);
      else if ((4 * j) / FT == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw[0], dst, 16, vo, so, 0,
                                                 MOE_WSTREAM_CPOL_GU);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw[GATEUP ? 1 : 0], dst, 16, vo, so, 0,
                                                 MOE_WSTREAM_CPOL_GU1);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) tk[n][ks] = sload(ra, past ? 0x80000000u : ao[n], so + ks * 64);
  };
  auto compute = [&](const char* slot, const uint4 (&tk)[NT][4]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const uint4 wf = *reinterpret_cast<const uint4*>(slot + fro[ks] + (w * FT + f * 16) * kRunBytes);
#pragma unroll
          for (int n = 0; n < NT; ++n) acc[w][f][n] = Elem<bf16_t>::mfma16(wf, tk[n][ks], acc[w][f][n]);
        }
  };
  // the scheduling barriers keep each run's loads (token rows included) where
  // they are written, a full run ahead of their use; the LDS wait before a
  // slot is refilled orders its last fragment reads before the DMA writes
  if (nb > 0) {
    issue(sl0, t0, 0);
    for (int i = 0; i < nb; i += 2) {
      issue(sl1, t1, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      compute(sl0, t0);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      issue(sl0, t0, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (i + 1 < nb) compute(sl1, t1);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no DMA left in flight
  }

  // cross-wave reduction in fixed order 0,1,2,3
  if (wave > 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int n = 0; n < NT; ++n) red[wave - 1][(w * NF + f) * NT + n][lane] = acc[w][f][n];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          f32x4 a = acc[w][f][n];
#pragma unroll
          for (int q = 0; q < NWAVE - 1; ++q) a += red[q][(w * NF + f) * NT + n][lane];
          acc[w][f][n] = a;
        }
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const size_t r = (size_t)(row0 + n * 16 + lr);
        const int col = f0 + f * 16 + 4 * kg;
        if constexpr (GATEUP) {
          bf16_t* h = reinterpret_cast<bf16_t*>(outp) + r * N + col;
          const f32x4 g = acc[0][f][n], u = acc[1][f][n];
          *reinterpret_cast<uint2*>(h) =
              make_uint2(pack_bf16x2(silu_f32(g[0]) * u[0], silu_f32(g[1]) * u[1]),
                         pack_bf16x2(silu_f32(g[2]) * u[2], silu_f32(g[3]) * u[3]));
        } else {
          float* y = reinterpret_cast<float*>(outp) + r * N + col;
          *reinterpret_cast<float4*>(y) =
              make_float4(acc[0][f][n][0], acc[0][f][n][1], acc[0][f][n][2], acc[0][f][n][3]);
        }
      }
  }
}

template <int BT, int FT, bool GATEUP>
__global__ __launch_bounds__(kStreamThreads) void stream_dma_kernel(
    const bf16_t* __restrict__ act, const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ num_tiles,
    const int32_t* __restrict__ tile_expert, int N, int K, const int32_t* __restrict__ row_token,
    int nT) {
  (void)num_tiles;
  stream_dma_body<BT, FT, GATEUP>(act, W0, W1, outp, counts, offsets, tile_expert, N, K,
                                  row_token, nT);
}

template <typename T, int BT>
static void gateup_stream(const Dims& D, const void* xs, const int32_t* row_token, const void* Wg,
                          const void* Wu, void* h, const int32_t* counts, const int32_t* offsets,
                          const int32_t* num_tiles, const int32_t* tile_expert, hipStream_t s) {
  constexpr int FT = MOE_STREAM_FT_GU;
  dim3 grid(D.f / FT, D.max_tiles);
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (D.d % 128 == 0) {
      stream_dma_kernel<BT, FT, true><<<grid, kStreamThreads, 0, s>>>(
          (const bf16_t*)xs, (const bf16_t*)Wg, (const bf16_t*)Wu, h, counts, offsets, num_tiles,
          tile_expert, D.f, D.d, row_token, D.T);
      return;
    }
  }
  stream_gemm_kernel<T, BT, FT, true, MOE_STREAM_U><<<grid, kStreamThreads, 0, s>>>(
      (const T*)xs, (const T*)Wg, (const T*)Wu, h, counts, offsets, num_tiles, tile_expert, D.f,
      D.d);
}

template <typename T, int BT>
static void down_stream(const Dims& D, const void* h, const void* Wd, float* y,
                        const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                        const int32_t* tile_expert, hipStream_t s) {
  constexpr int FT = MOE_STREAM_FT_DN;
  dim3 grid(D.d / FT, D.max_tiles);
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (D.f % 128 == 0) {
      constexpr int FTD = MOE_STREAM_DMA_FT_DN;
      stream_dma_kernel<BT, FTD, false><<<dim3(D.d / FTD, D.max_tiles), kStreamThreads, 0, s>>>(
          (const bf16_t*)h, (const bf16_t*)Wd, nullptr, y, counts, offsets, num_tiles,
          tile_expert, D.d, D.f, nullptr, 0);
      return;
    }
  }
  stream_gemm_kernel<T, BT, FT, false, MOE_STREAM_U><<<grid, kStreamThreads, 0, s>>>(
      (const T*)h, (const T*)Wd, nullptr, y, counts, offsets, num_tiles, tile_expert, D.d, D.f);
}

void launch_gateup_stream(const Dims& D, const void* act, const int32_t* row_token,
                          const void* Wg, const void* Wu, void* h, const int32_t* counts,
                          const int32_t* offsets, const int32_t* num_tiles,
                          const int32_t* tile_expert, hipStream_t s) {
  if (D.bf16) {
    if (D.BT == 16)
      gateup_stream<bf16_t, 16>(D, act, row_token, Wg, Wu, h, counts, offsets, num_tiles,
                                tile_expert, s);
    else
      gateup_stream<bf16_t, 32>(D, act, row_token, Wg, Wu, h, counts, offsets, num_tiles,
                                tile_expert, s);
  } else {
    if (D.BT == 16)
      gateup_stream<float, 16>(D, act, nullptr, Wg, Wu, h, counts, offsets, num_tiles,
                               tile_expert, s);
    else
      gateup_stream<float, 32>(D, act, nullptr, Wg, Wu, h, counts, offsets, num_tiles,
                               tile_expert, s);
  }
}

void launch_down_stream(const Dims& D, const void* h, const void* Wd, float* y,
                        const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                        const int32_t* tile_expert, hipStream_t s) {
  if (D.bf16) {
    if (D.BT == 16) down_stream<bf16_t, 16>(D, h, Wd, y, counts, offsets, num_tiles, tile_expert, s);
    else down_stream<bf16_t, 32>(D, h, Wd, y, counts, offsets, num_tiles, tile_expert, s);
  } else {
    if (D.BT == 16) down_stream<float, 16>(D, h, Wd, y, counts, offsets, num_tiles, tile_expert, s);
    else down_stream<float, 32>(D, h, Wd, y, counts, offsets, num_tiles, tile_expert, s);
  }
}

}  // namespace moe
