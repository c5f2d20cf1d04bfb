// Grouped expert GEMMs, weight-streaming form (few token rows per expert).
//
// "Mistral/Mixtralのアーキテクチャ", section "各エキスパートの構造":
//   E_i(x) = W2 (SiLU(W1 x) * W3 x), W1, W3: d_ff x d_model, W2: d_model x d_ff.
// Gate/up: H[r][f] = SiLU(sum_c W_gate[e][f][c] Xs[r][c]) * sum_c W_up[e][f][c] Xs[r][c]
// Down:    Y[r][o] = sum_f W_down[e][o][f] H[r][f]   (fp32 out)
// for every permuted row r of expert e's segment.
//
// Shape of the work: with a handful of rows per expert the weights are read
// exactly once and nothing is reused, so this form goes straight from HBM to
// registers (no LDS staging of weights): the MFMA A operand is 16 weight rows
// (output features), the B operand 16 token rows, both K-contiguous, 16 bytes
// per lane per load.  A workgroup owns FT output features of one token tile;
// its 4 waves split K by interleaved 16-byte k-groups so that the 4 waves
// together read contiguous 256-byte runs of each weight row; the partial sums
// are added in fixed wave order through LDS (deterministic), then the
// epilogue (SiLU(gate)*up, or plain fp32) is applied and stored.
//
// Token rows past the expert's count (segment padding) read as zero, so the
// padding rows of H are exactly zero and every row stored is in bounds.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kStreamThreads = 256;

template <typename T, int BT, int FT, bool GATEUP, int U>
__global__ __launch_bounds__(kStreamThreads) void stream_gemm_kernel(
    const T* __restrict__ act, const T* __restrict__ W0, const T* __restrict__ W1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ num_tiles,
    const int32_t* __restrict__ tile_expert, int N, int K) {
  constexpr int VEC = Elem<T>::kVec;
  constexpr int KSTEP = 4 * VEC;          // K covered by one 16x16 MFMA k-group set
  constexpr int NF = FT / 16;             // 16-row weight fragments per wave
  constexpr int NT = BT / 16;             // 16-row token fragments
  constexpr int NW = GATEUP ? 2 : 1;      // weight stacks (gate, up) or (down)
  constexpr int NWAVE = kStreamThreads / kWave;
  __shared__ f32x4 red[NWAVE - 1][NW * NF * NT][kWave];

  const int tile = blockIdx.y;
  if (tile >= *num_tiles) return;
  const int e = tile_expert[tile];
  const int row0 = tile * BT;
  const int valid_end = offsets[e] + counts[e];
  const int f0 = blockIdx.x * FT;
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int lr = lane & 15, kg = lane >> 4;

  const T* wp[NW];
  wp[0] = W0 + ((size_t)e * N + f0 + lr) * K + kg * VEC;
  if constexpr (GATEUP) wp[1] = W1 + ((size_t)e * N + f0 + lr) * K + kg * VEC;
  const T* ap[NT];
  bool aok[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int r = row0 + n * 16 + lr;
    aok[n] = r < valid_end;
    ap[n] = act + (size_t)r * K + kg * VEC;
  }

  f32x4 acc[NW][NF][NT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[w][f][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nks = K / KSTEP;
  const uint4 zero = make_uint4(0, 0, 0, 0);
  for (int ks0 = wave; ks0 < nks; ks0 += NWAVE * U) {
    uint4 wv[NW][NF][U];
    uint4 av[NT][U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + NWAVE * u;
      if (ks < nks) {
        const size_t ko = (size_t)ks * KSTEP;
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int f = 0; f < NF; ++f) wv[w][f][u] = ld16(wp[w] + (size_t)f * 16 * K + ko);
#pragma unroll
        for (int n = 0; n < NT; ++n) av[n][u] = aok[n] ? ld16(ap[n] + ko) : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ks0 + NWAVE * u < nks) {
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

template <typename T, int BT>
static void gateup_stream(const Dims& D, const void* xs, const void* Wg, const void* Wu, void* h,
                          const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                          const int32_t* tile_expert, hipStream_t s) {
  constexpr int FT = 32;
  dim3 grid(D.f / FT, D.max_tiles);
  stream_gemm_kernel<T, BT, FT, true, 8><<<grid, kStreamThreads, 0, s>>>(
      (const T*)xs, (const T*)Wg, (const T*)Wu, h, counts, offsets, num_tiles, tile_expert, D.f,
      D.d);
}

template <typename T, int BT>
static void down_stream(const Dims& D, const void* h, const void* Wd, float* y,
                        const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                        const int32_t* tile_expert, hipStream_t s) {
  constexpr int FT = 64;
  dim3 grid(D.d / FT, D.max_tiles);
  stream_gemm_kernel<T, BT, FT, false, 8><<<grid, kStreamThreads, 0, s>>>(
      (const T*)h, (const T*)Wd, nullptr, y, counts, offsets, num_tiles, tile_expert, D.d, D.f);
}

void launch_gateup_stream(const Dims& D, const void* xs, const void* Wg, const void* Wu, void* h,
                          const int32_t* counts, const int32_t* offsets,
                          const int32_t* num_tiles, const int32_t* tile_expert, hipStream_t s) {
  if (D.bf16) {
    if (D.BT == 16) gateup_stream<bf16_t, 16>(D, xs, Wg, Wu, h, counts, offsets, num_tiles, tile_expert, s);
    else gateup_stream<bf16_t, 32>(D, xs, Wg, Wu, h, counts, offsets, num_tiles, tile_expert, s);
  } else {
    if (D.BT == 16) gateup_stream<float, 16>(D, xs, Wg, Wu, h, counts, offsets, num_tiles, tile_expert, s);
    else gateup_stream<float, 32>(D, xs, Wg, Wu, h, counts, offsets, num_tiles, tile_expert, s);
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
