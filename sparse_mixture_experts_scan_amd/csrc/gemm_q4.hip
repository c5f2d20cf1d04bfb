// Weight-only INT4 expert weights: the quantizer, the dequantizer, and the
// weight-streaming grouped GEMMs that read INT4 weights (decode shapes).
//
// "Mixtral of Experts" (singularity-lens.com), list of limitations, memory
// item: the whole model fits in about 25-30 GB only with INT4 quantisation.
// The pages give no scheme; this library uses symmetric per-group absmax:
//   s   = max_{k in group} |w_k| / 7                 (float32, IEEE division)
//   q_k = clamp(rint(w_k / s), -8, 7)                (q = 0 when s = 0)
//   w~_k = s * q_k
// with groups of `group` consecutive input features of one weight row.
// Storage of a matrix [N][K]: packed[N][K/2] bytes, nibble u = q + 8,
// element 2b in the low nibble of byte b and element 2b + 1 in the high
// nibble; scales[K/group][N] float32, group-major, so that the scales of one
// group of 16 neighbouring rows sit in one 64-byte line.
//
// The GEMM: as the bf16 weight-streaming form, the MFMA A operand is 16
// weight rows and B 16 token rows.  One 16-byte load gives a lane 32
// consecutive INT4 weights of its row, which feed four 16x16x32 bf16 MFMAs;
// the lane's activation loads cover the same 32 K indices (four 16-byte
// loads), so A and B agree on every k.  Each weight is dequantized in
// registers to bf16(s * q) (one float32 fma, one rounding to bf16), the same
// value the dequantizer writes, so both GEMM forms see identical weights.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kQ4Threads = 256;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));


__device__ __forceinline__ uint4 q4_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                           uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float q4_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

// two float32 -> packed bf16 pair (round to nearest even), low half = a
__device__ inline uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// 8 nibbles (element i at bits 4i..4i+3) -> 8 bf16 weights s * (u - 8)
__device__ inline uint4 dequant8(uint32_t w, float s) {
  const uint32_t lo = w & 0x0F0F0F0Fu;          // elements 0, 2, 4, 6
  const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // elements 1, 3, 5, 7
  const float ns = -8.0f * s;                   // exact
  float e[8];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // fma(u, s, -8s) rounds s * (u - 8) once, as (u - 8) * s does
    e[2 * b] = fmaf((float)((lo >> (8 * b)) & 0xFFu), s, ns);
    e[2 * b + 1] = fmaf((float)((hi >> (8 * b)) & 0xFFu), s, ns);
  }
  return make_uint4(pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]), pack_bf16(e[4], e[5]),
                    pack_bf16(e[6], e[7]));
}

}  // namespace

// ---------------------------------------------------------------------------
// Quantizer: one block per weight row.  Pass 1: max |w| of every 8-element
// chunk into LDS; pass 2: one thread per group reduces its chunks and writes
// the scale; pass 3: the codes of each chunk, packed into one 32-bit word.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void quantize_int4_kernel(const T* __restrict__ W, int N, int K,
                                                            int G, uint32_t* __restrict__ packed,
                                                            float* __restrict__ scales) {
  extern __shared__ float q4_smem[];
  const int nch = K / 8, ngr = K / G, cpg = G / 8;
  float* cmax = q4_smem;
  float* gsc = q4_smem + nch;
  const size_t row = blockIdx.x;
  const size_t mat = row / N, n = row - mat * N;
  const T* w = W + row * (size_t)K;
  for (int c = threadIdx.x; c < nch; c += 256) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(Elem<T>::to_f32(w[c * 8 + i])));
    cmax[c] = m;
  }
  __syncthreads();
  for (int g = threadIdx.x; g < ngr; g += 256) {
    float m = 0.f;
    for (int c = g * cpg; c < (g + 1) * cpg; ++c) m = fmaxf(m, cmax[c]);
    const float s = m / 7.0f;
    gsc[g] = s;
    scales[(mat * ngr + g) * N + n] = s;
  }
  __syncthreads();
  for (int c = threadIdx.x; c < nch; c += 256) {
    const float s = gsc[c / cpg];
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int q = 0;
      if (s > 0.f) {
        const float r = rintf(Elem<T>::to_f32(w[c * 8 + i]) / s);
        q = (int)fminf(fmaxf(r, -8.f), 7.f);
      }
      word |= (uint32_t)(q + 8) << (4 * i);
    }
    packed[row * (size_t)nch + c] = word;
  }
}

// Dequantizer (for the LDS-tiled GEMMs): bf16(s * q) of every weight, 8 per
// thread, in the layout of the bf16 weights.
__global__ __launch_bounds__(256) void dequant_int4_kernel(const uint32_t* __restrict__ packed,
                                                           const float* __restrict__ scales,
                                                           int64_t nchunks, int N, int K, int G,
                                                           uint4* __restrict__ out) {
  const int cpr = K / 8, ngr = K / G;
  for (int64_t i = blockIdx.x * (int64_t)256 + threadIdx.x; i < nchunks;
       i += (int64_t)gridDim.x * 256) {
    const int64_t row = i / cpr;
    const int c = (int)(i - row * cpr);
    const int64_t mat = row / N, n = row - mat * N;
    const float s = scales[(mat * ngr + (c * 8) / G) * N + n];
    out[i] = dequant8(packed[i], s);
  }
}

// ---------------------------------------------------------------------------
// INT4 weight-streaming GEMM.  Chunk c of K (128 elements): lane (lr, kg) of
// a 16-row weight fragment loads bytes [c*64 + kg*16, +16) of row lr, i.e.
// K indices c*128 + kg*32 + [0, 32); word j of it feeds k-step j, whose
// activation operand is the 16 bytes at K index c*128 + kg*32 + 8j.
// Runs of U chunks interleave over the 4 waves; the next run's loads are in
// flight during the current run's dequantization and MFMAs.
// ---------------------------------------------------------------------------
template <int BT, int FT, bool GATEUP, int U>
struct Q4Batch {
  static constexpr int NF = FT / 16;
  static constexpr int NT = BT / 16;
  static constexpr int NW = GATEUP ? 2 : 1;
  uint4 wq[NW][NF][U];
  float sc[NW][NF][U];
  uint4 xv[NT][U][4];

  template <bool FULL>
  __device__ __forceinline__ void load(const __amdgpu_buffer_rsrc_t (&rw)[NW],
                                       const __amdgpu_buffer_rsrc_t (&rs)[NW],
                                       __amdgpu_buffer_rsrc_t ra, const uint32_t (&wo)[NF],
                                       const uint32_t (&so)[NF], const uint32_t (&ao)[NT],
                                       int run, int valid, int cpg, int gpc, uint32_t sgrp) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (FULL || u < valid) {
        const uint32_t c = (uint32_t)(run * U + u);
        const uint32_t wsoff = c * (kQ4Chunk / 2);
        const uint32_t ssoff = (c / cpg) * gpc * sgrp;
        const uint32_t asoff = c * kQ4Chunk * 2;
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            wq[w][f][u] = q4_load16(rw[w], wo[f], wsoff);
            sc[w][f][u] = q4_load4(rs[w], so[f], ssoff);
          }
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int j = 0; j < 4; ++j) xv[n][u][j] = q4_load16(ra, ao[n] + 16 * j, asoff);
      }
    }
  }

  // the first batch: codes and scales as soon as the expert is known,
  // activations once their row range is
  __device__ __forceinline__ void load_w(const __amdgpu_buffer_rsrc_t (&rw)[NW],
                                         const __amdgpu_buffer_rsrc_t (&rs)[NW],
                                         const uint32_t (&wo)[NF], const uint32_t (&so)[NF],
                                         int run, int cpg, int gpc, uint32_t sgrp) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = (uint32_t)(run * U + u);
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          wq[w][f][u] = q4_load16(rw[w], wo[f], c * (kQ4Chunk / 2));
          sc[w][f][u] = q4_load4(rs[w], so[f], (c / cpg) * gpc * sgrp);
        }
    }
  }
  __device__ __forceinline__ void load_x(__amdgpu_buffer_rsrc_t ra, const uint32_t (&ao)[NT],
                                         int run) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t c = (uint32_t)(run * U + u);
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) xv[n][u][j] = q4_load16(ra, ao[n] + 16 * j, c * kQ4Chunk * 2);
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
          for (int f = 0; f < NF; ++f) {
            const uint32_t words[4] = {wq[w][f][u].x, wq[w][f][u].y, wq[w][f][u].z,
                                       wq[w][f][u].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint4 a = dequant8(words[j], sc[w][f][u]);
#pragma unroll
              for (int n = 0; n < NT; ++n)
                acc[w][f][n] = Elem<bf16_t>::mfma16(a, xv[n][u][j], acc[w][f][n]);
            }
          }
      }
    }
  }
};

template <int BT, int FT, bool GATEUP, int U>
__device__ __forceinline__ void stream_q4_body(
    const bf16_t* __restrict__ act, const uint8_t* __restrict__ Q0,
    const float* __restrict__ S0, const uint8_t* __restrict__ Q1, const float* __restrict__ S1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ num_tiles,
    const int32_t* __restrict__ tile_expert, int N, int K, int G,
    const int32_t* __restrict__ row_token, int nT) {
  using QB = Q4Batch<BT, FT, GATEUP, U>;
  constexpr int NF = QB::NF, NT = QB::NT, NW = QB::NW;
  constexpr int NWAVE = kQ4Threads / kWave;
  __shared__ f32x4 red[NWAVE - 1][NW * NF * NT][kWave];

  // tiles past those in use have expert -1; the first weight loads wait only
  // for the expert lookup
  const int tile = blockIdx.y;
  const int row0 = tile * BT;
  const int lane = threadIdx.x & (kWave - 1);
  const int lr = lane & 15, kg = lane >> 4;
  // tokens read in place: the token of each of this lane's rows
  int tok[NT];
  if (row_token != nullptr) {
#pragma unroll
    for (int n = 0; n < NT; ++n) tok[n] = row_token[row0 + n * 16 + lr];
  }
  const int e = tile_expert[tile];
  if (e < 0) return;
  const int f0 = blockIdx.x * FT;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);

  const int ngr = K / G;
  const int cpg = G >= kQ4Chunk ? G / kQ4Chunk : 1;   // chunks per group
  const int gpc = G >= kQ4Chunk ? 1 : kQ4Chunk / G;   // groups per chunk
  // scales of expert e: [ngr][N]; this block's columns f0 .. f0 + FT - 1
  const uint32_t qrow = (uint32_t)K / 2, sgrp = (uint32_t)N * 4;
  const uint32_t sbytes = (uint32_t)(ngr - 1) * sgrp + FT * 4;
  __amdgpu_buffer_rsrc_t rw[NW], rs[NW];
  rw[0] = buffer_rsrc(Q0 + ((size_t)e * N + f0) * qrow, FT * qrow);
  rs[0] = buffer_rsrc(S0 + (size_t)e * ngr * N + f0, sbytes);
  if constexpr (GATEUP) {
    rw[1] = buffer_rsrc(Q1 + ((size_t)e * N + f0) * qrow, FT * qrow);
    rs[1] = buffer_rsrc(S1 + (size_t)e * ngr * N + f0, sbytes);
  }
  const uint32_t arow = (uint32_t)K * 2;
  uint32_t wo[NF], so[NF], ao[NT];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    wo[f] = (uint32_t)(f * 16 + lr) * qrow + kg * 16;
    so[f] = (uint32_t)(f * 16 + lr) * 4 + (uint32_t)((kg * 32) / G) * sgrp;
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) ao[n] = (uint32_t)(n * 16 + lr) * arow + kg * 64;

  f32x4 acc[NW][NF][NT];
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int n = 0; n < NT; ++n) acc[w][f][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nch = K / kQ4Chunk;
  const int nruns = nch / U, rem = nch % U;
  const int nb = nruns > wave ? (nruns - wave + NWAVE - 1) / NWAVE : 0;
  // Steady state with unconditional loads, so that the wait before each
  // compute counts only the other batch's loads; then a 1- or 2-batch tail.
  // Scheduling barriers keep each batch's loads ahead of the other batch's
  // compute (the scheduler would otherwise merge the two phases).
  QB A, B;
  int b = 0;
  if (nb > 0) A.load_w(rw, rs, wo, so, wave, cpg, gpc, sgrp);
  const int valid_end = offsets[e] + counts[e];
  const int nvalid = max(0, min(BT, valid_end - row0));
  // token rows past the expert's count load as zeros: outside the gathered
  // rows' range, or (in place) at an offset past the end of x
  __amdgpu_buffer_rsrc_t ra;
  if (row_token != nullptr) {
    ra = buffer_rsrc(act, (uint32_t)nT * arow);
#pragma unroll
    for (int n = 0; n < NT; ++n)
      ao[n] = (n * 16 + lr < nvalid && tok[n] >= 0) ? (uint32_t)tok[n] * arow + kg * 64
                                                     : 0x80000000u;
  } else {
    ra = buffer_rsrc(act + (size_t)row0 * K, (uint32_t)nvalid * arow);
  }
  if (nb > 0) A.load_x(ra, ao, wave);
  for (; b + 2 < nb; b += 2) {
    B.template load<true>(rw, rs, ra, wo, so, ao, wave + (b + 1) * NWAVE, U, cpg, gpc, sgrp);
    __builtin_amdgcn_sched_barrier(0);
    A.template compute<true>(acc, U);
    __builtin_amdgcn_sched_barrier(0);
    A.template load<true>(rw, rs, ra, wo, so, ao, wave + (b + 2) * NWAVE, U, cpg, gpc, sgrp);
    __builtin_amdgcn_sched_barrier(0);
    B.template compute<true>(acc, U);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (b + 1 < nb) {
    B.template load<true>(rw, rs, ra, wo, so, ao, wave + (b + 1) * NWAVE, U, cpg, gpc, sgrp);
    A.template compute<true>(acc, U);
    B.template compute<true>(acc, U);
  } else if (b < nb) {
    A.template compute<true>(acc, U);
  }
  if (rem > 0 && wave == nruns % NWAVE) {
    A.template load<false>(rw, rs, ra, wo, so, ao, nruns, rem, cpg, gpc, sgrp);
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
    // lane holds features f0 + f*16 + 4*kg + i (i = 0..3) of token row
    // row0 + n*16 + lr
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

// Decode shapes (16-row token tiles) are latency-bound on the weight stream:
// registers are capped so that 4 waves share each SIMD.
#ifndef MOE_Q4_WPE16
#define MOE_Q4_WPE16 4
#endif

#define MOE_Q4_PARAMS                                                                        \
  const bf16_t *__restrict__ act, const uint8_t *__restrict__ Q0,                            \
      const float *__restrict__ S0, const uint8_t *__restrict__ Q1,                          \
      const float *__restrict__ S1, void *__restrict__ outp,                                 \
      const int32_t *__restrict__ counts, const int32_t *__restrict__ offsets,               \
      const int32_t *__restrict__ num_tiles, const int32_t *__restrict__ tile_expert, int N, \
      int K, int G, const int32_t *__restrict__ row_token, int nT
#define MOE_Q4_ARGS \
  act, Q0, S0, Q1, S1, outp, counts, offsets, num_tiles, tile_expert, N, K, G, row_token, nT

template <int FT, bool GATEUP, int U>
__global__ __launch_bounds__(kQ4Threads)
__attribute__((amdgpu_waves_per_eu(MOE_Q4_WPE16, 8))) void stream_q4_kernel16(MOE_Q4_PARAMS) {
  stream_q4_body<16, FT, GATEUP, U>(MOE_Q4_ARGS);
}

template <int FT, bool GATEUP, int U>
__global__ __launch_bounds__(kQ4Threads) void stream_q4_kernel32(MOE_Q4_PARAMS) {
  stream_q4_body<32, FT, GATEUP, U>(MOE_Q4_ARGS);
}

#ifndef MOE_Q4_U
#define MOE_Q4_U 1
#endif
#ifndef MOE_Q4_FT_GU
#define MOE_Q4_FT_GU 32
#endif
#ifndef MOE_Q4_FT_DN
#define MOE_Q4_FT_DN 64
#endif

void launch_quantize_int4(const void* W, bool bf16, int64_t rows, int N, int K, int G,
                          void* packed, float* scales, hipStream_t s) {
  const size_t lds = sizeof(float) * ((size_t)K / 8 + (size_t)K / G);
  if (bf16)
    quantize_int4_kernel<bf16_t><<<(unsigned)rows, 256, lds, s>>>(
        (const bf16_t*)W, N, K, G, (uint32_t*)packed, scales);
  else
    quantize_int4_kernel<float><<<(unsigned)rows, 256, lds, s>>>((const float*)W, N, K, G,
                                                                  (uint32_t*)packed, scales);
}

void launch_dequant_int4(const void* packed, const float* scales, int64_t rows, int N, int K,
                         int G, void* out, hipStream_t s) {
  const int64_t nchunks = rows * (K / 8);
  const int64_t want = (nchunks + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  dequant_int4_kernel<<<grid, 256, 0, s>>>((const uint32_t*)packed, scales, nchunks, N, K, G,
                                           (uint4*)out);
}

template <int BT>
static void gateup_q4(const Dims& D, const void* xs, const int32_t* row_token,
                      const Q4Weights& Wg, const Q4Weights& Wu, void* h, const int32_t* counts,
                      const int32_t* offsets, const int32_t* num_tiles,
                      const int32_t* tile_expert, hipStream_t s) {
  constexpr int FT = MOE_Q4_FT_GU;
  dim3 grid(D.f / FT, D.max_tiles);
  auto kern = BT == 16 ? stream_q4_kernel16<FT, true, MOE_Q4_U>
                       : stream_q4_kernel32<FT, true, MOE_Q4_U>;
  kern<<<grid, kQ4Threads, 0, s>>>((const bf16_t*)xs, (const uint8_t*)Wg.q, Wg.s,
                                   (const uint8_t*)Wu.q, Wu.s, h, counts, offsets, num_tiles,
                                   tile_expert, D.f, D.d, D.group, row_token, D.T);
}

template <int BT>
static void down_q4(const Dims& D, const void* h, const Q4Weights& Wd, float* y,
                    const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                    const int32_t* tile_expert, hipStream_t s) {
  constexpr int FT = MOE_Q4_FT_DN;
  dim3 grid(D.d / FT, D.max_tiles);
  auto kern = BT == 16 ? stream_q4_kernel16<FT, false, MOE_Q4_U>
                       : stream_q4_kernel32<FT, false, MOE_Q4_U>;
  kern<<<grid, kQ4Threads, 0, s>>>((const bf16_t*)h, (const uint8_t*)Wd.q, Wd.s, nullptr,
                                   nullptr, y, counts, offsets, num_tiles, tile_expert, D.d,
                                   D.f, D.group, nullptr, 0);
}

void launch_gateup_q4(const Dims& D, const void* act, const int32_t* row_token,
                      const Q4Weights& Wg, const Q4Weights& Wu, void* h, const int32_t* counts,
                      const int32_t* offsets, const int32_t* num_tiles,
                      const int32_t* tile_expert, hipStream_t s) {
  if (D.BT == 16)
    gateup_q4<16>(D, act, row_token, Wg, Wu, h, counts, offsets, num_tiles, tile_expert, s);
  else
    gateup_q4<32>(D, act, row_token, Wg, Wu, h, counts, offsets, num_tiles, tile_expert, s);
}

void launch_down_q4(const Dims& D, const void* h, const Q4Weights& Wd, float* y,
                    const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                    const int32_t* tile_expert, hipStream_t s) {
  if (D.BT == 16) down_q4<16>(D, h, Wd, y, counts, offsets, num_tiles, tile_expert, s);
  else down_q4<32>(D, h, Wd, y, counts, offsets, num_tiles, tile_expert, s);
}

}  // namespace moe
