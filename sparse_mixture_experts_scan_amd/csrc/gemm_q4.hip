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
// loads), so A and B agree on every k.  Two forms of the dequantization:
//  - groups of a multiple of 128 (one group per chunk): the MFMAs take the
//    codes themselves and the scale multiplies the chunk's float32 partial
//    sum, s * sum_k q_k x_k, which is the group's share of the product with
//    the weights s * q_k exactly up to float32 rounding.  A code enters the
//    MFMA as bf16(128 + u) (u = q + 8 OR-ed into the mantissa of 128: one
//    and-or per pair of codes), and the chunk's accumulator starts at
//    -136 * sum_k x_k (one MFMA with a constant operand per k-step, shared by
//    all the weight rows), so that it ends at sum_k (u_k - 8) x_k;
//  - smaller groups (a chunk spans several groups, so an MFMA would mix
//    scales): each weight is dequantized in registers to bf16(s * q) (one
//    float32 fma, one rounding to bf16), the value the dequantizer writes.
#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kQ4Threads = 256;
// cache policy of the LDS-staged form's code DMA (gfx950 bits: 1 sc0, 2 nt,
// 16 sc1), measured on MI355X at the Mixtral decode shape with group 128:
// non-temporal for the down codes (50.6 -> 46.6 us); for gate/up on the up
// codes only (95 -> 91.6 us; on both 95, on neither 97, on the gate codes
// only 91.7)
#ifndef MOE_Q4_CPOL
#define MOE_Q4_CPOL 2                 // down codes
#endif
#ifndef MOE_Q4_CPOL_GU0
#define MOE_Q4_CPOL_GU0 0             // gate codes (Q1) of the gate/up kernel
#endif
#ifndef MOE_Q4_CPOL_GU1
#define MOE_Q4_CPOL_GU1 2             // up codes (Q3)
#endif

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

// 8 nibbles (element i at bits 4i) -> bf16(128 + u) of each, as the pairs
// (0, 4), (1, 5), (2, 6), (3, 7): 128 in bf16 is 0x4300 and its 7 mantissa
// bits count units of 1, so OR-ing u into bits 0..3 adds u exactly.
// The constants come in registers (CodeConsts): a VOP3 and-or cannot encode
// two literals, and with them inline the compiler emits a separate and + or.
struct CodeConsts {
  uint32_t mask, magic;   // 0x000F000F, 0x43004300
  __device__ static CodeConsts make() {
    CodeConsts c{0x000F000Fu, 0x43004300u};
    asm volatile("" : "+v"(c.mask), "+v"(c.magic));   // keep them in VGPRs
    return c;
  }
};
__device__ inline uint4 codes8(uint32_t w, CodeConsts c) {
  return make_uint4((w & c.mask) | c.magic, ((w >> 4) & c.mask) | c.magic,
                    ((w >> 8) & c.mask) | c.magic, ((w >> 12) & c.mask) | c.magic);
}

// 8 consecutive bf16 activations (pairs (0,1), (2,3), (4,5), (6,7)) into the
// order of codes8: (0,4), (1,5), (2,6), (3,7)
__device__ inline uint4 pair_like_codes(uint4 x) {
  constexpr uint32_t kLo = 0x05040100u, kHi = 0x07060302u;  // v_perm byte selectors
  return make_uint4(__builtin_amdgcn_perm(x.z, x.x, kLo), __builtin_amdgcn_perm(x.z, x.x, kHi),
                    __builtin_amdgcn_perm(x.w, x.y, kLo), __builtin_amdgcn_perm(x.w, x.y, kHi));
}

// -136 in bf16, in all eight halves: the MFMA operand of the offset term
constexpr uint32_t kNeg136x2 = 0xC308C308u;

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
// POST: groups of a multiple of 128; each lane then loads the four scales of
// its accumulator rows (f*16 + 4*kg + i) for the chunk's group, else the one
// scale of its weight row lr for its 32 K indices.
template <int BT, int FT, bool GATEUP, int U, bool POST>
struct Q4Batch {
  static constexpr int NF = FT / 16;
  static constexpr int NT = BT / 16;
  static constexpr int NW = GATEUP ? 2 : 1;
  uint4 wq[NW][NF][U];
  float sc[NW][NF][U];
  f32x4 sc4[NW][NF][U];
  uint4 xv[NT][U][4];

  __device__ __forceinline__ void load_scale(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                             uint32_t soff, int w, int f, int u) {
    if constexpr (POST) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
      sc4[w][f][u] = f32x4{__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                           __uint_as_float(v[3])};
    } else {
      sc[w][f][u] = q4_load4(r, voff, soff);
    }
  }

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
            load_scale(rs[w], so[f], ssoff, w, f, u);
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
          load_scale(rs[w], so[f], (c / cpg) * gpc * sgrp, w, f, u);
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
    if constexpr (POST) {
      compute_post<FULL>(acc, valid);
      return;
    }
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

  // one chunk = one group: t = sum_k (u_k - 8) x_k over the chunk's 128 K
  // indices (the offset term first, then the codes), acc += s * t per row
  template <bool FULL>
  __device__ __forceinline__ void compute_post(f32x4 (&acc)[NW][NF][NT], int valid) {
    const uint4 neg136 = make_uint4(kNeg136x2, kNeg136x2, kNeg136x2, kNeg136x2);
    const CodeConsts cc = CodeConsts::make();
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (FULL || u < valid) {
        f32x4 off[NT];
        uint4 xp[NT][4];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          off[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            off[n] = Elem<bf16_t>::mfma16(neg136, xv[n][u][j], off[n]);
            xp[n][j] = pair_like_codes(xv[n][u][j]);
          }
        }
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const uint32_t words[4] = {wq[w][f][u].x, wq[w][f][u].y, wq[w][f][u].z,
                                       wq[w][f][u].w};
            f32x4 t[NT];
#pragma unroll
            for (int n = 0; n < NT; ++n) t[n] = off[n];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint4 a = codes8(words[j], cc);
#pragma unroll
              for (int n = 0; n < NT; ++n) t[n] = Elem<bf16_t>::mfma16(a, xp[n][j], t[n]);
            }
            const f32x4 sv = sc4[w][f][u];
#pragma unroll
            for (int n = 0; n < NT; ++n)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc[w][f][n][i] = fmaf(sv[i], t[n][i], acc[w][f][n][i]);
          }
      }
    }
  }
};

template <int BT, int FT, bool GATEUP, int U, bool POST>
__device__ __forceinline__ void stream_q4_body(
    const bf16_t* __restrict__ act, const uint8_t* __restrict__ Q0,
    const float* __restrict__ S0, const uint8_t* __restrict__ Q1, const float* __restrict__ S1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ num_tiles,
    const int32_t* __restrict__ tile_expert, int N, int K, int G,
    const int32_t* __restrict__ row_token, int nT) {
  using QB = Q4Batch<BT, FT, GATEUP, U, POST>;
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
    so[f] = POST ? (uint32_t)(f * 16 + 4 * kg) * 4
                 : (uint32_t)(f * 16 + lr) * 4 + (uint32_t)((kg * 32) / G) * sgrp;
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

// ---------------------------------------------------------------------------
// INT4 weight streaming through LDS (groups of a multiple of 128, K a
// multiple of 256): a wave's run is 256 K indices, i.e. 128 bytes of each of
// the block's NW * FT weight rows, fetched by LDS DMA whole lines at a time
// (lane i of DMA j fills row 8 j + i / 8; stored 16-byte piece i % 8 holds
// global piece (i % 8) ^ (row % 8), so that the 16 rows of a fragment read
// 16 bytes each without bank conflicts), together with the run's two
// groups' scales of the block's rows (4-byte DMA, [matrix][group][row]).
// Only the token rows go to registers, so the bytes in flight do not
// compete with the accumulators for VGPRs.  Each wave owns a slot in each
// of two buffers and keeps the next run in flight while it computes the
// current one from the other buffer; the dequantization is the post-scaled
// form above, one chunk (128 K indices, one group) at a time.
// ---------------------------------------------------------------------------
template <int BT, int FT, bool GATEUP>
__device__ __forceinline__ void stream_q4_dma_body(
    const bf16_t* __restrict__ act, const uint8_t* __restrict__ Q0,
    const float* __restrict__ S0, const uint8_t* __restrict__ Q1, const float* __restrict__ S1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_expert, int N, int K,
    int G, const int32_t* __restrict__ row_token, int nT) {
  constexpr int NW = GATEUP ? 2 : 1, NF = FT / 16, NT = BT / 16;
  constexpr int NROW = NW * FT;                 // weight rows of the block
  constexpr int kRunK = 2 * kQ4Chunk;           // K indices per run
  constexpr int kRunBytes = kRunK / 2;          // bytes of a row per run
  constexpr int kSlot = NROW * kRunBytes;       // one wave's weight slot
  constexpr int kDma = kSlot / 1024;            // 16-byte DMAs per run
  // a matrix's scales of one run: [2 groups][FT rows], padded to whole
  // 64-lane 4-byte DMAs (lanes past 2 FT load out of range, into the pad)
  constexpr int kSReg = 2 * FT < 64 ? 64 : 2 * FT;
  constexpr int kSSlot = NW * kSReg;            // one wave's scales (floats)
  constexpr int kSDma = kSReg / 64;             // 4-byte DMAs per matrix per run
  constexpr int NWAVE = kQ4Threads / kWave;
  // loads of one run: all outstanding after the next run is issued
  constexpr int kIssue = kDma + NW * kSDma + NT * 8;
  static_assert(FT % 16 == 0 && NROW % 8 == 0 && kSReg % 64 == 0 && kIssue < 64, "block shape");
  static_assert(NW * NF * NT * kWave * 16 <= kSlot, "partial sums fit a wave's slot");
  __shared__ __attribute__((aligned(1024))) char sl0[NWAVE * kSlot];
  __shared__ __attribute__((aligned(1024))) char sl1[NWAVE * kSlot];
  __shared__ __attribute__((aligned(16))) float ss0[NWAVE * kSSlot];
  __shared__ __attribute__((aligned(16))) float ss1[NWAVE * kSSlot];

  const int tile = blockIdx.y;
  const int row0 = tile * BT;
  const int lane = threadIdx.x & (kWave - 1);
  const int lr = lane & 15, kg = lane >> 4;
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
  const int cpg = G / kQ4Chunk;                       // chunks per group
  const uint32_t qrow = (uint32_t)K / 2, sgrp = (uint32_t)N * 4;
  const uint32_t sbytes = (uint32_t)(ngr - 1) * sgrp + FT * 4;
  __amdgpu_buffer_rsrc_t rw[NW], rs[NW];
  rw[0] = buffer_rsrc(Q0 + ((size_t)e * N + f0) * qrow, FT * qrow);
  rs[0] = buffer_rsrc(S0 + (size_t)e * ngr * N + f0, sbytes);
  if constexpr (GATEUP) {
    rw[1] = buffer_rsrc(Q1 + ((size_t)e * N + f0) * qrow, FT * qrow);
    rs[1] = buffer_rsrc(S1 + (size_t)e * ngr * N + f0, sbytes);
  }
  // weight DMA j: row 8 j + lane / 8 of the block (matrix (8 j) / FT)
  uint32_t dvo[kDma];
#pragma unroll
  for (int j = 0; j < kDma; ++j) {
    const int rr = 8 * j + lane / 8;
    dvo[j] = (uint32_t)(rr % FT) * qrow + (uint32_t)(((lane & 7) ^ (rr & 7)) * 16);
  }
  // scale DMA m of a matrix: float m * 64 + lane of its [2][FT] run block
  // (sq = 2 or more: padding)
  int sq[kSDma], sr[kSDma];
#pragma unroll
  for (int m = 0; m < kSDma; ++m) {
    sq[m] = (m * 64 + lane) / FT;
    sr[m] = (m * 64 + lane) % FT;
  }
  // fragment (w, f) of chunk q: row w * FT + f * 16 + lr, piece q * 4 + kg
  uint32_t fro[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
    fro[q] = (uint32_t)wave * kSlot + (uint32_t)lr * kRunBytes +
             (uint32_t)(((q * 4 + kg) ^ (lr & 7)) * 16);
  const uint32_t sro = (uint32_t)(wave * kSSlot + 4 * kg);

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
  const uint32_t arow = (uint32_t)K * 2;
  uint32_t ao[NT];
  __amdgpu_buffer_rsrc_t ra;
  if (row_token != nullptr) {
    ra = buffer_rsrc(act, (uint32_t)nT * arow);
#pragma unroll
    for (int n = 0; n < NT; ++n)
      ao[n] = (n * 16 + lr < nvalid && tok[n] >= 0) ? (uint32_t)tok[n] * arow + kg * 64
                                                     : 0x80000000u;
  } else {
    ra = buffer_rsrc(act + (size_t)row0 * K, (uint32_t)nvalid * arow);
#pragma unroll
    for (int n = 0; n < NT; ++n) ao[n] = (uint32_t)(n * 16 + lr) * arow + kg * 64;
  }

  uint4 t0[NT][2][4], t1[NT][2][4];
  // run i of this wave (clamped to its last run, so that every issue has
  // the same number of loads); a run past the last (the steady state issues
  // one; nothing reads its slot) takes offsets past the buffer ranges: it
  // loads zeros and moves no bytes
  auto issue = [&](char* slot, float* ss, uint4 (&tk)[NT][2][4], int i) {
    const bool past = i >= nb;
    const int run = wave + NWAVE * min(i, nb - 1);
    const uint32_t so = (uint32_t)run * kRunBytes;
#pragma unroll
    for (int j = 0; j < kDma; ++j) {
      lds_void* dst = (lds_void*)(slot + wave * kSlot + j * 1024);
      const uint32_t vo = past ? 0x80000000u : dvo[j];
      if (!GATEUP)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw[0], dst, 16, vo, so, 0, MOE_Q4_CPOL);
      else if ((8 * j) / FT == 0)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw[0], dst, 16, vo, so, 0, MOE_Q4_CPOL_GU0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw[NW - 1], dst, 16, vo, so, 0,
                                                 MOE_Q4_CPOL_GU1);
    }
    // the groups of the run's two chunks
    const uint32_t g0 = (uint32_t)(2 * run) / (uint32_t)cpg;
    const uint32_t g1 = (uint32_t)(2 * run + 1) / (uint32_t)cpg;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int m = 0; m < kSDma; ++m)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs[w], (lds_void*)(ss + wave * kSSlot + w * kSReg + m * 64), 4,
            (sq[m] < 2 && !past) ? (uint32_t)sr[m] * 4 + (sq[m] ? g1 : g0) * sgrp : 0x80000000u,
            0, 0, 0);
    const uint32_t ab = (uint32_t)run * (kRunK * 2);
    const uint32_t aob = past ? 0x80000000u : 0u;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          tk[n][q][j] = q4_load16(ra, (ao[n] | aob) + 16 * j, ab + q * (kQ4Chunk * 2));
  };
  const uint4 neg136 = make_uint4(kNeg136x2, kNeg136x2, kNeg136x2, kNeg136x2);
  const CodeConsts cc = CodeConsts::make();
  // the LDS reads of the run's fragments and scales first; then per chunk
  // the codes, then the MFMAs with the fragments' accumulation chains
  // interleaved (no MFMA waits on the one before it)
  auto compute = [&](const char* slot, const float* ss, const uint4 (&tk)[NT][2][4]) {
    uint4 wqs[2][NW][NF];
    f32x4 svs[2][NW][NF];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          wqs[q][w][f] =
              *reinterpret_cast<const uint4*>(slot + fro[q] + (w * FT + f * 16) * kRunBytes);
          svs[q][w][f] = *reinterpret_cast<const f32x4*>(ss + sro + w * kSReg + q * FT + f * 16);
        }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 (&wq)[NW][NF] = wqs[q];
      const f32x4 (&sv)[NW][NF] = svs[q];
      f32x4 off[NT];
      uint4 xp[NT][4];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        off[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          off[n] = Elem<bf16_t>::mfma16(neg136, tk[n][q][j], off[n]);
          xp[n][j] = pair_like_codes(tk[n][q][j]);
        }
      }
      f32x4 t[NW][NF][NT];
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int n = 0; n < NT; ++n) t[w][f][n] = off[n];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 a[NW][NF];
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int f = 0; f < NF; ++f) {
            const uint32_t word = j == 0 ? wq[w][f].x : j == 1 ? wq[w][f].y
                                : j == 2 ? wq[w][f].z : wq[w][f].w;
            a[w][f] = codes8(word, cc);
          }
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int f = 0; f < NF; ++f)
#pragma unroll
            for (int n = 0; n < NT; ++n)
              t[w][f][n] = Elem<bf16_t>::mfma16(a[w][f], xp[n][j], t[w][f][n]);
      }
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int f = 0; f < NF; ++f)
#pragma unroll
          for (int n = 0; n < NT; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[w][f][n][i] = fmaf(sv[w][f][i], t[w][f][n][i], acc[w][f][n][i]);
    }
  };
  // vmcnt(kIssue) before a compute: the run it reads has landed in LDS (the
  // only loads still outstanding are the next run's); lgkmcnt(0) after it:
  // its LDS reads are done before the slot is refilled
  constexpr int kWaitRun = (kIssue & 0xF) | ((kIssue >> 4) << 14) | 0x0F70;
  if (nb > 0) {
    issue(sl0, ss0, t0, 0);
    for (int i = 0; i < nb; i += 2) {
      issue(sl1, ss1, t1, i + 1);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitRun);
      compute(sl0, ss0, t0);
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      issue(sl0, ss0, t0, i + 2);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(kWaitRun);
      if (i + 1 < nb) compute(sl1, ss1, t1);
      __builtin_amdgcn_s_waitcnt(0xC07F);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no DMA left in flight
  }

  // cross-wave reduction in fixed order 0,1,2,3, through each wave's own
  // first slot (its DMAs have all landed and its reads are done)
  f32x4* red = reinterpret_cast<f32x4*>(sl0);
  constexpr int kRedStride = kSlot / 16;   // f32x4 per wave slot
  if (wave > 0) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int f = 0; f < NF; ++f)
#pragma unroll
        for (int n = 0; n < NT; ++n)
          red[wave * kRedStride + ((w * NF + f) * NT + n) * kWave + lane] = acc[w][f][n];
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
          for (int q = 1; q < NWAVE; ++q) a += red[q * kRedStride + ((w * NF + f) * NT + n) * kWave + lane];
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
__global__ __launch_bounds__(kQ4Threads) void stream_q4_dma_kernel(
    const bf16_t* __restrict__ act, const uint8_t* __restrict__ Q0,
    const float* __restrict__ S0, const uint8_t* __restrict__ Q1, const float* __restrict__ S1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_expert, int N, int K,
    int G, const int32_t* __restrict__ row_token, int nT) {
  stream_q4_dma_body<BT, FT, GATEUP>(act, Q0, S0, Q1, S1, outp, counts, offsets, tile_expert, N,
                                     K, G, row_token, nT);
}

// Decode shapes (16-row token tiles) are latency-bound on the weight stream:
// registers are capped so that 4 waves share each SIMD (3 with the
// post-scaled form over more than two 16-row weight fragments, whose four
// scales per fragment would otherwise spill).
#ifndef MOE_Q4_WPE16
#define MOE_Q4_WPE16 4
#endif
#ifndef MOE_Q4_WPE16_POST
#define MOE_Q4_WPE16_POST 3
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

template <int FT, bool GATEUP, int U, bool POST>
__global__ __launch_bounds__(kQ4Threads)
__attribute__((amdgpu_waves_per_eu(POST && (GATEUP ? 2 : 1) * (FT / 16) > 2 ? MOE_Q4_WPE16_POST
                                                                            : MOE_Q4_WPE16,
                                   8))) void
stream_q4_kernel16(MOE_Q4_PARAMS) {
  stream_q4_body<16, FT, GATEUP, U, POST>(MOE_Q4_ARGS);
}

template <int FT, bool GATEUP, int U, bool POST>
__global__ __launch_bounds__(kQ4Threads) void stream_q4_kernel32(MOE_Q4_PARAMS) {
  stream_q4_body<32, FT, GATEUP, U, POST>(MOE_Q4_ARGS);
}

#ifndef MOE_Q4_U
#define MOE_Q4_U 1
#endif

// the kernel for a token tile of BT rows and the group size's form
template <int BT, int FT, bool GATEUP>
static auto q4_kernel(int G) {
  const bool post = G % kQ4Chunk == 0;
  if constexpr (BT == 16)
    return post ? stream_q4_kernel16<FT, GATEUP, MOE_Q4_U, true>
                : stream_q4_kernel16<FT, GATEUP, MOE_Q4_U, false>;
  else
    return post ? stream_q4_kernel32<FT, GATEUP, MOE_Q4_U, true>
                : stream_q4_kernel32<FT, GATEUP, MOE_Q4_U, false>;
}

#ifndef MOE_Q4_FT_GU
#define MOE_Q4_FT_GU 32
#endif
#ifndef MOE_Q4_FT_DN
#define MOE_Q4_FT_DN 64
#endif
// output features per block of the LDS-staged form (wave slots of
// NW * FT * 128 bytes)
#ifndef MOE_Q4_DMA_FT_GU
#define MOE_Q4_DMA_FT_GU 32
#endif
#ifndef MOE_Q4_DMA_FT_DN
#define MOE_Q4_DMA_FT_DN 64
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
  if (D.group % kQ4Chunk == 0 && D.d % (2 * kQ4Chunk) == 0 && D.f % MOE_Q4_DMA_FT_GU == 0) {
    constexpr int FTD = MOE_Q4_DMA_FT_GU;
    stream_q4_dma_kernel<BT, FTD, true><<<dim3(D.f / FTD, D.max_tiles), kQ4Threads, 0, s>>>(
        (const bf16_t*)xs, (const uint8_t*)Wg.q, Wg.s, (const uint8_t*)Wu.q, Wu.s, h, counts,
        offsets, tile_expert, D.f, D.d, D.group, row_token, D.T);
    return;
  }
  constexpr int FT = MOE_Q4_FT_GU;
  dim3 grid(D.f / FT, D.max_tiles);
  auto kern = q4_kernel<BT, FT, true>(D.group);
  kern<<<grid, kQ4Threads, 0, s>>>((const bf16_t*)xs, (const uint8_t*)Wg.q, Wg.s,
                                   (const uint8_t*)Wu.q, Wu.s, h, counts, offsets, num_tiles,
                                   tile_expert, D.f, D.d, D.group, row_token, D.T);
}

template <int BT>
static void down_q4(const Dims& D, const void* h, const Q4Weights& Wd, float* y,
                    const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                    const int32_t* tile_expert, hipStream_t s) {
  if (D.group % kQ4Chunk == 0 && D.f % (2 * kQ4Chunk) == 0 && D.d % MOE_Q4_DMA_FT_DN == 0) {
    constexpr int FTD = MOE_Q4_DMA_FT_DN;
    stream_q4_dma_kernel<BT, FTD, false><<<dim3(D.d / FTD, D.max_tiles), kQ4Threads, 0, s>>>(
        (const bf16_t*)h, (const uint8_t*)Wd.q, Wd.s, nullptr, nullptr, y, counts, offsets,
        tile_expert, D.d, D.f, D.group, nullptr, 0);
    return;
  }
  constexpr int FT = MOE_Q4_FT_DN;
  dim3 grid(D.d / FT, D.max_tiles);
  auto kern = q4_kernel<BT, FT, false>(D.group);
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
