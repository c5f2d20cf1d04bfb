// Router (scores -> top-k -> softmax over the k), permutation (histogram ->
// prefix scan -> padded offsets -> stable row maps -> gather) and the
// gate-weighted combine of the sparse MoE layer.
//
// "Mistral/Mixtralのアーキテクチャ" (disassemble-channel.com):
//   section "Top-2ゲーティングの定式化": s = W_g x (no bias), Top-k of s,
//     gates = softmax over the selected scores only, MoE(x) = sum_j g_j E_j(x);
//   section "MoEレイヤー全体の実装": the per-expert token mask and gather,
//     and the weighted scatter-add back into a zeros_like(x) output, which is
//     done here as a gather-sum (each token reads its k expert rows).
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moe {

// ---------------------------------------------------------------------------
// Block wrapper, before the layer: RMSNorm of each token ("Mistral/Mixtral
// のアーキテクチャ", section "Mixtralのアーキテクチャ": the MoE half of a
// block normalises, applies the layer, then adds the residual):
//   rs[t] = 1 / sqrt(mean_j x[t][j]^2 + eps)      (fp32, fixed-order sum)
//   xn[t][j] = x[t][j] * rs[t] * weight[j]        (rounded to the element type)
// xn feeds the experts; the router uses x, weight and rs directly so that
// its scores are not computed from the rounded xn.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* __restrict__ x,
                                                      const float* __restrict__ weight, float eps,
                                                      int d, float* __restrict__ rs_out,
                                                      T* __restrict__ xn) {
  // 16-byte chunks of the row (d is a multiple of 64): thread tid takes
  // chunks tid, tid + 256, ... in both passes; the second re-reads them
  constexpr int V = 16 / sizeof(T);
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float wsum[4];
  __shared__ float s_rs;
  const T* xr = x + (size_t)t * d;
  const int nch = d / V;
  auto widen = [](const uint4& raw, float (&v)[V]) {
    if constexpr (V == 8) {
      const uint32_t* p = &raw.x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(p[i] << 16);
        v[2 * i + 1] = __uint_as_float(p[i] & 0xffff0000u);
      }
    } else {
      v[0] = __uint_as_float(raw.x);
      v[1] = __uint_as_float(raw.y);
      v[2] = __uint_as_float(raw.z);
      v[3] = __uint_as_float(raw.w);
    }
  };
  float ss = 0.f;
  for (int c = tid; c < nch; c += 256) {
    float v[V];
    widen(*reinterpret_cast<const uint4*>(xr + (size_t)c * V), v);
#pragma unroll
    for (int i = 0; i < V; ++i) ss = fmaf(v[i], v[i], ss);
  }
  // fixed-order reduction: lanes by xor-shuffle, then the 4 waves in order
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) wsum[wave] = ss;
  __syncthreads();
  if (tid == 0) {
    const float tot = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
    s_rs = 1.0f / sqrtf(tot / (float)d + eps);
    rs_out[t] = s_rs;
  }
  __syncthreads();
  const float r = s_rs;
  const bool w16 = reinterpret_cast<uintptr_t>(weight) % 16 == 0;
  for (int c = tid; c < nch; c += 256) {
    float v[V];
    widen(*reinterpret_cast<const uint4*>(xr + (size_t)c * V), v);
    const float* wc = weight + (size_t)c * V;
    float o[V];
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      // the weight needs only 4-byte alignment: 16-byte loads when it has it
      const float4 w = w16 ? reinterpret_cast<const float4*>(wc)[q]
                           : make_float4(wc[4 * q], wc[4 * q + 1], wc[4 * q + 2], wc[4 * q + 3]);
      o[4 * q] = v[4 * q] * r * w.x;
      o[4 * q + 1] = v[4 * q + 1] * r * w.y;
      o[4 * q + 2] = v[4 * q + 2] * r * w.z;
      o[4 * q + 3] = v[4 * q + 3] * r * w.w;
    }
    uint4 out;
    if constexpr (V == 8) {
      out = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                       pack_bf16x2(o[6], o[7]));
    } else {
      out = make_uint4(__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                       __float_as_uint(o[3]));
    }
    *reinterpret_cast<uint4*>(xn + (size_t)t * d + (size_t)c * V) = out;
  }
}

// ---------------------------------------------------------------------------
// a1: router.  One block = kRouterTokens tokens (two 16-token MFMA columns) x
// all E experts (16-expert MFMA rows, zero-padded).  Scores are an fp32 GEMM:
// A = W_router^T (expert rows), B = x^T (token columns).  bf16 tokens: each
// fp32 weight is split exactly into three bf16 pieces, each multiplied on
// v_mfma_f32_16x16x32_bf16 (bf16 products are exact in fp32); float32
// tokens: v_mfma_f32_16x16x4_f32.  K = d_model split over 8 waves in
// interleaved 32- (bf16) or 16-element groups; wave partials are added in
// fixed order.
// Top-k: one thread per token, k passes of an arg-max over E (strict '>' in
// ascending expert order, so equal scores go to the lower index).
// Softmax over the selected k, shifted by the largest selected score.
// ---------------------------------------------------------------------------
template <typename T>
__device__ inline f32x4 load4_f32(const T* p);
template <>
__device__ inline f32x4 load4_f32<float>(const float* p) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  return f32x4{v.x, v.y, v.z, v.w};
}
template <>
__device__ inline f32x4 load4_f32<bf16_t>(const bf16_t* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u),
               __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xffff0000u)};
}

// Three bf16 pieces of an fp32 value, by truncation: hi keeps its sign,
// exponent and first 8 significant bits, mid the next 8 of the exact
// remainder, lo what is left (at most 8 bits), so w = hi + mid + lo exactly
// for |w| >= 2^-110 (below that lo falls under fp32's normal range and may
// lose bits).  Returned as bf16 bit patterns.
__device__ inline void split_bf16x3(float w, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t hb = __float_as_uint(w) & 0xffff0000u;
  const float r1 = w - __uint_as_float(hb);        // exact: the low 16 bits of w
  const uint32_t mb = __float_as_uint(r1) & 0xffff0000u;
  const float r2 = r1 - __uint_as_float(mb);       // exact, at most 8 significant bits
  hi = hb >> 16;
  mid = mb >> 16;
  lo = __float_as_uint(r2) >> 16;
}

constexpr int kRouterMfmaThreads = 512;  // 8 waves split K
// k-groups per batch of loads: the groups a wave accumulates, and their
// order, do not depend on it.  Measured on MI355X: 2 takes the decode router
// 1.3 us faster than 4 (a wave there has two groups per split); prefill is
// the same for 2, 4 and 8
#ifndef MOE_ROUTER_UNROLL
#define MOE_ROUTER_UNROLL 2
#endif
constexpr int kRouterUnroll = MOE_ROUTER_UNROLL;  // k-groups whose loads are issued together


// Top-k of one token's E scores, by the kSelGroup consecutive lanes of its
// group (lane q takes experts q, q + 8, ...): k rounds of an arg-max whose
// order is the larger score, then the lower expert index, reduced over the
// group with xor-shuffles, so every lane of the group ends each round with
// the same winner.  This is the choice of k passes of a sequential scan with
// strict '>' in ascending expert order: equal scores go to the lower index.
// Then the softmax over the selected k, shifted by the largest.  Lane q
// writes slot q (q < k) and counts it in the block histogram.  Called by
// whole waves (the shuffles need every lane of a group); valid = the token
// exists.
constexpr int kSelGroup = 8;
static_assert(MOE_MAX_EXPERTS <= 8 * kSelGroup && MOE_MAX_TOPK <= kSelGroup,
              "each lane holds at most 8 experts and writes at most one slot");
__device__ inline void select_topk_group(const float* srow, int E, int k, size_t t, bool valid,
                                         int32_t* __restrict__ idx_out,
                                         float* __restrict__ w_out, int* hist,
                                         int* s_sel = nullptr) {
  const int q = threadIdx.x & (kSelGroup - 1);
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = (q + kSelGroup * i < E) ? srow[q + kSelGroup * i] : 0.f;
  uint32_t taken = 0;            // bit i: expert q + 8 i already selected
  float sel[MOE_MAX_TOPK];
  int sid[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j < k) {
      float bv = 0.f;
      int bi = -1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = q + kSelGroup * i;
        if (e < E && !((taken >> i) & 1u) && (bi < 0 || v[i] > bv)) {
          bv = v[i];
          bi = e;
        }
      }
#pragma unroll
      for (int off = 1; off < kSelGroup; off <<= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (oi >= 0 && (bi < 0 || ov > bv || (ov == bv && oi < bi))) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & (kSelGroup - 1)) == q) taken |= 1u << (bi / kSelGroup);
      sel[j] = bv;
      sid[j] = bi;
    }
  }
  float sum = 0.f, zq = 0.f;
  int eq = 0;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j)
    if (j < k) {
      const float z = expf(sel[j] - sel[0]);
      sum += z;
      if (j == q) {
        zq = z;
        eq = sid[j];
      }
    }
  if (valid && q < k) {
    idx_out[t * k + q] = eq;
    w_out[t * k + q] = zq / sum;
    atomicAdd(&hist[eq], 1);
    if (s_sel) s_sel[t * k + q] = eq;
  }
}

// Router statistics of one block (load-balancing loss: p_i is the mean over
// tokens of softmax(s_t)_i over all N experts): for each expert, the sum over
// the block's valid tokens, in token order, of the full-softmax probability.
// Called by every thread of the block (contains barriers).
__device__ inline void block_prob_sums(const float (*slog)[65], int t0, int nT, int E,
                                       float* smax, float* sinv, float* __restrict__ out_row) {
  constexpr int TB = kRouterTokens;
  const int tid = threadIdx.x;
  if (tid < TB) {
    float m = slog[tid][0];
    for (int e = 1; e < E; ++e) m = fmaxf(m, slog[tid][e]);
    float z = 0.f;
    for (int e = 0; e < E; ++e) z += expf(slog[tid][e] - m);
    smax[tid] = m;
    sinv[tid] = 1.f / z;
  }
  __syncthreads();
  if (tid < E) {
    float acc = 0.f;
    for (int t = 0; t < TB; ++t)
      if (t0 + t < nT) acc += expf(slog[t][tid] - smax[t]) * sinv[t];
    out_row[tid] = acc;
  }
}

// Scores of kRouterTokens tokens over the d_model range of split blockIdx.y
// (all of d_model when splits == 1).  splits == 1: adds the bias, selects
// and writes the routing; splits > 1: writes the partial scores to `part`
// ([split][token][kRouterPartStride]) for router_select_kernel.  MB: 16-row
// expert blocks in use, (E + 15) / 16.
template <typename T, int MB>
__global__ __launch_bounds__(kRouterMfmaThreads) void router_topk_kernel(
    const T* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ bias,
    int nT, int d, int E, int k, int splits, float* __restrict__ part,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ blk_counts,
    float* __restrict__ blk_prob, const float* __restrict__ gamma, const float* __restrict__ rs,
    float* __restrict__ logits_out) {
  constexpr int TB = kRouterTokens;
  constexpr int NB = TB / 16;            // token column blocks
  static_assert(MB >= 1 && MB * 16 <= 64, "expert row blocks");
  constexpr int NWAVE = kRouterMfmaThreads / kWave;
  constexpr int U = kRouterUnroll;
  __shared__ f32x4 red[4][MB * NB][kWave];
  __shared__ float slog[TB][65];
  __shared__ int hist[64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TB;
  const int m = lane & 15, g = lane >> 4;
  if (tid < 64) hist[tid] = 0;

  f32x4 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool tok_ok[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) tok_ok[b] = t0 + b * 16 + m < nT;
  if constexpr (std::is_same<T, bf16_t>::value) {
    // bf16 tokens: each fp32 router weight (times gamma) is split into three
    // bf16 pieces (split_bf16x3) and every piece goes through a bf16 MFMA
    // 16x16x32 with the token values as they are.  bf16 products are exact
    // in fp32, so this is the fp32 product summed in fp32, at 3 bf16 MFMAs
    // (the pieces below hi in a second accumulator) per 32 k instead of 8
    // fp32 16x16x4 ones.  K in 32-element groups; lane group g holds k
    // 8 g .. 8 g + 7 of a group.
    f32x4 acc2[MB][NB];
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc2[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bf16_t* xp[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b)
      xp[b] = x + (size_t)(tok_ok[b] ? t0 + b * 16 + m : 0) * d + 8 * g;
    const int ngroups = d / 32;                    // 32-element k-groups
    const int gps = ngroups / splits;              // k-groups of this split
    const int g0 = blockIdx.y * gps, g1 = g0 + gps;
    for (int kb = g0 + wave; kb < g1; kb += NWAVE * U) {
      uint4 bv[U][NB];
      float wv[U][MB][8];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int kg = kb + NWAVE * u;
        const bool kok = kg < g1;
        const int k0 = kg * 32 + 8 * g;            // this lane's 8 consecutive k
#pragma unroll
        for (int b = 0; b < NB; ++b)
          bv[u][b] = (kok && tok_ok[b]) ? *reinterpret_cast<const uint4*>(xp[b] + kg * 32)
                                        : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int a = 0; a < MB; ++a) {
          const int ex = a * 16 + m;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            wv[u][a][i] = (kok && ex < E) ? (gamma ? Wr[(size_t)(k0 + i) * E + ex] * gamma[k0 + i]
                                                   : Wr[(size_t)(k0 + i) * E + ex])
                                          : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int a = 0; a < MB; ++a) {
          uint32_t ph[4], pm[4], pl[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t h0, m0, l0, h1, m1, l1;
            split_bf16x3(wv[u][a][2 * i], h0, m0, l0);
            split_bf16x3(wv[u][a][2 * i + 1], h1, m1, l1);
            ph[i] = h0 | (h1 << 16);
            pm[i] = m0 | (m1 << 16);
            pl[i] = l0 | (l1 << 16);
          }
          const uint4 ah = make_uint4(ph[0], ph[1], ph[2], ph[3]);
          const uint4 am = make_uint4(pm[0], pm[1], pm[2], pm[3]);
          const uint4 al = make_uint4(pl[0], pl[1], pl[2], pl[3]);
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            acc[a][b] = Elem<bf16_t>::mfma16(ah, bv[u][b], acc[a][b]);
            acc2[a][b] = Elem<bf16_t>::mfma16(am, bv[u][b], acc2[a][b]);
            acc2[a][b] = Elem<bf16_t>::mfma16(al, bv[u][b], acc2[a][b]);
          }
        }
    }
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[a][b] += acc2[a][b];
  } else {
  const T* xp[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int t = t0 + b * 16 + m;
    xp[b] = x + (size_t)(tok_ok[b] ? t : 0) * d + 4 * g;
  }
  const int ngroups = d / 16;                      // 16-element k-groups
  const int gps = ngroups / splits;                // k-groups of this split
  const int g0 = blockIdx.y * gps, g1 = g0 + gps;
  for (int kb = g0 + wave; kb < g1; kb += NWAVE * U) {
    // U k-groups of 16: all loads first, then the MFMAs
    f32x4 bv[U][NB];
    f32x4 av[U][MB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kg = kb + NWAVE * u;
      const bool kok = kg < g1;
      const int k0 = kg * 16 + 4 * g;     // this lane's 4 consecutive k
#pragma unroll
      for (int b = 0; b < NB; ++b)
        bv[u][b] = (kok && tok_ok[b]) ? load4_f32<T>(xp[b] + kg * 16) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int a = 0; a < MB; ++a) {
        const int ex = a * 16 + m;
        av[u][a] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (kok && ex < E) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            av[u][a][i] = gamma ? Wr[(size_t)(k0 + i) * E + ex] * gamma[k0 + i]
                                : Wr[(size_t)(k0 + i) * E + ex];
        }
      }
    }
    // k-step i outermost: consecutive MFMAs go to different accumulators, so
    // none waits on the one before it (each accumulator still sees the k
    // steps in the same order)
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int a = 0; a < MB; ++a)
#pragma unroll
          for (int b = 0; b < NB; ++b)
            acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u][a][i], bv[u][b][i], acc[a][b], 0, 0, 0);
  }
  }
  // fixed-order reduction of the 8 wave partials: (w + w+4), then 0 + 1 + 2 + 3
  static_assert(NWAVE == 8, "two-phase reduction assumes 8 waves");
  if (wave >= 4) {
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) red[wave - 4][a * NB + b][lane] = acc[a][b];
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[a][b] += red[wave][a * NB + b][lane];
  }
  __syncthreads();
  if (wave >= 1 && wave < 4) {
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) red[wave - 1][a * NB + b][lane] = acc[a][b];
  }
  __syncthreads();
  if (wave == 0) {
    // D[m][n]: lane holds experts a*16 + 4*g + i of token b*16 + m
#pragma unroll
    for (int a = 0; a < MB; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        f32x4 v = acc[a][b];
#pragma unroll
        for (int q = 0; q < 3; ++q) v += red[q][a * NB + b][lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ex = a * 16 + 4 * g + i;
          if (ex < E) {
            if (splits > 1)
              part[((size_t)blockIdx.y * gridDim.x * TB + t0 + b * 16 + m) * kRouterPartStride + ex] = v[i];
            else {
              const int t = t0 + b * 16 + m;
              const float sc = (rs && t < nT) ? rs[t] : 1.f;
              slog[b * 16 + m][ex] = v[i] * sc + (bias ? bias[ex] : 0.f);
            }
          }
        }
      }
  }
  if (splits > 1) return;
  __syncthreads();
  if (logits_out)
    for (int i = tid; i < TB * E; i += kRouterMfmaThreads)
      if (t0 + i / E < nT) logits_out[(size_t)(t0 + i / E) * E + i % E] = slog[i / E][i % E];
  if (tid < TB * kSelGroup)
    select_topk_group(slog[tid / kSelGroup], E, k, (size_t)(t0 + tid / kSelGroup),
                      t0 + tid / kSelGroup < nT, idx_out, w_out, hist);
  __syncthreads();
  if (tid < E) blk_counts[(size_t)blockIdx.x * E + tid] = hist[tid];
  if (blk_prob) {
    __shared__ float smax[TB], sinv[TB];
    block_prob_sums(slog, t0, nT, E, smax, sinv, blk_prob + (size_t)blockIdx.x * E);
  }
}

__device__ __forceinline__ void expert_scan_block(
    int32_t* __restrict__ blk, int nblk, int E, int Epow2, int BT, int max_rows, int max_tiles,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ tile_expert, int32_t* __restrict__ row_token,
    int32_t* __restrict__ counts_out, int nT, const float* __restrict__ blk_prob,
    float* __restrict__ prob_out, float* __restrict__ loss_out, const ScanArgs& sa);

// Schedule of the LDS-tiled down GEMM, from the ntiles token tiles in use and
// its n_ft feature tiles: whole rounds of kCus work-groups run unsplit tiles.
// The tiles left for a partial last round, rounded up to whole token tiles
// (the last ones), are split along K into 4 parts if the pieces fit one
// round, else into 2 if those fit, which fills that round with short pieces
// instead of leaving most CUs idle.  Writes the parts in use (1: none) and
// the first row of the split token tiles.
__device__ inline void write_down_schedule(const ScanArgs& sa, int ntiles, int BT) {
  const int n_ft = sa.down_n_ft;
  int parts = 1, split_tt = ntiles;
  const int rest = (ntiles * n_ft) % kCus;
  if (rest > 0) {
    const int n_sp_tt = min(ntiles, (rest + n_ft - 1) / n_ft);
    const int n_sp = n_sp_tt * n_ft;
    if (sa.down_max_parts >= 4 && 4 * n_sp <= kCus) parts = 4;
    else if (sa.down_max_parts >= 2 && 2 * n_sp <= kCus) parts = 2;
    if (parts > 1) split_tt = ntiles - n_sp_tt;
  }
  sa.down_sched[0] = parts;
  sa.down_sched[1] = split_tt * BT;
}

// Row maps of one router block (kRouterTokens tokens), run by all
// kRouterThreads threads (contains a barrier): thread p < kRouterTokens * k
// takes pair (t0 + p / k, p % k); its rank among the block's earlier pairs on
// the same expert (wave ballots per expert plus the counts of earlier waves)
// gives row offsets[e] + base[e] + rank, so rows inside an expert segment are
// in ascending (token, slot) order.  sRow[p], sTok[p] get the row and token
// (-1 past the batch); with write_maps, tok_row and row_token are written,
// and (row_w non-NULL) the pair's gate weight w as row_w of its row.
__device__ __forceinline__ void scatter_rows_block(
    const int32_t* __restrict__ idx, const float* __restrict__ w,
    const int32_t* __restrict__ base, const int32_t* __restrict__ offsets, int nT, int E, int k,
    int t0, bool write_maps, int32_t* __restrict__ tok_row, int32_t* __restrict__ row_token,
    float* __restrict__ row_w, int* sRow, int* sTok) {
  constexpr int NWAVE = kRouterThreads / kWave;
  __shared__ int wcnt[NWAVE][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int np = kRouterTokens * k;
  int e = -1, t = -1;
  if (tid < np) {
    t = t0 + tid / k;
    if (t < nT) e = idx[(size_t)t0 * k + tid];
    else t = -1;
  }
  int rank_w = 0;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int ex = 0; ex < E; ++ex) {
    const uint64_t msk = __ballot(e == ex);
    if (e == ex) rank_w = __popcll(msk & lt);
    if (lane == 0) wcnt[wave][ex] = __popcll(msk);
  }
  __syncthreads();
  int row = -1;
  if (e >= 0) {
    int rank = rank_w;
    for (int w = 0; w < wave; ++w) rank += wcnt[w][e];
    row = offsets[e] + base[e] + rank;
    if (write_maps) {
      tok_row[(size_t)t0 * k + tid] = row;
      row_token[row] = t;
      if (row_w) row_w[row] = w[(size_t)t0 * k + tid];
    }
  }
  sRow[tid] = row;
  sTok[tid] = t;
}

// The select pass of a batch that fits one router block, run by all
// kRouterThreads threads once slog holds the final scores: top-k and
// softmax, the router statistics, the expert scan and (sa.tok_row set) the
// row maps, with the same arithmetic as select_topk_group, block_prob_sums,
// expert_scan_block and scatter_rows_block for one block.  Every value that
// a later phase needs stays in LDS and the barriers are LDS-only, so the
// outputs' global stores drain once, at the end of the kernel.
// The expert whose padded segment holds row r < off[E]: the first x with
// off[x + 1] > r (empty segments are skipped), by binary search.
__device__ inline int tile_owner(const int* off, int E, int r) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (off[mid + 1] > r) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

__device__ __forceinline__ void select_single_block(
    const float (*slog)[65], int* hist, int nT, int E, int k, int BT, int max_rows,
    int max_tiles, int32_t* __restrict__ idx_out, float* __restrict__ w_out,
    int32_t* __restrict__ blk_counts, float* __restrict__ blk_prob, const ScanArgs& sa) {
  constexpr int TB = kRouterTokens;
  constexpr int NWAVE = kRouterThreads / kWave;
  __shared__ int s_sel[TB * MOE_MAX_TOPK];
  __shared__ int s_off[65];
  __shared__ float smax[TB], sinv[TB], s_p[64];
  __shared__ int wcnt[NWAVE][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  select_topk_group(slog[tid / kSelGroup], E, k, (size_t)(tid / kSelGroup), tid / kSelGroup < nT,
                    idx_out, w_out, hist, s_sel);
  if (blk_prob && tid < TB) {            // full-softmax constants of each token
    float m = slog[tid][0];
    for (int e = 1; e < E; ++e) m = fmaxf(m, slog[tid][e]);
    float z = 0.f;
    for (int e = 0; e < E; ++e) z += expf(slog[tid][e] - m);
    smax[tid] = m;
    sinv[tid] = 1.f / z;
  }
  lds_barrier();
  // expert scan: segments padded to BT rows, offsets by wave 0 (lane =
  // expert)
  if (tid < 64) {
    const int pad = tid < E ? (hist[tid] + BT - 1) / BT * BT : 0;
    int run = pad;
#pragma unroll
    for (int st = 1; st < 64; st <<= 1) {
      const int o = __shfl_up(run, st);
      if (tid >= st) run += o;
    }
    if (tid < E) s_off[tid] = run - pad;
    if (tid == E - 1) s_off[E] = run;
  }
  if (blk_prob && tid < E) {              // p_i: the mean full-softmax probability
    float acc = 0.f;
    for (int t = 0; t < TB; ++t)
      if (t < nT) acc += expf(slog[t][tid] - smax[t]) * sinv[t];
    blk_prob[tid] = acc;
    s_p[tid] = acc / (float)nT;
    if (sa.prob_out) sa.prob_out[tid] = s_p[tid];
  }
  lds_barrier();
  if (tid < E) {
    sa.counts[tid] = hist[tid];
    if (sa.counts_out) sa.counts_out[tid] = hist[tid];
    blk_counts[tid] = 0;                  // the one block's per-expert bases
  }
  if (tid <= E) sa.offsets[tid] = s_off[tid];
  const int P = s_off[E];
  const int ntiles = P / BT;
  if (tid == 0) {
    *sa.num_tiles = ntiles;
    if (sa.down_sched) write_down_schedule(sa, ntiles, BT);
  }
  for (int i = tid; i < max_tiles; i += kRouterThreads) {
    int ex = -1;
    if (i < ntiles) ex = tile_owner(s_off, E, i * BT);
    sa.tile_expert[i] = ex;
  }
  {
    // padding rows: expert x's by its kRouterThreads / Epow2 threads
    int ep = 1;
    while (ep < E) ep <<= 1;
    const int x = tid % ep;
    if (x < E)
      for (int r = s_off[x] + hist[x] + tid / ep; r < s_off[x + 1]; r += kRouterThreads / ep)
        sa.row_token[r] = -1;
  }
  for (int r = P + tid; r < max_rows; r += kRouterThreads) sa.row_token[r] = -1;
  if (blk_prob && tid == 0 && sa.loss_out) {   // N * sum_i f_i p_i
    float L = 0.f;
    for (int x = 0; x < E; ++x) L += ((float)hist[x] / (float)nT) * s_p[x];
    *sa.loss_out = (float)E * L;
  }
  if (sa.tok_row == nullptr) return;
  // row maps: rank of pair (t, j) among the earlier pairs on its expert
  const int np = TB * k;
  int e = -1, t = -1;
  if (tid < np) {
    t = tid / k;
    if (t < nT) e = s_sel[tid];
    else t = -1;
  }
  int rank_w = 0;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int ex = 0; ex < E; ++ex) {
    const uint64_t msk = __ballot(e == ex);
    if (e == ex) rank_w = __popcll(msk & lt);
    if (lane == 0) wcnt[wave][ex] = __popcll(msk);
  }
  lds_barrier();
  if (e >= 0) {
    int rank = rank_w;
    for (int w = 0; w < wave; ++w) rank += wcnt[w][e];
    const int row = s_off[e] + rank;
    sa.tok_row[tid] = row;
    sa.row_token[row] = t;
  }
}

// Second pass of a split router: per token, the split partial scores are
// added in split order (deterministic), the bias added, then top-k/softmax.
// With a single router block (do_scan) the same block then runs the expert
// scan (a2, part 1) on the counts it has just written, which saves a launch,
// and with sa.tok_row set the row maps as well (no scatter launch).
constexpr int kSelectThreads = 256;

__global__ __launch_bounds__(kSelectThreads) void router_select_kernel(
    const float* __restrict__ part, const float* __restrict__ bias, int nT, int E, int k,
    int splits, int32_t* __restrict__ idx_out, float* __restrict__ w_out,
    int32_t* __restrict__ blk_counts, float* __restrict__ blk_prob,
    const float* __restrict__ rs, float* __restrict__ logits_out, ScanArgs sa, int do_scan,
    int Epow2, int BT, int max_rows, int max_tiles) {
  static_assert(kSelectThreads == 256 && kSelectThreads == kRouterThreads,
                "the fused expert scan and row maps run on 256 threads");
  constexpr int TB = kRouterTokens;
  __shared__ float slog[TB][65];
  __shared__ int hist[64];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * TB;
  if (tid < 64) hist[tid] = 0;
  const size_t split_stride = (size_t)gridDim.x * TB * kRouterPartStride;
  for (int i = tid; i < TB * E; i += kSelectThreads) {
    const int tt = i / E, e = i % E;
    const size_t o = (size_t)(t0 + tt) * kRouterPartStride + e;
    float p[kMaxRouterSplits];
#pragma unroll
    for (int sp = 0; sp < kMaxRouterSplits; ++sp)   // all loads in flight together
      p[sp] = sp < splits ? part[sp * split_stride + o] : 0.f;
    float v = p[0];
#pragma unroll
    for (int sp = 1; sp < kMaxRouterSplits; ++sp)   // added in split order
      if (sp < splits) v += p[sp];
    const float sc = (rs && t0 + tt < nT) ? rs[t0 + tt] : 1.f;
    slog[tt][e] = v * sc + (bias ? bias[e] : 0.f);
  }
  __syncthreads();
  if (logits_out)
    for (int i = tid; i < TB * E; i += kSelectThreads)
      if (t0 + i / E < nT) logits_out[(size_t)(t0 + i / E) * E + i % E] = slog[i / E][i % E];
  if (do_scan) {   // one router block: select, statistics, scan and row maps here
    select_single_block(slog, hist, nT, E, k, BT, max_rows, max_tiles, idx_out, w_out,
                        blk_counts, blk_prob, sa);
    return;
  }
  if (tid < TB * kSelGroup)
    select_topk_group(slog[tid / kSelGroup], E, k, (size_t)(t0 + tid / kSelGroup),
                      t0 + tid / kSelGroup < nT, idx_out, w_out, hist);
  __syncthreads();
  if (tid < E) blk_counts[(size_t)blockIdx.x * E + tid] = hist[tid];
  if (blk_prob) {
    __shared__ float smax[TB], sinv[TB];
    block_prob_sums(slog, t0, nT, E, smax, sinv, blk_prob + (size_t)blockIdx.x * E);
  }
}

// ---------------------------------------------------------------------------
// a2 (part 1): one block.  counts[e] = sum over router blocks; the per-block
// counts are rewritten in place as exclusive per-expert bases; segments are
// padded to BT rows (offsets = exclusive scan of padded counts); each token
// tile gets its expert (or -1); padding rows of row_token are set to -1.
// ---------------------------------------------------------------------------
// Run by all 256 threads of one block (contains barriers).
__device__ __forceinline__ void expert_scan_block(
    int32_t* __restrict__ blk, int nblk, int E, int Epow2, int BT, int max_rows, int max_tiles,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ num_tiles,
    int32_t* __restrict__ tile_expert, int32_t* __restrict__ row_token,
    int32_t* __restrict__ counts_out, int nT, const float* __restrict__ blk_prob,
    float* __restrict__ prob_out, float* __restrict__ loss_out, const ScanArgs& sa) {
  constexpr int kBatch = 32;                  // block counts a thread holds in flight
  __shared__ int part[256];
  __shared__ int s_cnt[64];
  __shared__ int s_off[65];
  const int tid = threadIdx.x;
  // thread (e, c) = (tid % Epow2, tid / Epow2) sums chunk c of expert e's
  // per-block counts (C chunks, no more than blocks); its exclusive base is
  // then the sum of the earlier chunks
  const int C = min(256 / Epow2, max(nblk, 1));
  const int e = tid % Epow2, c = tid / Epow2;
  const int per = (nblk + C - 1) / C;
  const int b0 = min(nblk, c * per), b1 = min(nblk, b0 + per);
  int v[kBatch];
  int sum = 0;
  if (e < E) {
    for (int b = b0; b < b1; b += kBatch) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = b + i < b1 ? blk[(size_t)(b + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) sum += v[i];
    }
  }
  // inclusive scan over the chunks of each expert (Hillis-Steele)
  int incl = sum;
  part[tid] = incl;
  __syncthreads();
  for (int st = 1; st < C; st <<= 1) {
    const int add = c >= st ? part[tid - st * Epow2] : 0;
    __syncthreads();
    incl += add;
    part[tid] = incl;
    __syncthreads();
  }
  // per-block counts rewritten in place as exclusive per-expert bases (from
  // the registers when the chunk fits one batch)
  if (e < E) {
    int run = incl - sum;
    if (per <= kBatch) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (b0 + i < b1) {
          blk[(size_t)(b0 + i) * E + e] = run;
          run += v[i];
        }
    } else {
      for (int b = b0; b < b1; ++b) {
        const int x = blk[(size_t)b * E + e];
        blk[(size_t)b * E + e] = run;
        run += x;
      }
    }
  }
  // segments padded to BT rows; offsets = exclusive scan of the padded
  // counts, by wave 0 (lane = expert)
  if (tid < 64) {
    const int cnt = tid < E ? part[(C - 1) * Epow2 + tid] : 0;
    const int pad = (cnt + BT - 1) / BT * BT;
    int run = pad;
#pragma unroll
    for (int st = 1; st < 64; st <<= 1) {
      const int o = __shfl_up(run, st);
      if (tid >= st) run += o;
    }
    if (tid < E) {
      s_cnt[tid] = cnt;
      s_off[tid] = run - pad;
    }
    if (tid == E - 1) s_off[E] = run;
  }
  __syncthreads();
  if (tid < E) {
    counts[tid] = s_cnt[tid];
    if (counts_out) counts_out[tid] = s_cnt[tid];
  }
  if (tid <= E) offsets[tid] = s_off[tid];
  const int P = s_off[E];
  const int ntiles = P / BT;
  if (tid == 0) {
    *num_tiles = ntiles;
    if (sa.down_sched) write_down_schedule(sa, ntiles, BT);
  }
  // each token tile's expert
  for (int i = tid; i < max_tiles; i += 256) {
    int ex = -1;
    if (i < ntiles) {
      ex = tile_owner(s_off, E, i * BT);
    }
    tile_expert[i] = ex;
  }
  // padding rows: expert e's by its 256 / Epow2 threads
  if (e < E)
    for (int r = s_off[e] + s_cnt[e] + c; r < s_off[e + 1]; r += 256 / Epow2) row_token[r] = -1;
  for (int r = P + tid; r < max_rows; r += 256) row_token[r] = -1;

  // router statistics (the load-balancing loss): p_i = mean full-softmax
  // probability (block sums added in block order), f_i = counts_i / T,
  // loss = N * sum_i f_i p_i
  if (blk_prob) {
    __shared__ float s_p[64];
    if (tid < E) {
      float acc = 0.f;
      for (int b = 0; b < nblk; ++b) acc += blk_prob[(size_t)b * E + tid];
      s_p[tid] = acc / (float)nT;
      if (prob_out) prob_out[tid] = s_p[tid];
    }
    __syncthreads();
    if (tid == 0 && loss_out) {
      float L = 0.f;
      for (int x = 0; x < E; ++x) L += ((float)s_cnt[x] / (float)nT) * s_p[x];
      *loss_out = (float)E * L;
    }
  }
}

__global__ __launch_bounds__(256) void expert_scan_kernel(ScanArgs a, int32_t* __restrict__ blk,
                                                          int nblk, int E, int Epow2, int BT,
                                                          int max_rows, int max_tiles, int nT,
                                                          const float* __restrict__ blk_prob) {
  expert_scan_block(blk, nblk, E, Epow2, BT, max_rows, max_tiles, a.counts, a.offsets,
                    a.num_tiles, a.tile_expert, a.row_token, a.counts_out, nT, blk_prob,
                    a.prob_out, a.loss_out, a);
}

// ---------------------------------------------------------------------------
// a2 (part 2): per router block, rank of each (token, slot) among the
// block's earlier pairs routed to the same expert (wave ballots per expert,
// plus the counts of earlier waves) -> permuted row
// offsets[e] + base[blk][e] + rank, so rows inside an expert segment are in
// ascending (token, slot) order.  Then copy x[t] to Xs[row], 16 B per lane.
// blockIdx.y splits the row copy into column slices (small T has few token
// blocks); only slice 0 writes the row maps.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(kRouterThreads) void scatter_gather_kernel(
    const T* __restrict__ x, const int32_t* __restrict__ idx, const float* __restrict__ w,
    const int32_t* __restrict__ base, const int32_t* __restrict__ offsets, int nT, int d, int E,
    int k, int32_t* __restrict__ tok_row, int32_t* __restrict__ row_token,
    float* __restrict__ row_w, T* __restrict__ xs) {
  __shared__ int sRow[kRouterThreads];
  __shared__ int sTok[kRouterThreads];
  const int t0 = blockIdx.x * kRouterTokens;
  scatter_rows_block(idx, w, base + (size_t)blockIdx.x * E, offsets, nT, E, k, t0,
                     blockIdx.y == 0, tok_row, row_token, row_w, sRow, sTok);
  if (xs == nullptr) return;               // row maps only: the GEMM gathers in place
  __syncthreads();
  const int np = kRouterTokens * k;
  const int per_chunk = 16 / (int)sizeof(T);
  const int cpr = d / per_chunk;                       // 16-byte chunks per row
  const int cps = cpr / gridDim.y;                     // chunks in this column slice
  const int c0 = blockIdx.y * cps;
  for (int i = threadIdx.x; i < np * cps; i += kRouterThreads) {
    const int p = i / cps, c = c0 + (i - p * cps);
    const int r = sRow[p];
    if (r >= 0)
      st16(xs + (size_t)r * d + c * per_chunk, ld16(x + (size_t)sTok[p] * d + c * per_chunk));
  }
}

// ---------------------------------------------------------------------------
// a5: out[t] = sum_j w[t][j] * Y[tok_row[t][j]], fp32 in slot order, one
// rounding to the output type.  A gather, so no atomics.  Rows of the token
// tiles the down GEMM split along K (down_sched) sum their K parts in part
// order.  WEIGHTED (the LDS-tiled form): the down GEMM has already applied
// the gate weights and stored bf16 rows (float32 for the later K parts), so
// the rows are only summed; else fp32 FMA of w with the float32 rows.
// ---------------------------------------------------------------------------
// V columns per lane and step: 8 (one 16-byte load of a bf16 row) in the
// weighted form, else 4 (one 16-byte load of a float32 row).  KT > 0: the
// top-k at compile time, so that the loads of all k rows are in flight
// together before the sums (in the same order as with a runtime k).
template <typename T, bool WEIGHTED>
struct CombineCols {
  static constexpr int V = WEIGHTED ? 8 : 4;
  float v[V];
  // row r's columns V c .. V c + V - 1 (the first K part)
  __device__ __forceinline__ void load(const void* y, size_t r, int d, int c) {
    if constexpr (WEIGHTED) {
      const uint4 u = reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(y) + r * d)[c];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w4[i] << 16);
        v[2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
      }
    } else {
      const float4 f = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(y) + r * d)[c];
      v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    }
  }
  // plus a later K part (float32 rows)
  __device__ __forceinline__ void add_part(const float* yp, int d, int c) {
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
      const float4 q = reinterpret_cast<const float4*>(yp)[(size_t)c * (V / 4) + h];
      v[4 * h] += q.x; v[4 * h + 1] += q.y; v[4 * h + 2] += q.z; v[4 * h + 3] += q.w;
    }
  }
};

template <typename T, bool WEIGHTED, int KT>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ y,
                                                      const float* __restrict__ y_parts,
                                                      size_t part_stride,
                                                      const int32_t* __restrict__ down_sched,
                                                      const int32_t* __restrict__ tok_row,
                                                      const float* __restrict__ w, int d, int k,
                                                      const T* __restrict__ resid,
                                                      T* __restrict__ out) {
  using Cols = CombineCols<T, WEIGHTED>;
  constexpr int V = Cols::V;
  constexpr int KB = KT > 0 ? KT : MOE_MAX_TOPK;   // rows held at once
  const int t = blockIdx.x;
  const int kk = KT > 0 ? KT : k;
  __shared__ int s_row[MOE_MAX_TOPK];
  __shared__ float s_w[MOE_MAX_TOPK];
  __shared__ int s_parts[MOE_MAX_TOPK];
  if (threadIdx.x < kk) {
    const int r = tok_row[(size_t)t * kk + threadIdx.x];
    s_row[threadIdx.x] = r;
    s_w[threadIdx.x] = w[(size_t)t * kk + threadIdx.x];
    s_parts[threadIdx.x] = (down_sched && r >= down_sched[1]) ? down_sched[0] : 1;
  }
  __syncthreads();
  const int split_row0 = down_sched ? down_sched[1] : 0;
  // blockIdx.y: column slice (small T spreads a token over several blocks)
  for (int c = blockIdx.y * 256 + threadIdx.x; c < d / V; c += 256 * gridDim.y) {
    Cols rows[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if (KT > 0 || j < kk) rows[j].load(y, (size_t)s_row[j], d, c);
    float a[V];
#pragma unroll
    for (int i = 0; i < V; ++i) a[i] = 0.f;
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (KT == 0 && j >= kk) break;
      for (int p = 1; p < s_parts[j]; ++p)   // further K parts, in part order
        rows[j].add_part(y_parts + (p - 1) * part_stride + (size_t)(s_row[j] - split_row0) * d,
                         d, c);
#pragma unroll
      for (int i = 0; i < V; ++i) {
        if constexpr (WEIGHTED) a[i] += rows[j].v[i];
        else a[i] = fmaf(s_w[j], rows[j].v[i], a[i]);
      }
    }
    T* o = out + (size_t)t * d + V * c;
    if (resid) {   // block wrapper: x + MoE(RMSNorm(x)), one rounding
      const T* xr = resid + (size_t)t * d + V * c;
#pragma unroll
      for (int i = 0; i < V; ++i) a[i] += Elem<T>::to_f32(xr[i]);
    }
    if constexpr (sizeof(T) == 2) {
      if constexpr (V == 8)
        *reinterpret_cast<uint4*>(o) = make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                                                  pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7]));
      else
        *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
    } else {
#pragma unroll
      for (int h = 0; h < V / 4; ++h)
        reinterpret_cast<float4*>(o)[h] = make_float4(a[4 * h], a[4 * h + 1], a[4 * h + 2], a[4 * h + 3]);
    }
  }
}

// ---------------------------------------------------------------------------
void launch_rmsnorm(const Dims& D, const void* x, const float* weight, float eps, float* rs,
                    void* xn, hipStream_t s) {
  if (D.bf16)
    rmsnorm_kernel<bf16_t><<<D.T, 256, 0, s>>>((const bf16_t*)x, weight, eps, D.d, rs,
                                                (bf16_t*)xn);
  else
    rmsnorm_kernel<float><<<D.T, 256, 0, s>>>((const float*)x, weight, eps, D.d, rs, (float*)xn);
}

void launch_router(const Dims& D, const void* x, const float* Wr, const float* bias,
                   int32_t* idx, float* w, int32_t* blk_counts, float* part, float* blk_prob,
                   const float* gamma, const float* rs, float* logits_out, const ScanArgs& sa,
                   hipStream_t s) {
  const dim3 grid(D.nblk, D.router_splits);
  auto run = [&](auto mb) {
    constexpr int MB = decltype(mb)::value;
    if (D.bf16)
      router_topk_kernel<bf16_t, MB><<<grid, kRouterMfmaThreads, 0, s>>>(
          (const bf16_t*)x, Wr, bias, D.T, D.d, D.E, D.k, D.router_splits, part, idx, w,
          blk_counts, blk_prob, gamma, rs, logits_out);
    else
      router_topk_kernel<float, MB><<<grid, kRouterMfmaThreads, 0, s>>>(
          (const float*)x, Wr, bias, D.T, D.d, D.E, D.k, D.router_splits, part, idx, w,
          blk_counts, blk_prob, gamma, rs, logits_out);
  };
  switch ((D.E + 15) / 16) {
    case 1: run(std::integral_constant<int, 1>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    default: run(std::integral_constant<int, 4>{}); break;
  }
  if (D.router_splits > 1)
    router_select_kernel<<<D.nblk, kSelectThreads, 0, s>>>(
        part, bias, D.T, D.E, D.k, D.router_splits, idx, w, blk_counts, blk_prob, rs, logits_out,
        sa, router_fuses_scan(D) ? 1 : 0, D.Epow2, D.BT, D.max_rows, D.max_tiles);
}

void launch_scan(const Dims& D, int32_t* blk_counts, const ScanArgs& sa, const float* blk_prob,
                 hipStream_t s) {
  if (router_fuses_scan(D)) return;   // done by the router's select block
  expert_scan_kernel<<<1, 256, 0, s>>>(sa, blk_counts, D.nblk, D.E, D.Epow2, D.BT, D.max_rows,
                                       D.max_tiles, D.T, blk_prob);
}

// Column slices until about this many blocks run: each thread's 16-byte
// copies are a dependent load and store, so more blocks keep more loads in
// flight (measured on MI355X: 256 blocks took 0.035 ms on T = 4096, top-2,
// 1024 take 0.022 ms; 2048 and 4096 are slightly slower again)
#ifndef MOE_SCATTER_MIN_BLOCKS
#define MOE_SCATTER_MIN_BLOCKS 1024
#endif
void launch_scatter(const Dims& D, const void* x, const int32_t* idx, const float* w,
                    const int32_t* blk_base, const int32_t* offsets, int32_t* tok_row,
                    int32_t* row_token, float* row_w, void* xs, hipStream_t s) {
  // column slices so that small T still spreads the copy over many blocks
  const int cpr = D.d * (D.bf16 ? 2 : 4) / 16;
  int cs = 1;
  while (D.nblk * cs < MOE_SCATTER_MIN_BLOCKS && cs * 2 <= cpr / 16 && cpr % (cs * 2) == 0)
    cs *= 2;
  const dim3 grid(D.nblk, xs ? cs : 1);
  if (D.bf16)
    scatter_gather_kernel<bf16_t><<<grid, kRouterThreads, 0, s>>>(
        (const bf16_t*)x, idx, w, blk_base, offsets, D.T, D.d, D.E, D.k, tok_row, row_token,
        row_w, (bf16_t*)xs);
  else
    scatter_gather_kernel<float><<<grid, kRouterThreads, 0, s>>>(
        (const float*)x, idx, w, blk_base, offsets, D.T, D.d, D.E, D.k, tok_row, row_token,
        row_w, (float*)xs);
}

__global__ void empty_stats_kernel(int E, int32_t* counts_out, float* prob_out,
                                   float* loss_out) {
  const int e = threadIdx.x;
  if (e < E) {
    if (counts_out) counts_out[e] = 0;
    if (prob_out) prob_out[e] = 0.f;
  }
  if (e == 0 && loss_out) *loss_out = 0.f;
}

void launch_empty_stats(int E, int32_t* counts_out, float* prob_out, float* loss_out,
                        hipStream_t s) {
  empty_stats_kernel<<<1, 64, 0, s>>>(E, counts_out, prob_out, loss_out);
}

void launch_combine(const Dims& D, const void* y, bool weighted, const float* y_parts,
                    int64_t part_rows, const int32_t* down_sched, const int32_t* tok_row,
                    const float* w, const void* resid, void* out, hipStream_t s) {
  const size_t stride = (size_t)part_rows * D.d;
  const bool w8 = D.bf16 && weighted;   // 8 columns per lane and step, else 4
  const int V = w8 ? 8 : 4;
  // column slices of 256 chunks while the tokens alone give few blocks
  int cs = 1;
  while (D.T * cs < 256 && cs * 2 * 256 * V <= D.d) cs *= 2;
  const dim3 grid(D.T, cs);
#define MOE_COMBINE(TT, WW, KK)                                                             \
  combine_kernel<TT, WW, KK><<<grid, 256, 0, s>>>(y, y_parts, stride, down_sched, tok_row, w, \
                                                  D.d, D.k, (const TT*)resid, (TT*)out)
#define MOE_COMBINE_K(TT, WW)          \
  switch (D.k) {                       \
    case 1: MOE_COMBINE(TT, WW, 1); break; \
    case 2: MOE_COMBINE(TT, WW, 2); break; \
    case 4: MOE_COMBINE(TT, WW, 4); break; \
    case 8: MOE_COMBINE(TT, WW, 8); break; \
    default: MOE_COMBINE(TT, WW, 0); break; \
  }
  if (w8) {
    MOE_COMBINE_K(bf16_t, true)
  } else if (D.bf16) {
    MOE_COMBINE_K(bf16_t, false)
  } else {
    MOE_COMBINE_K(float, false)
  }
#undef MOE_COMBINE_K
#undef MOE_COMBINE
}

}  // namespace moe
