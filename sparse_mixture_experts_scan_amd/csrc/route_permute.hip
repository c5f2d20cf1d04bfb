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
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float wsum[4];
  __shared__ float s_rs;
  const T* xr = x + (size_t)t * d;
  float ss = 0.f;
  for (int j = tid; j < d; j += 256) {
    const float v = Elem<T>::to_f32(xr[j]);
    ss = fmaf(v, v, ss);
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
  for (int j = tid; j < d; j += 256)
    xn[(size_t)t * d + j] = Elem<T>::from_f32(Elem<T>::to_f32(xr[j]) * r * weight[j]);
}

// ---------------------------------------------------------------------------
// a1: router.  One block = kRouterTokens tokens (two 16-token MFMA columns) x
// all E experts (16-expert MFMA rows, zero-padded).  Scores are an fp32 GEMM
// on v_mfma_f32_16x16x4_f32: A = W_router^T (expert rows), B = x^T (token
// columns, bf16 widened exactly), K = d_model split over 8 waves in
// interleaved 16-element groups; wave partials are added in fixed order.
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

constexpr int kRouterMfmaThreads = 512;  // 8 waves split K
// k-groups per batch of loads: the groups a wave accumulates, and their
// order, do not depend on it.  Measured on MI355X: 2 takes the decode router
// 1.3 us faster than 4 (a wave there has two groups per split); prefill is
// the same for 2, 4 and 8
#ifndef MOE_ROUTER_UNROLL
#define MOE_ROUTER_UNROLL 2
#endif
constexpr int kRouterUnroll = MOE_ROUTER_UNROLL;  // k-groups whose loads are issued together


// Top-k of one token's E scores (k passes of an arg-max, strict '>' in
// ascending expert order: equal scores go to the lower index), then the
// softmax over the selected k shifted by the largest.  Counts the choices in
// the block histogram.
__device__ inline void select_topk_token(const float* srow, int E, int k, size_t t,
                                         int32_t* __restrict__ idx_out,
                                         float* __restrict__ w_out, int* hist,
                                         int* s_sel = nullptr) {
  uint64_t taken = 0;
  float sel[MOE_MAX_TOPK];
  int sid[MOE_MAX_TOPK];
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j) {
    if (j < k) {
      float best = 0.f;
      int bi = -1;
      for (int e = 0; e < E; ++e) {
        const float v = srow[e];
        if (!((taken >> e) & 1ull) && (bi < 0 || v > best)) {
          best = v;
          bi = e;
        }
      }
      taken |= 1ull << bi;
      sel[j] = best;
      sid[j] = bi;
    }
  }
  float z[MOE_MAX_TOPK];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j)
    if (j < k) {
      z[j] = expf(sel[j] - sel[0]);
      sum += z[j];
    }
#pragma unroll
  for (int j = 0; j < MOE_MAX_TOPK; ++j)
    if (j < k) {
      idx_out[t * k + j] = sid[j];
      w_out[t * k + j] = z[j] / sum;
      atomicAdd(&hist[sid[j]], 1);
      if (s_sel) s_sel[t * k + j] = sid[j];
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
// ([split][token][kRouterPartStride]) for router_select_kernel.
template <typename T>
__global__ __launch_bounds__(kRouterMfmaThreads) void router_topk_kernel(
    const T* __restrict__ x, const float* __restrict__ Wr, const float* __restrict__ bias,
    int nT, int d, int E, int k, int splits, float* __restrict__ part,
    int32_t* __restrict__ idx_out, float* __restrict__ w_out, int32_t* __restrict__ blk_counts,
    float* __restrict__ blk_prob, const float* __restrict__ gamma, const float* __restrict__ rs,
    float* __restrict__ logits_out) {
  constexpr int TB = kRouterTokens;
  constexpr int NB = TB / 16;            // token column blocks
  constexpr int MB = 64 / 16;            // expert row blocks (max)
  constexpr int NWAVE = kRouterMfmaThreads / kWave;
  constexpr int U = kRouterUnroll;
  __shared__ f32x4 red[4][MB * NB][kWave];
  __shared__ float slog[TB][65];
  __shared__ int hist[64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TB;
  const int mb_used = (E + 15) / 16;
  const int m = lane & 15, g = lane >> 4;
  if (tid < 64) hist[tid] = 0;

  f32x4 acc[MB][NB];
#pragma unroll
  for (int a = 0; a < MB; ++a)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool tok_ok[NB];
  const T* xp[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int t = t0 + b * 16 + m;
    tok_ok[b] = t < nT;
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
        if (kok && a < mb_used && ex < E) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            av[u][a][i] = gamma ? Wr[(size_t)(k0 + i) * E + ex] * gamma[k0 + i]
                                : Wr[(size_t)(k0 + i) * E + ex];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int a = 0; a < MB; ++a)
        if (a < mb_used) {
#pragma unroll
          for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i)
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
  if (tid < TB && t0 + tid < nT)
    select_topk_token(slog[tid], E, k, (size_t)(t0 + tid), idx_out, w_out, hist);
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
    float* __restrict__ prob_out, float* __restrict__ loss_out);

// Row maps of one router block (kRouterTokens tokens), run by all
// kRouterThreads threads (contains a barrier): thread p < kRouterTokens * k
// takes pair (t0 + p / k, p % k); its rank among the block's earlier pairs on
// the same expert (wave ballots per expert plus the counts of earlier waves)
// gives row offsets[e] + base[e] + rank, so rows inside an expert segment are
// in ascending (token, slot) order.  sRow[p], sTok[p] get the row and token
// (-1 past the batch); with write_maps, tok_row and row_token are written.
__device__ __forceinline__ void scatter_rows_block(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ base,
    const int32_t* __restrict__ offsets, int nT, int E, int k, int t0, bool write_maps,
    int32_t* __restrict__ tok_row, int32_t* __restrict__ row_token, int* sRow, int* sTok) {
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
    }
  }
  sRow[tid] = row;
  sTok[tid] = t;
}

// Workgroup barrier for data exchanged through LDS only: unlike
// __syncthreads it does not wait for the block's global stores to complete.
__device__ __forceinline__ void lds_only_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The select pass of a batch that fits one router block, run by all
// kRouterThreads threads once slog holds the final scores: top-k and
// softmax, the router statistics, the expert scan and (sa.tok_row set) the
// row maps, with the same arithmetic as select_topk_token, block_prob_sums,
// expert_scan_block and scatter_rows_block for one block.  Every value that
// a later phase needs stays in LDS and the barriers are LDS-only, so the
// outputs' global stores drain once, at the end of the kernel.
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
  if (tid < nT) select_topk_token(slog[tid], E, k, (size_t)tid, idx_out, w_out, hist, s_sel);
  if (blk_prob && tid < TB) {            // full-softmax constants of each token
    float m = slog[tid][0];
    for (int e = 1; e < E; ++e) m = fmaxf(m, slog[tid][e]);
    float z = 0.f;
    for (int e = 0; e < E; ++e) z += expf(slog[tid][e] - m);
    smax[tid] = m;
    sinv[tid] = 1.f / z;
  }
  lds_only_barrier();
  // expert scan: segments padded to BT rows
  if (tid == 0) {
    int off = 0;
    for (int x = 0; x < E; ++x) {
      s_off[x] = off;
      off += (hist[x] + BT - 1) / BT * BT;
    }
    s_off[E] = off;
  }
  if (blk_prob && tid < E) {              // p_i: the mean full-softmax probability
    float acc = 0.f;
    for (int t = 0; t < TB; ++t)
      if (t < nT) acc += expf(slog[t][tid] - smax[t]) * sinv[t];
    blk_prob[tid] = acc;
    s_p[tid] = acc / (float)nT;
    if (sa.prob_out) sa.prob_out[tid] = s_p[tid];
  }
  lds_only_barrier();
  if (tid < E) {
    sa.counts[tid] = hist[tid];
    if (sa.counts_out) sa.counts_out[tid] = hist[tid];
    blk_counts[tid] = 0;                  // the one block's per-expert bases
  }
  if (tid <= E) sa.offsets[tid] = s_off[tid];
  const int P = s_off[E];
  const int ntiles = P / BT;
  if (tid == 0) *sa.num_tiles = ntiles;
  for (int i = tid; i < max_tiles; i += kRouterThreads) {
    int ex = -1;
    if (i < ntiles) {
      const int r = i * BT;
      ex = 0;
      while (s_off[ex + 1] <= r) ++ex;
    }
    sa.tile_expert[i] = ex;
  }
  for (int x = 0; x < E; ++x)
    for (int r = s_off[x] + hist[x] + tid; r < s_off[x + 1]; r += kRouterThreads)
      sa.row_token[r] = -1;
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
  lds_only_barrier();
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
// d_model splits of the score GEMM at most (measured on MI355X at decode,
// one token block: 32 splits take the router stage 1 us longer than 16)
#ifndef MOE_ROUTER_MAX_SPLITS
#define MOE_ROUTER_MAX_SPLITS 16
#endif
constexpr int kMaxRouterSplits = MOE_ROUTER_MAX_SPLITS;

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
  if (tid < TB && t0 + tid < nT)
    select_topk_token(slog[tid], E, k, (size_t)(t0 + tid), idx_out, w_out, hist);
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
    float* __restrict__ prob_out, float* __restrict__ loss_out) {
  __shared__ int part[256];
  __shared__ int s_cnt[64];
  __shared__ int s_off[65];
  const int tid = threadIdx.x;
  // block chunks scanned in parallel per expert (no more chunks than blocks:
  // one thread per expert then walks the chunks in order)
  const int C = min(256 / Epow2, max(nblk, 1));
  const int e = tid % Epow2, c = tid / Epow2;
  const int per = (nblk + C - 1) / C;
  const int b0 = min(nblk, c * per), b1 = min(nblk, b0 + per);
  int sum = 0;
  // unrolled so that the loads of a chunk are in flight together (with 64
  // experts a thread walks 32 blocks per chunk)
  if (e < E) {
#pragma unroll 8
    for (int b = b0; b < b1; ++b) sum += blk[(size_t)b * E + e];
  }
  part[tid] = sum;
  __syncthreads();
  if (tid < E) {
    int run = 0;
    for (int cc = 0; cc < C; ++cc) {
      const int v = part[cc * Epow2 + tid];
      part[cc * Epow2 + tid] = run;
      run += v;
    }
    s_cnt[tid] = run;
  }
  __syncthreads();
  if (e < E) {
    int run = part[tid];
#pragma unroll 8
    for (int b = b0; b < b1; ++b) {
      const int v = blk[(size_t)b * E + e];
      blk[(size_t)b * E + e] = run;
      run += v;
    }
  }
  if (tid == 0) {
    int off = 0;
    for (int x = 0; x < E; ++x) {
      s_off[x] = off;
      off += (s_cnt[x] + BT - 1) / BT * BT;
    }
    s_off[E] = off;
  }
  __syncthreads();
  if (tid < E) {
    counts[tid] = s_cnt[tid];
    if (counts_out) counts_out[tid] = s_cnt[tid];
  }
  if (tid <= E) offsets[tid] = s_off[tid];
  const int P = s_off[E];
  const int ntiles = P / BT;
  if (tid == 0) *num_tiles = ntiles;
  for (int i = tid; i < max_tiles; i += 256) {
    int ex = -1;
    if (i < ntiles) {
      const int r = i * BT;
      ex = 0;
      while (s_off[ex + 1] <= r) ++ex;
    }
    tile_expert[i] = ex;
  }
  for (int x = 0; x < E; ++x)
    for (int r = s_off[x] + s_cnt[x] + tid; r < s_off[x + 1]; r += 256) row_token[r] = -1;
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
                    a.prob_out, a.loss_out);
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
    const T* __restrict__ x, const int32_t* __restrict__ idx, const int32_t* __restrict__ base,
    const int32_t* __restrict__ offsets, int nT, int d, int E, int k,
    int32_t* __restrict__ tok_row, int32_t* __restrict__ row_token, T* __restrict__ xs) {
  __shared__ int sRow[kRouterThreads];
  __shared__ int sTok[kRouterThreads];
  const int t0 = blockIdx.x * kRouterTokens;
  scatter_rows_block(idx, base + (size_t)blockIdx.x * E, offsets, nT, E, k, t0, blockIdx.y == 0,
                     tok_row, row_token, sRow, sTok);
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
// a5: out[t] = sum_j w[t][j] * Y[tok_row[t][j]], fp32 FMA in slot order,
// one rounding to the output type.  A gather, so no atomics.  When the down
// GEMM was split along K, Y[r] is the sum of its partial blocks, added in
// block order before the gate weight is applied.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ tok_row,
                                                      const float* __restrict__ w, int d, int k,
                                                      int splits, size_t split_stride,
                                                      const T* __restrict__ resid,
                                                      T* __restrict__ out) {
  const int t = blockIdx.x;
  __shared__ int s_row[MOE_MAX_TOPK];
  __shared__ float s_w[MOE_MAX_TOPK];
  if (threadIdx.x < k) {
    s_row[threadIdx.x] = tok_row[(size_t)t * k + threadIdx.x];
    s_w[threadIdx.x] = w[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  // blockIdx.y: column slice (small T spreads a token over several blocks)
  for (int c = blockIdx.y * 256 + threadIdx.x; c < d / 4; c += 256 * gridDim.y) {
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      float4 v = reinterpret_cast<const float4*>(y + (size_t)s_row[j] * d)[c];
      for (int p = 1; p < splits; ++p) {   // partial K blocks, fixed order
        const float4 q = reinterpret_cast<const float4*>(y + p * split_stride + (size_t)s_row[j] * d)[c];
        v.x += q.x;
        v.y += q.y;
        v.z += q.z;
        v.w += q.w;
      }
      const float g = s_w[j];
      a.x = fmaf(g, v.x, a.x);
      a.y = fmaf(g, v.y, a.y);
      a.z = fmaf(g, v.z, a.z);
      a.w = fmaf(g, v.w, a.w);
    }
    T* o = out + (size_t)t * d + 4 * c;
    if (resid) {   // block wrapper: x + MoE(RMSNorm(x)), one rounding
      const T* xr = resid + (size_t)t * d + 4 * c;
      a.x += Elem<T>::to_f32(xr[0]);
      a.y += Elem<T>::to_f32(xr[1]);
      a.z += Elem<T>::to_f32(xr[2]);
      a.w += Elem<T>::to_f32(xr[3]);
    }
    if constexpr (sizeof(T) == 2)
      *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
    else
      *reinterpret_cast<float4*>(o) = make_float4(a.x, a.y, a.z, a.w);
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

bool router_fuses_scan(const Dims& D) { return D.nblk == 1 && D.router_splits > 1; }

void launch_router(const Dims& D, const void* x, const float* Wr, const float* bias,
                   int32_t* idx, float* w, int32_t* blk_counts, float* part, float* blk_prob,
                   const float* gamma, const float* rs, float* logits_out, const ScanArgs& sa,
                   hipStream_t s) {
  const dim3 grid(D.nblk, D.router_splits);
  if (D.bf16)
    router_topk_kernel<bf16_t><<<grid, kRouterMfmaThreads, 0, s>>>(
        (const bf16_t*)x, Wr, bias, D.T, D.d, D.E, D.k, D.router_splits, part, idx, w, blk_counts,
        blk_prob, gamma, rs, logits_out);
  else
    router_topk_kernel<float><<<grid, kRouterMfmaThreads, 0, s>>>(
        (const float*)x, Wr, bias, D.T, D.d, D.E, D.k, D.router_splits, part, idx, w, blk_counts,
        blk_prob, gamma, rs, logits_out);
  if (D.router_splits > 1)
    router_select_kernel<<<D.nblk, kSelectThreads, 0, s>>>(
        part, bias, D.T, D.E, D.k, D.router_splits, idx, w, blk_counts, blk_prob, rs, logits_out,
        sa, router_fuses_scan(D) ? 1 : 0, D.Epow2, D.BT, D.max_rows, D.max_tiles);
}

#ifndef MOE_ROUTER_MIN_BLOCKS
#define MOE_ROUTER_MIN_BLOCKS 256
#endif
int router_splits_for(int nblk, int d) {
  // split d_model over blocks until about one block per CU runs (measured on
  // MI355X: 128 blocks left T = 4096 at 0.065 ms, 256 take 0.044 ms, 512 or
  // more are slower again); each split keeps a whole number of 16-element
  // k-groups
  const int groups = d / 16;
  int sp = 1;
  while (nblk * sp < MOE_ROUTER_MIN_BLOCKS && sp * 2 <= kMaxRouterSplits &&
         groups % (sp * 2) == 0)
    sp *= 2;
  return sp;
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
void launch_scatter(const Dims& D, const void* x, const int32_t* idx, const int32_t* blk_base,
                    const int32_t* offsets, int32_t* tok_row, int32_t* row_token, void* xs,
                    hipStream_t s) {
  // column slices so that small T still spreads the copy over many blocks
  const int cpr = D.d * (D.bf16 ? 2 : 4) / 16;
  int cs = 1;
  while (D.nblk * cs < MOE_SCATTER_MIN_BLOCKS && cs * 2 <= cpr / 16 && cpr % (cs * 2) == 0)
    cs *= 2;
  const dim3 grid(D.nblk, xs ? cs : 1);
  if (D.bf16)
    scatter_gather_kernel<bf16_t><<<grid, kRouterThreads, 0, s>>>(
        (const bf16_t*)x, idx, blk_base, offsets, D.T, D.d, D.E, D.k, tok_row, row_token,
        (bf16_t*)xs);
  else
    scatter_gather_kernel<float><<<grid, kRouterThreads, 0, s>>>(
        (const float*)x, idx, blk_base, offsets, D.T, D.d, D.E, D.k, tok_row, row_token,
        (float*)xs);
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

void launch_combine(const Dims& D, const float* y, const int32_t* tok_row, const float* w,
                    const void* resid, void* out, hipStream_t s) {
  const size_t stride = (size_t)D.max_rows * D.d;
  // column slices of 256 float4 chunks while the tokens alone give few blocks
  int cs = 1;
  while (D.T * cs < 256 && cs * 2 * 256 * 4 <= D.d) cs *= 2;
  const dim3 grid(D.T, cs);
  if (D.bf16)
    combine_kernel<bf16_t><<<grid, 256, 0, s>>>(y, tok_row, w, D.d, D.k, D.down_splits, stride,
                                                (const bf16_t*)resid, (bf16_t*)out);
  else
    combine_kernel<float><<<grid, 256, 0, s>>>(y, tok_row, w, D.d, D.k, D.down_splits, stride,
                                               (const float*)resid, (float*)out);
}

}  // namespace moe
