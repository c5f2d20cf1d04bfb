// Backward pass of the sparse MoE layer: a grouped bf16 GEMM for every
// contraction the chain rule needs, and the elementwise, router and gather
// steps around them.
//
// "Mistral/Mixtralのアーキテクチャ", sections "各エキスパートの構造" (E_i(x) =
// W2 (SiLU(W1 x) * W3 x)), "Top-2ゲーティングの定式化" (gates = softmax over
// the selected scores) and "ロードバランス損失" (the training loss adds
// alpha * N * sum_i f_i p_i).  Per routed row r = (t, j) of expert e, with
// a = W1 x_t, b = W3 x_t, h = SiLU(a) * b, upstream gradient dOut_t:
//   Z = W2^T dOut_t, dg_tj = <Z, h>, dA = g Z * b * SiLU'(a), dB = g Z * SiLU(a)
//   dX_r = W1^T dA + W3^T dB
//   dW2 += (g dOut_t) h^T, dW1 += dA x_t^T, dW3 += dB x_t^T
// then the softmax over the k gates, the balance term, the router weight
// gradient and dx_t = sum_j dX_r + W_router ds_t.
//
// The grouped GEMM: C[M][N] = sum_k A[m][k] B[k][n] on 128x128 tiles, K in
// steps of 32, four waves of 64x64 (v_mfma_f32_32x32x16_bf16), both operands
// staged in LDS as [row][k] with k contiguous (the MFMA operand layout).  An
// operand whose k is contiguous in memory is copied in 16-byte pieces; one
// whose k is the slow index (a row-major matrix read down its columns) is
// transposed on its way into LDS.  Groups are either row segments of the
// permuted layout (a tile table: expert, first row, rows) with the expert's
// weights as the other operand, or experts with the contraction running over
// the expert's rows (weight gradients).  Fixed summation order throughout.
#include <type_traits>

#include <climits>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

// Tile shape: kGM x kGN outputs per workgroup, K in steps of kGK, kGWM x kGWN
// waves each holding (kGM / kGWM) x (kGN / kGWN) in 32x32 fragments.
#ifndef MOE_BG_N
#define MOE_BG_N 128
#endif
#ifndef MOE_BG_K
#define MOE_BG_K 32
#endif
#ifndef MOE_BG_WM
#define MOE_BG_WM 4
#endif
#ifndef MOE_BG_WN
#define MOE_BG_WN 2
#endif
constexpr int kGM = MOE_BG_M;
constexpr int kDxTokens = 16;                // tokens per block of the dx kernel
constexpr int kGN = MOE_BG_N;
constexpr int kGK = MOE_BG_K;
constexpr int kGWM = MOE_BG_WM, kGWN = MOE_BG_WN;
constexpr int kGT = 64 * kGWM * kGWN;        // threads
constexpr int kGLd = kGK + 8;                // LDS row pitch in elements
constexpr int kGFA = kGM / kGWM / 32;        // 32-row fragments per wave (M)
constexpr int kGFB = kGN / kGWN / 32;        // 32-column fragments per wave (N)
static_assert(kGFA >= 1 && kGFB >= 1 && kGK % 16 == 0, "tile shape");


__device__ __forceinline__ uint4 g_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ inline f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// One operand tile (ROWS rows x kGK k) of one stage, in registers between
// the global load and the LDS store.
//   KC (k contiguous): ROWS rows of 2 kGK bytes, cut into 16-byte pieces;
//     piece p = thread + i * kGT is row p / (kGK / 8), piece p % (kGK / 8).
//   KS (k slow): kGK rows of k, ROWS contiguous elements each, cut into tasks
//     of two k rows by 8 elements; task p = thread + i * kGT is k pair
//     p % (kGK / 2), elements 8 (p / (kGK / 2)) .. +8; it stores eight
//     (k, k+1) pairs into eight LDS rows.
template <bool KC, int ROWS>
struct GOperand {
  static constexpr int TASKS = KC ? ROWS * kGK / 8 : (kGK / 2) * (ROWS / 8);
  static constexpr int PIECES = (TASKS + kGT - 1) / kGT;
  static constexpr bool EVEN = TASKS % kGT == 0;   // else the last round is partial
  uint4 v0[PIECES], v1[KC ? 1 : PIECES];
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t ld_bytes, int k0,
                                       int col0, int tid) {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = tid + i * kGT;
      if (!EVEN && p >= TASKS) break;
      if constexpr (KC) {
        const int row = p / (kGK / 8), piece = p % (kGK / 8);
        v0[i] = g_load16(r, (uint32_t)row * ld_bytes + (uint32_t)(k0 + piece * 8) * 2);
      } else {
        const int k = k0 + 2 * (p % (kGK / 2)), c8 = p / (kGK / 2);
        const uint32_t off = (uint32_t)k * ld_bytes + (uint32_t)(col0 + c8 * 8) * 2;
        v0[i] = g_load16(r, off);
        v1[i] = g_load16(r, off + ld_bytes);
      }
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PIECES; ++i) {
      const int p = tid + i * kGT;
      if (!EVEN && p >= TASKS) break;
      if constexpr (KC) {
        const int row = p / (kGK / 8), piece = p % (kGK / 8);
        *reinterpret_cast<uint4*>(lds + row * kGLd + piece * 8) = v0[i];
      } else {
        const int kk = 2 * (p % (kGK / 2)), c8 = p / (kGK / 2);
        const uint32_t a[4] = {v0[i].x, v0[i].y, v0[i].z, v0[i].w};
        const uint32_t b[4] = {v1[i].x, v1[i].y, v1[i].z, v1[i].w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t lo = (a[w] & 0xFFFFu) | (b[w] << 16);          // element 2w
          const uint32_t hi = (a[w] >> 16) | (b[w] & 0xFFFF0000u);      // element 2w + 1
          *reinterpret_cast<uint32_t*>(lds + (c8 * 8 + 2 * w) * kGLd + kk) = lo;
          *reinterpret_cast<uint32_t*>(lds + (c8 * 8 + 2 * w + 1) * kGLd + kk) = hi;
        }
      }
    }
  }
};

}  // namespace

// Grouped GEMM.  mode 0 (row segments): tile i of the table covers rows
// tb_row0[i] .. + tb_rows[i] of A and C, which belong to expert tb_exp[i];
// B is that expert's matrix (B + e * b_estride).  mode 1 (weight gradients):
// blockIdx.z = expert e, the contraction runs over rows offsets[e] ..
// offsets[e] + counts[e] of A and B (both k-slow), C = C + e * c_estride.
// A: k-contiguous (KCA) rows of lda elements, or k-slow rows of k.  B:
// k-contiguous rows of N (one row per output column) or k-slow rows of k.
// C: float (accumulate: C += result) or bf16, row pitch ldc.
template <bool KCA, bool KCB, int MODE, bool CBF16>
__global__ __launch_bounds__(kGT) void grouped_gemm_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ B, int ldb,
    size_t b_estride, void* __restrict__ C, int ldc, size_t c_estride, int M, int N, int K,
    bool accumulate, const int32_t* __restrict__ tb_count, const int32_t* __restrict__ tb_exp,
    const int32_t* __restrict__ tb_row0, const int32_t* __restrict__ tb_rows,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets) {
  __shared__ __attribute__((aligned(16))) bf16_t lA[2][kGM * kGLd];
  __shared__ __attribute__((aligned(16))) bf16_t lB[2][kGN * kGLd];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % kGWM, wn = wave / kGWM;
  const int n0 = blockIdx.x * kGN;

  int m0, rows, kn;
  __amdgpu_buffer_rsrc_t ra, rb;
  size_t c_base;
  if constexpr (MODE == 0) {
    const int i = blockIdx.y;
    if (i >= *tb_count) return;
    const int e = tb_exp[i];
    m0 = tb_row0[i];
    rows = tb_rows[i];
    kn = K;
    // A: rows m0 .. m0 + rows (k contiguous), past them zeros
    ra = buffer_rsrc(A + (size_t)m0 * lda, (uint32_t)rows * lda * 2);
    const bf16_t* Be = B + (size_t)e * b_estride;
    // (columns past N read as zeros or as a neighbour's data; never stored)
    if constexpr (KCB) rb = buffer_rsrc(Be + (size_t)n0 * ldb, (uint32_t)min(kGN, N - n0) * ldb * 2);
    else rb = buffer_rsrc(Be, (uint32_t)K * ldb * 2);
    c_base = (size_t)m0 * ldc;
  } else {
    const int e = blockIdx.z;
    m0 = blockIdx.y * kGM;
    rows = kGM;
    kn = counts[e];
    const int r0 = offsets[e];
    ra = buffer_rsrc(A + (size_t)r0 * lda, (uint32_t)kn * lda * 2);
    rb = buffer_rsrc(B + (size_t)r0 * ldb, (uint32_t)kn * ldb * 2);
    c_base = (size_t)e * c_estride + (size_t)m0 * ldc;
  }
  const uint32_t lda_b = (uint32_t)lda * 2, ldb_b = (uint32_t)ldb * 2;
  // A tile origin: k-contiguous rows start at m0 (already in the resource for
  // mode 0); k-slow columns start at m0
  const int a_col0 = KCA ? 0 : m0;
  const int b_col0 = KCB ? 0 : n0;

  f32x16 acc[kGFA][kGFB];
#pragma unroll
  for (int a = 0; a < kGFA; ++a)
#pragma unroll
    for (int b = 0; b < kGFB; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.f;

  GOperand<KCA, kGM> ga;
  GOperand<KCB, kGN> gb;
  const int nk = (kn + kGK - 1) / kGK;
  if (nk > 0) {
    ga.load(ra, lda_b, 0, a_col0, tid);
    gb.load(rb, ldb_b, 0, b_col0, tid);
    ga.store(lA[0], tid);
    gb.store(lB[0], tid);
  }
  __syncthreads();
  const int r32 = lane & 31, half = lane >> 5;
  const int arow0 = wm * (kGM / kGWM), brow0 = wn * (kGN / kGWN);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      ga.load(ra, lda_b, (kt + 1) * kGK, a_col0, tid);
      gb.load(rb, ldb_b, (kt + 1) * kGK, b_col0, tid);
    }
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      uint4 af[kGFA], bf[kGFB];
#pragma unroll
      for (int a = 0; a < kGFA; ++a)
        af[a] = *reinterpret_cast<const uint4*>(&lA[cur][(arow0 + a * 32 + r32) * kGLd +
                                                          ks * 16 + half * 8]);
#pragma unroll
      for (int b = 0; b < kGFB; ++b)
        bf[b] = *reinterpret_cast<const uint4*>(&lB[cur][(brow0 + b * 32 + r32) * kGLd +
                                                          ks * 16 + half * 8]);
#pragma unroll
      for (int a = 0; a < kGFA; ++a)
#pragma unroll
        for (int b = 0; b < kGFB; ++b) acc[a][b] = mfma32(af[a], bf[b], acc[a][b]);
    }
    if (kt + 1 < nk) {
      ga.store(lA[cur ^ 1], tid);
      gb.store(lB[cur ^ 1], tid);
    }
    __syncthreads();
  }

  // D of a 32x32 MFMA: lane holds column n = lane % 32 and rows
  // 8 * (j / 4) + 4 * (lane / 32) + j % 4.
#pragma unroll
  for (int a = 0; a < kGFA; ++a)
#pragma unroll
    for (int b = 0; b < kGFB; ++b) {
      const int n = n0 + brow0 + b * 32 + r32;
      if (n >= N) continue;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int m = arow0 + a * 32 + 8 * (j >> 2) + 4 * half + (j & 3);
        if (m >= rows || m0 + m >= M) continue;
        const size_t idx = c_base + (size_t)m * ldc + n;
        if constexpr (CBF16) {
          reinterpret_cast<bf16_t*>(C)[idx] = Elem<bf16_t>::from_f32(acc[a][b][j]);
        } else {
          float* c = reinterpret_cast<float*>(C) + idx;
          *c = accumulate ? *c + acc[a][b][j] : acc[a][b][j];
        }
      }
    }
}

// Tile table of mode 0: expert segments in order, each cut into kGM-row
// tiles.  One thread (the table is at most E + rows / kGM long).  Then the
// tiled dX GEMM's schedule (n_at feature tiles; two K halves per tile): the
// tiles of a partial last round of kCus work-groups, rounded up to whole
// token tiles (the last ones), run as four K quarters each if those fit the
// round and at most max_split token tiles are involved; sched = {split token
// tiles (0: none), first row of the first of them}.
__global__ void bwd_tile_table_kernel(const int32_t* __restrict__ counts,
                                      const int32_t* __restrict__ offsets, int E, int max_tiles,
                                      int n_at, int max_split, int parts,
                                      int32_t* __restrict__ tb_count,
                                      int32_t* __restrict__ tb_exp,
                                      int32_t* __restrict__ tb_row0,
                                      int32_t* __restrict__ tb_rows,
                                      int32_t* __restrict__ sched) {
  if (threadIdx.x != 0) return;
  int n = 0;
  for (int e = 0; e < E; ++e) {
    for (int r = 0; r < counts[e] && n < max_tiles; r += kGM, ++n) {
      tb_exp[n] = e;
      tb_row0[n] = offsets[e] + r;
      tb_rows[n] = min(kGM, counts[e] - r);
    }
  }
  *tb_count = n;
  // dX schedule: the last sp token tiles run each K part as two halves, so
  // that the pieces fill the last round of the CUs
  int sp = 0;
  const int rest = (parts * n * n_at) % kCus;
  if (rest > 0 && n_at > 0) {
    sp = min(n, (rest + parts * n_at - 1) / (parts * n_at));
    if (sp > max_split || 2 * parts * sp * n_at > kCus) sp = 0;
  }
  sched[0] = sp;
  sched[1] = sp > 0 ? tb_row0[n - sp] : 0;
}

// Permuted copy of the upstream gradient: Dp[r] = dOut[token of r], zero
// rows for padding.
__global__ __launch_bounds__(256) void bwd_gather_kernel(const bf16_t* __restrict__ src,
                                                         const int32_t* __restrict__ row_token,
                                                         int d, bf16_t* __restrict__ dst) {
  const int r = blockIdx.x;
  const int t = row_token[r];
  uint4* out = reinterpret_cast<uint4*>(dst + (size_t)r * d);
  const uint4* in = reinterpret_cast<const uint4*>(src + (size_t)(t < 0 ? 0 : t) * d);
  for (int c = threadIdx.x; c < d / 8; c += 256) out[c] = t < 0 ? make_uint4(0, 0, 0, 0) : in[c];
}

// Per permuted row: a, b (pre-activations from the recompute GEMMs) and
// Z = W2^T dOut_t, all bf16 (fp32 products rounded once).  dg[r] = <Z, h> (fixed-order block sum), dAB[r] = [g Z b
// SiLU'(a) | g Z SiLU(a)] and Hg[r] = g h (bf16), zeros on padding rows.
__global__ __launch_bounds__(256) void bwd_rows_kernel(
    const bf16_t* __restrict__ AB, const bf16_t* __restrict__ Z, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ tok_row, const float* __restrict__ gates, int f, int k,
    float* __restrict__ dg, bf16_t* __restrict__ dAB, bf16_t* __restrict__ Hg) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const int t = row_token[r];
  __shared__ float wsum[4];
  float g = 0.f;
  if (t >= 0)
    for (int j = 0; j < k; ++j)
      if (tok_row[(size_t)t * k + j] == r) g = gates[(size_t)t * k + j];
  const bf16_t* a_row = AB + (size_t)r * 2 * f;
  const bf16_t* b_row = a_row + f;
  const bf16_t* z_row = Z + (size_t)r * f;
  bf16_t* da_row = dAB + (size_t)r * 2 * f;
  bf16_t* db_row = da_row + f;
  bf16_t* hg_row = Hg + (size_t)r * f;
  float part = 0.f;
  // 8 consecutive columns per thread and step (f is a multiple of 64)
  for (int c = tid * 8; c < f; c += 256 * 8) {
    uint4 da = make_uint4(0, 0, 0, 0), db = da, hv = da;
    if (t >= 0) {
      const uint4 av = *reinterpret_cast<const uint4*>(a_row + c);
      const uint4 bv = *reinterpret_cast<const uint4*>(b_row + c);
      const uint4 zv = *reinterpret_cast<const uint4*>(z_row + c);
      const uint32_t* ap = &av.x;
      const uint32_t* bp = &bv.x;
      const uint32_t* zp = &zv.x;
      uint32_t* dap = &da.x;
      uint32_t* dbp = &db.x;
      uint32_t* hp = &hv.x;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t oa = 0, ob = 0, oh = 0;
#pragma unroll
        for (int hgh = 0; hgh < 2; ++hgh) {
          const float a = __uint_as_float((ap[i] >> (16 * hgh)) << 16);
          const float b = __uint_as_float((bp[i] >> (16 * hgh)) << 16);
          const float z = __uint_as_float((zp[i] >> (16 * hgh)) << 16);
          const float sig = 1.0f / (1.0f + expf(-a));
          const float sv = a * sig;
          const float h = sv * b;
          part = fmaf(z, h, part);
          const float dh = g * z;
          const float dav = dh * b * (sig * (1.0f + a * (1.0f - sig)));
          const float dbv = dh * sv;
          const float hgv = g * h;
          oa |= (uint32_t)Elem<bf16_t>::from_f32(dav) << (16 * hgh);
          ob |= (uint32_t)Elem<bf16_t>::from_f32(dbv) << (16 * hgh);
          oh |= (uint32_t)Elem<bf16_t>::from_f32(hgv) << (16 * hgh);
        }
        dap[i] = oa;
        dbp[i] = ob;
        hp[i] = oh;
      }
    }
    *reinterpret_cast<uint4*>(da_row + c) = da;
    *reinterpret_cast<uint4*>(db_row + c) = db;
    *reinterpret_cast<uint4*>(hg_row + c) = hv;
  }
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = part;
  __syncthreads();
  if (tid == 0) dg[r] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// Per token: ds_t over all E experts.  Selected experts: the softmax over the
// k gates, ds = g (dg - sum_l g_l dg_l); with alpha > 0 the balance term
// (alpha N / T) P_tm (f_m - sum_i f_i P_ti), P the full softmax of the scores.
__global__ __launch_bounds__(256) void bwd_router_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ gates, const int32_t* __restrict__ tok_row,
    const float* __restrict__ dg_row, const int32_t* __restrict__ counts, int T, int E, int k,
    float alpha, float* __restrict__ ds) {
  // one wave per token, lane e = expert e (E <= 64)
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int e = threadIdx.x & 63;
  if (t >= T) return;
  float sum = 0.f;                          // sum_j g_j dg_j, slot order (same in every lane)
  for (int j = 0; j < k; ++j)
    sum += gates[(size_t)t * k + j] * dg_row[tok_row[(size_t)t * k + j]];
  float v = 0.f;
  for (int j = 0; j < k; ++j)
    if (idx[(size_t)t * k + j] == e)
      v = gates[(size_t)t * k + j] * (dg_row[tok_row[(size_t)t * k + j]] - sum);
  if (alpha != 0.f) {
    // alpha N / T with f = counts / T; full-softmax p by wave reductions
    const float scale = alpha * (float)E / ((float)T * (float)T);
    const float se = e < E ? logits[(size_t)t * E + e] : -INFINITY;
    float m = se;
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    const float ex = e < E ? expf(se - m) : 0.f;
    float z = ex;
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
    const float inv = 1.f / z;
    const float p = ex * inv;
    float pc = e < E ? p * (float)counts[e] : 0.f;
    for (int off = 32; off > 0; off >>= 1) pc += __shfl_xor(pc, off);
    v += scale * p * ((e < E ? (float)counts[e] : 0.f) - pc);
  }
  if (e < E) ds[(size_t)t * E + e] = v;
}

// Router weight gradient, partial over a slice of tokens: part[s][j][e] =
// sum over tokens of slice s (in order) of x[t][j] ds[t][e]; and the bias
// gradient part (column j = d).  Thread per column j, every expert's sum in
// registers; the slice's ds rows are staged in LDS, kWgradChunk tokens at a
// time, and read as broadcasts.
constexpr int kWgradChunk = 128;       // tokens of a slice staged in LDS at once
constexpr int kWgradLoads = 32;        // tokens whose x loads a thread issues together
constexpr int kWgrad8Loads = 8;        // the same for the eight-column form (16-byte loads)
template <typename T, int EB>
__global__ __launch_bounds__(256) void bwd_router_wgrad_kernel(
    const T* __restrict__ x, const float* __restrict__ ds, int Tn, int d, int E, int tslice,
    float* __restrict__ part) {
  __shared__ float sds[kWgradChunk][EB];
  const int j = blockIdx.x * 256 + threadIdx.x;
  const int s = blockIdx.y;
  const int t0 = s * tslice, t1 = min(Tn, t0 + tslice);
  // all EB (>= E; zeros past E) accumulators at once, so x is read once
  float acc[EB];
#pragma unroll
  for (int q = 0; q < EB; ++q) acc[q] = 0.f;
  for (int c0 = t0; c0 < t1; c0 += kWgradChunk) {
    const int c1 = min(t1, c0 + kWgradChunk);
    __syncthreads();
    for (int i = threadIdx.x; i < (c1 - c0) * EB; i += 256) {
      const int t = c0 + i / EB, e = i % EB;
      sds[i / EB][e] = e < E ? ds[(size_t)t * E + e] : 0.f;
    }
    __syncthreads();
    if (j <= d) {
      // kWgradLoads tokens' x loads in flight together, then their FMAs in
      // token order (each accumulator still adds the tokens in order)
      auto fma_row = [&](float xv, int t) {
        const float4* row = reinterpret_cast<const float4*>(sds[t - c0]);
#pragma unroll
        for (int q4 = 0; q4 < EB / 4; ++q4) {
          const float4 v = row[q4];
          acc[4 * q4] = fmaf(xv, v.x, acc[4 * q4]);
          acc[4 * q4 + 1] = fmaf(xv, v.y, acc[4 * q4 + 1]);
          acc[4 * q4 + 2] = fmaf(xv, v.z, acc[4 * q4 + 2]);
          acc[4 * q4 + 3] = fmaf(xv, v.w, acc[4 * q4 + 3]);
        }
      };
      int t = c0;
      for (; t + kWgradLoads <= c1; t += kWgradLoads) {
        float xv[kWgradLoads];
#pragma unroll
        for (int u = 0; u < kWgradLoads; ++u)
          xv[u] = j < d ? Elem<T>::to_f32(x[(size_t)(t + u) * d + j]) : 1.0f;
#pragma unroll
        for (int u = 0; u < kWgradLoads; ++u) fma_row(xv[u], t + u);
      }
      for (; t < c1; ++t) fma_row(j < d ? Elem<T>::to_f32(x[(size_t)t * d + j]) : 1.0f, t);
    }
  }
  if (j <= d) {
    float* prow = part + ((size_t)s * (d + 1) + j) * E;
    if (E % 4 == 0 && reinterpret_cast<uintptr_t>(part) % 16 == 0) {
      // 16-byte stores of the row's E partial sums
#pragma unroll
      for (int q4 = 0; q4 < EB / 4; ++q4)
        if (4 * q4 < E)
          *reinterpret_cast<float4*>(prow + 4 * q4) =
              make_float4(acc[4 * q4], acc[4 * q4 + 1], acc[4 * q4 + 2], acc[4 * q4 + 3]);
    } else {
#pragma unroll
      for (int q = 0; q < EB; ++q)
        if (q < E) prow[q] = acc[q];
    }
  }
}

// The same partial sums for few experts (EB <= 16), eight consecutive
// columns per thread: one 16-byte load of x per token, 8 x EB accumulators.
// Chunk c = d / 8 is the bias column (x = 1) alone.  Same token order for
// every sum as bwd_router_wgrad_kernel, so the same results.
template <int EB>
__global__ __launch_bounds__(64) void bwd_router_wgrad8_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ ds, int Tn, int d, int E, int tslice,
    float* __restrict__ part) {
  __shared__ float sds[kWgradChunk][EB];
  const int c = blockIdx.x * 64 + threadIdx.x;   // 8-column chunk; d / 8 = the bias
  const int nch = d / 8;
  const int s = blockIdx.y;
  const int t0 = s * tslice, t1 = min(Tn, t0 + tslice);
  float acc[8][EB];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int q = 0; q < EB; ++q) acc[i][q] = 0.f;
  for (int c0 = t0; c0 < t1; c0 += kWgradChunk) {
    const int c1 = min(t1, c0 + kWgradChunk);
    __syncthreads();
    for (int i = threadIdx.x; i < (c1 - c0) * EB; i += 64) {
      const int t = c0 + i / EB, e = i % EB;
      sds[i / EB][e] = e < E ? ds[(size_t)t * E + e] : 0.f;
    }
    __syncthreads();
    if (c <= nch) {
      auto fma_row = [&](const uint4& xv, int t) {
        float xf[8];
        if (c < nch) {
          const uint32_t* p = &xv.x;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            xf[2 * i] = __uint_as_float(p[i] << 16);
            xf[2 * i + 1] = __uint_as_float(p[i] & 0xffff0000u);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) xf[i] = i == 0 ? 1.0f : 0.f;
        }
        const float4* row = reinterpret_cast<const float4*>(sds[t - c0]);
#pragma unroll
        for (int q4 = 0; q4 < EB / 4; ++q4) {
          const float4 v = row[q4];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            acc[i][4 * q4] = fmaf(xf[i], v.x, acc[i][4 * q4]);
            acc[i][4 * q4 + 1] = fmaf(xf[i], v.y, acc[i][4 * q4 + 1]);
            acc[i][4 * q4 + 2] = fmaf(xf[i], v.z, acc[i][4 * q4 + 2]);
            acc[i][4 * q4 + 3] = fmaf(xf[i], v.w, acc[i][4 * q4 + 3]);
          }
        }
      };
      int t = c0;
      for (; t + kWgrad8Loads <= c1; t += kWgrad8Loads) {
        uint4 xv[kWgrad8Loads];
#pragma unroll
        for (int u = 0; u < kWgrad8Loads; ++u)
          xv[u] = c < nch ? *reinterpret_cast<const uint4*>(x + (size_t)(t + u) * d + 8 * c)
                          : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kWgrad8Loads; ++u) fma_row(xv[u], t + u);
      }
      for (; t < c1; ++t)
        fma_row(c < nch ? *reinterpret_cast<const uint4*>(x + (size_t)t * d + 8 * c)
                        : make_uint4(0, 0, 0, 0), t);
    }
  }
  if (c < nch) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float* prow = part + ((size_t)s * (d + 1) + 8 * c + i) * E;
#pragma unroll
      for (int q = 0; q < EB; ++q)
        if (q < E) prow[q] = acc[i][q];
    }
  } else if (c == nch) {
    float* prow = part + ((size_t)s * (d + 1) + d) * E;
#pragma unroll
    for (int q = 0; q < EB; ++q)
      if (q < E) prow[q] = acc[0][q];
  }
}

__global__ __launch_bounds__(256) void bwd_router_wgrad_reduce(const float* __restrict__ part,
                                                               int slices, int d, int E,
                                                               float* __restrict__ dWr,
                                                               float* __restrict__ dbias) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= (d + 1) * E) return;
  float acc = 0.f;
  for (int s = 0; s < slices; ++s) acc += part[(size_t)s * (d + 1) * E + i];
  if (i < d * E) dWr[i] = acc;
  else if (dbias) dbias[i - d * E] = acc;
}

// dx_t = sum_j dX[tok_row[t][j]] (slot order) + sum_e W_router[.][e] ds_t[e]
template <typename T, int EB>
__global__ __launch_bounds__(256) void bwd_dx_kernel(int nplanes, const float* __restrict__ dX,
                                                     size_t plane,
                                                     const float* __restrict__ dX_extra,
                                                     size_t extra_plane,
                                                     const int32_t* __restrict__ sched,
                                                     const int32_t* __restrict__ tok_row,
                                                     const float* __restrict__ Wr,
                                                     const float* __restrict__ ds, int nT, int d,
                                                     int E, int k, T* __restrict__ dx) {
  // block: kDxTokens tokens x 256 columns; thread: one column, its E router
  // weights held in registers across the tokens (EB >= E of them, zeros past
  // E, which add exact zeros)
  __shared__ float sds[kDxTokens][EB];
  __shared__ int srow[kDxTokens][MOE_MAX_TOPK];
  const int t0 = blockIdx.x * kDxTokens, tid = threadIdx.x;
  for (int i = tid; i < kDxTokens * EB; i += 256) {
    const int t = t0 + i / EB, e = i % EB;
    sds[i / EB][e] = (t < nT && e < E) ? ds[(size_t)t * E + e] : 0.f;
  }
  for (int i = tid; i < kDxTokens * k; i += 256) {
    const int t = t0 + i / k;
    srow[i / k][i % k] = t < nT ? tok_row[(size_t)t * k + i % k] : 0;
  }
  const int c = blockIdx.y * 256 + tid;
  const int cc = min(c, d - 1);             // lanes past d load a valid column, unused
  // the column's E router weights (contiguous in W_router [d][E]): 16-byte
  // loads when rows are 16-byte aligned, so that a wave touches each of its
  // 64 rows' lines once per 4 experts rather than once per expert
  float wr[EB];
  if (E % 4 == 0 && reinterpret_cast<uintptr_t>(Wr) % 16 == 0) {
    const float4* wrow = reinterpret_cast<const float4*>(Wr + (size_t)cc * E);
#pragma unroll
    for (int j = 0; j < EB / 4; ++j) {
      const float4 v = 4 * j < E ? wrow[j] : make_float4(0.f, 0.f, 0.f, 0.f);
      wr[4 * j] = v.x;
      wr[4 * j + 1] = v.y;
      wr[4 * j + 2] = v.z;
      wr[4 * j + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < EB; ++e) wr[e] = e < E ? Wr[(size_t)cc * E + e] : 0.f;
  }
  __syncthreads();
  if (c >= d) return;
  // rows of split token tiles (from sched[1] on) add their second quarters
  const int split_row0 = (sched && sched[0] > 0) ? sched[1] : INT_MAX;
  const int nt = min(kDxTokens, nT - t0);
  // the row loads of token i: its planes (and a split row's extra planes),
  // all issued before any is used; a plane not in use reads as zero
  const bool two = nplanes > 1;
  auto load = [&](int i, float (&v)[MOE_MAX_TOPK][4]) {
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j) {
      if (j < k) {
        const int r = srow[i][j];
        const size_t o = (size_t)r * d + c;
        v[j][0] = dX[o];
        v[j][1] = two ? dX[plane + o] : 0.f;
        v[j][2] = v[j][3] = 0.f;
        if (r >= split_row0) {
          const size_t oe = (size_t)(r - split_row0) * d + c;
          v[j][2] = dX_extra[oe];
          if (two) v[j][3] = dX_extra[extra_plane + oe];
        }
      }
    }
  };
  // the slot-order sum plus W_router . ds in expert order
  auto finish = [&](int i, const float (&v)[MOE_MAX_TOPK][4]) {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < MOE_MAX_TOPK; ++j)
      if (j < k) acc += (srow[i][j] >= split_row0) ? (v[j][0] + v[j][2]) + (v[j][1] + v[j][3])
                                                   : v[j][0] + v[j][1];
    float rt = 0.f;
#pragma unroll
    for (int e = 0; e < EB; ++e) rt = fmaf(wr[e], sds[i][e], rt);
    dx[(size_t)(t0 + i) * d + c] = Elem<T>::from_f32(acc + rt);
  };
  // two tokens' loads in flight at a time
  float va[MOE_MAX_TOPK][4], vb[MOE_MAX_TOPK][4];
  int i = 0;
  for (; i + 1 < nt; i += 2) {
    load(i, va);
    load(i + 1, vb);
    finish(i, va);
    finish(i + 1, vb);
  }
  if (i < nt) {
    load(i, va);
    finish(i, va);
  }
}

__global__ __launch_bounds__(256) void zero_fill_kernel(uint4* __restrict__ p, size_t n16,
                                                        uint8_t* __restrict__ tail, int ntail) {
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n16; i += (size_t)gridDim.x * 256)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

// ---------------------------------------------------------------- launchers
void launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  if (!p || bytes == 0) return;
  const size_t n16 = bytes / 16;
  const size_t want = (n16 + 255) / 256;
  const unsigned grid = (unsigned)(want < 4096 ? (want > 0 ? want : 1) : 4096);
  zero_fill_kernel<<<grid, 256, 0, s>>>((uint4*)p, n16, (uint8_t*)p + n16 * 16,
                                        (int)(bytes - n16 * 16));
}



void launch_bwd_tile_table(const Dims& D, const int32_t* counts, const int32_t* offsets,
                           int max_tiles, int max_split, int dx_parts, int32_t* tb_count,
                           int32_t* tb_exp, int32_t* tb_row0, int32_t* tb_rows, int32_t* sched,
                           hipStream_t s) {
  bwd_tile_table_kernel<<<1, 64, 0, s>>>(counts, offsets, D.E, max_tiles, D.d / kBwdTileBT,
                                         max_split, dx_parts, tb_count, tb_exp, tb_row0, tb_rows,
                                         sched);
}

void launch_bwd_gather(const Dims& D, const void* src, const int32_t* row_token, void* dst,
                       hipStream_t s) {
  bwd_gather_kernel<<<D.max_rows, 256, 0, s>>>((const bf16_t*)src, row_token, D.d,
                                               (bf16_t*)dst);
}

void launch_bwd_gemm_rows(const void* A, int lda, const void* B, int ldb, bool b_kcontig,
                          size_t b_estride, void* C, bool c_bf16, int ldc, int M, int N,
                          int K, bool accumulate, int max_tiles, const int32_t* tb_count,
                          const int32_t* tb_exp, const int32_t* tb_row0, const int32_t* tb_rows,
                          hipStream_t s) {
  const dim3 grid((N + kGN - 1) / kGN, max_tiles);
  // bf16 output never accumulates
  auto run = [&](auto kc, auto cb) {
    grouped_gemm_kernel<true, decltype(kc)::value, 0, decltype(cb)::value><<<grid, kGT, 0, s>>>(
        (const bf16_t*)A, lda, (const bf16_t*)B, ldb, b_estride, C, ldc, 0, M, N, K,
        accumulate && !decltype(cb)::value, tb_count, tb_exp, tb_row0, tb_rows, nullptr, nullptr);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (b_kcontig) {
    if (c_bf16) run(T_{}, T_{});
    else run(T_{}, F_{});
  } else {
    if (c_bf16) run(F_{}, T_{});
    else run(F_{}, F_{});
  }
}

void launch_bwd_gemm_wgrad(const Dims& D, const void* A, int lda, const void* B, int ldb,
                           void* C, int M, int N, const int32_t* counts, const int32_t* offsets,
                           hipStream_t s) {
  const dim3 grid((N + kGN - 1) / kGN, (M + kGM - 1) / kGM, D.E);
  grouped_gemm_kernel<false, false, 1, true><<<grid, kGT, 0, s>>>(
      (const bf16_t*)A, lda, (const bf16_t*)B, ldb, 0, C, N, (size_t)M * N, M, N, 0, false,
      nullptr, nullptr, nullptr, nullptr, counts, offsets);
}

void launch_bwd_rows(const Dims& D, const void* AB, const void* Z, const int32_t* row_token,
                     const int32_t* tok_row, const float* gates, float* dg, void* dAB, void* Hg,
                     hipStream_t s) {
  bwd_rows_kernel<<<D.max_rows, 256, 0, s>>>((const bf16_t*)AB, (const bf16_t*)Z, row_token,
                                             tok_row, gates, D.f, D.k, dg, (bf16_t*)dAB,
                                             (bf16_t*)Hg);
}

void launch_bwd_router(const Dims& D, const float* logits, const int32_t* idx, const float* gates,
                       const int32_t* tok_row, const float* dg_row, const int32_t* counts,
                       float alpha, float* ds, hipStream_t s) {
  bwd_router_kernel<<<(D.T + 3) / 4, 256, 0, s>>>(logits, idx, gates, tok_row, dg_row, counts,
                                                  D.T, D.E, D.k, alpha, ds);
}

void launch_bwd_router_wgrad(const Dims& D, const void* x, const float* ds, float* part,
                             float* dWr, float* dbias, hipStream_t s) {
  const int slices = kBwdRouterSlices;
  const int tslice = (D.T + slices - 1) / slices;
  const dim3 grid((D.d + 1 + 255) / 256, slices);
  auto run = [&](auto eb) {
    bwd_router_wgrad_kernel<bf16_t, decltype(eb)::value><<<grid, 256, 0, s>>>(
        (const bf16_t*)x, ds, D.T, D.d, D.E, tslice, part);
  };
  // few experts: eight columns a thread (one 16-byte x load per token)
  const dim3 grid8((D.d / 8 + 1 + 63) / 64, slices);
  if (D.E <= 8)
    bwd_router_wgrad8_kernel<8><<<grid8, 64, 0, s>>>((const bf16_t*)x, ds, D.T, D.d, D.E, tslice,
                                                     part);
  else if (D.E <= 16)
    bwd_router_wgrad8_kernel<16><<<grid8, 64, 0, s>>>((const bf16_t*)x, ds, D.T, D.d, D.E,
                                                      tslice, part);
  else if (D.E <= 32) run(std::integral_constant<int, 32>{});
  else run(std::integral_constant<int, 64>{});
  bwd_router_wgrad_reduce<<<((D.d + 1) * D.E + 255) / 256, 256, 0, s>>>(part, slices, D.d, D.E,
                                                                       dWr, dbias);
}

void launch_bwd_dx(const Dims& D, int nplanes, const float* dX, size_t plane,
                   const float* dX_extra, size_t extra_plane, const int32_t* sched,
                   const int32_t* tok_row, const float* Wr, const float* ds, void* dx,
                   hipStream_t s) {
  const dim3 grid((D.T + kDxTokens - 1) / kDxTokens, (D.d + 255) / 256);
  auto run = [&](auto eb) {
    bwd_dx_kernel<bf16_t, decltype(eb)::value><<<grid, 256, 0, s>>>(
        nplanes, dX, plane, dX_extra, extra_plane, sched, tok_row, Wr, ds, D.T, D.d, D.E, D.k,
        (bf16_t*)dx);
  };
  if (D.E <= 8) run(std::integral_constant<int, 8>{});
  else if (D.E <= 16) run(std::integral_constant<int, 16>{});
  else if (D.E <= 32) run(std::integral_constant<int, 32>{});
  else run(std::integral_constant<int, 64>{});
}

}  // namespace moe
