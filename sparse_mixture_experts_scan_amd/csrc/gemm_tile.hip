// Grouped expert GEMMs, LDS-tiled form (many token rows per expert), bf16.
//
// "Mistral/Mixtralのアーキテクチャ", section "各エキスパートの構造":
//   E_i(x) = W2 (SiLU(W1 x) * W3 x).
// Gate/up: H[r][f] = SiLU(sum_c W_gate[e][f][c] Xs[r][c]) * sum_c W_up[e][f][c] Xs[r][c]
// Down:    Y[r][o] = sum_f W_down[e][o][f] H[r][f]   (fp32 out)
//
// Tile: 256 weight rows x 256 token rows per workgroup, K staged 64 at a time
// through double-buffered LDS (2 x 64 KiB), 4 waves as 2 (weights) x 2
// (tokens), each wave 128 x 128 outputs in sixteen 32x32 fp32 accumulators
// fed by v_mfma_f32_32x32x16_bf16 (A = weight rows, B = token rows, both
// K-contiguous).  For gate/up the 256 weight rows are 128 gate rows and the
// same 128 up rows, and each wave holds gate and up accumulators of the same
// features, so SiLU(gate) * up is applied in registers and only H is stored.
//
// LDS rows are 128 bytes (64 bf16); the eight 16-byte chunks of row r are
// XOR-swizzled by (r ^ r >> 3) & 7 so that the 32 rows one MFMA fragment
// reads, and the rows a wave writes, fall in distinct banks.
//
// Token rows past the expert's count read as zero; 32-row token fragments
// that are entirely past it skip their MFMAs.  Work-group ids are remapped
// so that consecutive tiles (same expert, neighbouring feature tiles) land on
// the same XCD and share its L2.
#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kTileThreads = 256;
constexpr int kTileBT = kTileTokens;  // token rows per tile (= padding unit)
constexpr int kTileBK = 64;           // K per LDS stage
constexpr int kTileRows = 256;        // weight rows per tile
constexpr int kTileStageBytes = 2 * kTileRows * kTileBK * 2;  // A + B per stage
constexpr int kTileLds = 2 * kTileStageBytes;                 // double buffered
constexpr int kXcds = 8;
constexpr int kFeatGroup = 8;         // feature tiles per XCD-local group

__device__ inline int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

__device__ inline f32x16 mfma32(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <bool GATEUP>
__global__ __launch_bounds__(kTileThreads, 1) void tile_gemm_kernel(
    const bf16_t* __restrict__ act, const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ num_tiles,
    const int32_t* __restrict__ tile_expert, int N, int K, int n_ft, int n_tt, int per_xcd) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int FB = GATEUP ? kTileRows / 2 : kTileRows;  // output features per tile

  // ---- tile id: XCD-contiguous remap, then groups of kFeatGroup feature tiles
  const int L = blockIdx.x;
  const int Lp = (L % kXcds) * per_xcd + L / kXcds;
  if (Lp >= n_ft * n_tt) return;
  const int grp = Lp / (kFeatGroup * n_tt);
  const int rem = Lp - grp * kFeatGroup * n_tt;
  const int gsize = min(kFeatGroup, n_ft - grp * kFeatGroup);
  const int tt = rem / gsize;
  const int ft = grp * kFeatGroup + rem % gsize;
  if (tt >= *num_tiles) return;
  const int e = tile_expert[tt];
  const int row0 = tt * kTileBT;
  const int valid_end = offsets[e] + counts[e];
  const int f0 = ft * FB;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave & 1, wt = wave >> 1;

  // ---- global -> register -> LDS staging: thread owns rows rbase + 32 i, chunk kc
  const int kc = tid & 7, rbase = tid >> 3;
  const bf16_t* gA0;
  const bf16_t* gA1;
  if constexpr (GATEUP) {
    gA0 = W0 + ((size_t)e * N + f0 + rbase) * K + kc * 8;   // gate rows 0..127
    gA1 = W1 + ((size_t)e * N + f0 + rbase) * K + kc * 8;   // up rows 128..255
  } else {
    gA0 = W0 + ((size_t)e * N + f0 + rbase) * K + kc * 8;
    gA1 = gA0 + (size_t)128 * K;
  }
  const bf16_t* gB = act + (size_t)(row0 + rbase) * K + kc * 8;
  const int bvalid = valid_end - row0 - rbase;  // token row rbase + 32 i valid iff 32 i < bvalid
  uint4 ra[8], rb[8];
  const uint4 zero = make_uint4(0, 0, 0, 0);

  auto gload = [&](int ks) {
    const size_t ko = (size_t)ks * kTileBK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = ld16(gA0 + (size_t)(32 * i) * K + ko);
      ra[i + 4] = ld16(gA1 + (size_t)(32 * i) * K + ko);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) rb[i] = (32 * i < bvalid) ? ld16(gB + (size_t)(32 * i) * K + ko) : zero;
  };
  auto sstore = [&](int buf) {
    char* A = smem + buf * kTileStageBytes;
    char* B = A + kTileStageBytes / 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int off = swz(rbase + 32 * i, kc);
      *reinterpret_cast<uint4*>(A + off) = ra[i];
      *reinterpret_cast<uint4*>(B + off) = rb[i];
    }
  };

  // ---- wave's fragments: A rows (weights), B rows (tokens)
  int arow[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    if constexpr (GATEUP) arow[a] = (a < 2 ? 0 : 128) + wf * 64 + (a & 1) * 32;
    else arow[a] = wf * 128 + a * 32;
  }
  const int nbv = max(0, min(4, (valid_end - (row0 + wt * 128) + 31) / 32));

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.f;

  auto compute = [&](int buf) {
    const char* A = smem + buf * kTileStageBytes;
    const char* B = A + kTileStageBytes / 2;
    const int r32 = lane & 31, khalf = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < kTileBK / 16; ++kk) {
      const int chunk = kk * 2 + khalf;
      uint4 af[4], bfr[4];
#pragma unroll
      for (int a = 0; a < 4; ++a)
        af[a] = *reinterpret_cast<const uint4*>(A + swz(arow[a] + r32, chunk));
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (b < nbv) bfr[b] = *reinterpret_cast<const uint4*>(B + swz(wt * 128 + b * 32 + r32, chunk));
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (b < nbv) {
#pragma unroll
          for (int a = 0; a < 4; ++a) acc[a][b] = mfma32(af[a], bfr[b], acc[a][b]);
        }
    }
  };

  const int nk = K / kTileBK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int ks = 0; ks < nk; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < nk) gload(ks + 1);
    compute(cur);
    if (ks + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  D of a 32x32 MFMA: lane holds column n = lane % 32 and rows
  // 8 * (j / 4) + 4 * (lane / 32) + j % 4, j = 0..15: four consecutive features.
  const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const size_t row = (size_t)(row0 + wt * 128 + b * 32 + r32);
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
      float* y = reinterpret_cast<float*>(outp) + row * N;
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
  const int total = n_ft * n_tt;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  static bool attr_set = false;
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&tile_gemm_kernel<GATEUP>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, kTileLds);
    attr_set = true;
  }
  tile_gemm_kernel<GATEUP><<<per_xcd * kXcds, kTileThreads, kTileLds, s>>>(
      (const bf16_t*)act, (const bf16_t*)W0, (const bf16_t*)W1, out, counts, offsets, num_tiles,
      tile_expert, N, K, n_ft, n_tt, per_xcd);
}

bool tile_shape_ok(const Dims& D) {
  return D.bf16 && D.BT == kTileBT && D.f % (kTileRows / 2) == 0 && D.d % kTileRows == 0 &&
         D.d % kTileBK == 0 && D.f % kTileBK == 0;
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
