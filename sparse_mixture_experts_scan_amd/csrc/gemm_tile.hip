// Grouped expert GEMMs, LDS-tiled form (many token rows per expert), bf16.
//
// "Mistral/Mixtralのアーキテクチャ", section "各エキスパートの構造":
//   E_i(x) = W2 (SiLU(W1 x) * W3 x).
// Gate/up: H[r][f] = SiLU(sum_c W_gate[e][f][c] Xs[r][c]) * sum_c W_up[e][f][c] Xs[r][c]
// Down:    Y[r][o] = sum_f W_down[e][o][f] H[r][f]   (fp32 out)
//
// Tile: 256 weight rows x 256 token rows per workgroup of 8 waves, each wave
// 128 weight rows x 64 token rows in eight 32x32 fp32 accumulators fed by
// v_mfma_f32_32x32x16_bf16 (A = weight rows, B = token rows, both
// K-contiguous).  For gate/up the 256 weight rows are 128 gate rows and the
// same 128 up rows, and each wave holds gate and up accumulators of the same
// features, so SiLU(gate) * up is applied in registers and only H is stored.
//
// K is staged 64 at a time through LDS buffers filled by gfx950 buffer loads
// straight to LDS (no VGPR staging): each lane fetches the 16 bytes that
// belong at its slot of the XOR-swizzled layout.  LDS rows are 128 bytes;
// chunk c of row r sits at c ^ ((r ^ r >> 3) & 7), so the 32 rows an MFMA
// fragment reads fall in distinct banks (no bank conflicts measured).
//
// Ping-pong: waves 0-3 (one per SIMD) and waves 4-7 run the same sequence per
// stage -- read the stage's fragments from LDS into registers, barrier, run
// the stage's 32 MFMAs, barrier -- but waves 4-7 pass one extra barrier first,
// so each SIMD's two waves alternate: one reads while the other keeps the
// matrix unit busy.  The DMA is split so that the CU's address unit is busy in
// both phases: waves 0-3 fetch the token operand (B, a pair of buffers, one
// stage ahead) as they start reading, waves 4-7 the weight operand (A, a ring
// of three buffers, two stages ahead) after their reads.  Data sent by waves
// 4-7 is read by waves 0-3 one phase later, so the deeper ring belongs there;
// it holds the weights.  Measured against the other way round on two MI355X
// boxes: E = 64 top-8 (few rows per expert, many weight panels in flight) 1.5%
// faster on both GEMMs; the 8-expert workloads from 1.4% faster to even.  The
// five 32 KiB buffers fill the 160 KiB of LDS.
//
// Token rows past the expert's count lie outside the token operand's buffer
// range, so the hardware loads zeros; 32-row token fragments entirely past it
// skip their reads and MFMAs (a wave's two fragments are 128 rows apart, so
// the two wave groups share a partly filled tile evenly).  Work-group ids are
// remapped so that the tiles an XCD runs together share weight and token
// panels in its L2.

#include <algorithm>
#include <cmath>

#include "common.h"
#include "launch.h"

namespace moe {

constexpr int kTileWaves = 8;                       // two per SIMD
constexpr int kTileThreads = 64 * kTileWaves;
constexpr int kBFrags = 2;                          // 32-row token fragments per wave
constexpr int kBStride = 128;                       // rows between a wave's token fragments
constexpr int kTileBT = kTileTokens;  // token rows per tile (= padding unit)
constexpr int kTileRows = 256;        // weight rows per tile
constexpr int kTileBK = 64;           // K per LDS stage
constexpr int kTileNS = 2;            // pair buffers (B): the K loop runs stages in pairs
constexpr int kKSteps = kTileBK / 16;               // 32x32x16 MFMA k-steps per stage
constexpr int kXcds = 8;

constexpr int kRowBytes = kTileBK * 2;              // LDS bytes per tile row
constexpr int kChunks = kRowBytes / 16;             // 16-byte chunks per row
constexpr int kOperBytes = 256 * kRowBytes;         // one operand tile (one buffer) in LDS
constexpr int kDmaWaves = 4;                        // waves issuing one operand's DMA
constexpr int kDmaPerWave = 256 * kChunks / 64 / kDmaWaves;  // 1 KiB DMA loads per wave per stage
static_assert(kChunks == 8 && kDmaPerWave == 8, "fragment and DMA addressing assume 8-chunk rows");
static_assert(5 * kOperBytes <= 160 * 1024, "LDS buffers exceed 160 KiB");

// XOR swizzle of the 16-byte chunks of LDS row r: the 32 rows an MFMA fragment
// reads (and the rows a DMA fills) fall in distinct banks.
__device__ inline int swz_key(int r) { return (r ^ (r >> 3)) & 7; }

// SiLU(z) = z * sigmoid(z) for the bf16 epilogue: sigmoid from the hardware
// base-2 exponential and reciprocal (about one fp32 ulp each, far below the
// bf16 rounding of the result); exp2 overflowing to +inf gives z * 0.
__device__ inline float silu_bf16_out(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
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
  // LDS byte offsets of this lane's first A and B fragment rows.  The swizzle
  // of row arow + r (arow a multiple of 32, r < 32) is key(r) ^ 4 (arow / 32
  // & 1), so a fragment at k-step kk sits at base ^ ((2 kk ^ that term) << 4)
  // plus a constant row offset: a few registers and immediate offsets serve
  // every read.
  uint32_t lbA, lbB;
  // B waves: whether this wave's 64 token rows start before the tile's last
  // valid row.  A wave whose rows are all past it issues no B at all (nobody
  // reads those rows: their fragments are skipped), for the whole tile, so
  // its waits on its own DMA pass at once.
  bool b_on;
};

// One operand of stage ks's DMA into buffer `buf`: op 0 = A (weights, sent
// by waves 4-7), op 1 = B (tokens, sent by waves 0-3).  Lane i of a wave's
// load j fetches the global 16 bytes that belong at LDS slot
// (dma_base + j) * 64 + i.
__device__ __forceinline__ void tile_issue_half(const TileCtx& c, char* buf, int ks, int op) {
  const uint32_t so = c.k_byte0 + (uint32_t)ks * kTileBK * 2;
  if (op == 0) {
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          c.rA, (lds_void*)(buf + (c.dma_base + j) * 1024), 16, c.voffA[j], so, 0, 0);
  } else if (c.b_on) {
#pragma unroll
    for (int j = 0; j < kDmaPerWave; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          c.rB, (lds_void*)(buf + (c.dma_base + j) * 1024), 16, c.voffB[j], so, 0, 0);
  }
}

// A stage's fragments (A from `buf`, B from `bbuf`): per k-step, the wave's
// four A fragments (32 weight rows each) and its NBV valid token fragments.  A fragment a starts at
// weight row arow(a) of the wave's half, token fragment b at row b * kBStride
// of the wave's slice.
template <int NBV, bool GATEUP>
__device__ __forceinline__ void tile_load(const TileCtx& c, const char* buf, const char* bbuf,
                                          uint4 (&fa)[kKSteps][4], uint4 (&fb)[kKSteps][kBFrags]) {
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int arow = GATEUP ? (a < 2 ? 0 : 128) + (a & 1) * 32 : a * 32;
      const uint32_t off = c.lbA ^ (uint32_t)(((2 * kk) ^ (4 * (a & 1))) << 4);
      fa[kk][a] = *reinterpret_cast<const uint4*>(buf + off + arow * kRowBytes);
    }
#pragma unroll
    for (int b = 0; b < NBV; ++b) {
      const uint32_t off = c.lbB ^ (uint32_t)((2 * kk) << 4);
      fb[kk][b] = *reinterpret_cast<const uint4*>(bbuf + off + b * kBStride * kRowBytes);
    }
    // keep the reads in k-step order
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NBV>
__device__ __forceinline__ void tile_mfma(const uint4 (&fa)[kKSteps][4],
                                          const uint4 (&fb)[kKSteps][kBFrags],
                                          f32x16 (&acc)[4][kBFrags]) {
#pragma unroll
  for (int kk = 0; kk < kKSteps; ++kk)
#pragma unroll
    for (int b = 0; b < NBV; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a][b] = mfma32(fa[kk][a], fb[kk][b], acc[a][b]);
}

// One stage s: B in the pair buffer `pcur` (stage s + 1's B goes to `pnxt`),
// A in the ring buffer `rcur`.  Waves 0-3 send B of stage s + 1 as they start
// reading stage s; waves 4-7 send A of stage s + 2 into `rnew` (the ring
// buffer of stage s - 1) after their reads.  XWAIT after the reads, then every
// wave waits for all of its DMA after the MFMAs (waves 0-3: B of stage s + 1;
// waves 4-7: A of s + 2).
template <int NBV, bool GATEUP, bool ISSUE_P, bool ISSUE_R, int XWAIT>
__device__ __forceinline__ void tile_stage(const TileCtx& c, char* pcur, char* pnxt,
                                           const char* rcur, char* rnew, int s, int g,
                                           uint4 (&fa)[kKSteps][4],
                                           uint4 (&fb)[kKSteps][kBFrags],
                                           f32x16 (&acc)[4][kBFrags]) {
  if (ISSUE_P && g == 0) tile_issue_half(c, pnxt, s + 1, 1);
  tile_load<NBV, GATEUP>(c, rcur, pcur, fa, fb);
  if (ISSUE_R && g == 1) tile_issue_half(c, rnew, s + 2, 0);
  wait_vmcnt<XWAIT>();
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  tile_mfma<NBV>(fa, fb, acc);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<0>();
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// Main loop over K (nk stages, a positive even number).  B of stage s lives
// in p0/p1 by s % 2 (compile-time), A in ring[s % 3] (run time); every wait
// count is a compile-time constant, the same in both wave groups.
template <int NBV, bool GATEUP>
__device__ __forceinline__ void tile_main_loop(const TileCtx& c, char* p0, char* p1, char* ring,
                                               int nk, int g, f32x16 (&acc)[4][kBFrags]) {
  uint4 fa[kKSteps][4], fb[kKSteps][kBFrags];
  if (g == 0) {
    tile_issue_half(c, p0, 0, 1);                  // B of stage 0
  } else {
    tile_issue_half(c, ring, 0, 0);                // A of stages 0 and 1
    tile_issue_half(c, ring + kOperBytes, 1, 0);
  }
  wait_vmcnt<0>();
  lds_barrier();                                   // stage 0 visible
  if (g == 1) lds_barrier();                       // waves 4-7 run one phase behind
  __builtin_amdgcn_sched_barrier(0);
  int bs = 0;                                      // s % 3
  auto bb = [&](int i) { return ring + i * kOperBytes; };
  auto inc3 = [](int i) { return i == 2 ? 0 : i + 1; };
  int s = 0;
  for (; s < nk - 2; s += 2) {
    const int b1 = inc3(bs), b2 = inc3(b1), b3 = inc3(b2);
    tile_stage<NBV, GATEUP, true, true, kDmaPerWave>(c, p0, p1, bb(bs), bb(b2), s, g, fa, fb, acc);
    tile_stage<NBV, GATEUP, true, true, kDmaPerWave>(c, p1, p0, bb(b1), bb(b3), s + 1, g, fa, fb,
                                                     acc);
    bs = b2;
  }
  tile_stage<NBV, GATEUP, true, false, 0>(c, p0, p1, bb(bs), nullptr, s, g, fa, fb, acc);
  tile_stage<NBV, GATEUP, false, false, 0>(c, p1, p0, bb(inc3(bs)), nullptr, s + 1, g, fa, fb,
                                           acc);
  if (g == 0) lds_barrier();                       // same barrier count in both groups
}

template <bool GATEUP>
__global__ __launch_bounds__(kTileThreads, 1) void tile_gemm_kernel(
    const bf16_t* __restrict__ act, const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1,
    void* __restrict__ outp, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ num_tiles,
    const int32_t* __restrict__ tile_expert, int N, int K, int n_ft, int n_tt, int per_xcd,
    int parts, size_t part_stride, int fgroup, const int32_t* __restrict__ row_token, int nT) {
  // separate __shared__ arrays for the token operand's pair of buffers and
  // the weight operand's ring, so that the compiler can tell which DMA each
  // LDS read depends on
  __shared__ __attribute__((aligned(1024))) char sa0[kOperBytes];
  __shared__ __attribute__((aligned(1024))) char sa1[kOperBytes];
  __shared__ __attribute__((aligned(1024))) char sbr[3 * kOperBytes];
  constexpr int FB = GATEUP ? kTileRows / 2 : kTileRows;  // output features per tile

  // ---- tile id: XCD-contiguous remap, then groups of `fgroup` feature tiles
  const int L = blockIdx.x;
  int Lp = (L % kXcds) * per_xcd + L / kXcds;
  if (Lp >= parts * n_ft * n_tt) return;
  const int part = Lp / (n_ft * n_tt);      // K-split part (slowest)
  Lp -= part * n_ft * n_tt;
  const int grp = Lp / (fgroup * n_tt);
  const int rem = Lp - grp * fgroup * n_tt;
  const int gsize = min(fgroup, n_ft - grp * fgroup);
  const int tt = rem / gsize;
  const int ft = grp * fgroup + rem % gsize;
  if (tt >= *num_tiles) return;             // past the token tiles in use
  const int e = tile_expert[tt];
  const int row0 = tt * kTileBT;
  const int valid_end = offsets[e] + counts[e];
  const int f0 = ft * FB;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wf = wave & 1, wt = wave >> 1;   // weight half, token slice
  const int g = wave >> 2;                   // wave group (ping-pong)

  // ---- DMA assignment: wave w fills LDS slots [(w % 4) * kDmaPerWave,
  // +kDmaPerWave) of its operand (1 KiB each); slot q's lane i holds LDS chunk
  // position p = q * 64 + i = row * kChunks + swizzled chunk.
  TileCtx c;
  c.dma_base = (wave & 3) * kDmaPerWave;
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
    if (GATEUP && row_token) {
      // token row of tile row r, read in place; a padding row has none and
      // points past the buffer range, which loads zeros
      const int t = row_token[row0 + r];
      c.voffB[j] = t >= 0 ? (uint32_t)t * row_bytes + cg * 16 : 0x80000000u;
    }
  }
  if constexpr (GATEUP) {
    // waves 4-5 fill A rows 0..127 (gate), waves 6-7 rows 128..255 (up);
    // waves 0-3 issue no A
    const bf16_t* Wsrc = ((wave & 3) < kDmaWaves / 2 ? W0 : W1) + ((size_t)e * N + f0) * K;
    c.rA = make_rsrc(Wsrc, 128 * row_bytes);
  } else {
    c.rA = make_rsrc(W0 + ((size_t)e * N + f0) * K, 256 * row_bytes);
  }
  // token rows past the expert's count fall outside the resource: read as 0
  const int nvalid = max(0, min(kTileBT, valid_end - row0));
  c.rB = (GATEUP && row_token) ? make_rsrc(act, (uint32_t)nT * row_bytes)
                               : make_rsrc(act + (size_t)row0 * K, (uint32_t)nvalid * row_bytes);
  c.b_on = c.dma_base * (1024 / kRowBytes) < nvalid;

  // ---- fragment rows: A fragment a of wave half wf, token fragments at rows
  // wt * 32 and wt * 32 + kBStride of the tile
  {
    const int r32 = lane & 31, h = lane >> 5;
    const uint32_t lrow = (uint32_t)r32 * kRowBytes + (uint32_t)((h ^ swz_key(r32)) << 4);
    c.lbA = (uint32_t)(GATEUP ? wf * 64 : wf * 128) * kRowBytes + lrow;
    c.lbB = (uint32_t)(wt * 32) * kRowBytes + (lrow ^ (uint32_t)((4 * (wt & 1)) << 4));
  }
  int nbv = 0;                              // valid token fragments of this wave
#pragma unroll
  for (int b = 0; b < kBFrags; ++b) nbv += row0 + wt * 32 + b * kBStride < valid_end;

  f32x16 acc[4][kBFrags];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < kBFrags; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.f;

  // wave-uniform choice; every variant runs the same DMA and barriers
  const int nk = Kp / kTileBK;
  switch (nbv) {
    case 2: tile_main_loop<2, GATEUP>(c, sa0, sa1, sbr, nk, g, acc); break;
    case 1: tile_main_loop<1, GATEUP>(c, sa0, sa1, sbr, nk, g, acc); break;
    default: tile_main_loop<0, GATEUP>(c, sa0, sa1, sbr, nk, g, acc); break;
  }

  // ---- epilogue.  D of a 32x32 MFMA: lane holds column n = lane % 32 and rows
  // 8 * (j / 4) + 4 * (lane / 32) + j % 4, j = 0..15: four consecutive
  // features.  Skipped fragments hold zeros (padding rows).  The tile is
  // staged in the (now idle) B ring and written back as whole rows with
  // 16-byte stores; every row of the tile is written, padding rows as zeros.
  const int r32 = lane & 31, half = lane >> 5;
  lds_barrier();                            // every wave is past its last LDS read
  if constexpr (GATEUP) {
    constexpr int kPitch = FB * 2 + 16;     // bf16 row of the h tile, padded
    static_assert(kTileBT * kPitch <= 3 * kOperBytes, "staging exceeds the B ring");
#pragma unroll
    for (int b = 0; b < kBFrags; ++b) {
      const int lrow = wt * 32 + b * kBStride + r32;
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int lfeat = wf * 64 + a * 32 + jj * 8 + half * 4;
          uint32_t p[2];
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const float g0 = acc[a][b][jj * 4 + 2 * q], u0 = acc[a + 2][b][jj * 4 + 2 * q];
            const float g1 = acc[a][b][jj * 4 + 2 * q + 1], u1 = acc[a + 2][b][jj * 4 + 2 * q + 1];
            p[q] = pack_bf16x2(silu_bf16_out(g0) * u0, silu_bf16_out(g1) * u1);
          }
          *reinterpret_cast<uint2*>(sbr + lrow * kPitch + lfeat * 2) = make_uint2(p[0], p[1]);
        }
    }
    lds_barrier();
    constexpr int kChunksRow = FB * 2 / 16;  // 16-byte pieces per h row
    bf16_t* h = reinterpret_cast<bf16_t*>(outp) + (size_t)row0 * N + f0;
#pragma unroll
    for (int it = 0; it < kTileBT * kChunksRow / kTileThreads; ++it) {
      const int q = it * kTileThreads + tid;
      const int lrow = q / kChunksRow, ch = q % kChunksRow;
      const uint4 v = *reinterpret_cast<const uint4*>(sbr + lrow * kPitch + ch * 16);
      *reinterpret_cast<uint4*>(h + (size_t)lrow * N + ch * 8) = v;
    }
  } else {
    // fp32: (token fragment b, feature half ch) = 128 rows x 128 features
    // at a time, written by the waves of that half
    constexpr int kPitch = 128 * 4 + 16;
    static_assert(128 * kPitch <= 3 * kOperBytes, "staging exceeds the B ring");
    float* y = reinterpret_cast<float*>(outp) + part * part_stride + (size_t)row0 * N + f0;
#pragma unroll
    for (int b = 0; b < kBFrags; ++b)
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        if (wf == ch) {
          const int lrow = wt * 32 + r32;
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int col = a * 32 + jj * 8 + half * 4;
              *reinterpret_cast<float4*>(sbr + lrow * kPitch + col * 4) =
                  make_float4(acc[a][b][jj * 4], acc[a][b][jj * 4 + 1], acc[a][b][jj * 4 + 2],
                              acc[a][b][jj * 4 + 3]);
            }
        }
        lds_barrier();
#pragma unroll
        for (int it = 0; it < 128 * 32 / kTileThreads; ++it) {
          const int q = it * kTileThreads + tid;
          const int lrow = q / 32, chunk = q % 32;
          const uint4 v = *reinterpret_cast<const uint4*>(sbr + lrow * kPitch + chunk * 16);
          *reinterpret_cast<uint4*>(y + (size_t)(b * kBStride + lrow) * N + ch * 128 +
                                    chunk * 4) = v;
        }
        lds_barrier();
      }
  }
}

// Feature tiles per XCD-local group of the tile order.  Consecutive
// workgroups of one XCD take the group's feature tiles for one token tile,
// then the next token tile, so about 32 / fgroup token tiles share each
// weight panel while they run.  Measured on MI355X: with about 1000 or more
// rows per expert (4+ token tiles) groups of 4 are best for both GEMMs; with
// about 500 (E = 64, top-8) groups of 3 for gate/up and 2 for down are 4% and
// 13% faster than 4, while 1 and wider groups (8 to 28) are slower.
static int tile_feat_group(const Dims& D, bool gateup) {
  const int64_t rows_per_expert = (int64_t)D.T * D.k / D.E;
  if (rows_per_expert >= 3 * kTileBT) return 4;
  return gateup ? 3 : 2;
}

template <bool GATEUP>
static void tile_launch(const Dims& D, const void* act, const int32_t* row_token, const void* W0,
                        const void* W1, void* out, const int32_t* counts,
                        const int32_t* offsets, const int32_t* num_tiles,
                        const int32_t* tile_expert, hipStream_t s) {
  const int N = GATEUP ? D.f : D.d;
  const int K = GATEUP ? D.d : D.f;
  const int FB = GATEUP ? kTileRows / 2 : kTileRows;
  const int n_ft = N / FB;
  const int n_tt = D.max_tiles;
  const int parts = GATEUP ? 1 : D.down_splits;
  const int total = parts * n_ft * n_tt;
  const int per_xcd = (total + kXcds - 1) / kXcds;
  const int grid = per_xcd * kXcds;
  tile_gemm_kernel<GATEUP><<<grid, kTileThreads, 0, s>>>(
      (const bf16_t*)act, (const bf16_t*)W0, (const bf16_t*)W1, out, counts, offsets, num_tiles,
      tile_expert, N, K, n_ft, n_tt, per_xcd, parts, (size_t)D.max_rows * N,
      tile_feat_group(D, GATEUP), row_token, D.T);
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

// Reading the tokens in place saves the scatter's copy of k rows per token
// but spreads each tile's token panel over x.  Measured on MI355X: with
// top-8 (E = 64) the step is 3.5% faster; with top-2 the gate/up GEMM loses
// about what the copy costs, so those keep the copy.
bool tile_gathers_in_place(const Dims& D) {
  return D.k >= 4 && (int64_t)D.T * D.d * 2 < (int64_t(1) << 31);
}

void launch_gateup_tile(const Dims& D, const void* x, const int32_t* row_token, const void* Wg,
                        const void* Wu, void* h, const int32_t* counts, const int32_t* offsets,
                        const int32_t* num_tiles, const int32_t* tile_expert, hipStream_t s) {
  tile_launch<true>(D, x, row_token, Wg, Wu, h, counts, offsets, num_tiles, tile_expert, s);
}

void launch_down_tile(const Dims& D, const void* h, const void* Wd, float* y,
                      const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                      const int32_t* tile_expert, hipStream_t s) {
  tile_launch<false>(D, h, nullptr, Wd, nullptr, y, counts, offsets, num_tiles, tile_expert, s);
}

}  // namespace moe
