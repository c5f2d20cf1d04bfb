// Backward GEMMs of the sparse MoE layer, LDS-tiled, bf16 in, fp32 accumulate.
//
// "Mistral/Mixtralのアーキテクチャ", section "各エキスパートの構造"
// (E_i(x) = W2 (SiLU(W1 x) * W3 x)): every contraction the chain rule needs
// is one launch of
//   C[brow][aidx] = sum_k A[aidx][k] B[brow][k]
// with aidx contiguous in C, on 256 x 256 tiles:
//   recompute  a | b  = W1 | W3 rows   . x_r rows          (token-tile groups)
//   Z          W2^T dOut               . dOut_r rows       (token-tile groups)
//   dX         [W1; W3]^T [dA | dB]    over K = 2 d_ff     (token-tile groups)
//   dW2        Hg^T . dOut             over the expert's rows
//   dW1 | dW3  x^T . [dA | dB]         over the expert's rows
// An operand is either k-contiguous in memory (KC: a row of k per index) or
// k-strided (KS: a row of indices per k, read down its columns).
//
// Structure as the forward's tiled GEMM: 8 waves of 128 (A) x 64 (B), two
// per SIMD in ping-pong (waves 4-7 one phase behind waves 0-3), operand A
// fetched by waves 0-3 one stage ahead into two LDS buffers, operand B by
// waves 4-7 two stages ahead into three, all by buffer loads straight to
// LDS; 64 k per stage.
//   KC tiles sit in LDS as [256 rows][64 k] with 16-byte chunks XOR-swizzled
//   by row and are read with ds_read_b128.
//   KS tiles sit as [64 k][256 indices] (512-byte rows) with 64-byte blocks
//   XOR-swizzled by k mod 4, and are read with gfx950's transposing
//   ds_read_b64_tr_b16: within each 16 lanes, lane 4 j + q addresses row
//   kb + j, columns cb + 4 q .. + 3, and lane i receives rows kb .. kb + 3 of
//   column cb + i -- four consecutive k of the lane's MFMA column; two such
//   reads give the eight k of a v_mfma_f32_32x32x16_bf16 operand.
// Rows of a k-strided operand past its end (an expert's rows) lie outside the
// buffer range, which the stage's resource is re-based to, so they load as
// zeros; so do token rows past a token tile's rows.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kBWaves = 8;
constexpr int kBThreads = 64 * kBWaves;
constexpr int kBT = 256;                    // tile extent in A and in B
constexpr int kBK = 64;                     // k per stage
constexpr int kBKSteps = kBK / 16;
constexpr int kBFragB = 2;                  // token fragments per wave
constexpr int kBStrideB = 128;              // rows between a wave's B fragments
constexpr int kBOper = kBT * kBK * 2;       // one operand tile in LDS (32 KiB)
constexpr int kBSlots = kBOper / 1024 / 4;  // 1 KiB DMA loads per wave per stage (8)
constexpr int kBXcds = 8;
#ifndef MOE_BWD_FEAT_GROUP
#define MOE_BWD_FEAT_GROUP 4
#endif
constexpr int kBFeatGroup = MOE_BWD_FEAT_GROUP;  // feature tiles per XCD-local group
constexpr int kBWgradGroup = 8;  // weight gradients with the wider B: B tiles per group
constexpr int kKCRow = kBK * 2;             // KC: bytes per LDS row (128)
constexpr int kKSRow = kBT * 2;             // KS: bytes per LDS row (512)
static_assert(5 * kBOper <= 160 * 1024, "LDS buffers exceed 160 KiB");

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;


__device__ inline int kc_key(int r) { return (r ^ (r >> 3)) & 7; }

__device__ inline f32x16 b_mfma(uint4 a, uint4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Two transposing 8-byte reads: the eight k of one MFMA operand lane.
__device__ __forceinline__ uint4 ks_frag(const char* p0, const char* p1) {
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p0));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(p1));
  const uint2 l = __builtin_bit_cast(uint2, lo), h = __builtin_bit_cast(uint2, hi);
  return make_uint4(l.x, l.y, h.x, h.y);
}

}  // namespace

struct BgArgs {
  const bf16_t* A0;     // operand A (mode 0: expert weights, e * a_estride apart)
  const bf16_t* A1;     // second A matrix: aidx tiles >= a_split_tile, or k >= a_split_k
  size_t a_estride;
  int lda;              // A row pitch (elements)
  int a_split_tile, a_split_k;
  const bf16_t* B;      // operand B (mode 0: permuted token rows)
  int ldb;
  void* C0;             // output; C1 for brow tiles >= c_split_tile (mode 1)
  void* C1;
  int ldc;
  size_t c_estride;     // mode 1: elements between experts' outputs
  int c_split_tile;
  int K;                // mode 0 contraction length
  int n_at, n_bt;       // tiles along aidx; along brow (mode 0: tile-table capacity)
  int per_xcd, total;   // tiles per XCD (mode 1: per expert); experts or K parts
  const int32_t* tb_count;
  const int32_t* tb_exp;
  const int32_t* tb_row0;
  const int32_t* tb_rows;
  const int32_t* counts;
  const int32_t* offsets;
  // mode 0: K split into `kparts` (1 or 2) equal parts, the slowest tile
  // dimension.  Part 1 takes A from A1, B from column K of its rows, and
  // writes the C plane c_pstride elements after C0.
  int kparts;
  size_t c_pstride;
  // mode 0 (dX): sched = {split token tiles sp, their first row} from the
  // tile table.  The last sp token tiles run each part as two K halves; a
  // part's second half goes to the extra plane C_extra + part *
  // extra_pstride, row r at r - sched[1].  NULL: none.
  const int32_t* sched;
  float* C_extra;
  size_t extra_pstride;
};

namespace {

// Per-wave state: the operand this wave fetches (A in waves 0-3, B in 4-7)
// and the LDS addressing of its fragments.
struct BCtx {
  __amdgpu_buffer_rsrc_t r;   // KC: fixed; KS: re-based each stage
  const char* ks_base;        // KS: operand's first k row (matrix 0)
  const char* ks_base1;       // KS A split: matrix 1's first k row
  uint32_t ld_bytes;
  int kn;                     // rows of k available (KS range)
  int split_k;                // KS A: first k of matrix 1 (kn if none)
  uint32_t voff[kBSlots];
  int dma_base;
  uint32_t lA[4];             // A fragment bases (KC: lA[0], lA[1] used)
  uint32_t lB;                // B fragment base
  // KC operand: false when all of this wave's 64 rows lie past the tile's
  // valid rows (token rows of a short tile); the wave then issues no DMA for
  // the tile, nobody reads those rows, and its waits pass at once
  bool on;
};

// One operand's DMA for stage s into `buf` (this wave's 8 slots).
template <bool KS>
__device__ __forceinline__ void b_issue(const BCtx& c, char* buf, int s) {
  const int k0 = s * kBK;
  if constexpr (KS) {
    // re-base the resource on the stage's first k row so that rows past the
    // operand's end fall outside it
    const char* base = c.ks_base;
    int kk0 = k0, kend = c.split_k;
    if (k0 >= c.split_k) { base = c.ks_base1; kk0 = k0 - c.split_k; kend = c.kn - c.split_k; }
    const int rows = max(0, min(kBK, kend - kk0));
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc(base + (size_t)kk0 * c.ld_bytes, rows * c.ld_bytes);
#pragma unroll
    for (int j = 0; j < kBSlots; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(buf + (c.dma_base + j) * 1024), 16,
                                               c.voff[j], 0, 0, 0);
  } else if (c.on) {
#pragma unroll
    for (int j = 0; j < kBSlots; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(c.r, (lds_void*)(buf + (c.dma_base + j) * 1024),
                                               16, c.voff[j], (uint32_t)k0 * 2, 0, 0);
  }
}

template <bool KSA, bool KSB, int NBV>
__device__ __forceinline__ void b_load(const BCtx& c, const char* abuf, const char* bbuf,
                                       uint4 (&fa)[kBKSteps][4],
                                       uint4 (&fb)[kBKSteps][kBFragB]) {
#pragma unroll
  for (int kk = 0; kk < kBKSteps; ++kk) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      if constexpr (KSA) {
        const char* p = abuf + c.lA[a] + kk * 16 * kKSRow;
        fa[kk][a] = ks_frag(p, p + 4 * kKSRow);
      } else {
        const uint32_t off = c.lA[0] ^ (uint32_t)(((2 * kk) ^ (4 * (a & 1))) << 4);
        fa[kk][a] = *reinterpret_cast<const uint4*>(abuf + off + a * 32 * kKCRow);
      }
    }
#pragma unroll
    for (int b = 0; b < NBV; ++b) {
      if constexpr (KSB) {
        const char* p = bbuf + c.lB + kk * 16 * kKSRow + b * 256;
        fb[kk][b] = ks_frag(p, p + 4 * kKSRow);
      } else {
        const uint32_t off = c.lB ^ (uint32_t)((2 * kk) << 4);
        fb[kk][b] = *reinterpret_cast<const uint4*>(bbuf + off + b * kBStrideB * kKCRow);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int NBV>
__device__ __forceinline__ void b_mfma_stage(const uint4 (&fa)[kBKSteps][4],
                                             const uint4 (&fb)[kBKSteps][kBFragB],
                                             f32x16 (&acc)[4][kBFragB]) {
#pragma unroll
  for (int kk = 0; kk < kBKSteps; ++kk)
#pragma unroll
    for (int b = 0; b < NBV; ++b)
#pragma unroll
      for (int a = 0; a < 4; ++a) acc[a][b] = b_mfma(fa[kk][a], fb[kk][b], acc[a][b]);
}

// One stage s (as the forward): waves 0-3 send the pair operand of s + 1 to
// `pnxt`, waves 4-7 the ring operand of s + 2 to `rnew` after their reads;
// XWAIT after the reads, then everything of this wave's DMA after the MFMAs.
// The pair operand is A and the ring operand B, or the other way round with
// SWAP (what waves 4-7 send is read one phase later, so the deeper ring goes
// to whichever operand waits longer on memory; chosen per GEMM by
// measurement).
template <bool KSA, bool KSB, bool SWAP, int NBV, bool ISSUE_P, bool ISSUE_R, int XWAIT>
__device__ __forceinline__ void b_stage(const BCtx& c, char* pcur, char* pnxt, const char* rcur,
                                        char* rnew, int s, int g, uint4 (&fa)[kBKSteps][4],
                                        uint4 (&fb)[kBKSteps][kBFragB],
                                        f32x16 (&acc)[4][kBFragB]) {
  if (ISSUE_P && g == 0) b_issue<SWAP ? KSB : KSA>(c, pnxt, s + 1);
  if constexpr (SWAP) b_load<KSA, KSB, NBV>(c, rcur, pcur, fa, fb);
  else b_load<KSA, KSB, NBV>(c, pcur, rcur, fa, fb);
  if (ISSUE_R && g == 1) b_issue<SWAP ? KSA : KSB>(c, rnew, s + 2);
  wait_vmcnt<XWAIT>();
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  b_mfma_stage<NBV>(fa, fb, acc);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt<0>();
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// nk stages (a positive even number); the pair operand of stage s in a0/a1
// by s % 2, the ring operand in bring[s % 3].
template <bool KSA, bool KSB, bool SWAP, int NBV>
__device__ __forceinline__ void b_main_loop(const BCtx& c, char* a0, char* a1, char* bring,
                                            int nk, int g, f32x16 (&acc)[4][kBFragB]) {
  uint4 fa[kBKSteps][4], fb[kBKSteps][kBFragB];
  if (g == 0) {
    b_issue<SWAP ? KSB : KSA>(c, a0, 0);
  } else {
    b_issue<SWAP ? KSA : KSB>(c, bring, 0);
    b_issue<SWAP ? KSA : KSB>(c, bring + kBOper, 1);
  }
  wait_vmcnt<0>();
  lds_barrier();
  if (g == 1) lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  int bs = 0;
  auto bb = [&](int i) { return bring + i * kBOper; };
  auto inc3 = [](int i) { return i == 2 ? 0 : i + 1; };
  int s = 0;
  for (; s < nk - 2; s += 2) {
    const int b1 = inc3(bs), b2 = inc3(b1), b3 = inc3(b2);
    b_stage<KSA, KSB, SWAP, NBV, true, true, kBSlots>(c, a0, a1, bb(bs), bb(b2), s, g, fa, fb,
                                                      acc);
    b_stage<KSA, KSB, SWAP, NBV, true, true, kBSlots>(c, a1, a0, bb(b1), bb(b3), s + 1, g, fa,
                                                      fb, acc);
    bs = b2;
  }
  b_stage<KSA, KSB, SWAP, NBV, true, false, 0>(c, a0, a1, bb(bs), nullptr, s, g, fa, fb, acc);
  b_stage<KSA, KSB, SWAP, NBV, false, false, 0>(c, a1, a0, bb(inc3(bs)), nullptr, s + 1, g, fa,
                                                fb, acc);
  if (g == 0) lds_barrier();
}

// LDS byte offset, inside a KS tile, of the first 8-byte piece lane l reads
// for a fragment of class q (the fragment's first index / 32, mod 4) at
// k-step 0, first half: row 8 (l / 32) + (l % 16) / 4, column block
// (q ^ row % 4), chunk 2 ((l / 16) % 2) + (l % 4) / 2, 8 bytes into it when
// l is odd.
__device__ inline uint32_t ks_lane_base(int lane, int q) {
  const int r = lane & 15, G = lane >> 4;
  const int row = 8 * (G >> 1) + (r >> 2);
  const int low = 2 * (G & 1) + ((r & 3) >> 1);
  const int within = 8 * (r & 1);
  return (uint32_t)row * kKSRow + (uint32_t)((((q ^ (row & 3)) << 2) | low) << 4) + within;
}

}  // namespace

// Epilogue stores of the weight gradients (written once, never read by the
// layer) are non-temporal: measured on MI355X, dW_gate | dW_up 1.3% faster
// on the Mixtral prefill shape and 2.5% on the 64-expert top-8 one.  The
// a | b, Z and dX outputs, read again by the next kernels, keep the default
// policy (non-temporal there: even, or slower overall).
typedef uint32_t bwd_u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ void bwd_store16(void* p, uint4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(bwd_u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<bwd_u32x4*>(p));
  else
    *reinterpret_cast<uint4*>(p) = v;
}

template <bool KSA, bool KSB, int MODE, bool CBF16, bool SWAP>
__global__ __launch_bounds__(kBThreads, 1) void bwd_tile_kernel(BgArgs p) {
  __shared__ __attribute__((aligned(1024))) char sa0[kBOper];
  __shared__ __attribute__((aligned(1024))) char sa1[kBOper];
  __shared__ __attribute__((aligned(1024))) char sbr[3 * kBOper];

  // ---- tile.  Work-groups go to the XCDs round robin.  Mode 1: XCD x takes
  // the x-th contiguous share of each expert's tiles, expert by expert, so
  // that every XCD gets the same work however unevenly the rows are spread
  // over the experts (with skewed routing, one expert per XCD left two XCDs
  // with most of it).  Mode 0: XCD-contiguous ranges of all tiles, K part
  // slowest (each XCD then streams one weight matrix of dX, which its L2
  // serves better).  Then groups of feature tiles.
  const int L = blockIdx.x;
  int e = 0, part = 0, Lp;
  int ntb = p.n_bt;                         // token tiles of the tile order
  int ksub = -1;                            // K half of a split tile's part (-1: unsplit)
  int bt, at;
  if constexpr (MODE == 1) {
    const int xcd = L % kBXcds, li = L / kBXcds;
    e = li / p.per_xcd;                     // per_xcd: tiles per expert and XCD
    Lp = xcd * p.per_xcd + (li - e * p.per_xcd);
    if (e >= p.total || Lp >= p.n_at * p.n_bt) return;
  } else if (p.sched == nullptr) {
    Lp = (L % kBXcds) * p.per_xcd + L / kBXcds;  // per_xcd: tiles per XCD
    if (Lp >= p.total * p.n_at * p.n_bt) return;
    part = Lp / (p.n_at * p.n_bt);
    Lp -= part * p.n_at * p.n_bt;
  } else {
    // the unsplit token tiles' tiles in XCD-contiguous ranges as above, then
    // the quarters of the split ones (quarter slowest) to fill the last round
    const int sp = p.sched[0];
    ntb = *p.tb_count - sp;
    const int n_un = p.total * p.n_at * ntb;
    const int per = (n_un + kBXcds - 1) / kBXcds;
    if (L < per * kBXcds) {
      Lp = (L % kBXcds) * per + L / kBXcds;
      if (Lp >= n_un) return;
      part = Lp / (p.n_at * ntb);
      Lp -= part * p.n_at * ntb;
    } else {
      const int i = L - per * kBXcds;
      if (i >= 2 * p.total * p.n_at * sp) return;
      const int q = i / (p.n_at * sp), j = i - q * (p.n_at * sp);
      part = q >> 1;
      ksub = q & 1;
      bt = ntb + j / p.n_at;
      at = j % p.n_at;
    }
  }
  if (MODE == 1 && ntb > p.n_at) {
    // weight gradients whose B operand has more tiles than A (dW1 | dW3:
    // 2 d_ff / 256 tiles of dA | dB against d / 256 of x): groups of
    // kBWgradGroup B tiles with every A tile, the group's B tiles fastest, so
    // that each B panel of the expert is read by tiles that run together and
    // the narrower A operand is the one re-read.  Measured on MI355X against
    // the A groups below: dW1 | dW3 2-2.6% faster on prefill and 5.5-7% on
    // the 64-expert top-8 shape with groups of 8 (2 and 4: slower to even);
    // dW2, whose A (H g) is the wider, 3-6% slower with B groups.
    const int grp = Lp / (kBWgradGroup * p.n_at);
    const int rem = Lp - grp * kBWgradGroup * p.n_at;
    const int gsize = min(kBWgradGroup, ntb - grp * kBWgradGroup);
    at = rem / gsize;
    bt = grp * kBWgradGroup + rem % gsize;
  } else if (ksub < 0) {
    const int grp = Lp / (kBFeatGroup * ntb);
    const int rem = Lp - grp * kBFeatGroup * ntb;
    const int gsize = min(kBFeatGroup, p.n_at - grp * kBFeatGroup);
    bt = rem / gsize;
    at = grp * kBFeatGroup + rem % gsize;
  }

  int row0 = 0, rows = kBT, kn, koff = 0;
  if constexpr (MODE == 0) {
    if (bt >= *p.tb_count) return;
    e = p.tb_exp[bt];
    row0 = p.tb_row0[bt];
    rows = p.tb_rows[bt];
    kn = p.K;
    if (ksub >= 0) {                        // a quarter: half of the part's K
      kn = p.K / 2;
      koff = ksub * kn;
    }
  } else {
    kn = p.counts[e];
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave & 1, wt = wave >> 1, g = wave >> 2;

  BCtx c;
  c.dma_base = (wave & 3) * kBSlots;
  c.split_k = kn;
  c.kn = kn;
  // ---- the operand this wave fetches
  const int ga = SWAP ? 1 : 0;               // the wave group that sends A
  if (g == ga) {
    // A: aidx tile `at`
    const bf16_t* Am = part == 0 ? p.A0 : p.A1;
    int a_tile = at;
    if (at >= p.a_split_tile) { Am = p.A1; a_tile = at - p.a_split_tile; }
    c.ld_bytes = (uint32_t)p.lda * 2;
    if constexpr (MODE == 0) Am += (size_t)e * p.a_estride;
    if constexpr (KSA) {
      // mode 0: the K range [koff, koff + kn) of A's rows; A1 takes over at
      // row a_split_k (from its own first row), so a range can lie in A0, in
      // A1, or cross from one to the other
      size_t first_row = (size_t)koff;
      if constexpr (MODE == 1) first_row = (size_t)p.offsets[e];
      const bf16_t* A1m = p.A1 + (MODE == 0 ? (size_t)e * p.a_estride : 0);
      if (MODE == 0 && koff >= p.a_split_k) {
        Am = A1m;
        first_row = (size_t)(koff - p.a_split_k);
      }
      c.ks_base = reinterpret_cast<const char*>(Am + first_row * p.lda + (size_t)a_tile * kBT);
      c.ks_base1 = c.ks_base;
      if (koff < p.a_split_k && p.a_split_k < koff + kn) {
        c.split_k = p.a_split_k - koff;
        c.ks_base1 = reinterpret_cast<const char*>(A1m + (size_t)a_tile * kBT);
      }
    } else {
      c.r = buffer_rsrc(Am + (size_t)a_tile * kBT * p.lda, kBT * c.ld_bytes);
    }
  } else {
    // B: brow tile `bt`
    c.ld_bytes = (uint32_t)p.ldb * 2;
    if constexpr (MODE == 0) {
      // token rows row0 .. + rows (k contiguous); past them zeros
      c.r = buffer_rsrc(p.B + (size_t)row0 * p.ldb + (size_t)part * p.K + koff,
                   (uint32_t)rows * c.ld_bytes);
    } else {
      c.ks_base = reinterpret_cast<const char*>(p.B + (size_t)p.offsets[e] * p.ldb +
                                                (size_t)bt * kBT);
      c.ks_base1 = c.ks_base;
    }
  }
  // DMA offsets: KC slot j lane i -> row (dma_base + j) * 8 + i / 8, chunk
  // i % 8 (swizzled); KS slot j lane i -> k row 2 (dma_base + j) + i / 32,
  // chunk i % 32 (64-byte blocks swizzled by k row mod 4)
  const bool ks_mine = g == ga ? KSA : KSB;
#pragma unroll
  for (int j = 0; j < kBSlots; ++j) {
    const int q = (c.dma_base + j) * 64 + lane;
    if (!ks_mine) {
      const int r = q / 8, cs = q % 8;
      c.voff[j] = (uint32_t)r * c.ld_bytes + (uint32_t)((cs ^ kc_key(r)) * 16);
    } else {
      const int kr = q / 32, cs = q % 32;
      c.voff[j] = (uint32_t)kr * c.ld_bytes + (uint32_t)((cs ^ ((kr & 3) << 2)) * 16);
    }
  }
  // a KC slot holds 8 rows; only the token rows of mode 0 can run short
  c.on = g == ga || MODE != 0 || KSB || c.dma_base * 8 < rows;
  // fragment bases
  {
    const int r32 = lane & 31, h = lane >> 5;
    const uint32_t lrow = (uint32_t)r32 * kKCRow + (uint32_t)((h ^ kc_key(r32)) << 4);
    if constexpr (KSA) {
#pragma unroll
      for (int a = 0; a < 4; ++a) c.lA[a] = ks_lane_base(lane, a) + (uint32_t)wf * 256;
    } else {
      c.lA[0] = (uint32_t)(wf * 128) * kKCRow + lrow;
    }
    if constexpr (KSB) c.lB = ks_lane_base(lane, wt);
    else c.lB = (uint32_t)(wt * 32) * kKCRow + (lrow ^ (uint32_t)((4 * (wt & 1)) << 4));
  }
  int nbv = 0;
#pragma unroll
  for (int b = 0; b < kBFragB; ++b) nbv += wt * 32 + b * kBStrideB < rows;

  f32x16 acc[4][kBFragB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < kBFragB; ++b)
#pragma unroll
      for (int j = 0; j < 16; ++j) acc[a][b][j] = 0.f;

  // stages: whole, and an even count (a zero stage past the end is harmless)
  int nk = (kn + kBK - 1) / kBK;
  nk += nk & 1;
  if (nk > 0) {
    switch (nbv) {
      case 2: b_main_loop<KSA, KSB, SWAP, 2>(c, sa0, sa1, sbr, nk, g, acc); break;
      case 1: b_main_loop<KSA, KSB, SWAP, 1>(c, sa0, sa1, sbr, nk, g, acc); break;
      default: b_main_loop<KSA, KSB, SWAP, 0>(c, sa0, sa1, sbr, nk, g, acc); break;
    }
  }

  // ---- epilogue: lane holds B row wt * 32 + b * kBStrideB + lane % 32 and,
  // per (a, jj), four consecutive aidx
  const int r32 = lane & 31, half = lane >> 5;
  char* Cb;
  int brow_base;
  if constexpr (MODE == 0) {
    if (ksub == 1) {                        // a part's second half: its extra plane
      Cb = reinterpret_cast<char*>(p.C_extra) + (size_t)part * p.extra_pstride * (CBF16 ? 2 : 4);
      brow_base = row0 - p.sched[1];
    } else {
      Cb = reinterpret_cast<char*>(p.C0) + (size_t)part * p.c_pstride * (CBF16 ? 2 : 4);
      brow_base = row0;
    }
  } else {
    int bt_out = bt;
    Cb = reinterpret_cast<char*>(p.C0);
    if (bt >= p.c_split_tile) { Cb = reinterpret_cast<char*>(p.C1); bt_out = bt - p.c_split_tile; }
    Cb += (size_t)e * p.c_estride * (CBF16 ? 2 : 4);
    brow_base = bt_out * kBT;
  }
  if constexpr (CBF16) {
    // stage each 128-row half of the bf16 tile in LDS (rows of kStagePitch
    // bytes) and write whole rows of the tile's valid rows with 16-byte
    // stores
    constexpr int kStagePitch = kBT * 2 + 16;
    static_assert(128 * kStagePitch <= 3 * kBOper, "staging exceeds the B ring");
    __syncthreads();                      // every wave is past its last LDS read
#pragma unroll
    for (int b = 0; b < kBFragB; ++b) {
      const int lrow = wt * 32 + r32;     // row within this half
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int aidx = wf * 128 + a * 32 + jj * 8 + half * 4;
          const f32x16& v = acc[a][b];
          const uint32_t lo = pack_bf16x2(v[jj * 4], v[jj * 4 + 1]);
          const uint32_t hi = pack_bf16x2(v[jj * 4 + 2], v[jj * 4 + 3]);
          *reinterpret_cast<uint2*>(sbr + lrow * kStagePitch + aidx * 2) = make_uint2(lo, hi);
        }
      __syncthreads();
#pragma unroll
      for (int it = 0; it < 128 * (kBT * 2 / 16) / kBThreads; ++it) {
        const int q = it * kBThreads + tid;
        const int lrow = q / (kBT * 2 / 16), chunk = q % (kBT * 2 / 16);
        const int brow = b * kBStrideB + lrow;
        if (brow < rows) {
          const uint4 v =
              *reinterpret_cast<const uint4*>(sbr + lrow * kStagePitch + chunk * 16);
          const size_t off =
              (size_t)(brow_base + brow) * p.ldc + (size_t)at * kBT + chunk * 8;
          bwd_store16<MODE == 1>(reinterpret_cast<bf16_t*>(Cb) + off, v);
        }
      }
      __syncthreads();
    }
    return;
  } else {
    // fp32: stage (token fragment b, column half ch) = 128 rows x 128 columns
    // at a time in LDS, written by the waves of that half, then store whole
    // 512-byte row pieces of the tile's valid rows
    constexpr int kStagePitch = 128 * 4 + 16;
    static_assert(128 * kStagePitch <= 3 * kBOper, "staging exceeds the B ring");
    __syncthreads();                      // every wave is past its last LDS read
#pragma unroll
    for (int b = 0; b < kBFragB; ++b)
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        if (wf == ch) {
          const int lrow = wt * 32 + r32;
#pragma unroll
          for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int col = a * 32 + jj * 8 + half * 4;
              const f32x16& v = acc[a][b];
              *reinterpret_cast<float4*>(sbr + lrow * kStagePitch + col * 4) =
                  make_float4(v[jj * 4], v[jj * 4 + 1], v[jj * 4 + 2], v[jj * 4 + 3]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < 128 * 32 / kBThreads; ++it) {
          const int q = it * kBThreads + tid;
          const int lrow = q / 32, chunk = q % 32;
          const int brow = b * kBStrideB + lrow;
          if (brow < rows) {
            const uint4 v =
                *reinterpret_cast<const uint4*>(sbr + lrow * kStagePitch + chunk * 16);
            const size_t off = (size_t)(brow_base + brow) * p.ldc + (size_t)at * kBT + ch * 128 +
                               chunk * 4;
            bwd_store16<false>(reinterpret_cast<float*>(Cb) + off, v);
          }
        }
        __syncthreads();
      }
  }
}

namespace {

template <bool KSA, bool KSB, int MODE, bool CBF16, bool SWAP = false>
void bg_launch(BgArgs p, int groups, hipStream_t s) {
  p.total = groups;                                  // experts or K parts
  const int tiles = p.n_at * p.n_bt;
  p.per_xcd = MODE == 1 ? (tiles + kBXcds - 1) / kBXcds              // per expert
                        : (groups * tiles + kBXcds - 1) / kBXcds;    // all tiles
  // with a schedule, kCus more work-groups for the split tiles' extra K
  // halves (at most kCus / 2 beyond the tiles they replace; the rest exit)
  const int grid = p.per_xcd * kBXcds * (MODE == 1 ? groups : 1) + (p.sched ? kCus : 0);
  if (grid > 0) bwd_tile_kernel<KSA, KSB, MODE, CBF16, SWAP><<<grid, kBThreads, 0, s>>>(p);
}

BgArgs bg_rows_args(const int32_t* tb_count, const int32_t* tb_exp, const int32_t* tb_row0,
                    const int32_t* tb_rows, int max_tiles) {
  BgArgs p{};
  p.tb_count = tb_count;
  p.tb_exp = tb_exp;
  p.tb_row0 = tb_row0;
  p.tb_rows = tb_rows;
  p.n_bt = max_tiles;
  p.a_split_tile = 1 << 30;
  p.a_split_k = 1 << 30;
  p.c_split_tile = 1 << 30;
  p.kparts = 1;
  return p;
}

}  // namespace

static_assert(kBT == kBwdTileBT, "the plan's tile extent");

// a | b = [W1 | W3] x_r: one launch, aidx over 2 d_ff (W1's tiles, then W3's)
void launch_bwd_recompute(const Dims& D, const void* xs, const void* Wg, const void* Wu, void* ab,
                          int max_tiles, const int32_t* tb_count, const int32_t* tb_exp,
                          const int32_t* tb_row0, const int32_t* tb_rows, hipStream_t s) {
  BgArgs p = bg_rows_args(tb_count, tb_exp, tb_row0, tb_rows, max_tiles);
  p.A0 = (const bf16_t*)Wg;
  p.A1 = (const bf16_t*)Wu;
  p.a_estride = (size_t)D.f * D.d;
  p.lda = D.d;
  p.a_split_tile = D.f / kBT;
  p.B = (const bf16_t*)xs;
  p.ldb = D.d;
  p.C0 = ab;
  p.ldc = 2 * D.f;
  p.K = D.d;
  p.n_at = 2 * D.f / kBT;
  bg_launch<false, false, 0, true, true>(p, 1, s);
}

// Z = W2^T dOut_r: A = W2 read down its columns (index f, k = d)
void launch_bwd_z(const Dims& D, const void* dp, const void* Wd, void* z, int max_tiles,
                  const int32_t* tb_count, const int32_t* tb_exp, const int32_t* tb_row0,
                  const int32_t* tb_rows, hipStream_t s) {
  BgArgs p = bg_rows_args(tb_count, tb_exp, tb_row0, tb_rows, max_tiles);
  p.A0 = (const bf16_t*)Wd;
  p.A1 = p.A0;
  p.a_estride = (size_t)D.d * D.f;
  p.lda = D.f;
  p.B = (const bf16_t*)dp;
  p.ldb = D.d;
  p.C0 = z;
  p.ldc = D.f;
  p.K = D.d;
  p.n_at = D.f / kBT;
  bg_launch<true, false, 0, true>(p, 1, s);
}

// dX_r = W1^T dA + W3^T dB: A = [W1; W3] down its columns (index d, k = 2 d_ff)
void launch_bwd_dxs(const Dims& D, int parts, const void* dab, const void* Wg, const void* Wu,
                    float* dxs, size_t plane, float* dxs_extra, size_t extra_plane,
                    const int32_t* sched, int max_tiles, const int32_t* tb_count,
                    const int32_t* tb_exp, const int32_t* tb_row0, const int32_t* tb_rows,
                    hipStream_t s) {
  // parts = 2: the d_ff of W1, then that of W3, one plane each, twice the
  // work-groups of one pass (on prefill 4.5 rounds of the CUs instead of
  // 2.25); parts = 1: one K = 2 d_ff pass, A switching from W1 to W3 at d_ff
  BgArgs p = bg_rows_args(tb_count, tb_exp, tb_row0, tb_rows, max_tiles);
  p.A0 = (const bf16_t*)Wg;
  p.A1 = (const bf16_t*)Wu;
  p.a_estride = (size_t)D.f * D.d;
  p.lda = D.d;
  p.B = (const bf16_t*)dab;
  p.ldb = 2 * D.f;
  p.C0 = dxs;
  p.ldc = D.d;
  p.K = parts == 1 ? 2 * D.f : D.f;
  if (parts == 1) p.a_split_k = D.f;
  p.n_at = D.d / kBT;
  p.kparts = parts;
  p.c_pstride = plane;
  p.sched = sched;
  p.C_extra = dxs_extra;
  p.extra_pstride = extra_plane;
  bg_launch<true, false, 0, false>(p, parts, s);
}

// dW2[e] = Hg^T dOut over the expert's rows: C[o][f], A = Hg (index f),
// B = dOut rows (index o)
void launch_bwd_wgrad_down(const Dims& D, const void* dp, const void* hg, void* dWd,
                           const int32_t* counts, const int32_t* offsets, hipStream_t s) {
  BgArgs p = bg_rows_args(nullptr, nullptr, nullptr, nullptr, D.d / kBT);
  p.A0 = (const bf16_t*)hg;
  p.A1 = p.A0;
  p.lda = D.f;
  p.B = (const bf16_t*)dp;
  p.ldb = D.d;
  p.C0 = dWd;
  p.C1 = dWd;
  p.ldc = D.f;
  p.c_estride = (size_t)D.d * D.f;
  p.n_at = D.f / kBT;
  p.counts = counts;
  p.offsets = offsets;
  bg_launch<true, true, 1, true>(p, D.E, s);
}

// dW1[e] | dW3[e] = [dA | dB]^T x over the expert's rows: C[f][c] with brow
// over 2 d_ff (dW1's tiles, then dW3's), A = x (index c)
void launch_bwd_wgrad_gate_up(const Dims& D, const void* dab, const void* xs, void* dWg,
                              void* dWu, const int32_t* counts, const int32_t* offsets,
                              hipStream_t s) {
  BgArgs p = bg_rows_args(nullptr, nullptr, nullptr, nullptr, 2 * D.f / kBT);
  p.A0 = (const bf16_t*)xs;
  p.A1 = p.A0;
  p.lda = D.d;
  p.B = (const bf16_t*)dab;
  p.ldb = 2 * D.f;
  p.C0 = dWg;
  p.C1 = dWu;
  p.c_split_tile = D.f / kBT;
  p.ldc = D.d;
  p.c_estride = (size_t)D.f * D.d;
  p.n_at = D.d / kBT;
  p.counts = counts;
  p.offsets = offsets;
  bg_launch<true, true, 1, true, true>(p, D.E, s);
}

}  // namespace moe
