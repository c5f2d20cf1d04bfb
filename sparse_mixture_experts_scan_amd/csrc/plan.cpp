// Launch plan of the MoE layer (see plan.h): validation, GEMM-form choices
// and workspace layouts.  Host code only; touches no HIP API.
#include "plan.h"

#include <algorithm>
#include <cmath>
#include <cstring>

namespace moe {

namespace {

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int fail(std::string* why, int status, const char* msg) {
  if (why) *why = msg;
  return status;
}

// Sequential 256-byte-aligned carving of a workspace.
struct Carver {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align256(off + bytes);
    return o;
  }
};

}  // namespace

int router_splits_for(int nblk, int d, int E) {
  // split d_model over blocks until about one block per CU runs, two with
  // few experts (measured on MI355X with d_model 4096: for 8 experts, 512
  // blocks take T = 4096 from 44 to 34 us and T = 8192 from 70 to 52 us
  // against 256; for 64 experts, whose blocks each do 8 times the MFMA work,
  // 256 stay faster); each split keeps a whole number of 32-element k-groups
  // (the K of one bf16 MFMA 16x16x32 of the score kernel)
  const int min_blocks = E <= 16 ? 2 * kCus : kCus;
  const int groups = d / 32;
  int sp = 1;
  while (nblk * sp < min_blocks && sp * 2 <= kMaxRouterSplits && groups % (sp * 2) == 0)
    sp *= 2;
  return sp;
}

bool router_fuses_scan(const Dims& D) { return D.nblk == 1 && D.router_splits > 1; }

// bf16 tokens: the LDS-staged bf16 kernel (d_model % 128 == 0) and the INT4
// kernel (whose group rule already makes d_model a multiple of 128) read
// them in place; offsets into x are 32-bit
bool stream_gathers_in_place(const Dims& D) {
  return D.bf16 && (D.w4 || D.d % 128 == 0) && (int64_t)D.T * D.d * 2 < (int64_t(1) << 31);
}

bool tile_shape_ok(const Dims& D) {
  // buffer offsets are 32-bit: 256 rows of either K must stay below 2 GiB
  const int64_t kmax = D.d > D.f ? D.d : D.f;
  return D.bf16 && D.BT == kTileTokens && D.f % (kTileRows / 2) == 0 && D.d % kTileRows == 0 &&
         D.d % (kTileBK * kTileNS) == 0 && D.f % (kTileBK * kTileNS) == 0 &&
         kTileRows * kmax * 2 < (int64_t(1) << 31);
}

// Each K part of a split tile must be whole pairs of K stages.
int tile_down_splits(const Dims& D) {
  if (D.f % (4 * kTileBK * kTileNS) == 0) return 4;
  if (D.f % (2 * kTileBK * kTileNS) == 0) return 2;
  return 1;
}

// The scan splits whole token tiles whose parts fit one round of kCus
// work-groups: at most kCus / 2 tiles (two parts each), kCus / 2 / n_ft
// token tiles.
int tile_down_split_tiles(const Dims& D) {
  const int n_ft = D.d / kTileRows;
  return std::max(1, std::min(D.max_tiles, kCus / 2 / n_ft));
}

// Reading the tokens in place saves the scatter's copy of k rows per token
// but spreads each tile's token panel over x.  Measured on MI355X: with
// top-8 (E = 64) the step is 3.5% faster; with top-2 the gate/up GEMM loses
// about what the copy costs, so those keep the copy.
bool tile_gathers_in_place(const Dims& D) {
  return D.k >= 4 && (int64_t)D.T * D.d * 2 < (int64_t(1) << 31);
}

bool q4_group_ok(int K, int G) {
  if (G < 32 || G % 32 || K % G || K % kQ4Chunk) return false;
  return G % kQ4Chunk == 0 || kQ4Chunk % G == 0;
}

bool bwd_tile_shape_ok(int64_t d, int64_t f) { return d % kBwdTileBT == 0 && f % kBwdTileBT == 0; }

// The dX GEMM runs two K halves of each (token tile, feature tile); the
// token tiles of a partial last round may instead run four K quarters each,
// if those quarters fit one round: kCus / 4 per feature-tile row.
// split token tiles whose 2 * parts K pieces per feature tile fit one round
int bwd_dx_split_tiles(int64_t d, int parts) {
  return (int)(kCus / (2 * parts * (d / kBwdTileBT)));
}

// dX = W1^T dA + W3^T dB in one K = 2 d_ff pass when the token tiles alone
// (at least T k / 256 of them) fill about MOE_DX_ONE_PART_ROUNDS rounds of
// the CUs: each routed row's dX is then one fp32 plane, half the GEMM's
// stores and half the dx kernel's loads.  Fewer tiles: two K parts (the W1
// and the W3 half), twice the work-groups.
#ifndef MOE_DX_ONE_PART_ROUNDS
#define MOE_DX_ONE_PART_ROUNDS 4
#endif
int bwd_dx_parts(int64_t T, int64_t d, int32_t k) {
  const int64_t tiles = (T * k / kBwdTileBT) * (d / kBwdTileBT);
  return tiles >= (int64_t)MOE_DX_ONE_PART_ROUNDS * kCus ? 1 : 2;
}

int make_plan(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, int32_t dtype, bool block,
              Plan* p, std::string* why) {
  if (T < 1 || d < 1 || f < 1 || E < 1 || k < 1)
    return fail(why, MOE_ERR_INVALID_ARG, "T must be >= 0; d_model, d_ff, E and k >= 1");
  if (k > E) return fail(why, MOE_ERR_INVALID_ARG, "k must be <= E");
  if (dtype != MOE_BF16 && dtype != MOE_F32 && dtype != MOE_W4A16)
    return fail(why, MOE_ERR_INVALID_ARG, "unknown dtype");
  if (E > MOE_MAX_EXPERTS) return fail(why, MOE_ERR_UNSUPPORTED, "E > 64");
  if (k > MOE_MAX_TOPK) return fail(why, MOE_ERR_UNSUPPORTED, "k > 8");
  if (d % MOE_DIM_ALIGN || f % MOE_DIM_ALIGN)
    return fail(why, MOE_ERR_UNSUPPORTED, "d_model and d_ff must be multiples of 64");
  if (T > (int64_t(1) << 24)) return fail(why, MOE_ERR_UNSUPPORTED, "T > 2^24");
  if (d > 32768 || f > 131072)
    return fail(why, MOE_ERR_UNSUPPORTED, "d_model > 32768 or d_ff > 131072");

  Dims& D = p->D;
  D.T = (int)T;
  D.d = (int)d;
  D.f = (int)f;
  D.E = E;
  D.k = k;
  D.bf16 = dtype != MOE_F32;
  D.w4 = dtype == MOE_W4A16;
  D.group = 0;
  D.Epow2 = 1;
  while (D.Epow2 < E) D.Epow2 *= 2;
  D.nblk = (D.T + kRouterTokens - 1) / kRouterTokens;
  D.router_splits = router_splits_for(D.nblk, D.d, E);
  const int64_t A = T * k;                       // (token, slot) assignments
  const int64_t rows_avg = (A + E - 1) / E;
  // GEMM form: weight-streaming for few rows per expert (weights read once,
  // HBM-bound), LDS-tiled MFMA for many (compute-bound).
  D.BT = kTileTokens;
  int variant = 1;
  if (!(D.bf16 && rows_avg >= kTileMinRows && tile_shape_ok(D))) {
    variant = 0;
    D.BT = rows_avg <= 16 ? 16 : 32;
  }
  D.down_splits = 1;
  int64_t max_rows = A + (int64_t)E * (D.BT - 1);
  max_rows = (max_rows + D.BT - 1) / D.BT * D.BT;
  if (max_rows > (int64_t(1) << 30)) return fail(why, MOE_ERR_UNSUPPORTED, "too many rows");
  D.max_rows = (int)max_rows;
  D.max_tiles = (int)(max_rows / D.BT);
  if (variant == 1) D.down_splits = tile_down_splits(D);

  moe_ws_layout_t& L = p->L;
  std::memset(&L, 0, sizeof(L));
  L.block_rows = D.BT;
  L.max_rows = D.max_rows;
  L.router_blocks = D.nblk;
  L.gemm_variant = variant;
  L.down_splits = D.down_splits;
  L.tokens_in_place = variant == 1 ? tile_gathers_in_place(D) : stream_gathers_in_place(D);
  const size_t es = D.bf16 ? 2 : 4;
  Carver c;
  L.topk_idx = c.take(sizeof(int32_t) * A);
  L.topk_w = c.take(sizeof(float) * A);
  L.block_counts = c.take(sizeof(int32_t) * D.nblk * E);
  L.counts = c.take(sizeof(int32_t) * E);
  L.offsets = c.take(sizeof(int32_t) * (E + 1));
  L.num_tiles = c.take(sizeof(int32_t));
  L.tile_expert = c.take(sizeof(int32_t) * D.max_tiles);
  L.row_token = c.take(sizeof(int32_t) * D.max_rows);
  L.tok_row = c.take(sizeof(int32_t) * A);
  // the LDS-tiled down GEMM applies the gate weights and stores bf16 rows
  L.y_weighted = variant == 1;
  L.row_w = c.take(L.y_weighted ? sizeof(float) * D.max_rows : 0);
  // gathered rows only when the gate/up GEMM does not read the tokens in place
  L.xs = c.take(L.tokens_in_place ? 0 : es * D.max_rows * d);
  L.h = c.take(es * D.max_rows * f);
  L.y = c.take((L.y_weighted ? sizeof(uint16_t) : sizeof(float)) * D.max_rows * d);
  L.y_part_rows = D.down_splits > 1 ? (int64_t)tile_down_split_tiles(D) * D.BT : 0;
  L.y_parts = c.take(sizeof(float) * (D.down_splits - 1) * L.y_part_rows * d);
  L.down_sched = c.take(variant == 1 ? 2 * sizeof(int32_t) : 0);
  L.block_probs = c.take(sizeof(float) * D.nblk * E);
  // the normalised tokens and their 1/rms only for the block wrapper
  L.norm_rs = c.take(block ? sizeof(float) * T : 0);
  L.xn = c.take(block ? es * T * d : 0);
  L.router_partial = c.take(D.router_splits > 1 ? sizeof(float) * D.router_splits * D.nblk *
                                                      kRouterTokens * kRouterPartStride
                                                : 0);
  L.wdeq = c.take(D.w4 && variant == 1 ? sizeof(uint16_t) * 3 * (size_t)E * d * f : 0);
  L.total = c.off;
  return MOE_OK;
}

int make_bwd_plan(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, BwdPlan* b,
                  std::string* why) {
  Plan p;
  int st = make_plan(T, d, f, E, k, MOE_BF16, false, &p, why);
  if (st != MOE_OK) return st;
  if (d % 128 || f % 128)
    return fail(why, MOE_ERR_UNSUPPORTED, "the backward needs d_model and d_ff multiples of 128");
  // 32-bit buffer ranges: one expert's rows of the widest row-major operand
  if ((int64_t)T * std::max<int64_t>(2 * f, d) * 4 >= (int64_t(1) << 31))
    return fail(why, MOE_ERR_UNSUPPORTED,
                "T * max(2 d_ff, d_model) too large for the backward");
  Dims& D = b->D;
  D = p.D;
  D.BT = kBwdPadRows;
  const int64_t A = T * k;
  int64_t max_rows = A + (int64_t)E * (D.BT - 1);
  max_rows = (max_rows + D.BT - 1) / D.BT * D.BT;
  D.max_rows = (int)max_rows;
  D.max_tiles = (int)(max_rows / D.BT);
  D.down_splits = 1;
  b->max_tiles = (int)((A + kBwdRowTile - 1) / kBwdRowTile + E);
  const size_t R = (size_t)max_rows;
  Carver c;
  b->topk_idx = c.take(4 * A);
  b->topk_w = c.take(4 * A);
  b->block_counts = c.take(4 * (size_t)D.nblk * E);
  b->counts = c.take(4 * (size_t)E);
  b->offsets = c.take(4 * (size_t)(E + 1));
  b->num_tiles = c.take(4);
  b->tile_expert = c.take(4 * (size_t)D.max_tiles);
  b->row_token = c.take(4 * R);
  b->tok_row = c.take(4 * A);
  b->xs = c.take(2 * R * d);
  b->logits = c.take(4 * (size_t)T * E);
  b->router_partial = c.take(D.router_splits > 1 ? sizeof(float) * D.router_splits * D.nblk *
                                                       kRouterTokens * kRouterPartStride
                                                 : 0);
  b->ab = c.take(2 * R * 2 * f);   // bf16 a | b
  b->z = c.take(2 * R * f);        // bf16 Z
  b->dab = c.take(2 * R * 2 * f);
  b->hg = c.take(2 * R * f);
  b->dp = c.take(2 * R * d);
  b->dxs = c.take(4 * 2 * R * d);   // two planes: the W1 and W3 halves of dX
  // (the tiled form with one K part uses the first)
  b->dx_parts = bwd_tile_shape_ok(d, f) ? bwd_dx_parts(T, d, k) : 2;
  // one more per part for the split token tiles' second K halves (tiled
  // form): their rows span at most the tiles plus the padding between experts
  b->dx_max_split = bwd_tile_shape_ok(d, f) ? bwd_dx_split_tiles(d, b->dx_parts) : 0;
  b->dx_split_rows = b->dx_max_split * (kBwdTileBT + kBwdPadRows);
  b->dxs_extra = c.take(4 * (size_t)b->dx_parts * b->dx_split_rows * d);
  b->dg = c.take(4 * R);
  b->ds = c.take(4 * (size_t)T * E);
  b->wpart = c.take(4 * (size_t)kBwdRouterSlices * (d + 1) * E);
  b->tb = c.take(4 * (size_t)(1 + 3 * b->max_tiles + 2));
  b->total = c.off;
  return MOE_OK;
}

}  // namespace moe
