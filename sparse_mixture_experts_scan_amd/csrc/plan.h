// Launch plan of the MoE layer: shape validation, the choice of GEMM forms,
// and the workspace layouts of the forward and backward passes.  Plain C++
// with no HIP types, so the same code is built into the library (by hipcc)
// and, for the CPU tests, into a host program under the address and
// undefined-behaviour sanitizers (by g++).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>

#include "moe_ffn.h"

namespace moe {

// ---- sizes shared by the plan and the kernels
constexpr int kRouterTokens = 32;      // tokens per router / scatter block
constexpr int kRouterPartStride = 64;  // floats per token row of the split router's partials
#ifndef MOE_ROUTER_MAX_SPLITS
#define MOE_ROUTER_MAX_SPLITS 16       // d_model splits of the score GEMM at most
#endif
constexpr int kMaxRouterSplits = MOE_ROUTER_MAX_SPLITS;
constexpr int kTileTokens = 256;       // token tile of the LDS-tiled form (= padding unit)
constexpr int kTileRows = 256;         // weight rows per tile of the LDS-tiled form
constexpr int kTileBK = 64;            // K per LDS stage of the LDS-tiled form
constexpr int kTileNS = 2;             // its K loop runs stages in pairs
constexpr int kQ4Chunk = 128;          // K per 16-byte INT4 weight load of a 4-lane row group
#ifndef MOE_BG_M
#define MOE_BG_M 256                   // row tile of the generic backward GEMM
#endif
constexpr int kBwdRowTile = MOE_BG_M;
constexpr int kBwdTileBT = 256;        // tile extent of the 256 x 256 backward GEMMs
constexpr int kBwdPadRows = 16;        // padding unit of the backward's expert segments
constexpr int kBwdRouterSlices = 32;   // token slices of the router weight gradient
constexpr int kTileMinRows = 96;       // average rows per expert from which the tiled form runs
constexpr int kCus = 256;              // compute units the tile schedules fill (MI355X)

struct Dims {
  int T, d, f, E, k;   // tokens, d_model, d_ff, experts, top-k
  int Epow2;           // smallest power of two >= E
  int nblk;            // router / scatter blocks (kRouterTokens tokens each)
  int BT;              // token tile = padding unit of expert segments
  int max_rows;        // rows reserved for the permuted layout
  int max_tiles;       // max_rows / BT
  int down_splits;     // K parts into which the down GEMM may split a token tile (1: never)
  int router_splits;   // d_model splits of the router scores (1 = fused kernel)
  bool bf16;           // element type of x / weights / out
  bool w4;             // expert weights in INT4 (bf16 activations)
  int group;           // INT4 scale group (input features per scale)
};

// ---- decisions the plan takes (also used by the launchers)
int router_splits_for(int nblk, int d, int E);
// with a single router block the select pass also runs the expert scan
bool router_fuses_scan(const Dims& D);
// whether the weight-streaming gate/up GEMM reads the tokens in place
bool stream_gathers_in_place(const Dims& D);
bool tile_shape_ok(const Dims& D);
// K parts into which the tiled down GEMM may split the token tiles of a
// partial last round (see expert_scan_kernel's schedule): 4 or 2 when d_ff
// splits into whole pairs of K stages, else 1
int tile_down_splits(const Dims& D);
// token tiles whose down-GEMM parts the extra Y planes hold at most
int tile_down_split_tiles(const Dims& D);
// whether the tiled gate/up GEMM reads the tokens in place
bool tile_gathers_in_place(const Dims& D);
bool q4_group_ok(int K, int G);
constexpr int q4_quantize_max_k() { return 65536; }
bool bwd_tile_shape_ok(int64_t d, int64_t f);
// token tiles whose dX work the tiled backward may split into K quarters to
// fill a partial last round of work-groups (0: never)
int bwd_dx_split_tiles(int64_t d, int parts);
// K parts of the tiled dX GEMM (1 or 2) for T tokens, top-k and d_model
int bwd_dx_parts(int64_t T, int64_t d, int32_t k);

// ---- forward plan
struct Plan {
  Dims D;
  moe_ws_layout_t L;
};
// Validates a forward shape and builds its plan.  block: the normalised
// block wrapper (reserves the normalised tokens and their 1/rms).  Returns a
// moe_status_t; on failure *why holds the reason.
int make_plan(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, int32_t dtype, bool block,
              Plan* p, std::string* why);

// ---- backward plan: the forward routing and permutation (16-row padding),
// the recomputed pre-activations and every gradient intermediate (byte
// offsets into the workspace)
struct BwdPlan {
  Dims D;
  int max_tiles;     // rows of the row-tile table
  int dx_parts;      // K parts of the tiled dX GEMM, one fp32 plane each (1 or 2)
  int dx_max_split;  // token tiles the dX schedule may split (0: none)
  int dx_split_rows; // rows of each extra dX plane (the split token tiles' span)
  // tb: [1 + 3 max_tiles + 2] int32: count, experts, first rows, row counts,
  // then the dX schedule (split token tiles, first row of the first one)
  size_t topk_idx, topk_w, block_counts, counts, offsets, num_tiles, tile_expert, row_token,
      tok_row, xs, logits, router_partial, ab, z, dab, hg, dp, dxs, dxs_extra, dg, ds, wpart, tb,
      total;
};
int make_bwd_plan(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, BwdPlan* b,
                  std::string* why);

}  // namespace moe
