// Host-side launchers of the MoE kernels (internal to libmoe_ffn.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.h"

namespace moe {


// INT4 weights of one matrix stack: packed codes and float32 scales
struct Q4Weights {
  const void* q;
  const float* s;
};

// a1: scores, top-k, softmax over the k, per-block expert histogram
// block wrapper: rs[t] = 1/rms(x[t]), xn = x * rs * weight (element type)
void launch_rmsnorm(const Dims& D, const void* x, const float* weight, float eps, float* rs,
                    void* xn, hipStream_t s);
// blk_prob: [nblk][E] per-block full-softmax probability sums, or NULL.
// gamma, rs (both or neither): scores of the RMS-normalised tokens,
// rs[t] * sum_j x[t][j] gamma[j] W[j][e]
// logits_out: [T][E] final scores (with bias), or NULL.
// outputs of the expert scan (a2, part 1); counts_out, prob_out, loss_out
// may be NULL
struct ScanArgs {
  int32_t* counts;
  int32_t* offsets;
  int32_t* num_tiles;
  int32_t* tile_expert;
  int32_t* row_token;
  int32_t* counts_out;
  float* prob_out;
  float* loss_out;
  // with a single router block: non-NULL makes the select pass also write the
  // row maps (tok_row, row_token), for a GEMM that reads the tokens in place
  int32_t* tok_row;
  // LDS-tiled form: the down GEMM's schedule (K parts in use, first split
  // row), from the token tiles in use, its feature tiles and the most parts
  // the plan allows; NULL otherwise
  int32_t* down_sched;
  int down_n_ft;
  int down_max_parts;
};
// With a single router block (router_fuses_scan) the select pass also runs
// the expert scan and launch_scan is a no-op, which saves a launch for small T.
void launch_router(const Dims& D, const void* x, const float* Wr, const float* bias,
                   int32_t* idx, float* w, int32_t* blk_counts, float* part, float* blk_prob,
                   const float* gamma, const float* rs, float* logits_out, const ScanArgs& sa,
                   hipStream_t s);
// a2: histogram reduce, padded offsets, per-block bases, tile table
// router statistics (when blk_prob is non-NULL): prob_out [E], loss_out [1]
void launch_scan(const Dims& D, int32_t* blk_counts, const ScanArgs& sa, const float* blk_prob,
                 hipStream_t s);
// a2: stable row maps and gather of x into expert-contiguous rows (xs NULL:
// the row maps only)
// (row_w non-NULL: also the gate weight w of each row)
void launch_scatter(const Dims& D, const void* x, const int32_t* idx, const float* w,
                    const int32_t* blk_base, const int32_t* offsets, int32_t* tok_row,
                    int32_t* row_token, float* row_w, void* xs, hipStream_t s);
// a3 + a4: grouped GEMMs, weight-streaming form (few rows per expert).
// row_token NULL: act is the gathered rows (xs); else act is x (or xn) and
// each row's token comes from row_token (only when stream_gathers_in_place).
void launch_gateup_stream(const Dims& D, const void* act, const int32_t* row_token,
                          const void* Wg, const void* Wu, void* h, const int32_t* counts,
                          const int32_t* offsets, const int32_t* num_tiles,
                          const int32_t* tile_expert, hipStream_t s);
void launch_down_stream(const Dims& D, const void* h, const void* Wd, float* y,
                        const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                        const int32_t* tile_expert, hipStream_t s);
// a3 + a4: grouped GEMMs, LDS-tiled MFMA form (many rows per expert, bf16)
// row_token non-NULL: `x` is the token matrix [T][d] and each tile gathers its
// rows through row_token; NULL: `x` is the gathered Xs
void launch_gateup_tile(const Dims& D, const void* x, const int32_t* row_token, const void* Wg,
                        const void* Wu, void* h, const int32_t* counts, const int32_t* offsets,
                        const int32_t* num_tiles, const int32_t* tile_expert, hipStream_t s);
// y: the first K part of every row; y_parts: [D.down_splits - 1][part_rows]
// further parts of the split token tiles' rows (see down_sched)
// (y: bf16 rows times their gate weight row_w; y_parts float32, weighted)
void launch_down_tile(const Dims& D, const void* h, const void* Wd, void* y, float* y_parts,
                      int64_t part_rows, const int32_t* down_sched, const float* row_w,
                      const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                      const int32_t* tile_expert, hipStream_t s);
// INT4 expert weights: quantizer, dequantizer (to bf16, for the tiled form)
// and the weight-streaming GEMMs that read INT4 directly
// rows = batch * N matrices rows; scales group-major per matrix ([K/G][N])
void launch_quantize_int4(const void* W, bool bf16, int64_t rows, int N, int K, int G,
                          void* packed, float* scales, hipStream_t s);
void launch_dequant_int4(const void* packed, const float* scales, int64_t rows, int N, int K,
                         int G, void* out, hipStream_t s);
// row_token as for launch_gateup_stream
void launch_gateup_q4(const Dims& D, const void* act, const int32_t* row_token,
                      const Q4Weights& Wg, const Q4Weights& Wu, void* h, const int32_t* counts,
                      const int32_t* offsets, const int32_t* num_tiles,
                      const int32_t* tile_expert, hipStream_t s);
void launch_down_q4(const Dims& D, const void* h, const Q4Weights& Wd, float* y,
                    const int32_t* counts, const int32_t* offsets, const int32_t* num_tiles,
                    const int32_t* tile_expert, hipStream_t s);
// backward (bf16): grouped GEMMs and the steps around them
// (and the dX schedule in sched[2] for a dX GEMM of dx_parts K parts; at
// most max_split split token tiles)
void launch_bwd_tile_table(const Dims& D, const int32_t* counts, const int32_t* offsets,
                           int max_tiles, int max_split, int dx_parts, int32_t* tb_count,
                           int32_t* tb_exp, int32_t* tb_row0, int32_t* tb_rows, int32_t* sched,
                           hipStream_t s);
void launch_bwd_gather(const Dims& D, const void* src, const int32_t* row_token, void* dst,
                       hipStream_t s);
// C[rows of tile][N] (+)= A[rows][K] (k contiguous) x B_e, per tile of the table
void launch_bwd_gemm_rows(const void* A, int lda, const void* B, int ldb, bool b_kcontig,
                          size_t b_estride, void* C, bool c_bf16, int ldc, int M, int N,
                          int K, bool accumulate, int max_tiles, const int32_t* tb_count,
                          const int32_t* tb_exp, const int32_t* tb_row0, const int32_t* tb_rows,
                          hipStream_t s);
// Backward GEMMs on 256 x 256 tiles (d_model and d_ff multiples of 256):
// one launch each for a | b, Z, dX (both terms), dW2, and dW1 | dW3.
void launch_bwd_recompute(const Dims& D, const void* xs, const void* Wg, const void* Wu, void* ab,
                          int max_tiles, const int32_t* tb_count, const int32_t* tb_exp,
                          const int32_t* tb_row0, const int32_t* tb_rows, hipStream_t s);
void launch_bwd_z(const Dims& D, const void* dp, const void* Wd, void* z, int max_tiles,
                  const int32_t* tb_count, const int32_t* tb_exp, const int32_t* tb_row0,
                  const int32_t* tb_rows, hipStream_t s);
// dX in `parts` K parts (1: K = 2 d_ff; 2: the W1 and the W3 half), one plane
// each; the split token tiles of sched run each part as two K halves, the
// second half of each part into its extra plane (row r at r - sched[1])
void launch_bwd_dxs(const Dims& D, int parts, const void* dab, const void* Wg, const void* Wu,
                    float* dxs, size_t plane, float* dxs_extra, size_t extra_plane,
                    const int32_t* sched, int max_tiles, const int32_t* tb_count,
                    const int32_t* tb_exp, const int32_t* tb_row0, const int32_t* tb_rows,
                    hipStream_t s);
void launch_bwd_wgrad_down(const Dims& D, const void* dp, const void* hg, void* dWd,
                           const int32_t* counts, const int32_t* offsets, hipStream_t s);
void launch_bwd_wgrad_gate_up(const Dims& D, const void* dab, const void* xs, void* dWg,
                              void* dWu, const int32_t* counts, const int32_t* offsets,
                              hipStream_t s);
void launch_bwd_gemm_wgrad(const Dims& D, const void* A, int lda, const void* B, int ldb,
                           void* C, int M, int N, const int32_t* counts, const int32_t* offsets,
                           hipStream_t s);
void launch_bwd_rows(const Dims& D, const void* AB, const void* Z, const int32_t* row_token,
                     const int32_t* tok_row, const float* gates, float* dg, void* dAB, void* Hg,
                     hipStream_t s);
void launch_bwd_router(const Dims& D, const float* logits, const int32_t* idx, const float* gates,
                       const int32_t* tok_row, const float* dg_row, const int32_t* counts,
                       float alpha, float* ds, hipStream_t s);
void launch_bwd_router_wgrad(const Dims& D, const void* x, const float* ds, float* part,
                             float* dWr, float* dbias, hipStream_t s);
// dX holds `nplanes` planes (1, or 2: the W1 and W3 halves of the
// contraction), `plane` elements apart, plus (sched non-NULL, sched[0] > 0)
// as many extra planes for the split rows, `extra_plane` apart
void launch_bwd_dx(const Dims& D, int nplanes, const float* dX, size_t plane,
                   const float* dX_extra, size_t extra_plane, const int32_t* sched,
                   const int32_t* tok_row, const float* Wr, const float* ds, void* dx,
                   hipStream_t s);
void launch_zero_fill(void* p, size_t bytes, hipStream_t s);
// a5: gate-weighted gather-sum back to token order
// resid: x for the block wrapper (out = x + layer), or NULL
// T = 0: zero the optional statistics outputs (any may be null).
void launch_empty_stats(int E, int32_t* counts_out, float* prob_out, float* loss_out,
                        hipStream_t s);

// y_parts / down_sched as for launch_down_tile (down_sched NULL: y alone).
// weighted: y is bf16 and already carries the gate weights (the LDS-tiled
// form); else float32 and the combine applies w
void launch_combine(const Dims& D, const void* y, bool weighted, const float* y_parts,
                    int64_t part_rows, const int32_t* down_sched, const int32_t* tok_row,
                    const float* w, const void* resid, void* out, hipStream_t s);

}  // namespace moe
