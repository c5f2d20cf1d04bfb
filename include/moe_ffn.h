/*
 * moe_ffn.h -- C ABI of the sparse Mixture-of-Experts feed-forward layer for
 * AMD Instinct MI355X (gfx950): the forward pass (bf16 or fp32), its
 * normalised-block wrapper, INT4 expert weights, and the backward pass.
 *
 * The layer ("Mistral/Mixtralのアーキテクチャ", disassemble-channel.com,
 * section "Top-2ゲーティングの定式化" and section "各エキスパートの構造";
 * "Mixtral of Experts", singularity-lens.com, the layer-output formula):
 *
 *   s_t      = x_t . W_router  (+ bias)                 router scores, [E]
 *   i_t1..k  = the k largest scores, descending; equal scores -> lower index
 *   g_tj     = exp(s_t,ij) / sum_l exp(s_t,il)           softmax over the k only
 *   E_e(x)   = W_down[e] (SiLU(W_gate[e] x) * W_up[e] x), SiLU(z) = z sigma(z)
 *   out_t    = sum_j g_tj E_ij(x_t)                      summed in slot order
 *
 * W_gate, W_up, W_down are the page's W1, W3, W2.  Every token is routed to
 * exactly k experts; nothing is dropped.  The router bias is an extension
 * (the pages' router has none) used to build skewed routing.
 *
 * Conventions for every entry point:
 *  - Tensor arguments are DEVICE pointers, row-major and contiguous, owned by
 *    the caller; x, W_router, W_gate, W_up, W_down and out 16-byte aligned,
 *    the bias and the optional outputs 4-byte aligned.  The library never
 *    frees them and keeps no reference after the work it enqueued has run.
 *  - Calls are asynchronous on the given stream (NULL = the default stream);
 *    device faults surface at the caller's next synchronisation.  No entry
 *    point synchronises with the host or calls hipMemset once its workspace
 *    exists, so a call with a caller-owned workspace can be captured into a
 *    HIP graph.
 *  - Workspace: a call that passes none uses one library-owned buffer per
 *    device, shared by every such call and grown on demand (growing
 *    synchronises the device).  Calls sharing it must be ordered (one stream,
 *    or synchronised between streams); concurrent calls on different streams
 *    must each pass their own workspace.
 *  - Arguments are validated on the host before any HIP call; a failed
 *    validation enqueues nothing.  Non-finite inputs give undefined results.
 *  - Return value: a moe_status_t.  On MOE_ERR_HIP, moe_last_error() holds
 *    the HIP error text (thread-local, valid until the next call on that
 *    thread); other failures also leave a short reason there.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, size out of range, k > E, ...  */
  MOE_ERR_UNSUPPORTED = 2, /* legal layer, but outside the library's limits */
  MOE_ERR_WORKSPACE = 3,   /* caller workspace too small or misaligned      */
  MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed    */
} moe_status_t;

/* Element type of x, W_gate, W_up, W_down and out.  W_router, the bias and
 * all accumulation are always float32.  MOE_W4A16 names the layer of
 * moe_ffn_forward_int4 (bf16 activations, INT4 expert weights) for the
 * workspace queries. */
typedef enum { MOE_BF16 = 0, MOE_F32 = 1, MOE_W4A16 = 2 } moe_dtype_t;

/* Limits (checked; MOE_ERR_UNSUPPORTED beyond them). */
#define MOE_MAX_EXPERTS 64
#define MOE_MAX_TOPK 8
#define MOE_DIM_ALIGN 64 /* d_model and d_ff must be multiples of this */

typedef struct moe_opts {
  int32_t dtype;              /* moe_dtype_t; default MOE_BF16                   */
  void* stream;               /* hipStream_t; NULL = default stream              */
  const float* router_bias;   /* [E] fp32 device pointer or NULL                 */
  void* workspace;            /* device buffer, 256-byte aligned, or NULL: then a
                                 library-owned buffer (per device, grown on demand,
                                 freed by moe_release) is used                   */
  size_t workspace_bytes;     /* size of `workspace`                             */
  int32_t* topk_idx_out;      /* [T][k] device or NULL: selected expert ids       */
  float* topk_w_out;          /* [T][k] device or NULL: their gate weights        */
  int32_t* expert_counts_out; /* [E] device or NULL: tokens routed to each expert */
  float* router_prob_out;     /* [E] device or NULL: router statistics p_i, the mean
                                 over tokens of the full softmax of the scores over
                                 all E experts ("ロードバランス損失")                */
  float* balance_loss_out;    /* [1] device or NULL: N * sum_i f_i p_i with
                                 f_i = tokens routed to i / T; times alpha this is
                                 the auxiliary load-balancing loss                */
  void* const* stage_events;  /* NULL, or MOE_NUM_STAGES + 1 hipEvent_t recorded on
                                 the stream before the first kernel and after each
                                 stage (router, scan, scatter, gate/up, down,
                                 combine), for per-kernel timing                 */
} moe_opts_t;

#define MOE_NUM_STAGES 6

/* Fill `opts` with the defaults (bf16, default stream, no bias, library
 * workspace, no extra outputs). */
void moe_opts_init(moe_opts_t* opts);

/*
 * The whole layer: router -> top-k -> gates -> permutation -> grouped
 * gate/up GEMM with SiLU(gate)*up -> grouped down GEMM -> gate-weighted
 * combine.  Matches the module call on "Mistral/Mixtralのアーキテクチャ",
 * section "MoEレイヤー全体の実装": out has x's shape and dtype, tokens
 * flattened to T = batch * seq_len.
 *
 *   x         [T][d_model]             dtype
 *   W_router  [d_model][E]             float32
 *   W_gate    [E][d_ff][d_model]       dtype  (W1, nn.Linear [out][in] layout)
 *   W_up      [E][d_ff][d_model]       dtype  (W3)
 *   W_down    [E][d_model][d_ff]       dtype  (W2)
 *   out       [T][d_model]             dtype  (written, never read)
 *   0 <= T <= 2^24; 1 <= k <= E <= 64; k <= 8; d_model, d_ff multiples of 64.
 *   opts      NULL = defaults.
 * T = 0 (an empty batch) is valid: nothing is read or written except the
 * optional statistics, which become zero counts, zero p_i and a zero loss.
 */
int moe_ffn_forward(const void* x, const float* W_router, const void* W_gate,
                    const void* W_up, const void* W_down, void* out, int64_t T,
                    int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                    const moe_opts_t* opts);

/*
 * moe_ffn_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * it calls no hipMalloc, hipFree or other allocating routine.  Arguments,
 * outputs, layouts and errors as moe_ffn_forward, except that
 * opts->workspace must be NULL: the intermediates live in a fixed array of
 * MOE_NOALLOC_SCRATCH_BYTES (64 MiB) of device memory that the library holds
 * on every GPU it runs on until the process ends.  That covers the layer's
 * workspace (moe_ffn_workspace_size) for decode-sized batches, e.g. T <= 256
 * at the Mixtral 8x7B shape; a larger shape returns MOE_ERR_WORKSPACE before
 * anything is enqueued.  Every call on one GPU shares that GPU's array, which
 * keeps the last call's contents (nothing in it needs clearing): calls that
 * overlap on one GPU (unordered streams, or several host threads) race and
 * give undefined results.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int moe_ffn_forward_noalloc(const void* x, const float* W_router, const void* W_gate,
                            const void* W_up, const void* W_down, void* out, int64_t T,
                            int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                            const moe_opts_t* opts);

/*
 * One MoE sub-block of a Mixtral transformer block: out = x + layer(RMSNorm(x)).
 * "Mistral/Mixtralのアーキテクチャ", section "Mixtralのアーキテクチャ",
 * lists the second half of each block as normalisation, then the MoE layer,
 * then a residual connection.  The pages name RMSNorm without a formula; the
 * plain (LLaMA) definition is taken: RMSNorm(x)[t][j] =
 * x[t][j] / sqrt(mean_j x[t][j]^2 + eps) * norm_weight[j].
 *   norm_weight [d_model] float32 device, 4-byte aligned; 0 <= eps <= 1.
 * The router scores the normalised tokens in fp32 (from x, norm_weight and
 * the per-token 1/rms); the experts take the normalised tokens rounded to
 * the element type; the residual is added in fp32 before the single rounding
 * of out.  out must not alias x.  A caller workspace is sized by
 * moe_block_workspace_size (the layer's plus the normalised tokens and their
 * 1/rms).  Other arguments, outputs, limits and errors as moe_ffn_forward.
 */
int moe_block_forward(const void* x, const float* norm_weight, float eps, const float* W_router,
                      const void* W_gate, const void* W_up, const void* W_down, void* out,
                      int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                      const moe_opts_t* opts);

/*
 * Weight-only INT4 quantisation of weight rows.  "Mixtral of Experts"
 * (singularity-lens.com), list of limitations, memory item: the model fits
 * in about 25-30 GB only with INT4 weights.  The pages fix no scheme; this
 * library's (symmetric, per group of `group` consecutive input features):
 *   s = max |w| / 7 over the group, q = clamp(rint(w / s), -8, 7), q = 0 when
 *   s = 0, both decided in float32 with IEEE division and ties to even;
 *   the weight stands for s * q.
 *   W       [batch][N][K] dtype (MOE_BF16 or MOE_F32), device, 16-byte aligned
 *   packed  [batch][N][K/2] uint8, device, 4-byte aligned (written): nibble
 *           q + 8; element 2b in the low nibble of byte b, 2b + 1 in the high
 *   scales  [batch][K/group][N] float32, device, 4-byte aligned (written):
 *           group-major, the scales of one group of neighbouring rows adjacent
 *   group: multiple of 32 dividing K, and either a multiple of 128 or 32/64;
 *   K a multiple of 128 and at most 65536; batch * N <= 2^31 - 1.
 * For an expert stack W_gate [E][d_ff][d_model] pass batch = E, N = d_ff,
 * K = d_model (W_down: N = d_model, K = d_ff).  Asynchronous on `stream`
 * (hipStream_t, NULL = default); validation as moe_ffn_forward.
 */
int moe_quantize_int4(const void* W, int32_t dtype, int64_t batch, int64_t N, int64_t K,
                      int32_t group, uint8_t* packed, float* scales, void* stream);

/*
 * The layer of moe_ffn_forward with INT4 expert weights as written by
 * moe_quantize_int4 (each expert matrix s * q); x and out bf16.
 *   Wg_q, Wu_q [E][d_ff][d_model/2] uint8, Wg_s, Wu_s [E][d_model/group][d_ff]
 *   Wd_q [E][d_model][d_ff/2] uint8, Wd_s [E][d_ff/group][d_model] float32
 * (16-byte aligned codes, 4-byte aligned scales); group as for
 * moe_quantize_int4 and dividing both d_model and d_ff, which must be
 * multiples of 128.  Few rows per expert (decode): the weight-streaming GEMMs
 * read the INT4 codes directly.  Many rows: the three stacks are first
 * dequantized to bf16 into the workspace (layout field wdeq, 6 * E * d_model
 * * d_ff bytes) and the LDS-tiled GEMMs run on them.  opts->dtype is ignored;
 * workspace sizes are those of MOE_W4A16.  Other arguments, outputs and
 * errors as moe_ffn_forward.
 */
int moe_ffn_forward_int4(const void* x, const float* W_router, const uint8_t* Wg_q,
                         const float* Wg_s, const uint8_t* Wu_q, const float* Wu_s,
                         const uint8_t* Wd_q, const float* Wd_s, int32_t group, void* out,
                         int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                         const moe_opts_t* opts);

/*
 * Backward pass of moe_ffn_forward (bf16 tensors): the gradients of
 *   L = <dout, out> + alpha * N * sum_i f_i p_i
 * ("Mistral/Mixtralのアーキテクチャ", section "ロードバランス損失": the
 * training loss adds the balance loss to the language-model loss, whose
 * gradient above the layer is dout).  f_i (the top-k counts over T) is
 * piecewise constant, so the balance term reaches only the router scores
 * through p_i.  The routing, the permutation and the pre-activations are
 * recomputed from x (nothing is kept from a forward call).
 *   x, W_router, W_gate, W_up, W_down, T .. k: as moe_ffn_forward, bf16
 *   dout        [T][d_model] bf16 device: gradient of the loss w.r.t. out
 *   alpha       >= 0, the balance-loss weight (0: no balance term)
 *   dx          [T][d_model] bf16 (written)
 *   dW_router   [d_model][E] float32 (written); dbias [E] float32 or NULL:
 *               the gradient w.r.t. an additive router bias (opts->router_bias)
 *   dW_gate, dW_up [E][d_ff][d_model], dW_down [E][d_model][d_ff] bf16 (written)
 * d_model and d_ff must be multiples of 128.  opts: dtype must be MOE_BF16;
 * stream, router_bias and workspace as for the forward, the workspace sized by
 * moe_ffn_backward_workspace_size; routing and statistics outputs are not
 * written; stage_events, if given, holds MOE_BWD_NUM_STAGES + 1 events
 * (routing, recompute, Z = W2^T dout, row/router gradients, dX GEMMs, dx,
 * dW_down, dW_gate and dW_up).  T = 0 writes zero weight gradients.
 * Deterministic: fixed summation orders, no atomics.
 */
#define MOE_BWD_NUM_STAGES 8
int moe_ffn_backward(const void* x, const float* W_router, const void* W_gate,
                     const void* W_up, const void* W_down, const void* dout, float alpha,
                     void* dx, float* dW_router, float* dbias, void* dW_gate, void* dW_up,
                     void* dW_down, int64_t T, int64_t d_model, int64_t d_ff, int32_t E,
                     int32_t k, const moe_opts_t* opts);

/* Bytes of workspace moe_ffn_backward needs (0 if the shape is invalid or
 * unsupported; T = 0 is sized as T = 1). */
size_t moe_ffn_backward_workspace_size(int64_t T, int64_t d_model, int64_t d_ff, int32_t E,
                                       int32_t k);

/* Bytes of workspace moe_ffn_forward (dtype MOE_BF16 or MOE_F32) or
 * moe_ffn_forward_int4 (MOE_W4A16) needs for this shape (0 if the shape is
 * invalid or unsupported; T = 0 is sized as T = 1). */
size_t moe_ffn_workspace_size(int64_t T, int64_t d_model, int64_t d_ff, int32_t E,
                              int32_t k, int32_t dtype);

/* Bytes of workspace moe_block_forward needs (dtype MOE_BF16 or MOE_F32; 0 if
 * the shape or dtype is invalid or unsupported; T = 0 is sized as T = 1). */
size_t moe_block_workspace_size(int64_t T, int64_t d_model, int64_t d_ff, int32_t E,
                                int32_t k, int32_t dtype);

/*
 * Where the forward pass keeps its intermediates inside a caller workspace,
 * for inspection after the call (byte offsets from the workspace start; all
 * int32 unless noted).  Row r of the permuted layout belongs to expert e when
 * offsets[e] <= r < offsets[e+1]; each expert's segment is padded to a
 * multiple of `block_rows`; rows at or beyond offsets[e] + counts[e] are
 * padding (row_token = -1, H rows zero).
 */
typedef struct moe_ws_layout {
  int64_t block_rows;       /* padding unit of expert segments (token tile)   */
  int64_t max_rows;         /* rows reserved for the permuted layout          */
  int64_t router_blocks;    /* token blocks of the router / scatter kernels   */
  int64_t y_part_rows;      /* rows of each extra down-GEMM part plane (y_parts) */
  int32_t gemm_variant;     /* 0 = weight-streaming, 1 = LDS-tiled             */
  int32_t down_splits;      /* K parts into which the down GEMM may split the
                               token tiles of a partial last round of work-
                               groups (1: never); see down_sched               */
  int32_t tokens_in_place;  /* 1: the gate/up GEMM reads each row's token from
                               x (or xn) through row_token and xs is not
                               written; 0: it reads the gathered rows of xs    */
  int32_t y_weighted;       /* 1 (LDS-tiled form): y holds bf16 rows that
                               already carry their gate weight (row_w), and
                               y_parts float32 rows likewise; 0: y holds
                               float32 W2 H and the combine applies the gates */
  size_t topk_idx;          /* [T][k]                                          */
  size_t topk_w;            /* [T][k] float32                                  */
  size_t block_counts;      /* [router_blocks][E]: per-block counts, then bases */
  size_t counts;            /* [E]                                             */
  size_t offsets;           /* [E+1] padded segment starts; offsets[E] = rows  */
  size_t num_tiles;         /* [1] token tiles in use                          */
  size_t tile_expert;       /* [max_rows / block_rows] expert of each tile     */
  size_t row_token;         /* [max_rows] token of each permuted row or -1     */
  size_t tok_row;           /* [T][k] permuted row of each (token, slot)       */
  size_t row_w;             /* [max_rows] float32, y_weighted only (else 0
                               bytes): the gate weight of each permuted row
                               (padding rows: not written; their y rows are
                               zeros)                                          */
  size_t xs;                /* [max_rows][d_model] dtype: gathered tokens.
                               0 bytes (not used) when tokens_in_place is 1:
                               bf16 tokens with T * d_model * 2 < 2^31, and
                               either the weight-streaming form (bf16 weights
                               with d_model a multiple of 128, or INT4
                               weights) or the LDS-tiled form with k >= 4      */
  size_t h;                 /* [max_rows][d_ff] dtype: SiLU(gate) * up         */
  size_t y;                 /* [max_rows][d_model]: expert outputs W2 H of
                               each row, float32; with y_weighted, bf16 and
                               times the row's gate weight (row_w).  For the
                               rows of a split token tile, the first of its K
                               parts                                           */
  size_t y_parts;           /* [down_splits - 1][y_part_rows][d_model] float32:
                               the other K parts of the split token tiles' rows
                               (times row_w when y_weighted), row r at
                               r - down_sched[1]; the row's output is their sum
                               with y, added in part order                     */
  size_t down_sched;        /* [2] int32, LDS-tiled form only (else 0 bytes):
                               written by the expert scan from the token tiles
                               in use: K parts s in use (1: none split) and the
                               first row of the split token tiles (the last
                               ones)                                           */
  size_t block_probs;       /* [router_blocks][E] float32: per-block sums of the
                               full-softmax probabilities (router statistics)  */
  size_t norm_rs;           /* [T] float32: 1/rms of each token; block wrapper
                               only (0 bytes in the layer's layout)            */
  size_t xn;                /* [T][d_model] dtype: RMS-normalised tokens; block
                               wrapper only (0 bytes in the layer's layout)    */
  size_t router_partial;    /* router scratch: partial scores when the score GEMM
                               is split over d_model (few token blocks)        */
  size_t wdeq;              /* MOE_W4A16 with the LDS-tiled form only: the three
                               weight stacks dequantized to bf16, W_gate, W_up,
                               W_down in their bf16 layouts (else 0 bytes)     */
  size_t total;             /* bytes                                           */
} moe_ws_layout_t;

int moe_ffn_workspace_layout(int64_t T, int64_t d_model, int64_t d_ff, int32_t E,
                             int32_t k, int32_t dtype, moe_ws_layout_t* layout);
/* The same for moe_block_forward (dtype MOE_BF16 or MOE_F32). */
int moe_block_workspace_layout(int64_t T, int64_t d_model, int64_t d_ff, int32_t E,
                               int32_t k, int32_t dtype, moe_ws_layout_t* layout);

/* Static, human-readable text for a status code. */
const char* moe_status_string(int status);

/* Thread-local text of the last failure on this thread ("" if none). */
const char* moe_last_error(void);

/* Free the library-owned workspaces (all devices).  The caller must make sure
 * no enqueued forward call still uses them (synchronise first). */
void moe_release(void);

/* Library version as "major.minor.patch" (static string). */
const char* moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
