// C ABI of the sparse MoE feed-forward layer: argument validation, the
// launch plan, the workspace layout and the launch sequence
//   router -> scan -> scatter/gather -> gate/up GEMM -> down GEMM -> combine,
// all asynchronous on the caller's stream with no host synchronisation.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>

#include "common.h"
#include "launch.h"
#include "moe_ffn.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const std::string& why) {
  g_last_error = why;
  return status;
}

using moe::BwdPlan;
using moe::Plan;

// make_plan / make_bwd_plan of plan.h, with the reason of a failure kept as
// this thread's last error
int plan_forward(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, int32_t dtype,
                 bool block, Plan* p) {
  std::string why;
  const int st = moe::make_plan(T, d, f, E, k, dtype, block, p, &why);
  return st == MOE_OK ? st : fail(st, why);
}

int plan_backward(int64_t T, int64_t d, int64_t f, int32_t E, int32_t k, BwdPlan* b) {
  std::string why;
  const int st = moe::make_bwd_plan(T, d, f, E, k, b, &why);
  return st == MOE_OK ? st : fail(st, why);
}

struct CachedWs {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::map<int, CachedWs> g_ws;

int hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// The library-owned workspace of the current device, grown to `bytes`.
int library_workspace(size_t bytes, char** ws) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  CachedWs& c = g_ws[dev];
  if (c.bytes < bytes) {
    if (c.ptr) {
      e = hipDeviceSynchronize();  // the old buffer may still be in use
      if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
      (void)hipFree(c.ptr);
      c.ptr = nullptr;
      c.bytes = 0;
    }
    e = hipMalloc(&c.ptr, bytes);
    if (e != hipSuccess) return hip_fail(e, "hipMalloc(workspace)");
    c.bytes = bytes;
  }
  *ws = static_cast<char*>(c.ptr);
  return MOE_OK;
}

}  // namespace

// Scratch memory of moe_ffn_forward_noalloc: a file-scope device array, so
// that entry point allocates nothing.  Each GPU the library runs on holds its
// own copy until the process ends.  In host code the array's name is only a
// stand-in for the symbol, never a device address: the address comes from
// hipGetSymbolAddress, once per device, and only that address is handed to
// kernels.
static __device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mutex;
std::map<int, char*> g_scratch;   // device -> device address of its scratch

// The current device's scratch address, looked up on the first call on that
// device (with it current) and kept.
int scratch_address(char** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    it = g_scratch.emplace(dev, static_cast<char*>(p)).first;
  }
  *ptr = it->second;
  return MOE_OK;
}

}  // namespace

extern "C" {

void moe_opts_init(moe_opts_t* o) {
  if (!o) return;
  std::memset(o, 0, sizeof(*o));
  o->dtype = MOE_BF16;
}

size_t moe_ffn_workspace_size(int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                              int32_t dtype) {
  Plan p;
  if (plan_forward(T == 0 ? 1 : T, d_model, d_ff, E, k, dtype, false, &p) != MOE_OK) return 0;
  return p.L.total;
}

int moe_ffn_workspace_layout(int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                             int32_t dtype, moe_ws_layout_t* layout) {
  g_last_error.clear();
  if (!layout) return fail(MOE_ERR_INVALID_ARG, "layout is NULL");
  Plan p;
  const int st = plan_forward(T == 0 ? 1 : T, d_model, d_ff, E, k, dtype, false, &p);
  if (st != MOE_OK) return st;
  *layout = p.L;
  return MOE_OK;
}

size_t moe_block_workspace_size(int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                                int32_t dtype) {
  Plan p;
  if (dtype == MOE_W4A16 ||
      plan_forward(T == 0 ? 1 : T, d_model, d_ff, E, k, dtype, true, &p) != MOE_OK)
    return 0;
  return p.L.total;
}

int moe_block_workspace_layout(int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                               int32_t dtype, moe_ws_layout_t* layout) {
  g_last_error.clear();
  if (!layout) return fail(MOE_ERR_INVALID_ARG, "layout is NULL");
  if (dtype == MOE_W4A16)
    return fail(MOE_ERR_INVALID_ARG, "the block wrapper takes bf16 or float32 weights");
  Plan p;
  const int st = plan_forward(T == 0 ? 1 : T, d_model, d_ff, E, k, dtype, true, &p);
  if (st != MOE_OK) return st;
  *layout = p.L;
  return MOE_OK;
}

}  // extern "C"

namespace {

// The whole launch sequence.  norm_w != NULL selects the block wrapper:
// out = x + layer(RMSNorm(x)).
// noalloc: the intermediates go to the device scratch array instead of a
// caller or library workspace (moe_ffn_forward_noalloc).
int run_layer(const void* x, const float* W_router, const void* W_gate, const void* W_up,
              const void* W_down, void* out, int64_t T, int64_t d_model, int64_t d_ff, int32_t E,
              int32_t k, const float* norm_w, float eps, const moe_opts_t* opts,
              const moe::Q4Weights* q4 = nullptr, int group = 0, bool noalloc = false) {
  moe_opts_t o;
  if (opts) o = *opts;
  else moe_opts_init(&o);
  if (q4) o.dtype = MOE_W4A16;
  Plan p;
  // an empty batch checks the other sizes as for one token, reads no tensor
  // and only clears the optional statistics
  int st = plan_forward(T == 0 ? 1 : T, d_model, d_ff, E, k, o.dtype, norm_w != nullptr, &p);
  if (st != MOE_OK) return st;
  if (noalloc) {
    if (o.workspace)
      return fail(MOE_ERR_INVALID_ARG,
                  "moe_ffn_forward_noalloc takes no workspace (opts->workspace must be NULL)");
    if (p.L.total > MOE_NOALLOC_SCRATCH_BYTES)
      return fail(MOE_ERR_WORKSPACE,
                  "this shape needs " + std::to_string(p.L.total) +
                      " bytes of workspace; moe_ffn_forward_noalloc's scratch holds " +
                      std::to_string((size_t)MOE_NOALLOC_SCRATCH_BYTES));
  }
  p.D.group = group;
  if (T == 0) {
    for (const void* ptr : {(const void*)o.expert_counts_out, (const void*)o.router_prob_out,
                            (const void*)o.balance_loss_out})
      if (reinterpret_cast<uintptr_t>(ptr) % 4)
        return fail(MOE_ERR_INVALID_ARG, "optional outputs must be 4-byte aligned");
    if (!o.expert_counts_out && !o.router_prob_out && !o.balance_loss_out) return MOE_OK;
    moe::launch_empty_stats(E, o.expert_counts_out, o.router_prob_out, o.balance_loss_out,
                            reinterpret_cast<hipStream_t>(o.stream));
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : hip_fail(e, "empty-batch launch");
  }
  if (!x || !W_router || !W_gate || !W_up || !W_down || !out)
    return fail(MOE_ERR_INVALID_ARG, "null tensor pointer");
  // rows are moved with 16-byte vector loads and stores
  for (const void* ptr : {x, (const void*)W_router, W_gate, W_up, W_down, (const void*)out})
    if (reinterpret_cast<uintptr_t>(ptr) % 16)
      return fail(MOE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  for (const void* ptr : {(const void*)o.router_bias, (const void*)o.topk_idx_out,
                          (const void*)o.topk_w_out, (const void*)o.expert_counts_out,
                          (const void*)o.router_prob_out, (const void*)o.balance_loss_out,
                          (const void*)norm_w})
    if (reinterpret_cast<uintptr_t>(ptr) % 4)
      return fail(MOE_ERR_INVALID_ARG, "optional outputs, bias and norm weight must be 4-byte aligned");
  if (o.workspace) {
    if (reinterpret_cast<uintptr_t>(o.workspace) % 256)
      return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (o.workspace_bytes < p.L.total)
      return fail(MOE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(p.L.total) +
                                         " bytes");
  }

  // ---- validated; from here on HIP calls
  hipStream_t s = reinterpret_cast<hipStream_t>(o.stream);
  char* ws = static_cast<char*>(o.workspace);
  if (noalloc) {
    if ((st = scratch_address(&ws)) != MOE_OK) return st;
  } else if (!ws && (st = library_workspace(p.L.total, &ws)) != MOE_OK) {
    return st;
  }
  const moe::Dims& D = p.D;
  const moe_ws_layout_t& L = p.L;
  int32_t* idx = o.topk_idx_out ? o.topk_idx_out : reinterpret_cast<int32_t*>(ws + L.topk_idx);
  float* w = o.topk_w_out ? o.topk_w_out : reinterpret_cast<float*>(ws + L.topk_w);
  int32_t* blk = reinterpret_cast<int32_t*>(ws + L.block_counts);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* num_tiles = reinterpret_cast<int32_t*>(ws + L.num_tiles);
  int32_t* tile_expert = reinterpret_cast<int32_t*>(ws + L.tile_expert);
  int32_t* row_token = reinterpret_cast<int32_t*>(ws + L.row_token);
  int32_t* tok_row = reinterpret_cast<int32_t*>(ws + L.tok_row);
  void* xs = ws + L.xs;
  void* h = ws + L.h;
  void* y = ws + L.y;
  float* y_parts = reinterpret_cast<float*>(ws + L.y_parts);
  float* row_w = L.y_weighted ? reinterpret_cast<float*>(ws + L.row_w) : nullptr;
  int32_t* down_sched = L.gemm_variant == 1 ? reinterpret_cast<int32_t*>(ws + L.down_sched)
                                            : nullptr;
  float* rpart = reinterpret_cast<float*>(ws + L.router_partial);
  float* bprob = (o.router_prob_out || o.balance_loss_out)
                     ? reinterpret_cast<float*>(ws + L.block_probs) : nullptr;
  float* rs = norm_w ? reinterpret_cast<float*>(ws + L.norm_rs) : nullptr;
  void* xn = ws + L.xn;

  hipError_t e;
  auto mark = [&](int i) -> hipError_t {
    return o.stage_events ? hipEventRecord(static_cast<hipEvent_t>(o.stage_events[i]), s)
                          : hipSuccess;
  };
  if ((e = mark(0)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  if (norm_w) {
    moe::launch_rmsnorm(D, x, norm_w, eps, rs, xn, s);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "rmsnorm launch");
  }
  // the gate/up GEMM reads token rows in place through row_token, so the
  // scatter then only writes the row maps, or (one router block) the
  // router's select pass does and there is no scatter launch
  const void* tok = norm_w ? xn : x;
  const bool gather = L.tokens_in_place != 0;
  const bool maps_in_router = gather && moe::router_fuses_scan(D);
  // one router block means at most 32 rows per expert: never the tiled form,
  // whose row weights the scatter writes
  if (maps_in_router && row_w) return fail(MOE_ERR_UNSUPPORTED, "row weights need the scatter");
  const moe::ScanArgs sa{counts,
                         offsets,
                         num_tiles,
                         tile_expert,
                         row_token,
                         o.expert_counts_out,
                         o.router_prob_out,
                         o.balance_loss_out,
                         maps_in_router ? tok_row : nullptr,
                         down_sched,
                         (int)(d_model / moe::kTileRows),
                         D.down_splits};
  moe::launch_router(D, x, W_router, o.router_bias, idx, w, blk, rpart, bprob, norm_w, rs,
                     nullptr, sa, s);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(1)) != hipSuccess)
    return hip_fail(e, "router launch");
  moe::launch_scan(D, blk, sa, bprob, s);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(2)) != hipSuccess)
    return hip_fail(e, "scan launch");
  if (!maps_in_router)
    moe::launch_scatter(D, tok, idx, w, blk, offsets, tok_row, row_token, row_w,
                        gather ? nullptr : xs, s);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(3)) != hipSuccess)
    return hip_fail(e, "scatter launch");
  if (q4 && L.gemm_variant == 1) {
    // many rows per expert: bf16 copies of the INT4 stacks for the tiled form
    char* wd = ws + L.wdeq;
    const size_t mat = sizeof(uint16_t) * (size_t)E * d_model * d_ff;
    moe::launch_dequant_int4(q4[0].q, q4[0].s, (int64_t)E * d_ff, (int)d_ff, (int)d_model,
                             group, wd, s);
    moe::launch_dequant_int4(q4[1].q, q4[1].s, (int64_t)E * d_ff, (int)d_ff, (int)d_model,
                             group, wd + mat, s);
    moe::launch_dequant_int4(q4[2].q, q4[2].s, (int64_t)E * d_model, (int)d_model, (int)d_ff,
                             group, wd + 2 * mat, s);
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "dequantize launch");
    W_gate = wd;
    W_up = wd + mat;
    W_down = wd + 2 * mat;
  }
  if (q4 && L.gemm_variant == 0)
    moe::launch_gateup_q4(D, gather ? tok : xs, gather ? row_token : nullptr, q4[0], q4[1], h,
                          counts, offsets, num_tiles, tile_expert, s);
  else if (L.gemm_variant == 1)
    moe::launch_gateup_tile(D, gather ? tok : xs, gather ? row_token : nullptr, W_gate, W_up,
                            h, counts, offsets, num_tiles, tile_expert, s);
  else
    moe::launch_gateup_stream(D, gather ? tok : xs, gather ? row_token : nullptr, W_gate, W_up,
                              h, counts, offsets, num_tiles, tile_expert, s);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(4)) != hipSuccess)
    return hip_fail(e, "gate/up launch");
  if (q4 && L.gemm_variant == 0)
    moe::launch_down_q4(D, h, q4[2], static_cast<float*>(y), counts, offsets, num_tiles,
                        tile_expert, s);
  else if (L.gemm_variant == 1)
    moe::launch_down_tile(D, h, W_down, y, y_parts, L.y_part_rows, down_sched, row_w, counts,
                          offsets, num_tiles, tile_expert, s);
  else
    moe::launch_down_stream(D, h, W_down, static_cast<float*>(y), counts, offsets, num_tiles,
                            tile_expert, s);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(5)) != hipSuccess)
    return hip_fail(e, "down launch");
  moe::launch_combine(D, y, L.y_weighted != 0, y_parts, L.y_part_rows, down_sched, tok_row, w,
                      norm_w ? x : nullptr, out, s);
  if ((e = hipGetLastError()) != hipSuccess || (e = mark(6)) != hipSuccess)
    return hip_fail(e, "combine launch");
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_ffn_forward(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                    const void* W_down, void* out, int64_t T, int64_t d_model, int64_t d_ff,
                    int32_t E, int32_t k, const moe_opts_t* opts) {
  g_last_error.clear();
  if (opts && opts->dtype == MOE_W4A16)
    return fail(MOE_ERR_INVALID_ARG, "MOE_W4A16 weights go through moe_ffn_forward_int4");
  return run_layer(x, W_router, W_gate, W_up, W_down, out, T, d_model, d_ff, E, k, nullptr, 0.f,
                   opts);
}

int moe_ffn_forward_noalloc(const void* x, const float* W_router, const void* W_gate,
                            const void* W_up, const void* W_down, void* out, int64_t T,
                            int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                            const moe_opts_t* opts) {
  g_last_error.clear();
  if (opts && opts->dtype == MOE_W4A16)
    return fail(MOE_ERR_INVALID_ARG, "MOE_W4A16 weights go through moe_ffn_forward_int4");
  return run_layer(x, W_router, W_gate, W_up, W_down, out, T, d_model, d_ff, E, k, nullptr, 0.f,
                   opts, nullptr, 0, true);
}

int moe_block_forward(const void* x, const float* norm_weight, float eps, const float* W_router,
                      const void* W_gate, const void* W_up, const void* W_down, void* out,
                      int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                      const moe_opts_t* opts) {
  g_last_error.clear();
  if (!norm_weight) return fail(MOE_ERR_INVALID_ARG, "norm_weight is NULL");
  if (!(eps >= 0.f) || eps > 1.f) return fail(MOE_ERR_INVALID_ARG, "eps must be in [0, 1]");
  if (T > 0 && x == out) return fail(MOE_ERR_INVALID_ARG, "out must not alias x");
  if (opts && opts->dtype == MOE_W4A16)
    return fail(MOE_ERR_INVALID_ARG, "the block wrapper takes bf16 or float32 weights");
  return run_layer(x, W_router, W_gate, W_up, W_down, out, T, d_model, d_ff, E, k, norm_weight,
                   eps, opts);
}

int moe_quantize_int4(const void* W, int32_t dtype, int64_t batch, int64_t N, int64_t K,
                      int32_t group, uint8_t* packed, float* scales, void* stream) {
  g_last_error.clear();
  if (!W || !packed || !scales) return fail(MOE_ERR_INVALID_ARG, "null pointer");
  if (dtype != MOE_BF16 && dtype != MOE_F32)
    return fail(MOE_ERR_INVALID_ARG, "dtype must be MOE_BF16 or MOE_F32");
  if (batch < 1 || N < 1 || K < 1 || group < 1)
    return fail(MOE_ERR_INVALID_ARG, "batch, N, K and group must be >= 1");
  if (N > 0x7fffffff || batch > 0x7fffffff / N)
    return fail(MOE_ERR_UNSUPPORTED, "batch * N > 2^31 - 1");
  if (K > moe::q4_quantize_max_k()) return fail(MOE_ERR_UNSUPPORTED, "K > 65536");
  if (!moe::q4_group_ok((int)K, group))
    return fail(MOE_ERR_UNSUPPORTED,
                "K must be a multiple of 128 and group a multiple of 32 that divides K and is "
                "32, 64 or a multiple of 128");
  if (reinterpret_cast<uintptr_t>(W) % 16 || reinterpret_cast<uintptr_t>(packed) % 4 ||
      reinterpret_cast<uintptr_t>(scales) % 4)
    return fail(MOE_ERR_INVALID_ARG, "W must be 16-byte aligned, packed and scales 4-byte");
  moe::launch_quantize_int4(W, dtype == MOE_BF16, batch * N, (int)N, (int)K, group, packed,
                            scales, reinterpret_cast<hipStream_t>(stream));
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : hip_fail(e, "quantize launch");
}

int moe_ffn_forward_int4(const void* x, const float* W_router, const uint8_t* Wg_q,
                         const float* Wg_s, const uint8_t* Wu_q, const float* Wu_s,
                         const uint8_t* Wd_q, const float* Wd_s, int32_t group, void* out,
                         int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                         const moe_opts_t* opts) {
  g_last_error.clear();
  if (d_model % 128 || d_ff % 128 || d_model < 128 || d_ff < 128)
    return fail(MOE_ERR_UNSUPPORTED, "INT4 weights need d_model and d_ff multiples of 128");
  if (!moe::q4_group_ok((int)d_model, group) || !moe::q4_group_ok((int)d_ff, group))
    return fail(MOE_ERR_UNSUPPORTED,
                "group must be a multiple of 32 dividing d_model and d_ff, and 32, 64 or a "
                "multiple of 128");
  if (T > 0) {
    if (!Wg_q || !Wg_s || !Wu_q || !Wu_s || !Wd_q || !Wd_s)
      return fail(MOE_ERR_INVALID_ARG, "null weight pointer");
    for (const void* ptr : {(const void*)Wg_q, (const void*)Wu_q, (const void*)Wd_q})
      if (reinterpret_cast<uintptr_t>(ptr) % 16)
        return fail(MOE_ERR_INVALID_ARG, "INT4 codes must be 16-byte aligned");
    for (const void* ptr : {(const void*)Wg_s, (const void*)Wu_s, (const void*)Wd_s})
      if (reinterpret_cast<uintptr_t>(ptr) % 4)
        return fail(MOE_ERR_INVALID_ARG, "scales must be 4-byte aligned");
  }
  const moe::Q4Weights q4[3] = {{Wg_q, Wg_s}, {Wu_q, Wu_s}, {Wd_q, Wd_s}};
  // the weight arguments of the plain path stand in for the non-null checks
  return run_layer(x, W_router, Wg_q, Wu_q, Wd_q, out, T, d_model, d_ff, E, k, nullptr, 0.f,
                   opts, q4, group);
}

}  // extern "C"

extern "C" {

size_t moe_ffn_backward_workspace_size(int64_t T, int64_t d_model, int64_t d_ff, int32_t E,
                                       int32_t k) {
  g_last_error.clear();
  BwdPlan b;
  if (plan_backward(T == 0 ? 1 : T, d_model, d_ff, E, k, &b) != MOE_OK) return 0;
  return b.total;
}

int moe_ffn_backward(const void* x, const float* W_router, const void* W_gate, const void* W_up,
                     const void* W_down, const void* dout, float alpha, void* dx,
                     float* dW_router, float* dbias, void* dW_gate, void* dW_up, void* dW_down,
                     int64_t T, int64_t d_model, int64_t d_ff, int32_t E, int32_t k,
                     const moe_opts_t* opts) {
  g_last_error.clear();
  moe_opts_t o;
  if (opts) o = *opts;
  else moe_opts_init(&o);
  if (o.dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "the backward takes bf16 tensors");
  if (!(alpha >= 0.f) || alpha > 1e30f) return fail(MOE_ERR_INVALID_ARG, "alpha must be >= 0");
  BwdPlan b;
  int st = plan_backward(T == 0 ? 1 : T, d_model, d_ff, E, k, &b);
  if (st != MOE_OK) return st;
  if (!dW_router || !dW_gate || !dW_up || !dW_down)
    return fail(MOE_ERR_INVALID_ARG, "null gradient pointer");
  for (const void* ptr : {(const void*)dW_router, (const void*)dbias, (const void*)o.router_bias})
    if (reinterpret_cast<uintptr_t>(ptr) % 4)
      return fail(MOE_ERR_INVALID_ARG, "dW_router, dbias and the bias must be 4-byte aligned");
  for (const void* ptr : {dW_gate, dW_up, dW_down})
    if (reinterpret_cast<uintptr_t>(ptr) % 16)
      return fail(MOE_ERR_INVALID_ARG, "weight gradients must be 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(o.stream);
  const size_t wbytes = sizeof(uint16_t) * (size_t)E * d_model * d_ff;
  hipError_t e;
  if (T == 0) {
    // an empty batch: every gradient is zero
    moe::launch_zero_fill(dW_router, sizeof(float) * (size_t)d_model * E, s);
    moe::launch_zero_fill(dbias, sizeof(float) * (size_t)E, s);
    moe::launch_zero_fill(dW_gate, wbytes, s);
    moe::launch_zero_fill(dW_up, wbytes, s);
    moe::launch_zero_fill(dW_down, wbytes, s);
    e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : hip_fail(e, "zero-fill launch");
  }
  if (!x || !W_router || !W_gate || !W_up || !W_down || !dout || !dx)
    return fail(MOE_ERR_INVALID_ARG, "null tensor pointer");
  for (const void* ptr : {x, (const void*)W_router, W_gate, W_up, W_down, dout, (const void*)dx})
    if (reinterpret_cast<uintptr_t>(ptr) % 16)
      return fail(MOE_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (o.workspace) {
    if (reinterpret_cast<uintptr_t>(o.workspace) % 256)
      return fail(MOE_ERR_WORKSPACE, "workspace must be 256-byte aligned");
    if (o.workspace_bytes < b.total)
      return fail(MOE_ERR_WORKSPACE, "workspace too small: need " + std::to_string(b.total) +
                                         " bytes");
  }
  char* ws = static_cast<char*>(o.workspace);
  if (!ws && (st = library_workspace(b.total, &ws)) != MOE_OK) return st;

  const moe::Dims& D = b.D;
  const int d = (int)d_model, f = (int)d_ff;
  auto I = [&](size_t off) { return reinterpret_cast<int32_t*>(ws + off); };
  auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  int32_t* idx = I(b.topk_idx);
  float* w = F(b.topk_w);
  int32_t* counts = I(b.counts);
  int32_t* offsets = I(b.offsets);
  int32_t* row_token = I(b.row_token);
  int32_t* tok_row = I(b.tok_row);
  int32_t* tb = I(b.tb);
  int32_t *tb_count = tb, *tb_exp = tb + 1, *tb_row0 = tb + 1 + b.max_tiles,
          *tb_rows = tb + 1 + 2 * b.max_tiles, *dx_sched = tb + 1 + 3 * b.max_tiles;
  char* xs = ws + b.xs;
  char* dp = ws + b.dp;
  char* dab = ws + b.dab;
  char* hg = ws + b.hg;
  moe::bf16_t* ab = reinterpret_cast<moe::bf16_t*>(ws + b.ab);
  moe::bf16_t* z = reinterpret_cast<moe::bf16_t*>(ws + b.z);
  float* dxs = F(b.dxs);
  const size_t dx_plane = (size_t)D.max_rows * d;   // dxs: [2][max_rows][d]
  float* dxs_extra = F(b.dxs_extra);                 // [dx_parts][dx_split_rows][d]
  const size_t dx_extra_plane = (size_t)b.dx_split_rows * d;
  float* dg = F(b.dg);
  float* ds = F(b.ds);
  const size_t wstride = (size_t)d * f;   // elements per expert matrix

  auto mark = [&](int i) -> hipError_t {
    return o.stage_events ? hipEventRecord(static_cast<hipEvent_t>(o.stage_events[i]), s)
                          : hipSuccess;
  };
  auto check = [&](int stage, const char* what) -> int {
    if ((e = hipGetLastError()) != hipSuccess || (e = mark(stage)) != hipSuccess)
      return hip_fail(e, what);
    return MOE_OK;
  };
  if ((e = mark(0)) != hipSuccess) return hip_fail(e, "hipEventRecord");
  // routing and permutation of the forward pass, the permuted upstream
  // gradient and the 128-row tile table
  const moe::ScanArgs sa{counts,  offsets, I(b.num_tiles), I(b.tile_expert), row_token,
                         nullptr, nullptr, nullptr,          nullptr,          nullptr,
                         0,       1};
  moe::launch_router(D, x, W_router, o.router_bias, idx, w, I(b.block_counts),
                     F(b.router_partial), nullptr, nullptr, nullptr, F(b.logits), sa, s);
  moe::launch_scan(D, I(b.block_counts), sa, nullptr, s);
  moe::launch_scatter(D, x, idx, nullptr, I(b.block_counts), offsets, tok_row, row_token, nullptr,
                      xs, s);
  moe::launch_bwd_gather(D, dout, row_token, dp, s);
  moe::launch_bwd_tile_table(D, counts, offsets, b.max_tiles, b.dx_max_split, b.dx_parts,
                             tb_count, tb_exp, tb_row0, tb_rows, dx_sched, s);
  if ((st = check(1, "routing launch")) != MOE_OK) return st;
  // the 256 x 256 ping-pong GEMMs when both widths allow, else the generic one
  const bool tiled = moe::bwd_tile_shape_ok(d, f);
  // pre-activations a = W1 x, b = W3 x of every routed row
  if (tiled) {
    moe::launch_bwd_recompute(D, xs, W_gate, W_up, ab, b.max_tiles, tb_count, tb_exp, tb_row0,
                              tb_rows, s);
  } else {
    moe::launch_bwd_gemm_rows(xs, d, W_gate, d, true, wstride, ab, true, 2 * f, D.max_rows, f,
                              d, false, b.max_tiles, tb_count, tb_exp, tb_row0, tb_rows, s);
    moe::launch_bwd_gemm_rows(xs, d, W_up, d, true, wstride, ab + f, true, 2 * f, D.max_rows, f,
                              d, false, b.max_tiles, tb_count, tb_exp, tb_row0, tb_rows, s);
  }
  if ((st = check(2, "recompute launch")) != MOE_OK) return st;
  // Z = W2^T dOut_t per routed row
  if (tiled)
    moe::launch_bwd_z(D, dp, W_down, z, b.max_tiles, tb_count, tb_exp, tb_row0, tb_rows, s);
  else
    moe::launch_bwd_gemm_rows(dp, d, W_down, f, false, wstride, z, true, f, D.max_rows, f, d,
                              false, b.max_tiles, tb_count, tb_exp, tb_row0, tb_rows, s);
  if ((st = check(3, "Z launch")) != MOE_OK) return st;
  // dg, dA, dB, g h; the router scores' gradient; the router weight gradient
  moe::launch_bwd_rows(D, ab, z, row_token, tok_row, w, dg, dab, hg, s);
  moe::launch_bwd_router(D, F(b.logits), idx, w, tok_row, dg, counts, alpha, ds, s);
  moe::launch_bwd_router_wgrad(D, x, ds, F(b.wpart), dW_router, dbias, s);
  if ((st = check(4, "row/router backward launch")) != MOE_OK) return st;
  // dX_r = W1^T dA + W3^T dB
  if (tiled) {
    moe::launch_bwd_dxs(D, b.dx_parts, dab, W_gate, W_up, dxs, dx_plane, dxs_extra,
                        dx_extra_plane, dx_sched, b.max_tiles, tb_count, tb_exp, tb_row0,
                        tb_rows, s);
  } else {
    moe::launch_bwd_gemm_rows(dab, 2 * f, W_gate, d, false, wstride, dxs, false, d, D.max_rows,
                              d, f, false, b.max_tiles, tb_count, tb_exp, tb_row0, tb_rows, s);
    moe::launch_bwd_gemm_rows(dab + 2 * (size_t)f, 2 * f, W_up, d, false, wstride,
                              dxs + dx_plane, false, d, D.max_rows, d, f, false, b.max_tiles,
                              tb_count, tb_exp, tb_row0, tb_rows, s);
  }
  if ((st = check(5, "dX launch")) != MOE_OK) return st;
  moe::launch_bwd_dx(D, tiled ? b.dx_parts : 2, dxs, dx_plane, dxs_extra, dx_extra_plane,
                     tiled ? dx_sched : nullptr, tok_row, W_router, ds, dx, s);
  if ((st = check(6, "dx launch")) != MOE_OK) return st;
  // weight gradients over each expert's rows
  if (tiled)
    moe::launch_bwd_wgrad_down(D, dp, hg, dW_down, counts, offsets, s);
  else
    moe::launch_bwd_gemm_wgrad(D, dp, d, hg, f, dW_down, d, f, counts, offsets, s);
  if ((st = check(7, "dW_down launch")) != MOE_OK) return st;
  if (tiled) {
    moe::launch_bwd_wgrad_gate_up(D, dab, xs, dW_gate, dW_up, counts, offsets, s);
  } else {
    moe::launch_bwd_gemm_wgrad(D, dab, 2 * f, xs, d, dW_gate, f, d, counts, offsets, s);
    moe::launch_bwd_gemm_wgrad(D, dab + 2 * (size_t)f, 2 * f, xs, d, dW_up, f, d, counts,
                               offsets, s);
  }
  return check(8, "dW_gate/dW_up launch");
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_WORKSPACE: return "workspace too small or misaligned";
    case MOE_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

void moe_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int cur = 0;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_ws) {
    if (kv.second.ptr) {
      if (hipSetDevice(kv.first) == hipSuccess) (void)hipFree(kv.second.ptr);
    }
    kv.second = CachedWs();
  }
  g_ws.clear();
  if (have_cur) (void)hipSetDevice(cur);
}

const char* moe_version(void) { return "0.1.0"; }

}  // extern "C"
