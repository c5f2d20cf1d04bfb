// Host-only driver of the launch plan (csrc/plan.cpp), built by the CPU tests
// with the address and undefined-behaviour sanitizers.  For every shape read
// from stdin ("T d_model d_ff E k dtype block", one per line) it prints one
// line: the status, then every field of the forward layout and the backward
// workspace size, so the test can compare them with the library's own
// answers through the C ABI.
#include <cstdio>
#include <string>

#include "plan.h"

int main() {
  long long T, d, f;
  int E, k, dtype, block;
  while (std::scanf("%lld %lld %lld %d %d %d %d", &T, &d, &f, &E, &k, &dtype, &block) == 7) {
    moe::Plan p{};
    std::string why;
    const int st = moe::make_plan(T == 0 ? 1 : T, d, f, E, k, dtype, block != 0, &p, &why);
    if (st != MOE_OK) {
      std::printf("%d\n", st);
      continue;
    }
    const moe_ws_layout_t& L = p.L;
    moe::BwdPlan b{};
    std::string why_b;
    const size_t bwd = moe::make_bwd_plan(T == 0 ? 1 : T, d, f, E, k, &b, &why_b) == MOE_OK
                           ? b.total : 0;
    std::printf("0 %lld %lld %lld %lld %d %d %d %d", (long long)L.block_rows,
                (long long)L.max_rows, (long long)L.router_blocks, (long long)L.y_part_rows,
                L.gemm_variant, L.down_splits, L.tokens_in_place, L.y_weighted);
    const size_t fields[] = {L.topk_idx,    L.topk_w,    L.block_counts, L.counts,
                             L.offsets,     L.num_tiles, L.tile_expert,  L.row_token,
                             L.tok_row,     L.row_w,     L.xs,           L.h,
                             L.y,
                             L.y_parts,     L.down_sched, L.block_probs, L.norm_rs,
                             L.xn,          L.router_partial, L.wdeq,    L.total};
    for (size_t v : fields) std::printf(" %zu", v);
    std::printf(" %zu\n", bwd);
  }
  return 0;
}
