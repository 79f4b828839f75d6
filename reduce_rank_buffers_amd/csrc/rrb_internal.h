// Internal declarations shared by the host-side plan builder, the C ABI and
// the HIP launchers of librrb.  Not installed; the public ABI is include/rrb.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "../../include/rrb.h"

namespace rrb {

// Records a failure message for rrb_last_error() and returns `s`.
rrb_status fail(rrb_status s, const char *fmt, ...);
// Clears the thread's last-error text.
void clear_error();

inline int elem_size(int32_t dtype) { return dtype == RRB_F32 ? 4 : 2; }

// An index-map entry at element granularity (the same fields rrb_segment
// exposes).  src_rank == -1 means "every rank 0..R-1, folded in rank order".
struct Segment {
  int64_t src_off;
  int64_t dst_off;
  int64_t len;
  int32_t src_rank;
  uint32_t dst_mask;
};

enum class PlanKind { Uniform, Rows, RowsDevice };

// Row maps of an expert-parallel plan, as uploaded to the device.
// Entry (t, i), i < topk, is token t's i-th expert in ascending expert id:
//   slot_rank[t*k+i], slot_row[t*k+i]  where the row sits in the dispatch
//   layout; weight[t*k+i] its combine weight; col[t*k+i] the column j of the
//   routing arrays (topk_idx[t][j]) it came from, so per-call weights given in
//   the routing order can be applied.
struct RowMaps {
  int64_t tokens = 0, hidden = 0;
  int32_t experts = 0, topk = 0, dir = 0;
  std::vector<int32_t> slot;    // [T*k] packed (rank << 26) | row
  std::vector<float> weight;    // [T*k]
  std::vector<int32_t> col;     // [T*k]
  std::vector<int64_t> rows_per_rank;
  // Byte offsets of the maps inside the workspace (host-built plans: slot,
  // weight and col; device-routed plans: all of them).
  int64_t nblk = 0;             // token blocks of kRouteBlock tokens
  size_t off_slot = 0, off_weight = 0, off_col = 0, off_counts = 0, off_expert = 0, off_rank = 0,
         off_bcounts = 0, off_bbase = 0, off_status = 0, off_bstatus = 0;
  // Co-resident capacity (workgroups) of the fused routing kernel, queried
  // once; 0 = not yet known.
  int64_t route_cap = 0;
};

// Tokens per block of the device-side routing kernels.
constexpr int kRouteBlock = 256;
// Largest expert count the device-side routing supports (one 256-bit token
// mask per expert in LDS).
constexpr int kRouteMaxExperts = 1024;
// Largest top-k the device-side routing supports.
constexpr int kRouteMaxTopk = 16;

struct Plan {
  PlanKind kind = PlanKind::Uniform;
  int32_t nranks = 0;
  int32_t dtype = RRB_BF16;
  int32_t op = RRB_COPY;
  int64_t count = 0;
  std::vector<Segment> segs;  // all of equal length for uniform plans
  std::vector<int64_t> in_count, out_count;
  RowMaps rows;
  void *d_ws = nullptr;       // bound device workspace (row plans)
  size_t ws_bytes = 0;
};

// One kernel launch, described rather than issued: kernel, grid, block and
// the kernel's single by-value argument struct.
struct LaunchDesc {
  const void *func = nullptr;
  dim3 grid, block;
  std::vector<unsigned char> args;
  std::string name;  // the kernel and its template arguments, for introspection
};

// The launches rrb_copy / rrb_reduce would issue for a uniform plan with
// these buffers, appended to `out` (rrb_atom.hip).
rrb_status describe_uniform(const struct Plan &plan, const void *const *in, void *const *out,
                            std::vector<LaunchDesc> &descs);

// Builds a uniform plan from a layout-naming spec (rrb_plan.cpp).
rrb_status build_uniform_plan(const rrb_spec &spec, Plan &plan);
// Builds a MoE row plan (rrb_plan.cpp).
rrb_status build_row_plan(int32_t nranks, int64_t tokens, int64_t hidden,
                          int32_t experts, int32_t topk, const int32_t *idx,
                          const float *w, int32_t dir, Plan &plan);

// Builds a MoE row plan whose maps are computed on the device (rrb_plan.cpp).
rrb_status build_row_plan_device(int32_t nranks, int64_t tokens, int64_t hidden,
                                 int32_t experts, int32_t topk, int32_t dir, Plan &plan);
// Enqueues the device-side routing kernels of a device row plan (rrb_moe.hip).
rrb_status launch_route(Plan &plan, const int32_t *d_idx, const float *d_w,
                        int32_t *d_rank_offsets, void *stream);

// Zero-fills a device row plan's slot map and status word on `stream`, so a
// copy or reduce before the first rrb_moe_route stays in bounds (rrb_moe.hip).
rrb_status clear_route_maps(const Plan &plan, void *stream);

// Launches a MoE row plan (rrb_moe.hip).  `stream` is a hipStream_t.
// d_weights (combine only, nullable): per-call weights [T][k] in the order of
// the routing arrays, in place of the plan's own.
rrb_status launch_rows(const Plan &plan, const void *const *in, void *const *out,
                       const float *d_weights, void *stream);

constexpr int kSlotRankShift = 26;
constexpr int32_t kSlotRowMask = (1 << kSlotRankShift) - 1;

}  // namespace rrb

struct rrb_plan_s {
  rrb::Plan p;
};
