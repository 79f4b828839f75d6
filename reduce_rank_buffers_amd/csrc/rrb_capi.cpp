// C ABI: error reporting and the plan entry points (host only).
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>

#include <hip/hip_runtime.h>

#include "rrb_internal.h"

namespace rrb {
namespace {
thread_local char g_last_error[512] = "";
}

rrb_status fail(rrb_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

void clear_error() { g_last_error[0] = '\0'; }

}  // namespace rrb

using namespace rrb;

extern "C" {

const char *rrb_status_string(rrb_status s) {
  switch (s) {
    case RRB_OK: return "ok";
    case RRB_EINVAL: return "invalid argument";
    case RRB_EUNSUPPORTED: return "unsupported";
    case RRB_EHIP: return "HIP runtime error";
    case RRB_ETIMEOUT: return "bounded wait timed out";
    case RRB_ENOMEM: return "host allocation failed";
    default: return "unknown status";
  }
}

const char *rrb_last_error(void) { return g_last_error; }

int32_t rrb_abi_version(void) { return RRB_ABI_VERSION; }

rrb_status rrb_plan_create(const rrb_spec *spec, rrb_plan_t *out) {
  clear_error();
  if (!spec || !out) return fail(RRB_EINVAL, "NULL spec or out");
  *out = nullptr;
  rrb_plan_s *p = new (std::nothrow) rrb_plan_s;
  if (!p) return fail(RRB_ENOMEM, "plan allocation failed");
  rrb_status s;
  try {
    s = build_uniform_plan(*spec, p->p);
  } catch (const std::bad_alloc &) {
    s = fail(RRB_ENOMEM, "plan allocation failed");
  }
  if (s != RRB_OK) {
    delete p;
    return s;
  }
  *out = p;
  return RRB_OK;
}

rrb_status rrb_plan_create_rows(int32_t nranks, int64_t tokens, int64_t hidden,
                                int32_t experts, int32_t topk, const int32_t *topk_idx,
                                const float *topk_w, int32_t dir, rrb_plan_t *out) {
  clear_error();
  if (!out) return fail(RRB_EINVAL, "NULL out");
  *out = nullptr;
  rrb_plan_s *p = new (std::nothrow) rrb_plan_s;
  if (!p) return fail(RRB_ENOMEM, "plan allocation failed");
  rrb_status s;
  try {
    s = build_row_plan(nranks, tokens, hidden, experts, topk, topk_idx, topk_w, dir, p->p);
  } catch (const std::bad_alloc &) {
    s = fail(RRB_ENOMEM, "plan allocation failed");
  }
  if (s != RRB_OK) {
    delete p;
    return s;
  }
  *out = p;
  return RRB_OK;
}

rrb_status rrb_plan_create_rows_device(int32_t nranks, int64_t tokens, int64_t hidden,
                                       int32_t experts, int32_t topk, int32_t dir,
                                       rrb_plan_t *out) {
  clear_error();
  if (!out) return fail(RRB_EINVAL, "NULL out");
  *out = nullptr;
  rrb_plan_s *p = new (std::nothrow) rrb_plan_s;
  if (!p) return fail(RRB_ENOMEM, "plan allocation failed");
  rrb_status s;
  try {
    s = build_row_plan_device(nranks, tokens, hidden, experts, topk, dir, p->p);
  } catch (const std::bad_alloc &) {
    s = fail(RRB_ENOMEM, "plan allocation failed");
  }
  if (s != RRB_OK) {
    delete p;
    return s;
  }
  *out = p;
  return RRB_OK;
}

rrb_status rrb_moe_route(rrb_plan_t plan, const int32_t *d_topk_idx, const float *d_topk_w,
                         int32_t *d_rank_offsets, rrb_stream_t stream) {
  clear_error();
  if (!plan) return fail(RRB_EINVAL, "NULL plan");
  Plan &p = plan->p;
  if (p.kind != PlanKind::RowsDevice) return fail(RRB_EINVAL, "rrb_moe_route needs a device row plan");
  if (!p.d_ws) return fail(RRB_EINVAL, "plan is not bound to a workspace");
  if (p.rows.tokens > 0 && (!d_topk_idx || !d_topk_w)) return fail(RRB_EINVAL, "NULL routing arrays");
  return launch_route(p, d_topk_idx, d_topk_w, d_rank_offsets, stream);
}

rrb_status rrb_moe_route_check(rrb_plan_t plan, rrb_stream_t stream) {
  clear_error();
  if (!plan) return fail(RRB_EINVAL, "NULL plan");
  const Plan &p = plan->p;
  if (p.kind != PlanKind::RowsDevice || !p.d_ws) return fail(RRB_EINVAL, "not a bound device row plan");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  int32_t st = 0;
  std::vector<int32_t> bst;
  try {
    bst.assign(static_cast<size_t>(p.rows.nblk), 0);
  } catch (const std::bad_alloc &) {
    return fail(RRB_ENOMEM, "route status buffer allocation failed");
  }
  if (e == hipSuccess)
    e = hipMemcpy(&st, static_cast<const char *>(p.d_ws) + p.rows.off_status, 4, hipMemcpyDeviceToHost);
  // Per-block words of the fused routing kernel (zero for the three-kernel path).
  if (e == hipSuccess && !bst.empty())
    e = hipMemcpy(bst.data(), static_cast<const char *>(p.d_ws) + p.rows.off_bstatus,
                  bst.size() * 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(RRB_EHIP, "route status read: %s", hipGetErrorString(e));
  for (int32_t b : bst) st |= b;
  if (st & 1) return fail(RRB_EINVAL, "routing names an expert outside 0..experts-1");
  if (st & 2) return fail(RRB_EINVAL, "routing selects an expert twice for one token");
  if (st & 4) return fail(RRB_ETIMEOUT, "routing grid barrier timed out; rebind the plan");
  return RRB_OK;
}

rrb_status rrb_plan_query(rrb_plan_t plan, size_t *workspace_bytes, int64_t *in_count,
                          int64_t *out_count) {
  clear_error();
  if (!plan) return fail(RRB_EINVAL, "NULL plan");
  const Plan &p = plan->p;
  if (workspace_bytes) *workspace_bytes = p.ws_bytes;
  for (int32_t r = 0; r < p.nranks; ++r) {
    if (in_count) in_count[r] = p.in_count[r];
    if (out_count) out_count[r] = p.out_count[r];
  }
  return RRB_OK;
}

rrb_status rrb_plan_bind(rrb_plan_t plan, void *d_workspace, size_t bytes, rrb_stream_t stream) {
  clear_error();
  if (!plan) return fail(RRB_EINVAL, "NULL plan");
  Plan &p = plan->p;
  if (p.ws_bytes == 0) return RRB_OK;
  if (!d_workspace || bytes < p.ws_bytes)
    return fail(RRB_EINVAL, "workspace of %zu bytes needed", p.ws_bytes);
  if (reinterpret_cast<uintptr_t>(d_workspace) % 256)
    return fail(RRB_EINVAL, "workspace must be 256-byte aligned");
  if (p.kind == PlanKind::RowsDevice) {
    // Maps are written by rrb_moe_route on the device; until then every slot
    // is row 0 of the arena (in bounds).
    p.d_ws = d_workspace;
    return clear_route_maps(p, stream);
  }
  const RowMaps &m = p.rows;
  const size_t n = m.slot.size();
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (n) {
    char *ws = static_cast<char *>(d_workspace);
    e = hipMemcpyAsync(ws + m.off_slot, m.slot.data(), n * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(ws + m.off_weight, m.weight.data(), n * 4, hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
      e = hipMemcpyAsync(ws + m.off_col, m.col.data(), n * 4, hipMemcpyHostToDevice, s);
    // The host maps belong to the plan; wait so a later destroy cannot free
    // them under an in-flight copy.
    if (e == hipSuccess) e = hipStreamSynchronize(s);
  }
  if (e != hipSuccess) return fail(RRB_EHIP, "map upload: %s", hipGetErrorString(e));
  p.d_ws = d_workspace;
  return RRB_OK;
}

rrb_status rrb_plan_segments(rrb_plan_t plan, rrb_segment *out, int32_t cap, int32_t *n) {
  clear_error();
  if (!plan || !n) return fail(RRB_EINVAL, "NULL plan or n");
  if (cap > 0 && !out) return fail(RRB_EINVAL, "NULL out with cap %d", cap);
  const Plan &p = plan->p;
  *n = static_cast<int32_t>(p.segs.size());
  for (int32_t i = 0; i < cap && i < *n; ++i) {
    const Segment &s = p.segs[i];
    out[i].src_off = s.src_off;
    out[i].dst_off = s.dst_off;
    out[i].len = s.len;
    out[i].src_rank = s.src_rank;
    out[i].dst_mask = s.dst_mask;
  }
  return RRB_OK;
}

void rrb_plan_destroy(rrb_plan_t plan) { delete plan; }

}  // extern "C"
