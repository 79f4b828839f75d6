// Plan builder: layout naming -> index map (host only, C++17).
//
// Purlin: Separating Orchestration from the Datapath of Collectives ("The
// Purlin PDF describes a three-layer design") specifies a collective as a
// naming of an input and an output layout plus copy or reduce, and has the
// orchestration derive everything else from that spec.  Here the derivation
// is: enumerate the names each rank's local blocks carry under both layouts,
// match every output block to its source block(s), then group output blocks
// that read the same source into one fan-out segment, and fuse the segments
// into a single one when they tile the buffers contiguously (All-Reduce,
// Reduce, Broadcast become one segment; the others keep one per block).
//
// Names live in one of two spaces:
//   X-space: blocks X[b] of the logical tensor (PARTIAL, REPLICATED, SHARD,
//            ROOT); PARTIAL blocks are rank q's contribution to X[b].
//   M-space: blocks M[r][q] of an R x R block matrix (BLOCK_ROW, BLOCK_COL).
// nb, the number of blocks X splits into, is R when either layout names
// blocks and 1 otherwise (so All-Reduce of any length needs no divisibility).
#include <algorithm>
#include <map>
#include <new>
#include <tuple>

#include "rrb_internal.h"

namespace rrb {
namespace {

struct Name {
  int32_t a, b;  // X-space: (-1, block); M-space: (row, col)
  bool operator<(const Name &o) const { return std::tie(a, b) < std::tie(o.a, o.b); }
};

bool names_blocks(int32_t k) {
  return k == RRB_SHARD || k == RRB_BLOCK_ROW || k == RRB_BLOCK_COL;
}
bool m_space(int32_t k) { return k == RRB_BLOCK_ROW || k == RRB_BLOCK_COL; }

// Names of rank q's local blocks, in local order.
std::vector<Name> local_names(const rrb_layout &l, int32_t q, int32_t R, int32_t nb) {
  std::vector<Name> v;
  switch (l.kind) {
    case RRB_PARTIAL:
    case RRB_REPLICATED:
      for (int32_t b = 0; b < nb; ++b) v.push_back({-1, b});
      break;
    case RRB_SHARD:
      v.push_back({-1, q});
      break;
    case RRB_ROOT:
      if (q == l.root)
        for (int32_t b = 0; b < nb; ++b) v.push_back({-1, b});
      break;
    case RRB_BLOCK_ROW:
      for (int32_t b = 0; b < R; ++b) v.push_back({q, b});
      break;
    case RRB_BLOCK_COL:
      for (int32_t b = 0; b < R; ++b) v.push_back({b, q});
      break;
  }
  return v;
}

bool valid_kind(int32_t k) { return k >= RRB_PARTIAL && k <= RRB_BLOCK_COL; }

// Fuse all segments into one when they share source rank and destination
// set and their source and destination offsets advance together by len.
void fuse_if_contiguous(std::vector<Segment> &segs) {
  if (segs.size() < 2) return;
  std::vector<Segment> s = segs;
  std::sort(s.begin(), s.end(),
            [](const Segment &x, const Segment &y) { return x.src_off < y.src_off; });
  for (size_t i = 1; i < s.size(); ++i) {
    if (s[i].src_rank != s[0].src_rank || s[i].dst_mask != s[0].dst_mask ||
        s[i].len != s[0].len || s[i].src_off != s[i - 1].src_off + s[i - 1].len ||
        s[i].dst_off != s[i - 1].dst_off + s[i - 1].len)
      return;
  }
  Segment one = s[0];
  one.len = s[0].len * static_cast<int64_t>(s.size());
  segs.assign(1, one);
}

}  // namespace

rrb_status build_uniform_plan(const rrb_spec &spec, Plan &plan) {
  const int32_t R = spec.nranks;
  if (R < 1 || R > RRB_MAX_RANKS)
    return fail(RRB_EINVAL, "nranks %d outside 1..%d", R, RRB_MAX_RANKS);
  if (spec.dtype != RRB_BF16 && spec.dtype != RRB_F32)
    return fail(RRB_EINVAL, "unknown dtype %d", spec.dtype);
  if (spec.op != RRB_COPY && spec.op != RRB_REDUCE_SUM && spec.op != RRB_REDUCE_SUM_TREE)
    return fail(RRB_EINVAL, "unknown op %d", spec.op);
  if (spec.count < 0) return fail(RRB_EINVAL, "negative count");
  if (spec.reserved != 0) return fail(RRB_EINVAL, "reserved field must be 0");
  const rrb_layout in = spec.in, out = spec.out;
  if (!valid_kind(in.kind) || !valid_kind(out.kind))
    return fail(RRB_EINVAL, "unknown layout kind (in %d, out %d)", in.kind, out.kind);
  for (const rrb_layout *l : {&in, &out})
    if (l->kind == RRB_ROOT && (l->root < 0 || l->root >= R))
      return fail(RRB_EINVAL, "root %d outside 0..%d", l->root, R - 1);
  if (out.kind == RRB_PARTIAL)
    return fail(RRB_EINVAL, "PARTIAL names contributions and cannot be an output layout");
  if (m_space(in.kind) != m_space(out.kind))
    return fail(RRB_EINVAL, "BLOCK_ROW/BLOCK_COL only pair with each other");
  const bool reduce = spec.op != RRB_COPY;
  if (reduce != (in.kind == RRB_PARTIAL))
    return fail(RRB_EINVAL, reduce ? "reduce needs a PARTIAL input layout"
                                   : "a PARTIAL input needs the reduce op");

  const int64_t n = spec.count;
  const bool blocked = names_blocks(in.kind) || names_blocks(out.kind);
  if (blocked && n % R != 0)
    return fail(RRB_EINVAL, "layouts that name blocks need count %% nranks == 0 "
                            "(count %lld, nranks %d)", (long long)n, R);
  const int32_t nb = blocked ? R : 1;
  const int64_t c = blocked ? n / R : n;

  plan.kind = PlanKind::Uniform;
  plan.nranks = R;
  plan.dtype = spec.dtype;
  plan.op = spec.op;
  plan.count = n;
  plan.in_count.assign(R, 0);
  plan.out_count.assign(R, 0);
  plan.segs.clear();

  std::vector<std::vector<Name>> in_names(R), out_names(R);
  for (int32_t q = 0; q < R; ++q) {
    in_names[q] = local_names(in, q, R, nb);
    out_names[q] = local_names(out, q, R, nb);
    plan.in_count[q] = static_cast<int64_t>(in_names[q].size()) * c;
    plan.out_count[q] = static_cast<int64_t>(out_names[q].size()) * c;
  }

  // Source of every name: (rank, local block); lowest rank wins.
  std::map<Name, std::pair<int32_t, int32_t>> where;
  for (int32_t r = 0; r < R; ++r)
    for (int32_t i = 0; i < static_cast<int32_t>(in_names[r].size()); ++i)
      where.emplace(in_names[r][i], std::make_pair(r, i));

  // Group output blocks by what they read: (src_rank, src_off, dst_off).
  std::map<std::tuple<int32_t, int64_t, int64_t>, uint32_t> groups;
  for (int32_t q = 0; q < R; ++q) {
    for (int32_t i = 0; i < static_cast<int32_t>(out_names[q].size()); ++i) {
      const Name nm = out_names[q][i];
      int32_t src_rank;
      int64_t src_off;
      if (reduce) {
        // Output X[b] folds every rank's partial of block b, which sits at
        // local block b of a PARTIAL buffer.
        src_rank = -1;
        src_off = static_cast<int64_t>(nm.b) * c;
      } else {
        auto it = where.find(nm);
        if (it == where.end())
          return fail(RRB_EINVAL, "output rank %d block %d names a block the input "
                                  "layout does not hold", q, i);
        src_rank = it->second.first;
        src_off = static_cast<int64_t>(it->second.second) * c;
      }
      groups[std::make_tuple(src_rank, src_off, static_cast<int64_t>(i) * c)] |= (1u << q);
    }
  }
  for (const auto &g : groups) {
    Segment s;
    s.src_rank = std::get<0>(g.first);
    s.src_off = std::get<1>(g.first);
    s.dst_off = std::get<2>(g.first);
    s.len = c;
    s.dst_mask = g.second;
    plan.segs.push_back(s);
  }
  fuse_if_contiguous(plan.segs);
  return RRB_OK;
}

rrb_status build_row_plan(int32_t R, int64_t T, int64_t h, int32_t E, int32_t k,
                          const int32_t *idx, const float *w, int32_t dir, Plan &plan) {
  if (R < 1 || R > RRB_MAX_RANKS)
    return fail(RRB_EINVAL, "nranks %d outside 1..%d", R, RRB_MAX_RANKS);
  if (T < 0 || h <= 0 || E < 1 || k < 1 || k > E)
    return fail(RRB_EINVAL, "bad MoE shape: tokens %lld hidden %lld experts %d topk %d",
                (long long)T, (long long)h, E, k);
  if (h >= (int64_t(1) << 30)) return fail(RRB_EUNSUPPORTED, "token rows of 2 GiB or more");
  if (T % R != 0) return fail(RRB_EINVAL, "tokens must divide evenly over the ranks");
  if (E % R != 0) return fail(RRB_EINVAL, "experts must divide evenly over the ranks");
  if (dir != RRB_MOE_DISPATCH && dir != RRB_MOE_COMBINE)
    return fail(RRB_EINVAL, "unknown MoE direction %d", dir);
  if (T > 0 && (idx == nullptr || (dir == RRB_MOE_COMBINE && w == nullptr)))
    return fail(RRB_EINVAL, "routing arrays are NULL");
  if (T * k >= (int64_t(1) << kSlotRankShift))
    return fail(RRB_EUNSUPPORTED, "more than 2^26 routed rows");
  const int32_t per = E / R;

  // Count tokens per expert, checking indices and distinctness per row.
  std::vector<int64_t> count(E, 0);
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < k; ++j) {
      const int32_t e = idx[t * k + j];
      if (e < 0 || e >= E) return fail(RRB_EINVAL, "token %lld routes to expert %d", (long long)t, e);
      for (int32_t j2 = 0; j2 < j; ++j2)
        if (idx[t * k + j2] == e)
          return fail(RRB_EINVAL, "token %lld selects expert %d twice", (long long)t, e);
      ++count[e];
    }
  }
  // Expert-major receive layout: offsets are exclusive prefix sums over the
  // experts of each rank.
  std::vector<int64_t> off(E, 0);
  RowMaps &m = plan.rows;
  m.rows_per_rank.assign(R, 0);
  for (int32_t e = 0; e < E; ++e) {
    const int32_t r = e / per;
    off[e] = m.rows_per_rank[r];
    m.rows_per_rank[r] += count[e];
  }
  // Slots: tokens visited in ascending order give ascending rows per expert.
  std::vector<int64_t> fill(E, 0);
  m.slot.assign(static_cast<size_t>(T * k), 0);
  m.weight.assign(static_cast<size_t>(T * k), 0.f);
  m.col.assign(static_cast<size_t>(T * k), 0);
  std::vector<std::pair<int32_t, int32_t>> order(k);
  for (int64_t t = 0; t < T; ++t) {
    for (int32_t j = 0; j < k; ++j) order[j] = {idx[t * k + j], j};
    std::sort(order.begin(), order.end());  // ascending expert id
    for (int32_t i = 0; i < k; ++i) {
      const int32_t e = order[i].first;
      const int64_t row = off[e] + fill[e]++;
      m.slot[t * k + i] = ((e / per) << kSlotRankShift) | static_cast<int32_t>(row);
      m.weight[t * k + i] = w ? w[t * k + order[i].second] : 0.f;
      m.col[t * k + i] = order[i].second;
    }
  }
  m.tokens = T;
  m.hidden = h;
  m.experts = E;
  m.topk = k;
  m.dir = dir;

  plan.kind = PlanKind::Rows;
  plan.nranks = R;
  plan.dtype = RRB_BF16;
  plan.op = dir == RRB_MOE_DISPATCH ? RRB_COPY : RRB_REDUCE_SUM;
  plan.count = T * h;
  plan.segs.clear();
  const int64_t Tr = T / R;
  plan.in_count.assign(R, 0);
  plan.out_count.assign(R, 0);
  for (int32_t r = 0; r < R; ++r) {
    const int64_t recv = m.rows_per_rank[r] * h;
    if (dir == RRB_MOE_DISPATCH) {
      plan.in_count[r] = Tr * h;
      plan.out_count[r] = recv;
    } else {
      plan.in_count[r] = recv;
      plan.out_count[r] = Tr * h;
    }
  }
  // Device map: slot[T*k] int32, weight[T*k] float, col[T*k] int32, each
  // 256-byte aligned.
  const size_t map_bytes = ((static_cast<size_t>(T * k) * 4 + 255) / 256) * 256;
  m.off_slot = 0;
  m.off_weight = map_bytes;
  m.off_col = 2 * map_bytes;
  plan.ws_bytes = 3 * map_bytes;
  return RRB_OK;
}

rrb_status build_row_plan_device(int32_t R, int64_t T, int64_t h, int32_t E, int32_t k,
                                 int32_t dir, Plan &plan) {
  if (R < 1 || R > RRB_MAX_RANKS)
    return fail(RRB_EINVAL, "nranks %d outside 1..%d", R, RRB_MAX_RANKS);
  if (T < 0 || h <= 0 || E < 1 || k < 1 || k > E)
    return fail(RRB_EINVAL, "bad MoE shape: tokens %lld hidden %lld experts %d topk %d",
                (long long)T, (long long)h, E, k);
  if (h >= (int64_t(1) << 30)) return fail(RRB_EUNSUPPORTED, "token rows of 2 GiB or more");
  if (T % R != 0) return fail(RRB_EINVAL, "tokens must divide evenly over the ranks");
  if (E % R != 0) return fail(RRB_EINVAL, "experts must divide evenly over the ranks");
  if (dir != RRB_MOE_DISPATCH && dir != RRB_MOE_COMBINE)
    return fail(RRB_EINVAL, "unknown MoE direction %d", dir);
  if (E > kRouteMaxExperts)
    return fail(RRB_EUNSUPPORTED, "device routing supports at most %d experts", kRouteMaxExperts);
  if (k > kRouteMaxTopk)
    return fail(RRB_EUNSUPPORTED, "device routing supports top-k up to %d", kRouteMaxTopk);
  if (T * k >= (int64_t(1) << kSlotRankShift) || T * k > 0x7fffffffLL)
    return fail(RRB_EUNSUPPORTED, "more than 2^26 routed rows");
  RowMaps &m = plan.rows;
  m = RowMaps();
  m.tokens = T;
  m.hidden = h;
  m.experts = E;
  m.topk = k;
  m.dir = dir;
  m.nblk = (T + kRouteBlock - 1) / kRouteBlock;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = 0;
  const size_t tk = static_cast<size_t>(T * k);
  m.off_slot = off;    off += up(tk * 4);
  m.off_weight = off;  off += up(tk * 4);
  m.off_col = off;     off += up(tk * 4);
  m.off_counts = off;  off += up(static_cast<size_t>(E) * 4);
  m.off_expert = off;  off += up(static_cast<size_t>(E) * 4);
  m.off_rank = off;    off += up(static_cast<size_t>(R + 1) * 4);
  m.off_bcounts = off; off += up(static_cast<size_t>(m.nblk) * E * 4);
  m.off_bbase = off;   off += up(static_cast<size_t>(m.nblk) * E * 4);
  m.off_status = off;  off += 256;  // status word; barrier counter at +128
  m.off_bstatus = off; off += up(static_cast<size_t>(m.nblk) * 4);
  plan.ws_bytes = off;
  plan.kind = PlanKind::RowsDevice;
  plan.nranks = R;
  plan.dtype = RRB_BF16;
  plan.op = dir == RRB_MOE_DISPATCH ? RRB_COPY : RRB_REDUCE_SUM;
  plan.count = T * h;
  plan.segs.clear();
  const int64_t Tr = T / R;
  plan.in_count.assign(R, 0);
  plan.out_count.assign(R, 0);
  // The receive side is one arena of exactly T*k rows: rank r's rows (its
  // experts in ascending id, tokens ascending within an expert) start at
  // rank_offsets[r].  It is rank 0's buffer in the pointer arrays.
  for (int32_t r = 0; r < R; ++r) {
    if (dir == RRB_MOE_DISPATCH) plan.in_count[r] = Tr * h;
    else plan.out_count[r] = Tr * h;
  }
  if (dir == RRB_MOE_DISPATCH) plan.out_count[0] = T * k * h;
  else plan.in_count[0] = T * k * h;
  return RRB_OK;
}

}  // namespace rrb
