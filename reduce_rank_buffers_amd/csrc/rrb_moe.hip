// Expert-parallel MoE dispatch and combine as Atom copy / reduce over row maps.
//
// The two datapath primitives of Purlin: Separating Orchestration from the
// Datapath of Collectives ("The Purlin PDF describes a three-layer design")
// carry the MoE all-to-all pair when the index map is a row map:
//   dispatch (copy):   every token row is read once and written to the
//                      receive slot of each of its k experts;
//   combine (reduce):  every token gathers its k expert rows, folds
//                      fl32(w * row) in ascending expert id with one multiply
//                      then one add per step, and rounds once to bf16.
// A token row is split into equal parts, one workgroup per (token, part), so
// the map entries a workgroup needs (k slots and weights) are uniform and
// come through scalar loads; the row itself moves as coalesced 16-byte
// vectors.  Both kernels are HBM-bound: dispatch reads T*h
// and writes T*k*h elements, combine the reverse.
#include <hip/hip_runtime.h>

#include <cstring>

#include "rrb_internal.h"
#include "rrb_kernels.h"

// Combine must not contract w * z + acc into a fused multiply-add.
#pragma clang fp contract(off)

namespace rrb {

struct RowArgs {
  const unsigned char *in[RRB_MAX_RANKS];
  unsigned char *out[RRB_MAX_RANKS];
  const int32_t *slot;   // [T*k] (rank << kSlotRankShift) | row, ascending expert
  const float *weight;   // [T*k]
  const int32_t *col;    // [T*k] routing-array column of each slot
  const float *wover;    // combine: per-call weights [T][k] in routing order, or NULL
  int64_t tokens_per_rank;
  int64_t row_bytes;     // hidden * 2
  int64_t nvec;          // whole 16-byte vectors per row
  int64_t hidden;
  int64_t part_vec;      // vector path: vectors per row part (one workgroup each)
  int32_t parts;         // vector path: parts per row
  int32_t k;
  // Device-routed plans: the routing status word; nonzero (a routing with an
  // invalid entry, or a barrier wait that ran out) stops the launch before
  // it writes anything.  NULL for host-built plans.
  const int32_t *route_status;
};

// True when the plan's last device-side routing failed: the kernel then
// leaves every output untouched (rrb_moe_route_check reports why).
__device__ __forceinline__ bool route_failed(const RowArgs &a) {
  return a.route_status && *a.route_status != 0;
}

// The routing status word, 0 for host-built plans.  The branch is on a
// kernel argument, so the load is a scalar load issued without a wait.
__device__ __forceinline__ int32_t route_status_word(const RowArgs &a) {
  int32_t st = 0;
  if (a.route_status) st = *a.route_status;
  return st;
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// One workgroup per part of a token row, one 16-byte vector per lane, each
// written to the token's k receive slots with non-temporal stores (the 1->k
// fan-out streams past the caches; measured 6.7 TB/s on MI355X for 1->8 vs
// 5.2 with plain stores).  Parts of at most 256 vectors: for a 7168-wide row,
// 4 parts of 224 vectors ran 4-7% ahead of one 128-lane workgroup with 8
// vectors per lane (interleaved A/B runs, 4096 tokens, top-8).
//
// The token's K slots are read before the first store.  Reads that no store
// precedes are scalar loads issued in one batch; a slot read between stores
// becomes a vector load, and the wait for it (vmcnt counts stores too) makes
// each of the K stores finish before the next one is issued.  Token and
// vector indices fit 32 bits (tokens * k < 2^26, rows < 2^31 bytes).
//
// The routing status is read in the same batch and decides without a branch:
// after a failed routing every slot reads as 0 (a failed routing may leave
// them unset) and the row loop is empty, so nothing is written.
template <int K>
__global__ void __launch_bounds__(256) moe_dispatch_kernel(RowArgs a) {
  const uint32_t parts = static_cast<uint32_t>(a.parts);
  const uint32_t t = blockIdx.x / parts;
  const int32_t status = route_status_word(a);
  const int32_t *slots = a.slot + static_cast<int64_t>(t) * K;
  int32_t s[K];
#pragma unroll
  for (int j = 0; j < K; ++j) s[j] = slots[j];
  const bool ok = status == 0;
#pragma unroll
  for (int j = 0; j < K; ++j) s[j] = ok ? s[j] : 0;
  const uint32_t tpr = static_cast<uint32_t>(a.tokens_per_rank);
  const uint32_t src_rank = t / tpr;
  const unsigned char *src = a.in[src_rank] + static_cast<int64_t>(t - src_rank * tpr) * a.row_bytes;
  unsigned char *dst[K];
#pragma unroll
  for (int j = 0; j < K; ++j)
    dst[j] = a.out[s[j] >> kSlotRankShift] + static_cast<int64_t>(s[j] & kSlotRowMask) * a.row_bytes;
  const uint32_t pv = static_cast<uint32_t>(a.part_vec), nv = static_cast<uint32_t>(a.nvec);
  const uint32_t v0 = (blockIdx.x - t * parts) * pv;
  const uint32_t v1 = !ok ? v0 : v0 + pv < nv ? v0 + pv : nv;
  for (uint32_t i = v0 + threadIdx.x; i < v1; i += blockDim.x) {
    const v4u x = *reinterpret_cast<const v4u *>(src + i * 16);
#pragma unroll
    for (int j = 0; j < K; ++j)
      __builtin_nontemporal_store(x, reinterpret_cast<v4u *>(dst[j] + i * 16));
  }
}

// Top-k above 16: the same copy with the slots read per store.
__global__ void __launch_bounds__(256) moe_dispatch_any_kernel(RowArgs a) {
  if (route_failed(a)) return;
  const int64_t t = blockIdx.x / a.parts;
  const int64_t v0 = (static_cast<int64_t>(blockIdx.x) - t * a.parts) * a.part_vec;
  const int64_t v1 = v0 + a.part_vec < a.nvec ? v0 + a.part_vec : a.nvec;
  const int64_t src_rank = t / a.tokens_per_rank;
  const unsigned char *src =
      a.in[src_rank] + (t - src_rank * a.tokens_per_rank) * a.row_bytes;
  const int32_t *slots = a.slot + t * a.k;
  for (int64_t i = v0 + threadIdx.x; i < v1; i += blockDim.x) {
    const v4u x = *reinterpret_cast<const v4u *>(src + i * 16);
    for (int j = 0; j < a.k; ++j) {
      const int32_t s = slots[j];
      unsigned char *dst = a.out[s >> kSlotRankShift] +
                           static_cast<int64_t>(s & kSlotRowMask) * a.row_bytes;
      __builtin_nontemporal_store(x, reinterpret_cast<v4u *>(dst + i * 16));
    }
  }
}

// Any hidden size: 2-byte units.
__global__ void __launch_bounds__(256) moe_dispatch_elem_kernel(RowArgs a) {
  if (route_failed(a)) return;
  const int64_t t = blockIdx.x;
  const int64_t src_rank = t / a.tokens_per_rank;
  const unsigned char *src =
      a.in[src_rank] + (t - src_rank * a.tokens_per_rank) * a.row_bytes;
  const int32_t *slots = a.slot + t * a.k;
  for (int64_t i = threadIdx.x; i < a.hidden; i += blockDim.x) {
    const uint16_t x = *reinterpret_cast<const uint16_t *>(src + i * 2);
    for (int j = 0; j < a.k; ++j) {
      const int32_t s = slots[j];
      unsigned char *dst = a.out[s >> kSlotRankShift] +
                           static_cast<int64_t>(s & kSlotRowMask) * a.row_bytes;
      *reinterpret_cast<uint16_t *>(dst + i * 2) = x;
    }
  }
}

// Fold of one 16-byte vector (8 bf16 lanes) over the K expert rows in
// ascending expert id: acc = w_0 * z_0, then acc = acc + w_j * z_j, each a
// separate fp32 multiply and add (contraction is off in this file).
template <int K>
__device__ __forceinline__ v4u combine_vec(const v4u (&z)[K], const float (&w)[K]) {
  float acc[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc[2 * q] = w[0] * bf16_lo(z[0][q]);
    acc[2 * q + 1] = w[0] * bf16_hi(z[0][q]);
  }
#pragma unroll
  for (int j = 1; j < K; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float lo = w[j] * bf16_lo(z[j][q]);
      const float hi = w[j] * bf16_hi(z[j][q]);
      acc[2 * q] = acc[2 * q] + lo;
      acc[2 * q + 1] = acc[2 * q + 1] + hi;
    }
  }
  const uint4 p = pack_bf16x8(acc);
  return v4u{p.x, p.y, p.z, p.w};
}

// One workgroup per part of a token row: CU vectors x K rows in flight per
// lane (K * CU >= 8), non-temporal loads (every expert row is read once) and
// write-through stores (the cache policy of agent-scope atomic stores, sc1):
// 88.2 us against 90.6 non-temporal and 94.2 plain, 4096 x 7168, top-8,
// interleaved A/B on MI355X.  Parts of 128 * CU
// vectors: for a 7168-wide row and top-8, 7 parts of 128 lanes ran 3-4% ahead
// of one 256-lane workgroup with 4 vectors per lane (interleaved A/B runs).
template <int K, int CU>
__global__ void __launch_bounds__(128) moe_combine_kernel(RowArgs a) {
  const uint32_t parts = static_cast<uint32_t>(a.parts);
  const uint32_t t = blockIdx.x / parts;
  const int64_t tk = static_cast<int64_t>(t) * K;
  // Routing status, slots and weights in one batch of scalar loads.  After a
  // failed routing (which may leave the maps unset) every slot reads as 0
  // and the row loop is empty, so nothing is read through the maps or
  // written.  Per-call weights follow their routing column.
  const int32_t status = route_status_word(a);
  int32_t s[K];
  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    s[j] = a.slot[tk + j];
    w[j] = a.weight[tk + j];
  }
  const bool ok = status == 0;
#pragma unroll
  for (int j = 0; j < K; ++j) s[j] = ok ? s[j] : 0;
  if (a.wover && ok) {
    int32_t c[K];
#pragma unroll
    for (int j = 0; j < K; ++j) c[j] = a.col[tk + j];
#pragma unroll
    for (int j = 0; j < K; ++j) w[j] = a.wover[tk + c[j]];
  }
  const uint32_t tpr = static_cast<uint32_t>(a.tokens_per_rank);
  const uint32_t dst_rank = t / tpr;
  unsigned char *dst = a.out[dst_rank] + static_cast<int64_t>(t - dst_rank * tpr) * a.row_bytes;
  const unsigned char *rows[K];
#pragma unroll
  for (int j = 0; j < K; ++j)
    rows[j] = a.in[s[j] >> kSlotRankShift] + static_cast<int64_t>(s[j] & kSlotRowMask) * a.row_bytes;
  const uint32_t pv = static_cast<uint32_t>(a.part_vec), nv = static_cast<uint32_t>(a.nvec);
  const uint32_t v0 = (blockIdx.x - t * parts) * pv;
  const uint32_t v1 = !ok ? v0 : v0 + pv < nv ? v0 + pv : nv;
  const uint32_t bs = blockDim.x;
  for (uint32_t i0 = v0 + threadIdx.x; i0 < v1; i0 += bs * CU) {
    v4u z[CU][K];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const uint32_t i = i0 + u * bs;
      if (i < v1) {
#pragma unroll
        for (int j = 0; j < K; ++j)
          z[u][j] = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(rows[j] + i * 16));
      }
    }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const uint32_t i = i0 + u * bs;
      if (i < v1)
        __builtin_amdgcn_raw_buffer_store_b128(
            combine_vec<K>(z[u], w),
            __builtin_amdgcn_make_buffer_rsrc(dst, static_cast<short>(0), static_cast<int>(a.row_bytes),
                                              0x00020000),
            static_cast<int32_t>(i * 16), 0, 16);
    }
  }
}

// Top-k above 16: the same combine, one vector per lane, with each row's
// slot and weight read as the fold reaches it (same terms, same order).
__global__ void __launch_bounds__(128) moe_combine_any_kernel(RowArgs a) {
  if (route_failed(a)) return;
  const int64_t t = blockIdx.x / a.parts;
  const int64_t tk = t * a.k;
  const int64_t dst_rank = t / a.tokens_per_rank;
  unsigned char *dst = a.out[dst_rank] + (t - dst_rank * a.tokens_per_rank) * a.row_bytes;
  const int64_t v0 = (static_cast<int64_t>(blockIdx.x) - t * a.parts) * a.part_vec;
  const int64_t v1 = v0 + a.part_vec < a.nvec ? v0 + a.part_vec : a.nvec;
  for (int64_t i = v0 + threadIdx.x; i < v1; i += blockDim.x) {
    float acc[8];
    for (int j = 0; j < a.k; ++j) {
      const int32_t s = a.slot[tk + j];
      const float w = a.wover ? a.wover[tk + a.col[tk + j]] : a.weight[tk + j];
      const v4u z = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(
          a.in[s >> kSlotRankShift] + static_cast<int64_t>(s & kSlotRowMask) * a.row_bytes + i * 16));
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = w * bf16_lo(z[q]);
        const float hi = w * bf16_hi(z[q]);
        acc[2 * q] = j == 0 ? lo : acc[2 * q] + lo;
        acc[2 * q + 1] = j == 0 ? hi : acc[2 * q + 1] + hi;
      }
    }
    const uint4 p = pack_bf16x8(acc);
    __builtin_amdgcn_raw_buffer_store_b128(
        v4u{p.x, p.y, p.z, p.w},
        __builtin_amdgcn_make_buffer_rsrc(dst, static_cast<short>(0), static_cast<int>(a.row_bytes), 0x00020000),
        static_cast<int32_t>(i * 16), 0, 16);
  }
}

// Rows that are not whole, aligned 16-byte vectors, any k: one element per
// lane, k rows folded in order.
__global__ void __launch_bounds__(256) moe_combine_elem_kernel(RowArgs a) {
  if (route_failed(a)) return;
  const int64_t t = blockIdx.x;
  const int64_t dst_rank = t / a.tokens_per_rank;
  unsigned char *dst = a.out[dst_rank] + (t - dst_rank * a.tokens_per_rank) * a.row_bytes;
  const int32_t *slots = a.slot + t * a.k;
  const float *ws = a.weight + t * a.k;
  const int32_t *cols = a.col + t * a.k;
  for (int64_t i = threadIdx.x; i < a.hidden; i += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j) {
      const int32_t s = slots[j];
      const unsigned char *row =
          a.in[s >> kSlotRankShift] + static_cast<int64_t>(s & kSlotRowMask) * a.row_bytes;
      const float wj = a.wover ? a.wover[t * a.k + cols[j]] : ws[j];
      const float term = wj * bf16_to_f32(*reinterpret_cast<const uint16_t *>(row + i * 2));
      acc = j == 0 ? term : acc + term;
    }
    *reinterpret_cast<uint16_t *>(dst + i * 2) = f32_to_bf16_rne(acc);
  }
}


// ---- device-side routing maps ----------------------------------------------
//
// Builds, on the GPU, the same maps rrb_plan_create_rows builds on the host:
// per-expert token counts, expert offsets in the expert-major receive arena,
// and for every (token, i) the arena row of the token's i-th expert in
// ascending id (tokens ascending within an expert) plus its weight.  Three
// kernels, all deterministic:
//   count: per block of kRouteBlock tokens, an LDS histogram of experts;
//   scan:  one workgroup per expert: exclusive prefix of its counts over
//          blocks, and its total;
//   slot:  per block, the exclusive prefix of the totals over experts (block
//          0 also stores it and the rank offsets: ranks hold contiguous
//          experts); a kRouteBlock-bit token mask per expert in LDS; a
//          token's position within its expert is the block base plus the
//          popcount of the mask bits below it.
// When the token blocks fit on the device at once, one fused kernel does all
// three (moe_route_fused_kernel): count, a grid-wide barrier, then every
// block computes the prefixes it needs itself and assigns its slots.

struct RouteArgs {
  const int32_t *idx;     // [T][k]
  const float *w;         // [T][k]
  int32_t *slot;          // [T][k] arena row, ascending expert per token
  float *weight;          // [T][k]
  int32_t *col;           // [T][k] routing-array column of each slot
  int32_t *rank_off;      // [R + 1]
  int32_t *bcounts;       // [nblk][E]
  int32_t *bbase;         // [nblk][E]
  int32_t *status;        // bit 0: expert out of range, bit 1: repeated expert
  int32_t *user_rank_off; // optional copy of rank_off
  int32_t *expert_off;    // [E]
  int32_t *counts;        // [E]
  int32_t *bstatus;       // [nblk] per-block error bits (fused kernel)
  unsigned long long *sync;  // grid-barrier arrivals, monotonic (fused kernel)
  int64_t T;
  int32_t E, k, R, per, nblk;
  uint32_t spin;          // polls before the barrier wait gives up
};

__global__ void moe_fill_kernel(int32_t *p, int64_t n, int32_t v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

// Exclusive prefix of one value per thread over the workgroup's
// kRouteBlock threads, and their total: a shuffle scan within each wave, then
// across the waves through part[kRouteBlock / 64] (one workgroup barrier).
__device__ __forceinline__ int32_t block_exclusive_prefix(int32_t v, int32_t *part, int32_t &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int32_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) part[wave] = incl;
  __syncthreads();
  total = 0;
#pragma unroll
  for (int q = 0; q < kRouteBlock / 64; ++q) {
    if (q < wave) incl += part[q];
    total += part[q];
  }
  return incl - v;
}

// Exclusive scan of v[0..n) in LDS, in place, by all kRouteBlock threads;
// returns the total.  Each thread takes a run of consecutive entries.
__device__ __forceinline__ int32_t lds_exclusive_scan(int32_t *v, int n, int32_t *part) {
  const int per_thread = (n + kRouteBlock - 1) / kRouteBlock;
  const int x0 = threadIdx.x * per_thread, x1 = min(n, x0 + per_thread);
  int32_t sum = 0;
  for (int x = x0; x < x1; ++x) sum += v[x];
  int32_t total;
  int32_t base = block_exclusive_prefix(sum, part, total);
  for (int x = x0; x < x1; ++x) {
    const int32_t c = v[x];
    v[x] = base;
    base += c;
  }
  __syncthreads();
  return total;
}

// One workgroup per expert x: bbase[b][x] = the sum of bcounts[b'][x] over
// b' < b, and counts[x] = the sum over all blocks.  Each thread takes a run
// of consecutive blocks, loaded eight at a time.
__global__ void __launch_bounds__(kRouteBlock) moe_route_scan_kernel(RouteArgs a) {
  __shared__ int32_t part[kRouteBlock / 64];
  const int x = blockIdx.x;
  const int per_thread = (a.nblk + kRouteBlock - 1) / kRouteBlock;
  const int b0 = threadIdx.x * per_thread, b1 = min(a.nblk, b0 + per_thread);
  const int32_t *__restrict__ col = a.bcounts + x;
  int32_t sum = 0;
  for (int b = b0; b < b1; b += 8) {
    int32_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = b + u < b1 ? col[static_cast<int64_t>(b + u) * a.E] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) sum += c[u];
  }
  int32_t total;
  int32_t run = block_exclusive_prefix(sum, part, total);
  for (int b = b0; b < b1; b += 8) {
    int32_t c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = b + u < b1 ? col[static_cast<int64_t>(b + u) * a.E] : 0;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (b + u < b1) a.bbase[static_cast<int64_t>(b + u) * a.E + x] = run;
      run += c[u];
    }
  }
  if (threadIdx.x == 0) a.counts[x] = total;
}

// A token's K routing entries.  They are contiguous: 16-byte loads when K
// is a multiple of 4 and the caller's arrays are 16-byte aligned.
template <int K>
__device__ __forceinline__ void load_topk(const RouteArgs &a, int64_t t, bool live, int32_t (&e)[K],
                                          float (&w)[K]) {
  const bool vec = K % 4 == 0 &&
                   ((reinterpret_cast<uintptr_t>(a.idx) | reinterpret_cast<uintptr_t>(a.w)) & 15u) == 0;
  if (vec) {
#pragma unroll
    for (int v = 0; v < K / 4; ++v) {
      int4 qi = make_int4(0, 0, 0, 0);
      float4 qw = make_float4(0.f, 0.f, 0.f, 0.f);
      if (live) {
        qi = reinterpret_cast<const int4 *>(a.idx + t * K)[v];
        qw = reinterpret_cast<const float4 *>(a.w + t * K)[v];
      }
      e[4 * v] = qi.x; e[4 * v + 1] = qi.y; e[4 * v + 2] = qi.z; e[4 * v + 3] = qi.w;
      w[4 * v] = qw.x; w[4 * v + 1] = qw.y; w[4 * v + 2] = qw.z; w[4 * v + 3] = qw.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      e[j] = live ? a.idx[t * K + j] : 0;
      w[j] = live ? a.w[t * K + j] : 0.f;
    }
  }
}

// Per block: an LDS histogram of its tokens' valid entries, stored as the
// block's row of bcounts, and the error bits of its invalid ones.
template <int K>
__global__ void __launch_bounds__(kRouteBlock) moe_route_count_kernel(RouteArgs a) {
  __shared__ int32_t hist[kRouteMaxExperts];
  __shared__ int32_t bad;
  for (int x = threadIdx.x; x < a.E; x += blockDim.x) hist[x] = 0;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteBlock + threadIdx.x;
  const bool live = t < a.T;
  int32_t e[K];
  float w[K];
  load_topk<K>(a, t, live, e, w);
  int32_t mybad = 0;
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const bool in_range = e[j] >= 0 && e[j] < a.E;
    bool dup = false;
#pragma unroll
    for (int j2 = 0; j2 < j; ++j2) dup = dup || e[j2] == e[j];
    if (live && !in_range) mybad |= 1;
    if (live && in_range && dup) mybad |= 2;
    if (live && in_range && !dup) atomicAdd(&hist[e[j]], 1);
  }
  if (mybad) atomicOr(&bad, mybad);
  __syncthreads();
  if (threadIdx.x == 0 && bad) atomicOr(a.status, bad);
  for (int x = threadIdx.x; x < a.E; x += blockDim.x)
    a.bcounts[static_cast<int64_t>(blockIdx.x) * a.E + x] = hist[x];
}

// Stable exchange sort of a token's entries by expert id (c: the entries'
// original positions), the swaps taken as selects rather than branches the
// lanes disagree on.
template <int K>
__device__ __forceinline__ void sort_by_expert(int32_t (&e)[K], float (&w)[K], bool (&ok)[K],
                                               int32_t (&c)[K]) {
#pragma unroll
  for (int j = 0; j < K; ++j) c[j] = j;
#pragma unroll
  for (int i = 0; i < K; ++i) {
#pragma unroll
    for (int j = 0; j + 1 < K - i; ++j) {
      const bool sw = e[j] > e[j + 1];
      const int32_t e0 = e[j], e1 = e[j + 1];
      const float w0 = w[j], w1 = w[j + 1];
      const bool o0 = ok[j], o1 = ok[j + 1];
      const int32_t c0 = c[j], c1 = c[j + 1];
      e[j] = sw ? e1 : e0; e[j + 1] = sw ? e0 : e1;
      w[j] = sw ? w1 : w0; w[j + 1] = sw ? w0 : w1;
      ok[j] = sw ? o1 : o0; ok[j + 1] = sw ? o0 : o1;
      c[j] = sw ? c1 : c0; c[j + 1] = sw ? c0 : c1;
    }
  }
}

// A token's slot, weight and column maps.  They are the library's own,
// 256-byte aligned: 16-byte stores when K is a multiple of 4.
template <int K>
__device__ __forceinline__ void store_maps(const RouteArgs &a, int64_t t, const int32_t (&row)[K],
                                           const float (&wt)[K], const int32_t (&c)[K]) {
  if (K % 4 == 0) {
#pragma unroll
    for (int v = 0; v < K / 4; ++v) {
      reinterpret_cast<int4 *>(a.slot + t * K)[v] =
          make_int4(row[4 * v], row[4 * v + 1], row[4 * v + 2], row[4 * v + 3]);
      reinterpret_cast<float4 *>(a.weight + t * K)[v] =
          make_float4(wt[4 * v], wt[4 * v + 1], wt[4 * v + 2], wt[4 * v + 3]);
      reinterpret_cast<int4 *>(a.col + t * K)[v] = make_int4(c[4 * v], c[4 * v + 1], c[4 * v + 2], c[4 * v + 3]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < K; ++j) {
      a.slot[t * K + j] = row[j];
      a.weight[t * K + j] = wt[j];
      a.col[t * K + j] = c[j];
    }
  }
}

template <int K>
__global__ void __launch_bounds__(kRouteBlock) moe_route_slot_kernel(RouteArgs a) {
  constexpr int W = kRouteBlock / 32;
  __shared__ uint32_t mask[kRouteMaxExperts * W];
  __shared__ uint16_t mpre[kRouteMaxExperts * W];  // tokens in the expert's earlier mask words
  __shared__ int32_t eoff[kRouteMaxExperts];       // exclusive offsets over experts
  __shared__ int32_t part[kRouteBlock / 64];
  for (int i = threadIdx.x; i < a.E * W; i += blockDim.x) mask[i] = 0;
  for (int x = threadIdx.x; x < a.E; x += blockDim.x) eoff[x] = a.counts[x];
  __syncthreads();
  const int32_t total = lds_exclusive_scan(eoff, a.E, part);
  if (blockIdx.x == 0) {
    for (int x = threadIdx.x; x < a.E; x += blockDim.x) a.expert_off[x] = eoff[x];
    if (static_cast<int>(threadIdx.x) <= a.R) {
      const int32_t v = static_cast<int>(threadIdx.x) < a.R ? eoff[threadIdx.x * a.per] : total;
      a.rank_off[threadIdx.x] = v;
      if (a.user_rank_off) a.user_rank_off[threadIdx.x] = v;
    }
  }
  const int local = threadIdx.x;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kRouteBlock + local;
  int32_t e[K];
  float w[K];
  bool ok[K];
  const bool live = t < a.T;
  load_topk<K>(a, t, live, e, w);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    ok[j] = live && e[j] >= 0 && e[j] < a.E;
#pragma unroll
    for (int j2 = 0; j2 < j; ++j2) ok[j] = ok[j] && e[j2] != e[j];
    if (ok[j]) atomicOr(&mask[e[j] * W + (local >> 5)], 1u << (local & 31));
  }
  __syncthreads();
  for (int x = local; x < a.E; x += blockDim.x) {
    int pre = 0;
#pragma unroll
    for (int q = 0; q < W; ++q) {
      mpre[x * W + q] = static_cast<uint16_t>(pre);
      pre += __popc(mask[x * W + q]);
    }
  }
  __syncthreads();
  if (!live) return;
  // Ascending expert id.
  int32_t c[K];
  sort_by_expert<K>(e, w, ok, c);
  int32_t row[K];
  float wt[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    row[j] = 0;
    wt[j] = 0.f;
    if (ok[j]) {
      const int q = local >> 5;
      const int pos = mpre[e[j] * W + q] + __popc(mask[e[j] * W + q] & ((1u << (local & 31)) - 1u));
      row[j] = eoff[e[j]] + a.bbase[static_cast<int64_t>(blockIdx.x) * a.E + e[j]] + pos;
      wt[j] = w[j];
    }
  }
  store_maps<K>(a, t, row, wt, c);
}

// Fused routing: one block of kRouteBlock tokens per workgroup, all blocks
// co-resident.  Phase 1 validates, counts (LDS histogram) and marks (LDS
// token masks) this block's tokens and publishes the counts; after a grid
// barrier, each block sums the counts of earlier blocks and of all blocks per
// expert itself, scans the totals over experts, and assigns its slots.  Block
// 0 also writes the expert counts, offsets, rank offsets and the status word.
// The barrier counter only grows: the blocks of one call take arrival numbers
// g * nblk .. g * nblk + nblk - 1, so each waits for (g + 1) * nblk.
template <int K>
__global__ void __launch_bounds__(kRouteBlock) moe_route_fused_kernel(RouteArgs a) {
  constexpr int W = kRouteBlock / 32;
  __shared__ uint32_t mask[kRouteMaxExperts * W];
  __shared__ uint16_t mpre[kRouteMaxExperts * W];  // tokens in the expert's earlier mask words
  __shared__ int32_t hist[kRouteMaxExperts];   // counts, then earlier-block prefix
  __shared__ int32_t eoff[kRouteMaxExperts];   // exclusive offsets over experts
  __shared__ int32_t part[kRouteBlock / 64];
  __shared__ int32_t bad;
  __shared__ int ok_all;
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  for (int i = tid; i < a.E * W; i += kRouteBlock) mask[i] = 0;
  for (int e = tid; e < a.E; e += kRouteBlock) hist[e] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();

  // Phase 1: this block's tokens.
  const int64_t t = static_cast<int64_t>(blk) * kRouteBlock + tid;
  const bool live = t < a.T;
  int32_t e[K];
  float w[K];
  bool ok[K];
  int32_t mybad = 0;
  load_topk<K>(a, t, live, e, w);
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const bool in_range = e[j] >= 0 && e[j] < a.E;
    bool dup = false;
#pragma unroll
    for (int j2 = 0; j2 < j; ++j2) dup = dup || e[j2] == e[j];
    if (live && !in_range) mybad |= 1;
    if (live && in_range && dup) mybad |= 2;
    ok[j] = live && in_range && !dup;
    if (ok[j]) {
      atomicAdd(&hist[e[j]], 1);
      atomicOr(&mask[e[j] * W + (tid >> 5)], 1u << (tid & 31));
    }
  }
  if (mybad) atomicOr(&bad, mybad);
  __syncthreads();
  // The counts other blocks read are stored with the agent-scope atomic
  // store policy (written through this XCD's L2).
  for (int x = tid; x < a.E; x += kRouteBlock)
    __hip_atomic_store(a.bcounts + static_cast<int64_t>(blk) * a.E + x, hist[x], __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  // This block's error bits, read by block 0 after the barrier: written
  // through like the counts.
  if (tid == 0)
    __hip_atomic_store(a.bstatus + blk, bad, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // Grid barrier without fences: every wave waits until its stores have
  // completed, thread 0 arrives and waits, and the counts are then read with
  // device-coherent (agent-scope atomic) loads.  The agent-scope release and
  // acquire fences this replaces write back and invalidate the whole L2 of
  // the XCD in every wave (kernel trace median 11.9 -> 11.3 us, 4096 tokens,
  // 256 experts, top-8, MI355X).
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (tid == 0) {
    const unsigned long long g =
        __hip_atomic_fetch_add(a.sync, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) /
        static_cast<unsigned long long>(a.nblk);
    const unsigned long long want = (g + 1) * static_cast<unsigned long long>(a.nblk);
    uint32_t spins = 0;
    int fine = 1;
    while (__hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
      if (++spins >= a.spin) {
        // This block writes no slots: say so where no later write can undo
        // it (its own status word; the check reads them all).
        __hip_atomic_store(a.bstatus + blk, bad | 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        atomicOr(a.status, 4);
        fine = 0;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    ok_all = fine;
  }
  __syncthreads();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (!ok_all) return;

  // Phase 2: per expert, the prefix counts of its mask words (so a slot
  // needs two LDS reads), the sum over earlier blocks and the total; eight
  // independent coherent loads in flight per step.
  for (int x = tid; x < a.E; x += kRouteBlock) {
    int pre = 0;
#pragma unroll
    for (int q = 0; q < W; ++q) {
      mpre[x * W + q] = static_cast<uint16_t>(pre);
      pre += __popc(mask[x * W + q]);
    }
  }
  for (int x = tid; x < a.E; x += kRouteBlock) {
    int32_t run = 0, tot = 0;
    for (int b0 = 0; b0 < a.nblk; b0 += 8) {
      int32_t c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        c[u] = b0 + u < a.nblk ? __hip_atomic_load(a.bcounts + static_cast<int64_t>(b0 + u) * a.E + x,
                                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                               : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (b0 + u < blk) run += c[u];
        tot += c[u];
      }
    }
    hist[x] = run;
    eoff[x] = tot;
  }
  __syncthreads();
  // Exclusive scan of the totals over experts (the shuffle scan went from
  // about 2.9 to 0.6 us of the kernel against a doubling scan, 256 experts).
  if (blk == 0)
    for (int x = tid; x < a.E; x += kRouteBlock) a.counts[x] = eoff[x];
  const int32_t total = lds_exclusive_scan(eoff, a.E, part);
  if (blk == 0)
    for (int x = tid; x < a.E; x += kRouteBlock) a.expert_off[x] = eoff[x];
  for (int x = tid; x < a.E; x += kRouteBlock) a.bbase[static_cast<int64_t>(blk) * a.E + x] = hist[x];
  if (blk == 0) {
    if (tid <= a.R) {
      const int32_t v = tid < a.R ? eoff[tid * a.per] : total;
      a.rank_off[tid] = v;
      if (a.user_rank_off) a.user_rank_off[tid] = v;
    }
    // Every block's error bits, read in parallel and combined in LDS.
    int32_t st = 0;
    for (int b = tid; b < a.nblk; b += kRouteBlock)
      st |= __hip_atomic_load(a.bstatus + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) bad = 0;
    __syncthreads();
    if (st) atomicOr(&bad, st);
    __syncthreads();
    if (tid == 0) *a.status = bad;
  }

  // Phase 3: this block's slots, experts in ascending id.
  if (!live) return;
  int32_t c[K];
  sort_by_expert<K>(e, w, ok, c);
  int32_t row[K];
  float wt[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    row[j] = 0;
    wt[j] = 0.f;
    if (ok[j]) {
      const int q = tid >> 5;
      const int pos = mpre[e[j] * W + q] + __popc(mask[e[j] * W + q] & ((1u << (tid & 31)) - 1u));
      row[j] = eoff[e[j]] + hist[e[j]] + pos;
      wt[j] = w[j];
    }
  }
  store_maps<K>(a, t, row, wt, c);
}

namespace {

using RouteFn = void (*)(RouteArgs);

RouteFn route_fused_for(int k) {
  switch (k) {
#define RRB_CASE(n) \
  case n:           \
    return moe_route_fused_kernel<n>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8) RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13)
    RRB_CASE(14) RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
  }
  return nullptr;
}

RouteFn route_count_for(int k) {
  switch (k) {
#define RRB_CASE(n) \
  case n:           \
    return moe_route_count_kernel<n>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8) RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13)
    RRB_CASE(14) RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
  }
  return nullptr;
}

RouteFn route_slot_for(int k) {
  switch (k) {
#define RRB_CASE(n) \
  case n:           \
    return moe_route_slot_kernel<n>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8) RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13)
    RRB_CASE(14) RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
  }
  return nullptr;
}

rrb_status route_launch_check(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RRB_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  return RRB_OK;
}

}  // namespace

rrb_status clear_route_maps(const Plan &p, void *stream) {
  const RowMaps &m = p.rows;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(p.d_ws);
  const int64_t n = m.tokens * m.topk;
  if (n > 0) {
    // Slots and columns: row 0 of the arena and column 0, both in bounds.
    hipLaunchKernelGGL(moe_fill_kernel, dim3(64), dim3(256), 0, s,
                       reinterpret_cast<int32_t *>(ws + m.off_slot), n, 0);
    hipLaunchKernelGGL(moe_fill_kernel, dim3(64), dim3(256), 0, s,
                       reinterpret_cast<int32_t *>(ws + m.off_col), n, 0);
  }
  // status word, barrier counter and per-block status words
  const int64_t words = (static_cast<int64_t>(m.off_bstatus - m.off_status) + m.nblk * 4) / 4;
  hipLaunchKernelGGL(moe_fill_kernel, dim3(1), dim3(256), 0, s,
                     reinterpret_cast<int32_t *>(ws + m.off_status), words, 0);
  return route_launch_check("route clear");
}

rrb_status launch_route(Plan &p, const int32_t *d_idx, const float *d_w, int32_t *d_rank_offsets,
                        void *stream) {
  const RowMaps &m = p.rows;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(p.d_ws);
  RouteArgs a;
  std::memset(&a, 0, sizeof a);
  a.idx = d_idx;
  a.w = d_w;
  a.slot = reinterpret_cast<int32_t *>(ws + m.off_slot);
  a.weight = reinterpret_cast<float *>(ws + m.off_weight);
  a.col = reinterpret_cast<int32_t *>(ws + m.off_col);
  a.counts = reinterpret_cast<int32_t *>(ws + m.off_counts);
  a.expert_off = reinterpret_cast<int32_t *>(ws + m.off_expert);
  a.rank_off = reinterpret_cast<int32_t *>(ws + m.off_rank);
  a.bcounts = reinterpret_cast<int32_t *>(ws + m.off_bcounts);
  a.bbase = reinterpret_cast<int32_t *>(ws + m.off_bbase);
  a.status = reinterpret_cast<int32_t *>(ws + m.off_status);
  a.bstatus = reinterpret_cast<int32_t *>(ws + m.off_bstatus);
  a.sync = reinterpret_cast<unsigned long long *>(ws + m.off_status + 128);
  a.spin = 1u << 22;
  a.user_rank_off = d_rank_offsets;
  a.T = m.tokens;
  a.E = m.experts;
  a.k = m.topk;
  a.R = p.nranks;
  a.per = m.experts / p.nranks;
  a.nblk = static_cast<int32_t>(m.nblk);
  // One fused kernel when every token block can be resident at once (half
  // the device's co-resident capacity, as a margin); its grid barrier waits
  // are bounded, so a grid that other work keeps apart times out (status
  // bit 4) instead of hanging.  Otherwise three kernels.
  if (m.tokens > 0) {
    RouteFn fused = route_fused_for(m.topk);
    if (m.route_cap == 0) {
      int dev = 0, cus = 0, perb = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e == hipSuccess)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&perb, reinterpret_cast<const void *>(fused),
                                                         kRouteBlock, 0);
      if (e != hipSuccess) return fail(RRB_EHIP, "route occupancy query: %s", hipGetErrorString(e));
      p.rows.route_cap = static_cast<int64_t>(perb) * cus;
    }
    if (2 * m.nblk <= p.rows.route_cap) {
      hipLaunchKernelGGL(fused, dim3(static_cast<unsigned>(m.nblk)), dim3(kRouteBlock), 0, s, a);
      return route_launch_check("route");
    }
  }
  hipLaunchKernelGGL(moe_fill_kernel, dim3(1), dim3(64), 0, s, a.status, static_cast<int64_t>(1), 0);
  rrb_status st = route_launch_check("route status clear");
  if (st != RRB_OK) return st;
  if (m.tokens > 0) {
    hipLaunchKernelGGL(route_count_for(m.topk), dim3(static_cast<unsigned>(m.nblk)), dim3(kRouteBlock),
                       0, s, a);
    if ((st = route_launch_check("route count")) != RRB_OK) return st;
  }
  hipLaunchKernelGGL(moe_route_scan_kernel, dim3(static_cast<unsigned>(m.experts)), dim3(kRouteBlock), 0, s, a);
  if ((st = route_launch_check("route scan")) != RRB_OK) return st;
  // With no tokens, one slot block still stores the (zero) expert and rank
  // offsets.
  hipLaunchKernelGGL(route_slot_for(m.topk), dim3(static_cast<unsigned>(m.nblk > 0 ? m.nblk : 1)),
                     dim3(kRouteBlock), 0, s, a);
  return route_launch_check("route slot");
}

namespace {

using RowFn = void (*)(RowArgs);

// Dispatch kernel for top-k up to 16 (nullptr above: the any-k kernel).
RowFn dispatch_for(int k) {
  switch (k) {
#define RRB_CASE(n) \
  case n:           \
    return moe_dispatch_kernel<n>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8) RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13)
    RRB_CASE(14) RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
    default: return nullptr;
  }
}

// Combine kernel for top-k up to 16 and its vectors per lane: CU = ceil(8 /
// k), so k * CU >= 8 loads are in flight per lane.
RowFn combine_for(int k, int *cu) {
  switch (k) {
#define RRB_CASE(n)                       \
  case n:                                 \
    *cu = (8 + (n) - 1) / (n);            \
    return moe_combine_kernel<n, (8 + (n) - 1) / (n)>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8) RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13)
    RRB_CASE(14) RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
    default: *cu = 0; return nullptr;
  }
}

// Row parts: the fewest parts of at most `cap` vectors, all of equal size
// (the last may be shorter).
void split_row(RowArgs &a, int64_t cap) {
  a.parts = static_cast<int32_t>((a.nvec + cap - 1) / cap);
  if (a.parts < 1) a.parts = 1;
  a.part_vec = (a.nvec + a.parts - 1) / a.parts;
}

}  // namespace

rrb_status launch_rows(const Plan &p, const void *const *in, void *const *out, const float *d_weights,
                       void *stream) {
  const RowMaps &m = p.rows;
  if (m.tokens == 0) return RRB_OK;
  if (!p.d_ws) return fail(RRB_EINVAL, "row plan is not bound to a workspace");
  RowArgs a;
  std::memset(&a, 0, sizeof a);
  bool vec = (m.hidden * 2) % 16 == 0;
  for (int32_t r = 0; r < p.nranks; ++r) {
    a.in[r] = static_cast<const unsigned char *>(in[r]);
    a.out[r] = static_cast<unsigned char *>(out[r]);
    if ((p.in_count[r] && (reinterpret_cast<uintptr_t>(in[r]) & 15)) ||
        (p.out_count[r] && (reinterpret_cast<uintptr_t>(out[r]) & 15)))
      vec = false;
  }
  // Device-routed plans: slots are arena rows (rank bits 0), the arena is
  // pointer 0.
  const char *ws = static_cast<const char *>(p.d_ws);
  a.slot = reinterpret_cast<const int32_t *>(ws + m.off_slot);
  a.weight = reinterpret_cast<const float *>(ws + m.off_weight);
  a.col = reinterpret_cast<const int32_t *>(ws + m.off_col);
  a.wover = m.dir == RRB_MOE_COMBINE ? d_weights : nullptr;
  if (p.kind == PlanKind::RowsDevice) a.route_status = reinterpret_cast<const int32_t *>(ws + m.off_status);
  a.tokens_per_rank = m.tokens / p.nranks;
  a.row_bytes = m.hidden * 2;
  a.nvec = a.row_bytes / 16;
  a.hidden = m.hidden;
  a.k = m.topk;
  RowFn kern = nullptr;
  int bs = 256;
  a.parts = 1;
  a.part_vec = a.nvec;
  if (m.dir == RRB_MOE_DISPATCH) {
    if (vec) {
      kern = dispatch_for(m.topk);
      if (!kern) kern = moe_dispatch_any_kernel;
      split_row(a, 256);
    } else {
      kern = moe_dispatch_elem_kernel;
    }
  } else {
    int cu = 0;
    if (vec) {
      kern = combine_for(m.topk, &cu);
      if (!kern) {
        kern = moe_combine_any_kernel;
        cu = 1;
      }
      bs = 128;
      split_row(a, 128LL * cu);
    } else {
      kern = moe_combine_elem_kernel;
    }
  }
  if (m.tokens * a.parts > 0x7fffffffLL) return fail(RRB_EUNSUPPORTED, "too many tokens for one launch");
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(m.tokens * a.parts)), dim3(bs), 0,
                     static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RRB_EHIP, "moe launch: %s", hipGetErrorString(e));
  return RRB_OK;
}

}  // namespace rrb
