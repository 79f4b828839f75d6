// Atom: the copy and reduce datapath on gfx950 (MI355X).
//
// Purlin: Separating Orchestration from the Datapath of Collectives ("The
// Purlin PDF describes a three-layer design"): below the orchestration sits a
// hardware-specific datapath with two primitives, copy and reduce.  On one
// MI355X both are HBM-streaming kernels: every source byte is read once with
// 128-bit loads, the reduce accumulates in fp32 registers in rank order
// 0..R-1 and rounds once to bf16 (round-to-nearest-even), and a fan-out
// segment writes its result to every destination rank from registers.  There
// is no contraction here, so no MFMA and no LDS: the work is bounded by HBM
// bandwidth (large payloads) or by launch and memory latency (decode sizes).
//
// A plan's segments ride in the kernel arguments (at most kMaxItems per
// launch), so a decode-size All-Reduce issues its loads without first
// fetching a table from memory.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <string>

#include "rrb_internal.h"
#include "rrb_kernels.h"

namespace rrb {

constexpr int kMaxItems = 64;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// 16-byte load / store with an optional non-temporal hint.  Streams larger
// than the caches use it: measured on MI355X, non-temporal stores lift a 1->8
// fan-out from 5.2 to 6.7 TB/s, and non-temporal loads help the 8-source
// reduce; both hurt when the data would otherwise be served from the
// Infinity Cache.
template <bool NT>
__device__ __forceinline__ uint4 ld16(const unsigned char *p) {
  if (NT) {
    const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u *>(p));
    return make_uint4(x[0], x[1], x[2], x[3]);
  }
  return *reinterpret_cast<const uint4 *>(p);
}
template <bool NT>
__device__ __forceinline__ void st16(unsigned char *p, uint4 v) {
  if (NT) {
    v4u x = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(x, reinterpret_cast<v4u *>(p));
  } else {
    *reinterpret_cast<uint4 *>(p) = v;
  }
}

struct KItem {
  int64_t src_off;  // bytes
  int64_t dst_off;  // bytes
  int32_t src_rank; // copy: source rank; reduce: unused (all ranks)
  uint32_t dst_mask;
};

struct UniArgs {
  const unsigned char *in[RRB_MAX_RANKS];
  unsigned char *out[RRB_MAX_RANKS];
  KItem items[kMaxItems];
  int64_t nvec;   // whole 16-byte vectors per item (vector path)
  int64_t tail;   // elements per item after those vectors (vector path)
  int64_t nelem;  // elements per item (element path)
  int32_t tiles;  // workgroups per item
  int32_t nranks;
  int32_t xcd_chunk;  // 0, or C: XCD-chunked tile order (tiles % (8 * C) == 0)
  int32_t fan;        // copy_split_kernel: workgroups per tile (largest fan-out)
};

// Workgroups are dealt to the 8 XCDs round-robin in blockIdx order.  With a
// chunk C, XCD x takes runs of C consecutive tiles in turn, so each XCD
// streams contiguous stretches of every buffer (a bijection on the item's
// tiles when tiles % (8 * C) == 0).
__device__ __forceinline__ int xcd_tile(int local, int C) {
  if (C == 0) return local;
  const int x = local & 7, k = local >> 3;
  return (k / C) * (8 * C) + x * C + (k % C);
}

// 16-byte store at byte `off` of the `span`-byte region at `base` with the
// cache policy of agent-scope atomic stores (sc1, through a buffer store):
// written through rather than left dirty in this XCD's L2.  `base` is the
// workgroup's tile, so offsets fit 32 bits for any buffer size.
__device__ __forceinline__ void st16_wt_at(unsigned char *base, int32_t span, int32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      v4u{v.x, v.y, v.z, v.w},
      __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), span, 0x00020000), off, 0, 16);
}

// Store v at byte offset off of every output whose bit is set in mask.  The
// loop runs over compile-time rank indices, so the output pointers come from
// one batch of scalar loads instead of a dependent load per set bit: that
// lifts the streaming 1->8 copy from 6.2 to 6.8 TB/s on MI355X (together with
// plain tile order).  The reduce keeps its bit loop, 3% faster there.
template <bool NTS>
__device__ __forceinline__ void st16_fan(unsigned char *const *out, uint32_t mask, int64_t off,
                                         uint4 v) {
#pragma unroll
  for (int q = 0; q < RRB_MAX_RANKS; ++q)
    if (mask >> q & 1u) st16<NTS>(out[q] + off, v);
}

// ---- kernels ---------------------------------------------------------------

// Body of the vector reduce; TREE selects the tree-order fold.
template <int R, int U, bool BF16, bool NTL, bool NTS, bool TREE, bool WT = false>
__device__ __forceinline__ void reduce_vec_body(const UniArgs &a) {
  const int bs = blockDim.x;
  const int item = blockIdx.x / a.tiles;
  const int tile = xcd_tile(blockIdx.x - item * a.tiles, a.xcd_chunk);
  const KItem it = a.items[item];
  const int64_t base = static_cast<int64_t>(tile) * bs * U + threadIdx.x;

  uint4 v[U][R];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * bs;
    if (i < a.nvec) {
#pragma unroll
      for (int r = 0; r < R; ++r)
        v[u][r] = ld16<NTL>(a.in[r] + it.src_off + i * 16);
    }
  }
  // Fold every vector first, then store output by output, each output's U
  // vectors back to back (measured on MI355X level with, or up to 1% ahead
  // of, interleaving the outputs vector by vector).
  uint4 res[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * bs;
    if (i < a.nvec) res[u] = fold_vec<R, BF16, TREE>(v[u]);
  }
  for (uint32_t m = it.dst_mask; m; m &= m - 1) {
    const int q = __builtin_ctz(m);
    unsigned char *tb = a.out[q] + it.dst_off + (base - threadIdx.x) * 16;  // this tile
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * bs;
      if (i < a.nvec) {
        if (WT)
          st16_wt_at(tb, bs * U * 16, static_cast<int32_t>((threadIdx.x + u * bs) * 16), res[u]);
        else
          st16<NTS>(a.out[q] + it.dst_off + i * 16, res[u]);
      }
    }
  }
  // Elements after the last whole vector of the item (single-segment plans
  // whose length is not a multiple of the vector width).
  if (a.tail && tile == a.tiles - 1 && threadIdx.x < a.tail) {
    const int64_t e = a.nvec * (BF16 ? 8 : 4) + threadIdx.x;
    const int esz = BF16 ? 2 : 4;
    float t[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      t[r] = BF16 ? bf16_to_f32(*reinterpret_cast<const uint16_t *>(a.in[r] + it.src_off + e * esz))
                  : *reinterpret_cast<const float *>(a.in[r] + it.src_off + e * esz);
    float acc;
    if (TREE) {
      acc = tree_sum<R>(t);
    } else {
      acc = t[0];
#pragma unroll
      for (int r = 1; r < R; ++r) acc = acc + t[r];
    }
    if (BF16) {
      const uint16_t b = f32_to_bf16_rne(acc);
      for (uint32_t m = it.dst_mask; m; m &= m - 1) {
        const int q = __builtin_ctz(m);
        *reinterpret_cast<uint16_t *>(a.out[q] + it.dst_off + e * esz) = b;
      }
    } else {
      for (uint32_t m = it.dst_mask; m; m &= m - 1) {
        const int q = __builtin_ctz(m);
        *reinterpret_cast<float *>(a.out[q] + it.dst_off + e * esz) = acc;
      }
    }
  }
}

template <int R, int U, bool BF16, bool NTL, bool NTS>
__global__ void __launch_bounds__(256) reduce_vec_kernel(UniArgs a) {
  reduce_vec_body<R, U, BF16, NTL, NTS, false>(a);
}

// Streaming single-destination reduce (Reduce-Scatter, Reduce to a root):
// non-temporal loads, write-through stores.  Measured on the sweep step on
// MI355X against plain stores: Reduce-Scatter 16 MiB 28.8 -> 27.4 us,
// 64 MiB 109.3 -> 103.6 us, 256 MiB 416 -> 410 us (4 MiB 10.0 -> 10.3), and
// the All-Gather that reads its output next kept its cache hits.
template <int R, int U, bool BF16>
__global__ void __launch_bounds__(256) reduce_wt_kernel(UniArgs a) {
  reduce_vec_body<R, U, BF16, true, false, false, true>(a);
}

// Tree-order reduce (opt-in op RRB_REDUCE_SUM_TREE), one vector per lane.
template <int R, bool BF16, bool NTL, bool NTS>
__global__ void __launch_bounds__(256) reduce_tree_vec_kernel(UniArgs a) {
  reduce_vec_body<R, 1, BF16, NTL, NTS, true>(a);
}

// Element-at-a-time reduce for buffers or offsets that are not 16-byte
// aligned: correct for any layout, not tuned.
template <bool BF16, bool TREE>
__device__ __forceinline__ void reduce_elem_body(const UniArgs &a) {
  const int item = blockIdx.x / a.tiles;
  const int tile = blockIdx.x - item * a.tiles;
  const KItem it = a.items[item];
  const int64_t e = static_cast<int64_t>(tile) * blockDim.x + threadIdx.x;
  if (e >= a.nelem) return;
  if (TREE) {
    float t[RRB_MAX_RANKS];
#pragma unroll
    for (int r = 0; r < RRB_MAX_RANKS; ++r)
      t[r] = r >= a.nranks ? 0.f
             : BF16 ? bf16_to_f32(*reinterpret_cast<const uint16_t *>(a.in[r] + it.src_off + e * 2))
                    : *reinterpret_cast<const float *>(a.in[r] + it.src_off + e * 4);
    const float acc = tree_sum_n<RRB_MAX_RANKS>(t, a.nranks);
    if (BF16) {
      const uint16_t b = f32_to_bf16_rne(acc);
      for (uint32_t m = it.dst_mask; m; m &= m - 1)
        *reinterpret_cast<uint16_t *>(a.out[__builtin_ctz(m)] + it.dst_off + e * 2) = b;
    } else {
      for (uint32_t m = it.dst_mask; m; m &= m - 1)
        *reinterpret_cast<float *>(a.out[__builtin_ctz(m)] + it.dst_off + e * 4) = acc;
    }
    return;
  }
  if (BF16) {
    float acc = bf16_to_f32(*reinterpret_cast<const uint16_t *>(a.in[0] + it.src_off + e * 2));
    for (int r = 1; r < a.nranks; ++r)
      acc = acc + bf16_to_f32(*reinterpret_cast<const uint16_t *>(a.in[r] + it.src_off + e * 2));
    const uint16_t b = f32_to_bf16_rne(acc);
    for (uint32_t m = it.dst_mask; m; m &= m - 1)
      *reinterpret_cast<uint16_t *>(a.out[__builtin_ctz(m)] + it.dst_off + e * 2) = b;
  } else {
    float acc = *reinterpret_cast<const float *>(a.in[0] + it.src_off + e * 4);
    for (int r = 1; r < a.nranks; ++r)
      acc = acc + *reinterpret_cast<const float *>(a.in[r] + it.src_off + e * 4);
    for (uint32_t m = it.dst_mask; m; m &= m - 1)
      *reinterpret_cast<float *>(a.out[__builtin_ctz(m)] + it.dst_off + e * 4) = acc;
  }
}

template <bool BF16>
__global__ void __launch_bounds__(256) reduce_elem_kernel(UniArgs a) {
  reduce_elem_body<BF16, false>(a);
}

template <bool BF16>
__global__ void __launch_bounds__(256) reduce_tree_elem_kernel(UniArgs a) {
  reduce_elem_body<BF16, true>(a);
}

template <int U, bool NTS>
__global__ void __launch_bounds__(256) copy_vec_kernel(UniArgs a) {
  const int bs = blockDim.x;
  const int item = blockIdx.x / a.tiles;
  const int tile = xcd_tile(blockIdx.x - item * a.tiles, a.xcd_chunk);
  const KItem it = a.items[item];
  const unsigned char *src = a.in[it.src_rank] + it.src_off;
  const int64_t base = static_cast<int64_t>(tile) * bs * U + threadIdx.x;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * bs;
    if (i < a.nvec) v[u] = *reinterpret_cast<const uint4 *>(src + i * 16);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * bs;
    if (i < a.nvec) st16_fan<NTS>(a.out, it.dst_mask, it.dst_off + i * 16, v[u]);
  }
  // Tail in 2-byte units (every element type is a multiple of 2 bytes).
  if (a.tail && tile == a.tiles - 1 && threadIdx.x < a.tail) {
    const int64_t off = a.nvec * 16 + static_cast<int64_t>(threadIdx.x) * 2;
    const uint16_t x = *reinterpret_cast<const uint16_t *>(src + off);
    for (uint32_t m = it.dst_mask; m; m &= m - 1)
      *reinterpret_cast<uint16_t *>(a.out[__builtin_ctz(m)] + it.dst_off + off) = x;
  }
}

// Copy with write-through stores for launches that do not stream past the
// caches (except small fan-out copies): the outputs are written through
// rather than left dirty in L2.  Measured on MI355X against plain stores:
// 4 MiB All-Gather 10.7 -> 9.4 us in the sweep step; 8 x 16 KiB All-to-All
// and Gather graph chains 1.89 -> 1.81 and 1.85 -> 1.81 us per launch.
template <int U>
__global__ void __launch_bounds__(256) copy_wt_kernel(UniArgs a) {
  const int bs = blockDim.x;
  const int item = blockIdx.x / a.tiles;
  const int tile = blockIdx.x - item * a.tiles;
  const KItem it = a.items[item];
  const unsigned char *src = a.in[it.src_rank] + it.src_off;
  const int64_t base = static_cast<int64_t>(tile) * bs * U + threadIdx.x;
  uint4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = base + static_cast<int64_t>(u) * bs;
    if (i < a.nvec) v[u] = *reinterpret_cast<const uint4 *>(src + i * 16);
  }
  const int64_t tile_off = it.dst_off + (base - threadIdx.x) * 16;
#pragma unroll
  for (int q = 0; q < RRB_MAX_RANKS; ++q) {
    if (it.dst_mask >> q & 1u) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i = base + static_cast<int64_t>(u) * bs;
        if (i < a.nvec)
          st16_wt_at(a.out[q] + tile_off, bs * U * 16, static_cast<int32_t>((threadIdx.x + u * bs) * 16),
                     v[u]);
      }
    }
  }
  if (a.tail && tile == a.tiles - 1 && threadIdx.x < a.tail) {
    const int64_t off = a.nvec * 16 + static_cast<int64_t>(threadIdx.x) * 2;
    const uint16_t x = *reinterpret_cast<const uint16_t *>(src + off);
    for (uint32_t m = it.dst_mask; m; m &= m - 1)
      *reinterpret_cast<uint16_t *>(a.out[__builtin_ctz(m)] + it.dst_off + off) = x;
  }
}

// Small fan-out copies: one workgroup per (item, destination, tile), each
// reading its tile and writing it to one destination, so a fan-out's stores
// spread over `fan` times more workgroups.  Graph-replayed All-Gather, 8
// ranks, MI355X: 8 x 256 B 2.69 -> 2.21 us per launch, 8 x 2 KiB 2.81 ->
// 2.31, 8 x 16 KiB 2.87 -> 2.41; at 8 x 64 KiB it lost (3.30 -> 3.50), so
// blocks above 1024 vectors keep one workgroup per tile.
__global__ void __launch_bounds__(256) copy_split_kernel(UniArgs a) {
  const int bs = blockDim.x;
  const int per_item = a.tiles * a.fan;
  const int item = blockIdx.x / per_item;
  const int rem = blockIdx.x - item * per_item;
  const int d = rem / a.tiles;
  const int tile = rem - d * a.tiles;
  const KItem it = a.items[item];
  uint32_t m = it.dst_mask;
  for (int j = 0; j < d && m; ++j) m &= m - 1;
  if (!m) return;  // this item fans out to fewer destinations
  unsigned char *dst = a.out[__builtin_ctz(m)] + it.dst_off;
  const unsigned char *src = a.in[it.src_rank] + it.src_off;
  const int64_t i = static_cast<int64_t>(tile) * bs + threadIdx.x;
  if (i < a.nvec) *reinterpret_cast<uint4 *>(dst + i * 16) = *reinterpret_cast<const uint4 *>(src + i * 16);
  if (a.tail && tile == a.tiles - 1 && threadIdx.x < a.tail) {
    const int64_t off = a.nvec * 16 + static_cast<int64_t>(threadIdx.x) * 2;
    *reinterpret_cast<uint16_t *>(dst + off) = *reinterpret_cast<const uint16_t *>(src + off);
  }
}

// 2-byte-unit copy for unaligned layouts.
__global__ void __launch_bounds__(256) copy_elem_kernel(UniArgs a) {
  const int item = blockIdx.x / a.tiles;
  const int tile = blockIdx.x - item * a.tiles;
  const KItem it = a.items[item];
  const int64_t e = static_cast<int64_t>(tile) * blockDim.x + threadIdx.x;
  if (e >= a.nelem) return;
  const uint16_t x = *reinterpret_cast<const uint16_t *>(a.in[it.src_rank] + it.src_off + e * 2);
  for (uint32_t m = it.dst_mask; m; m &= m - 1)
    *reinterpret_cast<uint16_t *>(a.out[__builtin_ctz(m)] + it.dst_off + e * 2) = x;
}

// Decode-size single-segment launches (All-Reduce, Reduce, Broadcast of a few
// KiB per rank): the pointers arrive already offset and the destinations as
// a compact list, so the wave issues its loads without a table lookup or an
// integer division first (measured 2.5 us vs 3.5 us per 8 x 8 KiB All-Reduce
// on MI355X, against a 1.3 us empty kernel).
struct OneArgs {
  int32_t nvec;   // whole 16-byte vectors (>= 1)
  int32_t ndst;   // >= 1
  int32_t tail;   // elements (reduce) or 2-byte units (copy) after the vectors
  int32_t pad;
  const unsigned char *in[RRB_MAX_RANKS];  // reduce: rank r's source; copy: [0]
  unsigned char *out[RRB_MAX_RANKS];       // the ndst destinations
};

constexpr int kOneBlock = 64;

// 16-byte store at byte `off` of a `bytes`-long buffer with the cache policy
// of agent-scope atomic stores (sc1, through a buffer store): written through
// rather than left dirty in this XCD's L2, so less is left to write back when
// the kernel completes.  Measured on MI355X: the 8 x 8 KiB All-Reduce
// replayed from a HIP graph, 1.858 -> 1.793 us per launch (plain and
// non-temporal stores were level), against 1.65 us for an empty kernel.
__device__ __forceinline__ void st16_wt(unsigned char *base, int32_t bytes, int32_t off, uint4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(
      v4u{v.x, v.y, v.z, v.w},
      __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), bytes, 0x00020000), off, 0, 16);
}

// The lane index is clamped instead of branched on, and the first store is
// unconditional, so the compiler issues every source load as soon as the
// kernel arguments arrive (one scalar round trip instead of three).  Lanes
// past the end repeat the last vector's work and store the same bits.
// ALL: every rank is a destination (ndst == R), so the stores unroll with
// all destination pointers fetched up front.
template <int R, bool BF16, bool ALL, bool TREE>
__device__ __forceinline__ void reduce_one_body(const OneArgs &a) {
  const int i = min(static_cast<int>(blockIdx.x) * kOneBlock + static_cast<int>(threadIdx.x),
                    a.nvec - 1);
  uint4 v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = *reinterpret_cast<const uint4 *>(a.in[r] + static_cast<int64_t>(i) * 16);
  const uint4 res = fold_vec<R, BF16, TREE>(v);
  const int32_t vb = a.nvec * 16;  // at most kOneMaxVectors vectors
  if (ALL) {
#pragma unroll
    for (int q = 0; q < R; ++q) st16_wt(a.out[q], vb, i * 16, res);
  } else {
    st16_wt(a.out[0], vb, i * 16, res);
    for (int q = 1; q < a.ndst; ++q) st16_wt(a.out[q], vb, i * 16, res);
  }
  if (a.tail && blockIdx.x == gridDim.x - 1 && static_cast<int>(threadIdx.x) < a.tail) {
    const int64_t e = static_cast<int64_t>(a.nvec) * (BF16 ? 8 : 4) + threadIdx.x;
    float t[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
      t[r] = BF16 ? bf16_to_f32(*reinterpret_cast<const uint16_t *>(a.in[r] + e * 2))
                  : *reinterpret_cast<const float *>(a.in[r] + e * 4);
    float acc;
    if (TREE) {
      acc = tree_sum<R>(t);
    } else {
      acc = t[0];
#pragma unroll
      for (int r = 1; r < R; ++r) acc = acc + t[r];
    }
    if (BF16) {
      const uint16_t b = f32_to_bf16_rne(acc);
      for (int q = 0; q < a.ndst; ++q) *reinterpret_cast<uint16_t *>(a.out[q] + e * 2) = b;
    } else {
      for (int q = 0; q < a.ndst; ++q) *reinterpret_cast<float *>(a.out[q] + e * 4) = acc;
    }
  }
}

template <int R, bool BF16, bool ALL>
__global__ void __launch_bounds__(kOneBlock) reduce_one_kernel(OneArgs a) {
  reduce_one_body<R, BF16, ALL, false>(a);
}

template <int R, bool BF16, bool ALL>
__global__ void __launch_bounds__(kOneBlock) reduce_tree_one_kernel(OneArgs a) {
  reduce_one_body<R, BF16, ALL, true>(a);
}

__global__ void __launch_bounds__(kOneBlock) copy_one_kernel(OneArgs a) {
  const int i = min(static_cast<int>(blockIdx.x) * kOneBlock + static_cast<int>(threadIdx.x),
                    a.nvec - 1);
  const uint4 x = *reinterpret_cast<const uint4 *>(a.in[0] + static_cast<int64_t>(i) * 16);
  const int32_t vb = a.nvec * 16;
  st16_wt(a.out[0], vb, i * 16, x);
  for (int q = 1; q < a.ndst; ++q) st16_wt(a.out[q], vb, i * 16, x);
  if (a.tail && blockIdx.x == gridDim.x - 1 && static_cast<int>(threadIdx.x) < a.tail) {
    const int64_t off = static_cast<int64_t>(a.nvec) * 16 + threadIdx.x * 2;
    const uint16_t y = *reinterpret_cast<const uint16_t *>(a.in[0] + off);
    for (int q = 0; q < a.ndst; ++q) *reinterpret_cast<uint16_t *>(a.out[q] + off) = y;
  }
}

__global__ void empty_kernel() {}

// ---- launchers -------------------------------------------------------------

namespace {

using ReduceFn = void (*)(UniArgs);

template <bool BF16, bool NTL, bool NTS>
ReduceFn reduce_tree_vec_for(int R) {
  switch (R) {
#define RRB_CASE(n) \
  case n:           \
    return reduce_tree_vec_kernel<n, BF16, NTL, NTS>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8) RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13)
    RRB_CASE(14) RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
  }
  return nullptr;
}

// Several vectors per lane (U > 1) only for R <= 8, where the R x U loads
// still leave room for occupancy; more ranks keep one vector per lane.
template <int U, bool BF16>
ReduceFn reduce_wt_for(int R) {
  switch (R) {
#define RRB_CASE(n) \
  case n:           \
    return reduce_wt_kernel<n, U, BF16>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8)
#undef RRB_CASE
  }
  if constexpr (U == 1) {
    switch (R) {
#define RRB_CASE(n) \
  case n:           \
    return reduce_wt_kernel<n, 1, BF16>;
      RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13) RRB_CASE(14)
      RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
    }
  }
  return nullptr;
}

template <int U, bool BF16, bool NTL, bool NTS>
ReduceFn reduce_vec_for(int R) {
  switch (R) {
#define RRB_CASE(n) \
  case n:           \
    return reduce_vec_kernel<n, U, BF16, NTL, NTS>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8)
#undef RRB_CASE
  }
  if constexpr (U == 1) {
    switch (R) {
#define RRB_CASE(n) \
  case n:           \
    return reduce_vec_kernel<n, 1, BF16, NTL, NTS>;
      RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13) RRB_CASE(14)
      RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
    }
  }
  return nullptr;
}

// The vector reduce for U vectors per lane and the element type.
template <bool NTL, bool NTS>
ReduceFn reduce_vec_pick(int U, bool bf16, int R) {
  if (U == 4) return bf16 ? reduce_vec_for<4, true, NTL, NTS>(R) : reduce_vec_for<4, false, NTL, NTS>(R);
  if (U == 2) return bf16 ? reduce_vec_for<2, true, NTL, NTS>(R) : reduce_vec_for<2, false, NTL, NTS>(R);
  return bf16 ? reduce_vec_for<1, true, NTL, NTS>(R) : reduce_vec_for<1, false, NTL, NTS>(R);
}

ReduceFn reduce_wt_pick(int U, bool bf16, int R) {
  if (U == 4) return bf16 ? reduce_wt_for<4, true>(R) : reduce_wt_for<4, false>(R);
  if (U == 2) return bf16 ? reduce_wt_for<2, true>(R) : reduce_wt_for<2, false>(R);
  return bf16 ? reduce_wt_for<1, true>(R) : reduce_wt_for<1, false>(R);
}

// When a launch streams past the caches (non-temporal hints).  A reduce
// streams from 64 MiB of traffic (one read and one write per element per
// rank), measured on the bandwidth sweep on MI355X.  A copy streams when the
// bytes it writes reach half the 256 MB Infinity Cache: output that large
// would only evict other lines.  Measured on the sweep step (All-Reduce ->
// Reduce-Scatter -> All-Gather at 1..256 MiB per rank), interleaved A/B:
// 2.577 -> 2.515 ms per step against counting copies at 512 MiB of one
// read and one write per element (64 MiB All-Gather 112 -> 92 us); a
// 256 MiB threshold gave 2.553 ms.
constexpr int64_t kStreamBytesReduce = 64LL << 20;
constexpr int64_t kStreamOutCopy = 128LL << 20;
// Tiles per XCD run in the chunked order of streaming launches.
constexpr int kXcdChunk = 16;
// Vectors per launch from which a reduce lane handles more than one vector:
// four up to kHugeVectors, two from there on.  Measured on MI355X with
// interleaved A/B runs of library builds, 8 ranks: four per lane is 2-4%
// ahead of two at 32, 64 and 128 MiB per rank, and 1-3% behind at 256 MiB.
constexpr int64_t kBigVectors = 2LL << 20;
constexpr int64_t kHugeVectors = 16LL << 20;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

rrb_status check_launch(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RRB_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  return RRB_OK;
}

// Checks the caller's pointer arrays against the plan's per-rank counts.
rrb_status check_buffers(const Plan &p, const void *const *in, void *const *out) {
  if (!in || !out) return fail(RRB_EINVAL, "NULL pointer array");
  for (int32_t r = 0; r < p.nranks; ++r) {
    if (p.in_count[r] > 0 && !in[r]) return fail(RRB_EINVAL, "input of rank %d is NULL", r);
    if (p.out_count[r] > 0 && !out[r]) return fail(RRB_EINVAL, "output of rank %d is NULL", r);
  }
  return RRB_OK;
}

using OneFn = void (*)(OneArgs);

template <bool BF16, bool ALL, bool TREE>
OneFn reduce_one_for(int R) {
  switch (R) {
#define RRB_CASE(n) \
  case n:           \
    if constexpr (TREE) return reduce_tree_one_kernel<n, BF16, ALL>; \
    else return reduce_one_kernel<n, BF16, ALL>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8) RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13)
    RRB_CASE(14) RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
  }
  return nullptr;
}

// Issues a launch on a stream, or records it when `descs` is set.
struct Emitter {
  hipStream_t stream = nullptr;
  std::vector<LaunchDesc> *descs = nullptr;
  template <class Args>
  rrb_status operator()(void (*kern)(Args), dim3 grid, dim3 block, const Args &a, const char *what,
                        const std::string &name) {
    if (descs) {
      LaunchDesc d;
      d.func = reinterpret_cast<const void *>(kern);
      d.grid = grid;
      d.block = block;
      d.args.assign(reinterpret_cast<const unsigned char *>(&a),
                    reinterpret_cast<const unsigned char *>(&a) + sizeof a);
      d.name = name;
      descs->push_back(std::move(d));
      return RRB_OK;
    }
    hipLaunchKernelGGL(kern, grid, block, 0, stream, a);
    return check_launch(what);
  }
};

// Single aligned segment of at most kOneMaxVectors vectors: the decode path.
constexpr int64_t kOneMaxVectors = 4096;

rrb_status launch_one(const Plan &p, const void *const *in, void *const *out, Emitter &emit) {
  const int esz = elem_size(p.dtype);
  const Segment &sg = p.segs[0];
  const bool reduce = p.op != RRB_COPY;
  const bool tree = p.op == RRB_REDUCE_SUM_TREE;
  OneArgs a;
  std::memset(&a, 0, sizeof a);
  if (reduce) {
    for (int32_t r = 0; r < p.nranks; ++r)
      a.in[r] = static_cast<const unsigned char *>(in[r]) + sg.src_off * esz;
  } else {
    a.in[0] = static_cast<const unsigned char *>(in[sg.src_rank]) + sg.src_off * esz;
  }
  for (int32_t q = 0; q < p.nranks; ++q)
    if (sg.dst_mask >> q & 1u) a.out[a.ndst++] = static_cast<unsigned char *>(out[q]) + sg.dst_off * esz;
  a.nvec = static_cast<int32_t>(sg.len * esz / 16);
  a.tail = reduce ? static_cast<int32_t>(sg.len - static_cast<int64_t>(a.nvec) * (16 / esz))
                  : static_cast<int32_t>((sg.len * esz - static_cast<int64_t>(a.nvec) * 16) / 2);
  const unsigned grid = static_cast<unsigned>((a.nvec + kOneBlock - 1) / kOneBlock);
  const bool all = a.ndst == p.nranks;
  const bool bf16 = p.dtype == RRB_BF16;
  OneFn kern = copy_one_kernel;
  if (reduce && !tree)
    kern = all ? (bf16 ? reduce_one_for<true, true, false>(p.nranks)
                       : reduce_one_for<false, true, false>(p.nranks))
               : (bf16 ? reduce_one_for<true, false, false>(p.nranks)
                       : reduce_one_for<false, false, false>(p.nranks));
  else if (reduce)
    kern = all ? (bf16 ? reduce_one_for<true, true, true>(p.nranks)
                       : reduce_one_for<false, true, true>(p.nranks))
               : (bf16 ? reduce_one_for<true, false, true>(p.nranks)
                       : reduce_one_for<false, false, true>(p.nranks));
  std::string name;  // built only when describing, not on the launch path
  if (emit.descs)
    name = !reduce ? std::string("copy_one_kernel")
                   : std::string(tree ? "reduce_tree_one_kernel<" : "reduce_one_kernel<") +
                         std::to_string(p.nranks) + (bf16 ? ",bf16" : ",f32") + (all ? ",all>" : ",list>");
  return emit(kern, dim3(grid), dim3(kOneBlock), a, reduce ? "reduce" : "copy", name);
}

rrb_status launch_uniform(const Plan &p, const void *const *in, void *const *out,
                          Emitter &emit) {
  const int esz = elem_size(p.dtype);
  if (p.segs.empty() || p.segs[0].len == 0) return RRB_OK;
  const int64_t len = p.segs[0].len;

  bool vec = true;
  for (int32_t r = 0; r < p.nranks; ++r) {
    if (p.in_count[r] > 0 && !aligned16(in[r])) vec = false;
    if (p.out_count[r] > 0 && !aligned16(out[r])) vec = false;
  }
  for (const Segment &s : p.segs)
    if ((s.src_off * esz) % 16 || (s.dst_off * esz) % 16) vec = false;
  if (vec && p.segs.size() == 1 && (len * esz) / 16 >= 1 && (len * esz) / 16 <= kOneMaxVectors &&
      p.segs[0].dst_mask != 0)
    return launch_one(p, in, out, emit);

  UniArgs a;
  std::memset(&a, 0, sizeof a);
  for (int32_t r = 0; r < p.nranks; ++r) {
    a.in[r] = static_cast<const unsigned char *>(in[r]);
    a.out[r] = static_cast<unsigned char *>(out[r]);
  }
  a.nranks = p.nranks;
  a.nelem = len;
  const bool reduce = p.op != RRB_COPY;
  const bool tree = p.op == RRB_REDUCE_SUM_TREE;
  const bool bf16 = p.dtype == RRB_BF16;

  int bs;
  int U;
  void (*kern)(UniArgs) = nullptr;
  // Kernel name for introspection, built only when describing.
  std::string name;
  const bool named = emit.descs != nullptr;
  const std::string R_ = named ? std::to_string(p.nranks) : std::string(),
                    dt = named ? (bf16 ? "bf16" : "f32") : "";
  if (vec) {
    a.nvec = (len * esz) / 16;
    a.tail = reduce ? (len - a.nvec * (16 / esz)) : ((len * esz - a.nvec * 16) / 2);
    // Decode-size items spread over more, smaller workgroups.  Streaming
    // launches (kStreamBytesReduce, kStreamOutCopy) take non-temporal hints:
    // loads and stores for a fan-out reduce, loads with write-through stores
    // for a single-destination reduce, stores for a copy; copies that do not
    // stream store write-through (measured best on MI355X for each shape).
    const bool small = a.nvec <= 4096;
    const int64_t traffic = static_cast<int64_t>(p.segs.size()) * len * esz *
                            (reduce ? p.nranks : 1) * 2;
    int64_t out_bytes = 0;
    for (const Segment &sg : p.segs) out_bytes += sg.len * esz * __builtin_popcount(sg.dst_mask);
    const bool stream = reduce ? traffic >= kStreamBytesReduce : out_bytes >= kStreamOutCopy;
    // Mid-size launches keep one vector per lane so the grid still covers
    // every CU several times over; only very large ones unroll.
    const bool big = static_cast<int64_t>(p.segs.size()) * a.nvec >= kBigVectors;
    bs = small ? 64 : 256;
    if (reduce) {
      const bool fan = __builtin_popcount(p.segs[0].dst_mask) > 1;
      const bool huge = static_cast<int64_t>(p.segs.size()) * a.nvec >= kHugeVectors;
      U = (small || !big || p.nranks > 8 || tree) ? 1 : huge ? 2 : 4;
      if (tree) {
        kern = stream ? (fan ? (bf16 ? reduce_tree_vec_for<true, true, true>(p.nranks)
                                     : reduce_tree_vec_for<false, true, true>(p.nranks))
                             : (bf16 ? reduce_tree_vec_for<true, true, false>(p.nranks)
                                     : reduce_tree_vec_for<false, true, false>(p.nranks)))
                      : (bf16 ? reduce_tree_vec_for<true, false, false>(p.nranks)
                              : reduce_tree_vec_for<false, false, false>(p.nranks));
        if (named) name = "reduce_tree_vec_kernel<" + R_ + "," + dt + (stream ? ",nt-load" : "") +
               (stream && fan ? ",nt-store>" : ">");
      } else if (stream && !fan) {
        kern = reduce_wt_pick(U, bf16, p.nranks);
        if (named) name = "reduce_wt_kernel<" + R_ + "," + std::to_string(U) + "," + dt + ">";
      } else if (stream) {
        kern = reduce_vec_pick<true, true>(U, bf16, p.nranks);
        if (named) name = "reduce_vec_kernel<" + R_ + "," + std::to_string(U) + "," + dt + ",nt-load,nt-store>";
      } else {
        // Below the streaming threshold a launch has under 2 M vectors, so
        // one vector per lane.
        kern = bf16 ? reduce_vec_for<1, true, false, false>(p.nranks)
                    : reduce_vec_for<1, false, false, false>(p.nranks);
        if (named) name = "reduce_vec_kernel<" + R_ + ",1," + dt + ">";
      }
    } else {
      // Streaming copies: one vector per lane on 128-lane workgroups (the
      // 64 MiB All-Gather 103 -> 92 us against 256 lanes, 8 ranks).
      // Small fan-out copies keep plain stores: write-through made the
      // 8 x 2 KiB All-Gather of a graph chain 2.5 -> 3.8 us per launch.
      // Single-destination copies below the streaming size (Gather,
      // All-to-All) take two vectors per lane on 128-lane workgroups:
      // Gather 8 x 2 MiB 5.61 -> 4.31 us, All-to-All 8 x 4 MiB 9.99 -> 7.72
      // us per launch (graph replays on MI355X; 8 x 128 KiB Gather 2.15 ->
      // 2.34, the one loss measured).
      int fan = 1;
      for (const Segment &sg : p.segs) fan = std::max(fan, __builtin_popcount(sg.dst_mask));
      const bool fan_any = fan > 1;
      const bool single = !stream && !small && !fan_any;
      const bool split = small && fan_any && a.nvec <= 1024;
      a.fan = fan;
      U = single ? 2 : (small || stream || !big) ? 1 : 4;
      kern = stream             ? copy_vec_kernel<1, true>
             : split            ? copy_split_kernel
             : (small && fan_any) ? copy_vec_kernel<1, false>
             : U == 1             ? copy_wt_kernel<1>
             : U == 2             ? copy_wt_kernel<2>
                                  : copy_wt_kernel<4>;
      if (named) name = stream ? "copy_vec_kernel<1,nt-store>"
             : split ? "copy_split_kernel"
             : (small && fan_any) ? "copy_vec_kernel<1>"
                                  : "copy_wt_kernel<" + std::to_string(U) + ">";
      if (stream || single) bs = 128;
    }
    const int64_t per_tile = static_cast<int64_t>(bs) * U;
    int64_t tiles = (a.nvec + per_tile - 1) / per_tile;
    if (tiles == 0) tiles = 1;  // tail-only item
    if (a.tail > bs) return fail(RRB_EUNSUPPORTED, "tail longer than a workgroup");
    a.tiles = static_cast<int32_t>(tiles);
    // XCD tile runs help streaming reduces; streaming copies run 9% faster
    // in plain order (measured on MI355X, 256 MiB per rank).
    a.xcd_chunk = (stream && reduce && tiles % (8 * kXcdChunk) == 0) ? kXcdChunk : 0;
  } else {
    bs = 256;
    U = 1;
    kern = !reduce ? copy_elem_kernel
           : tree  ? (bf16 ? reduce_tree_elem_kernel<true> : reduce_tree_elem_kernel<false>)
                   : (bf16 ? reduce_elem_kernel<true> : reduce_elem_kernel<false>);
    if (named) name = !reduce ? "copy_elem_kernel" : (tree ? "reduce_tree_elem_kernel<" : "reduce_elem_kernel<") + dt + ">";
    // the element copy moves 2-byte units
    if (!reduce) a.nelem = len * esz / 2;
    a.tiles = static_cast<int32_t>((a.nelem + bs - 1) / bs);
  }
  if (static_cast<int64_t>(a.tiles) * kMaxItems > 0x7fffffffLL)
    return fail(RRB_EUNSUPPORTED, "segment too long for one launch");

  const size_t nseg = p.segs.size();
  for (size_t first = 0; first < nseg; first += kMaxItems) {
    const int cnt = static_cast<int>(std::min<size_t>(kMaxItems, nseg - first));
    for (int i = 0; i < cnt; ++i) {
      const Segment &s = p.segs[first + i];
      a.items[i].src_off = s.src_off * esz;
      a.items[i].dst_off = s.dst_off * esz;
      a.items[i].src_rank = s.src_rank < 0 ? 0 : s.src_rank;
      a.items[i].dst_mask = s.dst_mask;
    }
    const unsigned grid = static_cast<unsigned>(cnt) * static_cast<unsigned>(a.tiles) *
                          static_cast<unsigned>(kern == copy_split_kernel ? a.fan : 1);
    const rrb_status st = emit(kern, dim3(grid), dim3(bs), a, reduce ? "reduce" : "copy", name);
    if (st != RRB_OK) return st;
  }
  return RRB_OK;
}

rrb_status launch_uniform_on(const Plan &p, const void *const *in, void *const *out,
                             hipStream_t stream) {
  Emitter e;
  e.stream = stream;
  return launch_uniform(p, in, out, e);
}

}  // namespace

rrb_status describe_uniform(const Plan &p, const void *const *in, void *const *out,
                            std::vector<LaunchDesc> &descs) {
  Emitter e;
  e.descs = &descs;
  return launch_uniform(p, in, out, e);
}

}  // namespace rrb

using namespace rrb;

extern "C" {

rrb_status rrb_copy(rrb_plan_t plan, const void *const *d_in, void *const *d_out,
                    rrb_stream_t stream) {
  clear_error();
  if (!plan) return fail(RRB_EINVAL, "NULL plan");
  const Plan &p = plan->p;
  if (p.op != RRB_COPY) return fail(RRB_EINVAL, "rrb_copy needs a copy plan");
  rrb_status s = check_buffers(p, d_in, d_out);
  if (s != RRB_OK) return s;
  if (p.kind != PlanKind::Uniform) return launch_rows(p, d_in, d_out, nullptr, stream);
  return launch_uniform_on(p, d_in, d_out, static_cast<hipStream_t>(stream));
}

rrb_status rrb_reduce(rrb_plan_t plan, const void *const *d_in, void *const *d_out,
                      const float *d_weights, rrb_stream_t stream) {
  clear_error();
  if (!plan) return fail(RRB_EINVAL, "NULL plan");
  const Plan &p = plan->p;
  if (p.op != RRB_REDUCE_SUM && p.op != RRB_REDUCE_SUM_TREE)
    return fail(RRB_EINVAL, "rrb_reduce needs a reduce plan");
  if (d_weights && p.kind == PlanKind::Uniform)
    return fail(RRB_EINVAL, "weights apply to MoE combine plans only (a layout-named reduce is an "
                            "unweighted sum)");
  if (d_weights && (reinterpret_cast<uintptr_t>(d_weights) & 3))
    return fail(RRB_EINVAL, "weights must be 4-byte aligned");
  rrb_status s = check_buffers(p, d_in, d_out);
  if (s != RRB_OK) return s;
  if (p.kind != PlanKind::Uniform) return launch_rows(p, d_in, d_out, d_weights, stream);
  return launch_uniform_on(p, d_in, d_out, static_cast<hipStream_t>(stream));
}

rrb_status rrb_plan_launch_info(rrb_plan_t plan, const void *const *d_in, void *const *d_out,
                                char *buf, int32_t cap) {
  clear_error();
  if (!plan || !buf || cap < 1) return fail(RRB_EINVAL, "NULL plan or buffer");
  buf[0] = 0;
  const Plan &p = plan->p;
  if (p.kind != PlanKind::Uniform) return fail(RRB_EUNSUPPORTED, "launch info covers layout-named plans");
  rrb_status s = check_buffers(p, d_in, d_out);
  if (s != RRB_OK) return s;
  std::string text;
  try {
    std::vector<LaunchDesc> descs;
    s = describe_uniform(p, d_in, d_out, descs);
    if (s != RRB_OK) return s;
    for (const LaunchDesc &d : descs) {
      if (!text.empty()) text += "; ";
      text += d.name + " grid=" + std::to_string(d.grid.x) + " block=" + std::to_string(d.block.x);
    }
  } catch (const std::bad_alloc &) {
    return fail(RRB_ENOMEM, "launch description allocation failed");
  }
  std::snprintf(buf, static_cast<size_t>(cap), "%s", text.c_str());
  return RRB_OK;
}

rrb_status rrb_empty_kernel(rrb_stream_t stream) {
  clear_error();
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  return check_launch("empty");
}

}  // extern "C"
