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
// One workgroup owns one token row, so the map entries it needs (k slots and
// weights) are uniform and come through scalar loads; the row itself moves as
// coalesced 16-byte vectors.  Both kernels are HBM-bound: dispatch reads T*h
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
  int64_t tokens_per_rank;
  int64_t row_bytes;     // hidden * 2
  int64_t nvec;          // whole 16-byte vectors per row
  int64_t hidden;
  int32_t k;
};

__device__ __forceinline__ const unsigned char *slot_row(const RowArgs &a, int32_t s,
                                                         const unsigned char *const *base) {
  return base[s >> kSlotRankShift] + static_cast<int64_t>(s & kSlotRowMask) * a.row_bytes;
}

__global__ void __launch_bounds__(256) moe_dispatch_kernel(RowArgs a) {
  const int64_t t = blockIdx.x;
  const int64_t src_rank = t / a.tokens_per_rank;
  const unsigned char *src =
      a.in[src_rank] + (t - src_rank * a.tokens_per_rank) * a.row_bytes;
  const int32_t *slots = a.slot + t * a.k;
  for (int64_t i = threadIdx.x; i < a.nvec; i += blockDim.x) {
    const uint4 x = *reinterpret_cast<const uint4 *>(src + i * 16);
    for (int j = 0; j < a.k; ++j) {
      const int32_t s = slots[j];
      unsigned char *dst = a.out[s >> kSlotRankShift] +
                           static_cast<int64_t>(s & kSlotRowMask) * a.row_bytes;
      *reinterpret_cast<uint4 *>(dst + i * 16) = x;
    }
  }
}

// Any hidden size: 2-byte units.
__global__ void __launch_bounds__(256) moe_dispatch_elem_kernel(RowArgs a) {
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

template <int K>
__global__ void __launch_bounds__(256) moe_combine_kernel(RowArgs a) {
  const int64_t t = blockIdx.x;
  const int64_t dst_rank = t / a.tokens_per_rank;
  unsigned char *dst = a.out[dst_rank] + (t - dst_rank * a.tokens_per_rank) * a.row_bytes;
  const int32_t *slots = a.slot + t * K;
  const float *ws = a.weight + t * K;
  const unsigned char *rows[K];
  float w[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const int32_t s = slots[j];
    rows[j] = a.in[s >> kSlotRankShift] + static_cast<int64_t>(s & kSlotRowMask) * a.row_bytes;
    w[j] = ws[j];
  }
  for (int64_t i = threadIdx.x; i < a.nvec; i += blockDim.x) {
    uint4 z[K];
#pragma unroll
    for (int j = 0; j < K; ++j) z[j] = *reinterpret_cast<const uint4 *>(rows[j] + i * 16);
    float acc[8];
    {
      const uint32_t zz[4] = {z[0].x, z[0].y, z[0].z, z[0].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = w[0] * bf16_lo(zz[q]);
        acc[2 * q + 1] = w[0] * bf16_hi(zz[q]);
      }
    }
#pragma unroll
    for (int j = 1; j < K; ++j) {
      const uint32_t zz[4] = {z[j].x, z[j].y, z[j].z, z[j].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = w[j] * bf16_lo(zz[q]);
        const float hi = w[j] * bf16_hi(zz[q]);
        acc[2 * q] = acc[2 * q] + lo;
        acc[2 * q + 1] = acc[2 * q + 1] + hi;
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4 *>(dst + i * 16) = o;
  }
}

// Any k and any hidden size: one element per lane, k rows folded in order.
__global__ void __launch_bounds__(256) moe_combine_elem_kernel(RowArgs a) {
  const int64_t t = blockIdx.x;
  const int64_t dst_rank = t / a.tokens_per_rank;
  unsigned char *dst = a.out[dst_rank] + (t - dst_rank * a.tokens_per_rank) * a.row_bytes;
  const int32_t *slots = a.slot + t * a.k;
  const float *ws = a.weight + t * a.k;
  for (int64_t i = threadIdx.x; i < a.hidden; i += blockDim.x) {
    float acc = 0.f;
    for (int j = 0; j < a.k; ++j) {
      const int32_t s = slots[j];
      const unsigned char *row =
          a.in[s >> kSlotRankShift] + static_cast<int64_t>(s & kSlotRowMask) * a.row_bytes;
      const float term = ws[j] * bf16_to_f32(*reinterpret_cast<const uint16_t *>(row + i * 2));
      acc = j == 0 ? term : acc + term;
    }
    *reinterpret_cast<uint16_t *>(dst + i * 2) = f32_to_bf16_rne(acc);
  }
}

namespace {

using RowFn = void (*)(RowArgs);

RowFn combine_for(int k) {
  switch (k) {
    case 1: return moe_combine_kernel<1>;
    case 2: return moe_combine_kernel<2>;
    case 4: return moe_combine_kernel<4>;
    case 6: return moe_combine_kernel<6>;
    case 8: return moe_combine_kernel<8>;
    case 16: return moe_combine_kernel<16>;
    default: return nullptr;
  }
}

}  // namespace

rrb_status launch_rows(const Plan &p, const void *const *in, void *const *out, void *stream) {
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
  const size_t n = m.slot.size();
  const size_t slot_bytes = ((n * 4 + 255) / 256) * 256;
  a.slot = static_cast<const int32_t *>(p.d_ws);
  a.weight = reinterpret_cast<const float *>(static_cast<const char *>(p.d_ws) + slot_bytes);
  a.tokens_per_rank = m.tokens / p.nranks;
  a.row_bytes = m.hidden * 2;
  a.nvec = a.row_bytes / 16;
  a.hidden = m.hidden;
  a.k = m.topk;
  RowFn kern;
  if (m.dir == RRB_MOE_DISPATCH) {
    kern = vec ? moe_dispatch_kernel : moe_dispatch_elem_kernel;
  } else {
    kern = vec ? combine_for(m.topk) : nullptr;
    if (!kern) kern = moe_combine_elem_kernel;
  }
  if (m.tokens > 0x7fffffffLL) return fail(RRB_EUNSUPPORTED, "too many tokens for one launch");
  hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(m.tokens)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RRB_EHIP, "moe launch: %s", hipGetErrorString(e));
  return RRB_OK;
}

}  // namespace rrb
