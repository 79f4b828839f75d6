// SNAC: stage / notify / consume orchestration of a decode All-Reduce chain.
//
// Purlin: Separating Orchestration from the Datapath of Collectives ("The
// Purlin PDF describes a three-layer design") names the orchestration layer
// Stage, Notify, And Consume.  SiFAR: Synchronization-Free All-Reduce for
// Low-Latency LLM Inference (review page: abstract; Fig. 1, Fig. 8, Fig. 14;
// the "Load-bearing premise"; referee report on §8.1) gives the protocol
// variants run here, over R simulated ranks in one GPU:
//
//   barrier      one staging buffer; top barrier (every source's flag) before
//                consuming, bottom barrier (every reader done) before the
//                next stage -- the write-after-read guard of Fig. 8.
//   dual         two staging buffers by epoch parity; the next epoch's top
//                barrier already proves the readers of this buffer finished,
//                so the bottom barrier goes.
//   speculative  dual buffers and no top barrier: one read of the sources'
//                flags, then the consume loads start at once and a reduced
//                validation flag (sum of the R sources' flags == R * epoch,
//                per workgroup slice) decides whether the result stands; on
//                mismatch only the stale sources are waited for and read
//                again.
//   twoshot      dual buffers; reduce-scatter into a reduced buffer, a second
//                flag round, then all-gather (SiFAR review, Fig. 6).
//   lamport      flag-in-data, the Lamport-style All-Reduce SiFAR compares
//                against (review page, Fig. 20): no flags, no fences.  Each
//                16-bit half of the payload is staged in a 32-bit word under
//                a 16-bit epoch tag; a reader polls every word it needs until
//                all carry this epoch's tag (lamport_chain_kernel below).
//   graph        no persistent kernel: one Atom All-Reduce launch per epoch,
//                chained in a cached HIP graph.
// Chains of any layout-named collective run the barrier, dual and
// speculative protocols over the plan's index map (snac_plan_kernel below).
//
// One persistent kernel runs the whole chain.  Rank r is a group of S
// workgroups; workgroup (r, s) stages slice s of rank r's payload, publishes
// flag[buf][r][s] = epoch, then reduces slice s of all R staged payloads in
// rank order 0..R-1 (fp32, one bf16 rounding) into rank r's output -- the
// oneshot All-Reduce of SiFAR's Fig. 5, every rank reducing the full payload.
//
// Speculation order.  The pages read the payload first and the flags after,
// and rely on no rank overtaking the reader between those two loads.  Here
// the flags are read first, and the payload loads are issued once the flag
// values have returned (loads from one wave may be served in any order, so
// issuing them together would rest on the memory system serving the flag
// first).  A flag equal to the epoch then proves the source finished staging
// before its payload loads were issued; the speculation is that the payload
// is loaded whatever the flags said, and the reduced flag decides afterwards.
// The speculative loads are device-coherent (the same cache policy as
// agent-scope atomic loads), so a line cached from an earlier epoch is never
// returned.

// Memory ordering without fences.  Every byte one workgroup writes for
// another (staged payloads, the twoshot reduced payload) is stored with the
// cache policy of agent-scope atomic stores (sc1): written through this XCD's
// L2 to the device's point of coherence.  notify() waits until all of the
// wave's memory operations have completed (s_waitcnt 0: the write-through
// stores acknowledged, the loads returned) before the flag store, and
// readers load that data, after the flag, with the policy of agent-scope
// atomic loads (sc1), which never returns a line cached from an earlier
// epoch.  The agent-scope release and acquire fences that would otherwise
// bracket each flag write back or invalidate the whole L2 of the XCD; with
// 8-64 workgroups per XCD taking them every epoch they dominated small
// payloads.  Measured on MI355X, 8 ranks, 64-epoch chains, per All-Reduce:
// dual 8 KiB 2.52 -> 2.09 us, barrier 256 KiB 13.7 -> 6.6 us, twoshot 512 KiB
// 21.0 -> 13.3 us, every result bit-exact (including 100k-epoch stress).  The
// same completion wait covers the write-after-read guards: a rank's flag of
// epoch e + 1 is stored only after its epoch-e loads have returned.
//
// This ordering rests on how the hardware completes a wave's memory
// operations, below the source-level memory model.  Built with
// RRB_SNAC_FENCES=1 (librrb_fenced.so), the flag-based chains take the
// memory model's own form instead: each flag is published with an
// agent-scope release store, and every wave that has seen flags (a wait, or
// the speculative flag read) takes an agent-scope acquire fence before it
// touches the data they announce or overwrites a buffer they release.  The
// kernels are otherwise the same.  The flag-in-data chain, whose ordering is
// per word, has no fenced form and is refused by that build.
//
// Every wait is bounded: a wait that exceeds its poll budget raises a status
// word that every other wait also watches, so the whole grid drains and the
// host sees RRB_ETIMEOUT.  The grid must be co-resident: it takes a plain
// launch when it fits well within the device (launch_persistent), else a
// cooperative one.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>

#include "rrb_internal.h"
#include "rrb_kernels.h"

namespace rrb {
namespace {

constexpr int kFlagStride = 32;          // u32 words: one 128-byte line per flag
constexpr uint32_t kDefaultSpin = 1u << 21;  // polls (about 1 us each)
constexpr int kMaxSlices = 256;
constexpr int64_t kSpecMaxBytes = 128 << 10;  // All-Reduce chains speculate up to this payload per rank
constexpr int64_t kLamportSettleVec = 4096;    // 64 KiB per rank (see lamport_chain_kernel)
constexpr int kStageU = 8;  // vectors in flight per lane in the stage copy

#ifndef RRB_SNAC_FENCES
#define RRB_SNAC_FENCES 0
#endif
constexpr bool kFences = RRB_SNAC_FENCES != 0;  // memory-model build (see above)

// Fenced build: agent-scope acquire after flags were seen; nothing otherwise.
__device__ __forceinline__ void acquire_if_fenced() {
  if constexpr (kFences) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// kLamportOne: the flag-in-data kernel shaped for slices of at most one
// vector per lane.
enum Variant : int32_t { kBarrier = 0, kDual = 1, kSpeculative = 2, kTwoshot = 3, kLamport = 4,
                         kLamportOne = 5 };

struct SnacArgs {
  const unsigned char *in;   // [E][R][count]
  unsigned char *out;        // [E][R][count]
  unsigned char *staging;    // [2][R][count]
  uint32_t *flag;            // [2][R][S] x kFlagStride
  uint32_t *done;            // [R][S] x kFlagStride
  uint32_t *status;          // [0]: nonzero once any wait timed out
  rrb_snac_stats *stats;
  const uint32_t *stagger;
  int64_t count;             // elements per rank payload
  int64_t rank_bytes;        // count * elem size
  int64_t nvec;              // 16-byte vectors per rank payload
  int64_t slice_vec;         // vectors per slice (the last slice may be short)
  unsigned char *reduced;    // twoshot: [2][count], chunk q owned by rank q
  uint32_t *flag2;           // twoshot: [2][R][S] x kFlagStride, chunk reduced
  int64_t chunk_vec;         // twoshot: vectors per chunk (ceil(nvec / R))
  int64_t piece_vec;         // twoshot: vectors per piece (ceil(chunk_vec / S))
  unsigned char *tagged;     // lamport: [2][R][2 * count * elem size] tagged words
  uint32_t epoch0;           // global number of this call's first epoch (>= 1)
  int32_t epochs;
  int32_t S;
  uint32_t spin_limit;
};

struct Layout {
  int64_t staging_off, entries_off, waits_off = 0, reduced_off, flag_off, flag2_off, done_off, tagged_off,
      status_off, total;
};

// staging [2][R][count] | reduced [2][count] | flags [2][R][S] | flags2 [2][R][S]
// | done [R][S] | tagged [2][R][2 count] | status; everything from flag_off
// on is cleared at bind.  The flag-in-data variant has only the tagged
// buffers (tag 0 after the clear, which no epoch uses before overwriting),
// the others have none.
Layout layout_for(int32_t R, int64_t count, int32_t dtype, int32_t S, bool lamport) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t rank_bytes = count * elem_size(dtype);
  Layout l;
  l.staging_off = 0;
  const int64_t staging = lamport ? 0 : up(2LL * R * rank_bytes);
  l.entries_off = staging;
  l.reduced_off = staging;
  const int64_t reduced = lamport ? 0 : up(2LL * rank_bytes);
  l.flag_off = l.reduced_off + reduced;
  const int64_t flags = lamport ? 0 : up(2LL * R * S * kFlagStride * 4);
  l.flag2_off = l.flag_off + flags;
  l.done_off = l.flag2_off + flags;
  const int64_t done = lamport ? 0 : up(1LL * R * S * kFlagStride * 4);
  l.tagged_off = l.done_off + done;
  const int64_t tagged = lamport ? up(2LL * R * 2 * rank_bytes) : 0;
  l.status_off = l.tagged_off + tagged;
  l.total = l.status_off + 256;
  return l;
}

// Chains of any uniform plan: one consume entry per (output rank, segment),
// offsets and lengths in 16-byte vectors.  src_rank < 0: reduce over all
// ranks in rank order.
struct PlanEntry {
  int64_t src_off, dst_off, len;
  int32_t src_rank, pad;
};

// staging [2][R][in_stride] | entries | wait lists | flags [2][R][S] |
// done [R][S] | status; the entries and wait lists are uploaded at bind,
// everything from flag_off on is cleared.
Layout layout_for_plan(int32_t R, int64_t in_stride, int32_t S, int64_t nentries,
                       int64_t nwait_words) {
  auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
  Layout l;
  l.staging_off = 0;
  l.entries_off = up(2LL * R * in_stride);
  l.waits_off = l.entries_off + up(nentries * static_cast<int64_t>(sizeof(PlanEntry)));
  l.reduced_off = l.waits_off + up(nwait_words * 4);
  l.flag_off = l.reduced_off;
  const int64_t flags = up(2LL * R * S * kFlagStride * 4);
  l.flag2_off = l.flag_off + flags;
  l.done_off = l.flag2_off;
  l.tagged_off = l.done_off + up(1LL * R * S * kFlagStride * 4);
  l.status_off = l.tagged_off;
  l.total = l.status_off + 256;
  return l;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// 16-byte store at byte offset `off` of a `bytes`-long buffer with the cache
// policy of agent-scope atomic stores (sc1): the line is written through
// rather than left dirty in this XCD's L2.  Every staged payload goes through
// here, since notify() takes no L2 write-back; the barrier, dual and
// speculative All-Reduce chains also store their outputs this way (4-13%
// less time per All-Reduce from 8 KiB to 2 MiB than plain output stores,
// measured on MI355X when the chains still took fences).
__device__ __forceinline__ void store_wt(unsigned char *base, int64_t bytes, int64_t off, v4u x) {
  __builtin_amdgcn_raw_buffer_store_b128(x, rsrc(base, bytes), static_cast<int32_t>(off), 0, 16);
}
// Write-through (WT) or plain 16-byte store.
template <bool WT>
__device__ __forceinline__ void store16(unsigned char *base, int64_t bytes, int64_t off, v4u x) {
  if (WT) store_wt(base, bytes, off, x);
  else *reinterpret_cast<v4u *>(base + off) = x;
}

// Device-coherent 16-byte load (cache policy sc1, as for agent-scope atomic
// loads): never served from a line another epoch left in this CU's caches.
__device__ __forceinline__ uint4 load_coherent(__amdgpu_buffer_rsrc_t r, int32_t off) {
  const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
  uint4 o;
  o.x = x[0];
  o.y = x[1];
  o.z = x[2];
  o.w = x[3];
  return o;
}

__device__ __forceinline__ uint32_t load_flag_relaxed(const uint32_t *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Keeps the compiler from moving later memory accesses above this point,
// without waiting for anything: for payload loads that must follow flag
// values the wave has already consumed (in a branch or a reduction), which
// the hardware only issues after those values have returned.  Loads from one
// wave to different addresses may be served in any order, so a payload load
// that must not see data older than a flag is issued only after the flag's
// value is back; issuing the two together would rest on service order.
__device__ __forceinline__ void order_after_values() {
  acquire_if_fenced();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// Reduced validation flag of the first N lanes' flag values f: their sum,
// and the set of lanes whose flag is not `ep`, both wave-uniform.  Each value
// is read into a scalar register (v_readlane, unrolled), so the reduction
// stays in registers and the results steer scalar branches; cross-lane
// shuffles through LDS cost about 0.5 us per epoch here.
template <int N>
__device__ __forceinline__ void flags_reduce(uint32_t f, uint32_t ep, uint32_t &sum, uint32_t &stale) {
  sum = 0;
  stale = 0;
#pragma unroll
  for (int l = 0; l < N; ++l) {
    const uint32_t fl = __builtin_amdgcn_readlane(f, l);
    sum += fl;
    if (fl != ep) stale |= 1u << l;
  }
}

// Polls *p until it reaches `want`; false if the budget ran out or another
// wait already timed out (then the status word is set).
__device__ bool wait_at_least(const uint32_t *p, uint32_t want, uint32_t *status,
                              uint32_t limit) {
  uint32_t spins = 0;
  // Relaxed (device-coherent) polls; what follows a successful wait reads
  // with device-coherent loads, issued after the flag value has returned.
  while (load_flag_relaxed(p) < want) {
    if ((spins & 63) == 0 && load_flag_relaxed(status) != 0) return false;
    if (++spins >= limit) {
      __hip_atomic_store(status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  return true;
}

// Threads 0..R-1 each wait for one rank's word at `base + t * stride_words`.
// Returns, in every thread, whether all R waits succeeded.  The chain
// workgroups are single waves: with VOTE the result is a wave vote; without
// it the R results meet in `ok`, an LDS array of R flags, behind a workgroup
// barrier.  The vote took the barrier chain 4-14% and twoshot 3-6% less time
// per All-Reduce at 8 KiB-1 MiB (MI355X, 8 ranks).  In the dual-buffer kernel
// it let the compiler hoist more work above the wait, 143 VGPRs against 112,
// so 2048-workgroup chains launched cooperatively (512 KiB 4.73 -> 5.07 us);
// that kernel keeps the LDS form.
template <int R, bool VOTE>
__device__ bool wait_all(const uint32_t *base, int64_t stride_words, uint32_t want,
                         uint32_t *status, uint32_t limit, int *ok) {
  if (VOTE) {
    bool mine = true;
    if (threadIdx.x < R) mine = wait_at_least(base + threadIdx.x * stride_words, want, status, limit);
    const bool all = __all(mine) != 0;
    // No acquire fence (but in the fenced build): the data that follows is
    // read with device-coherent loads, issued after the flags were seen.
    acquire_if_fenced();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    return all;
  }
  if (threadIdx.x < R)
    ok[threadIdx.x] = wait_at_least(base + threadIdx.x * stride_words, want, status, limit) ? 1 : 0;
  __syncthreads();
  // No acquire fence (as above).
  acquire_if_fenced();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  bool all = true;
#pragma unroll
  for (int t = 0; t < R; ++t) all = all && ok[t] != 0;
  return all;
}

// Publishes `ep` in *flag once every wave's earlier memory operations have
// completed: each wave waits for its own write-through stores to be
// acknowledged and its loads to return (s_waitcnt 0; no L2 write-back is
// needed, nothing the readers need sits dirty in L2), then thread 0 stores
// the flag after the workgroup barrier.
//
// With SETTLE the workgroup also waits for its own flag store to be
// acknowledged before it reads other flags.  A flag read issued right behind
// the store samples memory while the other ranks' flag stores of the same
// epoch are still on their way, and its value only returns after the store
// is acknowledged anyway (a wave's memory operations complete in issue
// order), so it mostly came back stale and was read again.  Measured on
// MI355X, 8 ranks, 64-epoch All-Reduce chains, us per All-Reduce: dual
// 8 KiB 1.99 -> 1.95, 128 KiB 2.72 -> 2.43; speculative 8 KiB 1.93 -> 1.80
// (failed validations 67% -> 14%), 128 KiB 2.78 -> 2.33 (74% -> 1%);
// barrier 8 KiB 3.09 -> 2.65; twoshot 128 KiB 5.07 -> 4.29.  The plan
// chains read their wait lists from memory after the flag store, and that
// load's completion wait already covers the store.
template <bool SETTLE = true>
__device__ __forceinline__ void notify(uint32_t *flag, uint32_t ep) {
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    if constexpr (kFences)
      __hip_atomic_store(flag, ep, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    else
      __hip_atomic_store(flag, ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (SETTLE) {
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  }
}

// Reduce one pass of this workgroup's slice: R loads in flight per lane, fold
// in rank order, store the result at byte `off` of the `bytes`-long `dst`.
template <int R, bool BF16, bool WT = true>
__device__ __forceinline__ void reduce_pass(const uint4 (&v)[R], unsigned char *dst, int64_t bytes,
                                            int64_t off) {
  const uint4 o = BF16 ? fold_bf16x8<R>(v) : fold_f32x4<R>(v);
  store16<WT>(dst, bytes, off, v4u{o.x, o.y, o.z, o.w});
}

// Stage: vectors [v0, v1) of a rank's payload `src` into its staged buffer
// `mine` (rank_bytes long), written through, by all the workgroup's lanes.
// Every pass issues all of its loads before its stores, a partial last pass
// included: a remainder loop of one load and one store per step put a slice
// of 2-7 vectors per lane through as many round trips (8 ranks, 512 KiB
// payload, 256 vectors per workgroup: 6.9 -> 5.4 us per All-Reduce, dual
// buffer).  A slice of at most one vector per lane takes a single load and
// store (2-6% less time per All-Reduce at 8-32 KiB than the masked pass).
__device__ __forceinline__ void stage_slice(const unsigned char *src, unsigned char *mine,
                                            int64_t rank_bytes, int64_t v0, int64_t v1) {
  const int bs = blockDim.x;
  if (v1 - v0 <= bs) {
    const int64_t i = v0 + threadIdx.x;
    if (i < v1) store_wt(mine, rank_bytes, i * 16, *reinterpret_cast<const v4u *>(src + i * 16));
    return;
  }
  for (int64_t i0 = v0 + threadIdx.x; i0 < v1; i0 += static_cast<int64_t>(bs) * kStageU) {
    v4u x[kStageU];  // (HIP's uint4 struct here would be placed in scratch)
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * bs;
      if (i < v1) x[u] = *reinterpret_cast<const v4u *>(src + i * 16);
    }
#pragma unroll
    for (int u = 0; u < kStageU; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * bs;
      if (i < v1) store_wt(mine, rank_bytes, i * 16, x[u]);
    }
  }
}

// Twoshot piece (q, s): slice s of chunk q, as a vector range [lo, hi).
__device__ __forceinline__ void piece_range(const SnacArgs &a, int q, int s, int64_t &lo,
                                            int64_t &hi) {
  const int64_t c0 = min(a.nvec, static_cast<int64_t>(q) * a.chunk_vec);
  const int64_t c1 = min(a.nvec, c0 + a.chunk_vec);
  lo = min(c1, c0 + static_cast<int64_t>(s) * a.piece_vec);
  hi = min(c1, lo + a.piece_vec);
}

// Copies pieces (q, s), q = 0..R-1, from `from` to `to` (both payload-shaped).
// COHERENT reads with the device-coherent policy (data another workgroup
// wrote this epoch); WT stores write through.  Byte offsets fit 31 bits
// (staging is below 2 GiB).
//
// Pieces of at least a workgroup's width: per pass, 2 vectors of every piece
// per lane in flight (2 R loads, no index division).  Narrower pieces are
// one flat index range of R x piece_vec vectors spread over all lanes,
// kCopyU per lane: a pass per piece left most lanes idle (8 KiB payload, 8
// ranks: stage and one flag round took 4.2 us per epoch, against 1.3 us for
// a contiguous slice; the whole twoshot epoch went 8.3 -> 4.2 us), while at
// 64-vector pieces the flat range ran 4% behind.
constexpr int kCopyU = 4;

template <int R, bool COHERENT, bool WT>
__device__ __forceinline__ void copy_pieces(const SnacArgs &a, int s, const unsigned char *from,
                                            unsigned char *to, int64_t bytes) {
  const int bs = blockDim.x;
  if (a.piece_vec >= bs) {
    int64_t lo[R], hi[R];
#pragma unroll
    for (int q = 0; q < R; ++q) piece_range(a, q, s, lo[q], hi[q]);
    for (int64_t base = threadIdx.x; base < a.piece_vec; base += 2LL * bs) {
      v4u x[R][2];
      int32_t at[R][2];
#pragma unroll
      for (int q = 0; q < R; ++q) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int64_t i = lo[q] + base + static_cast<int64_t>(u) * bs;
          at[q][u] = i < hi[q] ? static_cast<int32_t>(i * 16) : -1;
          if (at[q][u] >= 0) {
            if (COHERENT) {
              const uint4 y = load_coherent(rsrc(from, bytes), at[q][u]);
              x[q][u] = v4u{y.x, y.y, y.z, y.w};
            } else {
              x[q][u] = *reinterpret_cast<const v4u *>(from + at[q][u]);
            }
          }
        }
      }
#pragma unroll
      for (int q = 0; q < R; ++q)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (at[q][u] >= 0) store16<WT>(to, bytes, at[q][u], x[q][u]);
    }
    return;
  }
  const uint32_t pv = static_cast<uint32_t>(a.piece_vec);
  const uint32_t total = static_cast<uint32_t>(R) * pv;
  for (uint32_t f0 = threadIdx.x; f0 < total; f0 += static_cast<uint32_t>(bs) * kCopyU) {
    v4u x[kCopyU];
    int32_t at[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint32_t f = f0 + static_cast<uint32_t>(u * bs);
      at[u] = -1;
      if (f < total) {
        const int q = static_cast<int>(f / pv);
        int64_t lo, hi;
        piece_range(a, q, s, lo, hi);
        const int64_t i = lo + (f - static_cast<uint32_t>(q) * pv);
        if (i < hi) at[u] = static_cast<int32_t>(i * 16);
      }
      if (at[u] >= 0) {
        if (COHERENT) {
          const uint4 y = load_coherent(rsrc(from, bytes), at[u]);
          x[u] = v4u{y.x, y.y, y.z, y.w};
        } else {
          x[u] = *reinterpret_cast<const v4u *>(from + at[u]);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyU; ++u)
      if (at[u] >= 0) store16<WT>(to, bytes, at[u], x[u]);
  }
}

// One twoshot epoch of workgroup (r, s) (SiFAR review, Fig. 6: reduce-scatter
// then all-gather): stage slice s of every chunk of rank r's payload; once
// every rank has, reduce piece (r, s) -- slice s of chunk r -- over the R
// ranks into the reduced buffer; once every rank's piece s is reduced, copy
// pieces (q, s) of the reduced payload into rank r's output.  Two flag
// rounds per epoch, but each rank reads 2x its payload instead of R x.
template <int R, bool BF16>
__device__ bool twoshot_epoch(const SnacArgs &a, int r, int s, int k, uint32_t ep, int *lds_ok) {
  const int bs = blockDim.x;
  const int b = static_cast<int>(ep & 1u);
  const int64_t stride_rs = static_cast<int64_t>(a.S) * kFlagStride;
  unsigned char *stage_base = a.staging + static_cast<int64_t>(b) * R * a.rank_bytes;
  unsigned char *red = a.reduced + static_cast<int64_t>(b) * a.rank_bytes;
  uint32_t *flags_b = a.flag + static_cast<int64_t>(b) * R * stride_rs;
  uint32_t *flags2_b = a.flag2 + static_cast<int64_t>(b) * R * stride_rs;
  const unsigned char *src = a.in + (static_cast<int64_t>(k) * R + r) * a.rank_bytes;
  unsigned char *mine = stage_base + static_cast<int64_t>(r) * a.rank_bytes;
  unsigned char *dst = a.out + (static_cast<int64_t>(k) * R + r) * a.rank_bytes;

  // Stage pieces (q, s) of this rank's payload, written through for the
  // readers of other XCDs.
  copy_pieces<R, false, true>(a, s, src, mine, a.rank_bytes);
  notify(flags_b + r * stride_rs + s * kFlagStride, ep);
  if (!wait_all<R, true>(flags_b + s * kFlagStride, stride_rs, ep, a.status, a.spin_limit, lds_ok))
    return false;

  // Reduce-scatter: piece (r, s) over all ranks, into the reduced payload.
  {
    int64_t lo, hi;
    piece_range(a, r, s, lo, hi);
    // Two vectors per lane: 106 VGPRs, four waves per SIMD, so a grid of
    // 2048 workgroups (256 slices per rank from 512 KiB) launches plainly.
    constexpr int CU = 2;
    for (int64_t i0 = lo + threadIdx.x; i0 < hi; i0 += static_cast<int64_t>(bs) * CU) {
      uint4 v[CU][R];
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int64_t i = i0 + static_cast<int64_t>(u) * bs;
        if (i < hi) {
#pragma unroll
          for (int q = 0; q < R; ++q)
            v[u][q] = load_coherent(rsrc(stage_base + static_cast<int64_t>(q) * a.rank_bytes,
                                         a.rank_bytes),
                                    static_cast<int32_t>(i * 16));
        }
      }
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int64_t i = i0 + static_cast<int64_t>(u) * bs;
        if (i < hi) reduce_pass<R, BF16, true>(v[u], red, a.rank_bytes, i * 16);
      }
    }
  }
  notify(flags2_b + r * stride_rs + s * kFlagStride, ep);
  if (!wait_all<R, true>(flags2_b + s * kFlagStride, stride_rs, ep, a.status, a.spin_limit, lds_ok))
    return false;

  // All-gather: pieces (q, s) of the reduced payload into this rank's output.
  copy_pieces<R, true, false>(a, s, red, dst, a.rank_bytes);
  return true;
}

template <int R, bool BF16, int VAR>
__global__ void __launch_bounds__(64) snac_chain_kernel(SnacArgs a) {
  __shared__ int lds_ok[R];
  const int r = blockIdx.x / a.S;
  const int s = blockIdx.x - r * a.S;
  const int bs = blockDim.x;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_vec;
  const int64_t v1 = min(a.nvec, v0 + a.slice_vec);
  const int64_t stride_rs = static_cast<int64_t>(a.S) * kFlagStride;  // words per rank
  unsigned long long misspec = 0, retries = 0, timeouts = 0, done_epochs = 0;

  for (int k = 0; k < a.epochs; ++k) {
    const uint32_t ep = a.epoch0 + static_cast<uint32_t>(k);
    if constexpr (VAR == kTwoshot) {
      if (a.stagger) {
        const uint32_t d = a.stagger[r];
        for (uint32_t i = 0; i < d; ++i) __builtin_amdgcn_s_sleep(1);
      }
      if (!twoshot_epoch<R, BF16>(a, r, s, k, ep, lds_ok)) {
        ++timeouts;
        break;
      }
      ++done_epochs;
      continue;
    }
    const int b = VAR == kBarrier ? 0 : static_cast<int>(ep & 1u);
    unsigned char *stage_base = a.staging + static_cast<int64_t>(b) * R * a.rank_bytes;
    uint32_t *flags_b = a.flag + static_cast<int64_t>(b) * R * stride_rs;

    // Test hook: a late rank.
    if (a.stagger) {
      const uint32_t d = a.stagger[r];
      for (uint32_t i = 0; i < d; ++i) __builtin_amdgcn_s_sleep(1);
    }

    // Stage: this rank's slice lands in its staged buffer.
    stage_slice(a.in + (static_cast<int64_t>(k) * R + r) * a.rank_bytes,
                stage_base + static_cast<int64_t>(r) * a.rank_bytes, a.rank_bytes, v0, v1);

    // Notify.
    notify(flags_b + r * stride_rs + s * kFlagStride, ep);

    // Consume: fold the R staged slices in rank order, CU vectors x R
    // sources in flight per lane.  Two vectors keep the barrier and dual
    // kernels at 112 VGPRs, four waves per SIMD, so a chain of 2048
    // workgroups (256 slices per rank from 512 KiB) stays within half the
    // device and takes a plain launch; four vectors took 176 VGPRs and a
    // cooperative launch (dual, 8 ranks, us per All-Reduce: 512 KiB 5.01 ->
    // 4.68, 2 MiB 14.76 -> 13.98; barrier 5-10% faster from 256 KiB).
    unsigned char *dst_base = a.out + (static_cast<int64_t>(k) * R + r) * a.rank_bytes;
    constexpr int CU = 2;
    // The speculative first pass holds its loads across the flag wait: two
    // vectors per lane keep the kernel within 256 VGPRs, two waves per SIMD,
    // so a chain of 1024 workgroups stays within half the device and takes a
    // plain launch (four vectors took 310 VGPRs and a cooperative launch).
    constexpr int CUS = R <= 8 ? 2 : 1;
    int64_t first = v0 + threadIdx.x;  // first vector of the ordinary passes
    if (VAR == kSpeculative) {
      // No top barrier.  One read of the R sources' flags (lanes 0..R-1);
      // once those values have returned, the first pass loads every source
      // whatever its flag said.  The reduced validation flag (SiFAR review,
      // Fig. 14) decides: the flags must sum to R * epoch.  Every flag holds
      // epoch or epoch - 2 (dual buffering keeps each rank within one epoch
      // of its readers), so the sum is exact, and a valid sum also proves
      // every source's reads of this buffer two epochs ago returned before
      // its flag.  A source whose flag read as the epoch had finished staging
      // before its loads were issued, so on a mismatch only the stale sources
      // are waited for and read again; the others' data stays in registers.
      uint32_t f = 0;
      if (threadIdx.x < R) f = load_flag_relaxed(flags_b + threadIdx.x * stride_rs + s * kFlagStride);
      uint32_t sum, stale;
      flags_reduce<R>(f, ep, sum, stale);
      order_after_values();
      constexpr uint32_t kAll = R >= 32 ? ~0u : (1u << R) - 1u;
      const bool valid = sum == static_cast<uint32_t>(R) * ep;
      // re-read after the wait (a failed sum always has a stale flag; all,
      // should it not)
      const uint32_t late = valid ? 0u : (stale ? stale : kAll);
      uint4 v[CUS][R];
#pragma unroll
      for (int u = 0; u < CUS; ++u) {
        const int64_t i = first + static_cast<int64_t>(u) * bs;
        if (i < v1) {
#pragma unroll
          for (int q = 0; q < R; ++q)
            v[u][q] = load_coherent(rsrc(stage_base + static_cast<int64_t>(q) * a.rank_bytes, a.rank_bytes),
                                    static_cast<int32_t>(i * 16));
        }
      }
      bool ok = true;
      if (late) {
        ++misspec;
        retries += static_cast<unsigned long long>(__builtin_popcount(late));
        bool mine = true;
        if (threadIdx.x < R && (late >> threadIdx.x & 1u))
          mine = wait_at_least(flags_b + threadIdx.x * stride_rs + s * kFlagStride, ep, a.status,
                               a.spin_limit);
        ok = __all(mine) != 0;
        if (ok) {
          order_after_values();
#pragma unroll
          for (int q = 0; q < R; ++q) {
            if (late >> q & 1u) {
#pragma unroll
              for (int u = 0; u < CUS; ++u) {
                const int64_t i = first + static_cast<int64_t>(u) * bs;
                if (i < v1)
                  v[u][q] = load_coherent(rsrc(stage_base + static_cast<int64_t>(q) * a.rank_bytes,
                                               a.rank_bytes),
                                          static_cast<int32_t>(i * 16));
              }
            }
          }
        }
      }
      if (!ok) {
        ++timeouts;
        break;
      }
#pragma unroll
      for (int u = 0; u < CUS; ++u) {
        const int64_t i = first + static_cast<int64_t>(u) * bs;
        if (i < v1) reduce_pass<R, BF16>(v[u], dst_base, a.rank_bytes, i * 16);
      }
      first += static_cast<int64_t>(bs) * CUS;
    } else if (!wait_all<R, VAR == kBarrier>(flags_b + s * kFlagStride, stride_rs, ep, a.status,
                                             a.spin_limit, lds_ok)) {
      // the top barrier over the R sources' flags of this slice
      ++timeouts;
      break;
    }

    for (int64_t i0 = first; i0 < v1; i0 += static_cast<int64_t>(bs) * CU) {
      uint4 v[CU][R];
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int64_t i = i0 + static_cast<int64_t>(u) * bs;
        if (i < v1) {
#pragma unroll
          for (int q = 0; q < R; ++q)
            v[u][q] = load_coherent(rsrc(stage_base + static_cast<int64_t>(q) * a.rank_bytes,
                                         a.rank_bytes),
                                    static_cast<int32_t>(i * 16));
        }
      }
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int64_t i = i0 + static_cast<int64_t>(u) * bs;
        if (i < v1) reduce_pass<R, BF16>(v[u], dst_base, a.rank_bytes, i * 16);
      }
    }

    if (VAR == kBarrier) {
      // Bottom barrier: every reader of this rank's slice is done before the
      // next stage overwrites it.
      notify(a.done + (static_cast<int64_t>(r) * a.S + s) * kFlagStride, ep);
      if (!wait_all<R, true>(a.done + static_cast<int64_t>(s) * kFlagStride, stride_rs, ep, a.status,
                       a.spin_limit, lds_ok)) {
        ++timeouts;
        break;
      }
    }
    ++done_epochs;
  }

  if (a.stats && threadIdx.x == 0) {
    if (misspec) atomicAdd(&a.stats->misspec, misspec);
    if (retries) atomicAdd(&a.stats->retries, retries);
    if (timeouts) atomicAdd(&a.stats->timeouts, timeouts);
    atomicAdd(&a.stats->epochs, done_epochs);
  }
}

// ---- flag-in-data (Lamport-style) chain ----------------------------------
//
// The payload is viewed as 16-bit halves; half j of a rank's payload is
// staged as the 32-bit word (tag << 16) | half, tag = epoch mod 2^16, so 16
// payload bytes become 32 staged bytes.  Words are stored and polled with
// the agent-scope relaxed-atomic cache policy (sc1).  A 32-bit access is
// single-copy atomic, so a word that shows this epoch's tag holds this
// epoch's half, whatever became visible before or after it: nothing orders
// one word against another and nothing needs to, so the variant has no flag,
// no release and no acquire.  Two tagged buffers alternate by epoch parity.
// A rank stores into buffer e&1 at epoch e + 2 only after it has read every
// rank's epoch e + 1 words, and each rank stored those after its own epoch-e
// polls had returned (their tags decide when its consume ends), so no reader
// of epoch e is still waiting on that buffer.  The tags of e and e - 2
// differ, and the tag 0 left by bind is met only by epochs that already
// overwrote it.

__device__ __forceinline__ void store_tagged(__amdgpu_buffer_rsrc_t r, int32_t off, v4u w) {
  __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 16);
}

__device__ __forceinline__ v4u load_tagged(__amdgpu_buffer_rsrc_t r, int32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 16);
}

// 8 halves of a payload vector -> two vectors of tagged words (T = tag << 16).
__device__ __forceinline__ void tag_halves(v4u x, uint32_t T, v4u &lo, v4u &hi) {
  lo = v4u{T | (x[0] & 0xffffu), T | (x[0] >> 16), T | (x[1] & 0xffffu), T | (x[1] >> 16)};
  hi = v4u{T | (x[2] & 0xffffu), T | (x[2] >> 16), T | (x[3] & 0xffffu), T | (x[3] >> 16)};
}

__device__ __forceinline__ bool tagged_with(v4u w, uint32_t T) {
  return (((w[0] ^ T) | (w[1] ^ T) | (w[2] ^ T) | (w[3] ^ T)) >> 16) == 0;
}

__device__ __forceinline__ uint4 untag(v4u lo, v4u hi) {
  uint4 x;
  x.x = (lo[0] & 0xffffu) | (lo[1] << 16);
  x.y = (lo[2] & 0xffffu) | (lo[3] << 16);
  x.z = (hi[0] & 0xffffu) | (hi[1] << 16);
  x.w = (hi[2] & 0xffffu) | (hi[3] << 16);
  return x;
}

// Workgroup (r, s): stage slice s of rank r's payload as tagged words, then
// poll slice s of all R ranks' tagged payloads and fold it in rank order into
// rank r's output.  stats.retries counts poll rounds that found a word not yet
// tagged (lane 0 of each workgroup).  CU / kLU: payload vectors per lane per
// consume / stage pass (one each when a slice is one vector per lane).
template <int R, bool BF16, int CU, int kLU>
__global__ void __launch_bounds__(64) lamport_chain_kernel(SnacArgs a) {
  const int r = blockIdx.x / a.S;
  const int s = blockIdx.x - r * a.S;
  const int bs = blockDim.x;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_vec;
  const int64_t v1 = min(a.nvec, v0 + a.slice_vec);
  const int64_t tbytes = 2 * a.rank_bytes;  // tagged bytes per rank
  unsigned long long polls = 0, timeouts = 0, done_epochs = 0;

  for (int k = 0; k < a.epochs; ++k) {
    const uint32_t ep = a.epoch0 + static_cast<uint32_t>(k);
    const uint32_t T = (ep & 0xffffu) << 16;
    unsigned char *tb = a.tagged + static_cast<int64_t>(ep & 1u) * R * tbytes;

    // Test hook: a late rank.
    if (a.stagger) {
      const uint32_t d = a.stagger[r];
      for (uint32_t i = 0; i < d; ++i) __builtin_amdgcn_s_sleep(1);
    }

    // Stage: the store is the notification.
    const unsigned char *src = a.in + (static_cast<int64_t>(k) * R + r) * a.rank_bytes;
    const __amdgpu_buffer_rsrc_t mine = rsrc(tb + static_cast<int64_t>(r) * tbytes, tbytes);
    for (int64_t i0 = v0 + threadIdx.x; i0 < v1; i0 += static_cast<int64_t>(bs) * kLU) {
      v4u x[kLU];
#pragma unroll
      for (int u = 0; u < kLU; ++u) {
        const int64_t i = i0 + static_cast<int64_t>(u) * bs;
        if (i < v1) x[u] = *reinterpret_cast<const v4u *>(src + i * 16);
      }
#pragma unroll
      for (int u = 0; u < kLU; ++u) {
        const int64_t i = i0 + static_cast<int64_t>(u) * bs;
        if (i < v1) {
          v4u lo, hi;
          tag_halves(x[u], T, lo, hi);
          store_tagged(mine, static_cast<int32_t>(i * 32), lo);
          store_tagged(mine, static_cast<int32_t>(i * 32 + 16), hi);
        }
      }
    }

    // From kLamportSettleVec vectors per rank the first poll waits until this
    // lane's own tagged stores are acknowledged: issued right behind them it
    // samples the other ranks' words too early and is mostly polled again
    // (measured on MI355X, 8 ranks, 64-deep chains, us per All-Reduce:
    // 64 KiB 3.74 -> 3.18, 512 KiB 13.5 -> 12.0; below 64 KiB the wait cost
    // more than it saved, 8 KiB 1.77 -> 2.17).
    if (a.nvec >= kLamportSettleVec) {
      __builtin_amdgcn_s_waitcnt(0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
    // Consume: poll until every word this lane needs carries the tag, then
    // fold in rank order.
    unsigned char *dst = a.out + (static_cast<int64_t>(k) * R + r) * a.rank_bytes;
    bool ok = true;
    for (int64_t i0 = v0 + threadIdx.x; i0 < v1; i0 += static_cast<int64_t>(bs) * CU) {
      v4u lo[CU][R], hi[CU][R];
      uint32_t spins = 0;
      while (true) {
        bool ready = true;
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int64_t i = i0 + static_cast<int64_t>(u) * bs;
          if (i < v1) {
#pragma unroll
            for (int q = 0; q < R; ++q) {
              const __amdgpu_buffer_rsrc_t src_q = rsrc(tb + static_cast<int64_t>(q) * tbytes, tbytes);
              lo[u][q] = load_tagged(src_q, static_cast<int32_t>(i * 32));
              hi[u][q] = load_tagged(src_q, static_cast<int32_t>(i * 32 + 16));
            }
          }
        }
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int64_t i = i0 + static_cast<int64_t>(u) * bs;
          if (i < v1) {
#pragma unroll
            for (int q = 0; q < R; ++q)
              ready = ready && tagged_with(lo[u][q], T) && tagged_with(hi[u][q], T);
          }
        }
        if (ready) break;
        ++polls;
        if ((spins & 63) == 0 && load_flag_relaxed(a.status) != 0) {
          ok = false;
          break;
        }
        if (++spins >= a.spin_limit) {
          __hip_atomic_store(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (!ok) break;
#pragma unroll
      for (int u = 0; u < CU; ++u) {
        const int64_t i = i0 + static_cast<int64_t>(u) * bs;
        if (i < v1) {
          uint4 v[R];
#pragma unroll
          for (int q = 0; q < R; ++q) v[q] = untag(lo[u][q], hi[u][q]);
          // No fences here, so the output keeps plain stores.
          *reinterpret_cast<uint4 *>(dst + i * 16) = BF16 ? fold_bf16x8<R>(v) : fold_f32x4<R>(v);
        }
      }
    }
    // Every lane leaves together once any lane gave up.
    if (__any(!ok)) {
      ++timeouts;
      break;
    }
    ++done_epochs;
  }

  if (a.stats && threadIdx.x == 0) {
    if (polls) atomicAdd(&a.stats->retries, polls);
    if (timeouts) atomicAdd(&a.stats->timeouts, timeouts);
    atomicAdd(&a.stats->epochs, done_epochs);
  }
}

// ---- chains of any uniform plan ---------------------------------------------
//
// The same stage / notify / consume orchestration over a plan's index map
// (Purlin news page, "The Purlin PDF describes a three-layer design": the
// orchestration layer stays the same while the collective changes).
// Workgroup (r, s) stages slice s of rank r's input, publishes
// flag[buf][r][s] = epoch, then computes piece s of every map entry whose
// output is rank r (a copy from one staged rank, or a rank-order fold over
// all of them).  Its top barrier waits for the flags on its wait list (built
// at plan time, build_wait_lists): the slices its pieces read, and the
// workgroups whose pieces read its own slice -- with two buffers the latter
// proves that every reader of this workgroup's slice finished the previous
// epoch on this buffer, the write-after-read guard of dual buffering.
// Speculation reads the listed flags first, then consumes with
// device-coherent loads and keeps the result only if they summed to
// (list length) x epoch; otherwise it waits and consumes again (outputs are
// only read after the kernel).

struct PlanChainArgs {
  const unsigned char *in;   // [E][R][in_stride bytes]
  unsigned char *out;        // [E][R][out_stride bytes]
  unsigned char *staging;    // [2][R][in_stride bytes]
  uint32_t *flag;            // [2][R][S] x kFlagStride
  uint32_t *done;            // [R][S] x kFlagStride
  uint32_t *status;
  rrb_snac_stats *stats;
  const uint32_t *stagger;
  const PlanEntry *entries;  // rank r's entries at [first[r], first[r] + cnt[r])
  // Workgroup w waits on the flags wait_idx[wait_off[w] .. wait_off[w + 1]),
  // each a flag index r * S + s: the slices its consume reads and the
  // workgroups that read its own slice.
  const int32_t *wait_off;
  const int32_t *wait_idx;
  int64_t in_stride, out_stride;
  int64_t slice_vec;         // staging slice length in vectors
  int64_t in_vec[RRB_MAX_RANKS];
  int32_t first[RRB_MAX_RANKS], cnt[RRB_MAX_RANKS];
  // Vectors per entry when all of a rank's entries are copies of one length,
  // else 0.
  int64_t copy_len[RRB_MAX_RANKS];
  uint32_t epoch0;
  int32_t epochs;
  int32_t S;
  uint32_t spin_limit;
};

// A wait-list entry is a flag index r * S + s; entries that only guard the
// write-after-read order (a workgroup that reads this workgroup's slice, but
// whose own slice this workgroup does not read) also carry kGuardOnly.
constexpr int32_t kGuardOnly = 1 << 30;
constexpr int32_t kFlagIndexMask = kGuardOnly - 1;

// Every lane waits for its share of the n flags base + idx[i] * kFlagStride
// (no acquire fence: the staged data is read with device-coherent loads after
// the flags were seen).  True in every lane if all n waits succeeded.
__device__ bool wait_list(const uint32_t *base, const int32_t *idx, int n, uint32_t want,
                          uint32_t *status, uint32_t limit) {
  bool ok = true;
  for (int i = threadIdx.x; i < n && ok; i += blockDim.x)
    ok = wait_at_least(base + static_cast<int64_t>(idx[i] & kFlagIndexMask) * kFlagStride, want, status,
                       limit);
  const bool all = __all(ok) != 0;
  acquire_if_fenced();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return all;
}

// Piece s of the entries of rank r that read a rank in `stale` (a copy from
// such a rank, or any fold when `stale` is not empty) if `touching`, else of
// the others: staged data read with device-coherent loads, results stored to
// rank r's output of this epoch with plain stores (only the host reads
// outputs).  stale = 0 with touching = false selects every entry; the
// speculative consume runs the two halves on either side of its wait.
//
// The rank's entries are read from LDS (`ents`, at most kFlatEntries).  A
// rank whose entries are all copies of one length (All-Gather, All-to-All,
// Gather) takes its pieces as one flat index range over all lanes, kCopyU
// vectors per lane in flight: a pass per entry put the entries' round trips
// one after another, with most lanes idle when a piece is narrower than the
// workgroup.
constexpr int kFlatEntries = 64;

// A workgroup's piece [lo, hi) of one map entry, in vectors: slice s of the
// entry's ceil(len / S)-vector pieces.  Computed once per kernel, so no epoch
// divides.
struct Piece {
  int64_t lo, hi;
};

template <int R, bool BF16>
__device__ void plan_consume(const PlanChainArgs &a, int r, const unsigned char *stage_base,
                             unsigned char *dst, const PlanEntry *ents, const Piece *pieces,
                             uint32_t stale, bool touching) {
  const int bs = blockDim.x;
  constexpr int CU = R <= 8 ? 2 : 1;
  constexpr int CC = 4;  // copy vectors per lane in flight
  if (a.copy_len[r] > 0) {
    const int64_t lo = pieces[0].lo;  // every entry has the same piece
    const uint32_t w = static_cast<uint32_t>(pieces[0].hi - lo);
    const uint32_t total = static_cast<uint32_t>(a.cnt[r]) * w;
    // One descriptor over every rank's staged payload of this buffer.
    const __amdgpu_buffer_rsrc_t src = rsrc(stage_base, static_cast<int64_t>(R) * a.in_stride);
    for (uint32_t f0 = threadIdx.x; f0 < total; f0 += static_cast<uint32_t>(bs) * kCopyU) {
      uint4 x[kCopyU];
      int64_t at[kCopyU];
#pragma unroll
      for (int u = 0; u < kCopyU; ++u) {
        const uint32_t f = f0 + static_cast<uint32_t>(u * bs);
        at[u] = -1;
        if (f < total) {
          const uint32_t g = f / w;
          const PlanEntry e = ents[g];
          if ((stale >> e.src_rank & 1u) == static_cast<uint32_t>(touching)) {
            const int64_t i = lo + (f - g * w);
            x[u] = load_coherent(src, static_cast<int32_t>(e.src_rank * a.in_stride + (e.src_off + i) * 16));
            at[u] = (e.dst_off + i) * 16;
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kCopyU; ++u)
        if (at[u] >= 0) *reinterpret_cast<uint4 *>(dst + at[u]) = x[u];
    }
    return;
  }
  for (int g = 0; g < a.cnt[r]; ++g) {
    const PlanEntry e = ents[g];
    if ((e.src_rank < 0 ? stale != 0 : (stale >> e.src_rank & 1u) != 0) != touching) continue;
    const int64_t lo = pieces[g].lo;
    const int64_t hi = pieces[g].hi;
    if (e.src_rank < 0) {
      for (int64_t i0 = lo + threadIdx.x; i0 < hi; i0 += static_cast<int64_t>(bs) * CU) {
        uint4 v[CU][R];
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int64_t i = i0 + static_cast<int64_t>(u) * bs;
          if (i < hi) {
#pragma unroll
            for (int q = 0; q < R; ++q)
              v[u][q] = load_coherent(rsrc(stage_base + static_cast<int64_t>(q) * a.in_stride,
                                           a.in_stride),
                                      static_cast<int32_t>((e.src_off + i) * 16));
          }
        }
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int64_t i = i0 + static_cast<int64_t>(u) * bs;
          if (i < hi) reduce_pass<R, BF16, false>(v[u], dst, a.out_stride, (e.dst_off + i) * 16);
        }
      }
    } else {
      const __amdgpu_buffer_rsrc_t src =
          rsrc(stage_base + static_cast<int64_t>(e.src_rank) * a.in_stride, a.in_stride);
      for (int64_t i0 = lo + threadIdx.x; i0 < hi; i0 += static_cast<int64_t>(bs) * CC) {
        uint4 x[CC];
#pragma unroll
        for (int u = 0; u < CC; ++u) {
          const int64_t i = i0 + static_cast<int64_t>(u) * bs;
          if (i < hi) x[u] = load_coherent(src, static_cast<int32_t>((e.src_off + i) * 16));
        }
#pragma unroll
        for (int u = 0; u < CC; ++u) {
          const int64_t i = i0 + static_cast<int64_t>(u) * bs;
          if (i < hi) *reinterpret_cast<uint4 *>(dst + (e.dst_off + i) * 16) = x[u];
        }
      }
    }
  }
}

// The speculative consume of a workgroup whose work fits one round: the
// rank's copies at most kCopyU vectors per lane, or its one fold at most CU.
// Its addresses are worked out once per kernel (SpecPrep), so after the flag
// read only the loads remain: the flag read's ordering barrier keeps every
// instruction after it, and address work left there lengthened each epoch.
struct SpecPrep {
  int kind;  // 0: consume in two parts, 1: flat copies in one round, 2: one fold in one round
  int32_t off[kCopyU];   // copies: source byte offsets in the staged buffers
  int32_t rank[kCopyU];  // copies: source ranks
  int64_t at[kCopyU];    // copies: destination byte offsets, -1 for none
  int64_t src_off, dst_off, lo, hi;  // fold: the entry and this workgroup's piece
};

template <int R>
__device__ __forceinline__ void spec_prepare(const PlanChainArgs &a, int r, const PlanEntry *ents,
                                             const Piece *pieces, SpecPrep &p) {
  const int bs = blockDim.x;
  constexpr int CU = R <= 8 ? 2 : 1;
  p.kind = 0;
  p.src_off = p.dst_off = p.lo = p.hi = 0;
#pragma unroll
  for (int u = 0; u < kCopyU; ++u) {
    p.off[u] = 0;
    p.rank[u] = 0;
    p.at[u] = -1;
  }
  if (a.copy_len[r] > 0) {
    const int64_t lo = pieces[0].lo;  // every entry has the same piece
    const uint32_t w = static_cast<uint32_t>(pieces[0].hi - lo);
    const uint32_t total = static_cast<uint32_t>(a.cnt[r]) * w;
    if (total > static_cast<uint32_t>(bs) * kCopyU) return;
    p.kind = 1;
#pragma unroll
    for (int u = 0; u < kCopyU; ++u) {
      const uint32_t f = threadIdx.x + static_cast<uint32_t>(u * bs);
      if (f < total) {
        const uint32_t g = f / w;
        const PlanEntry e = ents[g];
        const int64_t i = lo + (f - g * w);
        p.off[u] = static_cast<int32_t>(e.src_rank * a.in_stride + (e.src_off + i) * 16);
        p.rank[u] = e.src_rank;
        p.at[u] = (e.dst_off + i) * 16;
      }
    }
    return;
  }
  if (a.cnt[r] != 1) return;
  const PlanEntry e = ents[0];
  if (e.src_rank >= 0) return;
  if (pieces[0].hi - pieces[0].lo > static_cast<int64_t>(bs) * CU) return;
  p.kind = 2;
  p.src_off = e.src_off;
  p.dst_off = e.dst_off;
  p.lo = pieces[0].lo;
  p.hi = pieces[0].hi;
}

// Every source is loaded once the flag values have returned.  After a failed
// sum the workgroup waits for its list and loads the stale ranks' sources
// again; the current ones' data stays in registers, so the wait overlaps
// their loads.  Outputs are stored once, after that.  Returns 0 when the work
// does not fit one round (the caller consumes in two parts around the wait),
// 1 when done, -1 when a wait ran out.
template <int R, bool BF16>
__device__ int plan_consume_spec(const PlanChainArgs &a, const SpecPrep &p, const unsigned char *stage_base,
                                 unsigned char *dst, const uint32_t *flags_b, const int32_t *wl, int nw,
                                 uint32_t ep, bool valid, uint32_t stale) {
  const int bs = blockDim.x;
  constexpr int CU = R <= 8 ? 2 : 1;
  if (p.kind == 1) {
    const __amdgpu_buffer_rsrc_t src = rsrc(stage_base, static_cast<int64_t>(R) * a.in_stride);
    uint4 x[kCopyU];
#pragma unroll
    for (int u = 0; u < kCopyU; ++u)
      if (p.at[u] >= 0) x[u] = load_coherent(src, p.off[u]);
    if (!valid) {
      if (!wait_list(flags_b, wl, nw, ep, a.status, a.spin_limit)) return -1;
      order_after_values();
#pragma unroll
      for (int u = 0; u < kCopyU; ++u)
        if (p.at[u] >= 0 && (stale >> p.rank[u] & 1u)) x[u] = load_coherent(src, p.off[u]);
    }
#pragma unroll
    for (int u = 0; u < kCopyU; ++u)
      if (p.at[u] >= 0) *reinterpret_cast<uint4 *>(dst + p.at[u]) = x[u];
    return 1;
  }
  if (p.kind != 2) return 0;
  uint4 v[CU][R];
#pragma unroll
  for (int u = 0; u < CU; ++u) {
    const int64_t i = p.lo + threadIdx.x + static_cast<int64_t>(u) * bs;
    if (i < p.hi) {
#pragma unroll
      for (int q = 0; q < R; ++q)
        v[u][q] = load_coherent(rsrc(stage_base + static_cast<int64_t>(q) * a.in_stride, a.in_stride),
                                static_cast<int32_t>((p.src_off + i) * 16));
    }
  }
  if (!valid) {
    if (!wait_list(flags_b, wl, nw, ep, a.status, a.spin_limit)) return -1;
    order_after_values();
#pragma unroll
    for (int q = 0; q < R; ++q) {
      if (stale >> q & 1u) {
#pragma unroll
        for (int u = 0; u < CU; ++u) {
          const int64_t i = p.lo + threadIdx.x + static_cast<int64_t>(u) * bs;
          if (i < p.hi)
            v[u][q] = load_coherent(rsrc(stage_base + static_cast<int64_t>(q) * a.in_stride, a.in_stride),
                                    static_cast<int32_t>((p.src_off + i) * 16));
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < CU; ++u) {
    const int64_t i = p.lo + threadIdx.x + static_cast<int64_t>(u) * bs;
    if (i < p.hi) reduce_pass<R, BF16, false>(v[u], dst, a.out_stride, (p.dst_off + i) * 16);
  }
  return 1;
}

template <int R, bool BF16, int VAR>
__global__ void __launch_bounds__(64) snac_plan_kernel(PlanChainArgs a) {
  const int r = blockIdx.x / a.S;
  const int s = blockIdx.x - r * a.S;
  const int bs = blockDim.x;
  const int64_t v0 = static_cast<int64_t>(s) * a.slice_vec;
  const int64_t v1 = min(a.in_vec[r], v0 + a.slice_vec);
  const int32_t w0 = a.wait_off[blockIdx.x];
  const int nw = a.wait_off[blockIdx.x + 1] - w0;
  const int32_t *wl = a.wait_idx + w0;
  unsigned long long misspec = 0, retries = 0, timeouts = 0, done_epochs = 0;
  // The rank's map entries (at most kFlatEntries, checked at plan time),
  // copied to LDS once, so no epoch waits on a global load for them.
  __shared__ PlanEntry ents[kFlatEntries];
  __shared__ Piece pieces[kFlatEntries];
  for (int g = threadIdx.x; g < a.cnt[r]; g += bs) {
    const PlanEntry e = a.entries[a.first[r] + g];
    const int64_t pl = (e.len + a.S - 1) / a.S;
    const int64_t lo = min(e.len, static_cast<int64_t>(s) * pl);
    ents[g] = e;
    pieces[g] = Piece{lo, min(e.len, lo + pl)};
  }
  __syncthreads();
  SpecPrep prep;
  if (VAR == kSpeculative) spec_prepare<R>(a, r, ents, pieces, prep);

  for (int k = 0; k < a.epochs; ++k) {
    const uint32_t ep = a.epoch0 + static_cast<uint32_t>(k);
    const int b = VAR == kBarrier ? 0 : static_cast<int>(ep & 1u);
    unsigned char *stage_base = a.staging + static_cast<int64_t>(b) * R * a.in_stride;
    uint32_t *flags_b = a.flag + static_cast<int64_t>(b) * R * a.S * kFlagStride;

    // Test hook: a late rank.
    if (a.stagger) {
      const uint32_t d = a.stagger[r];
      for (uint32_t i = 0; i < d; ++i) __builtin_amdgcn_s_sleep(1);
    }

    // Stage slice s of rank r's input.
    stage_slice(a.in + (static_cast<int64_t>(k) * R + r) * a.in_stride,
                stage_base + static_cast<int64_t>(r) * a.in_stride, a.in_stride, v0, v1);

    // Notify.
    notify<false>(flags_b + (static_cast<int64_t>(r) * a.S + s) * kFlagStride, ep);

    unsigned char *dst = a.out + (static_cast<int64_t>(k) * R + r) * a.out_stride;
    bool ok = true;
    if (VAR == kSpeculative && a.cnt[r] > 0) {
      // One read of the listed flags; once their values have returned, the
      // consume runs.  The reduced check covers the data flags (the slices
      // this workgroup's pieces read).  Each holds epoch or epoch - 2, so
      // their sum equals (their count) x epoch exactly when every one shows
      // the epoch; the check is taken in that form, as a count of the lanes
      // whose flag shows the epoch (two ballots), which cost 0.15-0.36 us
      // less per collective than summing the flags lane by lane through
      // scalar registers (a loop of v_readlane over the list).  Work that
      // fits one round loads every source at once and, on a mismatch, waits
      // for every listed flag and loads only the stale ranks' sources again
      // (plan_consume_spec).  Larger work leaves out the entries that read a
      // rank whose data flag read stale (copies from it, and every fold: a
      // fold run too early would be redone whole), waits, and then runs
      // those.  Either way the current sources' loads were issued after
      // their flags showed the epoch.  A write-after-read guard that read
      // stale holds back nothing of this epoch; it is waited for after the
      // consume, before the next stage.
      uint32_t stale = 0;
      int ndata = 0, ncur = 0;
      bool guard_late = false;
      for (int i0 = 0; i0 < nw; i0 += bs) {
        const int i = i0 + static_cast<int>(threadIdx.x);
        int32_t w = 0;
        uint32_t f = ep;
        if (i < nw) {
          w = wl[i];
          f = load_flag_relaxed(flags_b + static_cast<int64_t>(w & kFlagIndexMask) * kFlagStride);
        }
        const bool data = i < nw && !(w & kGuardOnly);
        ncur += __builtin_popcountll(__ballot(data && f == ep));
        ndata += __builtin_popcountll(__ballot(data));
        guard_late = guard_late || __ballot(i < nw && (w & kGuardOnly) && f != ep) != 0;
        // Lanes holding a stale data flag: their ranks' entries wait.
        for (uint64_t bad = __ballot(data && f != ep); bad; bad &= bad - 1) {
          const int l = __builtin_ctzll(bad);
          stale |= 1u << ((__builtin_amdgcn_readlane(w, l) & kFlagIndexMask) / a.S);
        }
      }
      order_after_values();
      const bool valid = ncur == ndata;
      if (!valid) {
        ++misspec;
        retries += static_cast<unsigned long long>(__builtin_popcount(stale));
      }
      const int one = plan_consume_spec<R, BF16>(a, prep, stage_base, dst, flags_b, wl, nw, ep, valid, stale);
      if (one < 0) {
        ok = false;
      } else if (one == 0) {
        plan_consume<R, BF16>(a, r, stage_base, dst, ents, pieces, stale, false);
        if (!valid) {
          ok = wait_list(flags_b, wl, nw, ep, a.status, a.spin_limit);
          if (ok) {
            order_after_values();
            if (stale) plan_consume<R, BF16>(a, r, stage_base, dst, ents, pieces, stale, true);
          }
        }
      }
      // A failed check already waited for the whole list.
      if (ok && valid && guard_late) ok = wait_list(flags_b, wl, nw, ep, a.status, a.spin_limit);
    } else {
      // (A speculative workgroup with no map entries only guards: it waits.)
      ok = wait_list(flags_b, wl, nw, ep, a.status, a.spin_limit);
      if (ok) plan_consume<R, BF16>(a, r, stage_base, dst, ents, pieces, 0u, false);
    }
    if (!ok) {
      ++timeouts;
      break;
    }
    if (VAR == kBarrier) {
      // Bottom barrier: every reader of this workgroup's slice is done.
      notify<false>(a.done + (static_cast<int64_t>(r) * a.S + s) * kFlagStride, ep);
      if (!wait_list(a.done, wl, nw, ep, a.status, a.spin_limit)) {
        ++timeouts;
        break;
      }
    }
    ++done_epochs;
  }

  if (a.stats && threadIdx.x == 0) {
    if (misspec) atomicAdd(&a.stats->misspec, misspec);
    if (retries) atomicAdd(&a.stats->retries, retries);
    if (timeouts) atomicAdd(&a.stats->timeouts, timeouts);
    atomicAdd(&a.stats->epochs, done_epochs);
  }
}

using PlanChainFn = void (*)(PlanChainArgs);

template <bool BF16, int VAR>
PlanChainFn snac_plan_for(int R) {
  switch (R) {
#define RRB_CASE(n) \
  case n:           \
    return snac_plan_kernel<n, BF16, VAR>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8) RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13)
    RRB_CASE(14) RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
  }
  return nullptr;
}

// Single-wave workgroups per rank: the caller's count, or chosen from the
// payload's vectors.
int32_t default_slices(int32_t slices, int64_t nvec, int32_t nranks, uint32_t flags, bool plan) {
  int32_t S = slices;
  if (S == 0) {
    if (flags & RRB_SNAC_LAMPORT) {
      // Flag-in-data has no fences; its time follows the coherent loads per
      // lane, so small payloads take one vector per lane (64 per workgroup),
      // then 32 per workgroup; above 256 KiB, 128 workgroups per rank (more
      // of them only add poll traffic).  Measured on MI355X, 8 ranks.
      if (nvec < 4096) {
        S = static_cast<int32_t>(std::max<int64_t>(1, nvec / 64));
      } else if (nvec <= 16384) {
        S = static_cast<int32_t>(std::min<int64_t>(256, nvec / 32));
      } else {
        S = 128;
      }
    } else if (!plan) {
      // Barrier, dual, speculative and twoshot All-Reduce chains: 64 vectors
      // per workgroup, up to 128 workgroups per rank, and 256 from 512 KiB
      // per rank.  Measured on MI355X, 8 ranks, us per All-Reduce by slices
      // per rank (two interleaved runs where two figures are given):
      //   dual     8 KiB    4: 2.82  8: 2.04  16: 2.11  32: 2.12
      //            32 KiB   16: 2.59  32: 2.13  64: 2.13  128: 2.37
      //            128 KiB  64: 2.81  128: 2.47  256: 3.18
      //            256 KiB  128: 3.33 / 3.47  256: 3.39 / 3.35
      //            512 KiB  128: 5.42 / 5.27  256: 5.01 / 5.01
      //            1 MiB    128: 8.67 / 8.36  256: 7.77 / 7.75
      //   twoshot  512 KiB  128: 7.16 / 7.19  256: 6.67 / 6.70
      //            1 MiB    128: 10.59 / 10.69  256: 9.02 / 9.06
      // (barrier and speculative follow dual).  Before the chains dropped
      // their fences, every extra workgroup added fence time and 8-32 per
      // rank were best; before the flag store settled (notify), 128 per rank
      // led at 1 MiB.
      S = nvec >= 32768 ? 256
                        : static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(128, nvec / 64)));
      // Speculation held at every size keeps 128 per rank: its kernel (244
      // VGPRs) fits 1024 workgroups in half the device, not 2048 (512 KiB:
      // 5.54 us at 128 against 5.72 at 256 cooperatively launched; 1 MiB:
      // 8.45 against 8.05).
      if ((flags & RRB_SNAC_SPEC_ALWAYS) && S > 128) S = 128;
    } else {
      // Plan chains: 64 vectors (of the larger of a rank's input and output)
      // per workgroup, up to 128 per rank.  Dual buffer, 8 ranks, us per
      // collective by slices per rank, measured on MI355X:
      //   512 KiB tensor  64: All-Reduce 6.91  All-Gather 4.32  All-to-All
      //                   6.25  Broadcast 4.53  Reduce 6.77  Gather 4.08
      //                   Reduce-Scatter 4.71
      //                  128: 5.50  3.40  5.50  3.50  4.88  3.07  4.75
      //   128 KiB tensor  64: 2.88  2.43  3.26  2.53  3.03  2.44  3.35
      //                  128: 2.87  2.38  3.25  2.30  2.77  2.42  3.53
      // (256 per rank was mixed at 512 KiB and slower at 128 KiB; 16 KiB
      // tensors, 16 per rank, were best or within 0.03 us.)
      S = static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(128, nvec / 64)));
    }
    if (kFences && !(flags & RRB_SNAC_LAMPORT)) {
      // The memory-model build writes back and invalidates an XCD's L2 per
      // workgroup and epoch, so fewer, larger workgroups: 64 vectors each,
      // up to 16 per rank below 128 KiB and 32 from there.  Measured on
      // MI355X, 8 ranks, dual, us per All-Reduce by slices per rank:
      //   8 KiB    4: 2.81  8: 2.50  16: 3.05
      //   32 KiB   8: 4.01  16: 3.83  32: 4.77
      //   128 KiB  16: 6.85  32: 6.79  64: 11.9  (128: 21.8)
      //   512 KiB  16: 21.5  32: 15.4  64: 17.9  (256: 65.9)
      // (barrier, speculative and twoshot follow dual within 10-30%).
      S = static_cast<int32_t>(
          std::max<int64_t>(1, std::min<int64_t>(nvec >= 8192 ? 32 : 16, nvec / 64)));
    }
    S = std::min<int32_t>(S, 2048 / nranks);
  }
  if (S > nvec) S = static_cast<int32_t>(nvec);
  return S;
}

__global__ void fill_u32_kernel(uint32_t *p, int64_t n, uint32_t v) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = v;
}

using SnacFn = void (*)(SnacArgs);

template <bool BF16, int VAR>
SnacFn snac_for(int R) {
  switch (R) {
#define RRB_CASE(n) \
  case n:           \
    if constexpr (VAR == kLamport) return lamport_chain_kernel<n, BF16, (n <= 8 ? 2 : 1), 4>; \
    else if constexpr (VAR == kLamportOne) return lamport_chain_kernel<n, BF16, 1, 1>; \
    else return snac_chain_kernel<n, BF16, VAR>;
    RRB_CASE(1) RRB_CASE(2) RRB_CASE(3) RRB_CASE(4) RRB_CASE(5) RRB_CASE(6) RRB_CASE(7)
    RRB_CASE(8) RRB_CASE(9) RRB_CASE(10) RRB_CASE(11) RRB_CASE(12) RRB_CASE(13)
    RRB_CASE(14) RRB_CASE(15) RRB_CASE(16)
#undef RRB_CASE
  }
  return nullptr;
}

}  // namespace
}  // namespace rrb

struct rrb_snac_s {
  int32_t R = 0;
  int64_t count = 0;
  int32_t dtype = RRB_BF16;
  uint32_t flags = 0;
  int32_t S = 1;
  int bs = 64;
  rrb::Layout lay{};
  unsigned char *ws = nullptr;
  uint32_t next_epoch = 1;
  // Bytes per rank per epoch in d_in / d_out (count * elem size for an
  // All-Reduce handle).
  int64_t in_stride = 0, out_stride = 0;
  // Chains of a plan (rrb_snac_create_plan): the consume entries per rank.
  bool from_plan = false;
  std::vector<rrb::PlanEntry> entries;
  // Per workgroup wait lists: R*S + 1 offsets, then the flag indices.
  std::vector<int32_t> wait_tab;
  int64_t slice_vec = 0;  // staging slice length in vectors
  int64_t in_vec[RRB_MAX_RANKS] = {};
  int32_t first[RRB_MAX_RANKS] = {}, cnt[RRB_MAX_RANKS] = {};
  int64_t copy_len[RRB_MAX_RANKS] = {};
  // Co-resident capacity (workgroups) of the last two persistent kernels
  // asked about.
  const void *cap_fn[2] = {nullptr, nullptr};
  int64_t cap[2] = {0, 0};
  // RRB_SNAC_GRAPH: one Atom All-Reduce kernel node per epoch, chained in a
  // HIP graph that is cached for the last (in, out, epochs).
  rrb::Plan ar_plan;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  const void *g_in = nullptr;
  void *g_out = nullptr;
  int32_t g_epochs = 0;
  std::vector<rrb::LaunchDesc> g_descs;

  void drop_graph() {
    if (exec) (void)hipGraphExecDestroy(exec);
    if (graph) (void)hipGraphDestroy(graph);
    exec = nullptr;
    graph = nullptr;
    g_in = nullptr;
    g_out = nullptr;
    g_epochs = 0;
    g_descs.clear();
  }
  ~rrb_snac_s() { drop_graph(); }
};

namespace rrb {
namespace {

// Wait lists of a plan chain.  Workgroup w = r * S + s consumes piece s of
// each of rank r's entries (the same piece bounds as plan_consume); reads(w)
// is the set of staging slices (q, s') those pieces touch.  w waits for
// reads(w) (its data is staged) and for every workgroup whose reads include
// w's own slice (they finished the previous epoch on this buffer before w
// stages over it).  The relation is symmetric, so no workgroup on w's list
// gets two epochs ahead of w, and with two buffers every flag w reads holds
// epoch or epoch - 2: the speculative sum check stays exact.
void build_wait_lists(rrb_snac_s &h) {
  const int R = h.R, S = h.S;
  const int W = R * S;
  std::vector<std::vector<int32_t>> lists(W);
  for (int r = 0; r < R; ++r) {
    for (int s = 0; s < S; ++s) {
      std::vector<int32_t> &l = lists[r * S + s];
      for (int g = h.first[r]; g < h.first[r] + h.cnt[r]; ++g) {
        const PlanEntry &e = h.entries[g];
        const int64_t pl = (e.len + S - 1) / S;
        const int64_t lo = std::min(e.len, static_cast<int64_t>(s) * pl);
        const int64_t hi = std::min(e.len, lo + pl);
        if (lo >= hi) continue;
        const int64_t s0 = (e.src_off + lo) / h.slice_vec;
        const int64_t s1 = (e.src_off + hi - 1) / h.slice_vec;
        for (int q = 0; q < R; ++q) {
          if (e.src_rank >= 0 && q != e.src_rank) continue;
          for (int64_t sp = s0; sp <= s1 && sp < S; ++sp) l.push_back(q * S + static_cast<int32_t>(sp));
        }
      }
      std::sort(l.begin(), l.end());
      l.erase(std::unique(l.begin(), l.end()), l.end());
    }
  }
  // Add the readers of each slice to that slice's own list.
  std::vector<std::vector<int32_t>> readers(W);
  for (int w = 0; w < W; ++w)
    for (int32_t f : lists[w]) readers[f].push_back(w);
  h.wait_tab.assign(1, 0);
  std::vector<int32_t> all;
  for (int w = 0; w < W; ++w) {
    std::vector<int32_t> m = lists[w];
    for (int32_t f : readers[w])
      if (!std::binary_search(lists[w].begin(), lists[w].end(), f)) m.push_back(f | kGuardOnly);
    std::sort(m.begin(), m.end(), [](int32_t x, int32_t y) {
      return (x & kFlagIndexMask) < (y & kFlagIndexMask);
    });
    m.erase(std::unique(m.begin(), m.end()), m.end());
    all.insert(all.end(), m.begin(), m.end());
    h.wait_tab.push_back(static_cast<int32_t>(all.size()));
  }
  h.wait_tab.insert(h.wait_tab.end(), all.begin(), all.end());
}

// Builds the chain's graph: epoch e's All-Reduce reads in[e][0..R-1] and
// writes out[e][0..R-1]; each epoch's kernels depend on the previous ones,
// as a decode step's All-Reduces do.
rrb_status build_chain_graph(rrb_snac_s *h, int32_t epochs, const void *d_in, void *d_out) {
  h->drop_graph();
  hipError_t e = hipGraphCreate(&h->graph, 0);
  if (e != hipSuccess) return fail(RRB_EHIP, "graph create: %s", hipGetErrorString(e));
  std::vector<const void *> in(h->R);
  std::vector<void *> out(h->R);
  for (int32_t k = 0; k < epochs; ++k) {
    for (int32_t r = 0; r < h->R; ++r) {
      in[r] = static_cast<const unsigned char *>(d_in) + (static_cast<int64_t>(k) * h->R + r) * h->in_stride;
      out[r] = static_cast<unsigned char *>(d_out) + (static_cast<int64_t>(k) * h->R + r) * h->out_stride;
    }
    const rrb_status st = describe_uniform(h->ar_plan, in.data(), out.data(), h->g_descs);
    if (st != RRB_OK) {
      h->drop_graph();
      return st;
    }
  }
  hipGraphNode_t prev = nullptr;
  for (LaunchDesc &d : h->g_descs) {
    hipKernelNodeParams np;
    std::memset(&np, 0, sizeof np);
    void *params[1] = {d.args.data()};
    np.func = const_cast<void *>(d.func);
    np.gridDim = d.grid;
    np.blockDim = d.block;
    np.sharedMemBytes = 0;
    np.kernelParams = params;
    np.extra = nullptr;
    hipGraphNode_t node = nullptr;
    e = hipGraphAddKernelNode(&node, h->graph, prev ? &prev : nullptr, prev ? 1 : 0, &np);
    if (e != hipSuccess) {
      h->drop_graph();
      return fail(RRB_EHIP, "graph kernel node: %s", hipGetErrorString(e));
    }
    prev = node;
  }
  e = hipGraphInstantiate(&h->exec, h->graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    h->drop_graph();
    return fail(RRB_EHIP, "graph instantiate: %s", hipGetErrorString(e));
  }
  h->g_in = d_in;
  h->g_out = d_out;
  h->g_epochs = epochs;
  return RRB_OK;
}

// Launches a chain kernel whose workgroups wait on each other, so the grid
// must be co-resident.  A grid within half the device's co-resident capacity
// for the kernel (occupancy limit x compute units, cached per handle) takes a
// plain launch.  Larger grids, and every launch with RRB_SNAC_COOPERATIVE,
// take a cooperative launch, which guarantees co-residency beside other work
// (or refuses) but costs about 13 us more per call on MI355X.  If other work
// keeps a plain-launched grid from becoming co-resident, its bounded waits
// run out and the call reports RRB_ETIMEOUT; it does not hang.
// Whether a persistent kernel `fn` of the handle's grid (R x S single-wave
// workgroups) takes a cooperative launch: when the grid exceeds half the
// device's co-resident capacity for fn (half, as a margin on the occupancy
// estimate).  The capacities of the last two kernels asked about are kept.
rrb_status needs_cooperative(rrb_snac_s *h, const void *fn, const char *what, bool *coop) {
  int slot = h->cap_fn[0] == fn ? 0 : h->cap_fn[1] == fn ? 1 : -1;
  if (slot < 0) {
    int dev = 0, cus = 0, per = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, fn, h->bs, 0);
    if (e != hipSuccess) return fail(RRB_EHIP, "%s occupancy query: %s", what, hipGetErrorString(e));
    h->cap_fn[1] = h->cap_fn[0];
    h->cap[1] = h->cap[0];
    h->cap_fn[0] = fn;
    h->cap[0] = static_cast<int64_t>(per) * cus;
    slot = 0;
  }
  *coop = 2 * static_cast<int64_t>(h->R) * h->S > h->cap[slot];
  return RRB_OK;
}

template <class Args>
rrb_status launch_persistent(rrb_snac_s *h, const void *fn, Args &a, hipStream_t stream,
                             const char *what) {
  const unsigned grid = static_cast<unsigned>(h->R * h->S);
  bool coop = (h->flags & RRB_SNAC_COOPERATIVE) != 0;
  if (!coop) {
    const rrb_status st = needs_cooperative(h, fn, what, &coop);
    if (st != RRB_OK) return st;
  }
  hipError_t e;
  if (coop) {
    void *args[] = {&a};
    e = hipLaunchCooperativeKernel(fn, dim3(grid), dim3(h->bs), args, 0, stream);
  } else {
    void *args[] = {&a};
    e = hipLaunchKernel(fn, dim3(grid), dim3(h->bs), args, 0, stream);
  }
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(RRB_EHIP, "%s launch: %s", what, hipGetErrorString(e));
  return RRB_OK;
}

// Issues one plan-chain call (the handle is bound and not in graph mode).
rrb_status launch_plan_chain(rrb_snac_s *h, int32_t epochs, const void *d_in, void *d_out,
                             rrb_snac_stats *d_stats, const uint32_t *d_stagger,
                             uint32_t spin_limit, rrb_stream_t stream) {
  PlanChainArgs a;
  std::memset(&a, 0, sizeof a);
  a.in = static_cast<const unsigned char *>(d_in);
  a.out = static_cast<unsigned char *>(d_out);
  a.staging = h->ws + h->lay.staging_off;
  a.flag = reinterpret_cast<uint32_t *>(h->ws + h->lay.flag_off);
  a.done = reinterpret_cast<uint32_t *>(h->ws + h->lay.done_off);
  a.status = reinterpret_cast<uint32_t *>(h->ws + h->lay.status_off);
  a.stats = d_stats;
  a.stagger = d_stagger;
  a.entries = reinterpret_cast<const PlanEntry *>(h->ws + h->lay.entries_off);
  a.wait_off = reinterpret_cast<const int32_t *>(h->ws + h->lay.waits_off);
  a.wait_idx = a.wait_off + (static_cast<int64_t>(h->R) * h->S + 1);
  a.in_stride = h->in_stride;
  a.out_stride = h->out_stride;
  for (int r = 0; r < h->R; ++r) {
    a.in_vec[r] = h->in_vec[r];
    a.first[r] = h->first[r];
    a.cnt[r] = h->cnt[r];
    a.copy_len[r] = h->copy_len[r];
  }
  a.slice_vec = h->slice_vec;
  a.epoch0 = h->next_epoch;
  a.epochs = epochs;
  a.S = h->S;
  a.spin_limit = spin_limit ? spin_limit : kDefaultSpin;
  const bool bf16 = h->dtype == RRB_BF16;
  // The memory-model build waits for the flags first: there the speculative
  // plan kernel trailed the dual wait at every tensor size measured (MI355X,
  // 8 ranks, 64-deep chains, 4-16 KiB tensors: 10-26% behind for five of the
  // seven collectives, level to 3% ahead for Broadcast, Reduce and Gather at
  // 4 KiB only).
  const int var = (h->flags & RRB_SNAC_SPECULATIVE) && !kFences ? kSpeculative
                  : (h->flags & (RRB_SNAC_DUAL_BUFFER | RRB_SNAC_SPECULATIVE)) ? kDual : kBarrier;
  PlanChainFn fn = nullptr;
  if (bf16)
    fn = var == kBarrier ? snac_plan_for<true, kBarrier>(h->R)
         : var == kDual  ? snac_plan_for<true, kDual>(h->R)
                         : snac_plan_for<true, kSpeculative>(h->R);
  else
    fn = var == kBarrier ? snac_plan_for<false, kBarrier>(h->R)
         : var == kDual  ? snac_plan_for<false, kDual>(h->R)
                         : snac_plan_for<false, kSpeculative>(h->R);
  const rrb_status st = launch_persistent(h, reinterpret_cast<const void *>(fn), a,
                                          static_cast<hipStream_t>(stream), "plan chain");
  if (st != RRB_OK) return st;
  h->next_epoch += static_cast<uint32_t>(epochs);
  return RRB_OK;
}

// Argument rules of an All-Reduce chain handle (rrb_snac_create).
rrb_status check_ar_chain_args(int32_t nranks, int64_t count, int32_t dtype, uint32_t flags,
                               int32_t slices) {
  if (nranks < 1 || nranks > RRB_MAX_RANKS)
    return fail(RRB_EINVAL, "nranks %d outside 1..%d", nranks, RRB_MAX_RANKS);
  if (dtype != RRB_BF16 && dtype != RRB_F32) return fail(RRB_EINVAL, "unknown dtype %d", dtype);
  if (flags & ~(RRB_SNAC_DUAL_BUFFER | RRB_SNAC_SPECULATIVE | RRB_SNAC_GRAPH | RRB_SNAC_TWOSHOT |
                RRB_SNAC_LAMPORT | RRB_SNAC_COOPERATIVE | RRB_SNAC_SPEC_ALWAYS))
    return fail(RRB_EINVAL, "unknown SNAC flags 0x%x", flags);
  if ((flags & RRB_SNAC_SPEC_ALWAYS) && !(flags & RRB_SNAC_SPECULATIVE))
    return fail(RRB_EINVAL, "RRB_SNAC_SPEC_ALWAYS goes with RRB_SNAC_SPECULATIVE");
  flags &= ~RRB_SNAC_SPEC_ALWAYS;
  if ((flags & RRB_SNAC_COOPERATIVE) && (flags & RRB_SNAC_GRAPH))
    return fail(RRB_EINVAL, "RRB_SNAC_GRAPH launches no persistent kernel");
  flags &= ~RRB_SNAC_COOPERATIVE;
  if ((flags & RRB_SNAC_LAMPORT) && flags != (RRB_SNAC_LAMPORT | RRB_SNAC_DUAL_BUFFER))
    return fail(RRB_EINVAL, "RRB_SNAC_LAMPORT goes with RRB_SNAC_DUAL_BUFFER only");
  if (kFences && (flags & RRB_SNAC_LAMPORT))
    return fail(RRB_EUNSUPPORTED, "the flag-in-data chain has no fenced build");
  if ((flags & RRB_SNAC_TWOSHOT) && flags != (RRB_SNAC_TWOSHOT | RRB_SNAC_DUAL_BUFFER))
    return fail(RRB_EINVAL, "RRB_SNAC_TWOSHOT goes with RRB_SNAC_DUAL_BUFFER only");
  if ((flags & RRB_SNAC_GRAPH) && flags != RRB_SNAC_GRAPH)
    return fail(RRB_EINVAL, "RRB_SNAC_GRAPH takes no other flag");
  if ((flags & RRB_SNAC_SPECULATIVE) && !(flags & RRB_SNAC_DUAL_BUFFER))
    return fail(RRB_EINVAL, "speculative reduction needs dual buffering");
  const int esz = elem_size(dtype);
  if (count <= 0 || (count * esz) % 16)
    return fail(RRB_EUNSUPPORTED, "chain payloads must be a positive multiple of 16 bytes");
  if (2LL * nranks * count * esz * ((flags & RRB_SNAC_LAMPORT) ? 2 : 1) > 0x7fffffffLL)
    return fail(RRB_EUNSUPPORTED, "staging above 2 GiB");
  if (slices < 0 || slices > kMaxSlices)
    return fail(RRB_EINVAL, "slices %d outside 0..%d", slices, kMaxSlices);
  return RRB_OK;
}

// Issues one All-Reduce chain call of a persistent variant on the handle's
// workspace h->ws (bound, not graph mode, not a plan chain).
rrb_status launch_ar_chain(rrb_snac_s *h, int32_t epochs, const void *d_in, void *d_out,
                           rrb_snac_stats *d_stats, const uint32_t *d_stagger, uint32_t spin_limit,
                           rrb_stream_t stream) {
  const int esz = elem_size(h->dtype);
  SnacArgs a;
  std::memset(&a, 0, sizeof a);
  a.in = static_cast<const unsigned char *>(d_in);
  a.out = static_cast<unsigned char *>(d_out);
  a.staging = h->ws + h->lay.staging_off;
  a.flag = reinterpret_cast<uint32_t *>(h->ws + h->lay.flag_off);
  a.done = reinterpret_cast<uint32_t *>(h->ws + h->lay.done_off);
  a.status = reinterpret_cast<uint32_t *>(h->ws + h->lay.status_off);
  a.stats = d_stats;
  a.stagger = d_stagger;
  a.count = h->count;
  a.rank_bytes = h->count * esz;
  a.nvec = a.rank_bytes / 16;
  a.slice_vec = (a.nvec + h->S - 1) / h->S;
  a.reduced = h->ws + h->lay.reduced_off;
  a.flag2 = reinterpret_cast<uint32_t *>(h->ws + h->lay.flag2_off);
  a.chunk_vec = (a.nvec + h->R - 1) / h->R;
  a.piece_vec = (a.chunk_vec + h->S - 1) / h->S;
  a.tagged = h->ws + h->lay.tagged_off;
  a.epoch0 = h->next_epoch;
  a.epochs = epochs;
  a.S = h->S;
  a.spin_limit = spin_limit ? spin_limit : kDefaultSpin;
  // Speculation overlaps the loads of the sources that are ready with the
  // wait for the late ones.  That pays while a chain is latency-bound; above
  // kSpecMaxBytes per rank it is bandwidth-bound, and the speculative loads
  // measured slower than waiting first on MI355X (8 ranks, 64-deep chains,
  // us per All-Reduce: 256 KiB 3.64 against 3.20, 512 KiB 5.50 against 5.31;
  // ahead at 8-128 KiB, 1.79 against 1.96 at 8 KiB).  There the speculative
  // variant runs the dual-buffer kernel: the same buffers and flags, a wait
  // before the loads.  The memory-model build pays an acquire fence for the
  // speculative read and another for a retry, and speculation leads there
  // only at 8 KiB (64-deep chains, dual against speculative, us per
  // All-Reduce: 8 KiB 2.36 / 2.28, 16 KiB 3.10 / 3.22, 32 KiB 3.68 / 4.13,
  // 128 KiB 6.70 / 7.52).
  const int64_t spec_max = kFences ? int64_t(8) << 10 : kSpecMaxBytes;
  const bool spec = (h->flags & RRB_SNAC_SPECULATIVE) &&
                    ((h->flags & RRB_SNAC_SPEC_ALWAYS) || a.rank_bytes <= spec_max);

  const bool bf16 = h->dtype == RRB_BF16;
  // Flag-in-data slices of at most one vector per lane: payloads up to
  // 16 KiB run 7-8% faster with one vector per lane in flight (measured on
  // MI355X); at 32-64 KiB the two-vector shape is as fast or faster.  Where
  // the two-vector instance (172 VGPRs) would need a cooperative launch, the
  // one-vector instance (85 VGPRs) still launches plainly: 2048 workgroups
  // at 128 KiB 4.60 -> 4.40 us per All-Reduce, 256 KiB 5.86-5.91 -> 5.53-5.59.
  bool one = a.nvec <= 1024 && a.slice_vec <= h->bs;
  if ((h->flags & RRB_SNAC_LAMPORT) && !one && a.slice_vec <= h->bs &&
      !(h->flags & RRB_SNAC_COOPERATIVE)) {
    bool coop_two = false;
    const rrb_status st = needs_cooperative(
        h, reinterpret_cast<const void *>(bf16 ? snac_for<true, kLamport>(h->R) : snac_for<false, kLamport>(h->R)),
        "chain", &coop_two);
    if (st != RRB_OK) return st;
    one = coop_two;
  }
  const int var = (h->flags & RRB_SNAC_LAMPORT) ? (one ? kLamportOne : kLamport)
                  : (h->flags & RRB_SNAC_TWOSHOT) ? kTwoshot
                  : spec                              ? kSpeculative
                  : (h->flags & RRB_SNAC_DUAL_BUFFER) ? kDual : kBarrier;
  SnacFn fn = nullptr;
  if (bf16) {
    fn = var == kBarrier ? snac_for<true, kBarrier>(h->R)
         : var == kDual  ? snac_for<true, kDual>(h->R)
         : var == kTwoshot ? snac_for<true, kTwoshot>(h->R)
         : var == kLamport ? snac_for<true, kLamport>(h->R)
         : var == kLamportOne ? snac_for<true, kLamportOne>(h->R)
                           : snac_for<true, kSpeculative>(h->R);
  } else {
    fn = var == kBarrier ? snac_for<false, kBarrier>(h->R)
         : var == kDual  ? snac_for<false, kDual>(h->R)
         : var == kTwoshot ? snac_for<false, kTwoshot>(h->R)
         : var == kLamport ? snac_for<false, kLamport>(h->R)
         : var == kLamportOne ? snac_for<false, kLamportOne>(h->R)
                           : snac_for<false, kSpeculative>(h->R);
  }
  // Every workgroup waits on others: the grid must be co-resident.
  const rrb_status st = launch_persistent(h, reinterpret_cast<const void *>(fn), a,
                                          static_cast<hipStream_t>(stream), "chain");
  if (st != RRB_OK) return st;
  h->next_epoch += static_cast<uint32_t>(epochs);
  return RRB_OK;
}

}  // namespace
}  // namespace rrb

using namespace rrb;

extern "C" {

int32_t rrb_snac_fenced(void) { return kFences ? 1 : 0; }

rrb_status rrb_snac_create(int32_t nranks, int64_t count, int32_t dtype, uint32_t flags,
                           int32_t slices, rrb_snac_t *out) {
  clear_error();
  if (!out) return fail(RRB_EINVAL, "NULL out");
  *out = nullptr;
  const rrb_status cs = check_ar_chain_args(nranks, count, dtype, flags, slices);
  if (cs != RRB_OK) return cs;
  const int esz = elem_size(dtype);
  const int64_t nvec = count * esz / 16;
  const int32_t S = default_slices(slices, nvec, nranks, flags, false);
  rrb_snac_s *h = new (std::nothrow) rrb_snac_s;
  if (!h) return fail(RRB_ENOMEM, "handle allocation failed");
  h->R = nranks;
  h->count = count;
  h->dtype = dtype;
  h->flags = flags;
  h->S = S;
  h->bs = 64;
  h->in_stride = h->out_stride = count * esz;
  h->lay = layout_for(nranks, count, dtype, S, (flags & RRB_SNAC_LAMPORT) != 0);
  if (flags & RRB_SNAC_GRAPH) {
    rrb_spec sp;
    std::memset(&sp, 0, sizeof sp);
    sp.nranks = nranks;
    sp.dtype = dtype;
    sp.count = count;
    sp.in.kind = RRB_PARTIAL;
    sp.out.kind = RRB_REPLICATED;
    sp.op = RRB_REDUCE_SUM;
    const rrb_status st = build_uniform_plan(sp, h->ar_plan);
    if (st != RRB_OK) {
      delete h;
      return st;
    }
  }
  *out = h;
  return RRB_OK;
}

rrb_status rrb_snac_create_plan(rrb_plan_t plan, uint32_t flags, int32_t slices, rrb_snac_t *out) {
  clear_error();
  if (!out) return fail(RRB_EINVAL, "NULL out");
  *out = nullptr;
  if (!plan) return fail(RRB_EINVAL, "NULL plan");
  const Plan &p = plan->p;
  if (p.kind != PlanKind::Uniform)
    return fail(RRB_EUNSUPPORTED, "chains take layout-named (uniform) plans, not MoE row plans");
  if (p.op == RRB_REDUCE_SUM_TREE)
    return fail(RRB_EUNSUPPORTED, "chains fold in the fixed rank order only");
  const uint32_t base = flags & ~RRB_SNAC_COOPERATIVE;
  if ((base != 0 && base != RRB_SNAC_DUAL_BUFFER &&
       base != (RRB_SNAC_DUAL_BUFFER | RRB_SNAC_SPECULATIVE) && base != RRB_SNAC_GRAPH) ||
      ((flags & RRB_SNAC_COOPERATIVE) && base == RRB_SNAC_GRAPH))
    return fail(RRB_EUNSUPPORTED,
                "plan chains take 0, DUAL_BUFFER, DUAL_BUFFER|SPECULATIVE (each optionally "
                "|COOPERATIVE) or GRAPH (flags 0x%x)", flags);
  if (slices < 0 || slices > kMaxSlices)
    return fail(RRB_EINVAL, "slices %d outside 0..%d", slices, kMaxSlices);
  const int R = p.nranks;
  const int esz = elem_size(p.dtype);
  int64_t in_max = 0, out_max = 0;
  for (int r = 0; r < R; ++r) {
    in_max = std::max(in_max, p.in_count[r] * esz);
    out_max = std::max(out_max, p.out_count[r] * esz);
  }
  if (in_max == 0 || out_max == 0) return fail(RRB_EINVAL, "the plan moves no data");
  for (const Segment &g : p.segs)
    if ((g.src_off * esz) % 16 || (g.dst_off * esz) % 16 || (g.len * esz) % 16)
      return fail(RRB_EUNSUPPORTED, "chains need every map entry on 16-byte boundaries");
  for (int r = 0; r < R; ++r)
    if ((p.in_count[r] * esz) % 16)
      return fail(RRB_EUNSUPPORTED, "chains need 16-byte multiples of input per rank");
  const int64_t in_stride = (in_max + 15) / 16 * 16;
  const int64_t out_stride = (out_max + 15) / 16 * 16;
  if (2LL * R * in_stride > 0x7fffffffLL) return fail(RRB_EUNSUPPORTED, "staging above 2 GiB");
  rrb_snac_s *h = new (std::nothrow) rrb_snac_s;
  if (!h) return fail(RRB_ENOMEM, "handle allocation failed");
  try {
    h->ar_plan = p;
    for (int r = 0; r < R; ++r) {
      h->in_vec[r] = p.in_count[r] * esz / 16;
      h->first[r] = static_cast<int32_t>(h->entries.size());
      for (const Segment &g : p.segs) {
        if (!(g.dst_mask >> r & 1u)) continue;
        PlanEntry e;
        e.src_off = g.src_off * esz / 16;
        e.dst_off = g.dst_off * esz / 16;
        e.len = g.len * esz / 16;
        e.src_rank = g.src_rank;
        e.pad = 0;
        h->entries.push_back(e);
      }
      h->cnt[r] = static_cast<int32_t>(h->entries.size()) - h->first[r];
      if (h->cnt[r] > kFlatEntries) {
        const int cnt = h->cnt[r];
        delete h;
        return fail(RRB_EUNSUPPORTED, "rank %d has %d map entries; a chain holds at most %d per rank", r,
                    cnt, kFlatEntries);
      }
      // Flat consume: copies of one length only.
      bool flat = h->cnt[r] >= 1;
      for (int g = h->first[r]; flat && g < h->first[r] + h->cnt[r]; ++g)
        flat = h->entries[g].src_rank >= 0 && h->entries[g].len == h->entries[h->first[r]].len;
      h->copy_len[r] = flat ? h->entries[h->first[r]].len : 0;
    }
  } catch (const std::bad_alloc &) {
    delete h;
    return fail(RRB_ENOMEM, "handle allocation failed");
  }
  const int64_t nvec = std::max(in_max, out_max) / 16;
  h->R = R;
  h->count = p.count;
  h->dtype = p.dtype;
  h->flags = flags;
  h->S = default_slices(slices, nvec, R, flags, true);
  h->bs = 64;
  h->in_stride = in_stride;
  h->out_stride = out_stride;
  h->from_plan = true;
  int64_t in_vec_max = 0;
  for (int r = 0; r < R; ++r) in_vec_max = std::max(in_vec_max, h->in_vec[r]);
  h->slice_vec = (in_vec_max + h->S - 1) / h->S;
  try {
    build_wait_lists(*h);
  } catch (const std::bad_alloc &) {
    delete h;
    return fail(RRB_ENOMEM, "handle allocation failed");
  }
  h->lay = layout_for_plan(R, in_stride, h->S, static_cast<int64_t>(h->entries.size()),
                           static_cast<int64_t>(h->wait_tab.size()));
  *out = h;
  return RRB_OK;
}

rrb_status rrb_snac_strides(rrb_snac_t h, int64_t *in_stride, int64_t *out_stride) {
  clear_error();
  if (!h) return fail(RRB_EINVAL, "NULL handle");
  if (in_stride) *in_stride = h->in_stride;
  if (out_stride) *out_stride = h->out_stride;
  return RRB_OK;
}

rrb_status rrb_snac_workspace(rrb_snac_t h, size_t *bytes) {
  clear_error();
  if (!h || !bytes) return fail(RRB_EINVAL, "NULL handle or bytes");
  *bytes = static_cast<size_t>(h->lay.total);
  return RRB_OK;
}

rrb_status rrb_snac_bind(rrb_snac_t h, void *d_ws, size_t bytes, rrb_stream_t stream) {
  clear_error();
  if (!h) return fail(RRB_EINVAL, "NULL handle");
  if (!d_ws || bytes < static_cast<size_t>(h->lay.total))
    return fail(RRB_EINVAL, "workspace of %lld bytes needed", (long long)h->lay.total);
  if (reinterpret_cast<uintptr_t>(d_ws) % 256) return fail(RRB_EINVAL, "workspace must be 256-byte aligned");
  h->ws = static_cast<unsigned char *>(d_ws);
  h->next_epoch = 1;
  h->drop_graph();
  hipError_t e = hipSuccess;
  if (h->from_plan && !(h->flags & RRB_SNAC_GRAPH) && !h->entries.empty()) {
    // The consume entries; synchronous so the host vector may change later.
    e = hipMemcpyAsync(h->ws + h->lay.entries_off, h->entries.data(),
                       h->entries.size() * sizeof(PlanEntry), hipMemcpyHostToDevice,
                       static_cast<hipStream_t>(stream));
    if (e == hipSuccess)
      e = hipMemcpyAsync(h->ws + h->lay.waits_off, h->wait_tab.data(), h->wait_tab.size() * 4,
                         hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    if (e == hipSuccess) e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(RRB_EHIP, "entry upload: %s", hipGetErrorString(e));
  }
  // Clear flags, done words and status with a fill kernel (graph-safe).
  uint32_t *p = reinterpret_cast<uint32_t *>(h->ws + h->lay.flag_off);
  const int64_t n = (h->lay.total - h->lay.flag_off) / 4;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(64), dim3(256), 0, static_cast<hipStream_t>(stream), p, n,
                     0u);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(RRB_EHIP, "flag clear: %s", hipGetErrorString(e));
  return RRB_OK;
}

rrb_status rrb_snac_allreduce_chain(rrb_snac_t h, int32_t epochs, const void *d_in, void *d_out,
                                    rrb_snac_stats *d_stats, const uint32_t *d_stagger,
                                    uint32_t spin_limit, rrb_stream_t stream) {
  clear_error();
  if (!h) return fail(RRB_EINVAL, "NULL handle");
  if (h->from_plan) return fail(RRB_EINVAL, "a plan chain runs through rrb_snac_chain");
  return rrb_snac_chain(h, epochs, d_in, d_out, d_stats, d_stagger, spin_limit, stream);
}

rrb_status rrb_snac_chain(rrb_snac_t h, int32_t epochs, const void *d_in, void *d_out,
                          rrb_snac_stats *d_stats, const uint32_t *d_stagger,
                          uint32_t spin_limit, rrb_stream_t stream) {
  clear_error();
  if (!h) return fail(RRB_EINVAL, "NULL handle");
  if (!h->ws) return fail(RRB_EINVAL, "handle is not bound to a workspace");
  if (epochs < 0) return fail(RRB_EINVAL, "negative epoch count");
  if (epochs == 0) return RRB_OK;
  if (!d_in || !d_out) return fail(RRB_EINVAL, "NULL payload pointer");
  if ((reinterpret_cast<uintptr_t>(d_in) | reinterpret_cast<uintptr_t>(d_out)) & 15)
    return fail(RRB_EINVAL, "payloads must be 16-byte aligned");
  if (h->flags & RRB_SNAC_GRAPH) {
    if (d_stagger) return fail(RRB_EINVAL, "the stagger hook applies to the flag protocol only");
    if (!(h->exec && h->g_in == d_in && h->g_out == d_out && h->g_epochs == epochs)) {
      rrb_status st;
      try {
        st = build_chain_graph(h, epochs, d_in, d_out);
      } catch (const std::bad_alloc &) {
        h->drop_graph();
        st = fail(RRB_ENOMEM, "graph description allocation failed");
      }
      if (st != RRB_OK) return st;
    }
    const hipError_t e = hipGraphLaunch(h->exec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(RRB_EHIP, "graph launch: %s", hipGetErrorString(e));
    return RRB_OK;
  }
  if (h->next_epoch > 0xffffffffu - static_cast<uint32_t>(epochs) - 2)
    return fail(RRB_EUNSUPPORTED, "epoch counter exhausted; rebind the handle");
  if (h->from_plan) return launch_plan_chain(h, epochs, d_in, d_out, d_stats, d_stagger, spin_limit, stream);
  return launch_ar_chain(h, epochs, d_in, d_out, d_stats, d_stagger, spin_limit, stream);
}

rrb_status rrb_snac_check(rrb_snac_t h, rrb_stream_t stream) {
  clear_error();
  if (!h || !h->ws) return fail(RRB_EINVAL, "NULL or unbound handle");
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  uint32_t st = 0;
  if (e == hipSuccess)
    e = hipMemcpy(&st, h->ws + h->lay.status_off, 4, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(RRB_EHIP, "status read: %s", hipGetErrorString(e));
  if (st) return fail(RRB_ETIMEOUT, "a SNAC wait exceeded its poll budget");
  return RRB_OK;
}

void rrb_snac_destroy(rrb_snac_t h) { delete h; }

}  // extern "C"

// ---- the All-Reduce chain without allocation ---------------------------------
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): the
// staging buffers, flags and status word of a chain call live in `scratch`, a
// file-scope device array of fixed size.  Each GPU the library runs on holds
// its own copy until the process ends; every call on a GPU shares it.

#include <mutex>

namespace {
// 8 ranks of up to 1 MiB each, twoshot included, fit (about 18.7 MiB).
constexpr int64_t kNoAllocScratchBytes = 20LL << 20;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
unsigned char *g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch`, by its device address, looked up
// once per device with that device current.  In host code the array's name
// is only a stand-in: it is never passed to a kernel or a copy.
rrb_status device_scratch(unsigned char **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(RRB_EHIP, "current device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(RRB_EUNSUPPORTED, "device %d: the static scratch covers devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(RRB_EHIP, "static scratch address on device %d: %s", dev, hipGetErrorString(e));
    g_scratch[dev] = static_cast<unsigned char *>(p);
  }
  *out = g_scratch[dev];
  return RRB_OK;
}

}  // namespace

extern "C" rrb_status rrb_snac_allreduce_chain_noalloc(int32_t nranks, int64_t count, int32_t dtype,
                                                       uint32_t flags, int32_t slices, int32_t epochs,
                                                       const void *d_in, void *d_out,
                                                       rrb_snac_stats *d_stats, uint32_t spin_limit,
                                                       rrb_stream_t stream) {
  clear_error();
  rrb_status st = check_ar_chain_args(nranks, count, dtype, flags, slices);
  if (st != RRB_OK) return st;
  if (flags & (RRB_SNAC_GRAPH | RRB_SNAC_LAMPORT))
    return fail(RRB_EUNSUPPORTED,
                "the allocation-free chain runs the flag protocols (barrier, dual, speculative, twoshot)");
  if (epochs < 0) return fail(RRB_EINVAL, "negative epoch count");
  const int esz = elem_size(dtype);
  // The handle's fields on the stack; its containers stay empty, so nothing
  // is allocated.
  rrb_snac_s h;
  h.R = nranks;
  h.count = count;
  h.dtype = dtype;
  h.flags = flags;
  h.S = default_slices(slices, count * esz / 16, nranks, flags, false);
  h.bs = 64;
  h.in_stride = h.out_stride = count * esz;
  h.lay = layout_for(nranks, count, dtype, h.S, false);
  if (h.lay.total > kNoAllocScratchBytes)
    return fail(RRB_EUNSUPPORTED,
                "this chain needs %lld bytes of scratch; the static scratch holds %lld (8 ranks of up "
                "to 1 MiB each)",
                (long long)h.lay.total, (long long)kNoAllocScratchBytes);
  if (epochs == 0) return RRB_OK;
  if (!d_in || !d_out) return fail(RRB_EINVAL, "NULL payload pointer");
  if ((reinterpret_cast<uintptr_t>(d_in) | reinterpret_cast<uintptr_t>(d_out)) & 15)
    return fail(RRB_EINVAL, "payloads must be 16-byte aligned");
  unsigned char *ws = nullptr;
  st = device_scratch(&ws);
  if (st != RRB_OK) return st;
  h.ws = ws;
  h.next_epoch = 1;
  // The array keeps the last call's contents: every call clears its flags,
  // done words and status word and starts again at epoch 1.  A fill kernel on
  // the stream, not a memset, so a captured graph replays it correctly.
  hipLaunchKernelGGL(fill_u32_kernel, dim3(64), dim3(256), 0, static_cast<hipStream_t>(stream),
                     reinterpret_cast<uint32_t *>(ws + h.lay.flag_off),
                     static_cast<int64_t>((h.lay.total - h.lay.flag_off) / 4), 0u);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(RRB_EHIP, "scratch flag clear: %s", hipGetErrorString(e));
  return launch_ar_chain(&h, epochs, d_in, d_out, d_stats, nullptr, spin_limit, stream);
}
