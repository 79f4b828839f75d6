/*
 * rrb.h -- C ABI of librrb, an MI355X (gfx950) collective datapath on one GPU.
 *
 * The R "ranks" are R buffers in one GPU's HBM.  The library follows the
 * three-way split of Purlin: Separating Orchestration from the Datapath of
 * Collectives ("The Purlin PDF describes a three-layer design"):
 *
 *   collective spec  -- a naming of an input layout and an output layout plus
 *                       a copy or a reduce            -> rrb_plan_create
 *   SNAC             -- stage / notify / consume orchestration, here as epoch
 *                       flags between workgroups      -> rrb_snac_*
 *   Atom             -- the copy and reduce datapath  -> rrb_copy, rrb_reduce
 *
 * Conventions for every function:
 *   - Return value: RRB_OK (0) or a negative rrb_status.  Nothing throws
 *     across the ABI.  rrb_last_error() returns a thread-local text for the
 *     last failure on the calling thread (including HIP's error string).
 *   - Ownership: the caller owns every device buffer and every stream.  The
 *     library never allocates, frees or reallocates device memory; it owns
 *     only the host-side plan / SNAC objects it creates.
 *   - Streams: an rrb_stream_t is a hipStream_t (NULL = the null stream).
 *     Entry points that launch work are asynchronous on that stream and do
 *     not synchronise it, except the *_check calls (which report a kernel's
 *     status) and binds that upload host data (which wait for the upload).
 *   - Pointers named d_* are device pointers; all others are host pointers.
 *   - Element types: RRB_BF16 (IEEE binary32's upper 16 bits) and RRB_F32.
 */
#ifndef RRB_H
#define RRB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RRB_ABI_VERSION 2
#define RRB_MAX_RANKS 16

typedef int32_t rrb_status;
#define RRB_OK            0
#define RRB_EINVAL       (-1) /* bad argument or an invalid layout naming          */
#define RRB_EUNSUPPORTED (-2) /* well formed, but outside what the library supports */
#define RRB_EHIP         (-3) /* a HIP runtime call failed; see rrb_last_error()    */
#define RRB_ETIMEOUT     (-4) /* a bounded wait in a SNAC kernel expired            */
#define RRB_ENOMEM       (-5) /* a host allocation failed                           */

typedef void *rrb_stream_t; /* hipStream_t */

typedef enum { RRB_BF16 = 0, RRB_F32 = 1 } rrb_dtype;
/* RRB_REDUCE_SUM folds in fixed rank order 0..R-1.  RRB_REDUCE_SUM_TREE is an
 * opt-in variant that folds pairwise, level by level (adjacent ranks pair up,
 * an odd last partial sum passes up unchanged: ((0+1)+(2+3))+((4+5)+(6+7))
 * for R = 8), still in fp32 with one final rounding; it may differ from the
 * fixed order by rounding, within max(1 bf16 ulp, 2 (R-1) 2^-24 sum |x|).
 * The tree is this library's reading: the pages name no order other than
 * the fixed one. */
typedef enum { RRB_COPY = 0, RRB_REDUCE_SUM = 1, RRB_REDUCE_SUM_TREE = 2 } rrb_op;

/*
 * Layout names.  The pages say only that a collective names an input and an
 * output layout (Purlin news page, "The Purlin PDF describes a three-layer
 * design"); this is the naming this library reads into that.  A logical
 * tensor X has `count` elements; layouts that name blocks split it into R
 * contiguous blocks of count / R elements.
 *
 *   PARTIAL     rank q holds a full-length partial of X (X = sum over ranks)
 *   REPLICATED  every rank holds all of X
 *   SHARD       rank q holds block q of X
 *   ROOT        rank `root` holds all of X; other ranks hold nothing
 *   BLOCK_ROW   X is an R x R matrix of blocks M[r][q]; rank r holds row r
 *   BLOCK_COL   rank q holds column q (its local block r is M[r][q])
 *
 * copy:   each output element receives the input element carrying the same
 *         name (the lowest rank's copy if several ranks hold it).
 * reduce: input must be PARTIAL; output element X[j] receives
 *         RNE_bf16(((P_0[j] + P_1[j]) + ...) + P_{R-1}[j]) accumulated in fp32
 *         in rank order 0..R-1 (fp32 data: the fp32 sum itself).
 * The seven collectives are: All-Reduce PARTIAL->REPLICATED reduce;
 * Reduce-Scatter PARTIAL->SHARD reduce; All-Gather SHARD->REPLICATED copy;
 * All-to-All BLOCK_ROW->BLOCK_COL copy; Broadcast ROOT(r)->REPLICATED copy;
 * Reduce ROOT: PARTIAL->ROOT(r) reduce; Gather SHARD->ROOT(r) copy.
 */
typedef enum {
  RRB_PARTIAL = 0,
  RRB_REPLICATED = 1,
  RRB_SHARD = 2,
  RRB_ROOT = 3,
  RRB_BLOCK_ROW = 4,
  RRB_BLOCK_COL = 5
} rrb_layout_kind;

typedef struct {
  int32_t kind; /* rrb_layout_kind */
  int32_t root; /* used by RRB_ROOT only */
} rrb_layout;

typedef struct {
  int32_t nranks; /* R, 1..RRB_MAX_RANKS */
  int32_t dtype;  /* rrb_dtype */
  int64_t count;  /* elements of the logical tensor X (per-rank buffer length
                     for BLOCK_ROW / BLOCK_COL); >= 0 */
  rrb_layout in;
  rrb_layout out;
  int32_t op;     /* rrb_op */
  int32_t reserved; /* must be 0 */
} rrb_spec;

/* One entry of a plan's index map, as returned by rrb_plan_segments: `len`
 * elements move from rank src_rank at element offset src_off (or, for a
 * reduce, from every rank 0..R-1 at src_off, folded in rank order) to every
 * rank set in dst_mask at element offset dst_off. */
typedef struct {
  int64_t src_off;
  int64_t dst_off;
  int64_t len;
  int32_t src_rank; /* -1: all ranks, folded in order (reduce) */
  uint32_t dst_mask;
} rrb_segment;

typedef struct rrb_plan_s *rrb_plan_t;

/* ---- errors --------------------------------------------------------------- */

/* Static text for a status code. */
const char *rrb_status_string(rrb_status s);
/* Thread-local text describing the last failure on this thread ("" if none). */
const char *rrb_last_error(void);
/* RRB_ABI_VERSION of the loaded library. */
int32_t rrb_abi_version(void);

/* ---- plans: layout naming -> index map (host only) ------------------------ */

/*
 * Validate `spec` and build its index map (Purlin news page, "The Purlin PDF
 * describes a three-layer design": a collective is a naming of input and
 * output layouts plus copy or reduce).  Rules: reduce iff the input layout is
 * PARTIAL; a reduce output must name elements of X (REPLICATED, SHARD, ROOT);
 * a copy output's every name must be held by the input; BLOCK_ROW/BLOCK_COL
 * only pair with each other; block-naming layouts need count % nranks == 0.
 * On success *out receives a new plan (free with rrb_plan_destroy).
 * Errors: RRB_EINVAL (message in rrb_last_error), RRB_ENOMEM.
 */
rrb_status rrb_plan_create(const rrb_spec *spec, rrb_plan_t *out);

/*
 * Row-map plan for expert-parallel MoE.  `tokens` rows of `hidden` elements
 * (dtype bf16) are sharded over `nranks` source ranks, tokens/nranks
 * consecutive rows each; `experts` experts live on the ranks in contiguous
 * groups of experts/nranks.  topk_idx[tokens][topk] (int32, distinct experts
 * per row) and topk_w[tokens][topk] (float32) are host arrays, copied.
 *   dir = RRB_MOE_DISPATCH: copy each token's row to every selected expert.
 *     Rank r's receive buffer is expert-major over its experts in ascending
 *     id, tokens ascending within an expert (in = token shards [tokens/R][h],
 *     out = receive buffers [rows_r][h]).
 *   dir = RRB_MOE_COMBINE: y[t] = RNE_bf16 of the fp32 fold, over t's experts
 *     in ascending id, of fl32(w * z[slot]) with one multiply then one add per
 *     step (no fused multiply-add) (in = expert outputs in the dispatch
 *     layout, out = token shards).
 * The maps are uploaded by rrb_plan_bind into caller-owned workspace.
 * Errors: RRB_EINVAL (shapes, indices out of range, repeated expert in a row);
 * RRB_EUNSUPPORTED for rows of 2 GiB or more (hidden >= 2^30) or
 * tokens*topk >= 2^26.
 */
#define RRB_MOE_DISPATCH 0
#define RRB_MOE_COMBINE 1
rrb_status rrb_plan_create_rows(int32_t nranks, int64_t tokens, int64_t hidden,
                                int32_t experts, int32_t topk,
                                const int32_t *topk_idx, const float *topk_w,
                                int32_t dir, rrb_plan_t *out);

/*
 * Row-map plan whose maps are built on the device from device routing arrays
 * (per step, with no host round trip): same layout rules as
 * rrb_plan_create_rows, except that the receive side is ONE arena of exactly
 * tokens*topk rows -- rank r's rows (its experts in ascending id, tokens
 * ascending within an expert) start at arena row rank_offsets[r] -- passed as
 * pointer 0 of the receive-side array (dispatch: d_out[0]; combine: d_in[0];
 * other ranks' entries are unused).  Limits: experts <= 1024, topk <= 16,
 * tokens*topk < 2^26, hidden < 2^30 (RRB_EUNSUPPORTED otherwise).  Bind a workspace with
 * rrb_plan_bind (it clears the maps: every slot is arena row 0 until routed);
 * a dispatch and a combine plan of the same shape may share one workspace.
 */
rrb_status rrb_plan_create_rows_device(int32_t nranks, int64_t tokens, int64_t hidden,
                                       int32_t experts, int32_t topk, int32_t dir,
                                       rrb_plan_t *out);

/*
 * Build a device row plan's maps on `stream` from d_topk_idx[tokens][topk]
 * (int32) and d_topk_w[tokens][topk] (float32), device arrays: expert
 * histogram, prefix offsets and the per-token slot list in ascending expert
 * id.  d_rank_offsets (nullable, nranks+1 int32, device) receives the arena
 * row where each rank's region starts, then tokens*topk.  An out-of-range or
 * repeated expert is recorded in the workspace's routing status, which
 * rrb_moe_route_check reports; while it is set, rrb_copy and rrb_reduce on
 * every device plan bound to that workspace write nothing (no valid row is
 * overwritten), until an rrb_moe_route without errors (or a rebind) clears
 * it.  Asynchronous; deterministic.  When
 * every block of 256 tokens fits on the device at once, one kernel with a
 * bounded grid barrier builds the maps; if other work keeps that grid apart,
 * the barrier wait runs out and rrb_moe_route_check reports RRB_ETIMEOUT
 * (rebind the plan then).
 */
rrb_status rrb_moe_route(rrb_plan_t plan, const int32_t *d_topk_idx, const float *d_topk_w,
                         int32_t *d_rank_offsets, rrb_stream_t stream);

/* Synchronise `stream` and report RRB_EINVAL if the last rrb_moe_route on
 * this plan's workspace saw an out-of-range or repeated expert, RRB_ETIMEOUT
 * if its grid barrier wait ran out. */
rrb_status rrb_moe_route_check(rrb_plan_t plan, rrb_stream_t stream);

/*
 * Sizes a plan needs.  *workspace_bytes: device workspace to pass to
 * rrb_plan_bind (0 if none).  in_count[R], out_count[R] (host arrays of
 * nranks entries, either may be NULL): elements each rank's input / output
 * buffer must hold (0: that rank's buffer is not read / not written and may
 * be NULL).
 */
rrb_status rrb_plan_query(rrb_plan_t plan, size_t *workspace_bytes,
                          int64_t *in_count, int64_t *out_count);

/*
 * Upload the plan's device-side map (row plans) into d_workspace (caller-owned,
 * >= workspace_bytes, 256-byte aligned) with a copy on `stream`, and wait for
 * that stream (the host-side map stays owned by the plan).  Device-routed row
 * plans instead zero their map on `stream` without waiting.  The plan keeps
 * d_workspace; it must stay allocated while the plan is used.  Plans with
 * workspace_bytes == 0 accept NULL and do nothing.
 */
rrb_status rrb_plan_bind(rrb_plan_t plan, void *d_workspace, size_t bytes,
                         rrb_stream_t stream);

/* Copy up to `cap` index-map segments into out[] (which may be NULL when
 * cap <= 0); *n receives the total. */
rrb_status rrb_plan_segments(rrb_plan_t plan, rrb_segment *out, int32_t cap,
                             int32_t *n);

void rrb_plan_destroy(rrb_plan_t plan);

/* ---- Atom: the datapath --------------------------------------------------- */

/*
 * Atom copy (Purlin news page, "The Purlin PDF describes a three-layer
 * design": copy is one of the two datapath primitives).  d_in[R] and d_out[R]
 * are host arrays of device pointers, sized per rrb_plan_query; entries for
 * ranks with a zero count may be NULL.  Outputs of ranks the plan does not
 * write are left untouched.  Input and output buffers must not overlap.
 * Requires a copy plan (RRB_EINVAL otherwise) that is bound if it needs a
 * workspace.  Asynchronous on `stream`.
 */
rrb_status rrb_copy(rrb_plan_t plan, const void *const *d_in,
                    void *const *d_out, rrb_stream_t stream);

/*
 * Atom reduce (same passage: reduce is the other primitive).  Same argument
 * rules as rrb_copy; requires a reduce plan (RRB_REDUCE_SUM or
 * RRB_REDUCE_SUM_TREE).  Elementwise fold in the plan's order with fp32
 * accumulation and one round-to-nearest-even to bf16 (the result is
 * bit-identical in every output that receives it).
 * d_weights (nullable, device, float32, 4-byte aligned): per-call combine
 * weights for an MoE combine plan, [tokens][topk] in the column order of the
 * routing arrays the plan was built from (topk_idx of rrb_plan_create_rows,
 * or d_topk_idx of the last rrb_moe_route for a device plan): the weight of
 * token t's expert topk_idx[t][j] is d_weights[t * topk + j].  They replace
 * the weights bound to the plan for this call only; NULL uses the plan's
 * (topk_w at creation, or d_topk_w at the last route).  The fold order stays
 * ascending expert id.  A layout-named reduce is an unweighted sum:
 * d_weights must be NULL for uniform plans (RRB_EINVAL otherwise).  The
 * buffer must stay valid until the launch completes.
 */
rrb_status rrb_reduce(rrb_plan_t plan, const void *const *d_in,
                      void *const *d_out, const float *d_weights,
                      rrb_stream_t stream);

/* Introspection: the kernel launches rrb_copy / rrb_reduce would issue for a
 * layout-named plan with these buffers (nothing is launched), as text --
 * "kernel<template arguments> grid=G block=B", several separated by "; " --
 * written NUL-terminated into buf (host, cap bytes, truncated to fit).
 * Errors: RRB_EINVAL, RRB_EUNSUPPORTED for MoE row plans, RRB_ENOMEM. */
rrb_status rrb_plan_launch_info(rrb_plan_t plan, const void *const *d_in,
                                void *const *d_out, char *buf, int32_t cap);

/* Launch an empty kernel (one workgroup) on `stream`: the launch floor that
 * decode-size collectives are measured against. */
rrb_status rrb_empty_kernel(rrb_stream_t stream);

/* ---- SNAC: stage / notify / consume chain --------------------------------- */

/*
 * A chain of back-to-back All-Reduces over R ranks of `count` elements, run
 * as one persistent kernel in which each rank is a group of `slices`
 * workgroups and the ranks coordinate only through epoch flags in device
 * memory (Purlin news page: Stage, Notify, And Consume; SiFAR:
 * Synchronization-Free All-Reduce for Low-Latency LLM Inference, abstract:
 * top and bottom barriers, dual buffering, speculative reduction).
 * flags:
 *   0                          top barrier + bottom barrier, one buffer
 *   RRB_SNAC_DUAL_BUFFER       two staging buffers by epoch parity; the
 *                              bottom barrier is dropped
 *   | RRB_SNAC_SPECULATIVE     (with DUAL_BUFFER) no top barrier: one read of
 *                              the R sources' flags, then the payload is read
 *                              whatever they said, and the reduced validation
 *                              flag (sum of the R flags == R * epoch) decides
 *                              (SiFAR review, Fig. 14); on a mismatch only the
 *                              stale sources are waited for and read again.
 *                              The payload loads are issued after the flag
 *                              values have returned, so the check holds under
 *                              any order in which the memory system serves
 *                              the loads.
 *                              All-Reduce chains speculate up to 128 KiB per
 *                              rank (8 KiB in the memory-model build, see
 *                              rrb_snac_fenced) and wait for the flags first
 *                              above that,
 *                              as DUAL_BUFFER does: there the chain is
 *                              bandwidth-bound and the early loads measured
 *                              slower.  Plan chains speculate at every size
 *                              (in the memory-model build they wait for the
 *                              flags first at every size).
 *   | RRB_SNAC_SPEC_ALWAYS     (with SPECULATIVE, All-Reduce chains) speculate
 *                              at every payload size
 *   RRB_SNAC_TWOSHOT | DUAL    twoshot (SiFAR review, Fig. 6): stage, then each
 *                              rank reduces chunk r of the payload over all
 *                              ranks, then every rank gathers the R reduced
 *                              chunks; two flag rounds per epoch, each rank
 *                              reads 2x its payload instead of R x
 *   RRB_SNAC_LAMPORT | DUAL    flag-in-data, the Lamport-style All-Reduce
 *                              (SiFAR review, Fig. 20): no flags and no
 *                              fences; each 16-bit half of the payload is
 *                              staged in a 32-bit word under a 16-bit epoch
 *                              tag and readers poll the words themselves
 *                              (staged bytes are 2x the payload);
 *                              stats.retries counts poll rounds that found an
 *                              untagged word.  On MI355X it leads
 *                              DUAL_BUFFER up to 32 KiB per rank and trails
 *                              it from 64 KiB, where polling every word
 *                              costs more than one flag per slice
 *   RRB_SNAC_GRAPH             (alone) orchestration by kernel boundaries on
 *                              one GPU: one Atom All-Reduce kernel per epoch,
 *                              reading d_in[e] in place and chained in a HIP
 *                              graph cached for the last (d_in, d_out,
 *                              epochs); no staging, no flags.  d_stats is not
 *                              written and d_stagger must be NULL.
 *   | RRB_SNAC_COOPERATIVE     (with any persistent variant) always launch
 *                              cooperatively: co-residency guaranteed beside
 *                              other work on the device, about 13 us more per
 *                              call.  Without it, a grid within half the
 *                              device's co-resident capacity takes a plain
 *                              launch (and
 *                              larger grids a cooperative one); if other work
 *                              keeps such a grid from becoming co-resident,
 *                              its bounded waits run out and the call reports
 *                              RRB_ETIMEOUT rather than hang.
 * slices: single-wave workgroups per rank (1..256; 0 = choose from count:
 *         1 KiB of payload per workgroup, up to 128, and 256 from 512 KiB
 *         (128 with RRB_SNAC_SPEC_ALWAYS);
 *         RRB_SNAC_LAMPORT: 1 KiB per workgroup below 64 KiB, then 512 B per
 *         workgroup up to 256, and 128 above 256 KiB; the memory-model build
 *         (rrb_snac_fenced() == 1): 1 KiB per workgroup, up to 16 below
 *         128 KiB and 32 from there; at most 2048 / nranks).
 *         The grid (nranks x slices) must be co-resident; a cooperative
 *         launch that cannot be fails with RRB_EHIP.
 */
#define RRB_SNAC_DUAL_BUFFER 1u
#define RRB_SNAC_SPECULATIVE 2u
#define RRB_SNAC_GRAPH 4u
#define RRB_SNAC_TWOSHOT 8u
#define RRB_SNAC_LAMPORT 16u
#define RRB_SNAC_COOPERATIVE 32u
#define RRB_SNAC_SPEC_ALWAYS 64u
typedef struct rrb_snac_s *rrb_snac_t;

/* Device-side counters a chain call may accumulate into (zeroed by the
 * caller).  misspec: speculative validations that failed; retries: stale
 * sources re-read after a failed validation (All-Reduce chains: source
 * slices; plan chains: source ranks whose entries waited), or for
 * RRB_SNAC_LAMPORT poll rounds that found an untagged word; timeouts:
 * bounded waits that expired; epochs: epochs completed (per rank and slice,
 * summed). */
typedef struct {
  unsigned long long misspec;
  unsigned long long retries;
  unsigned long long timeouts;
  unsigned long long epochs;
} rrb_snac_stats;

rrb_status rrb_snac_create(int32_t nranks, int64_t count, int32_t dtype,
                           uint32_t flags, int32_t slices, rrb_snac_t *out);
/* Device workspace the handle needs: two staging buffers of R x count
 * elements, two reduced buffers of count elements, flags and status words
 * (RRB_SNAC_LAMPORT: two tagged buffers of R x 2 x count elements and the
 * status word). */
rrb_status rrb_snac_workspace(rrb_snac_t h, size_t *bytes);
/* Attach caller-owned workspace (256-byte aligned) and clear its flags with a
 * fill kernel on `stream`; resets the handle's epoch counter. */
rrb_status rrb_snac_bind(rrb_snac_t h, void *d_workspace, size_t bytes,
                         rrb_stream_t stream);
/*
 * Run `epochs` All-Reduces.  d_in: [epochs][R][count] payloads; d_out:
 * [epochs][R][count], every rank's copy of each epoch's result.  d_stats
 * (nullable) accumulates counters.  d_stagger (nullable test hook, R uint32):
 * rank r sleeps about d_stagger[r] x 64 cycles before every stage.
 * spin_limit: polls before a wait gives up (0 = default, about 2 s); on
 * expiry every workgroup leaves, stats.timeouts counts it and
 * rrb_snac_check reports RRB_ETIMEOUT.  The epoch counter carries across
 * calls, so flags never need clearing between calls.  Calls on one handle
 * must be serialised on one stream.
 */
rrb_status rrb_snac_allreduce_chain(rrb_snac_t h, int32_t epochs,
                                    const void *d_in, void *d_out,
                                    rrb_snac_stats *d_stats,
                                    const uint32_t *d_stagger,
                                    uint32_t spin_limit, rrb_stream_t stream);
/*
 * Chains of any layout-named collective (Purlin news page, "The Purlin PDF
 * describes a three-layer design": the orchestration layer is the same
 * whatever collective the datapath runs).  `plan` is a uniform plan from
 * rrb_plan_create (copy or fixed-order reduce; the handle keeps its own copy,
 * so the plan may be destroyed afterwards).  Every map entry must start, end
 * and sit on 16-byte boundaries, and every rank's input must be a 16-byte
 * multiple (RRB_EUNSUPPORTED otherwise).  flags: 0 (top and bottom barrier),
 * RRB_SNAC_DUAL_BUFFER, RRB_SNAC_DUAL_BUFFER | RRB_SNAC_SPECULATIVE (one
 * read of the workgroup's listed flags and the reduced check on their sum;
 * once their values have returned the consume runs, leaving out the map
 * entries that read a rank whose flag read stale (copies from it, and every
 * fold); on a mismatch it waits for the list and then runs those), or
 * RRB_SNAC_GRAPH (one Atom launch per epoch in a cached HIP graph).  Workgroup (r, s) stages slice s of rank r's input and
 * computes piece s of every map entry whose output is rank r; it waits on a
 * list of flags built at create time: the staged slices its pieces read and
 * the workgroups that read its own slice.  slices = 0 gives each workgroup
 * 1 KiB of the larger of a rank's input and output, up to 128 per rank (the
 * memory-model build: up to 16 below 128 KiB and 32 from there).
 * Workspace, bind, check and destroy as for rrb_snac_create.
 */
rrb_status rrb_snac_create_plan(rrb_plan_t plan, uint32_t flags, int32_t slices,
                                rrb_snac_t *out);
/* Bytes between consecutive ranks' buffers in d_in / d_out of a chain: the
 * largest per-rank input (output) of the plan, rounded up to 16 bytes; for an
 * All-Reduce handle both are count x element size. */
rrb_status rrb_snac_strides(rrb_snac_t h, int64_t *in_stride, int64_t *out_stride);
/*
 * Run `epochs` collectives of the handle's plan (or All-Reduces of an
 * rrb_snac_create handle).  Rank r's input of epoch e starts at
 * d_in + (e * R + r) * in_stride bytes and holds in_count[r] elements; its
 * output at d_out + (e * R + r) * out_stride holds out_count[r] elements
 * (outputs of ranks the plan does not write are left untouched).  Other
 * arguments, the epoch counter and ordering rules as for
 * rrb_snac_allreduce_chain, which is this call restricted to All-Reduce
 * handles.
 */
rrb_status rrb_snac_chain(rrb_snac_t h, int32_t epochs, const void *d_in, void *d_out,
                          rrb_snac_stats *d_stats, const uint32_t *d_stagger,
                          uint32_t spin_limit, rrb_stream_t stream);
/*
 * rrb_snac_allreduce_chain without allocation, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Creates, binds and runs an All-Reduce
 * chain handle of (nranks, count, dtype, flags, slices) in one call, with the
 * staging buffers, flags and status word in a static device array of 20 MiB
 * per GPU (held until the process ends) instead of caller workspace; no
 * handle, no hipMalloc.  flags: 0, RRB_SNAC_DUAL_BUFFER,
 * RRB_SNAC_DUAL_BUFFER | RRB_SNAC_SPECULATIVE (optionally
 * | RRB_SNAC_SPEC_ALWAYS) or RRB_SNAC_TWOSHOT | RRB_SNAC_DUAL_BUFFER (each
 * optionally | RRB_SNAC_COOPERATIVE);
 * RRB_SNAC_GRAPH and RRB_SNAC_LAMPORT return RRB_EUNSUPPORTED.  A chain whose
 * staging and flags exceed the array (8 ranks of up to 1 MiB each fit)
 * returns RRB_EUNSUPPORTED with the bytes it needs.  d_in, d_out, d_stats,
 * spin_limit and the results as for rrb_snac_allreduce_chain; a wait that
 * ran out is reported in d_stats->timeouts (pass d_stats to see it).  Every
 * call on a GPU shares that GPU's array: each call clears the flags with a
 * fill kernel on `stream` and restarts at epoch 1, so calls that overlap on
 * one GPU (other streams, other host threads) race and must be serialised
 * by the caller.
 */
rrb_status rrb_snac_allreduce_chain_noalloc(int32_t nranks, int64_t count, int32_t dtype,
                                            uint32_t flags, int32_t slices, int32_t epochs,
                                            const void *d_in, void *d_out,
                                            rrb_snac_stats *d_stats, uint32_t spin_limit,
                                            rrb_stream_t stream);

/* Synchronise `stream` and report RRB_ETIMEOUT if any chain call on this
 * handle since bind timed out (the handle is unusable until rebound). */
rrb_status rrb_snac_check(rrb_snac_t h, rrb_stream_t stream);
void rrb_snac_destroy(rrb_snac_t h);

/* Which ordering this library's SNAC chains were built with.  0 (librrb.so):
 * no fences -- staged data is written through to the point of coherence,
 * each flag is stored once the wave's memory operations have completed, and
 * readers load the data with device-coherent loads issued after the flag
 * values have returned; this rests on how the hardware completes a wave's
 * memory operations, below the source-level memory model.  1
 * (librrb_fenced.so, built from the same sources with RRB_SNAC_FENCES=1):
 * each flag is published with an agent-scope release store, and a wave that
 * has seen flags takes an agent-scope acquire fence before it reads the
 * data they announce or overwrites a buffer they release -- the memory
 * model's own synchronisation for the notify step (Purlin news page: Stage,
 * Notify, And Consume; SiFAR review page, Fig. 8, the write-after-read
 * guard).  The results are bit-identical; the fenced chains are slower.
 * That build
 * refuses RRB_SNAC_LAMPORT (RRB_EUNSUPPORTED): the flag-in-data chain's
 * ordering is per word and has no fenced form.  No device, no errors. */
int32_t rrb_snac_fenced(void);

#ifdef __cplusplus
}
#endif

#endif /* RRB_H */
