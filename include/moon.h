/*
 * moon.h — C ABI of libmoon.so: balanced expert-parallel planning, dispatch
 * and combine for one MI355X (gfx950).
 *
 * The operations follow the "MoonEP Public API Visual Guide" page (sections
 * Notation, Buffer(...), Buffer.dispatch, Buffer.prefetch_weight,
 * Buffer.combine, Buffer.hidden_nvsh_buffer_view,
 * Buffer.router_weight_buffer_view, Buffer.destroy(), MoonEPCommPlan) and the
 * MoonEP README page (sections Performance, Integration / How to set B).
 *
 * The R expert-parallel ranks are emulated as R disjoint windows of one HBM
 * allocation: rank u's dispatched rows are rows [u*NvS, (u+1)*NvS) of a
 * [R*NvS, H] bf16 array.  One call serves all R ranks, so every per-rank
 * tensor of the pages gains a leading R dimension; rank r's plan is the [r]
 * slice.
 *
 * Shapes (all arrays C-contiguous):
 *   S tokens per rank, H hidden width, K routes per token, E experts
 *   (expert e is homed on rank e / (E/R), row e % (E/R) there), B prefetch
 *   slots per rank, P = token_padding, N = S*K routes per rank,
 *   NvS = dispatched-row capacity per rank, E+B physical groups per rank.
 *
 * Ownership: a context owns its windows and planner scratch; a plan owns its
 * arrays; every other pointer is caller-owned device memory, 16-byte aligned
 * for bf16 row arrays and 4-byte aligned otherwise.  Pointers into the
 * context windows are aliases that later dispatch calls overwrite.
 *
 * Streams: every call is asynchronous on the stream it is given; calls on one
 * stream run in order; no call synchronises the host except
 * moon_plan_status and moon_ctx_destroy.  A context's scratch is shared by
 * all its plans, so one context must not be used from two streams at once.
 *
 * Errors: problems visible on the host (null or misaligned pointers, bad
 * shapes, a plan of another context, a destroyed handle) return a negative
 * status before anything is launched.  Data-dependent problems found on the
 * GPU (an expert id out of range, a slot budget exceeded, a histogram that
 * disagrees with the routes) set the plan's device status word; every later
 * kernel that reads the plan sees it and writes nothing, and
 * moon_plan_status reports it.
 */
#ifndef MOON_H
#define MOON_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOON_OK = 0,
  MOON_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, bad flag, destroyed handle */
  MOON_ERR_TOPOLOGY = -2,      /* E not divisible by R (Guide, Buffer(...) validation) */
  MOON_ERR_UNSUPPORTED = -3,   /* sizes beyond the limits listed at moon_ctx_create */
  MOON_ERR_OOM = -4,           /* device allocation failed */
  MOON_ERR_HIP = -5,           /* a HIP runtime call failed */
  MOON_ERR_PLAN_MISMATCH = -6, /* plan belongs to another context */
  /* reported through the plan's device status word: */
  MOON_ERR_BAD_EXPERT = -7,    /* an expert id outside [0, E) */
  MOON_ERR_SLOT_BUDGET = -8,   /* a rank needs more than B slots (only when B < E/R) */
  MOON_ERR_HISTOGRAM = -9,     /* tokens_per_expert differs from the routes' histogram */
  MOON_ERR_NOT_PLANNED = -10,  /* the plan was never filled by moon_plan */
  MOON_ERR_INTERNAL = -11      /* an internal consistency check failed on the GPU */
} moon_status;

/* Combine flag: scale each routed row by the route weight stored at its row. */
#define MOON_COMBINE_WEIGHTED 0x1u
/* Combine flag: duplicate prologue (Guide, Buffer.combine).  Before the
 * gather, for every token and destination rank holding m >= 2 of its routes,
 * the m rows are summed in fp32 (ascending k, c_k * y with a separate
 * multiply and add, c_k as for the gather) and the bf16 result (nearest,
 * ties to even) is stored at the primary's row of the context's hidden
 * window, the persistent local shard; y_nvsh itself is written only when it
 * is that window.  The gather then adds folded primaries with coefficient 1
 * and skips duplicates.  The window's dispatched rows at those primaries are
 * overwritten. */
#define MOON_COMBINE_DUP_PROLOGUE 0x4u
/* Dispatch flags.  By default the scatter stores every route's row,
 * duplicates included, from registers (one pass; MOON_DISPATCH_FUSED_DUPS
 * names this default explicitly).  MOON_DISPATCH_DEDUP_EPILOGUE selects the
 * pages' two-pass structure (Guide, Buffer.dispatch): the scatter stores each
 * token's primary row once per destination rank, then an epilogue on the
 * receiving rank copies every primary into its duplicate rows.  Both give
 * the same windows; the two flags together are rejected. */
#define MOON_DISPATCH_FUSED_DUPS 0x2u
#define MOON_DISPATCH_DEDUP_EPILOGUE 0x8u

/* Constructor controls (Guide, Buffer(...)): R = number of EP ranks,
 * B <= 0 selects the default E/R, token_padding = alignment in rows of every
 * non-empty physical group.  flags: reserved, must be 0. */
typedef struct {
  int32_t R, E, K, S, H, B, token_padding;
  uint32_t flags;
} moon_config;

/* Zero-copy views (Guide, hidden_nvsh_buffer_view / router_weight_buffer_view):
 * rank u's [NvS, H] bf16 window starts at row u*NvS_padded of hidden_windows;
 * its [NvS] fp32 weights start at weight_windows + u*NvS_padded. */
typedef struct {
  int32_t N, NvS, NvS_padded, E_plus_B, B;
  void* hidden_windows;   /* bf16 [R*NvS_padded, H] */
  float* weight_windows;  /* fp32 [R*NvS_padded] */
} moon_layout;

/* Device pointers of a plan's arrays (Guide, MoonEPCommPlan field table),
 * each with a leading R: dst [R,N] (+G primary, -(G+1) local duplicate,
 * G = u*NvS_padded + local row), experts_to_copy [R,B] (-1 = unused),
 * zero_fill_ranges [R,E+B,2] (half-open padding rows), remote_stats [R,2]
 * (slots used, routes placed in slots), dup_groups [R,NvS,3] (primary local
 * row, first dup_loffs index, count), dup_loffs [R,NvS], dup_counts [R,2]
 * (valid prefix sizes), cu_seqlens [R,E+B] (inclusive padded end offsets),
 * status [1] (internal error bits), and one array the planner adds beside
 * the pages' fields: prefetch_index [R,B,2], for every (rank, slot) the
 * (owner rank, rank-local expert row) of experts_to_copy, or (-1,-1) for an
 * unused slot: the split of the expert id that Buffer.prefetch_weight
 * performs before its copy (written by moon_plan; moon_prefetch_index
 * computes the same into a caller's array). */
typedef struct {
  int32_t *dst, *experts_to_copy, *zero_fill_ranges, *remote_stats, *dup_groups, *dup_loffs,
      *dup_counts, *cu_seqlens, *status;
  int32_t N, R, E, B, NvS, K;
  int32_t* prefetch_index;
} moon_plan_arrays;

typedef struct moon_ctx moon_ctx;
typedef struct moon_comm_plan moon_comm_plan;

/* Validates the topology and sizes, derives N, NvS (= NvS_padded =
 * round_up(S*K + (E/R + B)*(token_padding - 1), token_padding)), allocates the
 * R windows and the planner scratch on the current device (Guide, Buffer(...)).
 * Limits: 1 <= R <= 32, E % R == 0, E <= 512, 1 <= K <= 64, S >= 1,
 * 8 <= H <= 65536 with H % 8 == 0, token_padding >= 1, R*B <= 8192,
 * R*NvS < 2^31, R*S*K < 2^31.  On error *out is NULL. */
moon_status moon_ctx_create(const moon_config* cfg, moon_ctx** out);

/* Window views and derived sizes; no allocation, no copy. */
moon_status moon_ctx_layout(const moon_ctx* ctx, moon_layout* out);

/* Synchronises the device, frees the windows and scratch, sets *ctx = NULL.
 * Idempotent: a NULL *ctx is a no-op (Guide, Buffer.destroy()).  Plans of the
 * context must be destroyed first; their later use is undefined. */
void moon_ctx_destroy(moon_ctx** ctx);

/* Device storage for one plan; its status reads MOON_ERR_NOT_PLANNED until
 * moon_plan fills it. */
moon_status moon_plan_create(moon_ctx* ctx, moon_comm_plan** out);

/* Deep copy of all plan arrays on `stream` (Guide, MoonEPCommPlan.clone()). */
moon_status moon_plan_clone(const moon_comm_plan* src, moon_comm_plan** out, hipStream_t stream);

/* Frees the plan and sets *plan = NULL; idempotent. */
void moon_plan_destroy(moon_comm_plan** plan);

moon_status moon_plan_view(const moon_comm_plan* plan, moon_plan_arrays* out);

/* Synchronises `stream` and returns the plan's device status as a
 * moon_status (MOON_OK when the plan is valid). */
moon_status moon_plan_status(const moon_comm_plan* plan, hipStream_t stream);

/* Planning (Guide, Buffer.dispatch, planning paragraph): reads
 * topk_rsk [R,S,K] int32 expert ids; tokens_per_expert_re [R,E] int32 is
 * optional (NULL) and, when given, is compared with the histogram the planner
 * builds.  Writes every array of `plan`.  Every rank receives exactly S*K
 * routes; a rank's overflow goes to at most B slots taken from one remote
 * home rank (README, Performance / How to set B). */
moon_status moon_plan(moon_ctx* ctx, const int32_t* topk_rsk, const int32_t* tokens_per_expert_re,
                      moon_comm_plan* plan, hipStream_t stream);

/* Planning that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  The same planning as moon_plan, without a context: cfg
 * gives the shapes (validated as by moon_ctx_create, nothing allocated);
 * `plan` holds caller-owned device arrays for every field of
 * moon_plan_arrays, sized for cfg, with N, R, E, B, NvS and K set to the
 * values cfg implies (NvS as at moon_ctx_create, B the effective slot count)
 * -- any other value is MOON_ERR_INVALID_ARG.  The planner's scratch is a
 * fixed 512 KB block in the library's device memory, one per GPU (its address
 * is taken once per device, on the first call with that device current); a
 * shape whose scratch exceeds it is refused with MOON_ERR_UNSUPPORTED.  Every
 * call on one GPU shares that block: calls that overlap on one GPU (two
 * streams, two host threads) race and their plans are undefined.  The
 * block keeps the last call's contents; each call resets what it reads.
 * Results (including the device status word, read by the caller from
 * plan->status: 0 = OK, else error bits) are bit-identical to moon_plan's. */
moon_status moon_plan_noalloc(const moon_config* cfg, const int32_t* topk_rsk,
                              const int32_t* tokens_per_expert_re, const moon_plan_arrays* plan,
                              hipStream_t stream);

/* Dispatch with a plan (Guide, Buffer.dispatch): hidden_rsh [R,S,H] bf16
 * token rows are copied once per destination rank to their primary rows,
 * weights_rsk [R,S,K] fp32 (optional) go to every route's row, padding rows
 * are zeroed; duplicate rows receive the same bits as their primaries (see
 * the dispatch flags).
 * hidden_out / weights_out: [R*NvS,H] bf16 / [R*NvS] fp32, or NULL for the
 * context windows.  Rows after a rank's last group are not written.  Passing
 * an existing plan again is the backward path (Guide: planning is skipped).
 * flags: 0, MOON_DISPATCH_FUSED_DUPS (the same as 0) or
 * MOON_DISPATCH_DEDUP_EPILOGUE. */
moon_status moon_dispatch(moon_ctx* ctx, const moon_comm_plan* plan, const void* hidden_rsh,
                          const float* weights_rsk, void* hidden_out, float* weights_out,
                          uint32_t flags, hipStream_t stream);

/* Combine (Guide, Buffer.combine): out_rsh[r][s] = bf16(sum over k of
 * c_k * y[row(r,s,k)]) accumulated in fp32 in ascending k, c_k = w_nvs[row]
 * with MOON_COMBINE_WEIGHTED, else 1; flags may add
 * MOON_COMBINE_DUP_PROLOGUE.  y_nvsh [R*NvS,H] bf16 (may be the
 * context window); w_nvs [R*NvS] fp32, required when weighted or when
 * w_rsk_out is given; w_rsk_out [R,S,K] (optional) receives the route
 * weights gathered back through the same dst encoding. */
moon_status moon_combine(moon_ctx* ctx, const moon_comm_plan* plan, const void* y_nvsh,
                         const float* w_nvs, uint32_t flags, void* out_rsh, float* w_rsk_out,
                         hipStream_t stream);

/* Prefetch index (Guide, Buffer.prefetch_weight): for every (rank, slot),
 * src_rb2 [R,B,2] int32 receives (owner rank, rank-local expert row) of
 * experts_to_copy, or (-1,-1) for an unused slot. */
moon_status moon_prefetch_index(moon_ctx* ctx, const moon_comm_plan* plan, int32_t* src_rb2,
                                hipStream_t stream);

/* One tensor of the expert weight buffer for moon_prefetch_weight (Guide,
 * Buffer.prefetch_weight; README, Weight buffer).  The pages give every rank
 * one [E+B, H, H'] tensor per projection whose rows [0, E) are the owners'
 * expert weights mapped on every rank and whose rows [E, E+B) are the rank's
 * prefetch slots.  With the R ranks on one GPU the shared rows are one array
 * and the slot rows of all ranks are another:
 *   experts  [E, row_bytes]     rows [0, E), read only
 *   slots    [R, B, row_bytes]  rank u's slot j at row u*B + j, written
 * row_bytes is the byte size of one expert row (H*H'*2 for bf16; any packed
 * format or block scales alike, the copy moves bytes), a positive multiple of
 * 16; both pointers 16-byte aligned.  Caller-owned device memory. */
typedef struct {
  const void* experts;
  void* slots;
  int64_t row_bytes;
} moon_weight_tensor;

/* Weight prefetch (Guide, Buffer.prefetch_weight): for every tensor and every
 * used slot j of every rank u, slots[u][j] <- experts[experts_to_copy[u][j]]
 * (the expert id names its home rank and its row there); unused (-1)
 * slots are not written.  n_tensors in [1, 8]: gate, up, down and, when
 * present, their scales.  Asynchronous on `stream`; uses context scratch
 * (the list of held experts and their slots), so calls on one context are
 * ordered on one stream.  A plan whose device status is not OK writes
 * nothing. */
moon_status moon_prefetch_weight(moon_ctx* ctx, const moon_comm_plan* plan,
                                 const moon_weight_tensor* tensors, int32_t n_tensors,
                                 hipStream_t stream);

/* One fp32 gradient tensor for moon_reduce_grad (Guide, Buffer.reduce_grad;
 * README, Gradient buffer), split like moon_weight_tensor:
 *   expert_grads [E, row_elems]     the owners' parameter gradients, updated
 *   slot_grads   [R, B, row_elems]  every rank's reduce buffer, used slots cleared
 * row_elems = H*H', a positive multiple of 4; both pointers 16-byte aligned. */
typedef struct {
  float* expert_grads;
  float* slot_grads;
  int64_t row_elems;
} moon_grad_tensor;

/* Gradient reduction (Guide, Buffer.reduce_grad): for every tensor and every
 * expert e held by at least one slot, expert_grads[e] <- expert_grads[e] +
 * slot_grads[u][j] for each rank u in ascending order whose slot j holds e
 * (fp32 adds, one after another, seeded with the expert's own gradient);
 * then every used slot's gradient row is set to +0.0.  Experts no slot holds
 * and unused slots are not touched.  n_tensors in [1, 8].  Asynchronous on
 * `stream`; uses context scratch.  A plan whose device status is not OK
 * writes nothing. */
moon_status moon_reduce_grad(moon_ctx* ctx, const moon_comm_plan* plan,
                             const moon_grad_tensor* tensors, int32_t n_tensors,
                             hipStream_t stream);

const char* moon_status_str(moon_status s);

/* Test hook, not part of the pages' interface: the planner's intermediate
 * per-tile histogram from the latest moon_plan call of this context.  The
 * planner cuts each rank's S tokens into *tiles_per_rank consecutive tiles of
 * *tile_tokens tokens (the last one may be shorter); tile t = r*tiles_per_rank
 * + i covers tokens [i*tile_tokens, min(S, (i+1)*tile_tokens)) of rank r.
 * counts_dev (optional, caller-owned device memory) is [E+1, R*tiles_per_rank]
 * int32: row e < E receives the routes to expert e in each tile, row E a 1 for
 * each tile that holds an id outside [0, E) and 0 otherwise.  A
 * device-to-device copy on `stream`, ordered after the moon_plan call when
 * both are on the same stream.  tile_tokens and tiles_per_rank are host
 * pointers and may be NULL. */
moon_status moon_debug_tile_counts(const moon_ctx* ctx, int32_t* counts_dev, int32_t* tile_tokens,
                                   int32_t* tiles_per_rank, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOON_H */
