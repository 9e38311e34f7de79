// moon_internal.h — shared definitions of libmoon's host code and kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moon.h"

namespace moon {

constexpr int kWave = 64;
constexpr int kMaxR = 32;
constexpr int kMaxE = 512;
constexpr int kMaxK = 64;
constexpr int kMaxTiles = 256;      // up to four tiles per lane in the cross-tile scan
constexpr int kPlanWaves = 16;      // waves per planner workgroup
constexpr int kPlanThreads = kPlanWaves * kWave;
constexpr int kMaxSlotsTotal = 8192;  // R * B

// Device status bits of a plan (reported by moon_plan_status).
constexpr int32_t kBadExpert = 1, kSlotBudget = 2, kHistogram = 4, kNotPlanned = 8, kInternal = 16;

// Sizes shared by all kernels of one context.
struct Dims {
  int32_t R, E, K, S, H, B, P;
  int32_t Eg, EB;          // E/R, E+B
  int32_t NvS;             // rows per rank window
  int32_t tile_tok;        // tokens per planner tile (a tile never spans two ranks)
  int32_t tiles_per_rank;
  int32_t ntiles;          // R * tiles_per_rank <= kMaxTiles
  int32_t ntiles_pad;      // ntiles rounded up to a multiple of 4 (row stride of tile counts)
  int32_t ebits;           // bits needed for an expert id
  int32_t rbits;           // bits needed for a rank id
  int32_t ctok;            // tokens per chunk (64 / K)
  int32_t tbits;           // bits needed for a token index inside a chunk
  int32_t ncu;             // compute units of the device the shapes were set up on
};

// Planner scratch: owned by a context (one allocation), or the library's
// static device array for moon_plan_noalloc.
struct Scratch {
  int32_t* tile_cnt;     // [E+1][ntiles_pad] routes of expert e in tile t; row E holds 1
                         // for a tile with an id outside [0,E); padding columns are 0
  uint64_t* tile_agg;    // [ntiles][R] packed (tag, duplicate groups, duplicate rows) per rank
  uint32_t* epoch;       // [1] tag of the latest planning call (low 16 bits never 0)
};

// Byte offsets of the planner scratch arrays inside one block, 256-byte
// aligned; `total` is the block size.
struct ScratchLayout {
  size_t cnt, agg, epoch, total;
};
ScratchLayout scratch_layout(const Dims& d);

// Slot index of a plan, rebuilt by every weight prefetch and gradient
// reduction call (context scratch).
struct SlotIndex {
  int32_t* used;       // [R*B] used slots u*B+j, ascending
  int32_t* act_e;      // [E] experts held by at least one slot, ascending
  int32_t* act_match;  // [E][R] slot the i-th held expert occupies on rank u (-1)
  int32_t* counts;     // [2] used slots, held experts
};

constexpr int kMaxWeightTensors = 8;  // tensors per prefetch / reduction call

// Words exchanged between workgroups of one launch: a 16-bit call tag and two
// 24-bit counts, so a reader knows when a word is current without fences.
__device__ __forceinline__ uint64_t pack_word(uint32_t tag, uint32_t a, uint32_t b) {
  return ((uint64_t)(tag & 0xFFFFu) << 48) | ((uint64_t)(a & 0xFFFFFFu) << 24) | (b & 0xFFFFFFu);
}

// Plan arrays (one allocation).  pidx [R,B,2]: (owner rank, rank-local row)
// of each slot's expert, (-1,-1) for an unused slot.
struct PlanArrays {
  int32_t *dst, *etc, *zfr, *rstats, *dup_groups, *dup_loffs, *dup_counts, *cu, *status, *pidx;
};

}  // namespace moon

struct moon_ctx {
  uint32_t magic;
  int device;
  moon::Dims d;
  void* hidden_win;      // bf16 [R*NvS, H]
  float* w_win;          // fp32 [R*NvS]
  void* scratch_mem;
  moon::Scratch sc;
  moon::SlotIndex si;
};

struct moon_comm_plan {
  uint32_t magic;
  moon_ctx* ctx;
  void* mem;
  size_t bytes;
  moon::PlanArrays a;
};

namespace moon {

// Kernel launchers (each returns a hipError_t from the launch).
hipError_t launch_plan(const Dims& d, const Scratch& sc, const PlanArrays& pa, const int32_t* topk,
                       const int32_t* tpe, hipStream_t s);
// epilogue: scatter primaries, then expand duplicates in a second kernel
// (else every route's row is stored by the scatter).
hipError_t launch_dispatch(const Dims& d, const PlanArrays& pa, const uint16_t* hidden,
                           const float* w, uint16_t* win, float* wwin, bool epilogue,
                           hipStream_t s);
// fold != NULL selects the duplicate prologue; folded primary rows are
// written there ([R*NvS, H], the context window).
hipError_t launch_combine(const Dims& d, const PlanArrays& pa, const uint16_t* y,
                          const float* wnvs, bool weighted, uint16_t* fold, uint16_t* out,
                          float* wsk, hipStream_t s);
// 16-byte vector of raw bits (eight bf16 values).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t dst_global_row(int32_t v) { return v >= 0 ? v : -(int64_t)v - 1; }

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts within
// rows of 16 lanes, then row broadcasts of lanes 15 and 31.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false); // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false); // row_bcast:31
  return v;
}

hipError_t launch_prefetch_index(const Dims& d, const PlanArrays& pa, int32_t* out, hipStream_t s);
// n tensors; row_bytes[t] is a multiple of 16 (reduction: fp32 rows).
hipError_t launch_prefetch_weight(const Dims& d, const PlanArrays& pa, const SlotIndex& si, int n,
                                  const void* const* experts, void* const* slots,
                                  const int64_t* row_bytes, hipStream_t s);
hipError_t launch_reduce_grad(const Dims& d, const PlanArrays& pa, const SlotIndex& si, int n,
                              float* const* grads, float* const* slot_grads,
                              const int64_t* row_bytes, hipStream_t s);

}  // namespace moon
