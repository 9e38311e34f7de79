// moon_weights.hip — weight prefetch into the slots and gradient reduction
// back from them.
//
// ("MoonEP Public API Visual Guide", Buffer.prefetch_weight: each used slot j
//  of rank u receives the weights of expert experts_to_copy[u][j], found
//  through its home rank and its row there; the same copy for gate, up,
//  down and optional scales.  Buffer.reduce_grad: each expert's own fp32
//  gradient is the seed, the slot gradients of every rank that held the
//  expert are added, the sum goes back to the expert's row and the consumed
//  slots are cleared.)
//
// On one GPU the expert rows [0, E) are one array that all emulated ranks
// share (the pages map the owner's memory on every rank), and the slot rows
// of all ranks are one [R, B, row] array, so the remote transfer becomes an
// HBM copy of whole expert rows.  Bound: HBM bandwidth.
//
//   k_slot_index    one workgroup: the list of used slots (ascending), and
//                   for every expert held by a slot, its slot on each rank
//                   (experts ascending).  Both lists go to context scratch.
//   k_prefetch_copy (up to 64 slots) persistent grid over (tensor, slot,
//                   8 KB chunk); items of unused slots (-1) end at once, the
//                   others copy their chunk with cached 16-byte loads and
//                   non-temporal stores.
//   k_prefetch_grouped  (more slots) after k_slot_index, a persistent grid
//                   over (tensor, held expert, 8 KB chunk): the chunk is read
//                   once and stored to every slot that holds the expert.
//   k_reduce_grad   persistent grid over (tensor, held expert, 2 KB chunk);
//                   one wave loads the expert's chunk, adds the matching
//                   slot chunks in ascending rank order (fp32, a + b), stores
//                   the sum and clears the slot chunks.  Each slot has one
//                   expert, so the wave that reads a slot chunk is its only
//                   reader and may clear it at once: the pages' barrier
//                   between reading and clearing is not needed on one GPU.
#include "moon_internal.h"

namespace moon {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWavesPerBlock * kWave;
constexpr int kIndexThreads = 1024;
// Chosen by a sweep on MI355X.  The copy loads expert rows through the
// caches: slots on several ranks often hold the same expert, and later
// copies of it then hit in the cache (non-temporal loads were 1.5x slower).
static_assert(kMaxSlotsTotal <= 65536 && kMaxE <= 32768,
              "a used slot and its expert pack into one int");
constexpr int kCopyVec = 8;          // 16-byte vectors per lane per copy chunk (8 KB per wave)
constexpr int kCopyBlocks = 8192;
constexpr bool kCopyNtLoad = false;
constexpr bool kCopyNtStore = true;
constexpr int kReduceVec = 2;        // 16-byte vectors per lane per reduction chunk (2 KB)
constexpr int kReduceBlocks = 8192;
constexpr bool kReduceNtLoad = true;

struct TensorArgs {
  int32_t n;
  const u32x4* src[kMaxWeightTensors];
  u32x4* dst[kMaxWeightTensors];
  int64_t vecs[kMaxWeightTensors];  // 16-byte vectors per expert row
};

// Ordered compaction of one 1024-entry round inside a workgroup: returns the
// exclusive position of this thread's flag among the flagged threads and the
// round's total.
__device__ int block_rank(bool flag, int* wave_tot, int* total) {
  const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  const uint64_t b = __ballot(flag);
  const int in_wave = __popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) wave_tot[w] = __popcll(b);
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < kIndexThreads / kWave; ++i) {
    const int c = wave_tot[i];
    before += i < w ? c : 0;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + in_wave;
}

__global__ void __launch_bounds__(kIndexThreads)
    k_slot_index(Dims d, PlanArrays pa, SlotIndex si) {
  __shared__ int16_t match[kMaxE * kMaxR];
  __shared__ int wave_tot[kIndexThreads / kWave];
  const bool ok = pa.status[0] == 0;
  const int RB = d.R * d.B;
  for (int i = threadIdx.x; i < d.E * d.R; i += kIndexThreads) match[i] = -1;
  __syncthreads();
  // used slots, ascending (u, j); the slot each expert holds on each rank
  int n_used = 0;
  for (int i0 = 0; i0 < RB; i0 += kIndexThreads) {
    const int i = i0 + threadIdx.x;
    const int e = (ok && i < RB) ? pa.etc[i] : -1;
    const bool used = e >= 0 && e < d.E;
    if (used) match[e * d.R + i / d.B] = (int16_t)(i % d.B);
    int tot;
    const int pos = block_rank(used, wave_tot, &tot);
    if (used) si.used[n_used + pos] = i;
    n_used += tot;
  }
  __syncthreads();
  // experts held by at least one slot, ascending, with their slot per rank
  int n_act = 0;
  for (int e0 = 0; e0 < d.E; e0 += kIndexThreads) {
    const int e = e0 + threadIdx.x;
    bool held = false;
    if (e < d.E)
      for (int u = 0; u < d.R; ++u) held = held || match[e * d.R + u] >= 0;
    int tot;
    const int pos = block_rank(held, wave_tot, &tot);
    if (held) {
      si.act_e[n_act + pos] = e;
      for (int u = 0; u < d.R; ++u) si.act_match[(n_act + pos) * d.R + u] = match[e * d.R + u];
    }
    n_act += tot;
  }
  if (threadIdx.x == 0) {
    si.counts[0] = n_used;
    si.counts[1] = n_act;
  }
}

__global__ void __launch_bounds__(kThreads)
    k_prefetch_copy(Dims d, PlanArrays pa, TensorArgs ta) {
  if (pa.status[0] != 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  for (int t = 0; t < ta.n; ++t) {
    const int64_t V = ta.vecs[t];
    const int64_t nch = (V + kWave * kCopyVec - 1) / (kWave * kCopyVec);
    const int64_t items = (int64_t)d.R * d.B * nch;  // every slot; unused ones are skipped
    for (int64_t it = wave; it < items; it += nwaves) {
      const int slot = (int)(it / nch);
      const int64_t c0 = (it - (int64_t)slot * nch) * kWave * kCopyVec;
      const int e = pa.etc[slot];
      if (e < 0) continue;
      const u32x4* sp = ta.src[t] + (int64_t)e * V;
      u32x4* dp = ta.dst[t] + (int64_t)slot * V;
      u32x4 buf[kCopyVec];
#pragma unroll
      for (int c = 0; c < kCopyVec; ++c) {
        const int64_t j = c0 + c * kWave + lane;
        if (j < V) buf[c] = kCopyNtLoad ? __builtin_nontemporal_load(sp + j) : sp[j];
      }
#pragma unroll
      for (int c = 0; c < kCopyVec; ++c) {
        const int64_t j = c0 + c * kWave + lane;
        if (j < V) {
          if (kCopyNtStore) __builtin_nontemporal_store(buf[c], dp + j);
          else dp[j] = buf[c];
        }
      }
    }
  }
}

// Large slot tables: a work item is one wave on an 8 KB chunk of one held
// expert's row (the slot index lists the held experts and, per expert, its
// slot on every rank); the chunk is read once, with non-temporal loads, and
// stored to every slot that holds the expert.  Measured against one copy per
// used slot (µs): R=16 shape, 15 slots / 6 experts of 3 x 29 MB rows, 367
// against 426; DSv3 shape, 7 / 5, 201 against 205.  Up to 64 slots the
// per-slot copy without the index launch stays faster (r8-e64-k6: 23.5
// against 26.1).
__global__ void __launch_bounds__(kThreads)
    k_prefetch_grouped(Dims d, PlanArrays pa, SlotIndex si, TensorArgs ta) {
  if (pa.status[0] != 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int n_act = si.counts[1];
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  for (int t = 0; t < ta.n; ++t) {
    const int64_t V = ta.vecs[t];
    const int64_t nch = (V + kWave * kCopyVec - 1) / (kWave * kCopyVec);
    const int64_t items = (int64_t)n_act * nch;
    for (int64_t it = wave; it < items; it += nwaves) {
      const int a = (int)(it / nch);
      const int64_t c0 = (it - (int64_t)a * nch) * kWave * kCopyVec;
      const int e = si.act_e[a];
      // lane u < R: the slot expert e holds on rank u (-1 if none)
      const int my_slot = lane < d.R ? si.act_match[a * d.R + lane] : -1;
      const u32x4* sp = ta.src[t] + (int64_t)e * V;
      u32x4 buf[kCopyVec];
#pragma unroll
      for (int c = 0; c < kCopyVec; ++c) {
        const int64_t j = c0 + c * kWave + lane;
        if (j < V) buf[c] = __builtin_nontemporal_load(sp + j);
      }
      uint64_t held = __ballot(my_slot >= 0);
      while (held != 0) {
        const int u = __builtin_ctzll(held);
        held &= held - 1;
        const int j_slot = __builtin_amdgcn_readlane(my_slot, u);
        u32x4* dp = ta.dst[t] + ((int64_t)u * d.B + j_slot) * V;
#pragma unroll
        for (int c = 0; c < kCopyVec; ++c) {
          const int64_t j = c0 + c * kWave + lane;
          if (j < V) __builtin_nontemporal_store(buf[c], dp + j);
        }
      }
    }
  }
}

__global__ void __launch_bounds__(kThreads)
    k_reduce_grad(Dims d, PlanArrays pa, SlotIndex si, TensorArgs ta) {
  if (pa.status[0] != 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int n_act = si.counts[1];
  const int64_t wave = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int t = 0; t < ta.n; ++t) {
    const int64_t V = ta.vecs[t];
    const int64_t nch = (V + kWave * kReduceVec - 1) / (kWave * kReduceVec);
    const int64_t items = (int64_t)n_act * nch;
    // src = expert gradient rows [E, V], dst = slot gradient rows [R, B, V]
    u32x4* grad = const_cast<u32x4*>(ta.src[t]);
    u32x4* slots = ta.dst[t];
    for (int64_t it = wave; it < items; it += nwaves) {
      const int a = (int)(it / nch);
      const int64_t c0 = (it - (int64_t)a * nch) * kWave * kReduceVec;
      const int e = si.act_e[a];
      // lane u < R: the slot expert e holds on rank u (-1 if none)
      const int my_slot = lane < d.R ? si.act_match[a * d.R + lane] : -1;
      u32x4* gp = grad + (int64_t)e * V;
      float acc[kReduceVec][4];
#pragma unroll
      for (int c = 0; c < kReduceVec; ++c) {
        const int64_t j = c0 + c * kWave + lane;
        u32x4 v = zero;
        if (j < V) v = gp[j];
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[c][q] = __uint_as_float(v[q]);
      }
      uint64_t held = __ballot(my_slot >= 0);
      while (held != 0) {
        const int u = __builtin_ctzll(held);
        held &= held - 1;
        const int j_slot = __builtin_amdgcn_readlane(my_slot, u);
        u32x4* sp = slots + ((int64_t)u * d.B + j_slot) * V;
#pragma unroll
        for (int c = 0; c < kReduceVec; ++c) {
          const int64_t j = c0 + c * kWave + lane;
          if (j < V) {
            const u32x4 v = kReduceNtLoad ? __builtin_nontemporal_load(sp + j) : sp[j];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[c][q] = acc[c][q] + __uint_as_float(v[q]);
          }
        }
#pragma unroll
        for (int c = 0; c < kReduceVec; ++c) {
          const int64_t j = c0 + c * kWave + lane;
          if (j < V) __builtin_nontemporal_store(zero, sp + j);
        }
      }
#pragma unroll
      for (int c = 0; c < kReduceVec; ++c) {
        const int64_t j = c0 + c * kWave + lane;
        if (j < V) {
          u32x4 v;
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = __float_as_uint(acc[c][q]);
          __builtin_nontemporal_store(v, gp + j);
        }
      }
    }
  }
}

hipError_t launch_index(const Dims& d, const PlanArrays& pa, const SlotIndex& si, hipStream_t s) {
  hipLaunchKernelGGL(k_slot_index, dim3(1), dim3(kIndexThreads), 0, s, d, pa, si);
  return hipGetLastError();
}

int grid_for(const Dims& d, const TensorArgs& ta, int vec, int max_blocks) {
  // enough waves for every (slot, chunk) item of the largest tensor, capped
  // to a persistent grid
  int64_t most = 0;
  for (int t = 0; t < ta.n; ++t) {
    const int64_t nch = (ta.vecs[t] + kWave * vec - 1) / (kWave * vec);
    most = nch > most ? nch : most;
  }
  const int64_t waves = most * (int64_t)d.R * d.B;
  const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
  return (int)(blocks < max_blocks ? (blocks > 0 ? blocks : 1) : max_blocks);
}

TensorArgs tensor_args(int n, const void* const* src, void* const* dst, const int64_t* bytes) {
  TensorArgs ta{};
  ta.n = n;
  for (int t = 0; t < n; ++t) {
    ta.src[t] = static_cast<const u32x4*>(src[t]);
    ta.dst[t] = static_cast<u32x4*>(dst[t]);
    ta.vecs[t] = bytes[t] / 16;
  }
  return ta;
}

}  // namespace

hipError_t launch_prefetch_weight(const Dims& d, const PlanArrays& pa, const SlotIndex& si, int n,
                                  const void* const* experts, void* const* slots,
                                  const int64_t* row_bytes, hipStream_t s) {
  if (d.B == 0) return hipSuccess;
  const TensorArgs ta = tensor_args(n, experts, slots, row_bytes);
  const int blocks = grid_for(d, ta, kCopyVec, kCopyBlocks);
  if (d.R * d.B <= kWave) {
    hipLaunchKernelGGL(k_prefetch_copy, dim3(blocks), dim3(kThreads), 0, s, d, pa, ta);
    return hipGetLastError();
  }
  hipError_t e = launch_index(d, pa, si, s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_prefetch_grouped, dim3(blocks), dim3(kThreads), 0, s, d, pa, si, ta);
  return hipGetLastError();
}

hipError_t launch_reduce_grad(const Dims& d, const PlanArrays& pa, const SlotIndex& si, int n,
                              float* const* grads, float* const* slot_grads,
                              const int64_t* row_bytes, hipStream_t s) {
  hipError_t e = launch_index(d, pa, si, s);
  if (e != hipSuccess || d.B == 0) return e;
  const TensorArgs ta = tensor_args(n, reinterpret_cast<const void* const*>(grads),
                                    reinterpret_cast<void* const*>(slot_grads), row_bytes);
  hipLaunchKernelGGL(k_reduce_grad, dim3(grid_for(d, ta, kReduceVec, kReduceBlocks)),
                     dim3(kThreads), 0, s, d, pa, si, ta);
  return hipGetLastError();
}

}  // namespace moon
