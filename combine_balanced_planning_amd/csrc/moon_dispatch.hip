// moon_dispatch.hip — dispatch scatter, padding zero-fill and dedup epilogue.
//
// ("MoonEP Public API Visual Guide", Buffer.dispatch: route i = s*K + k of a
//  token; its row goes once to each destination rank, every route weight to
//  its own row, padding rows become zero, and a second pass on the receiving
//  rank fills the duplicate routes from their primary row.)
//
// The rank windows are one HBM array, so the remote store of the pages is a
// scatter of 16-byte vectors.  Bound: HBM bandwidth, and about nine tenths
// of the bytes are writes to scattered rows.
//
//   k_dispatch_scatter<FUSED=true>   (the default) persistent grid; a work
//                       item is one wave on a 2 KB slice (128 vectors; 1 KB
//                       for rows of at most 4 KB) of one token's row, read once with plain loads and stored
//                       with non-temporal stores to the rows of all K routes
//                       (primaries and duplicates alike: a duplicate row gets
//                       the same bits from registers, so no second pass reads
//                       the primary back); slice 0 also scatters the K route
//                       weights.  Further items zero the padding rows of a
//                       rank's home-expert and slot groups (the only ones that
//                       can hold rows), two rows each.
//   k_dispatch_scatter<FUSED=false>  the pages' structure: as above on 7 KB
//                       slices, but only primary rows are stored (through the
//                       caches for primaries the epilogue re-reads, when all
//                       such rows fit in a budget of the last-level cache);
//   k_dispatch_expand   then the epilogue: persistent grid; a work item is one
//                       wave on a 4 KB slice of one duplicate group's primary
//                       row (plain loads where the scatter kept the primaries
//                       in the caches, non-temporal ones otherwise); the lanes
//                       also fetch the group's duplicate row offsets, then the
//                       slice is stored to each duplicate row.
//
// All copies move bits; no floating-point arithmetic is done.
#include "moon_internal.h"

namespace moon {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWavesPerBlock * kWave;
// 16-byte vectors per lane in a scatter slice.  Primaries only (the
// epilogue path), measured dispatch µs for widths 2 / 4 / 7 / 8 / 14:
// r8-e64-k6 94.8 / 87.1 / 86.0 / 85.9 / 86.3, where 7 makes a 4 KB row one
// item; DSv3 shape 1044 / 1056 / 1048 / 1051 / 1069; R=16 shape 3880 / 4306
// / 3875 / 3886 / 3874, where 4 leaves the last of four slices of a 14 KB row
// half empty.
constexpr int kSliceVec = 7;
// The same for the one-pass scatter, which stores each slice K times: 2 KB
// slices for wide rows, 1 KB slices for rows of at most 4 KB.  Measured
// dispatch µs for widths 1 / 2 / 4 / 7 (32768 workgroups; 8192 were 0.6 %
// slower at the R=16 shape): R=16 shape (14 KB rows) 3533 / 3403 / 3463 /
// 3568; r8-e64-k6 (4 KB rows) 77.9 / 80.7 / 84.0 / 85.0.
constexpr int kFusedSliceVec = 2;
constexpr int kFusedSliceVecNarrow = 1;
constexpr int kNarrowRowVec = 256;  // 4 KB rows
// Padding rows per zero-fill item (a sweep of 1, 2, 4, 8, 16: 2 is 5 % faster
// than 8 at serving decode, where padding dominates, and equal elsewhere).
constexpr int kZeroRows = 2;
constexpr int kScatterBlocks = 32768;  // persistent grids (a sweep of 2048, 8192, 32768)
constexpr int kExpandBlocks = 32768;
// Half of the 256 MB last-level cache (MI355X): the largest token-row size
// R*S*2H of a call for which the scatter caches the re-read primaries.
constexpr int64_t kKeepBudgetBytes = 128ll << 20;
constexpr int kExpandSliceVec = 4;  // 16-byte vectors per lane in an epilogue slice
constexpr int kExpandUnroll = 1;    // epilogue items a wave has in flight

// SV: vectors per lane in a slice.  FUSED: store the slice to every route's
// row (slice-major: for each of the lane's vectors, the K rows in turn);
// else to primary rows only (route-major), caching the primaries that the
// epilogue reads back when `keep_dup_primaries`.
template <int SV, bool FUSED>
__global__ void __launch_bounds__(kThreads)
    k_dispatch_scatter(Dims d, PlanArrays pa, const u32x4* __restrict__ hidden,
                       const float* __restrict__ w, u32x4* __restrict__ win,
                       float* __restrict__ wwin, int keep_dup_primaries) {
  // The plan's status is checked before the first store of each work item;
  // the item's loads do not depend on it, so they overlap with its load.
  const int status = pa.status[0];
  const int lane = threadIdx.x & (kWave - 1);
  const int V = d.H / 8;
  const int nsl = (V + kWave * SV - 1) / (kWave * SV);
  const int64_t tok_items = (int64_t)d.R * d.S * nsl;
  const int zpg = (d.P - 1 + kZeroRows - 1) / kZeroRows;  // zero items per group
  // Only a rank's own E/R home experts and its B slots can hold rows: the
  // groups of experts homed elsewhere are always empty and get no items.
  const int gpr = d.Eg + d.B;  // groups per rank that can hold rows
  const int64_t items = tok_items + (int64_t)d.R * gpr * zpg;
  const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t it = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; it < items;
       it += stride) {
    if (it < tok_items) {
      const int64_t t = it / nsl;
      const int sl = (int)(it - t * nsl);
      int dl = 0;
      float wk = 0.0f;
      const bool wlane = lane < d.K && w != nullptr && sl == 0;
      if (lane < d.K) dl = pa.dst[t * d.K + lane];
      if (wlane) wk = w[t * d.K + lane];
      const int c0 = sl * kWave * SV;
      const u32x4* src = hidden + t * V;
      u32x4 buf[SV];
      // (non-temporal loads: 1 % slower at the DSv3 and R=16 shapes)
#pragma unroll
      for (int c = 0; c < SV; ++c) {
        const int j = c0 + c * kWave + lane;
        if (j < V) buf[c] = src[j];
      }
      if (status != 0) return;
      if (wlane) wwin[dst_global_row(dl)] = wk;
      if (FUSED) {
#pragma unroll
        for (int c = 0; c < SV; ++c) {
          const int j = c0 + c * kWave + lane;
          for (int k = 0; k < d.K; ++k) {
            u32x4* dp = win + dst_global_row(__builtin_amdgcn_readlane(dl, k)) * V;
            if (j < V) __builtin_nontemporal_store(buf[c], dp + j);
          }
        }
        continue;
      }
      // Lanes k whose primary row the epilogue will read back (a later route
      // of the token goes to the same rank): stored through the caches when
      // the host judged that such rows fit in the last-level cache.
      uint64_t keep = 0;
      if (keep_dup_primaries) {
        const int64_t uk = dst_global_row(dl) / d.NvS;
        for (int k = 1; k < d.K; ++k) {
          const int dk = __builtin_amdgcn_readlane(dl, k);
          if (dk < 0) {
            const int64_t ud = dst_global_row(dk) / d.NvS;
            keep |= __ballot(lane < k && dl >= 0 && uk == ud);
          }
        }
      }
      for (int k = 0; k < d.K; ++k) {
        const int dk = __builtin_amdgcn_readlane(dl, k);
        if (dk < 0) continue;  // duplicate: written by the epilogue
        u32x4* dp = win + (int64_t)dk * V;
        if ((keep >> k) & 1) {
#pragma unroll
          for (int c = 0; c < SV; ++c) {
            const int j = c0 + c * kWave + lane;
            if (j < V) dp[j] = buf[c];
          }
        } else {
#pragma unroll
          for (int c = 0; c < SV; ++c) {
            const int j = c0 + c * kWave + lane;
            if (j < V) __builtin_nontemporal_store(buf[c], dp + j);
          }
        }
      }
    } else {
      if (status != 0) return;
      // Zero-fill: rows [a + kZeroRows*blk, ..) of one (rank, group) padding range.
      const int64_t z = it - tok_items;
      const int lg = (int)(z / zpg), blk = (int)(z - (int64_t)lg * zpg);
      const int u = lg / gpr, lj = lg - u * gpr;
      const int g = lj < d.Eg ? u * d.Eg + lj : d.E + (lj - d.Eg);
      const int grp = u * d.EB + g;
      const int a = pa.zfr[grp * 2 + 0] + blk * kZeroRows, b = pa.zfr[grp * 2 + 1];
      const int rows = min(kZeroRows, b - a);
      if (rows <= 0) continue;
      const u32x4 zero = {0u, 0u, 0u, 0u};
      for (int r = 0; r < rows; ++r) {
        u32x4* dp = win + ((int64_t)u * d.NvS + a + r) * V;
        for (int j = lane; j < V; j += kWave) __builtin_nontemporal_store(zero, dp + j);
      }
      if (w != nullptr && lane < rows) wwin[(int64_t)u * d.NvS + a + lane] = 0.0f;
    }
  }
}

// Work item = (duplicate group, slice of SW = 64*SV vectors).  A wave takes UI
// items at once: it loads their records, then their primary slices and (one
// lane per duplicate) their duplicate row offsets, then stores.  NTL: read
// the primaries with non-temporal loads (when the scatter did not keep them
// in the caches).
template <int SV, int UI, bool NTL>
__global__ void __launch_bounds__(kThreads) k_dispatch_expand(Dims d, PlanArrays pa,
                                                              u32x4* __restrict__ win) {
  constexpr int SW = kWave * SV;
  const int lane = threadIdx.x & (kWave - 1);
  const int V = d.H / 8;
  const int nsl = (V + SW - 1) / SW;
  // Groups of all ranks form one list: rank u's groups follow those of ranks < u.
  // (The counts are loaded alongside the plan's status word.)
  const int c = lane < d.R ? pa.dup_counts[lane * 2] : 0;
  if (pa.status[0] != 0) return;
  const int incl = wave_incl_scan(c);
  const int64_t items = (int64_t)__builtin_amdgcn_readlane(incl, kWave - 1) * nsl;
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t it0 = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; it0 < items;
       it0 += nwaves * UI) {
    int64_t base[UI];
    int prow[UI], m[UI], j0[UI], loff[UI];
#pragma unroll
    for (int i = 0; i < UI; ++i) {
      const int64_t it = it0 + i * nwaves;
      m[i] = 0;
      base[i] = 0;
      prow[i] = 0;
      j0[i] = 0;
      loff[i] = 0;
      if (it < items) {
        const int gi = (int)(it / nsl), sl = (int)(it - (int64_t)gi * nsl);
        const int u = __popcll(__ballot(lane < d.R && incl <= gi));  // uniform
        const int first = __builtin_amdgcn_readlane(incl - c, u);
        const int32_t* rec = pa.dup_groups + ((int64_t)u * d.NvS + (gi - first)) * 3;
        base[i] = (int64_t)u * d.NvS;
        prow[i] = rec[0];
        m[i] = rec[2];
        j0[i] = sl * SW + lane;
        loff[i] = lane < m[i] ? pa.dup_loffs[base[i] + rec[1] + lane] : 0;
      }
    }
    u32x4 buf[UI][SV];
#pragma unroll
    for (int i = 0; i < UI; ++i) {
      const u32x4* sp = win + (base[i] + prow[i]) * V;
#pragma unroll
      for (int cc = 0; cc < SV; ++cc) {
        const int j = j0[i] + cc * kWave;
        if (m[i] > 0 && j < V) buf[i][cc] = NTL ? __builtin_nontemporal_load(sp + j) : sp[j];
      }
    }
#pragma unroll
    for (int i = 0; i < UI; ++i) {
      for (int x = 0; x < m[i]; ++x) {
        u32x4* dp = win + (base[i] + __builtin_amdgcn_readlane(loff[i], x)) * V;
#pragma unroll
        for (int cc = 0; cc < SV; ++cc) {
          const int j = j0[i] + cc * kWave;
          if (j < V) __builtin_nontemporal_store(buf[i][cc], dp + j);
        }
      }
    }
  }
}

// Persistent scatter grid: enough 4-wave workgroups for every item, at most
// kScatterBlocks.
template <int SV>
int scatter_blocks(const Dims& d) {
  const int V = d.H / 8;
  const int nsl = (V + kWave * SV - 1) / (kWave * SV);
  const int zpg = (d.P - 1 + kZeroRows - 1) / kZeroRows;
  const int64_t items = (int64_t)d.R * d.S * nsl + (int64_t)d.R * (d.Eg + d.B) * zpg;
  const int64_t want = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  return (int)(want < kScatterBlocks ? (want > 0 ? want : 1) : kScatterBlocks);
}

}  // namespace

hipError_t launch_dispatch(const Dims& d, const PlanArrays& pa, const uint16_t* hidden,
                           const float* w, uint16_t* win, float* wwin, bool epilogue,
                           hipStream_t s) {
  const auto* hv = reinterpret_cast<const u32x4*>(hidden);
  auto* wv = reinterpret_cast<u32x4*>(win);
  if (!epilogue || d.K == 1) {
    if (d.H / 8 <= kNarrowRowVec)
      hipLaunchKernelGGL((k_dispatch_scatter<kFusedSliceVecNarrow, true>),
                         dim3(scatter_blocks<kFusedSliceVecNarrow>(d)), dim3(kThreads), 0, s, d,
                         pa, hv, w, wv, wwin, 0);
    else
      hipLaunchKernelGGL((k_dispatch_scatter<kFusedSliceVec, true>),
                         dim3(scatter_blocks<kFusedSliceVec>(d)), dim3(kThreads), 0, s, d, pa, hv,
                         w, wv, wwin, 0);
    return hipGetLastError();
  }
  // The epilogue re-reads one primary row per duplicate group (about 1.3
  // per token on uniform routing).  When the call's token rows fit a budget
  // of the last-level cache, the scatter stores those primaries through the
  // caches so the epilogue can find them there.
  const int V = d.H / 8;
  const int keep = (int64_t)d.R * d.S * d.H * 2 <= kKeepBudgetBytes;
  hipLaunchKernelGGL((k_dispatch_scatter<kSliceVec, false>), dim3(scatter_blocks<kSliceVec>(d)),
                     dim3(kThreads), 0, s, d, pa, hv, w, wv, wwin, keep);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The group count is only known on the device; size the persistent grid by
  // its bound R*S*(K/2) (a token has at most K/2 groups), times the slices.
  constexpr int SW = kWave * kExpandSliceVec;
  const int64_t bound = (int64_t)d.R * d.S * (d.K / 2) * ((V + SW - 1) / SW);
  const int64_t ewant = (bound + kWavesPerBlock * kExpandUnroll - 1) /
                        (kWavesPerBlock * kExpandUnroll);
  const int eblocks = (int)(ewant < kExpandBlocks ? (ewant > 0 ? ewant : 1) : kExpandBlocks);
  // Primaries the scatter kept in the caches are read with plain loads, the
  // others with non-temporal ones (2.4 % of dispatch at the DSv3 shape; 5 %
  // slower where the primaries are kept).
  if (keep)
    hipLaunchKernelGGL((k_dispatch_expand<kExpandSliceVec, kExpandUnroll, false>), dim3(eblocks),
                       dim3(kThreads), 0, s, d, pa, wv);
  else
    hipLaunchKernelGGL((k_dispatch_expand<kExpandSliceVec, kExpandUnroll, true>), dim3(eblocks),
                       dim3(kThreads), 0, s, d, pa, wv);
  return hipGetLastError();
}

}  // namespace moon
