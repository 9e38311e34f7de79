// moon_dispatch.hip — dispatch scatter, padding zero-fill and dedup epilogue.
//
// ("MoonEP Public API Visual Guide", Buffer.dispatch: route i = s*K + k of a
//  token; its row goes once to each destination rank, every route weight to
//  its own row, padding rows become zero, and a second pass on the receiving
//  rank fills the duplicate routes from their primary row.)
//
// The rank windows are one HBM array, so the remote store of the pages is a
// scatter of 16-byte vectors.  Bound: HBM bandwidth.
//
//   k_dispatch_scatter  persistent grid; a work item is one wave on a 2 KB
//                       slice (128 vectors) of one token's row, read once
//                       with plain loads and stored with non-temporal stores
//                       to each primary row of the token; slice 0 also
//                       scatters the K route weights.  Further items zero the
//                       padding rows of every (rank, group), eight rows each.
//   k_dispatch_expand   persistent grid; one wave per duplicate group reads
//                       the primary row and stores it to each duplicate row.
//
// All copies move bits; no floating-point arithmetic is done.
#include "moon_internal.h"

namespace moon {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWavesPerBlock * kWave;
constexpr int kSliceVec = 2;       // 16-byte vectors per lane in a scatter slice
constexpr int kZeroRows = 8;       // padding rows per zero-fill item
constexpr int kScatterBlocks = 8192;
constexpr int kExpandBlocks = 8192;

__global__ void __launch_bounds__(kThreads)
    k_dispatch_scatter(Dims d, PlanArrays pa, const u32x4* __restrict__ hidden,
                       const float* __restrict__ w, u32x4* __restrict__ win,
                       float* __restrict__ wwin, int fused) {
  if (pa.status[0] != 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int V = d.H / 8;
  const int nsl = (V + kWave * kSliceVec - 1) / (kWave * kSliceVec);
  const int64_t tok_items = (int64_t)d.R * d.S * nsl;
  const int zpg = (d.P - 1 + kZeroRows - 1) / kZeroRows;  // zero items per group
  const int64_t items = tok_items + (int64_t)d.R * d.EB * zpg;
  const int64_t stride = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t it = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; it < items;
       it += stride) {
    if (it < tok_items) {
      const int64_t t = it / nsl;
      const int sl = (int)(it - t * nsl);
      int dl = 0;
      if (lane < d.K) {
        dl = pa.dst[t * d.K + lane];
        if (w != nullptr && sl == 0) wwin[dst_global_row(dl)] = w[t * d.K + lane];
      }
      const int c0 = sl * kWave * kSliceVec;
      const u32x4* src = hidden + t * V;
      u32x4 buf[kSliceVec];
#pragma unroll
      for (int c = 0; c < kSliceVec; ++c) {
        const int j = c0 + c * kWave + lane;
        if (j < V) buf[c] = src[j];
      }
      for (int k = 0; k < d.K; ++k) {
        const int dk = __builtin_amdgcn_readlane(dl, k);
        if (dk < 0 && !fused) continue;  // duplicate: written by the epilogue
        u32x4* dp = win + dst_global_row(dk) * V;
#pragma unroll
        for (int c = 0; c < kSliceVec; ++c) {
          const int j = c0 + c * kWave + lane;
          if (j < V) __builtin_nontemporal_store(buf[c], dp + j);
        }
      }
    } else {
      // Zero-fill: rows [a + 8*blk, ..) of one (rank, group) padding range.
      const int64_t z = it - tok_items;
      const int grp = (int)(z / zpg), blk = (int)(z - (int64_t)grp * zpg);
      const int u = grp / d.EB;
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

template <int CH>
__global__ void __launch_bounds__(kThreads) k_dispatch_expand(Dims d, PlanArrays pa,
                                                              u32x4* __restrict__ win) {
  if (pa.status[0] != 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int V = d.H / 8;
  // Groups of all ranks form one list: rank u's groups follow those of ranks < u.
  const int c = lane < d.R ? pa.dup_counts[lane * 2] : 0;
  int incl = c;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += t;
  }
  const int total = __shfl(incl, kWave - 1, kWave);
  const int nwaves = gridDim.x * kWavesPerBlock;
  for (int gi = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; gi < total; gi += nwaves) {
    const int u = __popcll(__ballot(lane < d.R && incl <= gi));
    const int first = __shfl(incl - c, u, kWave);
    const int32_t* rec = pa.dup_groups + ((int64_t)u * d.NvS + (gi - first)) * 3;
    const int prow = rec[0], lb = rec[1], m = rec[2];
    const u32x4* sp = win + ((int64_t)u * d.NvS + prow) * V;
    const int32_t* lo = pa.dup_loffs + (int64_t)u * d.NvS + lb;
    for (int c0 = 0; c0 < V; c0 += kWave * CH) {
      u32x4 buf[CH];
#pragma unroll
      for (int cc = 0; cc < CH; ++cc) {
        const int j = c0 + cc * kWave + lane;
        if (j < V) buf[cc] = sp[j];
      }
      for (int i = 0; i < m; ++i) {
        u32x4* dp = win + ((int64_t)u * d.NvS + lo[i]) * V;
#pragma unroll
        for (int cc = 0; cc < CH; ++cc) {
          const int j = c0 + cc * kWave + lane;
          if (j < V) __builtin_nontemporal_store(buf[cc], dp + j);
        }
      }
    }
  }
}

template <int CH>
hipError_t launch_expand(const Dims& d, const PlanArrays& pa, uint16_t* win, hipStream_t s) {
  const int64_t tokens = (int64_t)d.R * d.S;
  const int64_t want = (tokens + kWavesPerBlock - 1) / kWavesPerBlock;
  const int blocks = (int)(want < kExpandBlocks ? (want > 0 ? want : 1) : kExpandBlocks);
  hipLaunchKernelGGL(k_dispatch_expand<CH>, dim3(blocks), dim3(kThreads), 0, s, d, pa,
                     reinterpret_cast<u32x4*>(win));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const Dims& d, const PlanArrays& pa, const uint16_t* hidden,
                           const float* w, uint16_t* win, float* wwin, bool fused, hipStream_t s) {
  const int V = d.H / 8;
  const int nsl = (V + kWave * kSliceVec - 1) / (kWave * kSliceVec);
  const int zpg = (d.P - 1 + kZeroRows - 1) / kZeroRows;
  const int64_t items = (int64_t)d.R * d.S * nsl + (int64_t)d.R * d.EB * zpg;
  const int64_t want = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  const int blocks = (int)(want < kScatterBlocks ? (want > 0 ? want : 1) : kScatterBlocks);
  hipLaunchKernelGGL(k_dispatch_scatter, dim3(blocks), dim3(kThreads), 0, s, d, pa,
                     reinterpret_cast<const u32x4*>(hidden), w, reinterpret_cast<u32x4*>(win),
                     wwin, fused ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fused || d.K == 1) return e;
  // Vectors per lane per pass of the epilogue: the smallest count covering a row.
  const int per_lane = (V + kWave - 1) / kWave;
  if (per_lane <= 1) return launch_expand<1>(d, pa, win, s);
  if (per_lane <= 2) return launch_expand<2>(d, pa, win, s);
  if (per_lane <= 4) return launch_expand<4>(d, pa, win, s);
  if (per_lane <= 8) return launch_expand<8>(d, pa, win, s);
  if (per_lane <= 14) return launch_expand<14>(d, pa, win, s);
  return launch_expand<16>(d, pa, win, s);
}

}  // namespace moon
