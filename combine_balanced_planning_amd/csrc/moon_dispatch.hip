// moon_dispatch.hip — dispatch scatter, padding zero-fill and dedup epilogue.
//
// ("MoonEP Public API Visual Guide", Buffer.dispatch: decode route
//  i = s*K + k, copy the primary hidden row to the destination rank, scatter
//  every routing weight, zero-fill padding, expand locally deduplicated routes
//  in an epilogue.)
//
// The rank windows are one HBM array, so the remote store of the pages is a
// scatter of 16-byte vectors.  Bound: HBM bandwidth.  One wave per token
// reads its row once into registers (H/8 vectors of 16 bytes, up to CH per
// lane per pass) and stores it to each primary row with non-temporal stores;
// lanes 0..K-1 scatter the K route weights.  Extra workgroups zero the padding
// rows of every (rank, group).  The epilogue is a grid-stride loop, one wave
// per duplicate group: read the primary row once, store it to each duplicate.
// All copies move bits; no floating-point arithmetic is done.
#include "moon_internal.h"

namespace moon {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWavesPerBlock * kWave;

template <int CH>
__global__ void __launch_bounds__(kThreads)
    k_dispatch_scatter(Dims d, PlanArrays pa, const u32x4* __restrict__ hidden,
                       const float* __restrict__ w, u32x4* __restrict__ win,
                       float* __restrict__ wwin, int fused, int token_blocks) {
  if (pa.status[0] != 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int V = d.H / 8;
  if ((int)blockIdx.x < token_blocks) {
    const int64_t t = (int64_t)blockIdx.x * kWavesPerBlock + wave;
    if (t >= (int64_t)d.R * d.S) return;
    int dl = 0;
    if (lane < d.K) {
      dl = pa.dst[t * d.K + lane];
      if (w != nullptr) wwin[dst_global_row(dl)] = w[t * d.K + lane];
    }
    const u32x4* src = hidden + t * V;
    for (int c0 = 0; c0 < V; c0 += kWave * CH) {
      u32x4 buf[CH];
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int j = c0 + c * kWave + lane;
        if (j < V) buf[c] = __builtin_nontemporal_load(src + j);
      }
      for (int k = 0; k < d.K; ++k) {
        const int dk = __builtin_amdgcn_readlane(dl, k);
        if (dk < 0 && !fused) continue;  // duplicate: written by the epilogue
        u32x4* dp = win + dst_global_row(dk) * V;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
          const int j = c0 + c * kWave + lane;
          if (j < V) __builtin_nontemporal_store(buf[c], dp + j);
        }
      }
    }
  } else {
    // Zero-fill: one workgroup per (rank, group), one wave per padding row.
    const int zb = blockIdx.x - token_blocks;
    const int u = zb / d.EB;
    const int a = pa.zfr[zb * 2 + 0], b = pa.zfr[zb * 2 + 1];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    for (int row = a + wave; row < b; row += kWavesPerBlock) {
      const int64_t G = (int64_t)u * d.NvS + row;
      u32x4* dp = win + G * V;
      for (int j = lane; j < V; j += kWave) __builtin_nontemporal_store(zero, dp + j);
      if (w != nullptr && lane == 0) wwin[G] = 0.0f;
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
hipError_t launch_ch(const Dims& d, const PlanArrays& pa, const uint16_t* hidden, const float* w,
                     uint16_t* win, float* wwin, bool fused, hipStream_t s) {
  const int64_t tokens = (int64_t)d.R * d.S;
  const int token_blocks = (int)((tokens + kWavesPerBlock - 1) / kWavesPerBlock);
  const int zero_blocks = d.R * d.EB;
  hipLaunchKernelGGL(k_dispatch_scatter<CH>, dim3(token_blocks + zero_blocks), dim3(kThreads), 0, s,
                     d, pa, reinterpret_cast<const u32x4*>(hidden), w,
                     reinterpret_cast<u32x4*>(win), wwin, fused ? 1 : 0, token_blocks);
  if (!fused && d.K > 1) {
    const int64_t want = (tokens + kWavesPerBlock - 1) / kWavesPerBlock;
    const int blocks = (int)(want < 2048 ? (want > 0 ? want : 1) : 2048);
    hipLaunchKernelGGL(k_dispatch_expand<CH>, dim3(blocks), dim3(kThreads), 0, s, d, pa,
                       reinterpret_cast<u32x4*>(win));
  }
  return hipGetLastError();
}

}  // namespace

// Vectors per lane per pass: the smallest instantiated count covering a row.
hipError_t launch_dispatch(const Dims& d, const PlanArrays& pa, const uint16_t* hidden,
                           const float* w, uint16_t* win, float* wwin, bool fused, hipStream_t s) {
  const int per_lane = (d.H / 8 + kWave - 1) / kWave;
  if (per_lane <= 1) return launch_ch<1>(d, pa, hidden, w, win, wwin, fused, s);
  if (per_lane <= 2) return launch_ch<2>(d, pa, hidden, w, win, wwin, fused, s);
  if (per_lane <= 4) return launch_ch<4>(d, pa, hidden, w, win, wwin, fused, s);
  if (per_lane <= 8) return launch_ch<8>(d, pa, hidden, w, win, wwin, fused, s);
  if (per_lane <= 14) return launch_ch<14>(d, pa, hidden, w, win, wwin, fused, s);
  return launch_ch<16>(d, pa, hidden, w, win, wwin, fused, s);
}

}  // namespace moon
