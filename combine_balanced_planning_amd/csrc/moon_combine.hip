// moon_combine.hip — gather-reduce combine, duplicate prologue, route-weight
// gather, prefetch index.
//
// ("MoonEP Public API Visual Guide", Buffer.combine: the reverse of dispatch;
//  each token's K routed rows, located through plan.dst, are summed back into
//  token order, and the route weights are read back through the same signed
//  entries.  A prologue may first fold the duplicate rows of a token on one
//  destination rank into that rank's primary row in fp32.)
//
// k_combine_staged (the default): a workgroup of 16 waves owns a run of
// consecutive tokens whose output rows fill up to 140 KB of LDS.  It first
// reads the run's dst entries (both signs: every route owns its row) and
// route weights into LDS and writes the weight gather w_sk from there.  A work
// item is one wave on a slice of 64 vectors (512 bf16) of one token's row: up
// to eight routed slices are loaded at a time with 16-byte loads, widened to
// fp32 and accumulated as c_k * y in ascending k with a separate multiply and
// add (the library is built with -ffp-contract=off), then rounded once to
// bf16 (nearest, ties to even) into LDS.  When all of its tokens are summed,
// the workgroup writes their rows as one contiguous run.  Bound: HBM
// bandwidth (K row reads + one row write per token); the long output runs
// write faster between the gathers than one 1 KB store per slice does.
// k_combine is the same sum, each wave fetching its token's dst entries and
// weights itself and loading two routed slices at a time, stored slice by
// slice; the duplicate-prologue path uses it.
//
// With the prologue, k_combine_fold first sums, per duplicate group and
// slice, the primary row and its duplicate rows (ascending k, c_k * y in
// fp32, separate multiply and add), rounds to bf16 and stores the result at
// the primary's row of the context window (the persistent local shard);
// k_combine then skips duplicate routes and reads a folded primary from the
// window with coefficient 1.  On one GPU this adds a row write and read per
// group: it is the pages' structure, kept for comparison.
#include "moon_internal.h"

namespace moon {
namespace {

constexpr int kWavesPerBlock = 16;  // one workgroup = 16 waves (chosen by a sweep of 4, 8, 16)
constexpr int kThreads = kWavesPerBlock * kWave;
constexpr int kUnroll = 2;  // rows in flight per wave in the prologue fold
constexpr int kCombineUnroll = 2;    // routed rows loaded before they are summed
constexpr bool kCombineNtLoad = true;   // routed rows are read once: non-temporal loads
constexpr bool kCombineNtStore = true;  // outputs are not read back here: non-temporal stores
constexpr int kFoldBlocks = 8192;  // persistent grid of the prologue
// Staged gather: one 16-wave workgroup per compute unit (its LDS block takes
// most of the unit's 160 KB), tokens per workgroup = the rows that fit.
constexpr int kStageThreads = 1024;
constexpr int kStageVec = 140 * 1024 / 16;  // 16-byte vectors of staged output
constexpr int kStageRoutes = 2048;          // routes whose dst and weight a workgroup stages
constexpr int kStageBatch = 8;              // vectors a thread moves per write step
constexpr int kStageUnroll = 8;             // routed rows loaded before they are summed

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// A duplicate group's position in the list of all ranks' groups (rank u's
// groups follow those of ranks < u): lanes < R hold the per-rank counts and
// their inclusive prefix; returns the record of group gi.
__device__ __forceinline__ const int32_t* group_record(const Dims& d, const PlanArrays& pa,
                                                      int lane, int cnt, int incl, int gi,
                                                      int* u_out) {
  const int u = __popcll(__ballot(lane < d.R && incl <= gi));  // uniform
  const int first = __builtin_amdgcn_readlane(incl - cnt, u);
  *u_out = u;
  return pa.dup_groups + ((int64_t)u * d.NvS + (gi - first)) * 3;
}

__global__ void __launch_bounds__(kThreads)
    k_combine_fold(Dims d, PlanArrays pa, const u32x4* y, const float* __restrict__ wnvs,
                   int weighted, u32x4* fold) {  // y may be fold (in-place prologue)
  if (pa.status[0] != 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int V = d.H / 8;
  const int nsl = (V + kWave - 1) / kWave;
  const int cnt = lane < d.R ? pa.dup_counts[lane * 2] : 0;
  const int incl = wave_incl_scan(cnt);
  const int64_t items = (int64_t)__builtin_amdgcn_readlane(incl, kWave - 1) * nsl;
  const int64_t nwaves = (int64_t)gridDim.x * kWavesPerBlock;
  for (int64_t it = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave; it < items;
       it += nwaves) {
    const int gi = (int)(it / nsl), sl = (int)(it - (int64_t)gi * nsl);
    int u;
    const int32_t* rec = group_record(d, pa, lane, cnt, incl, gi, &u);
    const int prow = rec[0], lb = rec[1], m = rec[2];
    const int64_t base = (int64_t)u * d.NvS;
    // member i: 0 = the primary, 1..m = the duplicates (ascending k)
    int gl = 0;
    float cl = 1.0f;
    if (lane <= m) {
      gl = (int)base + (lane == 0 ? prow : pa.dup_loffs[base + lb + lane - 1]);
      if (weighted) cl = wnvs[gl];
    }
    const int j = sl * kWave + lane;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int i0 = 0; i0 <= m; i0 += kUnroll) {
      u32x4 buf[kUnroll];
      float ck[kUnroll];
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu) {
        const int i = min(i0 + uu, m);
        const int G = __builtin_amdgcn_readlane(gl, i);
        ck[uu] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), i));
        if (j < V && i0 + uu <= m) buf[uu] = __builtin_nontemporal_load(y + (int64_t)G * V + j);
      }
#pragma unroll
      for (int uu = 0; uu < kUnroll; ++uu) {
        if (i0 + uu > m) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q + 0] = acc[2 * q + 0] + ck[uu] * bf16_lo(buf[uu][q]);
          acc[2 * q + 1] = acc[2 * q + 1] + ck[uu] * bf16_hi(buf[uu][q]);
        }
      }
    }
    if (j < V) {
      u32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = bf16_rne(acc[2 * q]) | (bf16_rne(acc[2 * q + 1]) << 16);
      fold[(base + prow) * V + j] = v;
    }
  }
}

// The sum of one token slice (64 vectors, one per lane: j = slice*64 + lane)
// over the token's K routes; dl/gl/wl are lane k's dst entry, its row and its
// route weight (lanes < K).  Routed slices are loaded KU at a time; fp32
// separate multiply and add in ascending k; one round to bf16.  Returns this
// lane's rounded vector (meaningful where j < V).
template <bool PROLOGUE, int KU>
__device__ __forceinline__ u32x4 combine_slice(const Dims& d, const u32x4* __restrict__ y,
                                               const u32x4* __restrict__ fold, int weighted,
                                               int lane, int dl, int gl, float wl, int j) {
  const int V = d.H / 8;
  // With the prologue: lane k is a folded primary when a duplicate route of
  // the token has the same destination rank; duplicates are skipped.
  int folded = 0;
  if (PROLOGUE) {
    const int rk = gl / d.NvS;
    for (int k = 0; k < d.K; ++k) {
      const int dk = __builtin_amdgcn_readlane(dl, k);
      const int gk = (int)dst_global_row(dk);
      if (dk < 0 && gk / d.NvS == rk) folded = 1;
    }
    folded = folded && dl >= 0 && lane < d.K;
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int k0 = 0; k0 < d.K; k0 += KU) {
    u32x4 buf[KU];
    float ck[KU];
    bool use[KU];
#pragma unroll
    for (int uu = 0; uu < KU; ++uu) {
      const int k = min(k0 + uu, d.K - 1);
      const int G = __builtin_amdgcn_readlane(gl, k);
      ck[uu] = weighted ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k)) : 1.0f;
      use[uu] = k0 + uu < d.K;
      const u32x4* src = y;
      if (PROLOGUE) {
        use[uu] = use[uu] && __builtin_amdgcn_readlane(dl, k) >= 0;
        if (__builtin_amdgcn_readlane(folded, k)) {
          src = fold;
          ck[uu] = 1.0f;
        }
      }
      const u32x4* row = src + (int64_t)G * V;
      if (j < V && use[uu])
        buf[uu] = kCombineNtLoad ? __builtin_nontemporal_load(row + j) : row[j];
    }
#pragma unroll
    for (int uu = 0; uu < KU; ++uu) {
      if (!use[uu]) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q + 0] = acc[2 * q + 0] + ck[uu] * bf16_lo(buf[uu][q]);
        acc[2 * q + 1] = acc[2 * q + 1] + ck[uu] * bf16_hi(buf[uu][q]);
      }
    }
  }
  u32x4 v;
#pragma unroll
  for (int q = 0; q < 4; ++q) v[q] = bf16_rne(acc[2 * q]) | (bf16_rne(acc[2 * q + 1]) << 16);
  return v;
}

// Lanes < K: the token's dst entry, its row, its route weight; slice 0 also
// writes the weight gather w_sk.
__device__ __forceinline__ void combine_routes(const Dims& d, const float* __restrict__ wnvs,
                                               float* __restrict__ wsk, int64_t t, int sl,
                                               int lane, int dl, int& gl, float& wl) {
  gl = 0;
  wl = 0.0f;
  if (lane < d.K) {
    gl = (int)dst_global_row(dl);
    if (wnvs != nullptr) wl = wnvs[gl];
    if (wsk != nullptr && sl == 0) wsk[t * d.K + lane] = wl;
  }
}

// One wave per (token, 1 KB slice); the slice is stored straight to `out`.
// The duplicate-prologue path (and rows too wide to stage) use it.
template <bool PROLOGUE, int KU>
__global__ void __launch_bounds__(kThreads)
    k_combine(Dims d, PlanArrays pa, const u32x4* __restrict__ y, const float* __restrict__ wnvs,
              int weighted, const u32x4* __restrict__ fold, u32x4* __restrict__ out,
              float* __restrict__ wsk) {
  const int lane = threadIdx.x & (kWave - 1);
  const int V = d.H / 8;
  const int nsl = (V + kWave - 1) / kWave;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (item >= (int64_t)d.R * d.S * nsl) return;
  const int64_t t = item / nsl;
  const int sl = (int)(item - t * nsl);
  const int j = sl * kWave + lane;
  // The dst entries are read before the plan's status is checked, so the two
  // loads overlap; nothing read before the check is used unless it is zero.
  int dl = 0;
  if (lane < d.K) dl = pa.dst[t * d.K + lane];
  if (pa.status[0] != 0) return;
  int gl;
  float wl;
  combine_routes(d, wnvs, wsk, t, sl, lane, dl, gl, wl);
  const u32x4 v = combine_slice<PROLOGUE, KU>(d, y, fold, weighted, lane, dl, gl, wl, j);
  if (j < V) {
    if (kCombineNtStore) __builtin_nontemporal_store(v, out + t * V + j);
    else out[t * V + j] = v;
  }
}

// Staged gather: a workgroup of 16 waves takes a run of consecutive tokens
// (the first `nhi` workgroups lo + 1 tokens, the others lo; at most about
// 140 KB of output rows).  It first reads the tokens' dst entries and route
// weights into LDS (and writes the weight gather w_sk, coalesced), so a work
// item then waits only for its routed rows; it sums every slice into LDS as
// k_combine does, then writes the run's rows to `out` as one contiguous run
// of non-temporal stores.
template <int KU>
__global__ void __launch_bounds__(kStageThreads)
    k_combine_staged(Dims d, PlanArrays pa, const u32x4* __restrict__ y,
                     const float* __restrict__ wnvs, int weighted, u32x4* __restrict__ out,
                     float* __restrict__ wsk, int lo, int nhi) {
  __shared__ u32x4 stage[kStageVec];
  __shared__ int sg[kStageRoutes];
  __shared__ float sw[kStageRoutes];
  if (pa.status[0] != 0) return;  // the same word for every thread of the grid
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  const int V = d.H / 8;
  const int nsl = (V + kWave - 1) / kWave;
  const int64_t b = blockIdx.x;
  const int64_t t0 = b < nhi ? b * (lo + 1) : (int64_t)nhi * (lo + 1) + (b - nhi) * lo;
  const int nt = b < nhi ? lo + 1 : lo;
  const int nr = nt * d.K;  // routes of the workgroup's tokens, at most kStageRoutes
  for (int i = threadIdx.x; i < nr; i += kStageThreads) {
    const int g = (int)dst_global_row(pa.dst[t0 * d.K + i]);
    const float w = wnvs != nullptr ? wnvs[g] : 0.0f;
    sg[i] = g;
    sw[i] = w;
    if (wsk != nullptr) wsk[t0 * d.K + i] = w;
  }
  __syncthreads();
  for (int it = wave; it < nt * nsl; it += kStageThreads / kWave) {
    const int lt = it / nsl, sl = it - lt * nsl;
    const int j = sl * kWave + lane;
    int gl = 0;
    float wl = 0.0f;
    if (lane < d.K) {
      gl = sg[lt * d.K + lane];
      wl = sw[lt * d.K + lane];
    }
    const u32x4 v = combine_slice<false, KU>(d, y, nullptr, weighted, lane, 0, gl, wl, j);
    if (j < V) stage[lt * V + j] = v;
  }
  __syncthreads();
  const int n = nt * V;
  u32x4* o = out + t0 * V;
  for (int b = 0; b < n; b += kStageThreads * kStageBatch) {
    u32x4 r[kStageBatch];
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
      const int i = b + u * kStageThreads + (int)threadIdx.x;
      if (i < n) r[u] = stage[i];
    }
#pragma unroll
    for (int u = 0; u < kStageBatch; ++u) {
      const int i = b + u * kStageThreads + (int)threadIdx.x;
      if (i < n) __builtin_nontemporal_store(r[u], o + i);
    }
  }
}

__global__ void k_prefetch_index(Dims d, PlanArrays pa, int32_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= d.R * d.B) return;
  const int ei = pa.etc[i];  // loaded alongside the status word
  const int e = pa.status[0] == 0 ? ei : -1;
  out[i * 2 + 0] = e >= 0 ? e / d.Eg : -1;
  out[i * 2 + 1] = e >= 0 ? e % d.Eg : -1;
}

// Staged workgroups: the fewest whole rounds of workgroups (one per compute
// unit at a time) whose runs fit the LDS block, at most one workgroup per
// token; the tokens are spread evenly over them (the first n % W get one
// more), so every round is full and the runs stay as long as they can be.
int64_t stage_groups(const Dims& d) {
  const int hi = min(kStageVec / (d.H / 8), kStageRoutes / d.K);
  const int64_t n = (int64_t)d.R * d.S;
  const int64_t ncu = d.ncu > 0 ? d.ncu : 256;
  const int64_t w = ((n + hi - 1) / hi + ncu - 1) / ncu * ncu;
  return w < n ? w : n;
}

}  // namespace

hipError_t launch_combine(const Dims& d, const PlanArrays& pa, const uint16_t* y,
                          const float* wnvs, bool weighted, uint16_t* fold, uint16_t* out,
                          float* wsk, hipStream_t s) {
  constexpr int KU = kCombineUnroll;
  const int V = d.H / 8;
  const int nsl = (V + kWave - 1) / kWave;
  const int64_t items = (int64_t)d.R * d.S * nsl;
  const int64_t blocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const auto* yv = reinterpret_cast<const u32x4*>(y);
  auto* fv = reinterpret_cast<u32x4*>(fold);
  auto* ov = reinterpret_cast<u32x4*>(out);
  if (fold != nullptr && d.K > 1) {
    // persistent grid over (duplicate group, slice) items, sized like the gather
    const int64_t want = (items + kWavesPerBlock - 1) / kWavesPerBlock;
    const int fblocks = (int)(want < kFoldBlocks ? (want > 0 ? want : 1) : kFoldBlocks);
    hipLaunchKernelGGL(k_combine_fold, dim3(fblocks), dim3(kThreads), 0, s, d, pa, yv, wnvs,
                       weighted ? 1 : 0, fv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_combine<true, KU>), dim3((unsigned)blocks), dim3(kThreads), 0, s, d,
                       pa, yv, wnvs, weighted ? 1 : 0, fv, ov, wsk);
    return hipGetLastError();
  }
  if (V <= kStageVec) {
    const int64_t n = (int64_t)d.R * d.S;
    const int64_t w = stage_groups(d);
    if (w > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_combine_staged<kStageUnroll>), dim3((unsigned)w), dim3(kStageThreads), 0,
                       s, d, pa, yv, wnvs, weighted ? 1 : 0, ov, wsk, (int)(n / w), (int)(n % w));
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_combine<false, KU>), dim3((unsigned)blocks), dim3(kThreads), 0, s, d, pa,
                     yv, wnvs, weighted ? 1 : 0, nullptr, ov, wsk);
  return hipGetLastError();
}

// Prefetch index (Guide, Buffer.prefetch_weight: a slot's global expert id
// names its home rank and its row on that rank; a -1 slot is unused).
hipError_t launch_prefetch_index(const Dims& d, const PlanArrays& pa, int32_t* out, hipStream_t s) {
  const int n = d.R * d.B;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(k_prefetch_index, dim3((n + 255) / 256), dim3(256), 0, s, d, pa, out);
  return hipGetLastError();
}

}  // namespace moon
