// moon_combine.hip — gather-reduce combine, duplicate prologue, route-weight
// gather, prefetch index.
//
// ("MoonEP Public API Visual Guide", Buffer.combine: the reverse of dispatch;
//  each token's K routed rows, located through plan.dst, are summed back into
//  token order, and the route weights are read back through the same signed
//  entries.  A prologue may first fold the duplicate rows of a token on one
//  destination rank into that rank's primary row in fp32.)
//
// k_combine: a work item is one wave on a slice of 64 vectors (512 bf16) of
// one token's row.  Lanes 0..K-1 decode the token's K dst entries (both
// signs: every route owns its row) and fetch the K route weights; the loop
// over k reads two routed slices at a time with 16-byte loads, widens bf16
// to fp32 and accumulates c_k * y in ascending k with a separate multiply
// and add (the library is built with -ffp-contract=off), then rounds once to
// bf16 (nearest, ties to even).  Bound: HBM bandwidth (K row reads + one row
// write per token).
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
constexpr int kCombineSliceVec = 1;  // 16-byte vectors per lane in a gather slice
constexpr int kCombineUnroll = 2;    // routed rows loaded before they are summed
constexpr bool kCombineNtLoad = true;   // routed rows are read once: non-temporal loads
constexpr bool kCombineNtStore = true;  // outputs are not read back here: non-temporal stores
constexpr int kFoldBlocks = 8192;  // persistent grid of the prologue

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

template <bool PROLOGUE, int SV, int KU>
__global__ void __launch_bounds__(kThreads)
    k_combine(Dims d, PlanArrays pa, const u32x4* __restrict__ y, const float* __restrict__ wnvs,
              int weighted, const u32x4* __restrict__ fold, u32x4* __restrict__ out,
              float* __restrict__ wsk) {
  constexpr int SW = kWave * SV;  // vectors per slice
  const int lane = threadIdx.x & (kWave - 1);
  const int V = d.H / 8;
  const int nsl = (V + SW - 1) / SW;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (item >= (int64_t)d.R * d.S * nsl) return;
  const int64_t t = item / nsl;
  const int sl = (int)(item - t * nsl);
  const int j0 = sl * SW + lane;  // this lane's vectors: j0 + c * kWave
  int gl = 0, dl = 0;
  float wl = 0.0f;
  // The dst entries are read before the plan's status is checked, so the two
  // loads overlap; nothing read before the check is used unless it is zero.
  if (lane < d.K) dl = pa.dst[t * d.K + lane];
  if (pa.status[0] != 0) return;
  if (lane < d.K) {
    gl = (int)dst_global_row(dl);
    if (wnvs != nullptr) wl = wnvs[gl];
    if (wsk != nullptr && sl == 0) wsk[t * d.K + lane] = wl;
  }
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
  float acc[SV][8];
#pragma unroll
  for (int c = 0; c < SV; ++c)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[c][e] = 0.0f;
  for (int k0 = 0; k0 < d.K; k0 += KU) {
    u32x4 buf[KU][SV];
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
#pragma unroll
      for (int c = 0; c < SV; ++c) {
        const int j = j0 + c * kWave;
        if (j < V && use[uu])
          buf[uu][c] = kCombineNtLoad ? __builtin_nontemporal_load(row + j) : row[j];
      }
    }
#pragma unroll
    for (int uu = 0; uu < KU; ++uu) {
      if (!use[uu]) continue;
#pragma unroll
      for (int c = 0; c < SV; ++c)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[c][2 * q + 0] = acc[c][2 * q + 0] + ck[uu] * bf16_lo(buf[uu][c][q]);
          acc[c][2 * q + 1] = acc[c][2 * q + 1] + ck[uu] * bf16_hi(buf[uu][c][q]);
        }
    }
  }
#pragma unroll
  for (int c = 0; c < SV; ++c) {
    const int j = j0 + c * kWave;
    if (j < V) {
      u32x4 v;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = bf16_rne(acc[c][2 * q]) | (bf16_rne(acc[c][2 * q + 1]) << 16);
      if (kCombineNtStore) __builtin_nontemporal_store(v, out + t * V + j);
      else out[t * V + j] = v;
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

}  // namespace

hipError_t launch_combine(const Dims& d, const PlanArrays& pa, const uint16_t* y,
                          const float* wnvs, bool weighted, uint16_t* fold, uint16_t* out,
                          float* wsk, hipStream_t s) {
  constexpr int SV = kCombineSliceVec, KU = kCombineUnroll;
  const int nsl = (d.H / 8 + kWave * SV - 1) / (kWave * SV);
  const int64_t items = (int64_t)d.R * d.S * nsl;
  const int64_t blocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const auto* yv = reinterpret_cast<const u32x4*>(y);
  auto* fv = reinterpret_cast<u32x4*>(fold);
  if (fold != nullptr && d.K > 1) {
    // persistent grid over (duplicate group, slice) items, sized like the gather
    const int fnsl = (d.H / 8 + kWave - 1) / kWave;
    const int64_t fw = (int64_t)d.R * d.S * fnsl;
    const int64_t want = (fw + kWavesPerBlock - 1) / kWavesPerBlock;
    const int fblocks = (int)(want < kFoldBlocks ? (want > 0 ? want : 1) : kFoldBlocks);
    hipLaunchKernelGGL(k_combine_fold, dim3(fblocks), dim3(kThreads), 0, s, d, pa, yv, wnvs,
                       weighted ? 1 : 0, fv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_combine<true, SV, KU>), dim3((unsigned)blocks), dim3(kThreads), 0, s, d,
                       pa, yv, wnvs, weighted ? 1 : 0, fv, reinterpret_cast<u32x4*>(out), wsk);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((k_combine<false, SV, KU>), dim3((unsigned)blocks), dim3(kThreads), 0, s, d,
                     pa, yv, wnvs, weighted ? 1 : 0, nullptr, reinterpret_cast<u32x4*>(out), wsk);
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
