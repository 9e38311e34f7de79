// moon_combine.hip — gather-reduce combine, route-weight gather, prefetch index.
//
// ("MoonEP Public API Visual Guide", Buffer.combine: the reverse of dispatch;
//  each token's K routed rows, located through plan.dst, are summed back into
//  token order, and the route weights are read back through the same signed
//  entries.)
//
// A work item is one wave on a slice of 64 vectors (512 bf16) of one token's
// row.  Lanes 0..K-1 decode the token's K dst entries (both signs: every
// route owns its row) and fetch the K route weights; the loop over k reads
// two routed slices at a time with 16-byte loads, widens bf16 to fp32 and
// accumulates c_k * y in ascending k with a separate multiply and add (the
// library is built with -ffp-contract=off), then rounds once to bf16
// (nearest, ties to even).  Bound: HBM bandwidth (K row reads + one row
// write per token).
#include "moon_internal.h"

namespace moon {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kThreads = kWavesPerBlock * kWave;
constexpr int kUnroll = 2;  // routed slices in flight per wave

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ void __launch_bounds__(kThreads)
    k_combine(Dims d, PlanArrays pa, const u32x4* __restrict__ y, const float* __restrict__ wnvs,
              int weighted, u32x4* __restrict__ out, float* __restrict__ wsk) {
  if (pa.status[0] != 0) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int V = d.H / 8;
  const int nsl = (V + kWave - 1) / kWave;
  const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (item >= (int64_t)d.R * d.S * nsl) return;
  const int64_t t = item / nsl;
  const int sl = (int)(item - t * nsl);
  const int j = sl * kWave + lane;  // this lane's vector of the row
  int gl = 0;
  float wl = 0.0f;
  if (lane < d.K) {
    gl = (int)dst_global_row(pa.dst[t * d.K + lane]);
    if (wnvs != nullptr) wl = wnvs[gl];
    if (wsk != nullptr && sl == 0) wsk[t * d.K + lane] = wl;
  }
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  for (int k0 = 0; k0 < d.K; k0 += kUnroll) {
    u32x4 buf[kUnroll];
    float ck[kUnroll];
#pragma unroll
    for (int uu = 0; uu < kUnroll; ++uu) {
      const int k = min(k0 + uu, d.K - 1);
      const int G = __builtin_amdgcn_readlane(gl, k);
      ck[uu] = weighted ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wl), k)) : 1.0f;
      if (j < V && k0 + uu < d.K) buf[uu] = __builtin_nontemporal_load(y + (int64_t)G * V + j);
    }
#pragma unroll
    for (int uu = 0; uu < kUnroll; ++uu) {
      if (k0 + uu >= d.K) break;
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
    __builtin_nontemporal_store(v, out + t * V + j);
  }
}

__global__ void k_prefetch_index(Dims d, PlanArrays pa, int32_t* __restrict__ out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= d.R * d.B) return;
  const bool ok = pa.status[0] == 0;
  const int e = ok ? pa.etc[i] : -1;
  out[i * 2 + 0] = e >= 0 ? e / d.Eg : -1;
  out[i * 2 + 1] = e >= 0 ? e % d.Eg : -1;
}

}  // namespace

hipError_t launch_combine(const Dims& d, const PlanArrays& pa, const uint16_t* y,
                          const float* wnvs, bool weighted, uint16_t* out, float* wsk,
                          hipStream_t s) {
  const int nsl = (d.H / 8 + kWave - 1) / kWave;
  const int64_t items = (int64_t)d.R * d.S * nsl;
  const int64_t blocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_combine, dim3((unsigned)blocks), dim3(kThreads), 0, s, d, pa,
                     reinterpret_cast<const u32x4*>(y), wnvs, weighted ? 1 : 0,
                     reinterpret_cast<u32x4*>(out), wsk);
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
