// moon_ceiling.hip — reference kernels for the benchmark (libmoon_ceiling.so,
// not part of libmoon): what the GPU's memory system delivers for the access
// patterns of dispatch and combine, each alone, on the same buffers and row
// lists the measured step uses.  They compute nothing of the method.
//
//   moon_ceiling_read        contiguous 16-byte non-temporal loads (discarded)
//   moon_ceiling_fill        contiguous 16-byte non-temporal stores of zero
//   moon_ceiling_copy        contiguous load + store
//   moon_ceiling_write_rows  dispatch's stores without its loads: for every
//                            token, a constant 2 KB slice stored to the rows
//                            of its K routes (the plan's dst), the same grid
//                            and order as the one-pass dispatch scatter
//   moon_ceiling_read_rows   combine's loads without its stores: for every
//                            token, 1 KB slices of its K routed rows loaded
//                            and discarded, one wave per token slice
//   moon_ceiling_scatter_cached  the one-pass dispatch scatter with its token
//                            rows served from the cache: token t stores the
//                            row of token t mod 4096 (58 MB at 14 KB rows,
//                            resident in the 256 MB last-level cache) to the
//                            rows of its K routes, same grid and order
//
// Loaded values are folded into one word that is stored only when `sink_on`
// is set (the host passes 0), so the loads cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWave = 64;

__device__ __forceinline__ int64_t row_of(int32_t v) { return v >= 0 ? v : -(int64_t)v - 1; }

__global__ void __launch_bounds__(256) k_read(const u32x4* __restrict__ p, int64_t n,
                                              uint32_t* sink, int sink_on) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (sink_on) sink[0] = acc;
}

__global__ void __launch_bounds__(256) k_fill(u32x4* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const u32x4 z = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(z, p + i);
}

__global__ void __launch_bounds__(256) k_copy(const u32x4* __restrict__ s, u32x4* __restrict__ d,
                                              int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(s + i), d + i);
}

constexpr int kRowSlice = 2;  // vectors per lane of a write_rows slice (as the dispatch scatter)

__global__ void __launch_bounds__(256) k_write_rows(u32x4* __restrict__ win,
                                                    const int32_t* __restrict__ dst, int64_t ntok,
                                                    int K, int V) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nsl = (V + kWave * kRowSlice - 1) / (kWave * kRowSlice);
  const int64_t items = ntok * nsl;
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t it = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; it < items;
       it += nw) {
    const int64_t t = it / nsl;
    const int c0 = (int)(it - t * nsl) * kWave * kRowSlice;
    const int dl = lane < K ? dst[t * K + lane] : 0;
    const u32x4 v = {(uint32_t)t, (uint32_t)c0, 0u, 0u};
#pragma unroll
    for (int c = 0; c < kRowSlice; ++c) {
      const int j = c0 + c * kWave + lane;
      for (int k = 0; k < K; ++k) {
        u32x4* dp = win + row_of(__builtin_amdgcn_readlane(dl, k)) * V;
        if (j < V) __builtin_nontemporal_store(v, dp + j);
      }
    }
  }
}

constexpr int64_t kCachedTokens = 4096;

__global__ void __launch_bounds__(256) k_scatter_cached(const u32x4* __restrict__ hidden,
                                                        u32x4* __restrict__ win,
                                                        const int32_t* __restrict__ dst,
                                                        int64_t ntok, int K, int V) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nsl = (V + kWave * kRowSlice - 1) / (kWave * kRowSlice);
  const int64_t items = ntok * nsl;
  const int64_t nw = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t it = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave; it < items;
       it += nw) {
    const int64_t t = it / nsl;
    const int c0 = (int)(it - t * nsl) * kWave * kRowSlice;
    const int dl = lane < K ? dst[t * K + lane] : 0;
    const u32x4* src = hidden + (t % kCachedTokens) * V;
    u32x4 buf[kRowSlice];
#pragma unroll
    for (int c = 0; c < kRowSlice; ++c) {
      const int j = c0 + c * kWave + lane;
      if (j < V) buf[c] = src[j];
    }
#pragma unroll
    for (int c = 0; c < kRowSlice; ++c) {
      const int j = c0 + c * kWave + lane;
      for (int k = 0; k < K; ++k) {
        u32x4* dp = win + row_of(__builtin_amdgcn_readlane(dl, k)) * V;
        if (j < V) __builtin_nontemporal_store(buf[c], dp + j);
      }
    }
  }
}

__global__ void __launch_bounds__(1024) k_read_rows(const u32x4* __restrict__ y,
                                                    const int32_t* __restrict__ dst, int64_t ntok,
                                                    int K, int V, uint32_t* sink, int sink_on) {
  const int lane = threadIdx.x & (kWave - 1);
  const int nsl = (V + kWave - 1) / kWave;
  const int64_t item = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (item >= ntok * nsl) return;
  const int64_t t = item / nsl;
  const int j = (int)(item - t * nsl) * kWave + lane;
  const int dl = lane < K ? dst[t * K + lane] : 0;
  uint32_t acc = 0;
  for (int k = 0; k < K; ++k) {
    const u32x4* row = y + row_of(__builtin_amdgcn_readlane(dl, k)) * V;
    if (j < V) {
      const u32x4 v = __builtin_nontemporal_load(row + j);
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (sink_on) sink[0] = acc;
}

int grid_for(int64_t n, int per_block, int cap) {
  const int64_t want = (n + per_block - 1) / per_block;
  return (int)(want < cap ? (want > 0 ? want : 1) : cap);
}

}  // namespace

extern "C" {

// Sizes in bytes must be positive multiples of 16 and pointers 16-byte
// aligned; returns a hipError_t value (0 on success).
int moon_ceiling_read(const void* p, int64_t bytes, void* sink4, hipStream_t s) {
  if (p == nullptr || sink4 == nullptr || bytes <= 0 || bytes % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read, dim3(grid_for(bytes / 16, 256, 32768)), dim3(256), 0, s,
                     static_cast<const u32x4*>(p), bytes / 16, static_cast<uint32_t*>(sink4), 0);
  return hipGetLastError();
}

int moon_ceiling_fill(void* p, int64_t bytes, hipStream_t s) {
  if (p == nullptr || bytes <= 0 || bytes % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_fill, dim3(grid_for(bytes / 16, 256, 32768)), dim3(256), 0, s,
                     static_cast<u32x4*>(p), bytes / 16);
  return hipGetLastError();
}

int moon_ceiling_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  if (src == nullptr || dst == nullptr || bytes <= 0 || bytes % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_copy, dim3(grid_for(bytes / 16, 256, 32768)), dim3(256), 0, s,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), bytes / 16);
  return hipGetLastError();
}

// win: [rows, H] bf16; dst [ntok, K] int32 entries +G or -(G+1) with every
// G a row of win (a plan of libmoon and its context windows); H a multiple
// of 8.
int moon_ceiling_write_rows(void* win, const int32_t* dst, int64_t ntok, int K, int H,
                            hipStream_t s) {
  if (win == nullptr || dst == nullptr || ntok <= 0 || K < 1 || K > kWave || H < 8 || H % 8)
    return hipErrorInvalidValue;
  const int V = H / 8;
  const int nsl = (V + kWave * kRowSlice - 1) / (kWave * kRowSlice);
  hipLaunchKernelGGL(k_write_rows, dim3(grid_for(ntok * nsl, 4, 32768)), dim3(256), 0, s,
                     static_cast<u32x4*>(win), dst, ntok, K, V);
  return hipGetLastError();
}

// hidden: [ntok, H] bf16 (only its first min(ntok, 4096) rows are read);
// win and dst as for moon_ceiling_write_rows.
int moon_ceiling_scatter_cached(const void* hidden, void* win, const int32_t* dst, int64_t ntok,
                                int K, int H, hipStream_t s) {
  if (hidden == nullptr || win == nullptr || dst == nullptr || ntok <= 0 || K < 1 || K > kWave ||
      H < 8 || H % 8)
    return hipErrorInvalidValue;
  const int V = H / 8;
  const int nsl = (V + kWave * kRowSlice - 1) / (kWave * kRowSlice);
  hipLaunchKernelGGL(k_scatter_cached, dim3(grid_for(ntok * nsl, 4, 32768)), dim3(256), 0, s,
                     static_cast<const u32x4*>(hidden), static_cast<u32x4*>(win), dst, ntok, K, V);
  return hipGetLastError();
}

// y: [rows, H] bf16 with the same condition on dst.
int moon_ceiling_read_rows(const void* y, const int32_t* dst, int64_t ntok, int K, int H,
                           void* sink4, hipStream_t s) {
  if (y == nullptr || dst == nullptr || sink4 == nullptr || ntok <= 0 || K < 1 || K > kWave ||
      H < 8 || H % 8)
    return hipErrorInvalidValue;
  const int V = H / 8;
  const int64_t items = ntok * ((V + kWave - 1) / kWave);
  const int64_t blocks = (items + 15) / 16;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_read_rows, dim3((unsigned)blocks), dim3(1024), 0, s,
                     static_cast<const u32x4*>(y), dst, ntok, K, V,
                     static_cast<uint32_t*>(sink4), 0);
  return hipGetLastError();
}

}  // extern "C"
