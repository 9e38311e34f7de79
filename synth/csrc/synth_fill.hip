// synth_fill.hip — GPU fill of the seeded bf16 "N(0,1)" input arrays.
//
// Input generation only: it draws synthetic activations and holds no part of
// the method.  Element j of a stream with key `key` is
//   table[ field (j mod 4) of  mix64(key + (j/4 + 1) * GAMMA) ]
// where mix64 is the SplitMix64 output function (Steele, Lea and Flood,
// OOPSLA 2014) and field f is bits [16f, 16f+16).  The same definition runs
// in numpy (synth.bf16_normal), so both produce identical bits.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// One thread per 64-bit word -> four consecutive bf16 values.  `start` is a
// multiple of 4 (checked on the host); `count` may end mid-word.
__global__ void __launch_bounds__(256) fill_bf16(uint16_t* __restrict__ out, int64_t count,
                                                 uint64_t key, uint64_t word0,
                                                 const uint16_t* __restrict__ table) {
  const int64_t nwords = (count + 3) / 4;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nwords;
       w += (int64_t)gridDim.x * blockDim.x) {
    uint64_t z = mix64(key + ((uint64_t)(word0 + w) + 1ull) * 0x9E3779B97F4A7C15ull);
    int64_t j = w * 4;
    if (j + 4 <= count) {
      ushort4 v;
      v.x = table[(z >> 0) & 0xFFFF];
      v.y = table[(z >> 16) & 0xFFFF];
      v.z = table[(z >> 32) & 0xFFFF];
      v.w = table[(z >> 48) & 0xFFFF];
      *reinterpret_cast<ushort4*>(out + j) = v;
    } else {
      for (int f = 0; f < 4 && j + f < count; ++f) out[j + f] = table[(z >> (16 * f)) & 0xFFFF];
    }
  }
}

}  // namespace

// Fill out[0..count) with elements start..start+count-1 of stream `key`.
// out must be 8-byte aligned; start must be a multiple of 4; table points to
// the 65536-entry device table.  Returns 0, or a HIP error code / -1.
extern "C" int synth_fill_bf16(uint16_t* out, int64_t count, uint64_t key, int64_t start,
                               const uint16_t* table, hipStream_t stream) {
  if (count < 0 || start < 0 || (start & 3) != 0 || out == nullptr || table == nullptr) return -1;
  if (((uintptr_t)out & 7) != 0) return -1;
  if (count == 0) return 0;
  int64_t nwords = (count + 3) / 4;
  int64_t blocks = (nwords + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(fill_bf16, dim3((unsigned)blocks), dim3(256), 0, stream, out, count, key,
                     (uint64_t)(start / 4), table);
  return (int)hipGetLastError();
}
