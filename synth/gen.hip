// GPU fill of synthetic tensors with the counter-based definition of synth/weights.py:
// element i = table[(mix64(key + (i/4 + 1) * GOLDEN) >> (16 * (i % 4))) & 0xFFFF],
// mix64 = the SplitMix64 finaliser.  Input generation only; bit-identical to the CPU generator.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ull;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBull;
  z ^= z >> 31;
  return z;
}

template <typename E>
__global__ void fill_kernel(E *dst, uint64_t n, uint64_t key, const E *table) {
  const uint64_t words = (n + 3) / 4;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < words; j += stride) {
    const uint64_t w = mix64(key + (j + 1) * 0x9E3779B97F4A7C15ull);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const uint64_t i = 4 * j + s;
      if (i < n) dst[i] = table[(w >> (16 * s)) & 0xFFFFu];
    }
  }
}

}  // namespace

extern "C" int synth_fill(void *dst, uint64_t n, uint64_t key, const void *table, int elem_bytes, hipStream_t s) {
  if (n == 0) return 0;
  const uint64_t words = (n + 3) / 4;
  const uint64_t blocks = words / 256 + 1;
  const unsigned grid = (unsigned)(blocks < 65536 ? blocks : 65536);
  if (elem_bytes == 2)
    hipLaunchKernelGGL(fill_kernel<uint16_t>, dim3(grid), dim3(256), 0, s, (uint16_t *)dst, n, key, (const uint16_t *)table);
  else if (elem_bytes == 4)
    hipLaunchKernelGGL(fill_kernel<uint32_t>, dim3(grid), dim3(256), 0, s, (uint32_t *)dst, n, key, (const uint32_t *)table);
  else
    return -1;
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
