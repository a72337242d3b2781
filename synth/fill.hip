// Device-side twin of synth.values(): fills a contiguous [n_tokens][heads][dim]
// buffer with the counter-based N(0,1) stream described in synth/__init__.py.
// Integer-only (hash + table lookup), so it is bit-identical to the numpy form.
#include <hip/hip_runtime.h>
#include <stdint.h>

__device__ __forceinline__ uint32_t lowbias32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

template <typename T>
__global__ void fill_kernel(T* __restrict__ dst, int64_t n, uint32_t e0, uint32_t key,
                            const T* __restrict__ table) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) {
    uint32_t e = e0 + (uint32_t)i + key;
    dst[i] = table[lowbias32(e) >> 16];
  }
}

extern "C" int synth_fill(void* dst, int64_t n_tokens, int64_t t0, int32_t heads, int32_t dim,
                          uint32_t key, int32_t elem_bytes, const void* table, void* stream) {
  if (n_tokens < 0 || heads <= 0 || dim <= 0 || !dst || !table) return -1;
  const int64_t n = n_tokens * heads * dim;
  if (n == 0) return 0;
  const uint32_t e0 = (uint32_t)((uint64_t)t0 * (uint64_t)heads * (uint64_t)dim);
  const int threads = 256;
  int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = (hipStream_t)stream;
  if (elem_bytes == 2) {
    hipLaunchKernelGGL(fill_kernel<uint16_t>, dim3((unsigned)blocks), dim3(threads), 0, s,
                       (uint16_t*)dst, n, e0, key, (const uint16_t*)table);
  } else if (elem_bytes == 4) {
    hipLaunchKernelGGL(fill_kernel<uint32_t>, dim3((unsigned)blocks), dim3(threads), 0, s,
                       (uint32_t*)dst, n, e0, key, (const uint32_t*)table);
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
