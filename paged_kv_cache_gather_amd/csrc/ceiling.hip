// Read-only bandwidth passes that the benchmark sets beside the decode
// kernels: the same (block, KV head) tiles a decode step reads through its
// block tables ("How the attention kernel actually reads paged blocks", vLLM
// Serving deep dive: block by block, wherever the table points), read once
// each with no attention arithmetic, and a plain contiguous read of the same
// number of bytes.  They measure what the chip gives for that access pattern
// (the practical ceiling of an HBM-bound kernel), not anything the method
// computes.
//
// One 256-thread workgroup takes kItems 16-byte chunks per thread round: item
// i of the launch is chunk i % C of list entry i / C (C = tile_bytes / 16),
// so consecutive lanes read consecutive bytes of a tile and a wave
// instruction covers 1 KiB.  Each thread has kUnroll loads in flight before
// it folds them into a running XOR; the result is stored only if it hits a
// constant, which keeps every load alive without a store per thread.
#include <string>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kCeilThreads = 256;
constexpr int kUnroll = 8;

__global__ void __launch_bounds__(kCeilThreads)
read_tiles_kernel(const unsigned char* __restrict__ kpool, const unsigned char* __restrict__ vpool,
                  const int64_t* __restrict__ tiles, int64_t n_k, int64_t n, int64_t tile_bytes,
                  uint32_t* __restrict__ sink) {
  const int64_t C = tile_bytes / 16;  // chunks per tile
  const int64_t total = n * C;
  const int64_t base = (int64_t)blockIdx.x * kCeilThreads * kUnroll + threadIdx.x;
  u32x4 v[kUnroll];
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) {
    const int64_t item = base + (int64_t)u * kCeilThreads;
    if (item < total) {
      const int64_t e = item / C, c = item % C;
      const int64_t t = tiles ? tiles[e] : e;
      const unsigned char* pool = e < n_k ? kpool : vpool;
      v[u] = ld16(pool + t * tile_bytes + c * 16);
    } else {
      v[u] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  uint32_t x = 0;
#pragma unroll
  for (int u = 0; u < kUnroll; ++u) x ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  if (x == 0x9e3779b9u) sink[0] = x;
}

}  // namespace
}  // namespace pkv

using pkv::fail;
using pkv::ok;

extern "C" int paged_kv_read_tiles(const void* k_pool, const void* v_pool, const int64_t* tiles, int64_t n_k_tiles,
                                   int64_t n_tiles, int64_t tile_bytes, uint32_t* sink, void* stream) {
  if (n_tiles < 0 || n_k_tiles < 0 || n_k_tiles > n_tiles)
    return fail(PKV_EINVAL, "paged_kv_read_tiles: bad tile counts");
  if (!tiles && n_k_tiles != n_tiles)
    return fail(PKV_EINVAL, "paged_kv_read_tiles: a contiguous read (tiles NULL) reads k_pool only");
  if (n_tiles == 0) return ok();
  if (!k_pool || !sink || (n_k_tiles < n_tiles && !v_pool))
    return fail(PKV_EINVAL, "paged_kv_read_tiles: NULL pointer");
  if (tile_bytes <= 0 || tile_bytes % 16 || !pkv::aligned16(k_pool) || (v_pool && !pkv::aligned16(v_pool)))
    return fail(PKV_EINVAL, "paged_kv_read_tiles: tiles must be 16-byte multiples at 16-byte aligned pools");
  const int64_t items = n_tiles * (tile_bytes / 16);
  const int64_t per_wg = (int64_t)pkv::kCeilThreads * pkv::kUnroll;
  const int64_t grid = (items + per_wg - 1) / per_wg;
  if (grid > 0x7fffffffll) return fail(PKV_EINVAL, "paged_kv_read_tiles: too many tiles for one launch");
  hipLaunchKernelGGL(pkv::read_tiles_kernel, dim3((unsigned)grid), dim3(pkv::kCeilThreads), 0, (hipStream_t)stream,
                     (const unsigned char*)k_pool, (const unsigned char*)v_pool, tiles, n_k_tiles, n_tiles,
                     tile_bytes, sink);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("paged_kv_read_tiles: ") + hipGetErrorString(e));
  return ok();
}
