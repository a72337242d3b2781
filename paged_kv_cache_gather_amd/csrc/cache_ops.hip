// Cache writes: reshape_and_cache (append new tokens' K/V into their slots),
// paged_kv_copy_blocks (whole-block copies for copy-on-write) and
// paged_kv_swap_blocks (whole-block copies between the HBM pools and pools of
// pinned host blocks, for swapping).
//
// reshape_and_cache and paged_kv_copy_blocks are byte copies;
// reshape_and_cache_fp8 quantises 32- or 16-bit rows into an 8-bit pool on the
// way (the 8-bit cache of "Quantization", vLLM Serving deep dive), with the
// same chunk walk.  reshape_and_cache reads each new token's K and V row
// in 16-byte chunks and writes them into the pool layout: a K chunk stays a
// contiguous 16-byte unit (the layout keeps x = 16/esize consecutive dims of
// one token together), while a V chunk is spread over x dim-rows, one
// element each, since V tiles are dim-major.  Consecutive lanes take
// consecutive tokens, so tokens that fill one block (a prefill chunk) write
// contiguous runs.  The per-item bodies (cache_write_chunk,
// cache_write_chunk_fp8) live in pkv_device.h: the decode launch of
// paged_attention_decode_append uses them too.
#include <cmath>
#include <string>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

template <int ES>
__global__ void __launch_bounds__(256)
reshape_and_cache_kernel(const unsigned char* __restrict__ key, const unsigned char* __restrict__ value,
                         int64_t kstride_b, int64_t vstride_b, unsigned char* __restrict__ kpool,
                         unsigned char* __restrict__ vpool, const int64_t* __restrict__ slots,
                         int64_t T, int64_t num_slots, int H, int D) {
  const int C = D * ES / 16;  // chunks per head row
  const int64_t total = T * H * C;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx % T;
    const int64_t rest = idx / T;
    cache_write_chunk<ES>(key, value, kstride_b, vstride_b, kpool, vpool, slots[i], num_slots, i,
                          (int)(rest % H), (int)(rest / H), H, D);
  }
}

// One work item = one 16-dim chunk of one token's head row: the K chunk is
// one 16-byte store, the V chunk 16 one-byte stores (dim-major V).
template <typename S>
__global__ void __launch_bounds__(256)
reshape_and_cache_fp8_kernel(const unsigned char* __restrict__ key, const unsigned char* __restrict__ value,
                             int64_t kstride_b, int64_t vstride_b, unsigned char* __restrict__ kpool,
                             unsigned char* __restrict__ vpool, const int64_t* __restrict__ slots, int64_t T,
                             int64_t num_slots, int H, int D, float k_inv, float v_inv) {
  const int C = D / 16;
  const int64_t total = T * H * C;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t i = idx % T;
    const int64_t rest = idx / T;
    cache_write_chunk_fp8<S>(key, value, kstride_b, vstride_b, kpool, vpool, slots[i], num_slots, i,
                             (int)(rest % H), (int)(rest / H), H, D, k_inv, v_inv);
  }
}

__global__ void __launch_bounds__(256)
copy_blocks_kernel(unsigned char* __restrict__ kpool, unsigned char* __restrict__ vpool,
                   const int32_t* __restrict__ pairs, int64_t num_blocks, int64_t block_bytes) {
  const int64_t src = pairs[2 * blockIdx.x];
  const int64_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks || src == dst) return;
  const int64_t n16 = block_bytes / 16;
  for (int64_t j = threadIdx.x; j < n16; j += blockDim.x) {
    st16(kpool + dst * block_bytes + j * 16, ld16(kpool + src * block_bytes + j * 16));
    st16(vpool + dst * block_bytes + j * 16, ld16(vpool + src * block_bytes + j * 16));
  }
}

// Whole blocks from one pool pair to another, either side in HBM or in pinned
// host memory (read and written by the kernel over the host link).  Grid
// (pair, K or V): 256 threads stream the block, four 16-byte loads in flight
// per thread before their stores.
__global__ void __launch_bounds__(256)
swap_blocks_kernel(const unsigned char* __restrict__ src_k, const unsigned char* __restrict__ src_v,
                   unsigned char* __restrict__ dst_k, unsigned char* __restrict__ dst_v,
                   const int32_t* __restrict__ pairs, int64_t src_num_blocks, int64_t dst_num_blocks,
                   int64_t block_bytes) {
  const int64_t src = pairs[2 * (int64_t)blockIdx.x];
  const int64_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  if (src < 0 || dst < 0 || src >= src_num_blocks || dst >= dst_num_blocks) return;
  const unsigned char* s = (blockIdx.y ? src_v : src_k) + src * block_bytes;
  unsigned char* d = (blockIdx.y ? dst_v : dst_k) + dst * block_bytes;
  const int64_t n16 = block_bytes / 16;
  for (int64_t j = threadIdx.x; j < n16; j += 4 * 256) {
    u32x4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j + u * 256 < n16) v[u] = ld16(s + (j + u * 256) * 16);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j + u * 256 < n16) st16(d + (j + u * 256) * 16, v[u]);
  }
}

// The address a kernel uses for p: device memory as is, pinned host memory
// through its device mapping; nullptr for memory a kernel cannot reach.
const void* device_view(const void* p) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess) {
    (void)hipGetLastError();  // do not leave the error for the next call
    return nullptr;
  }
  if (a.type == hipMemoryTypeDevice) return p;
  if (a.type == hipMemoryTypeHost && a.devicePointer) {
    const char* base_h = static_cast<const char*>(a.hostPointer ? a.hostPointer : p);
    return static_cast<const char*>(a.devicePointer) + (static_cast<const char*>(p) - base_h);
  }
  return nullptr;
}

}  // namespace
}  // namespace pkv

using pkv::fail;
using pkv::ok;

extern "C" int reshape_and_cache(const void* key, const void* value, int64_t key_token_stride,
                                 int64_t value_token_stride, void* k_pool, void* v_pool,
                                 const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                                 int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                 int32_t dtype, void* stream) {
  const int es = pkv::esize_of(dtype);
  if (!es) return fail(PKV_EINVAL, "reshape_and_cache: unknown dtype");
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size must be 16");
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (num_tokens < 0 || num_blocks < 1 || n_kv_heads < 1)
    return fail(PKV_EINVAL, "reshape_and_cache: bad sizes");
  if (num_tokens == 0) return ok();
  if (!key || !value || !k_pool || !v_pool || !slot_mapping)
    return fail(PKV_EINVAL, "reshape_and_cache: NULL pointer");
  const int64_t row = (int64_t)n_kv_heads * head_dim;
  if (key_token_stride < row || value_token_stride < row)
    return fail(PKV_EINVAL, "reshape_and_cache: token stride shorter than a row");
  if (!pkv::aligned16(key) || !pkv::aligned16(value) || !pkv::aligned16(k_pool) ||
      !pkv::aligned16(v_pool) || (key_token_stride * es) % 16 || (value_token_stride * es) % 16)
    return fail(PKV_EINVAL, "reshape_and_cache: pointers and strides must be 16-byte aligned");
  const int64_t total = num_tokens * n_kv_heads * (head_dim * es / 16);
  int64_t grid = (total + 255) / 256;
  if (grid > 16384) grid = 16384;
  hipStream_t s = (hipStream_t)stream;
  const int64_t num_slots = num_blocks * pkv::kBlockSize;
  if (es == 1) {
    hipLaunchKernelGGL(pkv::reshape_and_cache_kernel<1>, dim3((unsigned)grid), dim3(256), 0, s,
                       (const unsigned char*)key, (const unsigned char*)value, key_token_stride,
                       value_token_stride, (unsigned char*)k_pool, (unsigned char*)v_pool,
                       slot_mapping, num_tokens, num_slots, n_kv_heads, head_dim);
  } else if (es == 4) {
    hipLaunchKernelGGL(pkv::reshape_and_cache_kernel<4>, dim3((unsigned)grid), dim3(256), 0, s,
                       (const unsigned char*)key, (const unsigned char*)value, key_token_stride * 4,
                       value_token_stride * 4, (unsigned char*)k_pool, (unsigned char*)v_pool,
                       slot_mapping, num_tokens, num_slots, n_kv_heads, head_dim);
  } else {
    hipLaunchKernelGGL(pkv::reshape_and_cache_kernel<2>, dim3((unsigned)grid), dim3(256), 0, s,
                       (const unsigned char*)key, (const unsigned char*)value, key_token_stride * 2,
                       value_token_stride * 2, (unsigned char*)k_pool, (unsigned char*)v_pool,
                       slot_mapping, num_tokens, num_slots, n_kv_heads, head_dim);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("reshape_and_cache: ") + hipGetErrorString(e));
  return ok();
}

extern "C" int reshape_and_cache_fp8(const void* key, const void* value, int32_t src_dtype,
                                     int64_t key_token_stride, int64_t value_token_stride, void* k_pool,
                                     void* v_pool, const int64_t* slot_mapping, int64_t num_tokens,
                                     int64_t num_blocks, int32_t n_kv_heads, int32_t head_dim,
                                     int32_t block_size, float k_scale, float v_scale, void* stream) {
  if (src_dtype != PKV_F32 && src_dtype != PKV_F16 && src_dtype != PKV_BF16)
    return fail(PKV_EINVAL, "reshape_and_cache_fp8: source dtype must be f32, f16 or bf16");
  const int es = pkv::esize_of(src_dtype);
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size must be 16");
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (num_tokens < 0 || num_blocks < 1 || n_kv_heads < 1)
    return fail(PKV_EINVAL, "reshape_and_cache_fp8: bad sizes");
  if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f))
    return fail(PKV_EINVAL, "reshape_and_cache_fp8: scales must be finite and > 0");
  if (num_tokens == 0) return ok();
  if (!key || !value || !k_pool || !v_pool || !slot_mapping)
    return fail(PKV_EINVAL, "reshape_and_cache_fp8: NULL pointer");
  const int64_t row = (int64_t)n_kv_heads * head_dim;
  if (key_token_stride < row || value_token_stride < row)
    return fail(PKV_EINVAL, "reshape_and_cache_fp8: token stride shorter than a row");
  if (!pkv::aligned16(key) || !pkv::aligned16(value) || !pkv::aligned16(k_pool) ||
      !pkv::aligned16(v_pool) || (key_token_stride * es) % 16 || (value_token_stride * es) % 16)
    return fail(PKV_EINVAL, "reshape_and_cache_fp8: pointers and strides must be 16-byte aligned");
  // the reciprocals are rounded to nearest once, here (IEEE fp32 division)
  const float k_inv = 1.0f / k_scale, v_inv = 1.0f / v_scale;
  if (!std::isfinite(k_inv) || !std::isfinite(v_inv))
    return fail(PKV_EINVAL, "reshape_and_cache_fp8: scale too small");
  const int64_t total = num_tokens * n_kv_heads * (head_dim / 16);
  int64_t grid = (total + 255) / 256;
  if (grid > 16384) grid = 16384;
  hipStream_t s = (hipStream_t)stream;
  const int64_t num_slots = num_blocks * pkv::kBlockSize;
  auto launch = [&](auto src) {
    using S = decltype(src);
    hipLaunchKernelGGL(pkv::reshape_and_cache_fp8_kernel<S>, dim3((unsigned)grid), dim3(256), 0, s,
                       (const unsigned char*)key, (const unsigned char*)value, key_token_stride * es,
                       value_token_stride * es, (unsigned char*)k_pool, (unsigned char*)v_pool, slot_mapping,
                       num_tokens, num_slots, n_kv_heads, head_dim, k_inv, v_inv);
  };
  if (src_dtype == PKV_F32)
    launch(pkv::F32{});
  else if (src_dtype == PKV_F16)
    launch(pkv::F16{});
  else
    launch(pkv::BF16{});
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("reshape_and_cache_fp8: ") + hipGetErrorString(e));
  return ok();
}

extern "C" int paged_kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs_dev,
                                    int32_t n_pairs, int64_t num_blocks, int32_t n_kv_heads,
                                    int32_t head_dim, int32_t block_size, int32_t dtype,
                                    void* stream) {
  const int es = pkv::esize_of(dtype);
  if (!es) return fail(PKV_EINVAL, "paged_kv_copy_blocks: unknown dtype");
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size must be 16");
  if (n_pairs < 0 || num_blocks < 1 || n_kv_heads < 1 || head_dim < 1)
    return fail(PKV_EINVAL, "paged_kv_copy_blocks: bad sizes");
  if (n_pairs == 0) return ok();
  if (!k_pool || !v_pool || !pairs_dev) return fail(PKV_EINVAL, "paged_kv_copy_blocks: NULL pointer");
  if (!pkv::aligned16(k_pool) || !pkv::aligned16(v_pool))
    return fail(PKV_EINVAL, "paged_kv_copy_blocks: pools must be 16-byte aligned");
  const int64_t block_bytes = (int64_t)n_kv_heads * block_size * head_dim * es;
  if (block_bytes % 16) return fail(PKV_EINVAL, "paged_kv_copy_blocks: block not a multiple of 16 B");
  hipLaunchKernelGGL(pkv::copy_blocks_kernel, dim3((unsigned)n_pairs), dim3(256), 0,
                     (hipStream_t)stream, (unsigned char*)k_pool, (unsigned char*)v_pool, pairs_dev,
                     num_blocks, block_bytes);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("paged_kv_copy_blocks: ") + hipGetErrorString(e));
  return ok();
}

extern "C" int paged_kv_swap_blocks(const void* src_k_pool, const void* src_v_pool, int64_t src_num_blocks,
                                    void* dst_k_pool, void* dst_v_pool, int64_t dst_num_blocks,
                                    const int32_t* pairs, int32_t n_pairs, int32_t n_kv_heads, int32_t head_dim,
                                    int32_t block_size, int32_t dtype, void* stream) {
  const int es = pkv::esize_of(dtype);
  if (!es) return fail(PKV_EINVAL, "paged_kv_swap_blocks: unknown dtype");
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size must be 16");
  if (n_pairs < 0 || src_num_blocks < 1 || dst_num_blocks < 1 || n_kv_heads < 1 || head_dim < 1)
    return fail(PKV_EINVAL, "paged_kv_swap_blocks: bad sizes");
  if (n_pairs == 0) return ok();
  if (!src_k_pool || !src_v_pool || !dst_k_pool || !dst_v_pool || !pairs)
    return fail(PKV_EINVAL, "paged_kv_swap_blocks: NULL pointer");
  if (!pkv::aligned16(src_k_pool) || !pkv::aligned16(src_v_pool) || !pkv::aligned16(dst_k_pool) ||
      !pkv::aligned16(dst_v_pool))
    return fail(PKV_EINVAL, "paged_kv_swap_blocks: pools must be 16-byte aligned");
  const int64_t block_bytes = (int64_t)n_kv_heads * block_size * head_dim * es;
  if (block_bytes % 16) return fail(PKV_EINVAL, "paged_kv_swap_blocks: block not a multiple of 16 B");
  const void* v[5] = {src_k_pool, src_v_pool, dst_k_pool, dst_v_pool, pairs};
  for (auto& p : v) {
    p = pkv::device_view(p);
    if (!p) return fail(PKV_EINVAL, "paged_kv_swap_blocks: pools and pairs must be device or pinned host memory");
  }
  hipLaunchKernelGGL(pkv::swap_blocks_kernel, dim3((unsigned)n_pairs, 2), dim3(256), 0, (hipStream_t)stream,
                     (const unsigned char*)v[0], (const unsigned char*)v[1], (unsigned char*)const_cast<void*>(v[2]),
                     (unsigned char*)const_cast<void*>(v[3]), (const int32_t*)v[4], src_num_blocks, dst_num_blocks,
                     block_bytes);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("paged_kv_swap_blocks: ") + hipGetErrorString(e));
  return ok();
}
