// Device-side helpers for the gfx950 kernels: element types, 16-byte vector
// accesses, conversions, wave64 reductions, and the per-item bodies of the
// cache writes (plain and quantising), shared by the cache-write kernels and
// the decode launch that writes a step's new rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv.h"

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Storage types: raw bits, so the cache ops copy without conversion.
struct F32 {
  using bits = uint32_t;
  static constexpr int kCode = PKV_F32;
  static constexpr int kBytes = 4;
};
struct F16 {
  using bits = uint16_t;
  static constexpr int kCode = PKV_F16;
  static constexpr int kBytes = 2;
};
struct BF16 {
  using bits = uint16_t;
  static constexpr int kCode = PKV_BF16;
  static constexpr int kBytes = 2;
};
// OCP E4M3 codes of the 8-bit cache (values are code * the pool's scale).
struct FP8 {
  using bits = uint8_t;
  static constexpr int kCode = PKV_FP8_E4M3;
  static constexpr int kBytes = 1;
};

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float f16lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Two packed elements of a 32-bit word -> fp32.
template <typename T>
__device__ __forceinline__ void unpack2(uint32_t w, float& lo, float& hi) {
  if constexpr (T::kCode == PKV_BF16) {
    lo = bf16lo(w);
    hi = bf16hi(w);
  } else {
    lo = f16lo(w);
    hi = f16hi(w);
  }
}

// acc + a.lo*b.lo + a.hi*b.hi for two packed 16-bit elements, fp32 accumulate.
template <typename T>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  if constexpr (T::kCode == PKV_BF16) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
  } else {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  acc, false);
  }
}

// fp32 -> storage bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int OutCode>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v) {
  if constexpr (OutCode == PKV_F32) {
    reinterpret_cast<float*>(out)[idx] = v;
  } else if constexpr (OutCode == PKV_BF16) {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_bits(v);
  } else {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_f16_bits(v);
  }
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming (nontemporal) loads, for cache bytes a step reads once.  Used
// where one wave instruction takes whole 128-byte lines (a K row chunk of 16
// tokens, a 1 KiB K or V run, all four 8-byte pieces of a 16-bit V row,
// both halves of an 8-bit V row): the hint lets the caches drop the lines
// first.  Measured on scattered 4 KiB tiles it lifts what a read-only pass
// gets from ~6.1 to ~6.7 TB/s; on loads that take half a line per
// instruction (the other half in the next) it costs instead.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ uint64_t ld8_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Wave64 butterfly reductions (every lane receives the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int64_t clamp_block(int64_t b, int64_t num_blocks) {
  return b < 0 ? 0 : (b >= num_blocks ? num_blocks - 1 : b);
}

// One item of a cache write (a bit copy): the 16-byte chunk c of new token
// i's row for KV head g goes to its slot in the pool layout.  The K chunk
// stays one 16-byte unit (x = 16 / ES consecutive dims of one token); the V
// chunk is spread over its x dim-rows, one element each (V tiles are
// dim-major).  A slot outside [0, num_slots) is skipped (padding).
template <int ES>
__device__ __forceinline__ void cache_write_chunk(const unsigned char* __restrict__ key,
                                                  const unsigned char* __restrict__ value, int64_t kstride_b,
                                                  int64_t vstride_b, unsigned char* __restrict__ kpool,
                                                  unsigned char* __restrict__ vpool, int64_t slot, int64_t num_slots,
                                                  int64_t i, int g, int c, int H, int D) {
  constexpr int X = 16 / ES;  // elements per 16-byte chunk
  constexpr int BS = 16;      // tokens per block
  const int C = D / X;        // chunks per head row
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / BS;
  const int off = (int)(slot % BS);
  const int64_t tile = blk * H + g;
  const u32x4 kv = ld16(key + i * kstride_b + ((int64_t)g * D + c * X) * ES);
  const u32x4 vv = ld16(value + i * vstride_b + ((int64_t)g * D + c * X) * ES);
  st16(kpool + (((tile * C + c) * BS + off) * 16), kv);
  unsigned char* vrow = vpool + ((tile * D + (int64_t)c * X) * BS + off) * ES;
  if constexpr (ES == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) *reinterpret_cast<uint32_t*>(vrow + (int64_t)e * BS * ES) = vv[e];
  } else if constexpr (ES == 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) vrow[(int64_t)e * BS] = (unsigned char)(vv[e >> 2] >> (8 * (e & 3)));
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t h = (uint16_t)((e & 1) ? (vv[e >> 1] >> 16) : (vv[e >> 1] & 0xffffu));
      *reinterpret_cast<uint16_t*>(vrow + (int64_t)e * BS * ES) = h;
    }
  }
}

// fp32 -> E4M3 code of the nearest value (ties to even): finite magnitudes
// beyond 448 and infinities saturate first, NaN stays NaN.  Four values per
// 32-bit word, the first in the low byte.
__device__ __forceinline__ float e4m3_saturate(float y) {
  return y != y ? y : fminf(fmaxf(y, -448.f), 448.f);
}
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_saturate(a), e4m3_saturate(b), 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_saturate(c), e4m3_saturate(d), w, true);
}

// 16 source elements (one 16-dim chunk of a row) -> 16 codes, x * inv each.
template <typename S>
__device__ __forceinline__ u32x4 quantise16(const unsigned char* src, float inv) {
  float f[16];
  if constexpr (S::kBytes == 4) {
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const u32x4 w = ld16(src + 16 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) f[4 * h + e] = __uint_as_float(w[e]);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4 w = ld16(src + 16 * h);
#pragma unroll
      for (int e = 0; e < 4; ++e) unpack2<S>(w[e], f[8 * h + 2 * e], f[8 * h + 2 * e + 1]);
    }
  }
  u32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    r[e] = e4m3x4(f[4 * e] * inv, f[4 * e + 1] * inv, f[4 * e + 2] * inv, f[4 * e + 3] * inv);
  return r;
}

// One item of a quantising cache write into 8-bit pools: the 16-dim chunk c
// of new token i's row for KV head g (source type S) becomes 16 E4M3 codes
// of x * inv (inv = the host-rounded reciprocal of the pool's scale); the K
// chunk is one 16-byte store, the V chunk 16 one-byte stores (dim-major V).
// A slot outside [0, num_slots) is skipped.
template <typename S>
__device__ __forceinline__ void cache_write_chunk_fp8(const unsigned char* __restrict__ key,
                                                      const unsigned char* __restrict__ value, int64_t kstride_b,
                                                      int64_t vstride_b, unsigned char* __restrict__ kpool,
                                                      unsigned char* __restrict__ vpool, int64_t slot,
                                                      int64_t num_slots, int64_t i, int g, int c, int H, int D,
                                                      float k_inv, float v_inv) {
  constexpr int BS = 16;  // tokens per block
  const int C = D / 16;   // 16-dim chunks per head row
  if (slot < 0 || slot >= num_slots) return;
  const int64_t tile = (slot / BS) * H + g;
  const int off = (int)(slot % BS);
  const int64_t col = ((int64_t)g * D + c * 16) * S::kBytes;
  const u32x4 kq = quantise16<S>(key + i * kstride_b + col, k_inv);
  const u32x4 vq = quantise16<S>(value + i * vstride_b + col, v_inv);
  st16(kpool + ((tile * C + c) * BS + off) * 16, kq);
  unsigned char* vrow = vpool + (tile * D + (int64_t)c * 16) * BS + off;
#pragma unroll
  for (int e = 0; e < 16; ++e) vrow[(int64_t)e * BS] = (unsigned char)(vq[e >> 2] >> (8 * (e & 3)));
}

}  // namespace pkv
