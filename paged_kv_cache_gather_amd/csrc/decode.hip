// Decode attention over the paged KV cache (one query token per sequence).
//
// What is computed: for each sequence s and query head h (KV head
// g = h / G, G = n_q_heads / n_kv_heads), the softmax-weighted sum of the V
// rows of the sequence's L cached tokens, with weights softmax(scale*q.K).
// The kernel walks the block table block by block, reading K and V from the
// physical blocks it names ("How the attention kernel actually reads paged
// blocks", vLLM Serving deep dive; the decode shopping list of one query
// against the full K and V is in "The decode stage, and how to spot the
// waste", Life of a prompt).
//
// How (gfx950):
//  * Work unit = (partition p of 512 context tokens, KV head g, sequence s),
//    one 256-thread workgroup (4 wave64s).  All G query heads that share the
//    KV head are handled together, so every K/V byte is read once per step.
//  * Phase 1, scores: each thread takes one token, reads its whole K row
//    (16-byte chunks; the K layout keeps 8 dims of one token together) and
//    forms G dot products with packed dot2 instructions (fp32 accumulate).
//    The query is uniform across the workgroup and is read through the
//    scalar unit.  Scores, pre-multiplied by scale*log2(e), go to LDS.
//  * Phase 2, softmax: workgroup max per head, then p = 2^(s - max) in LDS and
//    the per-head sum.
//  * Phase 3, values: wave w takes blocks w, w+4, ...; lane l owns D/64
//    consecutive dims and reads their dim-major V rows (16 tokens each,
//    contiguous), accumulating p * v in fp32 with p broadcast from LDS.
//    The four waves' partial sums are added through LDS.
//  * A sequence that fits in one partition writes its normalised output
//    directly; otherwise each partition writes (max, sum, unnormalised o) to
//    the workspace and decode_reduce_kernel merges them:
//      M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
#include <math.h>

#include <cmath>
#include <string>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

constexpr int kPart = 512;        // context tokens per partition
constexpr int kThreads = 256;     // threads per workgroup
constexpr int kWaves = kThreads / 64;
constexpr int kTokPerThread = kPart / kThreads;

template <typename T, int D, int G, int OutCode>
__global__ void __launch_bounds__(kThreads, 2)
decode_partition_kernel(void* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
                        const typename T::bits* __restrict__ q, const unsigned char* __restrict__ kpool,
                        const unsigned char* __restrict__ vpool, const int32_t* __restrict__ tables,
                        int max_blocks, const int32_t* __restrict__ lens, int Hkv, int64_t num_blocks,
                        int max_context_len, float scale_log2, int max_parts) {
  constexpr int ES = T::kBytes;
  constexpr int X = 16 / ES;    // elements per 16-byte chunk
  constexpr int C = D / X;      // chunks per K row
  constexpr int DPL = D / 64;   // dims per lane in the V pass
  constexpr int VCH = DPL * kBlockSize * ES / 16;  // 16-byte V chunks per lane per block

  // Scores/probabilities [G][kPart]; after the V pass the same memory holds
  // the waves' partial outputs [kWaves][G][D] (kWaves * D <= kPart).
  static_assert(kWaves * D <= kPart, "partial outputs must fit in the score buffer");
  __shared__ float smem[G * kPart];
  __shared__ float wred[kWaves][G];
  float(*sc)[kPart] = reinterpret_cast<float(*)[kPart]>(smem);
  float(*red)[G][D] = reinterpret_cast<float(*)[G][D]>(smem);

  const int p = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int Hq = Hkv * G;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  int L = lens[s];
  L = L < 0 ? 0 : (L > max_context_len ? max_context_len : L);
  const int nparts = (L + kPart - 1) / kPart;
  if (p >= (nparts > 0 ? nparts : 1)) return;
  if (L == 0) {  // defined result for an empty context: zeros
    for (int i = tid; i < G * D; i += kThreads)
      store_out<OutCode>(out, ((int64_t)s * Hq + g * G) * D + i, 0.f);
    return;
  }
  const int t0 = p * kPart;
  const int n = (L - t0) < kPart ? (L - t0) : kPart;
  const int32_t* tab = tables + (int64_t)s * max_blocks;

  // ---- phase 1: scores ---------------------------------------------------
  float mx[G];
#pragma unroll
  for (int h = 0; h < G; ++h) mx[h] = -INFINITY;
  const typename T::bits* qg = q + ((int64_t)s * Hq + g * G) * D;

#pragma unroll 1
  for (int k = 0; k < kTokPerThread; ++k) {
    const int tl = tid + k * kThreads;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.f;
    if (tl < n) {
      const int t = t0 + tl;
      const int64_t blk = clamp_block(tab[t >> 4], num_blocks);
      const unsigned char* kp = kpool + (((blk * Hkv + g) * C) * kBlockSize + (t & 15)) * 16;
      u32x4 kc[C];
#pragma unroll
      for (int c = 0; c < C; ++c) kc[c] = ld16(kp + c * (kBlockSize * 16));
      if constexpr (ES == 2) {
        const uint32_t* qw = reinterpret_cast<const uint32_t*>(qg);
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[h] = dot2<T>(qw[h * (D / 2) + c * 4 + e], kc[c][e], acc[h]);
      } else {
        const float* qf = reinterpret_cast<const float*>(qg);
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              acc[h] = fmaf(qf[h * D + c * 4 + e], __uint_as_float(kc[c][e]), acc[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float sv = tl < n ? acc[h] * scale_log2 : -INFINITY;
      sc[h][tl] = sv;
      mx[h] = fmaxf(mx[h], sv);
    }
  }

  // ---- phase 2: softmax over the partition --------------------------------
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float m = wave_max(mx[h]);
    if (lane == 0) wred[w][h] = m;
  }
  __syncthreads();
  float M[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = wred[0][h];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) m = fmaxf(m, wred[i][h]);
    M[h] = m;
  }
  __syncthreads();
  float ls[G];
#pragma unroll
  for (int h = 0; h < G; ++h) ls[h] = 0.f;
#pragma unroll
  for (int k = 0; k < kTokPerThread; ++k) {
    const int tl = tid + k * kThreads;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float e = tl < n ? __builtin_amdgcn_exp2f(sc[h][tl] - M[h]) : 0.f;
      sc[h][tl] = e;
      ls[h] += e;
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float l = wave_sum(ls[h]);
    if (lane == 0) wred[w][h] = l;
  }
  __syncthreads();

  // ---- phase 3: values ---------------------------------------------------
  float o[G][DPL];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) o[h][dd] = 0.f;
  const int nblk = (n + kBlockSize - 1) / kBlockSize;
  const int b0 = t0 / kBlockSize;
#pragma unroll 1
  for (int b = w; b < nblk; b += kWaves) {
    const int64_t blk = clamp_block(tab[b0 + b], num_blocks);
    const unsigned char* vp =
        vpool + ((blk * Hkv + g) * D + (int64_t)lane * DPL) * kBlockSize * ES;
    u32x4 vv[VCH];
#pragma unroll
    for (int i = 0; i < VCH; ++i) vv[i] = ld16(vp + i * 16);
    const int ntok = (n - b * kBlockSize) < kBlockSize ? (n - b * kBlockSize) : kBlockSize;
    const float* pb = &sc[0][b * kBlockSize];
    auto vel = [&](int dd, int t) -> float {
      if constexpr (ES == 2) {
        const int wd = (dd * kBlockSize + t) >> 1;
        const uint32_t word = vv[wd >> 2][wd & 3];
        float lo, hi;
        unpack2<T>(word, lo, hi);
        return (t & 1) ? hi : lo;
      } else {
        const int wd = dd * kBlockSize + t;
        return __uint_as_float(vv[wd >> 2][wd & 3]);
      }
    };
    if (ntok == kBlockSize) {
#pragma unroll
      for (int t = 0; t < kBlockSize; ++t) {
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) {
          const float x = vel(dd, t);
#pragma unroll
          for (int h = 0; h < G; ++h) o[h][dd] = fmaf(pb[h * kPart + t], x, o[h][dd]);
        }
      }
    } else {
#pragma unroll
      for (int t = 0; t < kBlockSize; ++t) {
        if (t < ntok) {
#pragma unroll
          for (int dd = 0; dd < DPL; ++dd) {
            const float x = vel(dd, t);
#pragma unroll
            for (int h = 0; h < G; ++h) o[h][dd] = fmaf(pb[h * kPart + t], x, o[h][dd]);
          }
        }
      }
    }
  }
  __syncthreads();  // every wave is done reading sc
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) red[w][h][lane * DPL + dd] = o[h][dd];
  __syncthreads();

  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, j = i % D;
    float acc = red[0][h][j];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) acc += red[k][h][j];
    float l = wred[0][h];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) l += wred[k][h];
    const int64_t row = (int64_t)s * Hq + g * G + h;
    if (nparts == 1) {
      store_out<OutCode>(out, row * D + j, acc / l);
    } else {
      ws_o[(row * max_parts + p) * D + j] = acc;
      if (j == 0) {
        ws_ml[(row * max_parts + p) * 2 + 0] = M[h];
        ws_ml[(row * max_parts + p) * 2 + 1] = l;
      }
    }
  }
}

template <int D, int OutCode>
__global__ void __launch_bounds__(64)
decode_reduce_kernel(void* __restrict__ out, const float* __restrict__ ws_o,
                     const float* __restrict__ ws_ml, const int32_t* __restrict__ lens, int Hq, int G,
                     int max_context_len, int max_parts) {
  constexpr int DPL = D / 64;
  const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  int L = lens[s];
  L = L < 0 ? 0 : (L > max_context_len ? max_context_len : L);
  const int nparts = (L + kPart - 1) / kPart;
  if (nparts <= 1) return;
  const int64_t row = (int64_t)s * Hq + h;
  const float* ml = ws_ml + row * max_parts * 2;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  float den = 0.f, acc[DPL];
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) acc[dd] = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float wgt = __builtin_amdgcn_exp2f(ml[2 * p] - M);
    den = fmaf(wgt, ml[2 * p + 1], den);
    const float* op = ws_o + (row * max_parts + p) * D + lane * DPL;
#pragma unroll
    for (int dd = 0; dd < DPL; ++dd) acc[dd] = fmaf(wgt, op[dd], acc[dd]);
  }
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) store_out<OutCode>(out, row * D + lane * DPL + dd, acc[dd] / den);
  (void)G;
}

struct DecodeArgs {
  void* out;
  float* ws_o;
  float* ws_ml;
  const void* q;
  const unsigned char* kpool;
  const unsigned char* vpool;
  const int32_t* tables;
  int max_blocks;
  const int32_t* lens;
  int B, Hq, Hkv;
  int64_t num_blocks;
  int max_context_len;
  float scale_log2;
  int max_parts;
  hipStream_t stream;
};

template <typename T, int D, int G, int OutCode>
void launch_decode(const DecodeArgs& a) {
  hipLaunchKernelGGL((decode_partition_kernel<T, D, G, OutCode>),
                     dim3((unsigned)a.max_parts, (unsigned)a.Hkv, (unsigned)a.B), dim3(kThreads), 0,
                     a.stream, a.out, a.ws_o, a.ws_ml, (const typename T::bits*)a.q, a.kpool, a.vpool,
                     a.tables, a.max_blocks, a.lens, a.Hkv, a.num_blocks, a.max_context_len,
                     a.scale_log2, a.max_parts);
  if (a.max_parts > 1) {
    hipLaunchKernelGGL((decode_reduce_kernel<D, OutCode>), dim3((unsigned)a.Hq, (unsigned)a.B),
                       dim3(64), 0, a.stream, a.out, a.ws_o, a.ws_ml, a.lens, a.Hq, G,
                       a.max_context_len, a.max_parts);
  }
}

template <typename T, int D, int OutCode>
int dispatch_g(const DecodeArgs& a, int G) {
  switch (G) {
    case 1: launch_decode<T, D, 1, OutCode>(a); return 0;
    case 2: launch_decode<T, D, 2, OutCode>(a); return 0;
    case 4: launch_decode<T, D, 4, OutCode>(a); return 0;
    case 8: launch_decode<T, D, 8, OutCode>(a); return 0;
    case 16: launch_decode<T, D, 16, OutCode>(a); return 0;
    default: return -1;
  }
}

template <typename T, int OutCode>
int dispatch_d(const DecodeArgs& a, int D, int G) {
  if (D == 64) return dispatch_g<T, 64, OutCode>(a, G);
  if (D == 128) return dispatch_g<T, 128, OutCode>(a, G);
  return -1;
}

}  // namespace
}  // namespace pkv

using pkv::fail;
using pkv::ok;

extern "C" int32_t paged_attention_decode_partition_size(void) { return pkv::kPart; }

extern "C" int64_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t n_q_heads,
                                                          int32_t head_dim, int32_t max_context_len) {
  if (num_seqs <= 0 || n_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const int64_t parts = (max_context_len + pkv::kPart - 1) / pkv::kPart;
  if (parts <= 1) return 0;
  return (int64_t)num_seqs * n_q_heads * parts * (head_dim + 2) * (int64_t)sizeof(float);
}

extern "C" int paged_attention_decode(void* out, int32_t out_dtype, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                      int32_t max_context_len, float scale, int32_t kv_dtype,
                                      void* workspace, int64_t workspace_bytes, void* stream) {
  if (!pkv::esize_of(kv_dtype)) return fail(PKV_EINVAL, "paged_attention_decode: unknown kv dtype");
  if (out_dtype != PKV_F32 && out_dtype != kv_dtype)
    return fail(PKV_EINVAL, "paged_attention_decode: out dtype must be f32 or the kv dtype");
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size must be 16");
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (num_seqs < 0 || num_seqs > 65535 || n_kv_heads < 1 || n_q_heads < 1 || n_kv_heads > 65535)
    return fail(PKV_EINVAL, "paged_attention_decode: bad num_seqs or head counts");
  if (n_q_heads % n_kv_heads) return fail(PKV_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
  const int G = n_q_heads / n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PKV_EUNSUPPORTED, "n_q_heads / n_kv_heads must be 1, 2, 4, 8 or 16");
  if (num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_EINVAL, "paged_attention_decode: max_context_len exceeds the table width");
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "paged_attention_decode: NULL pointer");
  if (!pkv::aligned16(q) || !pkv::aligned16(k_pool) || !pkv::aligned16(v_pool) || !pkv::aligned16(out))
    return fail(PKV_EINVAL, "paged_attention_decode: q, out and pools must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "paged_attention_decode: scale not finite");
  const int max_parts = max_context_len > 0 ? (max_context_len + pkv::kPart - 1) / pkv::kPart : 1;
  const int64_t need = paged_attention_decode_workspace_bytes(num_seqs, n_q_heads, head_dim, max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need || !pkv::aligned16(workspace)))
    return fail(PKV_EINVAL, "paged_attention_decode: workspace missing or too small (need " +
                                std::to_string(need) + " bytes)");
  pkv::DecodeArgs a;
  a.out = out;
  a.ws_o = (float*)workspace;
  a.ws_ml = need > 0 ? (float*)workspace + (int64_t)num_seqs * n_q_heads * max_parts * head_dim : nullptr;
  a.q = q;
  a.kpool = (const unsigned char*)k_pool;
  a.vpool = (const unsigned char*)v_pool;
  a.tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.lens = context_lens;
  a.B = num_seqs;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.max_parts = max_parts;
  a.stream = (hipStream_t)stream;
  int rc = -1;
  switch (kv_dtype) {
    case PKV_F32: rc = pkv::dispatch_d<pkv::F32, PKV_F32>(a, head_dim, G); break;
    case PKV_F16:
      rc = out_dtype == PKV_F32 ? pkv::dispatch_d<pkv::F16, PKV_F32>(a, head_dim, G)
                                : pkv::dispatch_d<pkv::F16, PKV_F16>(a, head_dim, G);
      break;
    case PKV_BF16:
      rc = out_dtype == PKV_F32 ? pkv::dispatch_d<pkv::BF16, PKV_F32>(a, head_dim, G)
                                : pkv::dispatch_d<pkv::BF16, PKV_BF16>(a, head_dim, G);
      break;
  }
  if (rc) return fail(PKV_EUNSUPPORTED, "paged_attention_decode: configuration not built");
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, std::string("paged_attention_decode: ") + hipGetErrorString(e));
  return ok();
}
