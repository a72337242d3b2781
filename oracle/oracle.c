/*
 * fp64 CPU oracle for the paged KV-cache attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no source with the HIP path.
 *
 * What it computes, and where the pages define it:
 *
 *  - orc_attention: dense causal softmax attention in fp64 over logically
 *    contiguous K/V.  "Life of a prompt" (zamalbabar.com), sections "The
 *    detour, what really happens inside one forward pass" and "The decode
 *    stage, and how to spot the waste": scores are the query times K
 *    transposed, softmaxed, then multiplied by V; a decode step needs only the
 *    newest query against the full K and V after the new key and value are
 *    appended.  The causal rule (a token sees itself and earlier tokens only)
 *    follows from autoregressive generation ("How AI actually answers you",
 *    supraj.dev).  Scale 1/sqrt(d) and the contiguous grouping of query heads
 *    onto shared KV heads (grouped-query attention, "How big is the KV cache?"
 *    in the vLLM Serving deep dive) are readings the pages leave open.
 *
 *  - orc_gather / orc_slot: the block-table indirection of "PagedAttention in
 *    depth", Diagram-in-words (vLLM Serving deep dive, fahimfaisal.info):
 *    logical token t of a sequence lives in physical block table[t / bs] at
 *    offset t % bs.  The in-block byte layout is this project's own (the pages
 *    give none); it is restated here from its definition, see k_index/v_index.
 *
 *  - orc_scatter: the append of new keys/values into their cache slots
 *    ("Life of a prompt", "Back to the queue, and into vLLM proper": each new
 *    key and value vector goes into the next free slot of the sequence's
 *    blocks).  A byte copy; slot -1 means "no slot" and is skipped.
 *
 *  - orc_copy_blocks: copy-on-write copies a whole block ("Sharing and
 *    copy-on-write", vLLM Serving deep dive).
 *
 *  - orc_swap_blocks: swapping parks a preempted sequence's blocks in a pool
 *    of pinned host memory and restores them later ("The scheduler: waiting,
 *    running, swapped", vLLM Serving deep dive; the CPU blocks of "Back to
 *    the queue, and into vLLM proper", Life of a prompt): whole blocks are
 *    copied from one pool pair to another.
 *
 *  - e4m3_value / orc_quantize_e4m3: the 8-bit KV cache.  The pages say the
 *    cache may be kept in FP8 (one byte per element: the KV-size formula of
 *    "The hands-on guide to LLM Inference with vLLM"; "Quantization" in the
 *    vLLM Serving deep dive; "Trick 6, Quantization" in "How AI actually
 *    answers you") but fix neither the 8-bit format nor a scale rule.  The
 *    readings taken here: the OCP E4M3 format (bias 7, no infinities, largest
 *    finite 448), one fp32 scale per pool, stored code = the E4M3 value
 *    nearest to x * (1/scale) (both in fp32; ties to the even code; finite
 *    magnitudes beyond 448 and infinities saturate to 448), read back as
 *    value(code) * scale.
 *
 * Pool layout (per layer, elements of `esize` bytes, x = 16 / esize):
 *   K element (blk, head g, token t, dim j) at index
 *       ((((blk * H + g) * (d / x) + j / x) * bs + t) * x + j % x)
 *   V element (blk, g, t, j) at index
 *       (((blk * H + g) * d + j) * bs + t)
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_F16 = 1, ORC_BF16 = 2, ORC_FP8_E4M3 = 3 };

static int esize_of(int dtype) {
  switch (dtype) {
    case ORC_F32: return 4;
    case ORC_F16: return 2;
    case ORC_BF16: return 2;
    case ORC_FP8_E4M3: return 1;
    default: return 0;
  }
}

/* IEEE binary16 -> double, from the format's definition. */
static double f16_value(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = ldexp((double)m, -24); /* subnormal: m * 2^-14 * 2^-10 */
  } else if (e == 31) {
    v = m ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

/* bfloat16 -> double: the upper 16 bits of an IEEE binary32. */
static double bf16_value(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* OCP E4M3 -> double, from the format's definition: 1 sign bit, 4 exponent
 * bits (bias 7), 3 mantissa bits.  Exponent 0 holds the subnormals
 * m/8 * 2^-6; exponent 15 with mantissa 7 is NaN; there are no infinities. */
static double e4m3_value(uint8_t b) {
  int sign = (b >> 7) & 1;
  int e = (b >> 3) & 0xf;
  int m = b & 0x7;
  double v;
  if (e == 15 && m == 7) {
    v = NAN;
  } else if (e == 0) {
    v = ldexp((double)m, -9); /* m/8 * 2^-6 */
  } else {
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  }
  return sign ? -v : v;
}

static double f32_value(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

static double elem_value(int dtype, const unsigned char* base, int64_t idx) {
  if (dtype == ORC_F32) {
    uint32_t u;
    memcpy(&u, base + idx * 4, 4);
    return f32_value(u);
  }
  if (dtype == ORC_FP8_E4M3) return e4m3_value(base[idx]);
  uint16_t h;
  memcpy(&h, base + idx * 2, 2);
  return dtype == ORC_F16 ? f16_value(h) : bf16_value(h);
}

/* The E4M3 code nearest to y: the finite codes are searched one by one (ties
 * go to the even code, i.e. the even mantissa); magnitudes of 448 and beyond,
 * infinities included, give 448; NaN gives the NaN code 0x7f; the sign bit is
 * y's, so values that round to zero keep their sign. */
static uint8_t e4m3_nearest(float y) {
  const uint8_t sign = signbit(y) ? 0x80 : 0;
  if (isnan(y)) return sign | 0x7f;
  const double a = fabs((double)y);
  if (a >= 448.0) return sign | 0x7e;
  int best = 0;
  double best_d = a; /* distance to +0 */
  for (int c = 1; c <= 0x7e; ++c) {
    const double d = fabs(e4m3_value((uint8_t)c) - a);
    if (d < best_d || (d == best_d && (c & 1) == 0)) {
      best = c;
      best_d = d;
    }
  }
  return (uint8_t)(sign | best);
}

/* Quantise n fp32 values for the 8-bit cache: code = nearest E4M3 value of
 * the fp32 product x * inv_scale, where inv_scale is the fp32 reciprocal of
 * the pool's scale. */
int orc_quantize_e4m3(const float* x, int64_t n, float inv_scale, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    const float y = x[i] * inv_scale; /* one fp32 product, rounded to nearest even */
    out[i] = e4m3_nearest(y);
  }
  return 0;
}

int orc_decode(int dtype, const void* src, int64_t n, double* dst) {
  if (!esize_of(dtype)) return -1;
  for (int64_t i = 0; i < n; ++i) dst[i] = elem_value(dtype, (const unsigned char*)src, i);
  return 0;
}

static int64_t k_index(int64_t blk, int64_t g, int64_t t, int64_t j, int64_t H, int64_t d,
                       int64_t bs, int64_t x) {
  return (((blk * H + g) * (d / x) + j / x) * bs + t) * x + j % x;
}

static int64_t v_index(int64_t blk, int64_t g, int64_t t, int64_t j, int64_t H, int64_t d,
                       int64_t bs) {
  return ((blk * H + g) * d + j) * bs + t;
}

/* Physical slot of logical token t: block table[t / bs], offset t % bs. */
int64_t orc_slot(const int32_t* table, int64_t t, int32_t bs) {
  return (int64_t)table[t / bs] * bs + t % bs;
}

/*
 * Gather the first n_tokens logical tokens of one sequence from the pools into
 * contiguous fp64 arrays k_out/v_out of shape [n_tokens][H][d].
 * Returns -1 on a bad dtype or shape, -2 on a block id outside the pool.
 */
int orc_gather(int dtype, const void* k_pool, const void* v_pool, int64_t num_blocks, int32_t bs,
               int32_t H, int32_t d, const int32_t* table, int64_t n_table, int64_t n_tokens,
               double* k_out, double* v_out) {
  int es = esize_of(dtype);
  if (!es || bs <= 0 || H <= 0 || d <= 0 || (d * es) % 16) return -1;
  if (n_tokens > n_table * bs) return -1;
  int64_t x = 16 / es;
  for (int64_t t = 0; t < n_tokens; ++t) {
    int64_t blk = table[t / bs];
    int64_t off = t % bs;
    if (blk < 0 || blk >= num_blocks) return -2;
    for (int64_t g = 0; g < H; ++g)
      for (int64_t j = 0; j < d; ++j) {
        k_out[(t * H + g) * d + j] =
            elem_value(dtype, (const unsigned char*)k_pool, k_index(blk, g, off, j, H, d, bs, x));
        v_out[(t * H + g) * d + j] =
            elem_value(dtype, (const unsigned char*)v_pool, v_index(blk, g, off, j, H, d, bs));
      }
  }
  return 0;
}

/*
 * Write token i's key/value rows (key + i*key_stride elements, heads then dims)
 * into physical slot slots[i] of the pools, byte for byte.  slots[i] < 0 is
 * skipped.  Returns -2 when a slot lies outside the pool.
 */
int orc_scatter(int dtype, const void* key, const void* value, int64_t n_tokens,
                int64_t key_stride, int64_t value_stride, void* k_pool, void* v_pool,
                const int64_t* slots, int64_t num_blocks, int32_t bs, int32_t H, int32_t d) {
  int es = esize_of(dtype);
  if (!es || bs <= 0 || H <= 0 || d <= 0 || (d * es) % 16) return -1;
  int64_t x = 16 / es;
  for (int64_t i = 0; i < n_tokens; ++i) {
    int64_t s = slots[i];
    if (s < 0) continue;
    int64_t blk = s / bs, off = s % bs;
    if (blk >= num_blocks) return -2;
    for (int64_t g = 0; g < H; ++g)
      for (int64_t j = 0; j < d; ++j) {
        const unsigned char* ks = (const unsigned char*)key + (i * key_stride + g * d + j) * es;
        const unsigned char* vs = (const unsigned char*)value + (i * value_stride + g * d + j) * es;
        memcpy((unsigned char*)k_pool + k_index(blk, g, off, j, H, d, bs, x) * es, ks, es);
        memcpy((unsigned char*)v_pool + v_index(blk, g, off, j, H, d, bs) * es, vs, es);
      }
  }
  return 0;
}

/* Copy whole blocks src -> dst (pairs[2*i], pairs[2*i+1]) in both pools. */
int orc_copy_blocks(int dtype, void* k_pool, void* v_pool, const int32_t* pairs, int64_t n,
                    int64_t num_blocks, int32_t bs, int32_t H, int32_t d) {
  int es = esize_of(dtype);
  if (!es) return -1;
  int64_t block_bytes = (int64_t)H * bs * d * es;
  for (int64_t i = 0; i < n; ++i) {
    int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || dst < 0 || src >= num_blocks || dst >= num_blocks) return -2;
    memmove((unsigned char*)k_pool + dst * block_bytes, (unsigned char*)k_pool + src * block_bytes,
            block_bytes);
    memmove((unsigned char*)v_pool + dst * block_bytes, (unsigned char*)v_pool + src * block_bytes,
            block_bytes);
  }
  return 0;
}

/* Copy whole blocks from one pool pair to another: block pairs[2*i] of
 * (src_k, src_v) to block pairs[2*i+1] of (dst_k, dst_v).  Returns -2 when a
 * block lies outside its pool. */
int orc_swap_blocks(int dtype, const void* src_k, const void* src_v, int64_t src_num_blocks, void* dst_k,
                    void* dst_v, int64_t dst_num_blocks, const int32_t* pairs, int64_t n, int32_t bs, int32_t H,
                    int32_t d) {
  int es = esize_of(dtype);
  if (!es) return -1;
  int64_t block_bytes = (int64_t)H * bs * d * es;
  for (int64_t i = 0; i < n; ++i) {
    int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || dst < 0 || src >= src_num_blocks || dst >= dst_num_blocks) return -2;
    memcpy((unsigned char*)dst_k + dst * block_bytes, (const unsigned char*)src_k + src * block_bytes, block_bytes);
    memcpy((unsigned char*)dst_v + dst * block_bytes, (const unsigned char*)src_v + src * block_bytes, block_bytes);
  }
  return 0;
}

/*
 * Causal softmax attention, fp64.
 *   q     [n_rows][Hq][d]      query rows; row r sits at absolute position q_pos[r]
 *   k, v  [n_keys][Hkv][d]     logically contiguous keys / values
 *   out   [n_rows][Hq][d]
 *   wsum  [n_rows][Hq]         optional: sum of the softmax weights of each row
 * Row r, head h attends keys 0..q_pos[r] of KV head h / (Hq / Hkv):
 *   s_j = scale * sum_k q[h][k] * K_j[k]
 *   w_j = exp(s_j - max_i s_i) / sum_i exp(s_i - max_i s_i)
 *   out = sum_j w_j * V_j
 * Returns -1 on a bad shape or a position outside [0, n_keys).
 */
int orc_attention(int64_t n_rows, const double* q, const int64_t* q_pos, int64_t n_keys,
                  const double* k, const double* v, int32_t Hq, int32_t Hkv, int32_t d,
                  double scale, double* out, double* wsum, double* scratch /* [n_keys] per thread */,
                  int32_t n_threads) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0) return -1;
  for (int64_t r = 0; r < n_rows; ++r)
    if (q_pos[r] < 0 || q_pos[r] >= n_keys) return -1;
  const int32_t G = Hq / Hkv;
  const int64_t items = n_rows * Hq;
  if (n_threads < 1) n_threads = 1;
#pragma omp parallel for num_threads(n_threads) schedule(dynamic, 1)
  for (int64_t it = 0; it < items; ++it) {
    int tid = 0;
#ifdef _OPENMP
    tid = omp_get_thread_num();
#endif
    double* w = scratch + (int64_t)tid * n_keys;
    const int64_t r = it / Hq;
    const int32_t h = (int32_t)(it % Hq);
    const int32_t g = h / G;
    const int64_t p = q_pos[r];
    const double* qv = q + (r * Hq + h) * d;
    double m = -INFINITY;
    for (int64_t j = 0; j <= p; ++j) {
      const double* kj = k + (j * Hkv + g) * d;
      double s = 0.0;
      for (int32_t c = 0; c < d; ++c) s += qv[c] * kj[c];
      s *= scale;
      w[j] = s;
      if (s > m) m = s;
    }
    double z = 0.0;
    for (int64_t j = 0; j <= p; ++j) {
      w[j] = exp(w[j] - m);
      z += w[j];
    }
    double ws = 0.0;
    for (int64_t j = 0; j <= p; ++j) {
      w[j] /= z;
      ws += w[j];
    }
    double* o = out + (r * Hq + h) * d;
    for (int32_t c = 0; c < d; ++c) o[c] = 0.0;
    for (int64_t j = 0; j <= p; ++j) {
      const double* vj = v + (j * Hkv + g) * d;
      for (int32_t c = 0; c < d; ++c) o[c] += w[j] * vj[c];
    }
    if (wsum) wsum[r * Hq + h] = ws;
  }
  return 0;
}
