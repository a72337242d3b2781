// Decode attention over the paged KV cache (one query token per sequence),
// and verify attention (a few new query tokens per sequence) on the same
// split-context machinery.
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
// How (gfx950): three kernels per step on one stream.  decode_shared_kernel
// first serves the partitions that sequences of one run window share (see
// the section on shared partitions below) — and, when the step is one
// paged_attention_decode_append call, writes the new tokens' K/V rows with
// extra workgroups; decode_partition_kernel serves the rest;
// decode_reduce_kernel merges split-context partials.  Over an 8-bit
// (E4M3) cache the rest is served by decode_fp8_partition_kernel instead, on
// MFMA like the shared kernel: the codes are widened in registers, exactly,
// and the pools' scales fold into the softmax scale (keys) and the written
// partials (values).  Verify attention (verify_partition_kernel, further
// below) serves a sequence's new tokens with the same MFMA routine as the
// shared kernel (mfma_partition) and a causal limit per row.  Short contexts
// in a small batch skip all of that: decode_whole_kernel (further below)
// runs the per-sequence routine over a whole context of up to 2048 tokens
// on a 16-wave workgroup per (sequence, KV head), in one launch.
// decode_partition_kernel:
//  * Work unit = (KV head g, sequence s, partition p of 512 context tokens),
//    one 256-thread workgroup (4 wave64s).  All G query heads that share the
//    KV head are handled together, so every K/V byte is read once per step.
//    The grid runs KV head fastest: consecutive workgroups go round-robin to
//    the 8 XCDs, so with 8 KV heads every workgroup of one head lands on the
//    same XCD, and sequences that share prefix blocks (adjacent in the batch)
//    hit that XCD's L2.  Partitions run from the last to the first, so the
//    long sequences' extra partitions start early.
//  * The partition's blocks are dealt evenly to the four waves (up to 128
//    consecutive tokens each, so a partly filled last partition keeps every
//    wave busy); each wave takes its tokens end to end:
//    - scores: one token per lane; the lane reads its token's whole K row
//      (16-byte chunks; the K layout keeps x dims of one token together, so
//      each wave instruction reads 4 blocks x 256 contiguous bytes) and forms
//      G dot products with packed dot2 instructions (fp32 accumulate).  The
//      query is uniform across the workgroup and is read by the scalar unit.
//    - wave-local softmax in base 2 (scores pre-scaled by scale*log2 e):
//      max and sum by wave64 butterflies, probabilities to wave-private LDS.
//    - values: each wave instruction reads 1 KiB of a block's dim-major V
//      tile; lane l gets D/64 dims x (16/CPR) tokens and accumulates p*v in
//      fp32 with the probabilities read from LDS; the CPR lanes sharing a
//      dim are added with shuffles.  The next block's loads are issued
//      before this block's products where registers allow.
//  * The four waves' (max, sum, o) states are merged through LDS.  A sequence
//    that fits in one partition writes its normalised output; otherwise each
//    partition writes (max, sum, unnormalised o) to the workspace and
//    decode_reduce_kernel merges them:
//      M = max_p m_p,  out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
#include <math.h>

#include <cmath>
#include <mutex>
#include <string>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

// Tuning knobs (compile-time; the defaults are the measured best on MI355X).
#ifndef PKV_DECODE_PART
#define PKV_DECODE_PART 512
#endif
#ifndef PKV_DECODE_MIN_WAVES
#define PKV_DECODE_MIN_WAVES 2
#endif
// parts a wave's 128 tokens are processed in by the MFMA routine (1 or 2)
#ifndef PKV_SHARED_PARTS
#define PKV_SHARED_PARTS 2
#endif
#ifndef PKV_SHARED_WAVES
#define PKV_SHARED_WAVES 4
#endif
#ifndef PKV_FP8_PARTS
#define PKV_FP8_PARTS 2
#endif
// workgroups that share a run window's runs
#ifndef PKV_RUN_SLOTS
#define PKV_RUN_SLOTS 2
#endif
#ifndef PKV_VERIFY_PARTS
#define PKV_VERIFY_PARTS 2
#endif

constexpr int kPart = PKV_DECODE_PART;  // context tokens per partition
constexpr int kThreads = 256;           // threads per workgroup
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ int clamp_len(int L, int max_context_len) {
  return L < 0 ? 0 : (L > max_context_len ? max_context_len : L);
}

// The partition pass of sequence s, KV head g, partition p (n tokens) of PART
// context tokens, on WAVES waves: the G query heads of the KV head are the
// workgroup's R = G rows.
template <typename T, int D, int G, int OutCode, int PART = kPart, int WAVES = kWaves>
__device__ __forceinline__ void partition_rows(
    float* __restrict__ smem, float (*__restrict__ sml)[2], void* __restrict__ out, float* __restrict__ ws_o,
    float* __restrict__ ws_ml, const typename T::bits* __restrict__ q, const unsigned char* __restrict__ kpool,
    const unsigned char* __restrict__ vpool, const int32_t* __restrict__ tab, const int32_t* __restrict__ lens,
    int s, int g, int p, int n, int Hkv, int64_t num_blocks, int max_context_len, float scale_log2,
    int max_parts) {
  constexpr int R = G;                       // query rows served
  constexpr int ES = T::kBytes;
  constexpr int X = 16 / ES;                 // elements per 16-byte chunk
  constexpr int C = D / X;                   // chunks per K row
  constexpr int TPW = PART / WAVES;          // context tokens per wave
  constexpr int IT = TPW / 64;               // score iterations per wave (one token per lane)
  constexpr int CPR = ES;                    // 16-byte chunks per V dim-row of one block
  constexpr int TPC = kBlockSize / CPR;      // tokens per V chunk
  constexpr int NI = D * ES / 64;            // V chunks per lane per block (= dims per lane)
  constexpr int VTILE = D * kBlockSize * ES; // bytes of one (block, head) V tile

  const int Hq = Hkv * G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform per wave
  // the partition's blocks are dealt evenly to the waves, so a partly filled
  // (last) partition keeps every wave busy; wave w takes blocks [bw0, bw1),
  // at most TPW tokens
  const int nbp = (n + kBlockSize - 1) / kBlockSize;
  const int bw0 = (w * nbp) / WAVES, bw1 = ((w + 1) * nbp) / WAVES;
  const int wt0 = bw0 * kBlockSize;                         // wave's first token (partition-local)
  const int wend = bw1 * kBlockSize < n ? bw1 * kBlockSize : n;
  const int wn = wend - wt0 < 0 ? 0 : wend - wt0;            // its tokens
  float(*sp)[R] = reinterpret_cast<float(*)[R]>(smem) + w * TPW;
  // fp16 V: the probabilities go to LDS as fp16, [R][TPW] per wave, and the
  // products take two tokens per instruction (v_dot2_f32_f16 of a P pair and
  // a V pair, fp32 accumulate); the other types keep fp32 P, [TPW][R]
  constexpr bool kP16 = T::kCode == PKV_F16;
  _Float16* sp16 = reinterpret_cast<_Float16*>(smem) + w * TPW * R;

  // ---- scores: one token per lane, R rows, whole K row ---------------------
  float sreg[IT][R];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int tl = wt0 + it * 64 + lane;
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.f;
    if (it * 64 + lane < wn) {
      const int64_t blk = clamp_block(tab[tl >> 4], num_blocks);
      const unsigned char* kp = kpool + (((blk * Hkv + g) * C) * kBlockSize + (tl & 15)) * 16;
      u32x4 kc[C];
#pragma unroll
      for (int c = 0; c < C; ++c) kc[c] = ld16_stream(kp + c * (kBlockSize * 16));
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const typename T::bits* qr = q + ((int64_t)s * Hq + g * G + r) * D;
        if constexpr (ES == 2) {
          const uint32_t* qw = reinterpret_cast<const uint32_t*>(qr);
#pragma unroll
          for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r] = dot2<T>(qw[c * 4 + e], kc[c][e], acc[r]);
        } else {
          const float* qf = reinterpret_cast<const float*>(qr);
#pragma unroll
          for (int c = 0; c < C; ++c)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[r] = fmaf(qf[c * 4 + e], __uint_as_float(kc[c][e]), acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) sreg[it][r] = it * 64 + lane < wn ? acc[r] * scale_log2 : -INFINITY;
  }

  // ---- wave-local softmax state -------------------------------------------
  float mw[R], lw[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float m = sreg[0][r];
#pragma unroll
    for (int it = 1; it < IT; ++it) m = fmaxf(m, sreg[it][r]);
    mw[r] = wave_max(m);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const bool valid = it * 64 + lane < wn;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float e = valid ? __builtin_amdgcn_exp2f(sreg[it][r] - mw[r]) : 0.f;
      if constexpr (kP16)
        sp16[r * TPW + it * 64 + lane] = (_Float16)e;
      else
        sp[it * 64 + lane][r] = e;
      sreg[it][r] = e;
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float l = sreg[0][r];
#pragma unroll
    for (int it = 1; it < IT; ++it) l += sreg[it][r];
    lw[r] = wave_sum(l);
  }
  // the probabilities are read back by other lanes of this wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- values: lane owns NI dims x TPC tokens of each block -----------------
  // Chunk i of a block's V tile (1 KiB per wave instruction, fully coalesced)
  // gives lane l the dim (i*64 + l) / CPR and tokens (l % CPR) * TPC + [0, TPC).
  float o[R][NI];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int i = 0; i < NI; ++i) o[r][i] = 0.f;
  const int tg = lane % CPR;
  const int nbw = (wn + kBlockSize - 1) / kBlockSize;
  // V tiles, one block (D * 16 elements) per step of the wave.
  auto load_v = [&](int bl, u32x4 (&vv)[NI]) {
    const int64_t blk = clamp_block(tab[wt0 / kBlockSize + bl], num_blocks);
    const unsigned char* vp = vpool + (blk * Hkv + g) * (int64_t)VTILE + lane * 16;
#pragma unroll
    for (int i = 0; i < NI; ++i) vv[i] = ld16_stream(vp + i * 1024);
  };
  // block bl + 1's loads are issued before block bl's products while the
  // accumulators stay small (R * NI <= 16: G <= 4 at head_dim 128, G <= 8 at
  // 64); beyond, the second buffer costs occupancy or spills
  constexpr bool kPipeV = R * NI <= 16;
  u32x4 vcur[NI], vnxt[NI];
  if constexpr (kPipeV) {
    if (nbw > 0) load_v(0, vnxt);
  }
#pragma unroll 1
  for (int bl = 0; bl < nbw; ++bl) {
    if constexpr (kPipeV) {
#pragma unroll
      for (int i = 0; i < NI; ++i) vcur[i] = vnxt[i];
      if (bl + 1 < nbw) load_v(bl + 1, vnxt);
    } else {
      load_v(bl, vcur);
    }
    const int tb = wt0 / kBlockSize + bl;  // partition-local block
    const int ntok = n - tb * kBlockSize;
    const float(*pb)[R] = sp + bl * kBlockSize + tg * TPC;
    if constexpr (kP16) {
      // the lane's TPC = 8 tokens of the block: four fp16 P pairs per row
      u32x4 pp[R];
#pragma unroll
      for (int r = 0; r < R; ++r)
        pp[r] = *reinterpret_cast<const u32x4*>(sp16 + r * TPW + bl * kBlockSize + tg * TPC);
      if (ntok < kBlockSize) {  // zero V of slots past the context (they may hold anything)
        const int nv = ntok - tg * TPC;
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            vcur[i][e] &= 2 * e + 1 < nv ? 0xffffffffu : (2 * e < nv ? 0x0000ffffu : 0u);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int r = 0; r < R; ++r) o[r][i] = dot2<T>(pp[r][e], vcur[i][e], o[r][i]);
      continue;
    }
    auto accumulate = [&](auto masked) {
#pragma unroll
      for (int tt = 0; tt < TPC; ++tt) {
        float pv[R];
#pragma unroll
        for (int r = 0; r < R; ++r) pv[r] = pb[tt][r];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          float x;
          if constexpr (ES == 2) {
            float lo, hi;
            unpack2<T>(vcur[i][tt >> 1], lo, hi);
            x = (tt & 1) ? hi : lo;
          } else {
            x = __uint_as_float(vcur[i][tt]);
          }
          if constexpr (decltype(masked)::value) {
            x = tg * TPC + tt < ntok ? x : 0.f;  // slots past the context may hold anything
          }
#pragma unroll
          for (int r = 0; r < R; ++r) o[r][i] = fmaf(pv[r], x, o[r][i]);
        }
      }
    };
    if (ntok >= kBlockSize)
      accumulate(std::false_type{});
    else
      accumulate(std::true_type{});
  }
  // add the CPR lanes that share a dim
#pragma unroll
  for (int msk = 1; msk < CPR; msk <<= 1)
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < NI; ++i) o[r][i] += __shfl_xor(o[r][i], msk, 64);

  __syncthreads();  // all waves are done with the probabilities
  float(*so)[R][D] = reinterpret_cast<float(*)[R][D]>(smem);
  if (tg == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int i = 0; i < NI; ++i) so[w][r][(i * 64 + lane) / CPR] = o[r][i];
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      sml[w * R + r][0] = mw[r];
      sml[w * R + r][1] = lw[r];
    }
  }
  __syncthreads();

  // ---- merge the waves' partial softmax states ------------------------------
  for (int i = tid; i < R * D; i += WAVES * 64) {
    const int r = i / D, j = i % D;
    float Mx = sml[r][0];
#pragma unroll
    for (int k = 1; k < WAVES; ++k) Mx = fmaxf(Mx, sml[k * R + r][0]);
    float acc = 0.f, l = 0.f;
#pragma unroll
    for (int k = 0; k < WAVES; ++k) {
      const float f = __builtin_amdgcn_exp2f(sml[k * R + r][0] - Mx);  // 0 for a wave with no tokens
      acc = fmaf(f, so[k][r][j], acc);
      l = fmaf(f, sml[k * R + r][1], l);
    }
    const int64_t row = (int64_t)s * Hq + g * G + r;
    const int nparts = (clamp_len(lens[s], max_context_len) + PART - 1) / PART;
    if (nparts == 1) {
      store_out<OutCode>(out, row * D + j, acc / l);
    } else {
      ws_o[(row * max_parts + p) * D + j] = acc;
      if (j == 0) {
        ws_ml[(row * max_parts + p) * 2 + 0] = Mx;
        ws_ml[(row * max_parts + p) * 2 + 1] = l;
      }
    }
  }
}

// ---- partitions shared by sequences of one window ---------------------------
// Sequences forked from a common prefix name the same ref-counted physical
// blocks for it ("Memory sharing" with reference counts, vLLM Serving deep
// dive).  When several sequences of the batch name the same 32 blocks for a
// full partition p, one workgroup reads those K/V bytes once and serves all
// of them: with k sequences the partition is a (k G) x 512 x D contraction,
// done on MFMA by decode_shared_kernel.  Runs are formed inside aligned
// windows of KM = kRunRows / G sequences, in any order within the window:
//  * member i of the window is eligible for p when its context fills p;
//  * eligible members whose first block id for p is the same form a class,
//    led by its lowest member c;
//  * the run of the class is c and every other member whose 32 ids for p all
//    equal c's; a run of one sequence stays with the per-sequence kernel.
// Both kernels take this decision the same way, so each (sequence, p) is
// served by exactly one workgroup.
constexpr int kRunRows = 32;                     // query rows of a shared run (two 16-row MFMA tiles)
constexpr int kPartBlocks = kPart / kBlockSize;  // blocks per partition
static_assert(kPartBlocks <= 64, "one wave compares a partition's block ids");

// Is (s, p) served by a shared workgroup, i.e. is s in a run of two or more?
// The loads that decide it for most (s, p) — every window member's length
// and first block id for p, one member per lane — are issued together by
// probe_share, before the caller's own exits, so that the decision costs one
// round of loads; only a class of two or more compares all ids.  (Held as
// wave-uniform values read by the scalar unit instead, the window did not
// decide faster, and 32 members overflow the scalar registers.)
struct ShareProbe {
  int32_t id;  // lane i < KM: first block id of p for window member i
  int L;       // and its length (-1: past the batch, or not a member lane)
};

template <typename T, int G>
__device__ __forceinline__ ShareProbe probe_share(const int32_t* __restrict__ tables, int max_blocks,
                                                  const int32_t* __restrict__ lens, int B, int s, int p) {
  ShareProbe r{0, -1};
  if constexpr (T::kBytes != 4) {
    constexpr int KM = kRunRows / G;
    const int64_t col = (int64_t)p * kPartBlocks;  // < max_blocks for every p < max_parts
    const int lane = threadIdx.x & 63, a = s - s % KM + lane;
    if (lane < KM && a < B) {
      r.id = tables[(int64_t)a * max_blocks + col];
      r.L = lens[a];
    }
  }
  return r;
}

template <typename T, int G>
__device__ __forceinline__ bool in_shared_run(const ShareProbe& pr, const int32_t* __restrict__ tables,
                                              int max_blocks, int max_context_len, int s, int p, int L) {
  if constexpr (T::kBytes == 4) {
    return false;  // fp32 K/V: no MFMA path
  } else {
    constexpr int KM = kRunRows / G;
    const int need = (p + 1) * kPart;
    if (L < need) return false;
    const int me = s % KM, s_first = s - me;
    // s's class: eligible members with s's first block id (s is one of them)
    const int32_t id_s = __builtin_amdgcn_readlane(pr.id, me);
    const uint32_t cls =
        (uint32_t)__ballot(pr.L >= 0 && clamp_len(pr.L, max_context_len) >= need && pr.id == id_s);
    if (__popc(cls) < 2) return false;
    const int c = __builtin_ctz(cls);  // the class leader
    const int64_t col = (int64_t)p * kPartBlocks;
    const int lane = threadIdx.x & 63;
    const int32_t mine = lane < kPartBlocks ? tables[(int64_t)s * max_blocks + col + lane] : 0;
    if (me != c)  // a member: in the run when all its ids equal the leader's
      return __all(lane >= kPartBlocks || tables[(int64_t)(s_first + c) * max_blocks + col + lane] == mine);
    // the leader: a run when some other member's ids all equal its own
    for (uint32_t o = cls & (cls - 1u); o != 0u; o &= o - 1u) {
      const int t = __builtin_ctz(o);
      if (__all(lane >= kPartBlocks || tables[(int64_t)(s_first + t) * max_blocks + col + lane] == mine))
        return true;
    }
    return false;
  }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

template <typename T>
__device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (T::kCode == PKV_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2v_t));
}
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
// two fp32 -> two bf16 (round to nearest even), the first in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2v_t));
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}
// A probability p as a pair of bf16 values hi + lo with hi = bf16(p) and lo =
// bf16(p - hi): their sum carries p to about 2^-17 relative, so a bf16 V
// operand (exact, any finite value) and the pair give two exact-product
// MFMAs whose sum is p * v to that precision.
__device__ __forceinline__ void split_bf16x2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - bf16lo(hi), b - bf16hi(hi));
}
// Max / sum over lanes l, l^16, l^32, l^48 (the lanes holding one MFMA row).
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int ROWS, int NW = kWaves, int PBLK = kPartBlocks>
struct RunLds {
  float o[NW][ROWS][D + 4];  // the waves' unnormalised outputs (rows padded: LDS banks)
  float ml[NW][ROWS][2];     // and (max, sum) per row
  float wgt[ROWS][NW];       // merge weights 2^(m_w - M) per row
  float row_m[ROWS], row_l[ROWS];
  int row_parts[ROWS];        // partitions of the row's sequence
  int32_t blk[PBLK];          // the partition's block ids
};

// 8 E4M3 codes (two words, the first code in the low byte) -> one 8-element
// MFMA operand of fp16 or bf16 values.  Exact: both types hold every E4M3
// value.
template <typename QT>
__device__ __forceinline__ u32x4 e4m3x8_to(uint32_t w0, uint32_t w1) {
  u32x4 r;
  if constexpr (QT::kCode == PKV_BF16) {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true));
  } else {
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true));
  }
  return r;
}

__device__ __forceinline__ uint64_t ld8(const void* p) { return *reinterpret_cast<const uint64_t*>(p); }

// Which query rows an MFMA partition serves.  Row r of the 16 RT-row tile is
// member r / G, query head r % G of the KV head; a member owns one query
// token and a row of q / out in units of Hq rows (base).
//  * SeqRows: members are sequences s .. s + k - 1 of a decode batch, one
//    token each, sharing the partition's blocks (here k = 1);
//  * SetRows: members are the sequences of a shared run (below);
//  * TokenRows: members are query tokens q0 .. q0 + k - 1 of one sequence at
//    absolute positions pos0 .. pos0 + k - 1, each attending keys 0 .. its
//    position (causal), as in verifying several drafted tokens at once;
//  * WholeRows: one sequence over its whole context (the whole-context path).
struct SeqRows {
  static constexpr bool kCausal = false;
  int s, k;
  const int32_t* lens;
  int max_context_len;
  __device__ int table_row() const { return s; }
  __device__ int members() const { return k; }
  __device__ int64_t base(int mi) const { return (int64_t)s + mi; }
  __device__ int parts(int mi) const { return (clamp_len(lens[s + mi], max_context_len) + kPart - 1) / kPart; }
  __device__ int limit(int) const { return 0x7fffffff; }
};
// SetRows: members are the sequences s0 + idx[0], s0 + idx[1], .. of a run
// (idx ascending, in LDS), one token each, sharing the partition's blocks.
struct SetRows {
  static constexpr bool kCausal = false;
  int s0, k;
  const int* idx;
  const int32_t* lens;
  int max_context_len;
  __device__ int table_row() const { return s0 + idx[0]; }
  __device__ int members() const { return k; }
  __device__ int64_t base(int mi) const { return (int64_t)s0 + idx[mi]; }
  __device__ int parts(int mi) const {
    return (clamp_len(lens[s0 + idx[mi]], max_context_len) + kPart - 1) / kPart;
  }
  __device__ int limit(int) const { return 0x7fffffff; }
};
struct TokenRows {
  static constexpr bool kCausal = true;
  int s, q0, k, pos0;
  __device__ int table_row() const { return s; }
  __device__ int members() const { return k; }
  __device__ int64_t base(int mi) const { return (int64_t)q0 + mi; }
  __device__ int parts(int mi) const { return (pos0 + mi + kPart) / kPart; }  // partitions holding keys 0 .. pos
  __device__ int limit(int mi) const { return pos0 + mi + 1; }
};
// WholeRows: the G query heads of sequence s over its whole context, one
// "partition" of up to kWholeSpanM tokens whose result is final (no merge).
struct WholeRows {
  static constexpr bool kCausal = false;
  int s;
  __device__ int table_row() const { return s; }
  __device__ int members() const { return 1; }
  __device__ int64_t base(int) const { return s; }
  __device__ int parts(int) const { return 1; }
  __device__ int limit(int) const { return 0x7fffffff; }
};

// One partition on MFMA for the query rows R describes, whose members all
// read the same blocks for it (16 RT rows: row r = member r / G, head r % G;
// rows past k G repeat member 0 and are not stored).  The first n tokens of
// the partition are valid (Masked; otherwise all kPart), and with causal rows
// member m sees keys below R.limit(m) only.  K/V of the partition's blocks
// are read once.  Each of the NW waves takes kPart / NW tokens, in NH parts
// one after the other with a running softmax:
//  * S^T = K Q^T on MFMA 16x16x32 with K rows loaded from the pool straight
//    into operand layout (key order: see kNatural below).  8-bit keys are
//    widened to the query's type, and a lane's 16-byte K chunk (16 dims)
//    feeds two contraction slices; the query operands take the same dims;
//  * softmax over the wave's keys (base 2);
//  * O^T += V^T P^T with V loaded into operand layout: fp16 V with fp16
//    probabilities; bf16 V unconverted (any finite value) with each
//    probability split into a bf16 pair hi + lo, two products per tile;
//    8-bit V widened exactly to fp16, with fp16 probabilities;
//    the waves' (max, sum, o) are merged through LDS and written as each
//    member's partition result (8-bit values: times v_mul, the pool scale).
template <typename KV, typename QT, int D, int G, int RT, bool Masked, int OutCode, int NH, int NW,
          int PBLK = kPartBlocks, bool kEven = false, typename Rows>
__device__ __forceinline__ void mfma_partition(const Rows& R, int n, int g, int p, RunLds<D, 16 * RT, NW, PBLK>& sh,
                                               void* __restrict__ out, float* __restrict__ ws_o,
                                               float* __restrict__ ws_ml, const typename QT::bits* __restrict__ q,
                                               const unsigned char* __restrict__ kpool,
                                               const unsigned char* __restrict__ vpool,
                                               const int32_t* __restrict__ tables, int max_blocks, int Hkv,
                                               int64_t num_blocks, float scale_log2, float v_mul, int max_parts) {
  constexpr bool F8 = KV::kBytes == 1;
  constexpr bool kCausal = Rows::kCausal;
  // key order of the score tiles.  16-bit K/V, natural order: tile kt is
  // block kt of the part, row m its token m (a K operand instruction reads
  // 1 KiB, whole lines; a lane's eight keys of a product are four of each
  // block of a pair, two 8-byte V pieces).  8-bit K/V, line order: tile
  // 2 kp + h holds tokens 8 h .. 8 h + 7 of both blocks of pair kp (each
  // chunk group reads two whole 128-byte lines), and the probabilities are
  // realigned across lane groups before the value product so that a lane's
  // eight keys are eight consecutive keys of one block, one 8-byte V piece
  // (natural order would need 4-byte V pieces and twice the V instructions).
  static_assert(KV::kBytes != 4, "fp32 K/V have no MFMA path");
  constexpr bool kNatural = !F8;
  static_assert(F8 || (KV::kBytes == 2 && KV::kCode == QT::kCode), "16-bit K/V take queries of their type");
  constexpr bool kSplitP = !F8 && KV::kCode == PKV_BF16;  // bf16 V: exact operand, P as a bf16 pair
  static_assert(Masked || !kCausal, "causal rows need the masked path");
  constexpr int DC = D / 32;                         // 32-dim slices of the score contraction
  constexpr int DT = D / 16;                         // 16-dim tiles of the output
  constexpr int CH = D * KV::kBytes / 16;            // 16-byte K chunks per token
  constexpr int KC = F8 ? D / 64 : DC;               // K chunks per lane and score tile
  constexpr int VROW = kBlockSize * KV::kBytes;      // bytes of one dim of a V tile
  constexpr int TILE = D * VROW;                     // bytes of one (block, head) tile
  constexpr int WB = PBLK / NW;                      // blocks per wave (NW waves of 64 lanes)
  constexpr int HB = WB / NH;                        // blocks per part of a wave
  static_assert(HB % 2 == 0 && HB * NH == WB, "wave parts take whole block pairs");
  using vraw_t = typename std::conditional<F8, uint64_t, u32x4>::type;
  const int Hq = Hkv * G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, r16 = lane & 15;
  const int k = R.members();

  // query rows as B operands: lane (q4, r16) holds row 16 rt + r16 and the
  // dims of its K operand (16-bit K: 32 dc + 8 q4 ..; 8-bit K: 64 (dc/2) +
  // 16 q4 + 8 (dc%2) ..)
  u32x4 bq[RT][DC];
  int klim[RT];  // causal rows: keys of this partition the lane's row sees
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = 16 * rt + r16;
    const int mi = row / G < k ? row / G : 0;
    const int lim = R.limit(mi) - p * kPart;
    klim[rt] = lim < n ? lim : n;
    const typename QT::bits* qp = q + (R.base(mi) * Hq + g * G + row % G) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      bq[rt][dc] = ld16(qp + (F8 ? 64 * (dc >> 1) + 16 * q4 + 8 * (dc & 1) : 32 * dc + 8 * q4));
  }

  // the partition's block ids, read once into LDS (0 past the valid tokens)
  if (tid < PBLK)
    sh.blk[tid] = (!Masked || tid * kBlockSize < n) ? tables[(int64_t)R.table_row() * max_blocks + p * PBLK + tid] : 0;
  __syncthreads();
  // the wave's blocks: WB from block w WB, or (kEven) the valid blocks dealt
  // evenly in whole pairs, so that a short context keeps every wave busy;
  // nw = the end of the wave's tokens (partition-relative)
  int wb = WB;
  if constexpr (kEven) {
    const int per = ((n + kBlockSize - 1) / kBlockSize + NW - 1) / NW;
    wb = (per + 1) & ~1;
    wb = wb < WB ? wb : WB;
  }
  const int32_t* tab = sh.blk + w * wb;
  const int wbase = w * wb * kBlockSize;  // the wave's first token in the partition
  const int nw = kEven ? (n < wbase + wb * kBlockSize ? n : wbase + wb * kBlockSize) : n;
  float m[RT], l[RT];
  f32x4 o[RT][DT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (!Masked || wbase < nw) {  // uniform per wave
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      m[rt] = -INFINITY;
      l[rt] = 0.f;
    }
    // the wave's blocks in NH parts, one after the other with a running
    // softmax (fewer registers in flight per part)
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int hb = h * HB;                      // the part's first block (wave-local)
      const int hbase = wbase + hb * kBlockSize;  // and token (partition-local)
      if (Masked && hbase >= nw) break;           // uniform
      // K operands: score tile kt, row m
      u32x4 ka[HB][KC];
      if constexpr (kNatural) {
        // tile kt = block hb + kt, row m = its token m: an instruction reads
        // 4 chunks x 16 tokens = 1 KiB contiguous
#pragma unroll
        for (int kt = 0; kt < HB; ++kt) {
          const bool in = !Masked || hbase + kt * kBlockSize < nw;
          const int64_t kb = clamp_block(tab[hb + kt], num_blocks);
          const unsigned char* kr = kpool + ((kb * Hkv + g) * CH + q4) * (kBlockSize * 16) + r16 * 16;
#pragma unroll
          for (int c = 0; c < KC; ++c)
            ka[kt][c] = in ? ld16_stream(kr + c * 4 * kBlockSize * 16) : u32x4{0u, 0u, 0u, 0u};
        }
      } else {
        // line order: tile 2 kp + h, row m = block 2 kp + m / 8 of the part,
        // token 8 h + m % 8 (each chunk group reads two whole lines)
        const int k_half = r16 >> 3, k_tok = r16 & 7;
#pragma unroll
        for (int kp = 0; kp < HB / 2; ++kp) {
          const bool in = !Masked || hbase + (2 * kp + k_half) * kBlockSize < nw;
          const int64_t kb = clamp_block(tab[hb + 2 * kp + k_half], num_blocks);
          const unsigned char* kr = kpool + ((kb * Hkv + g) * CH + q4) * (kBlockSize * 16) + k_tok * 16;
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int c = 0; c < KC; ++c)
              ka[2 * kp + h][c] = in ? ld16_stream(kr + (8 * h + c * 4 * kBlockSize) * 16) : u32x4{0u, 0u, 0u, 0u};
        }
      }
      f32x4 st[HB][RT];
      if constexpr (F8) {
#pragma unroll
        for (int kt = 0; kt < HB; ++kt)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) st[kt][rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kt = 0; kt < HB; ++kt)
#pragma unroll
          for (int dc = 0; dc < DC; ++dc) {
            const u32x4 a = e4m3x8_to<QT>(ka[kt][dc >> 1][2 * (dc & 1)], ka[kt][dc >> 1][2 * (dc & 1) + 1]);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) st[kt][rt] = mfma_qk<QT>(a, bq[rt][dc], st[kt][rt]);
          }
      } else {
#pragma unroll
        for (int kt = 0; kt < HB; ++kt)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dc = 0; dc < DC; ++dc) acc = mfma_qk<QT>(ka[kt][dc], bq[rt][dc], acc);
            st[kt][rt] = acc;
          }
      }
      // V operands, issued next, ahead of the softmax: lane (q4, r16) takes
      // dim 16 dt + r16 and the eight keys its probabilities cover — natural
      // order: keys 4 q4 .. 4 q4 + 3 of both blocks of the pair (two 8-byte
      // pieces of the dim's rows); line order (8-bit): keys 8 q4 .. 8 q4 + 7
      // of the pair, after the realignment (one piece of block q4 / 2's row)
      vraw_t vraw[HB / 2][DT];
#pragma unroll
      for (int kp = 0; kp < HB / 2; ++kp) {
        if constexpr (kNatural) {
          const bool inA = !Masked || hbase + 2 * kp * kBlockSize < nw;
          const bool inB = !Masked || hbase + (2 * kp + 1) * kBlockSize < nw;
          const int64_t vbA = clamp_block(tab[hb + 2 * kp], num_blocks);
          const int64_t vbB = clamp_block(tab[hb + 2 * kp + 1], num_blocks);
          const unsigned char* vrA = vpool + (vbA * Hkv + g) * (int64_t)TILE + r16 * VROW + q4 * (VROW / 4);
          const unsigned char* vrB = vpool + (vbB * Hkv + g) * (int64_t)TILE + r16 * VROW + q4 * (VROW / 4);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const uint64_t a = inA ? ld8_stream(vrA + dt * 16 * VROW) : 0ull;
            const uint64_t b = inB ? ld8_stream(vrB + dt * 16 * VROW) : 0ull;
            vraw[kp][dt] = u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
          }
        } else {
          const bool in = !Masked || hbase + (2 * kp + (q4 >> 1)) * kBlockSize < nw;
          const int64_t vb = clamp_block(tab[hb + 2 * kp + (q4 >> 1)], num_blocks);
          const unsigned char* vr = vpool + (vb * Hkv + g) * (int64_t)TILE + r16 * VROW + (q4 & 1) * (VROW / 2);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            if constexpr (F8)
              vraw[kp][dt] = in ? ld8_stream(vr + dt * 16 * VROW) : 0ull;
            else
              vraw[kp][dt] = ld16(vr + dt * 16 * VROW);
          }
        }
      }
      // exact softmax over the wave's keys, per row (running over the parts)
      // bf16 V is kept exact: P goes to the matrix cores as a bf16 pair
      // (hi, lo), two products per tile; fp16 and 8-bit V take fp16 P
      u32x4 pb[HB / 2][RT];
      u32x4 pbl[kSplitP ? HB / 2 : 1][RT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < HB; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float x = st[kt][rt][r] * scale_log2;
            if constexpr (Masked) {  // keys past the context may hold anything
              const int key = kNatural ? hbase + kt * kBlockSize + 4 * q4 + r
                                       : hbase + ((kt >> 1) * 2 + (q4 >> 1)) * kBlockSize + 8 * (kt & 1) +
                                             4 * (q4 & 1) + r;
              x = key < (kCausal ? (klim[rt] < nw ? klim[rt] : nw) : nw) ? x : -INFINITY;
            }
            st[kt][rt][r] = x;
            mx = fmaxf(mx, x);
          }
        const float mnew = fmaxf(m[rt], rows4_max(mx));
        // a causal row may see none of the keys so far: its weights are 0
        const float mref = (kCausal && mnew == -INFINITY) ? 0.f : mnew;
        if (h > 0) {  // rescale what the earlier parts accumulated
          const float alpha = __builtin_amdgcn_exp2f(m[rt] - mref);
          l[rt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= alpha;
        }
        float ls = 0.f;
#pragma unroll
        for (int kt = 0; kt < HB; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            st[kt][rt][r] = __builtin_amdgcn_exp2f(st[kt][rt][r] - mref);
            ls += st[kt][rt][r];
          }
        l[rt] += rows4_sum(ls);
        m[rt] = mnew;
        // B operand of the pair: the lane's four keys of tile 2 kp, then of 2 kp + 1
#pragma unroll
        for (int kp = 0; kp < HB / 2; ++kp)
          if constexpr (kSplitP) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              uint32_t hi, lo;
              split_bf16x2(st[2 * kp + (e >> 1)][rt][2 * (e & 1)], st[2 * kp + (e >> 1)][rt][2 * (e & 1) + 1], hi,
                           lo);
              pb[kp][rt][e] = hi;
              pbl[kp][rt][e] = lo;
            }
          } else {
            pb[kp][rt] = u32x4{pack_f16x2(st[2 * kp][rt][0], st[2 * kp][rt][1]),
                               pack_f16x2(st[2 * kp][rt][2], st[2 * kp][rt][3]),
                               pack_f16x2(st[2 * kp + 1][rt][0], st[2 * kp + 1][rt][1]),
                               pack_f16x2(st[2 * kp + 1][rt][2], st[2 * kp + 1][rt][3])};
            if constexpr (!kNatural) {
              // line order: lane group q4 holds tokens 4 (q4 & 1) .. + 3 of
              // block q4 / 2 in each tile; the odd rows of tile 2 kp's words
              // trade with the even rows of tile 2 kp + 1's, leaving lane group
              // q4 tokens 8 (q4 & 1) .. + 7 of block q4 / 2, as its V piece
              const auto a0 = __builtin_amdgcn_permlane16_swap(pb[kp][rt][0], pb[kp][rt][2], false, false);
              const auto a1 = __builtin_amdgcn_permlane16_swap(pb[kp][rt][1], pb[kp][rt][3], false, false);
              pb[kp][rt] = u32x4{a0[0], a1[0], a0[1], a1[1]};
            }
          }
      }
      // O^T += V^T P^T over each pair's 32 keys
#pragma unroll
      for (int kp = 0; kp < HB / 2; ++kp)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          u32x4 va;
          if constexpr (F8) {
            uint64_t bytes = vraw[kp][dt];
            if constexpr (Masked) {  // zero the codes of keys past the context (they may be NaN codes)
              const int nv = nw - (hbase + kp * 2 * kBlockSize + 8 * q4);
              bytes &= nv >= 8 ? ~0ull : (nv <= 0 ? 0ull : (1ull << (8 * nv)) - 1ull);
            }
            va = e4m3x8_to<F16>((uint32_t)bytes, (uint32_t)(bytes >> 32));
          } else {
            u32x4 vv = vraw[kp][dt];
            if constexpr (Masked) {  // zero keys past the context (they may hold NaN)
#pragma unroll
              for (int half = 0; half < 2; ++half) {  // blocks 2 kp and 2 kp + 1
                const int nv = nw - (hbase + (2 * kp + half) * kBlockSize + 4 * q4);
#pragma unroll
                for (int e = 0; e < 2; ++e)
                  vv[2 * half + e] &= 2 * e + 1 < nv ? 0xffffffffu : (2 * e < nv ? 0x0000ffffu : 0u);
              }
            }
            va = vv;  // f16 V as it is; bf16 V with the split probabilities
          }
          if constexpr (kSplitP) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
              o[rt][dt] = mfma_bf16(va, pb[kp][rt], o[rt][dt]);
              o[rt][dt] = mfma_bf16(va, pbl[kp][rt], o[rt][dt]);
            }
          } else {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) o[rt][dt] = mfma_f16(va, pb[kp][rt], o[rt][dt]);
          }
        }
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      m[rt] = -INFINITY;  // a wave without keys: weight 0 in the merge
      l[rt] = 0.f;
    }
  }
  // merge the waves: lane (q4, r16) holds o^T[dim 16 dt + 4 q4 + r][row 16 rt + r16]
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int r = 0; r < 4; ++r) sh.o[w][16 * rt + r16][16 * dt + 4 * q4 + r] = o[rt][dt][r];
    if (q4 == 0) {
      sh.ml[w][16 * rt + r16][0] = m[rt];
      sh.ml[w][16 * rt + r16][1] = l[rt];
    }
  }
  __syncthreads();
  const int rows = k * G;
  if (tid < rows) {  // per row: merged max and sum, the waves' weights, the sequence's partitions
    float Mx = sh.ml[0][tid][0];
#pragma unroll
    for (int x = 1; x < NW; ++x) Mx = fmaxf(Mx, sh.ml[x][tid][0]);
    float den = 0.f;
#pragma unroll
    for (int x = 0; x < NW; ++x) {
      // 0 for a wave with no keys (a causal row may have none in the whole partition)
      const float mw = sh.ml[x][tid][0];
      const float f = (kCausal && mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - Mx);
      sh.wgt[tid][x] = f;
      den = fmaf(f, sh.ml[x][tid][1], den);
    }
    sh.row_m[tid] = Mx;
    sh.row_l[tid] = den;
    sh.row_parts[tid] = R.parts(tid / G);
  }
  __syncthreads();
  for (int i = tid; i < rows * D; i += NW * 64) {
    const int row = i / D, j = i % D;
    // a causal row whose keys all lie in earlier partitions has no result
    // here: the partitions that hold its keys write it (its partition count
    // is at most p)
    if (kCausal && p >= sh.row_parts[row]) continue;
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < NW; ++x) acc = fmaf(sh.wgt[row][x], sh.o[x][row][j], acc);
    if constexpr (F8) acc *= v_mul;
    const int64_t orow = R.base(row / G) * Hq + g * G + row % G;
    if (sh.row_parts[row] == 1) {
      store_out<OutCode>(out, orow * D + j, acc / sh.row_l[row]);
    } else {
      ws_o[(orow * max_parts + p) * D + j] = acc;
      if (j == 0) {
        ws_ml[(orow * max_parts + p) * 2 + 0] = sh.row_m[row];
        ws_ml[(orow * max_parts + p) * 2 + 1] = sh.row_l[row];
      }
    }
  }
  __syncthreads();  // the LDS is reused by the window's next run
}

// Grid (KV head, run window, slot).  The workgroups of a window find its
// runs for every partition the same way and deal them out: the window's
// candidate runs, counted over its partitions in order, go round-robin to the
// kRunSlots slots, so that runs of one window (and partitions) are served side
// by side instead of one after another.
// This step's new K/V rows can be written by extra workgroups of the
// shared-run launch (grid z >= kRunSlots), so that the cache write costs no
// launch of its own and fills CUs the runs leave idle.  A run never covers
// a new token's block — the block a sequence appends into is its own after
// copy-on-write, so its ids differ from every other sequence's — hence the write
// and the runs touch disjoint bytes, and the per-sequence pass, launched
// after, reads the new rows.
struct AppendArgs {
  const unsigned char* key = nullptr;    // new rows: token i's K row at key + i * kstride_b
  const unsigned char* value = nullptr;
  int64_t kstride_b = 0, vstride_b = 0;  // bytes between consecutive tokens' rows
  unsigned char* kpool = nullptr;        // the pools, written
  unsigned char* vpool = nullptr;
  const int64_t* slots = nullptr;        // slot of new token i (outside the pool: skipped)
  int64_t T = 0;                         // new tokens (0: no cache write)
  int64_t num_slots = 0;
  float k_inv = 1.f, v_inv = 1.f;        // 8-bit pools: the rows are quantised (x * inv), source type QT
};

constexpr int kSharedWaves = PKV_SHARED_WAVES;  // waves per shared-run workgroup (4 or 8)
constexpr int kRunSlots = PKV_RUN_SLOTS;        // workgroups per run window
constexpr int kProbeIds = 512;                  // window members x partitions probed per round
template <typename KV, typename QT, int D, int G, int OutCode>
__global__ void __launch_bounds__(kSharedWaves * 64, kSharedWaves == 8 ? 1 : 2)
decode_shared_kernel(void* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
                     const typename QT::bits* __restrict__ q, const unsigned char* __restrict__ kpool,
                     const unsigned char* __restrict__ vpool, const int32_t* __restrict__ tables,
                     int max_blocks, const int32_t* __restrict__ lens, int B, int Hkv, int64_t num_blocks,
                     int max_context_len, float scale_log2, float v_mul, int max_parts, AppendArgs app) {
  if constexpr (KV::kBytes == 4) {
    return;
  } else {
    constexpr int KM = kRunRows / G;
    static_assert(KM <= 32, "run window fits a 32-bit mask");
    constexpr int kThr = kSharedWaves * 64;
    if (blockIdx.z >= kRunSlots) {  // the cache write of this step's new tokens
      const int C = D * KV::kBytes / 16;  // 16-byte pool chunks per head row
      const int64_t total = app.T * Hkv * C;
      const int64_t wg = ((int64_t)(blockIdx.z - kRunSlots) * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x;
      const int64_t stride = (int64_t)(gridDim.z - kRunSlots) * gridDim.y * gridDim.x * kThr;
      for (int64_t idx = wg * kThr + threadIdx.x; idx < total; idx += stride) {
        const int64_t i = idx % app.T;  // tokens fastest, as in reshape_and_cache
        const int64_t rest = idx / app.T;
        if constexpr (KV::kBytes == 2)
          cache_write_chunk<2>(app.key, app.value, app.kstride_b, app.vstride_b, app.kpool, app.vpool, app.slots[i],
                               app.num_slots, i, (int)(rest % Hkv), (int)(rest / Hkv), Hkv, D);
        else
          cache_write_chunk_fp8<QT>(app.key, app.value, app.kstride_b, app.vstride_b, app.kpool, app.vpool,
                                    app.slots[i], app.num_slots, i, (int)(rest % Hkv), (int)(rest / Hkv), Hkv, D,
                                    app.k_inv, app.v_inv);
      }
      return;
    }
    constexpr int NP = kProbeIds / KM;  // partitions probed per round
    static_assert(NP <= kThr, "one thread clears each partition's mask");
    __shared__ __attribute__((aligned(16))) RunLds<D, kRunRows, kSharedWaves> sh;
    __shared__ int32_t fid[NP][KM];    // first block id of each (partition, member)
    __shared__ uint32_t clsm[NP][KM];  // members of the class that member c leads
    __shared__ uint32_t elig[NP];      // per partition: bit i = member i fills it
    __shared__ uint32_t lead[NP];      // per partition: bit c = c leads a class of two or more
    __shared__ uint32_t bad;         // members of a class whose ids differ from the leader's
    __shared__ int midx[KM];         // the run's members (window-relative, ascending)
    const int g = blockIdx.x, win = blockIdx.y, slot = blockIdx.z;
    const int s_first = win * KM;
    if (s_first >= B) return;
    const int tid = threadIdx.x;
    int unit = 0;  // candidate runs of the window so far, in (partition, leader) order
    for (int pc = 0; pc < max_parts; pc += NP) {
      const int np = max_parts - pc < NP ? max_parts - pc : NP;
      // one thread per (partition, member): its first block id and whether
      // it fills the partition (one round of loads, every one in bounds)
      if (tid < NP) {
        elig[tid] = 0u;
        lead[tid] = 0u;
      }
      for (int t = tid; t < np * KM; t += kThr) clsm[t / KM][t % KM] = 0u;
      __syncthreads();
      for (int t = tid; t < np * KM; t += kThr) {
        const int pp = t / KM, i = t % KM, a = s_first + i, p = pc + pp;
        if (a < B) {
          fid[pp][i] = tables[(int64_t)a * max_blocks + p * kPartBlocks];
          if (clamp_len(lens[a], max_context_len) >= (p + 1) * kPart) atomicOr(&elig[pp], 1u << i);
        }
      }
      __syncthreads();
      // the classes, a wave per partition: lane i finds its leader, the
      // lowest eligible member with the same first id (ids broadcast from
      // their lanes, no LDS round trips in the loop)
      {
        const int lane = tid & 63;
        for (int pp = tid >> 6; pp < np; pp += kSharedWaves) {
          const uint32_t el = elig[pp];
          const int32_t id = lane < KM ? fid[pp][lane] : 0;
          int c = lane;
          for (uint32_t x = el; x != 0u; x &= x - 1u) {
            const int j = __builtin_ctz(x);
            const int32_t idj = __builtin_amdgcn_readlane(id, j);
            c = (j < c && idj == id) ? j : c;
          }
          if (lane < KM && ((el >> lane) & 1u)) {
            atomicOr(&clsm[pp][c], 1u << lane);
            if (c != lane) atomicOr(&lead[pp], 1u << c);
          }
        }
      }
      __syncthreads();
      for (int pp = 0; pp < np; ++pp) {
        const int p = pc + pp;
        const int64_t col = (int64_t)p * kPartBlocks;
        // classes of two or more, lowest leader first (uniform)
        for (uint32_t ld = lead[pp]; ld != 0u; ld &= ld - 1u) {
          const int c = __builtin_ctz(ld);
          const uint32_t cls = clsm[pp][c];
          if (unit++ % kRunSlots != slot) continue;
          // full comparison of the class's ids for p against the leader's,
          // one thread per (member, entry): a mismatch drops the member
          if (tid == 0) bad = 0u;
          __syncthreads();
          for (int t = tid; t < KM * kPartBlocks; t += kThr) {
            const int i = t / kPartBlocks, e = t % kPartBlocks;
            if (i != c && ((cls >> i) & 1u) &&
                tables[(int64_t)(s_first + i) * max_blocks + col + e] !=
                    tables[(int64_t)(s_first + c) * max_blocks + col + e])
              atomicOr(&bad, 1u << i);
          }
          __syncthreads();
          const uint32_t run = cls & ~bad;  // the leader and the members that join it
          if (__popc(run) < 2) {
            __syncthreads();  // bad is rewritten by the next class
            continue;
          }
          if (tid == 0) {
            int k = 0;
            for (uint32_t x = run; x != 0u; x &= x - 1u) midx[k++] = __builtin_ctz(x);
          }
          __syncthreads();
          mfma_partition<KV, QT, D, G, kRunRows / 16, false, OutCode, PKV_SHARED_PARTS, kSharedWaves>(
              SetRows{s_first, (int)__popc(run), midx, lens, max_context_len}, kPart, g, p, sh, out, ws_o, ws_ml, q,
              kpool, vpool, tables, max_blocks, Hkv, num_blocks, scale_log2, v_mul, max_parts);
          // (mfma_partition ends with a barrier: bad and midx may be rewritten)
        }
      }
      __syncthreads();  // fid, clsm, elig and lead are rewritten by the next round
    }
  }
}

// The per-sequence partitions of an 8-bit cache, on MFMA as well: widening
// the codes costs one conversion per two values, more than the VALU kernel's
// issue budget leaves at full bandwidth, while the matrix cores have room to
// pad the G query rows of a KV head to 16.
template <typename QT, int D, int G, int OutCode>
__global__ void __launch_bounds__(kThreads, 2)
decode_fp8_partition_kernel(void* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
                            const typename QT::bits* __restrict__ q, const unsigned char* __restrict__ kpool,
                            const unsigned char* __restrict__ vpool, const int32_t* __restrict__ tables,
                            int max_blocks, const int32_t* __restrict__ lens, int Hkv, int64_t num_blocks,
                            int max_context_len, float scale_log2, float v_mul, int max_parts) {
  static_assert(G <= 16, "one 16-row tile");
  __shared__ __attribute__((aligned(16))) RunLds<D, 16> sh;
  // last partitions first, as in decode_partition_kernel
  const int g = blockIdx.x, s = blockIdx.y, p = gridDim.z - 1 - blockIdx.z;
  const int Hq = Hkv * G;
  const int Lraw = lens[s];
  const ShareProbe pr = probe_share<FP8, G>(tables, max_blocks, lens, gridDim.y, s, p);
  const int L = clamp_len(Lraw, max_context_len);
  const int nparts = (L + kPart - 1) / kPart;
  if (p >= (nparts > 0 ? nparts : 1)) return;
  if (L == 0) {  // defined result for an empty context: zeros
    for (int i = threadIdx.x; i < G * D; i += kThreads)
      store_out<OutCode>(out, ((int64_t)s * Hq + g * G) * D + i, 0.f);
    return;
  }
  if (in_shared_run<FP8, G>(pr, tables, max_blocks, max_context_len, s, p, L)) return;
  const int t0 = p * kPart;
  const int n = (L - t0) < kPart ? (L - t0) : kPart;  // tokens in this partition, >= 1
  mfma_partition<FP8, QT, D, G, 1, true, OutCode, PKV_FP8_PARTS, kWaves>(SeqRows{s, 1, lens, max_context_len}, n, g, p, sh, out, ws_o,
                                                  ws_ml, q, kpool, vpool, tables, max_blocks, Hkv, num_blocks,
                                                  scale_log2, v_mul, max_parts);
}

// The per-sequence partitions of 16-bit pools: the vector routine for G <= 4
// query rows per KV head; from G = 8 on the MFMA routine (the G rows padded to
// one 16-row tile, at most half of it idle), where the vector units' G
// products per cached element, not the reads, would set the pace.
constexpr int kSeqMfmaMinG = 8;
template <typename T, int D, int G, int OutCode>
__global__ void __launch_bounds__(kThreads, PKV_DECODE_MIN_WAVES)
decode_partition_kernel(void* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
                        const typename T::bits* __restrict__ q, const unsigned char* __restrict__ kpool,
                        const unsigned char* __restrict__ vpool, const int32_t* __restrict__ tables,
                        int max_blocks, const int32_t* __restrict__ lens, int Hkv, int64_t num_blocks,
                        int max_context_len, float scale_log2, int max_parts) {

  // last partitions first: long sequences' work starts early, the tail is
  // made of partitions every sequence has
  const int g = blockIdx.x, s = blockIdx.y, p = gridDim.z - 1 - blockIdx.z;
  const int Hq = Hkv * G;

  const int Lraw = lens[s];
  const ShareProbe pr = probe_share<T, G>(tables, max_blocks, lens, gridDim.y, s, p);
  const int L = clamp_len(Lraw, max_context_len);
  const int nparts = (L + kPart - 1) / kPart;
  if (p >= (nparts > 0 ? nparts : 1)) return;
  if (L == 0) {  // defined result for an empty context: zeros
    for (int i = threadIdx.x; i < G * D; i += kThreads)
      store_out<OutCode>(out, ((int64_t)s * Hq + g * G) * D + i, 0.f);
    return;
  }
  if (in_shared_run<T, G>(pr, tables, max_blocks, max_context_len, s, p, L)) return;
  const int t0 = p * kPart;
  const int n = (L - t0) < kPart ? (L - t0) : kPart;  // tokens in this partition
  if constexpr (T::kBytes == 2 && G >= kSeqMfmaMinG) {
    __shared__ __attribute__((aligned(16))) RunLds<D, 16> sh;
    mfma_partition<T, T, D, G, 1, true, OutCode, 2, kWaves>(SeqRows{s, 1, lens, max_context_len}, n, g, p, sh, out,
                                                           ws_o, ws_ml, q, kpool, vpool, tables, max_blocks, Hkv,
                                                           num_blocks, scale_log2, 1.f, max_parts);
  } else {
    // Per-wave probabilities [kWaves][TPW][R]; after the V pass the same
    // memory holds the waves' partial outputs [kWaves][R][D].
    constexpr int SMEM = (kPart > kWaves * D ? kPart : kWaves * D) * G;
    __shared__ __attribute__((aligned(16))) float smem[SMEM];
    __shared__ float sml[kWaves * G][2];
    const int32_t* tab = tables + (int64_t)s * max_blocks + t0 / kBlockSize;
    partition_rows<T, D, G, OutCode>(smem, sml, out, ws_o, ws_ml, q, kpool, vpool, tab, lens, s, g, p, n, Hkv,
                                     num_blocks, max_context_len, scale_log2, max_parts);
  }
}

// ---- short contexts in a small batch: one launch, no merge ------------------
// When every context fits the span (kWholeSpanM tokens on the MFMA routine,
// kWholeSpan on the vector one) and the batch has few (sequence, KV head)
// pairs, split partitions and the merge would leave the chip idle between
// three launches.  Instead one workgroup of kWholeWaves waves takes a whole
// (sequence, KV head), the waves' softmax states merge in LDS and the output
// is written directly.  Partitions that sequences share are read per sequence
// on this path.  16-bit and 8-bit pools run the MFMA partition routine (the G
// query rows padded to one 16-row tile: with G = 8 the vector routine's
// products, not the reads, set its pace), fp32 pools the vector routine;
// both deal the sequence's blocks evenly to the waves (the MFMA routine in
// whole block pairs), so a short context keeps every wave busy.
constexpr int kWholeSpan = 2048;      // context tokens one workgroup takes (vector routine)
constexpr int kWholeSpanM = 4096;     // and on the MFMA routine (16-bit and 8-bit pools)
constexpr int kWholeWaves = 16;       // its waves (4 per SIMD)

// Does a batch take the whole-context path?  One workgroup fills a CU and the
// 256 CUs take P = (sequence, KV head) pairs in rounds of 256.  16-bit and
// 8-bit pools take any G (one 16-row MFMA tile) and contexts up to 4096
// tokens; on fp32 pools the vector routine's per-wave accumulators must stay
// within 128 registers (G x D x 4 <= 1024) and its span is 2048.  Measured
// against the split path on uniform and prefix-sharing batches: up to 256
// pairs — one round — the whole-context launch wins except when fewer than
// 128 pairs hold contexts past 1536 tokens (too few CUs take part; the split
// path's 4x more workgroups win).  A second round: on the MFMA routine it
// wins from 384 pairs on at every length up to 2048 (TinyLlama and
// Llama-3-8B heads, 384 to 640 pairs) and loses at 320; it stops at 512
// pairs and 2048 tokens, past which reading shared partitions once and the
// split path's finer work units win on prefix-sharing batches.  The vector
// routine (fp32 pools) keeps the band it was measured for: 448 to 512 pairs
// with at least 384 KiB per pair.
inline bool whole_context(int B, int Hkv, int G, int D, int es, int max_context_len) {
  const int64_t units = (int64_t)B * Hkv;
  if (es == 4) {
    if (max_context_len > kWholeSpan || G * D * es > 1024) return false;
    if (units <= 256) return units >= 128 || max_context_len <= 1536;
    return units >= 448 && units <= 512 && (int64_t)max_context_len * 2 * D * es >= 384 * 1024;
  }
  if (max_context_len > kWholeSpanM) return false;
  if (units <= 256) return units >= 128 || max_context_len <= 1536;
  return units >= 384 && units <= 512 && max_context_len <= kWholeSpan;
}

// With this step's new rows (app.T > 0), the workgroup of (sequence s, KV
// head g) first writes head g of sequence s's new row into the pool: the
// row's block is the sequence's own (copy-on-write done before the append),
// so no other workgroup reads it, and a workgroup-scope release / acquire
// around a barrier orders the write before this workgroup's reads.
// KV is the pools' type, QT the queries' (the same for 16-bit and fp32
// pools; fp16 or bf16 queries over 8-bit pools, whose values are scaled by
// v_mul and whose new rows are quantised on the way in).
// SPAN: the launch's span (kWholeSpan, or kWholeSpanM when a context of the
// batch needs it): a wave takes at most SPAN / 16 / kWholeWaves blocks.
template <typename KV, typename QT, int D, int G, int OutCode, int SPAN>
__global__ void __launch_bounds__(kWholeWaves * 64, 1)
decode_whole_kernel(void* __restrict__ out, const typename QT::bits* __restrict__ q, const unsigned char* kpool,
                    const unsigned char* vpool, const int32_t* __restrict__ tables, int max_blocks,
                    const int32_t* __restrict__ lens, int Hkv, int64_t num_blocks, int max_context_len,
                    float scale_log2, float v_mul, AppendArgs app) {
  static_assert(G <= 16, "one 16-row tile");
  const int g = blockIdx.x, s = blockIdx.y;
  if (app.T > 0) {  // uniform
    constexpr int C = D * KV::kBytes / 16;  // 16-byte pool chunks per head row
    if (s < app.T && threadIdx.x < C) {
      if constexpr (KV::kBytes == 1)
        cache_write_chunk_fp8<QT>(app.key, app.value, app.kstride_b, app.vstride_b, app.kpool, app.vpool,
                                  app.slots[s], app.num_slots, s, g, threadIdx.x, Hkv, D, app.k_inv, app.v_inv);
      else
        cache_write_chunk<KV::kBytes>(app.key, app.value, app.kstride_b, app.vstride_b, app.kpool, app.vpool,
                                      app.slots[s], app.num_slots, s, g, threadIdx.x, Hkv, D);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  }
  const int L = clamp_len(lens[s], max_context_len);
  if (L == 0) {  // defined result for an empty context: zeros
    for (int i = threadIdx.x; i < G * D; i += kWholeWaves * 64)
      store_out<OutCode>(out, ((int64_t)s * Hkv * G + g * G) * D + i, 0.f);
    return;
  }
  if constexpr (KV::kBytes != 4) {
    // each wave's blocks in parts of 4 (head_dim 64, and 8-bit pools) or 2
    // (16-bit at 128): within 128 registers at 4 waves per SIMD
    constexpr int PB = SPAN / kBlockSize;
    __shared__ __attribute__((aligned(16))) RunLds<D, 16, kWholeWaves, PB> sh;
    mfma_partition<KV, QT, D, G, 1, true, OutCode, (PB / kWholeWaves) / ((D == 64 || KV::kBytes == 1) ? 4 : 2),
                   kWholeWaves, PB, true>(WholeRows{s}, L, g, 0, sh, out, nullptr, nullptr, q, kpool, vpool, tables,
                                       max_blocks, Hkv, num_blocks, scale_log2, v_mul, 1);
  } else {
    using T = KV;
    static_assert(SPAN == kWholeSpan, "the vector routine's span");
    constexpr int RMAX = G;
    constexpr int SMEM = (kWholeSpan > kWholeWaves * D ? kWholeSpan : kWholeWaves * D) * RMAX;
    __shared__ __attribute__((aligned(16))) float smem[SMEM];
    __shared__ float sml[kWholeWaves * RMAX][2];
    partition_rows<T, D, G, OutCode, kWholeSpan, kWholeWaves>(smem, sml, out, nullptr, nullptr, q, kpool, vpool,
                                                              tables + (int64_t)s * max_blocks, lens, s, g, 0, L,
                                                              Hkv, num_blocks, max_context_len, scale_log2, 1);
  }
}


template <int D, int OutCode, bool PerToken>
__global__ void __launch_bounds__(64)
decode_reduce_kernel(void* __restrict__ out, const float* __restrict__ ws_o, const float* __restrict__ ws_ml,
                     const int32_t* __restrict__ lens, const int32_t* __restrict__ tok_parts, int Hq,
                     int max_context_len, int max_parts) {
  // row blockIdx.y: a sequence (decode) or a query token (verify: its own
  // partition count, written by the partition pass)
  constexpr int DPL = D / 64;
  const int h = blockIdx.x, s = blockIdx.y, lane = threadIdx.x;
  int nparts;
  if constexpr (PerToken) {
    // clamped: a row no sequence covers (cu_q_lens breaks its contract)
    // reads nothing beyond its own workspace row
    nparts = tok_parts[s];
    nparts = nparts < 0 ? 0 : (nparts > max_parts ? max_parts : nparts);
  } else {
    int L = lens[s];
    L = L < 0 ? 0 : (L > max_context_len ? max_context_len : L);
    nparts = (L + kPart - 1) / kPart;
  }
  if (nparts <= 1) return;
  const int64_t row = (int64_t)s * Hq + h;
  const float* ml = ws_ml + row * max_parts * 2;
  const float* ob = ws_o + row * max_parts * D + lane * DPL;
  // The partials of PB partitions are loaded together (indexes clamped to
  // the last partition, so every load is in bounds and none waits on
  // another); the arithmetic is the plain two passes, partitions in order.
  constexpr int PB = 8;
  float mp[PB], lp[PB], op[PB][DPL];
  auto load = [&](int p0, bool with_o) {
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      const int p = p0 + j < nparts ? p0 + j : nparts - 1;
      mp[j] = ml[2 * p];
      lp[j] = ml[2 * p + 1];
      if (with_o)
#pragma unroll
        for (int dd = 0; dd < DPL; ++dd) op[j][dd] = ob[(int64_t)p * D + dd];
    }
  };
  load(0, true);
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < PB; ++j)
    if (j < nparts) M = fmaxf(M, mp[j]);
  for (int p0 = PB; p0 < nparts; p0 += PB) {  // more than PB partitions: the maxima first
    load(p0, false);
#pragma unroll
    for (int j = 0; j < PB; ++j)
      if (p0 + j < nparts) M = fmaxf(M, mp[j]);
  }
  if (nparts > PB) load(0, true);
  float den = 0.f, acc[DPL];
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) acc[dd] = 0.f;
  for (int p0 = 0; p0 < nparts; p0 += PB) {
    if (p0 > 0) load(p0, true);
#pragma unroll
    for (int j = 0; j < PB; ++j) {
      if (p0 + j >= nparts) break;
      const float wgt = __builtin_amdgcn_exp2f(mp[j] - M);
      den = fmaf(wgt, lp[j], den);
#pragma unroll
      for (int dd = 0; dd < DPL; ++dd) acc[dd] = fmaf(wgt, op[j][dd], acc[dd]);
    }
  }
#pragma unroll
  for (int dd = 0; dd < DPL; ++dd) store_out<OutCode>(out, row * D + lane * DPL + dd, acc[dd] / den);
}

// ---- verify attention: several new query tokens per sequence ---------------
// Checking drafted tokens ("speculative decoding": a small model drafts k
// tokens, the large one checks them in one pass) appends k + 1 tokens to a
// sequence and attends each of them causally to the cached keys and the new
// keys before it — a prefill chunk with a tiny q_len.  Its bytes are those of
// a decode step (the whole context once per KV head), its contraction
// (q_len G) rows deep: the same MFMA partition routine as the shared decode
// runs, with the sequence's new tokens as the members and a causal limit per
// row.  Grid (KV head, sequence, partition), partitions last to first; a
// workgroup serves the query tokens in groups of 32 / G (32 rows), each group
// reading the partition's K/V (the second from L2).  Rows whose keys span
// several partitions leave partial states merged by decode_reduce_kernel,
// which learns each token's own partition count from tok_parts.
template <typename KV, typename QT, int D, int G, int OutCode>
__global__ void __launch_bounds__(kThreads, 2)
verify_partition_kernel(void* __restrict__ out, float* __restrict__ ws_o, float* __restrict__ ws_ml,
                        int32_t* __restrict__ tok_parts, const typename QT::bits* __restrict__ q,
                        const unsigned char* __restrict__ kpool, const unsigned char* __restrict__ vpool,
                        const int32_t* __restrict__ tables, int max_blocks, const int32_t* __restrict__ cu_q,
                        const int32_t* __restrict__ lens, int total_q, int max_q_len, int Hkv, int64_t num_blocks,
                        int max_context_len, float scale_log2, float v_mul, int max_parts) {
  constexpr int TPG = kRunRows / G;  // query tokens per 32-row group
  __shared__ __attribute__((aligned(16))) RunLds<D, kRunRows> sh;
  const int g = blockIdx.x, s = blockIdx.y, p = gridDim.z - 1 - blockIdx.z;
  int q0 = cu_q[s], q1 = cu_q[s + 1];
  q0 = q0 < 0 ? 0 : (q0 > total_q ? total_q : q0);
  q1 = q1 < q0 ? q0 : (q1 > total_q ? total_q : q1);
  const int L = clamp_len(lens[s], max_context_len);
  int ql = q1 - q0;
  ql = ql > max_q_len ? max_q_len : ql;
  ql = ql > L ? L : ql;
  const int pos_first = L - ql;  // absolute position of the first new token
  if (tok_parts && g == 0 && p == 0 && (int)threadIdx.x < ql)
    tok_parts[q0 + threadIdx.x] = (pos_first + (int)threadIdx.x + kPart) / kPart;
  const int nparts = (L + kPart - 1) / kPart;
  if (ql == 0 || p >= nparts) return;
  const int t0 = p * kPart;
  const int n = (L - t0) < kPart ? (L - t0) : kPart;
  for (int tg = 0; tg * TPG < ql; ++tg) {
    const int k = ql - tg * TPG < TPG ? ql - tg * TPG : TPG;
    const int pos0 = pos_first + tg * TPG;
    if (pos0 + k - 1 < t0) continue;  // no token of the group reaches this partition (uniform)
    mfma_partition<KV, QT, D, G, kRunRows / 16, true, OutCode, PKV_VERIFY_PARTS, kWaves>(
        TokenRows{s, q0 + tg * TPG, k, pos0}, n, g, p, sh, out, ws_o, ws_ml, q, kpool, vpool, tables, max_blocks, Hkv,
        num_blocks, scale_log2, v_mul, max_parts);
  }
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
  float v_mul;  // 8-bit cache: the V pool's scale
  int max_parts;
  hipStream_t stream;
  AppendArgs app;  // this step's cache write, done by the shared-run launch (16-bit pools)
  // verify attention
  const int32_t* cu_q = nullptr;
  int total_q = 0, max_q_len = 0;
  int32_t* tok_parts = nullptr;
};

template <typename KV, typename QT, int D, int G, int OutCode>
void launch_shared(const DecodeArgs& a) {
  constexpr int KM = kRunRows / G;
  const int64_t windows = (a.B + KM - 1) / KM;
  // z layers of cache-write workgroups: one thread per 16-byte pool chunk of
  // the new rows (grid-stride beyond 64 layers)
  int64_t nz = 0;
  if (a.app.T > 0) {
    const int64_t items = a.app.T * a.Hkv * (D * KV::kBytes / 16);
    const int64_t per_layer = (int64_t)a.Hkv * windows * kSharedWaves * 64;
    nz = (items + per_layer - 1) / per_layer;
    nz = nz > 64 ? 64 : nz;
  }
  hipLaunchKernelGGL((decode_shared_kernel<KV, QT, D, G, OutCode>),
                     dim3((unsigned)a.Hkv, (unsigned)windows, (unsigned)(kRunSlots + nz)),
                     dim3(kSharedWaves * 64),
                     0, a.stream, a.out, a.ws_o, a.ws_ml, (const typename QT::bits*)a.q, a.kpool, a.vpool,
                     a.tables, a.max_blocks, a.lens, a.B, a.Hkv, a.num_blocks, a.max_context_len, a.scale_log2,
                     a.v_mul, a.max_parts, a.app);
}

template <int D, int OutCode>
void launch_reduce(const DecodeArgs& a, int G) {
  (void)G;
  if (a.max_parts > 1)
    hipLaunchKernelGGL((decode_reduce_kernel<D, OutCode, false>), dim3((unsigned)a.Hq, (unsigned)a.B), dim3(64),
                       0, a.stream, a.out, a.ws_o, a.ws_ml, a.lens, (const int32_t*)nullptr, a.Hq,
                       a.max_context_len, a.max_parts);
}

template <typename KV, typename QT, int D, int G, int OutCode>
void launch_whole(const DecodeArgs& a) {
  const dim3 grid((unsigned)a.Hkv, (unsigned)a.B), block(kWholeWaves * 64);
  const auto* q = (const typename QT::bits*)a.q;
  if constexpr (KV::kBytes != 4) {
    if (a.max_context_len > kWholeSpan) {
      hipLaunchKernelGGL((decode_whole_kernel<KV, QT, D, G, OutCode, kWholeSpanM>), grid, block, 0, a.stream, a.out,
                         q, a.kpool, a.vpool, a.tables, a.max_blocks, a.lens, a.Hkv, a.num_blocks, a.max_context_len,
                         a.scale_log2, a.v_mul, a.app);
      return;
    }
  }
  if constexpr (KV::kBytes != 4 || G * D * KV::kBytes <= 1024)
    hipLaunchKernelGGL((decode_whole_kernel<KV, QT, D, G, OutCode, kWholeSpan>), grid, block, 0, a.stream, a.out, q,
                       a.kpool, a.vpool, a.tables, a.max_blocks, a.lens, a.Hkv, a.num_blocks, a.max_context_len,
                       a.scale_log2, a.v_mul, a.app);
}

template <typename T, int D, int G, int OutCode>
void launch_decode(const DecodeArgs& a, bool partitions, bool reduce) {
  // the one-call form (partitions and merge together) of a short, small batch
  if (partitions && reduce && whole_context(a.B, a.Hkv, G, D, T::kBytes, a.max_context_len)) {
    launch_whole<T, T, D, G, OutCode>(a);
    return;
  }
  if (partitions && T::kBytes == 2) launch_shared<T, T, D, G, OutCode>(a);
  if (partitions)
    hipLaunchKernelGGL((decode_partition_kernel<T, D, G, OutCode>),
                       dim3((unsigned)a.Hkv, (unsigned)a.B, (unsigned)a.max_parts), dim3(kThreads), 0,
                       a.stream, a.out, a.ws_o, a.ws_ml, (const typename T::bits*)a.q, a.kpool, a.vpool,
                       a.tables, a.max_blocks, a.lens, a.Hkv, a.num_blocks, a.max_context_len,
                       a.scale_log2, a.max_parts);
  if (reduce) launch_reduce<D, OutCode>(a, G);
}

// 8-bit cache: shared runs, then the per-sequence MFMA partitions, then the
// reduction (a short, small batch: the whole-context launch instead).
template <typename QT, int D, int G, int OutCode>
void launch_decode_fp8(const DecodeArgs& a, bool partitions, bool reduce) {
  if (partitions && reduce && whole_context(a.B, a.Hkv, G, D, FP8::kBytes, a.max_context_len)) {
    launch_whole<FP8, QT, D, G, OutCode>(a);
    return;
  }
  if (partitions) {
    launch_shared<FP8, QT, D, G, OutCode>(a);
    hipLaunchKernelGGL((decode_fp8_partition_kernel<QT, D, G, OutCode>),
                       dim3((unsigned)a.Hkv, (unsigned)a.B, (unsigned)a.max_parts), dim3(kThreads), 0, a.stream,
                       a.out, a.ws_o, a.ws_ml, (const typename QT::bits*)a.q, a.kpool, a.vpool, a.tables,
                       a.max_blocks, a.lens, a.Hkv, a.num_blocks, a.max_context_len, a.scale_log2, a.v_mul,
                       a.max_parts);
  }
  if (reduce) launch_reduce<D, OutCode>(a, G);
}

// verify attention: the partition pass, then the per-token merge
template <typename KV, typename QT, int D, int G, int OutCode>
void launch_verify(const DecodeArgs& a) {
  hipLaunchKernelGGL((verify_partition_kernel<KV, QT, D, G, OutCode>),
                     dim3((unsigned)a.Hkv, (unsigned)a.B, (unsigned)a.max_parts), dim3(kThreads), 0, a.stream, a.out,
                     a.ws_o, a.ws_ml, a.tok_parts, (const typename QT::bits*)a.q, a.kpool, a.vpool, a.tables,
                     a.max_blocks, a.cu_q, a.lens, a.total_q, a.max_q_len, a.Hkv, a.num_blocks, a.max_context_len,
                     a.scale_log2, a.v_mul, a.max_parts);
  if (a.max_parts > 1)
    hipLaunchKernelGGL((decode_reduce_kernel<D, OutCode, true>), dim3((unsigned)a.Hq, (unsigned)a.total_q),
                       dim3(64), 0, a.stream, a.out, a.ws_o, a.ws_ml, a.lens, a.tok_parts, a.Hq, a.max_context_len,
                       a.max_parts);
}

// Launcher<T, D, G, OutCode>::run(args, partitions, reduce)
template <typename T, int D, int G, int OutCode>
struct Plain {
  static void run(const DecodeArgs& a, bool pa, bool re) { launch_decode<T, D, G, OutCode>(a, pa, re); }
};
template <typename QT, int D, int G, int OutCode>
struct Fp8 {
  static void run(const DecodeArgs& a, bool pa, bool re) { launch_decode_fp8<QT, D, G, OutCode>(a, pa, re); }
};

template <typename T, int D, int G, int OutCode>
struct Verify {
  static void run(const DecodeArgs& a, bool, bool) { launch_verify<T, T, D, G, OutCode>(a); }
};
template <typename QT, int D, int G, int OutCode>
struct VerifyFp8 {
  static void run(const DecodeArgs& a, bool, bool) { launch_verify<FP8, QT, D, G, OutCode>(a); }
};

template <template <typename, int, int, int> class Launcher, typename T, int D, int OutCode>
int dispatch_g(const DecodeArgs& a, int G, bool pa, bool re) {
  switch (G) {
    case 1: Launcher<T, D, 1, OutCode>::run(a, pa, re); return 0;
    case 2: Launcher<T, D, 2, OutCode>::run(a, pa, re); return 0;
    case 4: Launcher<T, D, 4, OutCode>::run(a, pa, re); return 0;
    case 8: Launcher<T, D, 8, OutCode>::run(a, pa, re); return 0;
    case 16: Launcher<T, D, 16, OutCode>::run(a, pa, re); return 0;
    default: return -1;
  }
}

template <template <typename, int, int, int> class Launcher, typename T, int OutCode>
int dispatch_d(const DecodeArgs& a, int D, int G, bool pa, bool re) {
  if (D == 64) return dispatch_g<Launcher, T, 64, OutCode>(a, G, pa, re);
  if (D == 128) return dispatch_g<Launcher, T, 128, OutCode>(a, G, pa, re);
  return -1;
}

}  // namespace
}  // namespace pkv

using pkv::fail;
using pkv::ok;

extern "C" int32_t paged_attention_decode_partition_size(void) { return pkv::kPart; }

extern "C" int32_t paged_attention_decode_whole_context(int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                                        int32_t head_dim, int32_t kv_dtype, int32_t max_context_len) {
  const int es = pkv::esize_of(kv_dtype);
  if (num_seqs <= 0 || n_kv_heads <= 0 || n_q_heads <= 0 || n_q_heads % n_kv_heads || max_context_len < 0 || !es)
    return 0;
  return pkv::whole_context(num_seqs, n_kv_heads, n_q_heads / n_kv_heads, head_dim, es, max_context_len) ? 1 : 0;
}

extern "C" int64_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t n_q_heads,
                                                          int32_t head_dim, int32_t max_context_len) {
  if (num_seqs <= 0 || n_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const int64_t parts = (max_context_len + pkv::kPart - 1) / pkv::kPart;
  if (parts <= 1) return 0;
  return (int64_t)num_seqs * n_q_heads * parts * (head_dim + 2) * (int64_t)sizeof(float);
}

// Validation and dispatch shared by the 16-bit/fp32 entry points (fp8 =
// false: q in the KV dtype, unit scales) and the 8-bit one.
static int decode_impl(const char* fn, bool pa, bool re, bool fp8, void* out, int32_t out_dtype, const void* q,
                       int32_t q_dtype, const void* k_pool, const void* v_pool, float k_scale, float v_scale,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                       int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                       int32_t block_size, int64_t num_blocks, int32_t max_context_len, float scale,
                       int32_t kv_dtype, void* workspace, int64_t workspace_bytes, void* stream,
                       const pkv::AppendArgs* app = nullptr) {
  const std::string F(fn);
  if (!pkv::esize_of(kv_dtype)) return fail(PKV_EINVAL, F + ": unknown kv dtype");
  if (fp8 != (kv_dtype == PKV_FP8_E4M3))
    return fail(PKV_EINVAL, fp8 ? F + ": pools must hold E4M3 codes"
                                : F + ": 8-bit pools are read by paged_attention_decode_fp8");
  if (fp8 && q_dtype != PKV_F16 && q_dtype != PKV_BF16)
    return fail(PKV_EINVAL, F + ": q dtype must be f16 or bf16");
  if (out_dtype != PKV_F32 && out_dtype != q_dtype)
    return fail(PKV_EINVAL, F + ": out dtype must be f32 or the query's dtype");
  if (fp8 && (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f)))
    return fail(PKV_EINVAL, F + ": k_scale and v_scale must be finite and > 0");
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size must be 16");
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (num_seqs < 0 || num_seqs > 65535 || n_kv_heads < 1 || n_q_heads < 1 || n_kv_heads > 65535 ||
      (int64_t)max_context_len > 65535ll * pkv::kPart)
    return fail(PKV_EINVAL, F + ": bad num_seqs or head counts");
  if (n_q_heads % n_kv_heads) return fail(PKV_EINVAL, "n_q_heads must be a multiple of n_kv_heads");
  const int G = n_q_heads / n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PKV_EUNSUPPORTED, "n_q_heads / n_kv_heads must be 1, 2, 4, 8 or 16");
  if (num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_EINVAL, F + ": max_context_len exceeds the table width");
  if (num_seqs == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return fail(PKV_EINVAL, F + ": NULL pointer");
  if (!pkv::aligned16(q) || !pkv::aligned16(k_pool) || !pkv::aligned16(v_pool) || !pkv::aligned16(out))
    return fail(PKV_EINVAL, F + ": q, out and pools must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, F + ": scale not finite");
  const int max_parts = max_context_len > 0 ? (max_context_len + pkv::kPart - 1) / pkv::kPart : 1;
  const int64_t need = paged_attention_decode_workspace_bytes(num_seqs, n_q_heads, head_dim, max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need || !pkv::aligned16(workspace)))
    return fail(PKV_EINVAL, F + ": workspace missing or too small (need " +
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
  // scores in base 2; an 8-bit key pool's scale folds into the softmax scale
  a.scale_log2 = (float)((double)scale * (double)k_scale * 1.4426950408889634);
  if (!std::isfinite(a.scale_log2)) return fail(PKV_EINVAL, F + ": scale * k_scale overflows");
  a.v_mul = v_scale;
  a.max_parts = max_parts;
  a.stream = (hipStream_t)stream;
  if (app) a.app = *app;
  using pkv::dispatch_d;
  using pkv::Fp8;
  using pkv::Plain;
  auto dispatch = [&](bool do_pa, bool do_re) -> int {
    switch (kv_dtype) {
      case PKV_F32: return dispatch_d<Plain, pkv::F32, PKV_F32>(a, head_dim, G, do_pa, do_re);
      case PKV_F16:
        return out_dtype == PKV_F32 ? dispatch_d<Plain, pkv::F16, PKV_F32>(a, head_dim, G, do_pa, do_re)
                                    : dispatch_d<Plain, pkv::F16, PKV_F16>(a, head_dim, G, do_pa, do_re);
      case PKV_BF16:
        return out_dtype == PKV_F32 ? dispatch_d<Plain, pkv::BF16, PKV_F32>(a, head_dim, G, do_pa, do_re)
                                    : dispatch_d<Plain, pkv::BF16, PKV_BF16>(a, head_dim, G, do_pa, do_re);
      case PKV_FP8_E4M3:
        if (q_dtype == PKV_BF16)
          return out_dtype == PKV_F32 ? dispatch_d<Fp8, pkv::BF16, PKV_F32>(a, head_dim, G, do_pa, do_re)
                                      : dispatch_d<Fp8, pkv::BF16, PKV_BF16>(a, head_dim, G, do_pa, do_re);
        return out_dtype == PKV_F32 ? dispatch_d<Fp8, pkv::F16, PKV_F32>(a, head_dim, G, do_pa, do_re)
                                    : dispatch_d<Fp8, pkv::F16, PKV_F16>(a, head_dim, G, do_pa, do_re);
    }
    return -1;
  };
  const int rc = dispatch(pa, re);
  if (rc) return fail(PKV_EUNSUPPORTED, F + ": configuration not built");
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, std::string(F + ": ") + hipGetErrorString(e));
  return ok();
}

#define PKV_DECODE_PARAMS                                                                          \
  void *out, int32_t out_dtype, const void *q, const void *k_pool, const void *v_pool,             \
      const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,        \
      int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,                   \
      int32_t block_size, int64_t num_blocks, int32_t max_context_len, float scale,                \
      int32_t kv_dtype, void *workspace, int64_t workspace_bytes, void *stream
#define PKV_DECODE_ARGS                                                                            \
  out, out_dtype, q, kv_dtype, k_pool, v_pool, 1.0f, 1.0f, block_tables, max_blocks_per_seq,       \
      context_lens, num_seqs, n_q_heads, n_kv_heads, head_dim, block_size, num_blocks,             \
      max_context_len, scale, kv_dtype, workspace, workspace_bytes, stream

// Fused cache write + decode: the new rows go in with the shared-run launch
// (16-bit pools) or a cache-write launch first (fp32 pools).
extern "C" int paged_attention_decode_append(void* out, int32_t out_dtype, const void* q, const void* k_new,
                                             const void* v_new, int64_t k_new_stride, int64_t v_new_stride,
                                             const int64_t* slot_mapping, void* k_pool, void* v_pool,
                                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                                             const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads,
                                             int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                             int64_t num_blocks, int32_t max_context_len, float scale,
                                             int32_t kv_dtype, void* workspace, int64_t workspace_bytes,
                                             void* stream) {
  const std::string F("paged_attention_decode_append");
  if (kv_dtype == PKV_FP8_E4M3)
    return fail(PKV_EINVAL, F + ": 8-bit pools take reshape_and_cache_fp8, then paged_attention_decode_fp8");
  const int es = pkv::esize_of(kv_dtype);
  if (!es) return fail(PKV_EINVAL, F + ": unknown kv dtype");
  if (num_seqs > 0) {
    if (!k_new || !v_new || !slot_mapping) return fail(PKV_EINVAL, F + ": NULL new rows or slot mapping");
    const int64_t row = (int64_t)n_kv_heads * head_dim;
    if (n_kv_heads < 1 || k_new_stride < row || v_new_stride < row)
      return fail(PKV_EINVAL, F + ": token stride shorter than a row");
    if (!pkv::aligned16(k_new) || !pkv::aligned16(v_new) || (k_new_stride * es) % 16 || (v_new_stride * es) % 16)
      return fail(PKV_EINVAL, F + ": new rows and their strides must be 16-byte aligned");
  }
  if (kv_dtype == PKV_F32) {  // no shared-run launch: the cache write goes first
    // the attention's arguments are checked before anything is launched
    const int vr = decode_impl(F.c_str(), false, false, false, out, out_dtype, q, kv_dtype, k_pool, v_pool, 1.0f,
                               1.0f, block_tables, max_blocks_per_seq, context_lens, num_seqs, n_q_heads,
                               n_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale, kv_dtype,
                               workspace, workspace_bytes, stream);
    if (vr != PKV_OK) return vr;
    if (num_seqs > 0) {
      const int rc = reshape_and_cache(k_new, v_new, k_new_stride, v_new_stride, k_pool, v_pool, slot_mapping,
                                       num_seqs, num_blocks, n_kv_heads, head_dim, block_size, kv_dtype, stream);
      if (rc != PKV_OK) return rc;
    }
    return decode_impl(F.c_str(), true, true, false, out, out_dtype, q, kv_dtype, k_pool, v_pool, 1.0f, 1.0f,
                       block_tables, max_blocks_per_seq, context_lens, num_seqs, n_q_heads, n_kv_heads, head_dim,
                       block_size, num_blocks, max_context_len, scale, kv_dtype, workspace, workspace_bytes,
                       stream);
  }
  pkv::AppendArgs app;
  app.key = (const unsigned char*)k_new;
  app.value = (const unsigned char*)v_new;
  app.kstride_b = k_new_stride * es;
  app.vstride_b = v_new_stride * es;
  app.kpool = (unsigned char*)k_pool;
  app.vpool = (unsigned char*)v_pool;
  app.slots = slot_mapping;
  app.T = num_seqs;
  app.num_slots = num_blocks * (int64_t)pkv::kBlockSize;
  return decode_impl(F.c_str(), true, true, false, out, out_dtype, q, kv_dtype, k_pool, v_pool, 1.0f, 1.0f,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, n_q_heads, n_kv_heads, head_dim,
                     block_size, num_blocks, max_context_len, scale, kv_dtype, workspace, workspace_bytes, stream,
                     &app);
}

// ---- the decode step for callers that cannot allocate ----------------------
// paged_attention_decode_append with its workspace (the split-context
// partials) in device memory the library itself holds: a file-scope array,
// one copy per GPU, present from the moment the library's code is loaded on
// that GPU until the process ends.  Host code never names the array in a
// kernel argument or copy: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and that address is used.
// Nothing in it must start at zero: every partial a merge reads is written by
// the same call's partition pass first.
namespace {
constexpr int64_t kNoAllocScratchBytes = 64ll << 20;
constexpr int kMaxDevices = 64;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Device address of this GPU's scratch, looked up on the first call per
// device (the current device: the one the caller's stream belongs to).
static int scratch_for_current_device(const std::string& F, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_EHIP, F + ": hipGetDevice: " + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_EUNSUPPORTED, F + ": device index beyond 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_EHIP, F + ": hipGetSymbolAddress(scratch): " + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ok();
}

extern "C" int64_t paged_attention_decode_noalloc_max_workspace_bytes(void) { return kNoAllocScratchBytes; }

extern "C" int paged_attention_decode_append_noalloc(void* out, int32_t out_dtype, const void* q, const void* k_new,
                                                     const void* v_new, int64_t k_new_stride, int64_t v_new_stride,
                                                     const int64_t* slot_mapping, void* k_pool, void* v_pool,
                                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                     const int32_t* context_lens, int32_t num_seqs,
                                                     int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                                     int32_t block_size, int64_t num_blocks,
                                                     int32_t max_context_len, float scale, int32_t kv_dtype,
                                                     void* stream) {
  const std::string F("paged_attention_decode_append_noalloc");
  const int64_t need = paged_attention_decode_workspace_bytes(num_seqs, n_q_heads, head_dim, max_context_len);
  if (need > kNoAllocScratchBytes)
    return fail(PKV_EINVAL, F + ": the split-context partials need " + std::to_string(need) +
                                " bytes, more than the library's " + std::to_string(kNoAllocScratchBytes) +
                                "-byte scratch (use paged_attention_decode_append with a workspace)");
  void* ws = nullptr;
  if (need > 0) {
    const int rc = scratch_for_current_device(F, &ws);
    if (rc != PKV_OK) return rc;
  }
  return paged_attention_decode_append(out, out_dtype, q, k_new, v_new, k_new_stride, v_new_stride, slot_mapping,
                                       k_pool, v_pool, block_tables, max_blocks_per_seq, context_lens, num_seqs,
                                       n_q_heads, n_kv_heads, head_dim, block_size, num_blocks, max_context_len,
                                       scale, kv_dtype, ws, need > 0 ? kNoAllocScratchBytes : 0, stream);
}

extern "C" int paged_attention_decode(PKV_DECODE_PARAMS) {
  return decode_impl("paged_attention_decode", true, true, false, PKV_DECODE_ARGS);
}
extern "C" int paged_attention_decode_partitions(PKV_DECODE_PARAMS) {
  return decode_impl("paged_attention_decode_partitions", true, false, false, PKV_DECODE_ARGS);
}
extern "C" int paged_attention_decode_reduce(PKV_DECODE_PARAMS) {
  return decode_impl("paged_attention_decode_reduce", false, true, false, PKV_DECODE_ARGS);
}
#define PKV_DECODE_FP8_PARAMS                                                                      \
  void *out, int32_t out_dtype, const void *q, int32_t q_dtype, const void *k_pool,                \
      const void *v_pool, float k_scale, float v_scale, const int32_t *block_tables,               \
      int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_seqs, int32_t n_q_heads, \
      int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,                \
      int32_t max_context_len, float scale, void *workspace, int64_t workspace_bytes, void *stream
#define PKV_DECODE_FP8_ARGS                                                                        \
  out, out_dtype, q, q_dtype, k_pool, v_pool, k_scale, v_scale, block_tables, max_blocks_per_seq,  \
      context_lens, num_seqs, n_q_heads, n_kv_heads, head_dim, block_size, num_blocks,             \
      max_context_len, scale, PKV_FP8_E4M3, workspace, workspace_bytes, stream

extern "C" int paged_attention_decode_fp8(PKV_DECODE_FP8_PARAMS) {
  return decode_impl("paged_attention_decode_fp8", true, true, true, PKV_DECODE_FP8_ARGS);
}
// Fused quantising cache write + decode over 8-bit pools: the new rows (in
// the query's type) are quantised by the shared-run launch.
extern "C" int paged_attention_decode_fp8_append(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                                                 const void* k_new, const void* v_new, int64_t k_new_stride,
                                                 int64_t v_new_stride, const int64_t* slot_mapping, void* k_pool,
                                                 void* v_pool, float k_scale, float v_scale,
                                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                                 const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads,
                                                 int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                                 int64_t num_blocks, int32_t max_context_len, float scale,
                                                 void* workspace, int64_t workspace_bytes, void* stream) {
  const std::string F("paged_attention_decode_fp8_append");
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16) return fail(PKV_EINVAL, F + ": q dtype must be f16 or bf16");
  const int es = pkv::esize_of(q_dtype);
  pkv::AppendArgs app;
  if (num_seqs > 0) {
    if (!k_new || !v_new || !slot_mapping) return fail(PKV_EINVAL, F + ": NULL new rows or slot mapping");
    const int64_t row = (int64_t)n_kv_heads * head_dim;
    if (n_kv_heads < 1 || k_new_stride < row || v_new_stride < row)
      return fail(PKV_EINVAL, F + ": token stride shorter than a row");
    if (!pkv::aligned16(k_new) || !pkv::aligned16(v_new) || (k_new_stride * es) % 16 || (v_new_stride * es) % 16)
      return fail(PKV_EINVAL, F + ": new rows and their strides must be 16-byte aligned");
    if (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f))
      return fail(PKV_EINVAL, F + ": k_scale and v_scale must be finite and > 0");
    // the reciprocals are rounded to nearest once, here, as by reshape_and_cache_fp8
    app.k_inv = 1.0f / k_scale;
    app.v_inv = 1.0f / v_scale;
    if (!std::isfinite(app.k_inv) || !std::isfinite(app.v_inv)) return fail(PKV_EINVAL, F + ": scale too small");
  }
  app.key = (const unsigned char*)k_new;
  app.value = (const unsigned char*)v_new;
  app.kstride_b = k_new_stride * es;
  app.vstride_b = v_new_stride * es;
  app.kpool = (unsigned char*)k_pool;
  app.vpool = (unsigned char*)v_pool;
  app.slots = slot_mapping;
  app.T = num_seqs;
  app.num_slots = num_blocks * (int64_t)pkv::kBlockSize;
  return decode_impl(F.c_str(), true, true, true, out, out_dtype, q, q_dtype, k_pool, v_pool, k_scale, v_scale,
                     block_tables, max_blocks_per_seq, context_lens, num_seqs, n_q_heads, n_kv_heads, head_dim,
                     block_size, num_blocks, max_context_len, scale, PKV_FP8_E4M3, workspace, workspace_bytes,
                     stream, &app);
}

extern "C" int paged_attention_decode_fp8_partitions(PKV_DECODE_FP8_PARAMS) {
  return decode_impl("paged_attention_decode_fp8_partitions", true, false, true, PKV_DECODE_FP8_ARGS);
}
extern "C" int paged_attention_decode_fp8_reduce(PKV_DECODE_FP8_PARAMS) {
  return decode_impl("paged_attention_decode_fp8_reduce", false, true, true, PKV_DECODE_FP8_ARGS);
}

// ---- verify attention entry points ------------------------------------------
extern "C" int64_t paged_attention_verify_workspace_bytes(int32_t total_q, int32_t n_q_heads, int32_t head_dim,
                                                          int32_t max_context_len) {
  if (total_q <= 0 || n_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0) return 0;
  const int64_t parts = (max_context_len + pkv::kPart - 1) / pkv::kPart;
  if (parts <= 1) return 0;
  return (int64_t)total_q * n_q_heads * parts * (head_dim + 2) * (int64_t)sizeof(float) + (int64_t)total_q * 4;
}

static int verify_impl(const char* fn, bool fp8, void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                       const void* k_pool, const void* v_pool, float k_scale, float v_scale,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                       const int32_t* context_lens, int32_t n_seqs, int32_t total_q, int32_t max_q_len,
                       int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                       int64_t num_blocks, int32_t max_context_len, float scale, int32_t kv_dtype, void* workspace,
                       int64_t workspace_bytes, void* stream) {
  const std::string F(fn);
  if (!fp8 && kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(kv_dtype == PKV_F32 ? PKV_EUNSUPPORTED : PKV_EINVAL,
                F + (kv_dtype == PKV_FP8_E4M3 ? ": 8-bit pools are read by paged_attention_verify_fp8"
                                              : ": kv dtype must be f16 or bf16"));
  if (q_dtype != PKV_F16 && q_dtype != PKV_BF16) return fail(PKV_EINVAL, F + ": q dtype must be f16 or bf16");
  if (out_dtype != PKV_F32 && out_dtype != q_dtype)
    return fail(PKV_EINVAL, F + ": out dtype must be f32 or the query's dtype");
  if (fp8 && (!std::isfinite(k_scale) || !std::isfinite(v_scale) || !(k_scale > 0.f) || !(v_scale > 0.f)))
    return fail(PKV_EINVAL, F + ": k_scale and v_scale must be finite and > 0");
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size must be 16");
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (n_kv_heads < 1 || n_q_heads < 1 || n_kv_heads > 65535 || n_q_heads % n_kv_heads)
    return fail(PKV_EINVAL, F + ": n_q_heads must be a positive multiple of n_kv_heads");
  const int G = n_q_heads / n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PKV_EUNSUPPORTED, F + ": n_q_heads / n_kv_heads must be 1, 2, 4, 8 or 16");
  if (n_seqs < 0 || n_seqs > 65535 || total_q < 0 || total_q > 65535 || max_q_len < 0)
    return fail(PKV_EINVAL, F + ": bad n_seqs, total_q or max_q_len");
  if (max_q_len > 64)
    return fail(PKV_EUNSUPPORTED, F + ": more than 64 query tokens per sequence (use paged_attention_prefill_chunk)");
  if (num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size ||
      (int64_t)max_context_len > 65535ll * pkv::kPart)
    return fail(PKV_EINVAL, F + ": max_context_len exceeds the table width");
  if (n_seqs == 0 || total_q == 0 || max_q_len == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !cu_q_lens || !context_lens)
    return fail(PKV_EINVAL, F + ": NULL pointer");
  if (!pkv::aligned16(q) || !pkv::aligned16(k_pool) || !pkv::aligned16(v_pool) || !pkv::aligned16(out))
    return fail(PKV_EINVAL, F + ": q, out and pools must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, F + ": scale not finite");
  const int max_parts = max_context_len > 0 ? (max_context_len + pkv::kPart - 1) / pkv::kPart : 1;
  const int64_t need = paged_attention_verify_workspace_bytes(total_q, n_q_heads, head_dim, max_context_len);
  if (need > 0 && (!workspace || workspace_bytes < need || !pkv::aligned16(workspace)))
    return fail(PKV_EINVAL, F + ": workspace missing or too small (need " + std::to_string(need) + " bytes)");
  pkv::DecodeArgs a;
  a.out = out;
  const int64_t rows = (int64_t)total_q * n_q_heads;
  a.ws_o = (float*)workspace;
  a.ws_ml = need > 0 ? a.ws_o + rows * max_parts * head_dim : nullptr;
  a.tok_parts = need > 0 ? (int32_t*)(a.ws_ml + rows * max_parts * 2) : nullptr;
  a.q = q;
  a.kpool = (const unsigned char*)k_pool;
  a.vpool = (const unsigned char*)v_pool;
  a.tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.lens = context_lens;
  a.B = n_seqs;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.scale_log2 = (float)((double)scale * (double)k_scale * 1.4426950408889634);
  if (!std::isfinite(a.scale_log2)) return fail(PKV_EINVAL, F + ": scale * k_scale overflows");
  a.v_mul = v_scale;
  a.max_parts = max_parts;
  a.stream = (hipStream_t)stream;
  a.cu_q = cu_q_lens;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  using pkv::dispatch_d;
  using pkv::Verify;
  using pkv::VerifyFp8;
  int rc;
  const bool f32o = out_dtype == PKV_F32;
  if (fp8) {
    if (q_dtype == PKV_BF16)
      rc = f32o ? dispatch_d<VerifyFp8, pkv::BF16, PKV_F32>(a, head_dim, G, true, true)
                : dispatch_d<VerifyFp8, pkv::BF16, PKV_BF16>(a, head_dim, G, true, true);
    else
      rc = f32o ? dispatch_d<VerifyFp8, pkv::F16, PKV_F32>(a, head_dim, G, true, true)
                : dispatch_d<VerifyFp8, pkv::F16, PKV_F16>(a, head_dim, G, true, true);
  } else if (kv_dtype == PKV_BF16) {
    rc = f32o ? dispatch_d<Verify, pkv::BF16, PKV_F32>(a, head_dim, G, true, true)
              : dispatch_d<Verify, pkv::BF16, PKV_BF16>(a, head_dim, G, true, true);
  } else {
    rc = f32o ? dispatch_d<Verify, pkv::F16, PKV_F32>(a, head_dim, G, true, true)
              : dispatch_d<Verify, pkv::F16, PKV_F16>(a, head_dim, G, true, true);
  }
  if (rc) return fail(PKV_EUNSUPPORTED, F + ": configuration not built");
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, F + ": " + hipGetErrorString(e));
  return ok();
}

extern "C" int paged_attention_verify(void* out, int32_t out_dtype, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* cu_q_lens, const int32_t* context_lens, int32_t n_seqs,
                                      int32_t total_q, int32_t max_q_len, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                      int32_t max_context_len, float scale, int32_t kv_dtype, void* workspace,
                                      int64_t workspace_bytes, void* stream) {
  return verify_impl("paged_attention_verify", false, out, out_dtype, q, kv_dtype, k_pool, v_pool, 1.f, 1.f,
                     block_tables, max_blocks_per_seq, cu_q_lens, context_lens, n_seqs, total_q, max_q_len, n_q_heads,
                     n_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale, kv_dtype, workspace,
                     workspace_bytes, stream);
}

extern "C" int paged_attention_verify_fp8(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                                          const void* k_pool, const void* v_pool, float k_scale, float v_scale,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* cu_q_lens, const int32_t* context_lens, int32_t n_seqs,
                                          int32_t total_q, int32_t max_q_len, int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                          int32_t max_context_len, float scale, void* workspace,
                                          int64_t workspace_bytes, void* stream) {
  return verify_impl("paged_attention_verify_fp8", true, out, out_dtype, q, q_dtype, k_pool, v_pool, k_scale,
                     v_scale, block_tables, max_blocks_per_seq, cu_q_lens, context_lens, n_seqs, total_q, max_q_len,
                     n_q_heads, n_kv_heads, head_dim, block_size, num_blocks, max_context_len, scale, PKV_FP8_E4M3,
                     workspace, workspace_bytes, stream);
}
