// Chunked-prefill attention over the paged KV cache, on MFMA (gfx950).
//
// What is computed: chunk c holds q_len query tokens of one sequence whose
// keys/values (the cached context plus the chunk itself, appended before the
// call) number L.  Query i sits at absolute position p = L - q_len + i and
// attends causally to keys 0..p:  out = softmax(scale * q K^T) V  row by row
// ("The detour, what really happens inside one forward pass", Life of a
// prompt, for the Q K^T -> softmax -> V contraction; "Chunked prefill" in The
// hands-on guide to LLM Inference with vLLM: each chunk's attention reads the
// KV cache of every chunk before it).  Keys and values are gathered block by
// block through the chunk's block table ("How the attention kernel actually
// reads paged blocks", vLLM Serving deep dive).
//
// How (gfx950, MFMA 16x16x32):
//  * Workgroup = 8 wave64s over (KV head, 64 query tokens, chunk) for a GQA
//    group of 4 query heads (more tokens when fewer heads share a KV head).
//    Each wave owns 2 row tiles of 16 query rows (token tile x head): the
//    heads of one KV head are stacked so every K/V tile staged in LDS serves
//    all of them.
//  * Keys advance 64 at a time (4 blocks).  The step's K and V tiles are
//    staged in LDS with direct global->LDS loads issued three steps ahead
//    (rings of four K and five V buffers, no registers); each thread rewrites
//    the V chunks it loaded as fp16, because the P.V product runs in fp16
//    (see below).
//  * Scores are formed transposed, S^T = K Q^T (A = K tile from LDS, B = the
//    wave's Q rows kept in registers), so each lane owns one query row: the
//    online softmax (base 2) needs one cross-lane max per row tile and step,
//    and the probabilities feed the next product from the lane's registers.
//    The running max only moves when a score exceeds it by more than 2^8, so
//    the output accumulators are rarely rescaled.
//  * O^T += V^T P^T with A = V^T (16 dims x 32 keys) and B = P^T.  The key
//    order inside each block pair is permuted identically in both operands
//    so that a lane's 8 contraction slots are 8 consecutive keys of one block:
//    each V^T operand is one 16-byte LDS read.  P is rounded to fp16
//    (u = 2^-11) rather than bf16 (u = 2^-8): the latter's error on short
//    causal rows comes close to the 2e-3 tolerance.  Row sums of P come from
//    an MFMA against ones.
//  * A step is two phases between workgroup barriers: the products (this
//    step's QK, then the previous step's PV) and the vector work (softmax,
//    staging); waves 4..7, which share SIMDs with waves 0..3, run one phase
//    behind, so in every phase each SIMD has one wave on the matrix cores and
//    one on the vector units.
//  * The causal mask is applied only on steps that reach the diagonal; keys
//    past the context are masked and their V entries zeroed when staged.
#include <math.h>

#include <cmath>
#include <string>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#ifndef PKV_PREFILL_WAVES
#define PKV_PREFILL_WAVES 8
#endif
constexpr int kPfWaves = PKV_PREFILL_WAVES;  // waves per workgroup (4: one per SIMD, 8: two)
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kStepKeys = 64;  // keys per step: 4 blocks of 16
constexpr float kSlack = 8.f;  // log2 headroom before the running max is moved

template <typename T>
__device__ __forceinline__ f32x4 mfma_qk(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (T::kCode == PKV_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_pv(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed fp16, round to nearest even (one v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2v_t));
}

// Two fp32 -> packed fp16, round toward zero: exact for values fp16 holds and
// saturating (to +-65504) for finite values beyond its range.
__device__ __forceinline__ uint32_t pack_f16x2_rtz(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// One 16-byte chunk of a V tile (8 consecutive keys of one dim) -> fp16 bits,
// keys at or past `valid` zeroed.
template <typename T>
__device__ __forceinline__ u32x4 v_chunk_to_f16(u32x4 v, int valid) {
  u32x4 r;
  if constexpr (T::kCode == PKV_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_f16x2_rtz(bf16lo(v[i]), bf16hi(v[i]));
  } else {
    r = v;
  }
  if (valid < 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = 2 * i < valid ? 0xffffu : 0u;
      const uint32_t hi = 2 * i + 1 < valid ? 0xffff0000u : 0u;
      r[i] &= lo | hi;
    }
  }
  return r;
}

// Max over lanes l, l^16, l^32, l^48 (the four lanes that hold one score row),
// with gfx950's cross-row lane swaps instead of a round trip through LDS.
__device__ __forceinline__ float row_max4(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Byte offset of an LDS location (its address in the LDS aperture).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane
// (lds_base wave-uniform).  Issued as inline asm so the compiler's wait-count
// pass does not see an LDS write in flight (it would then wait for every LDS
// read to drain before the first use of any); completion is tracked here with
// explicit vmcnt waits and workgroup barriers.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_base)
               : "memory", "m0");
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

template <typename T, int D, int GW, int OutCode>
__global__ void __launch_bounds__(kPfThreads, 1)
prefill_chunk_kernel(void* __restrict__ out, const uint16_t* __restrict__ q,
                     const unsigned char* __restrict__ kpool, const unsigned char* __restrict__ vpool,
                     const int32_t* __restrict__ tables, int max_blocks, const int32_t* __restrict__ cu_q,
                     const int32_t* __restrict__ lens, int total_q, int Hkv, int G, int64_t num_blocks,
                     int max_context_len, float scale_log2) {
  constexpr int RT = 16 / kPfWaves;        // row tiles (16 query rows each) per wave
  constexpr int HW = GW < RT ? GW : RT;    // heads per wave
  constexpr int TTW = RT / HW;             // 16-token tiles per wave
  constexpr int WPT = GW / HW;             // waves sharing a token tile (different heads)
  constexpr int TW = 16 * TTW;             // query tokens per wave
  constexpr int TWG = 16 * TTW * (kPfWaves / WPT);  // query tokens per workgroup
  constexpr int DC = D / 32;               // 32-dim slices of the score contraction
  constexpr int DT = D / 16;               // 16-dim tiles of the output
  constexpr int TILE = D * kBlockSize * 2; // bytes of one (block, head) tile
  constexpr int CPT = TILE / 16;           // 16-byte chunks per tile
  constexpr int NCH = 4 * CPT / kPfThreads;  // staging chunks per thread per step (K and V each)

  constexpr int kAhead = 3;           // steps whose loads are in flight while a step is consumed
  // K(t) is read one step before V(t), so V keeps one buffer more
  constexpr int NK = kAhead + 1, NV = kAhead + 2;
  __shared__ __attribute__((aligned(16))) unsigned char ldsK[NK][4 * TILE];
  __shared__ __attribute__((aligned(16))) unsigned char ldsV[NV][4 * TILE];
  auto kbuf = [&](int t) -> unsigned char* { return ldsK[t % NK]; };
  auto vbuf = [&](int t) -> unsigned char* { return ldsV[t % NV]; };
  static_assert(kPfWaves == 8, "the phase schedule pairs waves w and w + 4 on one SIMD");

  // Longest work first.  The causal work of a (chunk, query tile) unit grows
  // with the chunk's context length L, and the chunks of one call can differ
  // by two orders of magnitude; dispatched in index order, a long chunk that
  // comes late sets the kernel's length.  So grid slot z takes the chunk of
  // rank z in decreasing L (ties by index) and slot y the chunk's y-th tile
  // from the end.  Every workgroup ranks the chunks itself (each thread one
  // chunk, against a copy of all L in LDS), so nothing is precomputed; with
  // more chunks than threads the chunks keep their index order.
  __shared__ int rank_len[kPfThreads];
  __shared__ int rank_pick;
  int c = blockIdx.z;
  if (gridDim.z <= (unsigned)kPfThreads) {
    const int n = gridDim.z, t = threadIdx.x;
    if (t < n) {
      const int l = lens[t];
      rank_len[t] = l < 0 ? 0 : (l > max_context_len ? max_context_len : l);
    }
    __syncthreads();
    if (t < n) {
      const int mine = rank_len[t];
      int r = 0;
      for (int j = 0; j < n; ++j) {
        const int other = rank_len[j];
        r += (other > mine) | ((other == mine) & (j < t));
      }
      if (r == (int)blockIdx.z) rank_pick = t;
    }
    __syncthreads();
    c = rank_pick;
  }
  const int qs = cu_q[c];
  int qlen = cu_q[c + 1] - qs;
  int L = lens[c];
  L = L < 0 ? 0 : (L > max_context_len ? max_context_len : L);
  qlen = qlen < 0 ? 0 : (qlen > L ? L : qlen);
  const int ctx = L - qlen;
  const int tile_idx = (qlen + TWG - 1) / TWG - 1 - (int)blockIdx.y;
  if (tile_idx < 0) return;
  const int tile0 = tile_idx * TWG;

  const int hgroups = G / GW;
  const int g = blockIdx.x / hgroups;
  const int h0 = g * G + (blockIdx.x % hgroups) * GW;  // first query head of this workgroup
  const int Hq = Hkv * G;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, r16 = lane & 15;

  const int i0 = tile0 + (w / WPT) * TW;           // wave's first query token (chunk-local)
  const int hb = (w % WPT) * HW;                   // wave's first head within the workgroup
  const int wg_end = qlen < tile0 + TWG ? qlen : tile0 + TWG;
  const int nsteps = (ctx + wg_end + kStepKeys - 1) / kStepKeys;
  const bool active = i0 < qlen;
  const int wave_end = qlen < i0 + TW ? qlen : i0 + TW;
  const int kmax_w = ctx + wave_end;                // keys this wave needs: [0, kmax_w)
  const int32_t* tab = tables + (int64_t)c * max_blocks;
  const int nblk = (L + kBlockSize - 1) / kBlockSize;

  // ---- the wave's query rows as B operands of S^T = K Q^T -------------------
  u32x4 bq[RT][DC];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int tt = rt / HW, hh = hb + rt % HW;
    int tok = i0 + 16 * tt + r16;
    tok = tok < qlen ? tok : qlen - 1;
    int row = qs + tok;
    row = row < 0 ? 0 : (row >= total_q ? total_q - 1 : row);
    const uint16_t* qp = q + ((int64_t)row * Hq + h0 + hh) * D + 8 * q4;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) bq[rt][dc] = active ? ld16(qp + 32 * dc) : u32x4{0, 0, 0, 0};
  }

  // Key order inside the 32 keys of a block pair (2kh, 2kh+1) of a step.  Row
  // m = 4a + r of score tile kt = 2kh + sub holds the pair's key
  //   16 (a>>1) + 8 (a&1) + 4 (sub ^ (a>>1)) + r,
  // so (i) the 16 rows of one tile sit at 16 distinct token offsets, which
  // keeps the K reads free of LDS bank conflicts, and (ii) the lanes of group
  // a (q4 = a) own, across the pair's two tiles, the 8 consecutive keys
  // 8(a&1)..8(a&1)+7 of block 2kh + (a>>1): exactly one 16-byte chunk of a V
  // row, read whole as the V^T operand.  For odd blocks the two 4-key halves
  // arrive in the order (4..7, 0..3); the staging stores their V chunks that
  // way round.
  auto pair_key = [](int m, int sub) {
    const int a = m >> 2;
    return 16 * (a >> 1) + 8 * (a & 1) + 4 * (sub ^ (a >> 1)) + (m & 3);
  };
  int k_row_off[2], key_base[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int kr = pair_key(r16, sub);  // key whose K row this lane loads
    k_row_off[sub] = (kr >> 4) * TILE + ((kr & 15) + q4 * kBlockSize) * 16;
    key_base[sub] = pair_key(4 * q4, sub);  // key of score element r = 0 held by this lane
  }
  // V^T operand: dims 16dt + r16, the lane group's 8 keys.  A dim row is 32
  // bytes (16 keys); lane group q4 reads half q4 & 1 of the rows of block
  // q4 >> 1.  Unswizzled rows measure free of LDS bank conflicts for this
  // pattern on gfx950; swapping the halves of every other group of 8 rows
  // made these reads 2-way bank conflicted.
  const int v_off = (q4 >> 1) * TILE + r16 * 32 + (q4 & 1) * 16;
  const u32x4 ones = {0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u};  // fp16 1.0 x 8

  f32x4 o[RT][DT];
  f32x4 lsum[RT];  // element 0: running row sum of the fp16 probabilities (an MFMA against ones)
  float m[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m[rt] = -INFINITY;
    lsum[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- staging of one step's K/V tiles (4 blocks) --------------------------
  // Chunk ci = tid + kPfThreads k of a step: tile bi = ci / CPT (uniform per
  // wave), byte offset (ci % CPT) * 16 in it.  Direct global -> LDS loads (no
  // registers); a wave's 64 chunks land contiguously at a wave-uniform base.
  // Block ids of step t for this thread's chunks, -1 past the context; read
  // through the scalar unit a phase before they are used.
  // The table entry is read unconditionally (index clamped to the last
  // block) so nothing waits for it until issue_blocks uses it.
  auto load_blocks = [&](int t, int32_t (&blk)[NCH]) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int lb = 4 * t + __builtin_amdgcn_readfirstlane((tid + kPfThreads * k) / CPT);
      blk[k] = tab[lb < nblk ? lb : nblk - 1];
    }
  };
  auto issue_blocks = [&](int t, const int32_t (&blk)[NCH]) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int lb = 4 * t + __builtin_amdgcn_readfirstlane((tid + kPfThreads * k) / CPT);
      if (t < nsteps && lb < nblk) {
        const int off = ((tid + kPfThreads * k) % CPT) * 16;
        const int64_t base = (clamp_block(blk[k], num_blocks) * Hkv + g) * (int64_t)TILE + off;
        const int wbase = (kPfThreads * k + 64 * w) * 16;
        dma16(kpool + base, lds_offset(kbuf(t) + wbase));
        dma16(vpool + base, lds_offset(vbuf(t) + wbase));
      }
    }
  };
  // Number of loads issue_blocks issues for this thread at step t.
  auto n_loads = [&](int t) -> int {
    int n = 0;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int lb = 4 * t + __builtin_amdgcn_readfirstlane((tid + kPfThreads * k) / CPT);
      n += (t < nsteps && lb < nblk) ? 2 : 0;
    }
    return n;
  };
  // This thread's raw V chunks of a staged step (after its loads landed).
  auto read_raw = [&](int t, u32x4 (&raw)[NCH]) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) raw[k] = *reinterpret_cast<const u32x4*>(vbuf(t) + (tid + kPfThreads * k) * 16);
  };
  // Raw V chunks -> fp16, keys at or past the context zeroed (blocks past the
  // end become zeros), written back in place (each thread rewrites the 16
  // bytes it read); odd blocks with their 4-key halves swapped.
  auto finish_step = [&](int s, const u32x4 (&raw)[NCH]) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int ci = tid + kPfThreads * k;
      const int bi = __builtin_amdgcn_readfirstlane(ci / CPT), off = (ci % CPT) * 16;
      const int lb = 4 * s + bi;
      const int j = off / 32, hf = (off % 32) / 16;  // dim j, keys 8hf..8hf+7
      u32x4 v = lb < nblk ? v_chunk_to_f16<T>(raw[k], L - (lb * kBlockSize + 8 * hf)) : u32x4{0, 0, 0, 0};
      if (bi & 1) v = u32x4{v[2], v[3], v[0], v[1]};
      *reinterpret_cast<u32x4*>(vbuf(s) + bi * TILE + j * 32 + hf * 16) = v;
    }
  };
  // Wait until at most `keep` vector-memory operations of this wave are
  // outstanding (loads complete in issue order, so every earlier one is done).
  auto wait_vm = [](int keep) {
    // s_waitcnt immediate: vmcnt in bits 3:0, expcnt 6:4 and lgkmcnt 11:8 left at their maxima
    switch (keep) {
      case 0: __builtin_amdgcn_s_waitcnt(0xF70); break;
      case 1: __builtin_amdgcn_s_waitcnt(0xF71); break;
      case 2: __builtin_amdgcn_s_waitcnt(0xF72); break;
      case 3: __builtin_amdgcn_s_waitcnt(0xF73); break;
      case 4: __builtin_amdgcn_s_waitcnt(0xF74); break;
      case 5: __builtin_amdgcn_s_waitcnt(0xF75); break;
      case 6: __builtin_amdgcn_s_waitcnt(0xF76); break;
      case 7: __builtin_amdgcn_s_waitcnt(0xF77); break;
      default: __builtin_amdgcn_s_waitcnt(0xF78); break;
    }
  };
  static_assert(4 * NCH <= 8, "wait_vm covers at most 8 loads in flight per thread");
  // Workgroup barrier for LDS hand-off only: waits for this thread's LDS
  // writes (lgkmcnt) but, unlike __syncthreads(), not for the global->LDS
  // loads still in flight for later steps.
  // It also closes a phase: no instruction is scheduled across it.
  auto lds_barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- the three compute phases of a 64-key step ----------------------------
  f32x4 st[RT][4];  // S^T tiles: st[rt][kt] holds, for row r16, keys 32(kt/2) + key_base[kt%2] + r
  u32x4 pb[RT][2];  // fp16 probabilities as B operands of O^T += V^T P^T, per 32-key half
  // The K operand reads go in dim-slice order, four (one per key tile) ahead
  // of the 4 x RT MFMAs that use them, so the LDS reads of later slices
  // overlap the products of earlier ones; the MFMAs run dim-slice outermost
  // so 4 x RT accumulation chains are in flight.
  auto phase_qk = [&](const unsigned char* kl) {
    u32x4 ka[4][DC];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
        ka[kt][dc] = *reinterpret_cast<const u32x4*>(kl + (kt >> 1) * 2 * TILE + k_row_off[kt & 1] +
                                                     dc * 4 * kBlockSize * 16);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) st[rt][kt] = mfma_qk<T>(ka[kt][0], bq[rt][0], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int dc = 1; dc < DC; ++dc)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) st[rt][kt] = mfma_qk<T>(ka[kt][dc], bq[rt][dc], st[rt][kt]);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4 * RT, 0);
    }
  };
  // Online softmax, one row per lane; kDiag: the step reaches the causal
  // diagonal (or the end of the context) and needs the mask.  The reference
  // max m only moves when a score exceeds it by more than 2^kSlack, so the
  // accumulators are rescaled rarely; probabilities stay <= 2^kSlack.
  auto phase_softmax = [&](auto diag_tag, int s) __attribute__((always_inline)) {
    constexpr bool kDiag = decltype(diag_tag)::value;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      if constexpr (kDiag) {
        // last visible key of the step; rows past the chunk's last query
        // repeat that query (their loads were clamped) and take its limit,
        // so no key past the context (a stale slot, or a tile this call did
        // not stage) enters their scores or the wave's rescale vote
        int tok = i0 + 16 * (rt / HW) + r16;
        tok = tok < qlen ? tok : qlen - 1;
        const int lim = ctx + tok - kStepKeys * s;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            st[rt][kt][r] = 32 * (kt >> 1) + key_base[kt & 1] + r <= lim ? st[rt][kt][r] : -INFINITY;
      }
      // max over raw scores (scale > 0, so it commutes with the scaling),
      // then moved to base-2 units
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[rt][kt][r]);
      mx = row_max4(mx) * scale_log2;
      if (__any(mx > m[rt] + kSlack)) {
        const float mn = fmaxf(m[rt], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[rt] - mn);
        lsum[rt][0] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rt][dt] *= alpha;
        m[rt] = mn;
      }
      const float mr = m[rt];
      float e[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) e[kt][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(st[rt][kt][r], scale_log2, -mr));
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        pb[rt][kh][0] = pack_f16x2(e[2 * kh][0], e[2 * kh][1]);
        pb[rt][kh][1] = pack_f16x2(e[2 * kh][2], e[2 * kh][3]);
        pb[rt][kh][2] = pack_f16x2(e[2 * kh + 1][0], e[2 * kh + 1][1]);
        pb[rt][kh][3] = pack_f16x2(e[2 * kh + 1][2], e[2 * kh + 1][3]);
      }
    }
  };
  // O^T += V^T P^T, and the row sums as ones . P^T.  Per 32-key half, the V
  // operand reads go in two groups of DT / 2, the first ahead of the row-sum
  // MFMAs (which need none), the second ahead of the first DT / 2 dim tiles'
  // products, so LDS reads and MFMAs overlap.
  auto phase_pv = [&](const unsigned char* vl) {
    u32x4 va[2][DT];
#pragma unroll
    for (int kh = 0; kh < 2; ++kh)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        va[kh][dt] = *reinterpret_cast<const u32x4*>(vl + 2 * kh * TILE + dt * 16 * 32 + v_off);
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) lsum[rt] = mfma_pv(ones, pb[rt][kh], lsum[rt]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) o[rt][dt] = mfma_pv(va[kh][dt], pb[rt][kh], o[rt][dt]);
    }
#pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, DT / 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, RT, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, DT / 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, RT * DT / 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, RT * DT / 2, 0);
    }
  };

  // ---- schedule ----------------------------------------------------------------
  // A step s is two phases separated by workgroup barriers:
  //  * M(s), on the matrix cores: S(s) = K(s) Q^T, then O += P(s-1) V(s-1);
  //  * X(s), on the vector units: issue the loads of step s + kAhead, the
  //    softmax of step s, and the fp16 rewrite of this thread's V chunks of
  //    step s + 1.
  // Waves 4..7 run one phase behind waves 0..3; as waves w and w + 4 share a
  // SIMD, one of them issues MFMAs while the other runs vector work.  Every
  // wave passes the same number of barriers (2 per step plus one).
  //
  // Hazards, with phase k of the workgroup between barriers k and k + 1 and
  // M(s) in phase 2s (waves 0..3) or 2s + 1 (waves 4..7):
  //  * K(t) and V(t) are issued in X(t - 3); each thread waits for its own
  //    loads of step t at the start of M(t - 1) (phase <= 2t - 1), so K(t) is
  //    complete when read in phases 2t and 2t + 1;
  //  * V(t) is rewritten as fp16 by its loaders in X(t - 1) (phase <= 2t) and
  //    read in M(t + 1) (phases 2t + 2, 2t + 3);
  //  * K(t)'s buffer is reloaded (for K(t + NK)) in X(t + 1), phase >= 2t + 3;
  //    V(t)'s (for V(t + NV)) in X(t + 2), phase >= 2t + 5.
  const int grp = w >> 2;
  int s_diag = (ctx + i0 + 1) / kStepKeys;  // first step with a key past row i0's position
  s_diag = s_diag < nsteps ? s_diag : nsteps;

  for (int t = 0; t < kAhead && t < nsteps; ++t) {
    int32_t blk[NCH];
    load_blocks(t, blk);
    issue_blocks(t, blk);
  }
  {
    wait_vm(n_loads(1) + n_loads(2));  // step 0's loads have landed
    u32x4 raw[NCH];
    read_raw(0, raw);
    finish_step(0, raw);
  }
  lds_barrier();
  if (grp) lds_barrier();

  // Steps before s_diag lie wholly below this wave's first query row and need
  // no mask; the two ranges run as separate loops (one code path each keeps
  // the register budget).
  auto run_steps = [&](auto diag_tag, int s_begin, int s_end) __attribute__((always_inline)) {
#pragma unroll 1
    for (int s = s_begin; s < s_end; ++s) {
      const bool work = active && kStepKeys * s < kmax_w;
      const bool work_prev = s > 0 && active && kStepKeys * (s - 1) < kmax_w;
      wait_vm(n_loads(s + 2));  // this thread's loads of step s + 1 have landed
      int32_t blk[NCH];
      load_blocks(s + kAhead, blk);  // in flight during the products
      if (work) phase_qk(kbuf(s));
      if (work_prev) phase_pv(vbuf(s - 1));
      lds_barrier();
      issue_blocks(s + kAhead, blk);
      if (work) phase_softmax(diag_tag, s);
      if (s + 1 < nsteps) {
        u32x4 raw[NCH];
        read_raw(s + 1, raw);
        finish_step(s + 1, raw);
      }
      if (grp == 0 || s + 1 < nsteps) lds_barrier();
    }
  };
  run_steps(std::false_type{}, 0, s_diag);
  run_steps(std::true_type{}, s_diag, nsteps);
  if (active && kStepKeys * (nsteps - 1) < kmax_w) phase_pv(vbuf(nsteps - 1));

  // ---- normalise and write the wave's rows ---------------------------------
  if (!active) return;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float inv = 1.f / lsum[rt][0];
    const int tok = i0 + 16 * (rt / HW) + r16;
    if (tok < qlen && qs + tok < total_q) {
      const int64_t rowbase = ((int64_t)(qs + tok) * Hq + h0 + hb + rt % HW) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) store_out<OutCode>(out, rowbase + 16 * dt + 4 * q4 + r, o[rt][dt][r] * inv);
    }
  }
}

struct PrefillArgs {
  void* out;
  const uint16_t* q;
  const unsigned char* kpool;
  const unsigned char* vpool;
  const int32_t* tables;
  int max_blocks;
  const int32_t* cu_q;
  const int32_t* lens;
  int n_chunks, total_q, max_q_len, Hkv, G;
  int64_t num_blocks;
  int max_context_len;
  float scale_log2;
  hipStream_t stream;
};

template <typename T, int D, int GW, int OutCode>
void launch_prefill(const PrefillArgs& a) {
  constexpr int RT = 16 / kPfWaves;
  constexpr int HW = GW < RT ? GW : RT;
  constexpr int TWG = 16 * (RT / HW) * (kPfWaves / (GW / HW));
  const unsigned gy = (unsigned)((a.max_q_len + TWG - 1) / TWG);
  hipLaunchKernelGGL((prefill_chunk_kernel<T, D, GW, OutCode>),
                     dim3((unsigned)(a.Hkv * (a.G / GW)), gy, (unsigned)a.n_chunks), dim3(kPfThreads), 0,
                     a.stream, a.out, a.q, a.kpool, a.vpool, a.tables, a.max_blocks, a.cu_q, a.lens, a.total_q,
                     a.Hkv, a.G, a.num_blocks, a.max_context_len, a.scale_log2);
}

template <typename T, int D, int OutCode>
int prefill_dispatch_g(const PrefillArgs& a) {
  switch (a.G) {
    case 1: launch_prefill<T, D, 1, OutCode>(a); return 0;
    case 2: launch_prefill<T, D, 2, OutCode>(a); return 0;
    case 4:
    case 8:
    case 16: launch_prefill<T, D, 4, OutCode>(a); return 0;
    default: return -1;
  }
}

template <typename T, int OutCode>
int prefill_dispatch_d(const PrefillArgs& a, int D) {
  if (D == 64) return prefill_dispatch_g<T, 64, OutCode>(a);
  if (D == 128) return prefill_dispatch_g<T, 128, OutCode>(a);
  return -1;
}

}  // namespace
}  // namespace pkv

using pkv::fail;
using pkv::ok;

extern "C" int paged_attention_prefill_chunk(void* out, int32_t out_dtype, const void* q, const void* k_pool,
                                             const void* v_pool, const int32_t* block_tables,
                                             int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                                             const int32_t* context_lens, int32_t n_chunks, int32_t total_q,
                                             int32_t max_q_len, int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                             int32_t max_context_len, float scale, int32_t kv_dtype,
                                             void* stream) {
  const std::string F("paged_attention_prefill_chunk");
  if (kv_dtype != PKV_F16 && kv_dtype != PKV_BF16)
    return fail(kv_dtype == PKV_F32 ? PKV_EUNSUPPORTED : PKV_EINVAL, F + ": kv dtype must be f16 or bf16");
  if (out_dtype != PKV_F32 && out_dtype != kv_dtype)
    return fail(PKV_EINVAL, F + ": out dtype must be f32 or the kv dtype");
  if (block_size != pkv::kBlockSize) return fail(PKV_EUNSUPPORTED, "block_size must be 16");
  if (head_dim != 64 && head_dim != 128) return fail(PKV_EUNSUPPORTED, "head_dim must be 64 or 128");
  if (n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads)
    return fail(PKV_EINVAL, F + ": n_q_heads must be a positive multiple of n_kv_heads");
  const int G = n_q_heads / n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(PKV_EUNSUPPORTED, F + ": n_q_heads / n_kv_heads must be 1, 2, 4, 8 or 16");
  if (n_chunks < 0 || n_chunks > 65535 || total_q < 0 || max_q_len < 0)
    return fail(PKV_EINVAL, F + ": bad n_chunks, total_q or max_q_len");
  if (num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 0 ||
      (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_EINVAL, F + ": max_context_len exceeds the table width");
  if ((int64_t)n_kv_heads * (G >= 4 ? G / 4 : 1) > 65535 || max_q_len / 64 > 65535)
    return fail(PKV_EINVAL, F + ": grid too large");
  if (n_chunks == 0 || total_q == 0 || max_q_len == 0) return ok();
  if (!out || !q || !k_pool || !v_pool || !block_tables || !cu_q_lens || !context_lens)
    return fail(PKV_EINVAL, F + ": NULL pointer");
  if (!pkv::aligned16(q) || !pkv::aligned16(k_pool) || !pkv::aligned16(v_pool))
    return fail(PKV_EINVAL, F + ": q and pools must be 16-byte aligned");
  if (!std::isfinite(scale) || !(scale > 0.f)) return fail(PKV_EINVAL, F + ": scale must be finite and > 0");
  pkv::PrefillArgs a;
  a.out = out;
  a.q = (const uint16_t*)q;
  a.kpool = (const unsigned char*)k_pool;
  a.vpool = (const unsigned char*)v_pool;
  a.tables = block_tables;
  a.max_blocks = max_blocks_per_seq;
  a.cu_q = cu_q_lens;
  a.lens = context_lens;
  a.n_chunks = n_chunks;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.Hkv = n_kv_heads;
  a.G = G;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634);
  a.stream = (hipStream_t)stream;
  int rc;
  if (kv_dtype == PKV_BF16)
    rc = out_dtype == PKV_F32 ? pkv::prefill_dispatch_d<pkv::BF16, PKV_F32>(a, head_dim)
                              : pkv::prefill_dispatch_d<pkv::BF16, PKV_BF16>(a, head_dim);
  else
    rc = out_dtype == PKV_F32 ? pkv::prefill_dispatch_d<pkv::F16, PKV_F32>(a, head_dim)
                              : pkv::prefill_dispatch_d<pkv::F16, PKV_F16>(a, head_dim);
  if (rc) return fail(PKV_EUNSUPPORTED, F + ": configuration not built");
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, F + ": " + hipGetErrorString(e));
  return ok();
}
