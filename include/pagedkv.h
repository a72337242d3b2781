/*
 * pagedkv.h — C ABI of the MI355X (gfx950) paged KV-cache attention library.
 *
 * The library implements the PagedAttention hot path: a host-side block
 * manager that maps each sequence's logical KV blocks to physical blocks of a
 * shared pool, the cache-write kernel that appends new keys/values into their
 * slots, decode attention over the paged cache (split-context partitions plus
 * a reduction pass), and chunked-prefill attention (MFMA).
 *
 * Conventions for every entry point
 *   - Return value: PKV_OK (0) or a negative PKV_E* code.  pkv_last_error()
 *     returns a thread-local message for the last failing call.  Arguments are
 *     validated on the host before anything is launched; on error nothing is
 *     launched and no state changes.
 *   - Device pointers (pools, q, out, tables, lens, slot mappings, workspace)
 *     are owned by the caller (allocated e.g. with PyTorch) and must stay valid
 *     until the work queued on `stream` has finished.  The library owns only
 *     its host-side block-manager state.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.
 *     Kernels are queued asynchronously; PKV_EHIP reports a launch failure.
 *   - Block ids, slot numbers and lengths read from device memory are the
 *     caller's contract: kernels clamp block ids into [0, num_blocks) and
 *     lengths into [0, max_context_len] so that a bad value can never make
 *     them touch memory outside the buffers they were given, but the numbers
 *     produced in that case are unspecified.
 *   - block_size must be 16 (the pages' default block of 16 tokens).
 *
 * KV pool layout (one layer; the pages fix none, this is the library's own).
 * Elements are `esize` bytes (4 for PKV_F32, 2 for PKV_F16 / PKV_BF16, 1 for
 * PKV_FP8_E4M3) and x = 16 / esize elements form one 16-byte chunk:
 *   K element (block b, kv head g, token slot t, dim j) at element index
 *       ((((b * n_kv_heads + g) * (head_dim / x) + j / x) * block_size + t) * x + j % x)
 *   V element (b, g, t, j) at element index
 *       (((b * n_kv_heads + g) * head_dim + j) * block_size + t)
 * so one (block, kv head) tile of K or of V is block_size * head_dim * esize
 * contiguous bytes, and a pool holds num_blocks * n_kv_heads such tiles.
 * The token in physical slot s lives in block s / block_size at offset
 * s % block_size.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define PKV_OK 0
#define PKV_EINVAL (-1)        /* bad argument: null, shape, dtype, range */
#define PKV_ENOMEM_BLOCKS (-2) /* the pool has too few free blocks; nothing changed */
#define PKV_EUNSUPPORTED (-3)  /* valid but not built: head_dim, group size, block size */
#define PKV_EHIP (-4)          /* a HIP call or kernel launch failed */
#define PKV_ESTATE (-5)        /* unknown sequence id, or a pool in the wrong state */

/* element types */
#define PKV_F32 0
#define PKV_F16 1
#define PKV_BF16 2
/* 8-bit cache: OCP E4M3 codes (1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits; no infinities; 0x7f / 0xff are NaN; largest finite 448).
 * The pages allow an 8-bit cache ("Quantization", vLLM Serving deep dive:
 * about twice the tokens per byte of HBM) without fixing the format; each
 * pool carries one fp32 scale, a cached value being value(code) * scale. */
#define PKV_FP8_E4M3 3

/* Text of the last error on this thread ("" after a success).  A failing
 * call changes nothing and reports why, so that the caller can react instead
 * of crashing — as the scheduler of "The skeleton of a scheduler" (LLM
 * Serving from Scratch) reacts to running out of blocks by preempting.  The
 * string is owned by the library and valid until this thread's next call. */
const char* pkv_last_error(void);

/* ------------------------------------------------------------------------
 * Pool sizing and the host block manager
 * ------------------------------------------------------------------------ */

/* Bytes of K plus V per token across n_layers layers:
 * 2 * n_layers * n_kv_heads * head_dim * esize.
 * ("How big is the KV cache?", vLLM Serving deep dive, bytes/token formula.) */
int paged_kv_bytes_per_token(int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                             int32_t dtype, int64_t* bytes);

/* Whole blocks of block_size tokens, spanning n_layers layers, that fit in
 * budget_bytes: floor(budget / (block_size * bytes_per_token)).
 * ("Worked memory example" and "Reading the startup logs", vLLM Serving deep
 * dive: the "# GPU blocks" figure.) */
int paged_kv_blocks_for_budget(int64_t budget_bytes, int32_t n_layers, int32_t n_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t dtype,
                               int64_t* num_blocks);

typedef struct pkv_pool pkv_pool; /* opaque host state */

typedef struct pkv_pool_desc {
  int64_t num_blocks;  /* physical blocks in the pool, >= 1 */
  int32_t block_size;  /* tokens per block; must be 16 */
  int32_t n_kv_heads;  /* >= 1 */
  int32_t head_dim;    /* 64 or 128 */
  int32_t dtype;       /* PKV_F32, PKV_F16 or PKV_BF16 */
  int32_t n_layers;    /* layers whose per-layer pools share these block ids, >= 1 */
  int32_t reserved;    /* must be 0 */
  /* Host array [num_blocks]: initial order of the free-block queue (a
   * permutation of 0..num_blocks-1; copied).  NULL means 0, 1, ..., num_blocks-1. */
  const int32_t* initial_free_order;
} pkv_pool_desc;

/* Create the block manager of one pool ("PagedAttention in depth", vLLM
 * Serving deep dive: a global pool of fixed-size blocks and one block table
 * per sequence; "Back to the queue, and into vLLM proper", Life of a prompt:
 * the free block queue).  It owns host memory only; the device pools are
 * caller-allocated buffers of paged_kv_pool_bytes() bytes each, per layer.
 * *out receives the handle; release it with paged_kv_destroy. */
int paged_kv_alloc(const pkv_pool_desc* desc, pkv_pool** out);

/* Bytes of one layer's K pool and of one layer's V pool for desc:
 * num_blocks * n_kv_heads * block_size * head_dim * esize each. */
int paged_kv_pool_bytes(const pkv_pool_desc* desc, int64_t* k_bytes, int64_t* v_bytes);

/* Free the host state: the per-sequence block tables and the free block
 * queue, the small CPU-side bookkeeping of "Back to the queue, and into vLLM
 * proper" (Life of a prompt).  Device pools are untouched (the caller owns
 * them).  PKV_EINVAL for NULL; the handle is invalid afterwards. */
int paged_kv_destroy(pkv_pool* pool);

/* New empty sequence with an empty block table: a request admitted from the
 * waiting queue gets its own ordered list of block ids ("admit" in "The
 * skeleton of a scheduler", LLM Serving from Scratch; the page table of "Back
 * to the queue, and into vLLM proper", Life of a prompt).  No block is taken
 * until tokens are appended.  *seq receives its id (ids count up from 0). */
int paged_kv_seq_create(pkv_pool* pool, int64_t* seq);

/* New sequence that shares the physical blocks holding the parent's first
 * n_prefix_tokens tokens (ceil(n / block_size) blocks, each reference count
 * +1); its length is n_prefix_tokens.  ("Sharing and copy-on-write", vLLM
 * Serving deep dive.)  PKV_ESTATE if parent is unknown, PKV_EINVAL if
 * n_prefix_tokens is outside [0, parent length]. */
int paged_kv_seq_fork(pkv_pool* pool, int64_t parent, int64_t n_prefix_tokens, int64_t* child);

/* Reserve slots for n_tokens new tokens at the end of seq.
 *   - A new block is taken from the head of the free queue only when the
 *     sequence's last block is full (so L tokens own ceil(L / 16) blocks).
 *   - If the last block is partly filled and shared (reference count > 1),
 *     it is copied first: a fresh block replaces it in this sequence's table
 *     only, the old block's count drops by one, and the pair (old, new) is
 *     reported so the caller can copy the device data (paged_kv_copy_blocks)
 *     before writing.  A full shared block is never written, so no copy.
 *   ("PagedAttention in depth" and "Sharing and copy-on-write", vLLM Serving
 *   deep dive; "Back to the queue, and into vLLM proper", Life of a prompt.)
 * slot_mapping_out: host [n_tokens], receives physical slot
 *   table[t / 16] * 16 + t % 16 of each new token t (may be NULL).
 * cow_pairs_out: host [2 * max_cow] int32 (src, dst) pairs (may be NULL when
 *   max_cow is 0); *n_cow receives the number written (0 or 1).
 * All or nothing: PKV_ENOMEM_BLOCKS if the free queue cannot supply every
 * block the append needs — nothing changes, so the caller can preempt
 * ("The skeleton of a scheduler", LLM Serving from Scratch).  PKV_EINVAL if
 * max_cow is too small for the copy the append needs (again no change). */
int paged_kv_seq_append(pkv_pool* pool, int64_t seq, int64_t n_tokens, int64_t* slot_mapping_out,
                        int32_t* cow_pairs_out, int32_t max_cow, int32_t* n_cow);

/* A step's appends in one call (the per-step host work of "The skeleton of a
 * scheduler", LLM Serving from Scratch: every running sequence gets its next
 * token's slot).  Sequence seqs[i] gets n_tokens[i] new tokens (one each when
 * n_tokens is NULL), in list order, each exactly as paged_kv_seq_append would
 * append it (new blocks from the head of the free queue, copy-on-write of a
 * shared partly filled last block).
 *   seqs            host int64 [n]
 *   n_tokens        host int64 [n], >= 0, or NULL
 *   slot_mapping_out host int64 [sum of the counts] (may be NULL): the slots
 *                   of sequence 0's new tokens, then sequence 1's, ...
 *   cow_pairs_out   host int32 [2 * max_cow] (src, dst) pairs in order (may
 *                   be NULL when max_cow is 0); *n_cow receives their number
 *   *n_done         receives the number of sequences appended.
 * The sequences are appended one after another; the first that cannot be
 * stops the call with its code — PKV_ENOMEM_BLOCKS (the free queue is
 * short), PKV_ESTATE (unknown or swapped-out sequence) or PKV_EINVAL (no
 * room left in cow_pairs_out) — with the earlier ones appended and reported
 * (*n_done, their slots and pairs) and that one and the later ones
 * unchanged, so the caller can preempt and call again for the rest.
 * PKV_EINVAL before any change for a negative count or NULL list. */
int paged_kv_seqs_append(pkv_pool* pool, const int64_t* seqs, int32_t n, const int64_t* n_tokens,
                         int64_t* slot_mapping_out, int32_t* cow_pairs_out, int32_t max_cow, int32_t* n_cow,
                         int32_t* n_done);

/* Blocks the append of n_tokens would take from the free queue (new blocks
 * plus a copy-on-write block), without changing anything. */
int paged_kv_seq_blocks_needed(pkv_pool* pool, int64_t seq, int64_t n_tokens, int64_t* n_blocks);

/* Finish seq: every block's reference count drops by one and blocks reaching
 * zero rejoin the tail of the free queue at once, in the sequence's logical
 * order ("Back to the queue, and into vLLM proper", Life of a prompt).  With
 * prefix caching on, a released labelled block keeps its label while it
 * waits in the queue (see paged_kv_prefix_cache_enable). */
int paged_kv_seq_free(pkv_pool* pool, int64_t seq);

/* Automatic prefix caching ("Trick 3, Prefix caching", How AI actually
 * answers you; "Prefix caching (automatic KV reuse)", vLLM Serving deep dive;
 * The hands-on guide to LLM Inference with vLLM, Automatic Prefix Caching).
 * Off by default.  When on, every full block of a sequence whose token ids
 * are known is labelled with a fingerprint of its 16 tokens chained with the
 * fingerprint of the block before it (a 64-bit mix; a lookup also compares
 * the stored tokens and previous fingerprint).  Only full blocks are
 * labelled, and a block whose content is already labelled elsewhere is not.
 * A released labelled block stays reusable while it waits in the free queue
 * and loses its label when the queue hands it out again, so unused cached
 * blocks are evicted least recently released first.  Turning caching off
 * drops every label.  Token ids are known for sequences made by
 * paged_kv_seq_create / paged_kv_seq_create_cached and extended only with
 * paged_kv_seq_append_tokens (forks inherit the parent's); a plain
 * paged_kv_seq_append makes the rest of that sequence unlabelled. */
int paged_kv_prefix_cache_enable(pkv_pool* pool, int32_t enable);

/* New sequence for a prompt of n_tokens token ids: its leading full blocks
 * whose labels are cached are reused (reference count +1; a cached block
 * waiting in the free queue leaves it), stopping at the first miss and
 * leaving at least the prompt's last token uncached.  *n_cached receives the
 * number of reused tokens (a multiple of 16), which is the new sequence's
 * length: append the remaining n_tokens - *n_cached tokens with
 * paged_kv_seq_append_tokens and compute only those.  With caching off the
 * sequence starts empty.  tokens is host int32 [n_tokens]. */
int paged_kv_seq_create_cached(pkv_pool* pool, const int32_t* tokens, int64_t n_tokens, int64_t* seq,
                               int64_t* n_cached);

/* paged_kv_seq_append with the new tokens' ids (host int32 [n_tokens]), so
 * that the blocks it fills can be labelled for prefix caching.  Same slots,
 * copy-on-write and all-or-nothing behaviour as paged_kv_seq_append. */
int paged_kv_seq_append_tokens(pkv_pool* pool, int64_t seq, const int32_t* tokens, int64_t n_tokens,
                               int64_t* slot_mapping_out, int32_t* cow_pairs_out, int32_t max_cow,
                               int32_t* n_cow);

/* Prefix-cache counters: labelled blocks now, full prompt blocks looked up
 * and found by paged_kv_seq_create_cached so far (any pointer may be NULL). */
int paged_kv_prefix_cache_stats(pkv_pool* pool, int64_t* cached_blocks, int64_t* queried_blocks,
                                int64_t* hit_blocks);

/* Length (tokens) of seq. */
int paged_kv_seq_len(pkv_pool* pool, int64_t seq, int64_t* len);

/* Copy seq's block table (logical order) into blocks_out[cap]; *n receives
 * its length (PKV_EINVAL if cap is smaller; blocks_out may then be NULL to
 * query the length). */
int paged_kv_seq_table(pkv_pool* pool, int64_t seq, int32_t* blocks_out, int64_t cap, int64_t* n);

/* Export the block tables of n sequences as a host int32 [n][max_blocks]
 * array, rows padded with -1, and their lengths as host int32 [n]
 * (the table the attention kernels read, "How the attention kernel actually
 * reads paged blocks", vLLM Serving deep dive).  PKV_EINVAL if a table is
 * longer than max_blocks. */
int paged_kv_block_tables(pkv_pool* pool, const int64_t* seqs, int32_t n, int32_t max_blocks,
                          int32_t* tables_out, int32_t* lens_out);

/* Free blocks in the queue (*n): what an admission test such as
 * can_allocate, or the out_of_blocks check before preempting, compares a
 * request's needs with ("The skeleton of a scheduler", LLM Serving from
 * Scratch; the free block queue of "Back to the queue, and into vLLM proper",
 * Life of a prompt). */
int paged_kv_num_free(pkv_pool* pool, int64_t* n);

/* Reference count of one block (0 for a free block). */
int paged_kv_block_refcount(pkv_pool* pool, int64_t block, int32_t* ref);

/* Copy the free queue, head first, into out[cap]; *n receives its length. */
int paged_kv_free_queue(pkv_pool* pool, int32_t* out, int64_t cap, int64_t* n);

/* ------------------------------------------------------------------------
 * Swap space: host ("CPU") blocks for preempted sequences
 * ("The scheduler: waiting, running, swapped", vLLM Serving deep dive: a
 * preempted sequence's blocks are copied to CPU swap space and restored
 * later; "Back to the queue, and into vLLM proper", Life of a prompt: the CPU
 * blocks are a pool of pinned host memory sized like the GPU pool,
 * paged_kv_blocks_for_budget of the swap space).  The host pools themselves
 * (one K and one V pool per layer, same layout and block size as the GPU
 * pools) are caller-allocated pinned memory; the block manager only hands out
 * their block ids, FIFO, and reports the copies to run with
 * paged_kv_swap_blocks.
 * ------------------------------------------------------------------------ */

/* Give the pool num_cpu_blocks host blocks, queued 0, 1, ..., n-1 (0 removes
 * the swap space).  PKV_ESTATE while any sequence is swapped out. */
int paged_kv_swap_space(pkv_pool* pool, int64_t num_cpu_blocks);

/* Swap a sequence out: each of its blocks, in logical order, gets a host
 * block from the head of the host queue (a private copy, also of blocks it
 * shares with other sequences), then its GPU blocks are released as by
 * paged_kv_seq_free (reference counts drop; blocks reaching zero join the
 * free queue's tail, where they keep their bytes and any prefix-cache label
 * until the queue hands them out).  pairs_out (host int32 [cap][2]) receives
 * the copies (GPU block, host block), *n_pairs their number (= the table
 * length).  Queue the copy (paged_kv_swap_blocks, GPU pools -> host pools)
 * before any later write into blocks allocated after this call, on the same
 * stream.  All or nothing: PKV_ENOMEM_BLOCKS if the host queue is too short,
 * PKV_EINVAL if cap is smaller than the table, PKV_ESTATE if the sequence is
 * unknown or already swapped out.  While swapped out a sequence can only be
 * swapped in, freed (its host blocks rejoin their queue) or read with
 * paged_kv_seq_table / paged_kv_seq_len (the table then names host blocks);
 * appends, forks, paged_kv_seq_blocks_needed and paged_kv_block_tables return
 * PKV_ESTATE. */
int paged_kv_seq_swap_out(pkv_pool* pool, int64_t seq, int32_t* pairs_out, int64_t cap, int64_t* n_pairs);

/* Swap a sequence back in: each host block, in logical order, gets a GPU
 * block from the head of the free queue, then the host blocks rejoin their
 * queue's tail.  pairs_out receives (host block, GPU block); queue the copy
 * (host pools -> GPU pools) before anything reads the sequence.  Its full
 * blocks are labelled again for prefix caching when their tokens are known and
 * the same text is not cached already.  All or nothing: PKV_ENOMEM_BLOCKS if
 * the free queue is too short, PKV_EINVAL if cap is too small, PKV_ESTATE if
 * the sequence is not swapped out. */
int paged_kv_seq_swap_in(pkv_pool* pool, int64_t seq, int32_t* pairs_out, int64_t cap, int64_t* n_pairs);

/* *swapped = 1 if the sequence is swapped out, else 0. */
int paged_kv_seq_is_swapped(pkv_pool* pool, int64_t seq, int32_t* swapped);

/* Copy the host block queue, head first, into out[cap]; *n receives its
 * length (out may be NULL to query it). */
int paged_kv_cpu_free_queue(pkv_pool* pool, int32_t* out, int64_t cap, int64_t* n);

/* ------------------------------------------------------------------------
 * Device operations (HIP, gfx950)
 * ------------------------------------------------------------------------ */

/* Append new tokens' keys and values into their cache slots (the write that
 * fills the blocks: "Back to the queue, and into vLLM proper" and "The
 * decode stage, and how to spot the waste", Life of a prompt — each new key
 * and value row is appended to the cached ones).
 *   key, value   device, token i's row at key + i * key_token_stride
 *                elements: [n_kv_heads][head_dim] contiguous, dtype elements;
 *                pointers and strides 16-byte aligned.
 *   k_pool, v_pool  device pools in the layout above (num_blocks blocks).
 *   slot_mapping device int64 [num_tokens]; slot -1 means skip the token.
 * A bit-exact copy: no conversion.  Slots >= num_blocks * block_size are
 * skipped (caller contract). */
int reshape_and_cache(const void* key, const void* value, int64_t key_token_stride,
                      int64_t value_token_stride, void* k_pool, void* v_pool,
                      const int64_t* slot_mapping, int64_t num_tokens, int64_t num_blocks,
                      int32_t n_kv_heads, int32_t head_dim, int32_t block_size, int32_t dtype,
                      void* stream);

/* reshape_and_cache into an 8-bit pool pair (dtype PKV_FP8_E4M3): the new
 * rows are quantised on the way in.  Element x of a key row is stored as the
 * E4M3 code nearest to fp32(x) * fp32(1 / k_scale) (the reciprocal rounded to
 * nearest once, the product rounded to nearest; ties to the even code;
 * finite magnitudes beyond 448 and infinities saturate to +-448; NaN gives a
 * NaN code; a value that rounds to zero keeps its sign), values likewise with
 * v_scale.  The pages allow the 8-bit cache ("Quantization", vLLM Serving deep
 * dive) but give no rounding or scale rule: this is the library's reading.
 *   key, value   device rows as for reshape_and_cache, in src_dtype
 *                (PKV_F32, PKV_F16 or PKV_BF16).
 *   k_pool, v_pool  device 8-bit pools (num_blocks * n_kv_heads * block_size
 *                * head_dim bytes each) in the layout above with esize 1.
 *   k_scale, v_scale  finite and > 0 (PKV_EINVAL otherwise).
 * Rows that are already E4M3 codes are copied unchanged by reshape_and_cache
 * with dtype PKV_FP8_E4M3. */
int reshape_and_cache_fp8(const void* key, const void* value, int32_t src_dtype,
                          int64_t key_token_stride, int64_t value_token_stride, void* k_pool,
                          void* v_pool, const int64_t* slot_mapping, int64_t num_tokens,
                          int64_t num_blocks, int32_t n_kv_heads, int32_t head_dim,
                          int32_t block_size, float k_scale, float v_scale, void* stream);

/* Copy whole blocks of one layer's K and V pools: pairs_dev is device int32
 * [n_pairs][2] (src, dst), as reported by paged_kv_seq_append for a
 * copy-on-write ("Sharing and copy-on-write", vLLM Serving deep dive).
 * Pairs with an id outside [0, num_blocks) are skipped. */
int paged_kv_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs_dev, int32_t n_pairs,
                         int64_t num_blocks, int32_t n_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t dtype, void* stream);

/* Copy whole blocks from one pool pair to another: for each pair i, block
 * pairs[2i] of (src_k_pool, src_v_pool) to block pairs[2i+1] of (dst_k_pool,
 * dst_v_pool) — the swap-out / swap-in copies of paged_kv_seq_swap_out /
 * _swap_in ("The scheduler: waiting, running, swapped", vLLM Serving deep
 * dive).  Pools and pairs may be device memory or pinned host memory
 * (hipHostMalloc, e.g. PyTorch's pin_memory): the kernel reads and writes
 * host blocks over the host link itself, all pairs in one launch.  Block
 * bytes = n_kv_heads * block_size * head_dim * esize(dtype) per pool.  Pairs
 * with an id outside [0, src_num_blocks) / [0, dst_num_blocks) are skipped;
 * pairs must name distinct destination blocks.  PKV_EINVAL for memory the GPU
 * cannot reach (pageable host memory). */
int paged_kv_swap_blocks(const void* src_k_pool, const void* src_v_pool, int64_t src_num_blocks,
                         void* dst_k_pool, void* dst_v_pool, int64_t dst_num_blocks,
                         const int32_t* pairs, int32_t n_pairs, int32_t n_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t dtype, void* stream);

/* Context tokens one decode partition covers (the split-context unit). */
int32_t paged_attention_decode_partition_size(void);

/* 1 when paged_attention_decode and paged_attention_decode_append take the
 * whole-context path for these sizes, 0 otherwise (the split-context path;
 * paged_attention_decode_partitions / _reduce always split).  The path is
 * taken, with P = num_seqs * n_kv_heads, for 16-bit and 8-bit pools when
 * max_context_len <= 4096 and either P <= 256 and (P >= 128 or
 * max_context_len <= 1536), or 384 <= P <= 512 and max_context_len <= 2048;
 * for fp32 pools when max_context_len <= 2048, (n_q_heads / n_kv_heads) *
 * head_dim * 4 <= 1024 and either P <= 256 and (P >= 128 or max_context_len
 * <= 1536), or 448 <= P <= 512 with max_context_len * 2 * head_dim * 4 >= 384
 * KiB (the decode of a small batch
 * is bound by the latency of one or two rounds of reads, not by HBM
 * bandwidth).  ("The decode stage, and how to spot the
 * waste", Life of a prompt: the same attention, one query per sequence.)
 * Invalid sizes give 0. */
int32_t paged_attention_decode_whole_context(int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                             int32_t head_dim, int32_t kv_dtype, int32_t max_context_len);

/* Device workspace bytes paged_attention_decode needs for these sizes
 * (0 when every sequence fits in one partition): the partial softmax states
 * (max, sum and unnormalised output, fp32) of every partition of every
 * (sequence, query head), num_seqs * n_q_heads * ceil(max_context_len /
 * partition size) * (head_dim + 2) * 4 bytes.  The attention is the decode
 * step of "The decode stage, and how to spot the waste" (Life of a prompt):
 * one query against the sequence's full K and V; splitting the context into
 * partitions whose states are merged afterwards is this library's way of
 * spreading one long sequence over many compute units (the pages give no
 * kernel design).  0 for non-positive arguments. */
int64_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t n_q_heads,
                                               int32_t head_dim, int32_t max_context_len);

/* Decode attention over the paged cache: one query token per sequence
 * attends to all context_lens[s] cached keys of its sequence, the newest
 * (already appended) included.  For query head h, KV head g = h / (n_q_heads
 * / n_kv_heads):  out[s][h] = sum_j softmax_j(scale * q[s][h] . K_j) V_j.
 * ("The decode stage, and how to spot the waste", Life of a prompt: one new
 * query against the full K and V; "How the attention kernel actually reads
 * paged blocks", vLLM Serving deep dive: the kernel reads the block table and
 * works block by block.)  Long contexts are split into partitions of
 * paged_attention_decode_partition_size() tokens whose partial softmax
 * states are merged by a second reduction kernel.
 * Shared blocks: when sequences of one aligned window of 32 / G batch
 * entries (G = n_q_heads / n_kv_heads), in any order within it, name the
 * same blocks for a whole partition (sequences forked from one prefix:
 * "Memory sharing", vLLM Serving deep dive), one workgroup reads that
 * partition once for all of them (up to 32 query rows, on MFMA; 16-bit and
 * 8-bit K/V): a third kernel, queued on `stream` before the per-sequence
 * partition pass.
 * Short contexts in a small batch (paged_attention_decode_whole_context
 * says when): one launch instead, one workgroup per (sequence, KV head)
 * taking the whole context with its blocks dealt to 16 waves (16-bit K/V
 * on MFMA, the G query rows in one 16-row tile; fp32 K/V on the vector
 * units) and the waves' softmax states merged on chip; no partition is
 * split or shared, the workspace is not touched.
 *   out           device [num_seqs][n_q_heads][head_dim], out_dtype
 *                 (PKV_F32, or the KV dtype).
 *   q             device [num_seqs][n_q_heads][head_dim], kv_dtype.
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq].
 *   context_lens  device int32 [num_seqs]; each in [1, max_context_len]
 *                 (a sequence with 0 gets zeros).
 *   max_context_len <= max_blocks_per_seq * block_size.
 *   workspace     device, >= paged_attention_decode_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0); contents need no
 *                 initialisation and are overwritten.
 * Supported: kv_dtype PKV_F32, PKV_F16 or PKV_BF16 (8-bit pools go to
 * paged_attention_decode_fp8), head_dim 64/128, n_q_heads / n_kv_heads in
 * {1, 2, 4, 8, 16}, block_size 16.  Accumulation is fp32. */
int paged_attention_decode(void* out, int32_t out_dtype, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           int32_t max_context_len, float scale, int32_t kv_dtype, void* workspace,
                           int64_t workspace_bytes, void* stream);

/* One decode step's cache write and attention in one call:
 * reshape_and_cache of each sequence's new token (k_new / v_new row s into
 * slot_mapping[s]), then paged_attention_decode, with the same results (the
 * step of "The decode stage, and how to spot the waste", Life of a prompt:
 * append the new key and value, then attend over all of them).  With f16 /
 * bf16 pools the rows are written by extra workgroups of the shared-run
 * kernel, or on the whole-context path by the workgroup of each (sequence,
 * KV head) before it reads, so the write needs no launch of its own; with
 * f32 pools the write is launched first.  The new token's block must be the sequence's own (as
 * paged_kv_seq_append leaves it, copy-on-write done) and context_lens must
 * already count the new token.
 *   k_new, v_new   device [num_seqs][n_kv_heads * head_dim] rows, kv_dtype,
 *                  token strides k_new_stride / v_new_stride in elements
 *                  (16-byte aligned rows).
 *   slot_mapping   device int64 [num_seqs]; a slot outside the pool skips
 *                  that row's write.
 * Everything else as paged_attention_decode.  Every argument is checked
 * before anything is launched.  8-bit pools: PKV_EINVAL (use
 * reshape_and_cache_fp8, then paged_attention_decode_fp8). */
int paged_attention_decode_append(void* out, int32_t out_dtype, const void* q, const void* k_new,
                                  const void* v_new, int64_t k_new_stride, int64_t v_new_stride,
                                  const int64_t* slot_mapping, void* k_pool, void* v_pool,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads,
                                  int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                  int64_t num_blocks, int32_t max_context_len, float scale,
                                  int32_t kv_dtype, void* workspace, int64_t workspace_bytes,
                                  void* stream);

/* paged_attention_decode_append for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, the same
 * results.  The split-context partials go to a scratch array the library
 * holds in device memory, one copy per GPU, of
 * paged_attention_decode_noalloc_max_workspace_bytes() bytes (64 MiB); its
 * address is looked up on the first call on each device (the current device,
 * which must be the one `stream` belongs to).  PKV_EINVAL when
 * paged_attention_decode_workspace_bytes(num_seqs, n_q_heads, head_dim,
 * max_context_len) exceeds it.  Nothing is allocated.  Every call on one GPU
 * shares that GPU's scratch, so calls that overlap on one GPU (different
 * streams, or threads without ordering) race; calls queued on one stream are
 * ordered and safe. */
int paged_attention_decode_append_noalloc(void* out, int32_t out_dtype, const void* q, const void* k_new,
                                          const void* v_new, int64_t k_new_stride, int64_t v_new_stride,
                                          const int64_t* slot_mapping, void* k_pool, void* v_pool,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads,
                                          int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                          int64_t num_blocks, int32_t max_context_len, float scale,
                                          int32_t kv_dtype, void* stream);

/* Bytes of the scratch paged_attention_decode_append_noalloc uses per GPU. */
int64_t paged_attention_decode_noalloc_max_workspace_bytes(void);

/* Decode attention over an 8-bit cache (PKV_FP8_E4M3 pools written by
 * reshape_and_cache_fp8): the same result as paged_attention_decode with
 * every cached key and value replaced by value(code) * k_scale (resp.
 * v_scale).  The query stays in q_dtype (PKV_F16 or PKV_BF16); out_dtype is
 * PKV_F32 or q_dtype.  Other arguments, the workspace size
 * (paged_attention_decode_workspace_bytes) and the supported shapes are those
 * of paged_attention_decode.  The codes are widened exactly to q_dtype for the
 * score products and to fp16 for the value products (both on MFMA, fp32
 * accumulation, probabilities in fp16); k_scale folds into the softmax scale
 * and v_scale into the output.  Short contexts in a small batch take the
 * whole-context launch as paged_attention_decode does
 * (paged_attention_decode_whole_context with PKV_FP8_E4M3 says when).
 * k_scale, v_scale finite and > 0.  Half the
 * bytes of a 16-bit cache per decode step ("Quantization", vLLM Serving deep
 * dive). */
int paged_attention_decode_fp8(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                               const void* k_pool, const void* v_pool, float k_scale,
                               float v_scale, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* context_lens,
                               int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               int32_t max_context_len, float scale, void* workspace,
                               int64_t workspace_bytes, void* stream);
/* The decode step over 8-bit pools in one call: reshape_and_cache_fp8 of
 * each sequence's new row (k_new / v_new in q_dtype, quantised with the
 * pools' scales), then paged_attention_decode_fp8, with the same results.
 * The rows are quantised by extra workgroups of the shared-run kernel (no
 * launch of their own), as in paged_attention_decode_append, whose
 * conditions hold here too (the new token's block is the sequence's own,
 * context_lens count it).  k_new / v_new: device [num_seqs][n_kv_heads *
 * head_dim] rows of q_dtype with token strides in elements (16-byte aligned);
 * slot_mapping device int64 [num_seqs] (a slot outside the pool skips that
 * row).  Everything else as paged_attention_decode_fp8; every argument is
 * checked before anything is launched. */
int paged_attention_decode_fp8_append(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                                      const void* k_new, const void* v_new, int64_t k_new_stride,
                                      int64_t v_new_stride, const int64_t* slot_mapping, void* k_pool,
                                      void* v_pool, float k_scale, float v_scale,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                                      int64_t num_blocks, int32_t max_context_len, float scale,
                                      void* workspace, int64_t workspace_bytes, void* stream);

/* Its two passes, as paged_attention_decode_partitions / _reduce are for
 * paged_attention_decode (same arguments and ordering rule). */
int paged_attention_decode_fp8_partitions(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                                          const void* k_pool, const void* v_pool, float k_scale,
                                          float v_scale, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                          int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                          int32_t max_context_len, float scale, void* workspace,
                                          int64_t workspace_bytes, void* stream);
int paged_attention_decode_fp8_reduce(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                                      const void* k_pool, const void* v_pool, float k_scale,
                                      float v_scale, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* context_lens,
                                      int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                      int32_t max_context_len, float scale, void* workspace,
                                      int64_t workspace_bytes, void* stream);

/* The two passes of paged_attention_decode, for callers that schedule them
 * separately (same arguments, same validation).  _partitions runs the
 * partition pass: sequences that fit in one partition get their final output,
 * longer ones leave partial softmax states in the workspace.  _reduce then
 * merges those states into out (a no-op when max_context_len fits one
 * partition).  Queue _reduce after _partitions on the same stream (or order
 * them with events) and do not touch the workspace in between. */
int paged_attention_decode_partitions(void* out, int32_t out_dtype, const void* q,
                                      const void* k_pool, const void* v_pool,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                      int32_t block_size, int64_t num_blocks,
                                      int32_t max_context_len, float scale, int32_t kv_dtype,
                                      void* workspace, int64_t workspace_bytes, void* stream);
int paged_attention_decode_reduce(void* out, int32_t out_dtype, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* context_lens,
                                  int32_t num_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                  int32_t max_context_len, float scale, int32_t kv_dtype,
                                  void* workspace, int64_t workspace_bytes, void* stream);

/* Chunked-prefill attention: chunk c holds the query tokens
 * cu_q_lens[c] .. cu_q_lens[c+1]-1 (rows of q/out) of one sequence whose
 * keys and values — the cached context plus the chunk itself, already
 * appended with reshape_and_cache — number context_lens[c].  Query i of
 * the chunk sits at absolute position p = context_lens[c] - q_len + i and
 * attends causally to keys 0..p.  ("Chunked prefill" in The hands-on guide
 * to LLM Inference with vLLM: each chunk's attention reads the KV of every
 * chunk before it; "The detour, what really happens inside one forward
 * pass", Life of a prompt: the Q K^T -> softmax -> V contraction.)
 *   out, q        device [total_q][n_q_heads][head_dim] (out in out_dtype,
 *                 q in kv_dtype).
 *   block_tables  device int32 [n_chunks][max_blocks_per_seq].
 *   cu_q_lens     device int32 [n_chunks + 1], cu_q_lens[0] = 0,
 *                 non-decreasing, cu_q_lens[n_chunks] = total_q,
 *                 each q_len <= max_q_len and <= context_lens[c].
 *   context_lens  device int32 [n_chunks], <= max_context_len
 *                 <= max_blocks_per_seq * block_size.
 * Supported: kv_dtype PKV_F16 or PKV_BF16, head_dim 64/128, n_q_heads /
 * n_kv_heads in {1, 2, 4, 8, 16}, block_size 16, scale finite and > 0
 * (PKV_EINVAL otherwise).  Products on MFMA, fp32 accumulation and softmax;
 * the P.V product takes V and the probabilities in fp16, so bf16 V entries
 * beyond fp16's range (|v| > 65504) are clamped to it.  8-bit pools: chunks
 * over an E4M3 cache go through paged_attention_verify_fp8, the same causal
 * attention for up to 64 query tokens per sequence (a longer chunk in pieces
 * of at most 64 queries, each with context_lens counting keys up to the
 * piece's last query). */
int paged_attention_prefill_chunk(void* out, int32_t out_dtype, const void* q, const void* k_pool,
                                  const void* v_pool, const int32_t* block_tables,
                                  int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                                  const int32_t* context_lens, int32_t n_chunks, int32_t total_q,
                                  int32_t max_q_len, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int32_t block_size, int64_t num_blocks,
                                  int32_t max_context_len, float scale, int32_t kv_dtype,
                                  void* stream);

/* Device workspace bytes paged_attention_verify needs for these sizes (0 when
 * every context fits in one partition). */
int64_t paged_attention_verify_workspace_bytes(int32_t total_q, int32_t n_q_heads, int32_t head_dim,
                                               int32_t max_context_len);

/* Verify attention: a few new query tokens per sequence (the drafted tokens
 * of speculative decoding plus one, checked by the large model in one pass:
 * "Speculative decoding" in the vLLM Serving deep dive and in How AI
 * actually answers you), each attending causally to the sequence's cached
 * keys and the new keys before it.  The same arguments and result as
 * paged_attention_prefill_chunk (sequence c's new tokens are rows
 * cu_q_lens[c] .. cu_q_lens[c+1]-1 of q / out, query i at absolute position
 * context_lens[c] - q_len + i, keys already appended), computed the way a
 * decode step is: 512-token split-context partitions read once per KV head
 * for all of the sequence's new tokens (MFMA, fp32 accumulation; bf16 values
 * are exact operands with each probability split into a bf16 pair, fp16
 * values take fp16 probabilities), partial states merged per token.
 *   workspace  device, >= paged_attention_verify_workspace_bytes(total_q,
 *              n_q_heads, head_dim, max_context_len) bytes (NULL when 0).
 * Supported: kv_dtype PKV_F16 or PKV_BF16 (out PKV_F32 or kv_dtype),
 * head_dim 64/128, n_q_heads / n_kv_heads in {1, 2, 4, 8, 16}, max_q_len <=
 * 64 (PKV_EUNSUPPORTED above: use paged_attention_prefill_chunk), n_seqs and
 * total_q <= 65535, scale finite. */
int paged_attention_verify(void* out, int32_t out_dtype, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* cu_q_lens,
                           const int32_t* context_lens, int32_t n_seqs, int32_t total_q,
                           int32_t max_q_len, int32_t n_q_heads, int32_t n_kv_heads,
                           int32_t head_dim, int32_t block_size, int64_t num_blocks,
                           int32_t max_context_len, float scale, int32_t kv_dtype, void* workspace,
                           int64_t workspace_bytes, void* stream);

/* paged_attention_verify over an 8-bit cache (PKV_FP8_E4M3 pools, scales as
 * for paged_attention_decode_fp8): queries and output in q_dtype (PKV_F16 or
 * PKV_BF16; out PKV_F32 or q_dtype); everything else as paged_attention_verify. */
int paged_attention_verify_fp8(void* out, int32_t out_dtype, const void* q, int32_t q_dtype,
                               const void* k_pool, const void* v_pool, float k_scale, float v_scale,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* cu_q_lens, const int32_t* context_lens, int32_t n_seqs,
                               int32_t total_q, int32_t max_q_len, int32_t n_q_heads,
                               int32_t n_kv_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks, int32_t max_context_len, float scale,
                               void* workspace, int64_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Measurement
 * ------------------------------------------------------------------------ */

/* A read-only pass over tiles of one or two pools: the bandwidth an
 * HBM-bound kernel with this access pattern can reach, with no attention
 * arithmetic (the decode kernels read the (block, KV head) tiles a step's
 * block tables name, "How the attention kernel actually reads paged blocks",
 * vLLM Serving deep dive).  Entry e of tiles (device int64 [n_tiles]) names
 * tile tiles[e], the tile_bytes bytes at pool + tiles[e] * tile_bytes, of
 * k_pool for e < n_k_tiles and of v_pool after; tiles NULL reads tiles 0,
 * 1, ..., n_tiles - 1 of k_pool, a contiguous read of n_tiles * tile_bytes
 * bytes (n_k_tiles must then equal n_tiles, PKV_EINVAL otherwise).  Every tile byte is loaded once, 16 bytes
 * per lane, with streaming (nontemporal) loads as the decode kernels read
 * K/V when streaming is nonzero, with plain loads otherwise (a plain pass
 * over an unrelated buffer is what leaves the caches full of other data);
 * sink (device uint32 [1]) is written only when the bytes' XOR hits
 * a fixed value (it keeps the loads alive).  tile_bytes a positive multiple of
 * 16, pools 16-byte aligned; tiles outside the pools are the caller's
 * contract. */
int paged_kv_read_tiles(const void* k_pool, const void* v_pool, const int64_t* tiles, int64_t n_k_tiles,
                        int64_t n_tiles, int64_t tile_bytes, int32_t streaming, uint32_t* sink, void* stream);

/* The matrix-core rate beside the chunked-prefill kernel, whose Q K^T and
 * P V products ("The detour, what really happens inside one forward pass",
 * Life of a prompt) are 16x16x32 bf16/fp16 MFMAs issued by two waves per SIMD
 * while the partner wave runs the softmax.  n_workgroups workgroups of 512
 * threads, one per CU, each of whose waves 0..3 issues iters x 8 independent
 * 16x16x32 bf16 MFMAs (16384 flops each); mode 0: waves 4..7 idle; mode 1:
 * waves 4..7 issue the same MFMAs; mode 2: waves 4..7 run, per eight partner
 * MFMAs, 4 exps and 14 other vector operations (the prefill softmax's mix);
 * mode 3: that vector work alone.  Matrix flops per launch: n_workgroups *
 * W * iters * 8 * 16384 with W = 8 in mode 1, 4 in modes 0 and 2, 0 in mode 3.
 * sink (device float [1]) is written only if a result hits a fixed value.
 * Errors: PKV_EINVAL for a mode outside 0..3, n_workgroups outside
 * [1, 65535], iters outside [1, 2^24] or a NULL sink. */
int paged_kv_mfma_rate(int32_t mode, int32_t n_workgroups, int32_t iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
