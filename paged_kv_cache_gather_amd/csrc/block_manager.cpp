// Host block manager: the free-block queue, per-block reference counts and
// per-sequence block tables of one KV pool, with optional automatic prefix
// caching.
//
// Rules (restated from the pages):
//  - a new block comes from the head of the free queue, and only when the
//    sequence's last block is full; finished sequences return their blocks at
//    once ("Back to the queue, and into vLLM proper", Life of a prompt;
//    "PagedAttention in depth", vLLM Serving deep dive);
//  - block tables may share physical blocks, counted by reference counts;
//    appending into a shared, partly filled block copies that block for the
//    appending sequence only ("Sharing and copy-on-write", vLLM Serving deep
//    dive);
//  - running out of blocks is reported, not fatal, and leaves the state as it
//    was so the caller can preempt ("The skeleton of a scheduler", LLM
//    Serving from Scratch);
//  - prefix caching ("Trick 3, Prefix caching", How AI actually answers you;
//    "Prefix caching (automatic KV reuse)", vLLM Serving deep dive; the
//    Automatic Prefix Caching paragraph of The hands-on guide to LLM
//    Inference with vLLM): a full block is labelled by a fingerprint of its
//    own tokens chained with the fingerprint of the block before it; a new
//    prompt reuses every leading full block whose label is known; only full
//    blocks are labelled; unused labelled blocks are thrown out least
//    recently used first;
//  - swapping ("The scheduler: waiting, running, swapped", vLLM Serving deep
//    dive; the CPU blocks of "Back to the queue, and into vLLM proper", Life
//    of a prompt): a preempted sequence's blocks are parked in a pool of
//    pinned host blocks and restored later.  The host blocks have their own
//    FIFO queue; swapping out gives each block of the sequence, in logical
//    order, a host block (a private copy, also of shared blocks) and releases
//    the GPU blocks as a finished sequence would; swapping in takes GPU
//    blocks from the head of the free queue and returns the host blocks to
//    their queue's tail.  Both are all or nothing.
//
// The free queue is a doubly linked list over block ids (a block is either
// queued or referenced, never both), so a cache hit can take a free block out
// of the middle.  A freed labelled block keeps its label while it waits in
// the queue; it loses the label only when the queue hands it out again, so
// the queue's FIFO order is the eviction order (least recently released
// first).  Every operation is O(blocks touched).
#include <algorithm>
#include <cstdint>
#include <deque>
#include <string>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

namespace {

thread_local std::string g_last_error;

struct Sequence {
  std::vector<int32_t> table;
  int64_t len = 0;
  // token ids of every position, while they are all known (sequences
  // created from tokens and extended with paged_kv_seq_append_tokens); the
  // fingerprints of the full blocks among them
  bool tracked = true;
  std::vector<int32_t> tokens;
  std::vector<uint64_t> fp;
  // swapped out: `table` holds host (CPU) block ids
  bool swapped = false;
};

// Fingerprint of a full block: a 64-bit chained mix of the previous block's
// fingerprint and the block's tokens (splitmix64 finaliser per token).  A
// lookup also compares the stored tokens and previous fingerprint, so a
// label match means equal tokens here and an equal chain before.
constexpr uint64_t kFpRoot = 0x243f6a8885a308d3ull;
uint64_t mix64(uint64_t x) {
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}
uint64_t block_fp(uint64_t prev, const int32_t* tok, int n) {
  uint64_t h = mix64(prev);
  for (int i = 0; i < n; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tok[i]);
  return h;
}

}  // namespace

namespace pkv {
int fail(int code, const std::string& msg) {
  g_last_error = msg;
  return code;
}
int ok() {
  g_last_error.clear();
  return PKV_OK;
}
}  // namespace pkv

struct pkv_pool {
  int64_t num_blocks = 0;
  int32_t block_size = 16;
  int32_t n_kv_heads = 0;
  int32_t head_dim = 0;
  int32_t dtype = 0;
  int32_t n_layers = 1;
  // free queue: doubly linked list, head first
  std::vector<int32_t> nxt, prv;
  int32_t qhead = -1, qtail = -1;
  int64_t count = 0;  // blocks in the queue
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Sequence> seqs;
  int64_t next_id = 0;
  // prefix cache: label -> block; per labelled block its label, the previous
  // block's label and its tokens
  bool caching = false;
  std::unordered_map<uint64_t, int32_t> labels;
  std::vector<char> labelled;
  std::vector<uint64_t> blabel, bprev;
  std::vector<int32_t> btok;
  int64_t queried = 0, hits = 0;
  // swap space: host blocks, FIFO
  int64_t num_cpu_blocks = 0;
  std::deque<int32_t> cpu_free;
  int64_t n_swapped = 0;
  std::mutex mu;

  void unlink(int32_t b) {
    const int32_t p = prv[b], n = nxt[b];
    if (p >= 0) nxt[p] = n; else qhead = n;
    if (n >= 0) prv[n] = p; else qtail = p;
    prv[b] = nxt[b] = -1;
    --count;
  }
  void push(int32_t b) {
    prv[b] = qtail;
    nxt[b] = -1;
    if (qtail >= 0) nxt[qtail] = b; else qhead = b;
    qtail = b;
    ++count;
  }
  void drop_label(int32_t b) {
    if (!labelled.empty() && labelled[b]) {
      auto it = labels.find(blabel[b]);
      if (it != labels.end() && it->second == b) labels.erase(it);
      labelled[b] = 0;
    }
  }
  int32_t pop() {
    const int32_t b = qhead;
    unlink(b);
    drop_label(b);  // evicted: the block is about to hold new data
    ref[b] = 1;
    return b;
  }
  int64_t need(const Sequence& s, int64_t n) const {
    const int64_t L = s.len, bs = block_size;
    int64_t blocks = (L + n + bs - 1) / bs - (L + bs - 1) / bs;
    if (n > 0 && L % bs != 0 && ref[s.table[L / bs]] > 1) ++blocks;
    return blocks;
  }
  // label the full blocks of s from index `from` on (its tokens are known)
  void label_full_blocks(Sequence& s, int64_t from) {
    const int64_t bs = block_size, nfull = s.len / bs;
    for (int64_t i = (int64_t)s.fp.size(); i < nfull; ++i) {
      const uint64_t prev = i ? s.fp[i - 1] : kFpRoot;
      s.fp.push_back(block_fp(prev, s.tokens.data() + i * bs, (int)bs));
    }
    if (!caching) return;
    for (int64_t i = from; i < nfull; ++i) {
      const int32_t b = s.table[i];
      if (labelled[b] || labels.count(s.fp[i])) continue;  // already known content
      labels.emplace(s.fp[i], b);
      labelled[b] = 1;
      blabel[b] = s.fp[i];
      bprev[b] = i ? s.fp[i - 1] : kFpRoot;
      std::copy(s.tokens.begin() + i * bs, s.tokens.begin() + (i + 1) * bs, btok.begin() + (int64_t)b * bs);
    }
  }
};

using pkv::fail;
using pkv::ok;

extern "C" {

const char* pkv_last_error(void) { return g_last_error.c_str(); }

int paged_kv_bytes_per_token(int32_t n_layers, int32_t n_kv_heads, int32_t head_dim,
                             int32_t dtype, int64_t* bytes) {
  const int es = pkv::esize_of(dtype);
  if (!bytes || n_layers <= 0 || n_kv_heads <= 0 || head_dim <= 0 || !es)
    return fail(PKV_EINVAL, "paged_kv_bytes_per_token: bad argument");
  *bytes = 2ll * n_layers * n_kv_heads * head_dim * es;
  return ok();
}

int paged_kv_blocks_for_budget(int64_t budget_bytes, int32_t n_layers, int32_t n_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t dtype,
                               int64_t* num_blocks) {
  int64_t per_token = 0;
  if (!num_blocks || budget_bytes < 0 || block_size <= 0)
    return fail(PKV_EINVAL, "paged_kv_blocks_for_budget: bad argument");
  int rc = paged_kv_bytes_per_token(n_layers, n_kv_heads, head_dim, dtype, &per_token);
  if (rc) return rc;
  *num_blocks = budget_bytes / (per_token * block_size);
  return ok();
}

static int check_desc(const pkv_pool_desc* d) {
  if (!d) return fail(PKV_EINVAL, "pool descriptor is NULL");
  if (d->num_blocks < 1 || d->num_blocks > INT32_MAX)
    return fail(PKV_EINVAL, "num_blocks must be in [1, 2^31)");
  if (d->block_size != pkv::kBlockSize)
    return fail(PKV_EUNSUPPORTED, "block_size must be 16");
  if (d->n_kv_heads < 1 || d->n_layers < 1 || d->reserved != 0)
    return fail(PKV_EINVAL, "n_kv_heads and n_layers must be >= 1, reserved 0");
  if (!pkv::esize_of(d->dtype)) return fail(PKV_EINVAL, "unknown dtype");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "head_dim must be 64 or 128");
  return PKV_OK;
}

int paged_kv_pool_bytes(const pkv_pool_desc* desc, int64_t* k_bytes, int64_t* v_bytes) {
  int rc = check_desc(desc);
  if (rc) return rc;
  const int64_t b = desc->num_blocks * desc->n_kv_heads * desc->block_size * desc->head_dim *
                    pkv::esize_of(desc->dtype);
  if (k_bytes) *k_bytes = b;
  if (v_bytes) *v_bytes = b;
  return ok();
}

int paged_kv_alloc(const pkv_pool_desc* desc, pkv_pool** out) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!out) return fail(PKV_EINVAL, "out is NULL");
  pkv_pool* p = new (std::nothrow) pkv_pool();
  if (!p) return fail(PKV_EINVAL, "host allocation failed");
  p->num_blocks = desc->num_blocks;
  p->block_size = desc->block_size;
  p->n_kv_heads = desc->n_kv_heads;
  p->head_dim = desc->head_dim;
  p->dtype = desc->dtype;
  p->n_layers = desc->n_layers;
  try {
    p->nxt.assign(p->num_blocks, -1);
    p->prv.assign(p->num_blocks, -1);
    p->ref.assign(p->num_blocks, 0);
  } catch (...) {
    delete p;
    return fail(PKV_EINVAL, "host allocation failed");
  }
  if (desc->initial_free_order) {
    std::vector<char> seen(p->num_blocks, 0);
    for (int64_t i = 0; i < p->num_blocks; ++i) {
      const int32_t b = desc->initial_free_order[i];
      if (b < 0 || b >= p->num_blocks || seen[b]) {
        delete p;
        return fail(PKV_EINVAL, "initial_free_order is not a permutation of the pool");
      }
      seen[b] = 1;
    }
    for (int64_t i = 0; i < p->num_blocks; ++i) p->push(desc->initial_free_order[i]);
  } else {
    for (int64_t i = 0; i < p->num_blocks; ++i) p->push((int32_t)i);
  }
  *out = p;
  return ok();
}

int paged_kv_destroy(pkv_pool* pool) {
  if (!pool) return fail(PKV_EINVAL, "pool is NULL");
  delete pool;
  return ok();
}

int paged_kv_seq_create(pkv_pool* pool, int64_t* seq) {
  if (!pool || !seq) return fail(PKV_EINVAL, "paged_kv_seq_create: NULL argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  const int64_t id = pool->next_id++;
  pool->seqs.emplace(id, Sequence{});
  *seq = id;
  return ok();
}

int paged_kv_seq_fork(pkv_pool* pool, int64_t parent, int64_t n_prefix_tokens, int64_t* child) {
  if (!pool || !child) return fail(PKV_EINVAL, "paged_kv_seq_fork: NULL argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(parent);
  if (it == pool->seqs.end()) return fail(PKV_ESTATE, "paged_kv_seq_fork: unknown parent");
  if (it->second.swapped) return fail(PKV_ESTATE, "paged_kv_seq_fork: parent is swapped out");
  if (n_prefix_tokens < 0 || n_prefix_tokens > it->second.len)
    return fail(PKV_EINVAL, "paged_kv_seq_fork: prefix longer than the parent");
  const int64_t nb = (n_prefix_tokens + pool->block_size - 1) / pool->block_size;
  Sequence s;
  s.table.assign(it->second.table.begin(), it->second.table.begin() + nb);
  s.len = n_prefix_tokens;
  s.tracked = it->second.tracked;
  if (s.tracked) {
    s.tokens.assign(it->second.tokens.begin(), it->second.tokens.begin() + n_prefix_tokens);
    s.fp.assign(it->second.fp.begin(), it->second.fp.begin() + n_prefix_tokens / pool->block_size);
  }
  for (int32_t b : s.table) ++pool->ref[b];
  const int64_t id = pool->next_id++;
  pool->seqs.emplace(id, std::move(s));
  *child = id;
  return ok();
}

int paged_kv_seq_blocks_needed(pkv_pool* pool, int64_t seq, int64_t n_tokens, int64_t* n_blocks) {
  if (!pool || !n_blocks) return fail(PKV_EINVAL, "paged_kv_seq_blocks_needed: NULL argument");
  if (n_tokens < 0) return fail(PKV_EINVAL, "n_tokens < 0");
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ESTATE, "unknown sequence");
  if (it->second.swapped) return fail(PKV_ESTATE, "paged_kv_seq_blocks_needed: sequence is swapped out");
  *n_blocks = pool->need(it->second, n_tokens);
  return ok();
}

// The append of n_tokens to s, the pool's lock held: all or nothing (the
// checks come before any change).  Writes the slots, and at most one
// copy-on-write pair if max_cow allows it; *n_cow receives 0 or 1.
static int append_locked(const std::string& F, pkv_pool* pool, Sequence& s, const int32_t* tokens,
                         int64_t n_tokens, int64_t* slot_mapping_out, int32_t* cow_pairs_out, int32_t max_cow,
                         int32_t* n_cow) {
  if (s.swapped) return fail(PKV_ESTATE, F + ": sequence is swapped out");
  const int64_t bs = pool->block_size;
  const int64_t L = s.len;
  const bool cow = n_tokens > 0 && L % bs != 0 && pool->ref[s.table[L / bs]] > 1;
  if (cow && max_cow < 1)
    return fail(PKV_EINVAL, F + ": the append needs a copy-on-write pair and max_cow leaves no room");
  const int64_t need = pool->need(s, n_tokens);
  if (need > pool->count)
    return fail(PKV_ENOMEM_BLOCKS, "out of KV blocks: need " + std::to_string(need) + ", free " +
                                       std::to_string(pool->count));
  int32_t ncow = 0;
  if (cow) {
    const int32_t old = s.table[L / bs];
    const int32_t fresh = pool->pop();
    --pool->ref[old];
    s.table[L / bs] = fresh;
    cow_pairs_out[0] = old;
    cow_pairs_out[1] = fresh;
    ncow = 1;
  }
  s.table.reserve((L + n_tokens + bs - 1) / bs);
  for (int64_t t = L; t < L + n_tokens; ++t) {
    if (t % bs == 0) s.table.push_back(pool->pop());
    if (slot_mapping_out) slot_mapping_out[t - L] = (int64_t)s.table[t / bs] * bs + t % bs;
  }
  s.len = L + n_tokens;
  if (tokens && s.tracked) {
    s.tokens.insert(s.tokens.end(), tokens, tokens + n_tokens);
    pool->label_full_blocks(s, L / bs);
  } else if (n_tokens > 0) {
    s.tracked = false;  // contents unknown from here on: nothing of it is labelled
    s.tokens.clear();
    s.tokens.shrink_to_fit();
  }
  *n_cow = ncow;
  return ok();
}

static int append_impl(const char* fn, pkv_pool* pool, int64_t seq, const int32_t* tokens, int64_t n_tokens,
                       int64_t* slot_mapping_out, int32_t* cow_pairs_out, int32_t max_cow, int32_t* n_cow) {
  const std::string F(fn);
  if (!pool) return fail(PKV_EINVAL, F + ": pool is NULL");
  if (n_tokens < 0) return fail(PKV_EINVAL, F + ": n_tokens < 0");
  if (max_cow < 0 || (max_cow > 0 && !cow_pairs_out))
    return fail(PKV_EINVAL, F + ": cow_pairs_out is NULL with max_cow > 0");
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ESTATE, F + ": unknown sequence");
  int32_t ncow = 0;
  const int rc = append_locked(F, pool, it->second, tokens, n_tokens, slot_mapping_out, cow_pairs_out, max_cow,
                               &ncow);
  if (rc == PKV_OK && n_cow) *n_cow = ncow;
  return rc;
}

int paged_kv_seqs_append(pkv_pool* pool, const int64_t* seqs, int32_t n, const int64_t* n_tokens,
                         int64_t* slot_mapping_out, int32_t* cow_pairs_out, int32_t max_cow, int32_t* n_cow,
                         int32_t* n_done) {
  const std::string F("paged_kv_seqs_append");
  if (n_done) *n_done = 0;
  if (n_cow) *n_cow = 0;
  if (!pool) return fail(PKV_EINVAL, F + ": pool is NULL");
  if (n < 0 || (n > 0 && !seqs)) return fail(PKV_EINVAL, F + ": bad sequence list");
  if (max_cow < 0 || (max_cow > 0 && !cow_pairs_out))
    return fail(PKV_EINVAL, F + ": cow_pairs_out is NULL with max_cow > 0");
  if (n_tokens)
    for (int32_t i = 0; i < n; ++i)
      if (n_tokens[i] < 0) return fail(PKV_EINVAL, F + ": n_tokens < 0");
  std::lock_guard<std::mutex> lk(pool->mu);
  int64_t off = 0;
  int32_t ncow = 0;
  for (int32_t i = 0; i < n; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end()) return fail(PKV_ESTATE, F + ": unknown sequence " + std::to_string(seqs[i]));
    const int64_t nt = n_tokens ? n_tokens[i] : 1;
    int32_t c = 0;
    const int rc = append_locked(F, pool, it->second, nullptr, nt, slot_mapping_out ? slot_mapping_out + off : nullptr,
                                 cow_pairs_out ? cow_pairs_out + 2 * ncow : nullptr, max_cow - ncow, &c);
    if (rc != PKV_OK) return rc;  // sequences 0 .. i-1 stay appended and reported
    off += nt;
    ncow += c;
    if (n_cow) *n_cow = ncow;
    if (n_done) *n_done = i + 1;
  }
  return ok();
}

int paged_kv_seq_append(pkv_pool* pool, int64_t seq, int64_t n_tokens, int64_t* slot_mapping_out,
                        int32_t* cow_pairs_out, int32_t max_cow, int32_t* n_cow) {
  return append_impl("paged_kv_seq_append", pool, seq, nullptr, n_tokens, slot_mapping_out, cow_pairs_out,
                     max_cow, n_cow);
}

int paged_kv_seq_append_tokens(pkv_pool* pool, int64_t seq, const int32_t* tokens, int64_t n_tokens,
                               int64_t* slot_mapping_out, int32_t* cow_pairs_out, int32_t max_cow,
                               int32_t* n_cow) {
  if (n_tokens > 0 && !tokens) return fail(PKV_EINVAL, "paged_kv_seq_append_tokens: tokens is NULL");
  return append_impl("paged_kv_seq_append_tokens", pool, seq, tokens, n_tokens, slot_mapping_out,
                     cow_pairs_out, max_cow, n_cow);
}

int paged_kv_prefix_cache_enable(pkv_pool* pool, int32_t enable) {
  if (!pool) return fail(PKV_EINVAL, "pool is NULL");
  std::lock_guard<std::mutex> lk(pool->mu);
  if (enable && !pool->caching) {
    try {
      pool->labelled.assign(pool->num_blocks, 0);
      pool->blabel.assign(pool->num_blocks, 0);
      pool->bprev.assign(pool->num_blocks, 0);
      pool->btok.assign(pool->num_blocks * pool->block_size, 0);
    } catch (...) {
      return fail(PKV_EINVAL, "paged_kv_prefix_cache_enable: host allocation failed");
    }
    pool->caching = true;
  } else if (!enable && pool->caching) {
    pool->labels.clear();
    std::vector<char>().swap(pool->labelled);
    std::vector<uint64_t>().swap(pool->blabel);
    std::vector<uint64_t>().swap(pool->bprev);
    std::vector<int32_t>().swap(pool->btok);
    pool->caching = false;
  }
  return ok();
}

int paged_kv_seq_create_cached(pkv_pool* pool, const int32_t* tokens, int64_t n_tokens, int64_t* seq,
                               int64_t* n_cached) {
  if (!pool || !seq || !n_cached || (n_tokens > 0 && !tokens) || n_tokens < 0)
    return fail(PKV_EINVAL, "paged_kv_seq_create_cached: bad argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  const int64_t bs = pool->block_size;
  Sequence s;
  if (pool->caching && n_tokens > 0) {
    const int64_t nq = (n_tokens - 1) / bs;  // the last token is always computed
    uint64_t prev = kFpRoot;
    for (int64_t i = 0; i < nq; ++i) {
      const int32_t* tk = tokens + i * bs;
      const uint64_t fp = block_fp(prev, tk, (int)bs);
      ++pool->queried;
      auto hit = pool->labels.find(fp);
      if (hit == pool->labels.end()) break;
      const int32_t b = hit->second;
      if (pool->bprev[b] != prev || !std::equal(tk, tk + bs, pool->btok.begin() + (int64_t)b * bs)) break;
      ++pool->hits;
      if (pool->ref[b] == 0) pool->unlink(b);  // an unused cached block leaves the free queue
      ++pool->ref[b];
      s.table.push_back(b);
      s.fp.push_back(fp);
      prev = fp;
    }
  }
  s.len = (int64_t)s.table.size() * bs;
  s.tokens.assign(tokens, tokens + s.len);
  const int64_t id = pool->next_id++;
  pool->seqs.emplace(id, std::move(s));
  *seq = id;
  *n_cached = (int64_t)pool->seqs[id].len;
  return ok();
}

int paged_kv_prefix_cache_stats(pkv_pool* pool, int64_t* cached_blocks, int64_t* queried_blocks,
                                int64_t* hit_blocks) {
  if (!pool) return fail(PKV_EINVAL, "pool is NULL");
  std::lock_guard<std::mutex> lk(pool->mu);
  if (cached_blocks) *cached_blocks = (int64_t)pool->labels.size();
  if (queried_blocks) *queried_blocks = pool->queried;
  if (hit_blocks) *hit_blocks = pool->hits;
  return ok();
}

int paged_kv_seq_free(pkv_pool* pool, int64_t seq) {
  if (!pool) return fail(PKV_EINVAL, "pool is NULL");
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ESTATE, "paged_kv_seq_free: unknown sequence");
  if (it->second.swapped) {  // its host blocks rejoin their queue
    for (int32_t c : it->second.table) pool->cpu_free.push_back(c);
    --pool->n_swapped;
  } else {
    for (int32_t b : it->second.table) {
      if (--pool->ref[b] == 0) pool->push(b);
    }
  }
  pool->seqs.erase(it);
  return ok();
}

int paged_kv_swap_space(pkv_pool* pool, int64_t num_cpu_blocks) {
  if (!pool) return fail(PKV_EINVAL, "pool is NULL");
  if (num_cpu_blocks < 0 || num_cpu_blocks > INT32_MAX)
    return fail(PKV_EINVAL, "paged_kv_swap_space: num_cpu_blocks must be in [0, 2^31)");
  std::lock_guard<std::mutex> lk(pool->mu);
  if (pool->n_swapped) return fail(PKV_ESTATE, "paged_kv_swap_space: sequences are swapped out");
  pool->num_cpu_blocks = num_cpu_blocks;
  pool->cpu_free.clear();
  for (int64_t c = 0; c < num_cpu_blocks; ++c) pool->cpu_free.push_back((int32_t)c);
  return ok();
}

int paged_kv_seq_swap_out(pkv_pool* pool, int64_t seq, int32_t* pairs_out, int64_t cap, int64_t* n_pairs) {
  if (!pool || !n_pairs) return fail(PKV_EINVAL, "paged_kv_seq_swap_out: NULL argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ESTATE, "paged_kv_seq_swap_out: unknown sequence");
  Sequence& s = it->second;
  if (s.swapped) return fail(PKV_ESTATE, "paged_kv_seq_swap_out: already swapped out");
  const int64_t n = (int64_t)s.table.size();
  if (n > 0 && (!pairs_out || cap < n))
    return fail(PKV_EINVAL, "paged_kv_seq_swap_out: pairs_out holds fewer than " + std::to_string(n) + " pairs");
  if (n > (int64_t)pool->cpu_free.size())
    return fail(PKV_ENOMEM_BLOCKS, "out of CPU blocks: need " + std::to_string(n) + ", free " +
                                       std::to_string(pool->cpu_free.size()));
  for (int64_t i = 0; i < n; ++i) {
    const int32_t c = pool->cpu_free.front();
    pool->cpu_free.pop_front();
    pairs_out[2 * i] = s.table[i];
    pairs_out[2 * i + 1] = c;
  }
  for (int64_t i = 0; i < n; ++i) {  // release the GPU blocks, in logical order
    const int32_t b = s.table[i];
    if (--pool->ref[b] == 0) pool->push(b);
    s.table[i] = pairs_out[2 * i + 1];
  }
  s.swapped = true;
  ++pool->n_swapped;
  *n_pairs = n;
  return ok();
}

int paged_kv_seq_swap_in(pkv_pool* pool, int64_t seq, int32_t* pairs_out, int64_t cap, int64_t* n_pairs) {
  if (!pool || !n_pairs) return fail(PKV_EINVAL, "paged_kv_seq_swap_in: NULL argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ESTATE, "paged_kv_seq_swap_in: unknown sequence");
  Sequence& s = it->second;
  if (!s.swapped) return fail(PKV_ESTATE, "paged_kv_seq_swap_in: not swapped out");
  const int64_t n = (int64_t)s.table.size();
  if (n > 0 && (!pairs_out || cap < n))
    return fail(PKV_EINVAL, "paged_kv_seq_swap_in: pairs_out holds fewer than " + std::to_string(n) + " pairs");
  if (n > pool->count)
    return fail(PKV_ENOMEM_BLOCKS, "out of KV blocks: need " + std::to_string(n) + ", free " +
                                       std::to_string(pool->count));
  for (int64_t i = 0; i < n; ++i) {
    const int32_t c = s.table[i];
    const int32_t g = pool->pop();
    pairs_out[2 * i] = c;
    pairs_out[2 * i + 1] = g;
    s.table[i] = g;
    pool->cpu_free.push_back(c);
  }
  s.swapped = false;
  --pool->n_swapped;
  if (s.tracked) pool->label_full_blocks(s, 0);
  *n_pairs = n;
  return ok();
}

int paged_kv_seq_is_swapped(pkv_pool* pool, int64_t seq, int32_t* swapped) {
  if (!pool || !swapped) return fail(PKV_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ESTATE, "unknown sequence");
  *swapped = it->second.swapped ? 1 : 0;
  return ok();
}

int paged_kv_cpu_free_queue(pkv_pool* pool, int32_t* out, int64_t cap, int64_t* n) {
  if (!pool || !n) return fail(PKV_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  *n = (int64_t)pool->cpu_free.size();
  if (!out) return ok();
  if (cap < *n) return fail(PKV_EINVAL, "paged_kv_cpu_free_queue: cap too small");
  std::copy(pool->cpu_free.begin(), pool->cpu_free.end(), out);
  return ok();
}

int paged_kv_seq_len(pkv_pool* pool, int64_t seq, int64_t* len) {
  if (!pool || !len) return fail(PKV_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ESTATE, "unknown sequence");
  *len = it->second.len;
  return ok();
}

int paged_kv_seq_table(pkv_pool* pool, int64_t seq, int32_t* blocks_out, int64_t cap, int64_t* n) {
  if (!pool || !n) return fail(PKV_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->seqs.find(seq);
  if (it == pool->seqs.end()) return fail(PKV_ESTATE, "unknown sequence");
  const auto& t = it->second.table;
  *n = (int64_t)t.size();
  if (!blocks_out) return ok();
  if (cap < (int64_t)t.size()) return fail(PKV_EINVAL, "paged_kv_seq_table: cap too small");
  std::copy(t.begin(), t.end(), blocks_out);
  return ok();
}

int paged_kv_block_tables(pkv_pool* pool, const int64_t* seqs, int32_t n, int32_t max_blocks,
                          int32_t* tables_out, int32_t* lens_out) {
  if (!pool || (n > 0 && (!seqs || !tables_out)) || n < 0 || max_blocks < 0)
    return fail(PKV_EINVAL, "paged_kv_block_tables: bad argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  for (int32_t i = 0; i < n; ++i) {
    auto it = pool->seqs.find(seqs[i]);
    if (it == pool->seqs.end()) return fail(PKV_ESTATE, "paged_kv_block_tables: unknown sequence");
    if (it->second.swapped) return fail(PKV_ESTATE, "paged_kv_block_tables: a sequence is swapped out");
    if ((int64_t)it->second.table.size() > max_blocks)
      return fail(PKV_EINVAL, "paged_kv_block_tables: table longer than max_blocks");
    if (it->second.len > INT32_MAX) return fail(PKV_EINVAL, "sequence too long for int32 lens");
  }
  for (int32_t i = 0; i < n; ++i) {
    const Sequence& s = pool->seqs.find(seqs[i])->second;
    int32_t* row = tables_out + (int64_t)i * max_blocks;
    std::fill(row, row + max_blocks, -1);
    std::copy(s.table.begin(), s.table.end(), row);
    if (lens_out) lens_out[i] = (int32_t)s.len;
  }
  return ok();
}

int paged_kv_num_free(pkv_pool* pool, int64_t* n) {
  if (!pool || !n) return fail(PKV_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  *n = pool->count;
  return ok();
}

int paged_kv_block_refcount(pkv_pool* pool, int64_t block, int32_t* ref) {
  if (!pool || !ref) return fail(PKV_EINVAL, "NULL argument");
  if (block < 0 || block >= pool->num_blocks) return fail(PKV_EINVAL, "block outside the pool");
  std::lock_guard<std::mutex> lk(pool->mu);
  *ref = pool->ref[block];
  return ok();
}

int paged_kv_free_queue(pkv_pool* pool, int32_t* out, int64_t cap, int64_t* n) {
  if (!pool || !n) return fail(PKV_EINVAL, "NULL argument");
  std::lock_guard<std::mutex> lk(pool->mu);
  *n = pool->count;
  if (!out) return ok();
  if (cap < pool->count) return fail(PKV_EINVAL, "paged_kv_free_queue: cap too small");
  int64_t i = 0;
  for (int32_t b = pool->qhead; b >= 0; b = pool->nxt[b]) out[i++] = b;
  return ok();
}

}  // extern "C"
