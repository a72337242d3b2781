// Host-only driver for the sanitizer build: the block manager of the C ABI
// (block_manager.cpp) and the test oracle (oracle/oracle.c), compiled with
// AddressSanitizer and UndefinedBehaviorSanitizer, exercised with seeded
// random operation sequences, bad arguments and edge-case inputs.  Every
// invariant the allocator states is checked after each operation; any
// memory or UB error aborts the run with the sanitizer's report.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "pagedkv.h"

extern "C" {
int orc_decode(int dtype, const void* src, int64_t n, double* dst);
int64_t orc_slot(const int32_t* table, int64_t t, int32_t bs);
int orc_gather(int dtype, const void* k_pool, const void* v_pool, int64_t num_blocks, int32_t bs, int32_t H,
               int32_t d, const int32_t* table, int64_t n_table, int64_t n_tokens, double* k_out, double* v_out);
int orc_scatter(int dtype, const void* key, const void* value, int64_t n_tokens, int64_t key_stride,
                int64_t value_stride, void* k_pool, void* v_pool, const int64_t* slots, int64_t num_blocks, int32_t bs,
                int32_t H, int32_t d);
int orc_copy_blocks(int dtype, void* k_pool, void* v_pool, const int32_t* pairs, int64_t n, int64_t num_blocks,
                    int32_t bs, int32_t H, int32_t d);
int orc_swap_blocks(int dtype, const void* src_k, const void* src_v, int64_t src_num_blocks, void* dst_k, void* dst_v,
                    int64_t dst_num_blocks, const int32_t* pairs, int64_t n, int32_t bs, int32_t H, int32_t d);
int orc_attention(int64_t n_rows, const double* q, const int64_t* q_pos, int64_t n_keys, const double* k,
                  const double* v, int32_t Hq, int32_t Hkv, int32_t d, double scale, double* out, double* wsum,
                  double* scratch, int32_t n_threads);
int orc_quantize_e4m3(const float* x, int64_t n, float inv_scale, uint8_t* out);
}

static int g_fail = 0;
#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      std::fprintf(stderr, "CHECK failed at line %d: %s\n", __LINE__, #c);    \
      g_fail = 1;                                                             \
      std::exit(2);                                                           \
    }                                                                         \
  } while (0)

struct Seq {
  int64_t id;
  bool swapped;
};

// After every operation: blocks held (reference count > 0) plus the free
// queue make up the pool, every free-queue entry is a block with count 0, and
// each sequence's table has ceil(len / 16) entries.
static void check_invariants(pkv_pool* p, int64_t nb, const std::vector<Seq>& seqs) {
  int64_t nfree = -1;
  CHECK(paged_kv_num_free(p, &nfree) == PKV_OK);
  std::vector<int32_t> q(nb + 1);
  int64_t qn = -1;
  CHECK(paged_kv_free_queue(p, q.data(), nb + 1, &qn) == PKV_OK);
  CHECK(qn == nfree);
  int64_t held = 0;
  for (int64_t b = 0; b < nb; ++b) {
    int32_t r = -1;
    CHECK(paged_kv_block_refcount(p, b, &r) == PKV_OK);
    CHECK(r >= 0);
    held += r > 0;
  }
  CHECK(held + nfree == nb);
  for (int64_t i = 0; i < qn; ++i) {
    int32_t r = -1;
    CHECK(paged_kv_block_refcount(p, q[i], &r) == PKV_OK && r == 0);
  }
  for (const Seq& s : seqs) {
    int64_t len = -1, n = -1;
    CHECK(paged_kv_seq_len(p, s.id, &len) == PKV_OK);
    CHECK(paged_kv_seq_table(p, s.id, nullptr, 0, &n) == PKV_OK || n >= 0);
    std::vector<int32_t> t(n > 0 ? n : 1);
    CHECK(paged_kv_seq_table(p, s.id, t.data(), n, &n) == PKV_OK);
    CHECK(n == (len + 15) / 16);
  }
}

static void fuzz_block_manager(uint64_t seed, int steps) {
  std::mt19937_64 rng(seed);
  auto rnd = [&](int64_t a, int64_t b) { return std::uniform_int_distribution<int64_t>(a, b)(rng); };
  const int64_t nb = rnd(8, 96);
  std::vector<int32_t> order(nb);
  for (int64_t i = 0; i < nb; ++i) order[i] = (int32_t)i;
  std::shuffle(order.begin(), order.end(), rng);
  pkv_pool_desc d{};
  d.num_blocks = nb;
  d.block_size = 16;
  d.n_kv_heads = 2;
  d.head_dim = 64;
  d.dtype = PKV_F16;
  d.n_layers = 1;
  d.initial_free_order = rnd(0, 1) ? order.data() : nullptr;
  pkv_pool* p = nullptr;
  CHECK(paged_kv_alloc(&d, &p) == PKV_OK && p);
  std::vector<Seq> seqs;
  std::vector<std::vector<int32_t>> prompts;
  for (int f = 0; f < 3; ++f) {  // token families, so that cached prefixes recur
    std::vector<int32_t> t(200);
    for (auto& x : t) x = (int32_t)rnd(0, 20);
    prompts.push_back(t);
  }
  int swap_cap = 0;
  for (int step = 0; step < steps; ++step) {
    const int op = (int)rnd(0, 13);
    const int64_t pick = seqs.empty() ? -1 : rnd(0, (int64_t)seqs.size() - 1);
    int rc = PKV_OK;
    if (op == 0 || seqs.empty()) {
      int64_t id = -1;
      CHECK(paged_kv_seq_create(p, &id) == PKV_OK);
      seqs.push_back({id, false});
    } else if (op == 1) {  // fork
      Seq& s = seqs[pick];
      int64_t len = 0, child = -1;
      paged_kv_seq_len(p, s.id, &len);
      rc = paged_kv_seq_fork(p, s.id, rnd(0, len), &child);
      if (rc == PKV_OK) seqs.push_back({child, false});
      else CHECK(s.swapped);
    } else if (op == 2 || op == 3) {  // append
      Seq& s = seqs[pick];
      const int64_t n = rnd(0, 40);
      std::vector<int64_t> slots(n + 1);
      int32_t cow[2];
      int32_t ncow = -1;
      rc = paged_kv_seq_append(p, s.id, n, slots.data(), cow, 1, &ncow);
      CHECK(rc == PKV_OK || rc == PKV_ENOMEM_BLOCKS || (rc == PKV_ESTATE && s.swapped));
    } else if (op == 4) {  // batched append
      std::vector<int64_t> ids, counts;
      for (auto& s : seqs)
        if (!s.swapped && rnd(0, 1)) {
          ids.push_back(s.id);
          counts.push_back(rnd(0, 20));
        }
      int64_t tot = 0;
      for (auto c : counts) tot += c;
      std::vector<int64_t> slots(tot + 1);
      std::vector<int32_t> cow(2 * (ids.size() + 1));
      int32_t ncow = -1, ndone = -1;
      rc = paged_kv_seqs_append(p, ids.data(), (int32_t)ids.size(), counts.data(), slots.data(), cow.data(),
                                (int32_t)ids.size() + 1, &ncow, &ndone);
      CHECK(rc == PKV_OK || rc == PKV_ENOMEM_BLOCKS);
      CHECK(ndone >= 0 && ndone <= (int32_t)ids.size());
    } else if (op == 5) {  // free
      rc = paged_kv_seq_free(p, seqs[pick].id);
      CHECK(rc == PKV_OK);
      seqs.erase(seqs.begin() + pick);
    } else if (op == 6) {  // cached prompt
      const auto& t = prompts[rnd(0, 2)];
      const int64_t n = rnd(0, (int64_t)t.size());
      int64_t id = -1, cached = -1;
      CHECK(paged_kv_seq_create_cached(p, t.data(), n, &id, &cached) == PKV_OK);
      CHECK(cached >= 0 && cached <= n && cached % 16 == 0);
      seqs.push_back({id, false});
      std::vector<int64_t> slots(n - cached + 1);
      int32_t cow[2];
      int32_t ncow = -1;
      rc = paged_kv_seq_append_tokens(p, id, t.data() + cached, n - cached, slots.data(), cow, 1, &ncow);
      CHECK(rc == PKV_OK || rc == PKV_ENOMEM_BLOCKS);
    } else if (op == 7) {
      CHECK(paged_kv_prefix_cache_enable(p, (int32_t)rnd(0, 3) != 0) == PKV_OK);
    } else if (op == 8) {  // swap space
      const int64_t n = rnd(0, 64);
      bool any = false;
      for (auto& s : seqs) any |= s.swapped;
      rc = paged_kv_swap_space(p, n);
      CHECK(any ? rc == PKV_ESTATE : rc == PKV_OK);
      if (rc == PKV_OK) swap_cap = (int)n;
    } else if (op == 9) {  // swap out / in
      Seq& s = seqs[pick];
      std::vector<int32_t> pairs(2 * (nb + swap_cap + 1));
      int64_t np = -1;
      if (!s.swapped) {
        rc = paged_kv_seq_swap_out(p, s.id, pairs.data(), nb + swap_cap + 1, &np);
        CHECK(rc == PKV_OK || rc == PKV_ENOMEM_BLOCKS);
        if (rc == PKV_OK) s.swapped = true;
      } else {
        rc = paged_kv_seq_swap_in(p, s.id, pairs.data(), nb + swap_cap + 1, &np);
        CHECK(rc == PKV_OK || rc == PKV_ENOMEM_BLOCKS);
        if (rc == PKV_OK) s.swapped = false;
      }
    } else if (op == 10) {  // export tables
      std::vector<int64_t> ids;
      for (auto& s : seqs)
        if (!s.swapped) ids.push_back(s.id);
      const int32_t mb = (int32_t)rnd(0, 20);
      std::vector<int32_t> tab(ids.size() * (mb > 0 ? mb : 1) + 1), lens(ids.size() + 1);
      rc = paged_kv_block_tables(p, ids.data(), (int32_t)ids.size(), mb, tab.data(), lens.data());
      CHECK(rc == PKV_OK || rc == PKV_EINVAL);
    } else if (op == 11) {  // bad arguments: every one rejected, nothing changes
      int64_t x = 0;
      int32_t r = 0;
      CHECK(paged_kv_seq_append(p, 1ll << 40, 1, nullptr, nullptr, 0, nullptr) != PKV_OK);
      CHECK(paged_kv_seq_append(p, seqs[pick].id, -1, nullptr, nullptr, 0, nullptr) != PKV_OK);
      CHECK(paged_kv_seq_fork(p, -5, 0, &x) != PKV_OK);
      CHECK(paged_kv_seq_free(p, 1ll << 40) != PKV_OK);
      CHECK(paged_kv_block_refcount(p, nb, &r) != PKV_OK);
      CHECK(paged_kv_block_refcount(p, -1, &r) != PKV_OK);
      CHECK(paged_kv_seq_len(nullptr, 0, &x) != PKV_OK);
      CHECK(paged_kv_seqs_append(p, nullptr, 3, nullptr, nullptr, nullptr, 0, nullptr, nullptr) != PKV_OK);
      CHECK(paged_kv_seq_create_cached(p, nullptr, 5, &x, &x) != PKV_OK);
      CHECK(std::strlen(pkv_last_error()) > 0);
    } else {  // blocks needed
      Seq& s = seqs[pick];
      int64_t need = -1;
      rc = paged_kv_seq_blocks_needed(p, s.id, rnd(0, 50), &need);
      CHECK(rc == PKV_OK ? need >= 0 : s.swapped);
    }
    check_invariants(p, nb, seqs);
  }
  int64_t st[3];
  CHECK(paged_kv_prefix_cache_stats(p, &st[0], &st[1], &st[2]) == PKV_OK);
  CHECK(paged_kv_destroy(p) == PKV_OK);
}

static void exercise_oracle(uint64_t seed) {
  std::mt19937_64 rng(seed);
  std::normal_distribution<double> nd;
  auto rnd = [&](int64_t a, int64_t b) { return std::uniform_int_distribution<int64_t>(a, b)(rng); };
  // decoders on every 16-bit pattern and random words
  std::vector<uint16_t> h(65536);
  for (int i = 0; i < 65536; ++i) h[i] = (uint16_t)i;
  std::vector<double> dv(65536);
  CHECK(orc_decode(1, h.data(), 65536, dv.data()) == 0);
  CHECK(orc_decode(2, h.data(), 65536, dv.data()) == 0);
  std::vector<uint8_t> b8(256);
  for (int i = 0; i < 256; ++i) b8[i] = (uint8_t)i;
  CHECK(orc_decode(3, b8.data(), 256, dv.data()) == 0);
  CHECK(orc_decode(9, h.data(), 4, dv.data()) != 0);
  // quantiser: random values, infinities, NaN, signed zeros, huge values
  std::vector<float> x(4096);
  for (auto& v : x) v = (float)(nd(rng) * std::pow(10.0, (double)rnd(-12, 6)));
  x[0] = INFINITY;
  x[1] = -INFINITY;
  x[2] = NAN;
  x[3] = -0.0f;
  x[4] = 3.0e38f;
  std::vector<uint8_t> codes(x.size());
  CHECK(orc_quantize_e4m3(x.data(), (int64_t)x.size(), 1.0f / 0.0103f, codes.data()) == 0);
  // scatter -> gather round trip, block copies and swaps, attention
  for (int trial = 0; trial < 20; ++trial) {
    const int H = (int)rnd(1, 3), dd = rnd(0, 1) ? 64 : 128, bs = 16, dtype = (int)rnd(0, 2);
    const int es = dtype == 0 ? 4 : 2;
    const int64_t nbk = rnd(2, 12);
    const int64_t elems = nbk * H * bs * dd;
    std::vector<uint8_t> kp(elems * es), vp(elems * es);
    const int64_t T = rnd(1, nbk * bs);
    std::vector<int32_t> table(nbk);
    for (int64_t i = 0; i < nbk; ++i) table[i] = (int32_t)i;
    std::shuffle(table.begin(), table.end(), rng);
    std::vector<int64_t> slots(T);
    for (int64_t t = 0; t < T; ++t) slots[t] = orc_slot(table.data(), t, bs);
    if (T > 1) slots[rnd(0, T - 1)] = -1;  // a padding slot
    std::vector<uint8_t> key(T * H * dd * es), val(T * H * dd * es);
    for (auto& c : key) c = (uint8_t)rnd(0, 255);
    for (auto& c : val) c = (uint8_t)rnd(0, 255);
    CHECK(orc_scatter(dtype, key.data(), val.data(), T, (int64_t)H * dd, (int64_t)H * dd, kp.data(), vp.data(),
                      slots.data(), nbk, bs, H, dd) == 0);
    std::vector<double> kg(T * H * dd), vg(T * H * dd);
    CHECK(orc_gather(dtype, kp.data(), vp.data(), nbk, bs, H, dd, table.data(), nbk, T, kg.data(), vg.data()) == 0);
    std::vector<int32_t> bad = table;
    bad[0] = (int32_t)nbk;  // a block outside the pool
    CHECK(orc_gather(dtype, kp.data(), vp.data(), nbk, bs, H, dd, bad.data(), nbk, T, kg.data(), vg.data()) == -2);
    int32_t pairs[4] = {0, (int32_t)(nbk - 1), 1, 0};
    CHECK(orc_copy_blocks(dtype, kp.data(), vp.data(), pairs, 2, nbk, bs, H, dd) == 0);
    int32_t badp[2] = {0, (int32_t)nbk};
    CHECK(orc_copy_blocks(dtype, kp.data(), vp.data(), badp, 1, nbk, bs, H, dd) == -2);
    std::vector<uint8_t> hk(elems * es), hv(elems * es);
    CHECK(orc_swap_blocks(dtype, kp.data(), vp.data(), nbk, hk.data(), hv.data(), nbk, pairs, 2, bs, H, dd) == 0);
    // attention over finite values
    const int G = (int)rnd(1, 4), Hq = H * G;
    std::vector<double> kk(T * H * dd), vv(T * H * dd), q(3 * Hq * dd), out(3 * Hq * dd), ws(3 * Hq);
    for (auto& v : kk) v = nd(rng);
    for (auto& v : vv) v = nd(rng);
    for (auto& v : q) v = nd(rng);
    int64_t pos[3] = {0, T - 1, rnd(0, T - 1)};
    std::vector<double> scratch(T * 4);
    CHECK(orc_attention(3, q.data(), pos, T, kk.data(), vv.data(), Hq, H, dd, 1.0 / std::sqrt((double)dd), out.data(),
                        ws.data(), scratch.data(), 4) == 0);
    for (double w : ws) CHECK(std::fabs(w - 1.0) < 1e-9);
    int64_t badpos[1] = {T};
    CHECK(orc_attention(1, q.data(), badpos, T, kk.data(), vv.data(), Hq, H, dd, 0.1, out.data(), ws.data(),
                        scratch.data(), 1) != 0);
  }
}

int main(int argc, char** argv) {
  const int runs = argc > 1 ? std::atoi(argv[1]) : 40;
  for (int r = 0; r < runs; ++r) fuzz_block_manager(1000 + r, 400);
  exercise_oracle(7);
  std::printf("sanitize driver: %d allocator runs and the oracle routines passed\n", runs);
  return g_fail;
}
