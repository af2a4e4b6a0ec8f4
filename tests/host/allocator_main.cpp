// CPU test of the host runtime's paged KV bookkeeping through the C ABI, built with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).
//
// No GPU: the KV pool, workspace and weights are bound as fake, never-dereferenced
// device addresses, and every call that would enqueue device work stops at the runtime's
// first HIP allocation with DORY_ERR_HIP, before it commits. What runs is the host side:
// configuration checks, the page allocator (full-attention streams, sliding-window rings,
// per_loop / last_loop slot counts), page-table delta lists, truncation and release. A
// seeded sequence of random operations is checked after every step against a model kept
// here: the pages a sequence holds are those a sequence of its longest length ever
// reached holds (truncation keeps pages), counted by dory_kv_pages_needed.
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <vector>

#include "../../include/dory.h"

static int failures = 0;
static long n_grown = 0, n_out_of_kv = 0, n_released = 0, n_truncated = 0;
#define EXPECT(cond, ...)                                                  \
  do {                                                                     \
    if (!(cond)) {                                                         \
      ++failures;                                                          \
      std::fprintf(stderr, "line %d: check failed: %s: ", __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                                   \
      std::fprintf(stderr, "\n");                                          \
    }                                                                      \
  } while (0)

struct Model {
  int64_t len = 0, max_len = 0;
  int k_built = 1;
};

static dory_config make_cfg(int window, int max_rows) {
  dory_config c{};
  c.hidden = 256;
  c.n_q_heads = 4;
  c.n_kv_heads = 1;
  c.head_dim = 64;
  c.intermediate = 1024;
  c.n_in = 2;
  c.n_rec = 4;
  c.n_out = 2;
  c.window = window;
  c.full_period = 4;
  c.theta_swa = 1e4;
  c.theta_full = 1e7;
  c.attn_scale = 8.f;
  c.qk_norm = 1;
  c.attn_gate = DORY_GATE_ELEMENTWISE;
  c.act_dtype = DORY_DTYPE_F32;
  c.weight_format = DORY_WFMT_F32;
  c.max_loops = 4;
  c.max_seqs = 6;
  c.max_seq_len = 3000;
  c.max_rows = max_rows;
  return c;
}

static int run(int window, int max_rows, int mode, unsigned seed, int n_ops) {
  dory_config cfg = make_cfg(window, max_rows);
  dory_ctx* ctx = nullptr;
  EXPECT(dory_create(&cfg, &ctx) == DORY_OK, "create: %s", dory_last_error(nullptr));
  size_t page_bytes = 0, ws_bytes = 0;
  EXPECT(dory_query_sizes(&cfg, &page_bytes, &ws_bytes) == DORY_OK, "query_sizes");
  // fake device addresses (never dereferenced on the host)
  const size_t n_pages = 300;
  void* pool = (void*)(uintptr_t)0x7f0000000000ull;
  void* ws = (void*)(uintptr_t)0x7e0000000000ull;
  EXPECT(dory_bind_kv_pool(ctx, pool, n_pages * page_bytes) == DORY_OK, "pool");
  EXPECT(dory_bind_workspace(ctx, ws, ws_bytes) == DORY_OK, "workspace");
  float fake_f[64];
  dory_layer_weights w{};
  w.w_qkvg = w.w_o = w.w_gu = w.w_down = (const void*)(uintptr_t)0x7d0000000000ull;
  w.alpha_attn = w.alpha_mlp = w.s_qk = fake_f;
  for (int l = 0; l < cfg.n_in + cfg.n_rec + cfg.n_out; ++l) EXPECT(dory_bind_weights(ctx, l, &w) == DORY_OK, "w");
  EXPECT(dory_set_kv_mode(ctx, mode) == DORY_OK, "mode");

  std::mt19937 rng(seed);
  auto rnd = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  std::map<int32_t, Model> live;
  auto held = [&]() {
    int64_t pages = 0;
    for (auto& kv : live) {
      int64_t p = 0;
      EXPECT(dory_kv_pages_needed(&cfg, mode, kv.second.k_built, kv.second.max_len, 1, &p) == DORY_OK, "needed");
      pages += p;
    }
    return pages;
  };
  auto check = [&](const char* after) {
    size_t bytes = 0;
    EXPECT(dory_kv_bytes_in_use(ctx, &bytes) == DORY_OK, "in use");
    EXPECT((int64_t)(bytes / page_bytes) == held(), "after %s: %zu pages in use, model %lld", after,
           bytes / page_bytes, (long long)held());
    int32_t n = -1;
    EXPECT(dory_live_seqs(ctx, &n) == DORY_OK && n == (int32_t)live.size(), "after %s: live %d, model %zu", after, n,
           live.size());
    for (auto& kv : live) {
      int64_t len = -1;
      EXPECT(dory_seq_len(ctx, kv.first, &len) == DORY_OK && len == kv.second.len, "after %s: seq %d len %lld != %lld",
             after, kv.first, (long long)len, (long long)kv.second.len);
    }
  };
  int k_ctx = 2;
  EXPECT(dory_set_loops(ctx, k_ctx) == DORY_OK, "loops");
  for (int op = 0; op < n_ops; ++op) {
    const int kind = rnd(0, 9);
    const int32_t id = rnd(0, 7);
    auto it = live.find(id);
    if (kind <= 3) {  // grow by reserve
      const int n = rnd(1, 400);
      const int r = dory_test_reserve(ctx, id, n);
      const bool fits_seqs = it != live.end() || (int)live.size() < cfg.max_seqs;
      const int64_t len0 = it == live.end() ? 0 : it->second.len;
      if (!fits_seqs || len0 + n > cfg.max_seq_len) {
        EXPECT(r == DORY_ERR_INVALID_ARG, "reserve %d +%d: %d", id, n, r);
      } else if (r == DORY_OK) {
        Model& m = live[id];
        if (it == live.end()) m.k_built = mode == DORY_KV_PER_LOOP ? k_ctx : 1;
        m.len += n;
        m.max_len = std::max(m.max_len, m.len);
        ++n_grown;
      } else {
        EXPECT(r == DORY_ERR_OUT_OF_KV, "reserve %d +%d: %d (%s)", id, n, r, dory_last_error(ctx));
        ++n_out_of_kv;
      }
      check("reserve");
    } else if (kind == 4 && it != live.end()) {  // release
      EXPECT(dory_release_seq(ctx, id) == DORY_OK, "release");
      live.erase(it);
      ++n_released;
      check("release");
    } else if (kind == 5 && it != live.end()) {  // truncate
      const int64_t len = rnd(1, (int)it->second.len);
      EXPECT(dory_truncate_seq(ctx, id, len) == DORY_OK, "truncate");
      it->second.len = len;
      ++n_truncated;
      check("truncate");
    } else if (kind == 6) {  // a prefill: fails at the first device allocation, unchanged state
      const int32_t ids[2] = {id, (int32_t)((id + 1) % 8)};
      const int32_t nn[2] = {rnd(1, 64), rnd(1, 64)};
      const int r = dory_prefill(ctx, nullptr, 2, ids, nn, fake_f, fake_f);
      EXPECT(r != DORY_OK, "prefill without a GPU returned OK");
      check("prefill");
    } else if (kind == 7) {  // argument errors
      const int32_t ids[2] = {id, id};
      const int32_t nn[2] = {1, 1};
      EXPECT(dory_prefill(ctx, nullptr, 2, ids, nn, fake_f, fake_f) == DORY_ERR_INVALID_ARG, "repeated id");
      const int32_t big[1] = {cfg.max_rows + 1};
      EXPECT(dory_prefill(ctx, nullptr, 1, ids, big, fake_f, fake_f) == DORY_ERR_INVALID_ARG, "rows > max_rows");
      if (!live.empty()) {
        EXPECT(dory_set_kv_mode(ctx, mode) == DORY_ERR_STATE, "mode change while live");
        EXPECT(dory_bind_kv_pool(ctx, pool, n_pages * page_bytes) == DORY_ERR_STATE, "rebind pool while live");
      }
      check("argument errors");
    } else if (kind == 8) {  // the context's loop count (new per_loop sequences build that many slots)
      k_ctx = rnd(1, 4);
      EXPECT(dory_set_loops(ctx, k_ctx) == DORY_OK, "set loops");
      EXPECT(dory_set_loops(ctx, 5) == DORY_ERR_INVALID_ARG, "k > max_loops");
    } else if (kind == 9 && it != live.end()) {  // per-sequence loop counts
      const int k = rnd(0, 4);
      const int r = dory_set_seq_loops(ctx, id, k);
      if (mode == DORY_KV_PER_LOOP && k > it->second.k_built) EXPECT(r == DORY_ERR_STATE, "seq loops above built");
      else EXPECT(r == DORY_OK, "seq loops");
    }
  }
  for (auto& kv : live) EXPECT(dory_release_seq(ctx, kv.first) == DORY_OK, "final release");
  live.clear();
  check("final release");
  size_t bytes = 1;
  EXPECT(dory_kv_bytes_in_use(ctx, &bytes) == DORY_OK && bytes == 0, "pages left after releasing everything");
  EXPECT(dory_destroy(ctx) == DORY_OK, "destroy");
  return failures;
}

int main() {
  // full and sliding streams, window shorter and longer than a page, both KV modes
  for (int mode : {DORY_KV_PER_LOOP, DORY_KV_LAST_LOOP})
    for (int window : {16, 200})
      for (unsigned seed : {1u, 2u}) run(window, 128, mode, seed, 3000);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("allocator checks passed: %ld grows, %ld refused for lack of pages, %ld releases, %ld truncations\n",
              n_grown, n_out_of_kv, n_released, n_truncated);
  if (n_grown < 1000 || n_out_of_kv < 10 || n_released < 100 || n_truncated < 100) {
    std::fprintf(stderr, "too few operations of some kind\n");
    return 1;
  }
  return 0;
}
