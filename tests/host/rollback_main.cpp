// CPU test of the boundary's error contract, built with AddressSanitizer and
// UndefinedBehaviorSanitizer: a prefill or decode call that fails after committing
// (its sequences created and grown, pages taken, page-table updates consumed) leaves the
// context as it was. The HIP runtime is a stand-in (tests/host/fake_hip.cpp) that
// records every host-to-device upload instead of performing it, and the kernel
// launchers succeed without doing anything, so the host runtime runs every step of a
// call. dory_test_inject_failure makes a call fail at a chosen point (the metadata
// upload, or layer call n). Context A fails and retries each such call; context B, with
// the same configuration, makes the same calls and never fails. After every failure
// A's host state must equal its state before the call, and every successful call must
// upload exactly the same bytes on A as on B: the same positions, tiles, page ids and
// page-table updates (a lost or duplicated update, or pages handed out in another order,
// would show there).
#include <cstdio>
#include <cstdlib>
#include <functional>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "../../include/dory.h"

extern std::vector<std::vector<unsigned char>> g_uploads;
extern hipError_t g_stub_launch;

static int failures = 0, n_failed_calls = 0, n_compared = 0;
#define EXPECT(cond, ...)                                                  \
  do {                                                                     \
    if (!(cond)) {                                                         \
      ++failures;                                                          \
      std::fprintf(stderr, "line %d: check failed: %s: ", __LINE__, #cond); \
      std::fprintf(stderr, __VA_ARGS__);                                   \
      std::fprintf(stderr, "\n");                                          \
    }                                                                      \
  } while (0)

static dory_config make_cfg() {
  dory_config c{};
  c.hidden = 256;
  c.n_q_heads = 4;
  c.n_kv_heads = 1;
  c.head_dim = 64;
  c.intermediate = 1024;
  c.n_in = 2;
  c.n_rec = 4;
  c.n_out = 2;
  c.window = 64;
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
  c.max_seq_len = 1024;
  c.max_rows = 256;
  return c;
}

struct State {
  int32_t live = -1;
  size_t bytes = 0;
  std::vector<int64_t> lens;
  bool operator==(const State& o) const { return live == o.live && bytes == o.bytes && lens == o.lens; }
};

static State state_of(dory_ctx* c) {
  State s;
  dory_live_seqs(c, &s.live);
  dory_kv_bytes_in_use(c, &s.bytes);
  for (int id = 0; id < 8; ++id) {
    int64_t len = -1;
    if (dory_seq_len(c, id, &len) != DORY_OK) len = -1;
    s.lens.push_back(len);
  }
  return s;
}

static dory_ctx* make_ctx(int mode, int k) {
  dory_config cfg = make_cfg();
  dory_ctx* ctx = nullptr;
  EXPECT(dory_create(&cfg, &ctx) == DORY_OK, "create");
  size_t page_bytes = 0, ws_bytes = 0;
  EXPECT(dory_query_sizes(&cfg, &page_bytes, &ws_bytes) == DORY_OK, "sizes");
  EXPECT(dory_bind_kv_pool(ctx, (void*)(uintptr_t)0x7f0000000000ull, 400 * page_bytes) == DORY_OK, "pool");
  EXPECT(dory_bind_workspace(ctx, (void*)(uintptr_t)0x7e0000000000ull, ws_bytes) == DORY_OK, "ws");
  static float fake_f[64];
  dory_layer_weights w{};
  w.w_qkvg = w.w_o = w.w_gu = w.w_down = (const void*)(uintptr_t)0x7d0000000000ull;
  w.alpha_attn = w.alpha_mlp = w.s_qk = fake_f;
  for (int l = 0; l < cfg.n_in + cfg.n_rec + cfg.n_out; ++l) EXPECT(dory_bind_weights(ctx, l, &w) == DORY_OK, "w");
  EXPECT(dory_set_kv_mode(ctx, mode) == DORY_OK, "mode");
  EXPECT(dory_set_loops(ctx, k) == DORY_OK, "loops");
  return ctx;
}

using Call = std::function<int(dory_ctx*)>;

static void run(int mode) {
  const int k = 2;
  const int calls = 2 + k * 4 + 2;  // layer calls of a step
  dory_ctx* A = make_ctx(mode, k);
  dory_ctx* B = make_ctx(mode, k);
  static float x[256 * 256], y[256 * 256];  // never read: the launchers do nothing

  // the same successful call on both contexts, uploads compared byte for byte
  auto both = [&](const char* what, const Call& f) {
    g_uploads.clear();
    const int ra = f(A);
    const auto ua = g_uploads;
    g_uploads.clear();
    const int rb = f(B);
    const auto ub = g_uploads;
    EXPECT(ra == DORY_OK && rb == DORY_OK, "%s: %d %d (%s)", what, ra, rb, dory_last_error(A));
    EXPECT(ua == ub, "%s: %zu uploads on the retried context, %zu on the control; contents differ", what,
           ua.size(), ub.size());
    EXPECT(state_of(A) == state_of(B), "%s: host states differ", what);
    ++n_compared;
  };
  // a call that fails at `at` on A only, then the same call on both
  auto fail_then = [&](const char* what, int at, const Call& f) {
    const State before = state_of(A);
    EXPECT(dory_test_inject_failure(A, at) == DORY_OK, "inject");
    const int r = f(A);
    EXPECT(r == DORY_ERR_HIP, "%s at %d: returned %d", what, at, r);
    EXPECT(state_of(A) == before, "%s at %d: state changed by a failed call", what, at);
    ++n_failed_calls;
    both(what, f);
  };
  auto prefill = [&](std::vector<int32_t> ids, std::vector<int32_t> n) {
    return [ids, n](dory_ctx* c) { return dory_prefill(c, nullptr, (int)ids.size(), ids.data(), n.data(), x, y); };
  };
  auto decode = [&](std::vector<int32_t> ids) {
    return [ids](dory_ctx* c) { return dory_decode_step(c, nullptr, (int)ids.size(), ids.data(), x, y); };
  };

  both("first prefill", prefill({0, 1}, {100, 30}));
  for (int at : {0, 1, 3, calls}) {
    fail_then("prefill crossing a page, new sequence", at, prefill({0, 2 + at % 2}, {40, 10}));
    fail_then("decode", at, decode({0, 1}));
  }
  // page-table updates queued outside a call (a reservation) must survive a failure
  both("reserve", [](dory_ctx* c) { return dory_test_reserve(c, 1, 70); });
  fail_then("prefill after a reservation", 0, prefill({1, 4}, {20, 64}));
  both("reserve again", [](dory_ctx* c) { return dory_test_reserve(c, 4, 1); });
  fail_then("decode after a reservation", calls, decode({0, 1, 4}));
  // release and truncation, then regrowth into the sequence's own pages
  both("release", [](dory_ctx* c) { return dory_release_seq(c, 2); });
  both("truncate", [](dory_ctx* c) { return dory_truncate_seq(c, 0, 50); });
  fail_then("regrowth after truncation", 1, prefill({0}, {60}));
  fail_then("long chunk", 5, prefill({5}, {256}));
  both("decode all", decode({0, 1, 3, 4, 5}));
  EXPECT(dory_destroy(A) == DORY_OK && dory_destroy(B) == DORY_OK, "destroy");
}

int main() {
  g_stub_launch = hipSuccess;
  for (int mode : {DORY_KV_PER_LOOP, DORY_KV_LAST_LOOP}) run(mode);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("rollback checks passed: %d failed calls rolled back, %d call pairs compared\n", n_failed_calls,
              n_compared);
  return 0;
}
