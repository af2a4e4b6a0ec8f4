// CPU driver for the trace-range test: one prefill and one decode step at k = 2 through
// the C ABI, on the stand-in HIP runtime (tests/host/fake_hip.cpp) and kernel launchers
// (tests/host/stub_launchers.cpp). The ranges themselves are printed by the stand-in
// marker library (tests/host/roctx_stub.cpp) that DORY_TRACE_LIB names.
#include <cstdint>
#include <cstdio>

#include <hip/hip_runtime_api.h>

#include "../../include/dory.h"

extern hipError_t g_stub_launch;

int main() {
  g_stub_launch = hipSuccess;
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
  c.max_loops = 2;
  c.max_seqs = 2;
  c.max_seq_len = 256;
  c.max_rows = 256;
  dory_ctx* ctx = nullptr;
  size_t page_bytes = 0, ws_bytes = 0;
  if (dory_create(&c, &ctx) != DORY_OK || dory_query_sizes(&c, &page_bytes, &ws_bytes) != DORY_OK) return 2;
  // addresses the stand-in launchers never dereference
  if (dory_bind_kv_pool(ctx, (void*)(uintptr_t)0x7f0000000000ull, 64 * page_bytes) != DORY_OK ||
      dory_bind_workspace(ctx, (void*)(uintptr_t)0x7e0000000000ull, ws_bytes) != DORY_OK)
    return 3;
  static float fake_f[64];
  dory_layer_weights w{};
  w.w_qkvg = w.w_o = w.w_gu = w.w_down = (const void*)(uintptr_t)0x7d0000000000ull;
  w.alpha_attn = w.alpha_mlp = w.s_qk = fake_f;
  for (int l = 0; l < c.n_in + c.n_rec + c.n_out; ++l)
    if (dory_bind_weights(ctx, l, &w) != DORY_OK) return 4;
  if (dory_set_kv_mode(ctx, DORY_KV_PER_LOOP) != DORY_OK || dory_set_loops(ctx, 2) != DORY_OK) return 5;
  static float x[256 * 256], y[256 * 256];
  const int32_t ids[2] = {0, 1}, n_new[2] = {100, 30};
  if (dory_prefill(ctx, nullptr, 2, ids, n_new, x, y) != DORY_OK) return 6;
  if (dory_decode_step(ctx, nullptr, 2, ids, x, y) != DORY_OK) return 7;
  if (dory_destroy(ctx) != DORY_OK) return 8;
  std::printf("trace main done\n");
  return 0;
}
