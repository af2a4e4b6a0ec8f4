// Host runtime behind include/dory.h: context, argument checks, the paged KV cache
// (page allocator, per-(layer, slot) page tables, sliding-window rings) and the layer
// schedule of the looped forward pass.
//
// Schedule ("Dory1.0-4B", paper summary core-method equation; arXiv §3.2): input block
// layers once (KV slot 0); x saved at its end and u_1 = N(x + x); the recurrent block
// k times with KV slot t-1 (per_loop) or 0 (last_loop), ending each loop with
// s_t = N(.) and u_{t+1} = N(s_t + x); the output block once (slot 0).
// KV slots (arXiv §6.1): per_loop keeps k slots per recurrent attention layer,
// last_loop one slot that every loop overwrites.
#include <dlfcn.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <set>
#include <string>
#include <vector>

#include "../../include/dory.h"
#include "kernels.h"

using namespace dory;

namespace {

constexpr int NSTAGE = 4;          // pinned staging buffers in rotation
constexpr int DELTA_CAP = 65536;   // page-table updates per upload
constexpr int ACT_STATE_MIN_ROWS = 512;  // rows from which a prefill keeps its state in fp16
constexpr int SKINNY_M = 256;      // rows up to which projections use split-K tiles
constexpr size_t ALIGN = 256;
constexpr int ROPE_INTS = 2 * 128 * 2;  // two tables of up to 128 doubles

thread_local std::string g_create_err;

size_t al(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

struct Dims {
  int H, Hq, Hkv, d, I, Nq, Nkv, Ng, Nqkvg, L;
  int n_streams, tab_len, ring_swa;
  size_t esz;          // act element size
  size_t page_elems;   // elements per page (K and V)
  size_t page_bytes;
  int max_tiles;
};

struct WsLayout {
  size_t table, meta, s, x, sb, s16, qkvg, q, o, h, part, apart, wexp, rcs, total;
  size_t part_floats, apart_floats;
  size_t meta_ints;
};

Dims dims_of(const dory_config& c) {
  Dims D{};
  D.H = c.hidden;
  D.Hq = c.n_q_heads;
  D.Hkv = c.n_kv_heads;
  D.d = c.head_dim;
  D.I = c.intermediate;
  D.Nq = D.Hq * D.d;
  D.Nkv = D.Hkv * D.d;
  D.Ng = c.attn_gate == DORY_GATE_ELEMENTWISE ? D.Nq : 0;
  D.Nqkvg = D.Nq + 2 * D.Nkv + D.Ng;
  D.L = c.n_in + c.n_rec + c.n_out;
  D.n_streams = c.n_in + c.n_rec * c.max_loops + c.n_out;
  D.tab_len = (c.max_seq_len + DORY_PAGE_TOKENS - 1) / DORY_PAGE_TOKENS;
  const int ring = (c.window + c.max_rows - 1 + DORY_PAGE_TOKENS - 1) / DORY_PAGE_TOKENS + 1;
  D.ring_swa = std::min(ring, D.tab_len);
  D.esz = c.act_dtype == DORY_DTYPE_F32 ? 4 : 2;
  D.page_elems = (size_t)2 * D.Hkv * DORY_PAGE_TOKENS * D.d;
  D.page_bytes = D.page_elems * D.esz;
  D.max_tiles = (c.max_rows + 63) / 64 + c.max_seqs;
  return D;
}

// floats of one base's RoPE (cos, sin) table: a block of 64 rows x d/2 pairs per tile
size_t rope_table_floats(const Dims& D) { return (size_t)D.max_tiles * 64 * D.d; }

WsLayout layout_of(const dory_config& c, const Dims& D) {
  WsLayout W{};
  const size_t R = (size_t)c.max_rows;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al(bytes);
    return o;
  };
  W.table = take((size_t)c.max_seqs * D.n_streams * D.tab_len * 4);
  // metadata per call: positions, row -> sequence slot, prefill tiles, RoPE frequency
  // tables (2 bases x 128 doubles), page-table updates
  W.meta_ints = 3 * R + 4 * (size_t)D.max_tiles + ROPE_INTS + 2 * (size_t)DELTA_CAP;
  W.meta = take(W.meta_ints * 4);
  W.s = take(R * D.H * 4);
  W.x = take(R * D.H * 4);
  W.sb = take(R * D.H * D.esz);
  W.s16 = take(c.act_dtype == DORY_DTYPE_BF16 ? R * D.H * 2 : 0);  // fp16 state of long prefills
  W.qkvg = take(R * D.Nqkvg * D.esz);
  W.q = take(R * D.Nq * D.esz);
  W.o = take(R * D.Nq * D.esz);
  W.h = take(R * D.I * D.esz);
  const size_t maxN = std::max({(size_t)D.Nqkvg, (size_t)2 * D.I, (size_t)D.H});
  size_t pf = R * maxN;  // one split at max rows (fp32 path, prefill outputs)
  if (c.act_dtype == DORY_DTYPE_BF16) pf = std::max(pf, (size_t)32 * std::min<size_t>(R, SKINNY_M) * maxN);  // <= 32 splits
  W.part_floats = pf;
  W.part = take(pf * 4);
  W.apart_floats = std::max<size_t>(R, 256) * D.Hq * (D.d + 2) * 8;
  W.apart = take(W.apart_floats * 4);
  // MXFP8 / NVFP4: one weight matrix expanded to bf16 for the large-M GEMMs
  const size_t wmax = std::max({(size_t)D.Nqkvg * D.H, (size_t)D.H * D.Nq, (size_t)2 * D.I * D.H,
                                (size_t)D.H * D.I});
  const bool quant = c.weight_format == DORY_WFMT_NVFP4 || c.weight_format == DORY_WFMT_MXFP8;
  W.wexp = take(quant && c.max_rows > SKINNY_M ? wmax * 2 : 0);
  // (cos, sin) of the prefill tiles' RoPE angles for both bases (64-row blocks per tile)
  W.rcs = take(2 * rope_table_floats(D) * 4);
  W.total = off;
  return W;
}

struct Seq {
  int32_t id = 0;
  int slot = 0;
  int64_t len = 0;
  int k_built = 1;
  int rec_slots = 1;
  int k_set = 0;  // loop count set for this sequence (0: the default of its mode)
  std::vector<std::vector<int32_t>> pages;  // per stream: table entries (-1 = none)
};

}  // namespace

struct dory_ctx {
  dory_config cfg{};
  Dims D{};
  WsLayout W{};
  int k = 2;
  int mode = DORY_KV_PER_LOOP;
  std::vector<dory_layer_weights> lw;
  std::vector<bool> lw_bound;
  dory_vocab_weights vocab{};
  bool vocab_bound = false;
  void* pool = nullptr;
  size_t pool_bytes = 0;
  int64_t n_pages = 0;
  std::vector<int32_t> free_pages;
  char* ws = nullptr;
  size_t ws_bytes = 0;
  std::map<int32_t, Seq> seqs;
  std::vector<int> free_slots;
  std::vector<int32_t> pending;  // (flat table index, page) pairs
  std::string err;
  int64_t last_calls = 0;
  // one-shot options of the next prefill / decode call (speculative activation reuse)
  float* cap_x = nullptr;
  float* cap_s1 = nullptr;
  bool cap_skip_out = false;
  const float* res_x = nullptr;
  const float* res_s1 = nullptr;
  bool dev_ready = false;
  int32_t* stage[NSTAGE] = {};
  hipEvent_t ev[NSTAGE] = {};
  int stage_i = 0;
  std::vector<int32_t> scratch;
  // calls are ordered across streams: each call's device work ends with done_ev on its
  // stream, and a call on another stream first waits for it (the workspace is shared)
  hipEvent_t done_ev = nullptr;
  hipStream_t last_st = nullptr;
  bool have_last = false;
  // test hook: fail the next prefill/decode call after it has committed (0: at the
  // metadata upload; n >= 1: before layer call n), then disarm
  int inject_at = -1;
  // tracing
  int prof = 0;  // bit mask of kernel classes being timed
  struct ProfRec { int kc; int ev; double flops, bytes; };
  std::vector<hipEvent_t> pev;
  int pev_used = 0;
  std::vector<ProfRec> precs;

  int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    err = buf;
    return code;
  }
  bool is_full(int l) const { return l % cfg.full_period == cfg.full_period - 1; }
  int stream_of(int l, int slot) const {
    if (l < cfg.n_in) return l;
    if (l < cfg.n_in + cfg.n_rec) return cfg.n_in + (l - cfg.n_in) * cfg.max_loops + slot;
    return cfg.n_in + cfg.n_rec * cfg.max_loops + (l - cfg.n_in - cfg.n_rec);
  }
  int ring_of(int l) const { return is_full(l) ? D.tab_len : D.ring_swa; }
  int layer_of_stream(int s) const {
    if (s < cfg.n_in) return s;
    if (s < cfg.n_in + cfg.n_rec * cfg.max_loops) return cfg.n_in + (s - cfg.n_in) / cfg.max_loops;
    return s - cfg.n_rec * cfg.max_loops + cfg.n_rec;
  }
  bool stream_used(const Seq& q, int s) const {
    if (s < cfg.n_in || s >= cfg.n_in + cfg.n_rec * cfg.max_loops) return true;
    return (s - cfg.n_in) % cfg.max_loops < q.rec_slots;
  }
};

namespace {

int hip_fail(dory_ctx* c, hipError_t e, const char* what) {
  return c->fail(DORY_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define HIPCHK(expr, what)                      \
  do {                                          \
    hipError_t e_ = (expr);                     \
    if (e_ != hipSuccess) return hip_fail(ctx, e_, what); \
  } while (0)

// Record a launch bracket: begin() before the launch, end() after it.
int prof_event(dory_ctx* ctx, hipStream_t st) {
  if (ctx->pev_used == (int)ctx->pev.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return -1;
    ctx->pev.push_back(e);
  }
  const int i = ctx->pev_used++;
  if (hipEventRecord(ctx->pev[i], st) != hipSuccess) return -1;
  return i;
}

// Optional marker ranges (DORY_TRACE=1 in the environment): one range per boundary
// call, per block of the schedule (input block, each loop, output block) and per layer
// call, named after what they cover; rocprofv3 --marker-trace shows them beside the
// kernels. The marker library (librocprofiler-sdk-roctx, or the one DORY_TRACE_LIB
// names) is opened on the first traced call, so the library does not link against it
// and an untraced call costs one environment lookup per range.
struct TraceApi {
  int (*push)(const char*);
  int (*pop)();
};
const TraceApi* trace_api() {
  static const TraceApi* api = []() -> const TraceApi* {
    const char* lib = std::getenv("DORY_TRACE_LIB");
    void* h = dlopen(lib && *lib ? lib : "librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_LOCAL);
    if (!h) return nullptr;
    static TraceApi a;
    a.push = (int (*)(const char*))dlsym(h, "roctxRangePushA");
    a.pop = (int (*)())dlsym(h, "roctxRangePop");
    return a.push && a.pop ? &a : nullptr;
  }();
  return api;
}
struct Trace {
  const TraceApi* api = nullptr;
  explicit Trace(const char* fmt, ...) {
    const char* e = std::getenv("DORY_TRACE");
    if (!e || !*e || (e[0] == '0' && !e[1]) || !(api = trace_api())) return;
    char buf[128];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    api->push(buf);
  }
  ~Trace() {
    if (api) api->pop();
  }
  Trace(const Trace&) = delete;
  Trace& operator=(const Trace&) = delete;
};

struct Prof {
  dory_ctx* ctx;
  hipStream_t st;
  int kc;
  int ev0 = -1;
  Prof(dory_ctx* c, hipStream_t s, int k) : ctx(c), st(s), kc(k) {
    if (ctx->prof & (1 << kc)) ev0 = prof_event(ctx, st);
  }
  void end(double flops, double bytes) {
    if (ev0 < 0) return;
    const int ev1 = prof_event(ctx, st);
    if (ev1 == ev0 + 1) ctx->precs.push_back({kc, ev0, flops, bytes});
  }
};

int check_config(const dory_config* c, std::string& msg) {
  auto bad = [&](const char* m) {
    msg = m;
    return DORY_ERR_INVALID_ARG;
  };
  auto uns = [&](const char* m) {
    msg = m;
    return DORY_ERR_UNSUPPORTED;
  };
  if (!c) return bad("null config");
  if (c->hidden < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 2 ||
      c->intermediate < 1)
    return bad("shape fields must be positive");
  if (c->n_q_heads % c->n_kv_heads) return bad("n_q_heads must be a multiple of n_kv_heads");
  if (c->head_dim % 2) return bad("head_dim must be even");
  if (c->n_in < 1 || c->n_rec < 1 || c->n_out < 1) return bad("each block needs >= 1 layer");
  if (c->window < 1 || c->full_period < 1) return bad("window and full_period must be >= 1");
  if (!(c->theta_swa > 0) || !(c->theta_full > 0) || !std::isfinite(c->attn_scale))
    return bad("RoPE bases must be > 0 and attn_scale finite");
  if (c->qk_norm != 0 && c->qk_norm != 1) return bad("qk_norm must be 0 or 1");
  if (c->attn_gate != DORY_GATE_NONE && c->attn_gate != DORY_GATE_ELEMENTWISE)
    return bad("attn_gate must be DORY_GATE_NONE or DORY_GATE_ELEMENTWISE");
  if (c->act_dtype != DORY_DTYPE_F32 && c->act_dtype != DORY_DTYPE_BF16) return bad("bad act_dtype");
  if (c->weight_format < DORY_WFMT_F32 || c->weight_format > DORY_WFMT_NVFP4)
    return bad("bad weight_format");
  if ((c->weight_format == DORY_WFMT_F32) != (c->act_dtype == DORY_DTYPE_F32))
    return bad("F32 weights go with F32 activations; BF16/MXFP8/NVFP4 weights with BF16");
  if (c->max_loops < 1 || c->max_loops > DORY_MAX_LOOPS) return bad("max_loops must be 1..8");
  if (c->max_seqs < 1 || c->max_rows < 1) return bad("max_seqs and max_rows must be >= 1");
  if (c->max_seq_len < 1 || c->max_seq_len > DORY_MAX_POSITIONS)
    return bad("max_seq_len must be 1..262144");
  // what the kernels of this library run
  const int G = c->n_q_heads / c->n_kv_heads;
  if (G > 4) return uns("more than 4 query heads per KV head");
  if (c->head_dim % 32 || c->head_dim > 256) return uns("head_dim must be a multiple of 32, <= 256 (KV page fragments)");
  if (c->hidden > 4096) return uns("hidden > 4096");
  if (c->act_dtype == DORY_DTYPE_BF16) {
    const int Nq = c->n_q_heads * c->head_dim;
    const int Nqkvg = Nq + 2 * c->n_kv_heads * c->head_dim +
                      (c->attn_gate == DORY_GATE_ELEMENTWISE ? Nq : 0);
    if (c->hidden % 128 || Nq % 64 || c->intermediate % 64 || Nqkvg % 128)
      return uns("bf16 shapes need hidden % 128, Hq*d % 64, I % 64, qkvg rows % 128 == 0");
  }
  if (c->act_dtype == DORY_DTYPE_F32 && c->head_dim * 4 * 2 * 64 > 49152)
    return uns("fp32 head_dim too large for the attention tile");
  const double tab = (double)c->max_seqs * (c->n_in + c->n_out + c->n_rec * c->max_loops) *
                     ((c->max_seq_len + 63) / 64);
  if (tab > 2e9) return uns("page table too large");
  return DORY_OK;
}

int64_t pages_for_stream(int64_t len, bool full, int ring) {
  const int64_t np = (len + DORY_PAGE_TOKENS - 1) / DORY_PAGE_TOKENS;
  return full ? np : std::min<int64_t>(np, ring);
}

// Pages a sequence must newly allocate to grow from its length to len1: the page-table
// entries grow() would fill that hold no page yet (a truncated sequence keeps the pages
// past its length, so only the others count).
int64_t pages_to_grow(const dory_ctx* c, const Seq& q, int64_t len1) {
  int64_t need = 0;
  const int64_t lp0 = (q.len + DORY_PAGE_TOKENS - 1) / DORY_PAGE_TOKENS;
  const int64_t lp1 = (len1 + DORY_PAGE_TOKENS - 1) / DORY_PAGE_TOKENS;
  for (int s = 0; s < c->D.n_streams; ++s) {
    if (!c->stream_used(q, s)) continue;
    const int l = c->layer_of_stream(s);
    const int ring = c->ring_of(l);
    const bool full = c->is_full(l);
    const std::vector<int32_t>* tab = (size_t)s < q.pages.size() ? &q.pages[s] : nullptr;
    // a ring stream visits each entry at most once however far it grows
    const int64_t end = full ? lp1 : std::min(lp1, lp0 + ring);
    for (int64_t lp = lp0; lp < end; ++lp) {
      const int64_t idx = full ? lp : lp % ring;
      if (!tab || (int64_t)tab->size() <= idx || (*tab)[idx] < 0) ++need;
    }
  }
  return need;
}

// One page a call took from the free list: enough to give it back (rollback).
struct Taken {
  int32_t id;
  int stream;
  int idx;
  int32_t page;
};

void grow(dory_ctx* c, Seq& q, int64_t len1, std::vector<Taken>* journal = nullptr) {
  const int64_t len0 = q.len;
  for (int s = 0; s < c->D.n_streams; ++s) {
    if (!c->stream_used(q, s)) continue;
    const int l = c->layer_of_stream(s);
    const int ring = c->ring_of(l);
    auto& tab = q.pages[s];
    const bool full = c->is_full(l);
    if (!full && tab.empty()) tab.assign(ring, -1);
    // logical pages [ceil(len0/64), ceil(len1/64)) are new; page lp lives in entry lp % ring
    const int64_t lp0 = (len0 + DORY_PAGE_TOKENS - 1) / DORY_PAGE_TOKENS;
    const int64_t lp1 = (len1 + DORY_PAGE_TOKENS - 1) / DORY_PAGE_TOKENS;
    for (int64_t lp = lp0; lp < lp1; ++lp) {
      const int idx = (int)(lp % ring);
      if (full && (int64_t)tab.size() <= lp) tab.resize(lp + 1, -1);
      if (tab[idx] < 0) {
        tab[idx] = c->free_pages.back();
        c->free_pages.pop_back();
        if (journal) journal->push_back({q.id, s, idx, tab[idx]});
        const int64_t flat = ((int64_t)q.slot * c->D.n_streams + s) * c->D.tab_len + idx;
        c->pending.push_back((int32_t)flat);
        c->pending.push_back(tab[idx]);
      }
    }
  }
  q.len = len1;
}

void release(dory_ctx* c, Seq& q) {
  for (auto& tab : q.pages)
    for (int32_t p : tab)
      if (p >= 0) c->free_pages.push_back(p);
  c->free_slots.push_back(q.slot);
}

int dev_init(dory_ctx* ctx) {
  if (ctx->dev_ready) return DORY_OK;
  const size_t bytes = ctx->W.meta_ints * 4;
  for (int i = 0; i < NSTAGE; ++i) {
    HIPCHK(hipHostMalloc((void**)&ctx->stage[i], bytes, hipHostMallocDefault), "hipHostMalloc");
    HIPCHK(hipEventCreateWithFlags(&ctx->ev[i], hipEventDisableTiming), "hipEventCreate");
  }
  HIPCHK(hipEventCreateWithFlags(&ctx->done_ev, hipEventDisableTiming), "hipEventCreate");
  ctx->dev_ready = true;
  return DORY_OK;
}

// Start of a call's device work on st: wait for the previous call's work if it ran on
// another stream.
int enter(dory_ctx* ctx, hipStream_t st) {
  int r = dev_init(ctx);
  if (r) return r;
  if (ctx->have_last && ctx->last_st != st) HIPCHK(hipStreamWaitEvent(st, ctx->done_ev, 0), "hipStreamWaitEvent");
  return DORY_OK;
}

// End of a call's device work on st (also after a failure part-way: whatever was
// enqueued is ordered before the next call).
int leave(dory_ctx* ctx, hipStream_t st) {
  HIPCHK(hipEventRecord(ctx->done_ev, st), "hipEventRecord");
  ctx->last_st = st;
  ctx->have_last = true;
  return DORY_OK;
}

// Copy n ints to the workspace's metadata area through a pinned staging buffer.
int upload(dory_ctx* ctx, hipStream_t st, const int32_t* src, size_t n) {
  if (n == 0) return DORY_OK;
  const int i = ctx->stage_i++ % NSTAGE;
  HIPCHK(hipEventSynchronize(ctx->ev[i]), "hipEventSynchronize");
  memcpy(ctx->stage[i], src, n * 4);
  HIPCHK(hipMemcpyAsync(ctx->ws + ctx->W.meta, ctx->stage[i], n * 4, hipMemcpyHostToDevice, st),
         "hipMemcpyAsync");
  HIPCHK(hipEventRecord(ctx->ev[i], st), "hipEventRecord");
  return DORY_OK;
}

// Apply pending page-table updates beyond what fits with the call's own metadata.
int flush_deltas(dory_ctx* ctx, hipStream_t st, size_t keep) {
  while (ctx->pending.size() / 2 > keep) {
    const size_t n = std::min<size_t>(ctx->pending.size() / 2, DELTA_CAP);
    const size_t start = ctx->pending.size() - 2 * n;
    int r = upload(ctx, st, ctx->pending.data() + start, 2 * n);
    if (r) return r;
    HIPCHK(launch_apply_deltas((int32_t*)(ctx->ws + ctx->W.table), (const int32_t*)(ctx->ws + ctx->W.meta),
                               (int)n, ctx->pool, ctx->D.page_bytes, st), "apply_deltas");
    ctx->pending.resize(start);
  }
  return DORY_OK;
}

bool bound(dory_ctx* ctx) {
  if (!ctx->pool || !ctx->ws) return false;
  for (bool b : ctx->lw_bound)
    if (!b) return false;
  return true;
}

// Host state a prefill/decode call changes when it commits.
struct Journal {
  std::vector<Taken> taken;                       // pages taken, in order
  std::vector<std::pair<int32_t, int64_t>> lens;  // (id, length before) of live sequences
  std::vector<int32_t> created;                   // ids the call created, in order
  std::vector<int32_t> pending;                   // page-table deltas queued before the call
};

// Undo a committed call that failed before finishing: the pages go back to the free list
// in reverse order (restoring it exactly), lengths are reset, new sequences are removed
// and the page-table deltas queued before the call are queued again (re-applying one
// only clears a page that holds no entry a sequence can read). The device table may
// still hold entries of the returned pages; they sit past the sequences' lengths, are
// never read, and are overwritten when the sequences grow into them again.
void rollback(dory_ctx* ctx, Journal&& jr) {
  for (auto it = jr.taken.rbegin(); it != jr.taken.rend(); ++it) {
    ctx->seqs[it->id].pages[it->stream][it->idx] = -1;
    ctx->free_pages.push_back(it->page);
  }
  for (auto& l : jr.lens) ctx->seqs[l.first].len = l.second;
  for (auto it = jr.created.rbegin(); it != jr.created.rend(); ++it) {
    auto q = ctx->seqs.find(*it);
    ctx->free_slots.push_back(q->second.slot);
    ctx->seqs.erase(q);
  }
  ctx->pending = std::move(jr.pending);
}

struct CallPlan {
  int M = 0;
  int inject_at = -1;  // test hook: fail before layer call inject_at (>= 1)
  int max_pos = 0;
  int n_tiles = 0;
  int max_tile_rows = 0;
  int n_quads = 0;  // sum over tiles of ceil(rows / 4)
  std::vector<std::pair<int64_t, int>> chunks;  // (first position, rows) per sequence
  // Loop counts: sequences are ordered by loop count, largest first, so the rows still
  // looping in loop t are a prefix: loop_rows[t], loop_tiles[t], loop_seqs[t] (t >= 1).
  int k_max = 1;
  std::vector<int> loop_rows, loop_tiles, loop_seqs, loop_quads;
  bool reordered = false;  // rows are not in the caller's order (row map in the metadata)
  // activation reuse: capture x and s_1 (caller order), skip the output block; or start
  // at loop 2 from given x and s_1
  float* cap_x = nullptr;
  float* cap_s1 = nullptr;
  bool skip_out = false;
  const float* res_x = nullptr;
  const float* res_s1 = nullptr;
  // the state between sublayers is kept in fp16 beside its bf16 GEMM copy (every layer
  // call of the call takes the vectorised prefill update); the last layer writes floats
  bool act_state = false;
};

// Algorithmic attention work of one layer call: visible (query, key) pairs and the
// distinct cached entries the call must read.
void attn_work(const CallPlan& P, bool full, int W, double* pairs, double* keys) {
  *pairs = 0;
  *keys = 0;
  for (auto& c : P.chunks) {
    const int64_t p0 = c.first, n = c.second, p1 = p0 + n - 1;
    if (full) {
      *pairs += (double)n * (p0 + 1) + (double)n * (n - 1) / 2;
      *keys += (double)(p1 + 1);
    } else {
      for (int64_t p = p0; p <= p1; ++p) *pairs += (double)std::min<int64_t>(p + 1, W);
      *keys += (double)(p1 - std::max<int64_t>(0, p0 - W + 1) + 1);
    }
  }
}

KVLayout kv_layout(dory_ctx* ctx, int l) {
  KVLayout kv;
  kv.pool = ctx->pool;
  kv.act = ctx->cfg.act_dtype == DORY_DTYPE_F32 ? ACT_F32 : ACT_BF16;
  kv.Hkv = ctx->D.Hkv;
  kv.d = ctx->D.d;
  kv.page_elems = ctx->D.page_elems;
  kv.table = (const int32_t*)(ctx->ws + ctx->W.table);
  kv.n_streams = ctx->D.n_streams;
  kv.tab_len = ctx->D.tab_len;
  kv.ring = ctx->ring_of(l);
  return kv;
}

int run_layer(dory_ctx* ctx, hipStream_t st, const CallPlan& P, int l, int slot, int bnd,
              float* out, int final_from = 0x7fffffff) {
  const dory_config& c = ctx->cfg;
  const Dims& D = ctx->D;
  const WsLayout& W = ctx->W;
  char* ws = ctx->ws;
  const dory_layer_weights& w = ctx->lw[l];
  const int M = P.M;
  Trace tr("layer %d, KV slot %d, %d rows", l, slot, M);
  const int act = c.act_dtype == DORY_DTYPE_F32 ? ACT_F32 : ACT_BF16;
  const int wf = c.weight_format == DORY_WFMT_F32   ? W_F32
                 : c.weight_format == DORY_WFMT_BF16 ? W_BF16
                 : c.weight_format == DORY_WFMT_MXFP8 ? W_MXFP8
                                                      : W_NVFP4;
  const bool f32 = act == ACT_F32;
  const bool skinny = !f32 && M <= SKINNY_M;
  const int32_t* meta = (const int32_t*)(ws + W.meta);
  float* part = (float*)(ws + W.part);
  float* s = (float*)(ws + W.s);

  auto gemm = [&](const void* A, int K, const void* B, const uint8_t* Bs, int N, int epi, void* C,
                  int ldc, int splits) {
    GemmArgs g;
    g.A = A;
    g.lda = K;
    g.B = B;
    g.Bs = Bs;
    g.M = M;
    g.N = N;
    g.K = K;
    g.act = act;
    g.wfmt = wf;
    g.epi = epi;
    g.splits = splits;
    g.C = C;
    g.ldc = ldc;
    return g;
  };
  const double wbytes = wf == W_F32 ? 4.0 : wf == W_BF16 ? 2.0 : wf == W_MXFP8 ? 1.0 + 1.0 / 32 : 0.5 + 1.0 / 16;
  // NVFP4: the matrix scale that goes with a weight matrix of this layer
  auto nv_scale = [&](const void* B) -> const float* {
    return B == w.w_qkvg ? w.g_qkvg : B == w.w_o ? w.g_o : B == w.w_gu ? w.g_gu : w.g_down;
  };
  // bf16: the fragment-order copy of a weight matrix of this layer, if bound
  auto frag_of = [&](const void* B) -> const void* {
    return B == w.w_qkvg ? w.f_qkvg : B == w.w_o ? w.f_o : B == w.w_gu ? w.f_gu : B == w.w_down ? w.f_down : nullptr;
  };
  auto run_gemm = [&](const GemmArgs& g0) -> hipError_t {
    Prof pr(ctx, st, DORY_KC_GEMM);
    GemmArgs g = g0;
    if (wf == W_NVFP4) g.Bg = nv_scale(g0.B);
    if (wf == W_BF16 && g.epi == EPI_PARTIAL) g.Bf = frag_of(g0.B);
    if ((wf == W_NVFP4 || wf == W_MXFP8) && g.epi != EPI_PARTIAL) {
      // large M: expand the matrix to bf16 (exact), then the bf16 tiles
      const hipError_t x = wf == W_NVFP4 ? launch_expand_nvfp4((const uint8_t*)g.B, g.Bs, g.Bg, g.N, g.K, ws + W.wexp, st)
                                         : launch_expand_mxfp8((const uint8_t*)g.B, g.Bs, g.N, g.K, ws + W.wexp, st);
      if (x != hipSuccess) return x;
      g.B = ws + W.wexp;
      g.Bs = nullptr;
      g.Bg = nullptr;
      g.wfmt = W_BF16;
    }
    const hipError_t e = launch_gemm(g, st);
    const double outb = g.epi == EPI_STORE_ACT || g.epi == EPI_SWIGLU ? 2.0 : 4.0 * g.splits;
    const double ncols = g.epi == EPI_SWIGLU ? g.n_half : g.N;
    pr.end(2.0 * g.M * g.N * (double)g.K,
           (double)g.N * g.K * wbytes + (double)g.M * g.K * D.esz + (double)g.M * ncols * outb);
    return e;
  };
  auto update = [&](int splits, const float* alpha, int b, float* sout, bool ybf = false) {
    UpdateArgs u;
    u.y = part;
    u.splits = splits;
    u.y_bf16 = ybf;
    u.s = s;
    u.s_out = sout ? sout : P.act_state ? nullptr : s;
    u.state_act = P.act_state;
    u.s16 = ws + W.s16;
    u.sb = ws + W.sb;
    u.x = (float*)(ws + W.x);
    u.alpha = alpha;
    u.M = M;
    u.H = D.H;
    u.act = act;
    u.bnd = b;
    u.final_from = final_from;
    Prof pr(ctx, st, DORY_KC_UPDATE);
    const hipError_t e = launch_update(u, st);
    const double sbytes = P.act_state ? 4.0 + D.esz + (sout ? 4 : 0) : 4 + 4 + D.esz;
    pr.end(0, (double)M * D.H * ((ybf ? 2.0 : 4.0 * splits) + sbytes));
    return e;
  };

  // ---- attention sublayer: [q|k|v|g] projection
  int S = 1;
  RopeArgs ra;
  if (f32) {
    HIPCHK(run_gemm(gemm(ws + W.sb, D.H, w.w_qkvg, nullptr, D.Nqkvg, EPI_F32, part, D.Nqkvg, 1)), "gemm qkvg");
    ra.qkvg = part;
    ra.in_f32 = 1;
  } else if (skinny) {
    S = gemm_pick_splits(M, D.Nqkvg, D.H, wf);
    HIPCHK(run_gemm(gemm(ws + W.sb, D.H, w.w_qkvg, w.s_qkvg, D.Nqkvg, EPI_PARTIAL, part, D.Nqkvg, S)), "gemm qkvg");
    ra.qkvg = part;
    ra.in_f32 = 1;
  } else {
    HIPCHK(run_gemm(gemm(ws + W.sb, D.H, w.w_qkvg, w.s_qkvg, D.Nqkvg, EPI_STORE_ACT, ws + W.qkvg, D.Nqkvg, 1)), "gemm qkvg");
    ra.qkvg = ws + W.qkvg;
    ra.in_f32 = 0;
  }
  const bool full = ctx->is_full(l);
  const int sidx = ctx->stream_of(l, slot);
  ra.splits = S;
  ra.M = M;
  ra.Hq = D.Hq;
  ra.Hkv = D.Hkv;
  ra.d = D.d;
  ra.Nqkvg = D.Nqkvg;
  ra.gate = D.Ng > 0;
  ra.pos = meta;
  ra.row_seq = meta + c.max_rows;
  ra.freq = (const double*)(meta + 2 * c.max_rows + 4 * D.max_tiles) + (full ? 128 : 0);
  ra.qk_norm = c.qk_norm;
  ra.s_qk = w.s_qk;
  ra.q_out = ws + W.q;
  ra.kv = kv_layout(ctx, l);
  ra.stream_idx = sidx;
  ra.tiles = meta + 2 * c.max_rows;
  ra.n_tiles = P.n_tiles;
  const bool tiled = !ra.in_f32 && P.max_tile_rows > 1 && (D.d == 64 || D.d == 128 || D.d == 160);
  // the MFMA prefill kernel takes the gate in bf16: small chunks, whose projection
  // leaves float split partials, use the row-wise kernels
  const bool mfma_attn = !f32 && !(ra.in_f32 && D.Ng) && P.max_tile_rows > 1 && D.Hq == 4 * D.Hkv &&
                         (D.d == 64 || D.d == 128 || D.d == 160);
  // with both, the attention rotates q as it loads it and the RoPE kernel does K and V
  const bool q_in_attn = tiled && mfma_attn;
  if (tiled) ra.cs = (const float*)(ws + W.rcs) + (full ? rope_table_floats(D) : 0);
  if (q_in_attn) ra.q_out = nullptr;
  {
    Prof pr(ctx, st, DORY_KC_ROPE);
    HIPCHK(tiled ? launch_rope_kv_tiles(ra, st) : launch_rope_kv(ra, st), "rope_kv");
    const double qb = q_in_attn ? 0.0 : 2.0 * D.Nq * D.esz;  // q read and written
    pr.end(0, tiled ? (double)M * (qb + 4.0 * D.Nkv * D.esz)
                    : (double)M * (D.Nqkvg * (ra.in_f32 ? 4.0 * S : D.esz) + (2 * D.Nq + 2 * D.Nkv) * D.esz));
  }

  AttnArgs aa;
  aa.q = ws + W.q;
  if (q_in_attn) {
    aa.q_raw = ws + W.qkvg;
    aa.q_ld = D.Nqkvg;
    aa.rope_cs = ra.cs;
  }
  if (D.Ng) {  // the gate columns of the [q|k|v|gate] projection output
    const int gcol = D.Nq + 2 * D.Nkv;
    aa.g_ld = D.Nqkvg;
    if (ra.in_f32) {
      aa.g = (const float*)ra.qkvg + gcol;
      aa.g_f32 = 1;
      aa.g_splits = S;
      aa.g_sstride = (size_t)M * D.Nqkvg;
    } else {
      aa.g = (const uint16_t*)ra.qkvg + gcol;  // bf16 elements
    }
  }
  aa.M = M;
  aa.Hq = D.Hq;
  aa.Hkv = D.Hkv;
  aa.d = D.d;
  aa.pos = meta;
  aa.row_seq = meta + c.max_rows;
  aa.window = full ? 0 : c.window;
  aa.scale = c.attn_scale;
  aa.s_qk = c.qk_norm ? w.s_qk : nullptr;
  aa.kv = ra.kv;
  aa.stream_idx = sidx;
  aa.max_pos = P.max_pos;
  aa.part = (float*)(ws + W.apart);
  aa.part_cap = (int)std::min<size_t>(W.apart_floats, 0x7fffffff);
  aa.o = ws + W.o;
  aa.tiles = meta + 2 * c.max_rows;
  aa.n_tiles = P.n_tiles;
  aa.max_tile_rows = P.max_tile_rows;
  aa.n_quads = P.n_quads;
  {
    double pairs, keys;
    attn_work(P, full, c.window, &pairs, &keys);
    int splits = 1;
    {
      // the prefill kernel also applies the gate and writes o; the split-key kernel reads
      // K, V and q and leaves the rest to the merge
      Prof pr(ctx, st, DORY_KC_ATTN);
      if (mfma_attn)
        HIPCHK(launch_attn_prefill(aa, st), "attention (prefill)");
      else
        HIPCHK(launch_attn_rows(aa, ATTN_SPLITS, &splits, st), "attention");
      pr.end(4.0 * D.Hq * D.d * pairs,
             keys * 2.0 * D.Nkv * D.esz + (double)M * (mfma_attn ? 3 : 1) * D.Nq * D.esz);
    }
    if (!mfma_attn) {
      Prof pr(ctx, st, DORY_KC_MERGE);
      HIPCHK(launch_attn_rows(aa, ATTN_MERGE, &splits, st), "attention merge");
      pr.end(0, (double)M * D.Hq * splits * (D.d + 2) * 4 + (double)M * D.Nq * (2 * D.esz + (f32 ? 4.0 * S : 0)));
    }
  }

  // ---- output projection + nGPT update (the pre-projection norm cancels in N(y))
  if (f32) {
    HIPCHK(run_gemm(gemm(ws + W.o, D.Nq, w.w_o, nullptr, D.H, EPI_F32, part, D.H, 1)), "gemm o");
    HIPCHK(update(1, w.alpha_attn, BND_NONE, nullptr), "update attn");
  } else if (skinny) {
    S = gemm_pick_splits(M, D.H, D.Nq, wf);
    HIPCHK(run_gemm(gemm(ws + W.o, D.Nq, w.w_o, w.s_o, D.H, EPI_PARTIAL, part, D.H, S)), "gemm o");
    HIPCHK(update(S, w.alpha_attn, BND_NONE, nullptr), "update attn");
  } else {  // prefill: the sublayer output in the activation type (bf16)
    HIPCHK(run_gemm(gemm(ws + W.o, D.Nq, w.w_o, w.s_o, D.H, EPI_STORE_ACT, part, D.H, 1)), "gemm o");
    HIPCHK(update(1, w.alpha_attn, BND_NONE, nullptr, true), "update attn");
  }

  // ---- MLP sublayer
  if (f32 || skinny) {
    S = f32 ? 1 : gemm_pick_splits(M, 2 * D.I, D.H, wf);
    HIPCHK(run_gemm(gemm(ws + W.sb, D.H, w.w_gu, w.s_gu, 2 * D.I, f32 ? EPI_F32 : EPI_PARTIAL, part, 2 * D.I, S)), "gemm gu");
    {
      Prof pr(ctx, st, DORY_KC_SWIGLU);
      HIPCHK(launch_swiglu(part, S, M, D.I, ws + W.h, act, st), "swiglu");
      pr.end(0, (double)M * (2.0 * D.I * 4 * S + D.I * D.esz));
    }
    S = f32 ? 1 : gemm_pick_splits(M, D.H, D.I, wf);
    HIPCHK(run_gemm(gemm(ws + W.h, D.I, w.w_down, w.s_down, D.H, f32 ? EPI_F32 : EPI_PARTIAL, part, D.H, S)), "gemm down");
    HIPCHK(update(S, w.alpha_mlp, bnd, out), "update mlp");
  } else {
    GemmArgs g = gemm(ws + W.sb, D.H, w.w_gu, w.s_gu, 2 * D.I, EPI_SWIGLU, ws + W.h, D.I, 1);
    g.n_half = D.I;
    HIPCHK(run_gemm(g), "gemm gu");
    HIPCHK(run_gemm(gemm(ws + W.h, D.I, w.w_down, w.s_down, D.H, EPI_STORE_ACT, part, D.H, 1)), "gemm down");
    HIPCHK(update(1, w.alpha_mlp, bnd, out, true), "update mlp");
  }
  return DORY_OK;
}

int run_forward(dory_ctx* ctx, hipStream_t st, const CallPlan& P, const float* x_in, float* y_out) {
  const dory_config& c = ctx->cfg;
  char* ws = ctx->ws;
  const int act = c.act_dtype == DORY_DTYPE_F32 ? ACT_F32 : ACT_BF16;
  const int R = c.max_rows;
  const int32_t* rowmap = P.reordered ? (const int32_t*)(ws + ctx->W.meta) + 2 * R + 4 * ctx->D.max_tiles + ROPE_INTS
                                      : nullptr;
  const int H = ctx->D.H;
  // rows of the workspace state (internal order) into a caller-order array
  auto export_rows = [&](size_t off, float* dst, const char* what) -> int {
    Prof pr(ctx, st, DORY_KC_UPDATE);
    if (rowmap)
      HIPCHK(launch_scatter_rows((const float*)(ws + off), rowmap, P.M, H, dst, st), what);
    else
      HIPCHK(hipMemcpyAsync(dst, ws + off, (size_t)P.M * H * 4, hipMemcpyDeviceToDevice, st), what);
    pr.end(0, (double)P.M * H * 8.0);
    return DORY_OK;
  };
  if (act == ACT_BF16 && P.max_tile_rows > 1 && P.n_tiles > 0) {  // RoPE (cos, sin) of every tile row, both bases
    const int half = ctx->D.d / 2;
    const int32_t* meta = (const int32_t*)(ws + ctx->W.meta);
    Prof pr(ctx, st, DORY_KC_ROPE);
    HIPCHK(launch_rope_table(meta + 2 * R, P.n_tiles, (const double*)(meta + 2 * R + 4 * ctx->D.max_tiles), half,
                             rope_table_floats(ctx->D), (float*)(ws + ctx->W.rcs), st),
           "rope table");
    pr.end(0, (double)P.M * half * 16.0);
  }
  int64_t calls = 0;
  int r;
  auto injected = [&]() {
    return P.inject_at == calls + 1 ? ctx->fail(DORY_ERR_HIP, "injected failure before layer call %lld", (long long)(calls + 1))
                                    : DORY_OK;
  };
  if (P.res_x) {  // start at loop 2 from the given x and s_1
    Prof pr(ctx, st, DORY_KC_UPDATE);
    HIPCHK(launch_resume_state(P.res_x, P.res_s1, rowmap, P.M, H, (float*)(ws + ctx->W.x), (float*)(ws + ctx->W.s),
                               ws + ctx->W.sb, act, st),
           "resume state");
    pr.end(0, (double)P.M * H * (16.0 + 8.0 + ctx->D.esz));
  } else {
    Trace tb("input block");
    {
      Prof pr(ctx, st, DORY_KC_UPDATE);
      HIPCHK(launch_stage_input(x_in, P.act_state ? nullptr : (float*)(ws + ctx->W.s), ws + ctx->W.sb, P.M, H, act,
                                st, rowmap, P.act_state ? ws + ctx->W.s16 : nullptr),
             "stage_input");
      pr.end(0, (double)P.M * H * ((P.act_state ? 6.0 : 8.0) + ctx->D.esz));
    }
    for (int l = 0; l < c.n_in; ++l) {
      if ((r = injected()) || (r = run_layer(ctx, st, P, l, 0, l == c.n_in - 1 ? BND_SAVE_X : BND_NONE, nullptr))) return r;
      ++calls;
    }
    if (P.cap_x && (r = export_rows(ctx->W.x, P.cap_x, "capture x"))) return r;
  }
  // loop t runs the recurrent block on the rows of the sequences with k >= t (a prefix);
  // rows whose sequence ends at loop t take the final boundary there
  for (int t = P.res_x ? 2 : 1; t <= P.k_max; ++t) {
    Trace tt("loop %d of %d", t, P.k_max);
    CallPlan Pt = P;
    Pt.M = P.loop_rows[t];
    Pt.n_tiles = P.loop_tiles[t];
    Pt.n_quads = P.loop_quads[t];
    Pt.chunks.resize(P.loop_seqs[t]);
    const int slot = ctx->mode == DORY_KV_PER_LOOP ? t - 1 : 0;
    const int next = t < P.k_max ? P.loop_rows[t + 1] : 0;
    for (int l = c.n_in; l < c.n_in + c.n_rec; ++l) {
      int b = BND_NONE;
      if (l == c.n_in + c.n_rec - 1) b = t < P.k_max ? BND_LOOP_CONTINUE : BND_LOOP_FINAL;
      if ((r = injected()) || (r = run_layer(ctx, st, Pt, l, slot, b, nullptr, next))) return r;
      ++calls;
    }
    if (t == 1 && P.cap_s1 && (r = export_rows(ctx->W.s, P.cap_s1, "capture s1"))) return r;
  }
  if (P.skip_out) {
    ctx->last_calls = calls;
    return DORY_OK;
  }
  Trace to("output block");
  const int L = c.n_in + c.n_rec + c.n_out;
  for (int l = c.n_in + c.n_rec; l < L; ++l) {
    // the last layer's update writes the float result: into the caller's array, or into
    // the state array that the row scatter reads
    float* out = l < L - 1 ? nullptr : P.reordered ? (float*)(ws + ctx->W.s) : y_out;
    if ((r = injected()) || (r = run_layer(ctx, st, P, l, 0, BND_NONE, out))) return r;
    ++calls;
  }
  if (P.reordered) {
    Prof pr(ctx, st, DORY_KC_UPDATE);
    HIPCHK(launch_scatter_rows((const float*)(ws + ctx->W.s), rowmap, P.M, ctx->D.H, y_out, st), "output rows");
    pr.end(0, (double)P.M * ctx->D.H * 8.0);
  }
  ctx->last_calls = calls;
  return DORY_OK;
}

// Loop count a sequence runs with: the count set for it, else per_loop sequences the k
// their cache was built for and last_loop sequences the context's.
int loops_of(const dory_ctx* ctx, const Seq& q) {
  if (ctx->mode == DORY_KV_PER_LOOP) return q.k_set ? q.k_set : q.k_built;
  return q.k_set ? q.k_set : ctx->k;
}

// Shared body of prefill and decode: rows of each sequence, grown by n_new[i].
int step(dory_ctx* ctx, hipStream_t st, int n, const int32_t* ids, const int32_t* n_new,
         const float* x_in, float* y_out, bool decode) {
  Trace tc("%s: %d sequences", decode ? "dory_decode_step" : "dory_prefill", n);
  const dory_config& c = ctx->cfg;
  float* const cap_x = ctx->cap_x;  // one-shot: consumed by this call whatever its outcome
  float* const cap_s1 = ctx->cap_s1;
  const bool skip_out = ctx->cap_skip_out;
  const float* const res_x = ctx->res_x;
  const float* const res_s1 = ctx->res_s1;
  ctx->cap_x = ctx->cap_s1 = nullptr;
  ctx->cap_skip_out = false;
  ctx->res_x = ctx->res_s1 = nullptr;
  if (!bound(ctx)) return ctx->fail(DORY_ERR_STATE, "weights, KV pool and workspace must be bound");
  if (n < 1 || !ids || (!decode && !n_new) || !x_in || !y_out)
    return ctx->fail(DORY_ERR_INVALID_ARG, "null argument or n_seqs < 1");
  if (((uintptr_t)x_in | (uintptr_t)y_out) & 15) return ctx->fail(DORY_ERR_INVALID_ARG, "x_in and y_out must be 16-byte aligned");
  std::set<int32_t> seen;
  int64_t rows = 0;
  int n_newseq = 0;
  for (int i = 0; i < n; ++i) {
    if (!seen.insert(ids[i]).second) return ctx->fail(DORY_ERR_INVALID_ARG, "sequence id %d repeated", ids[i]);
    const int64_t nn = decode ? 1 : n_new[i];
    if (nn < 1) return ctx->fail(DORY_ERR_INVALID_ARG, "n_new[%d] < 1", i);
    auto it = ctx->seqs.find(ids[i]);
    const int64_t len = it == ctx->seqs.end() ? 0 : it->second.len;
    if (it == ctx->seqs.end()) {
      if (decode) return ctx->fail(DORY_ERR_INVALID_ARG, "decode of unknown sequence %d", ids[i]);
      ++n_newseq;
    }
    if (len + nn > c.max_seq_len)
      return ctx->fail(DORY_ERR_INVALID_ARG, "sequence %d would reach position %lld >= max_seq_len %d",
                       ids[i], (long long)(len + nn - 1), c.max_seq_len);
    rows += nn;
  }
  if (rows > c.max_rows) return ctx->fail(DORY_ERR_INVALID_ARG, "%lld rows > max_rows %d", (long long)rows, c.max_rows);
  if ((int64_t)ctx->seqs.size() + n_newseq > c.max_seqs)
    return ctx->fail(DORY_ERR_INVALID_ARG, "more than max_seqs %d live sequences", c.max_seqs);
  // pages (transactional)
  int64_t need = 0;
  for (int i = 0; i < n; ++i) {
    auto it = ctx->seqs.find(ids[i]);
    Seq probe;
    if (it != ctx->seqs.end()) probe = it->second;
    else probe.rec_slots = ctx->mode == DORY_KV_PER_LOOP ? ctx->k : 1;
    need += pages_to_grow(ctx, probe, probe.len + (decode ? 1 : n_new[i]));
  }
  if (need > (int64_t)ctx->free_pages.size())
    return ctx->fail(DORY_ERR_OUT_OF_KV, "need %lld KV pages, %zu free", (long long)need, ctx->free_pages.size());
  const int inject = ctx->inject_at;  // test hook, consumed by this call
  ctx->inject_at = -1;

  // commit: create, grow, build row metadata
  std::vector<int32_t>& meta = ctx->scratch;
  const int R = c.max_rows;
  meta.assign(3 * (size_t)R + 4 * (size_t)ctx->D.max_tiles + ROPE_INTS, 0);
  {  // RoPE frequencies theta^(-2i/d), sliding base then full base
    double* fr = (double*)(meta.data() + 2 * (size_t)R + 4 * (size_t)ctx->D.max_tiles);
    const int d = ctx->D.d;
    for (int i = 0; i < d / 2; ++i) {
      fr[i] = std::pow(c.theta_swa, -2.0 * i / d);
      fr[128 + i] = std::pow(c.theta_full, -2.0 * i / d);
    }
  }
  // loop count of each sequence of the call; the plan orders sequences by it, largest
  // first (stable), so that the rows still looping in loop t form a prefix
  std::vector<int> kseq(n), order(n);
  std::vector<int64_t> caller_row(n);
  {
    int64_t cr = 0;
    for (int i = 0; i < n; ++i) {
      auto it = ctx->seqs.find(ids[i]);
      kseq[i] = it == ctx->seqs.end() ? ctx->k : loops_of(ctx, it->second);
      caller_row[i] = cr;
      cr += decode ? 1 : n_new[i];
      order[i] = i;
    }
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return kseq[a] > kseq[b]; });
  }
  for (int i = 0; i < n; ++i) {
    if (cap_x && kseq[i] != 1)
      return ctx->fail(DORY_ERR_INVALID_ARG, "capture needs every sequence at one loop (sequence %d runs %d)", ids[i],
                       kseq[i]);
    if (res_x && kseq[i] < 2)
      return ctx->fail(DORY_ERR_INVALID_ARG, "resume needs every sequence at two loops or more (sequence %d runs %d)",
                       ids[i], kseq[i]);
  }
  int r = enter(ctx, st);
  if (r) return r;
  // what the commit changes, so that a failure after it can be undone
  Journal jr;
  jr.pending = ctx->pending;
  CallPlan P;
  P.inject_at = inject;
  P.cap_x = cap_x;
  P.cap_s1 = cap_s1;
  P.skip_out = skip_out;
  P.res_x = res_x;
  P.res_s1 = res_s1;
  P.k_max = kseq[order[0]];
  P.loop_rows.assign(P.k_max + 2, 0);
  P.loop_tiles.assign(P.k_max + 2, 0);
  P.loop_quads.assign(P.k_max + 2, 0);
  P.loop_seqs.assign(P.k_max + 2, 0);
  for (int i = 0; i < n; ++i) P.reordered |= order[i] != i;
  int row = 0;
  for (int oi = 0; oi < n; ++oi) {
    const int i = order[oi];
    auto it = ctx->seqs.find(ids[i]);
    if (it == ctx->seqs.end()) {
      Seq q;
      q.id = ids[i];
      q.slot = ctx->free_slots.back();
      ctx->free_slots.pop_back();
      q.k_built = ctx->k;
      q.rec_slots = ctx->mode == DORY_KV_PER_LOOP ? ctx->k : 1;
      q.pages.assign(ctx->D.n_streams, {});
      it = ctx->seqs.emplace(ids[i], std::move(q)).first;
      jr.created.push_back(ids[i]);
    } else {
      jr.lens.emplace_back(ids[i], it->second.len);
    }
    Seq& q = it->second;
    const int nn = decode ? 1 : n_new[i];
    const int64_t p0 = q.len;
    grow(ctx, q, q.len + nn, &jr.taken);
    for (int j = 0; j < nn; ++j) {
      meta[row + j] = (int32_t)(p0 + j);
      meta[R + row + j] = q.slot;
      meta[2 * R + 4 * ctx->D.max_tiles + ROPE_INTS + row + j] = (int32_t)(caller_row[i] + j);
    }
    for (int j = 0; j < nn; j += 64) {  // prefill tiles of <= 64 rows
      int32_t* tl = &meta[2 * R + 4 * P.n_tiles];
      tl[0] = row + j;
      tl[1] = std::min(64, nn - j);
      tl[2] = (int32_t)(p0 + j);
      tl[3] = q.slot;
      ++P.n_tiles;
      P.n_quads += (tl[1] + 3) / 4;
    }
    P.max_tile_rows = std::min(64, std::max(P.max_tile_rows, nn));
    P.chunks.emplace_back(p0, nn);
    P.max_pos = std::max<int>(P.max_pos, (int)(p0 + nn - 1));
    row += nn;
    for (int t = 1; t <= kseq[i]; ++t) {  // prefixes: this sequence loops in loops 1..k
      P.loop_rows[t] = row;
      P.loop_tiles[t] = P.n_tiles;
      P.loop_quads[t] = P.n_quads;
      P.loop_seqs[t] = oi + 1;
    }
  }
  P.M = row;
  {  // fp16 state when every layer call of this call takes the vectorised prefill update
    int min_rows = P.M;
    for (int t = 1; t <= P.k_max; ++t) min_rows = std::min(min_rows, P.loop_rows[t]);
    P.act_state = c.act_dtype != DORY_DTYPE_F32 && min_rows >= ACT_STATE_MIN_ROWS && !P.cap_x && !P.cap_s1 &&
                  !P.res_x && !P.skip_out;
  }
  r = [&]() -> int {
    // deltas: whatever does not fit goes first in separate uploads
    int rr;
    if ((rr = flush_deltas(ctx, st, DELTA_CAP))) return rr;
    const size_t nd = ctx->pending.size() / 2;
    meta.insert(meta.end(), ctx->pending.begin(), ctx->pending.end());
    ctx->pending.clear();
    if (inject == 0) return ctx->fail(DORY_ERR_HIP, "injected failure at the metadata upload");
    if ((rr = upload(ctx, st, meta.data(), meta.size()))) return rr;
    if (nd)
      HIPCHK(launch_apply_deltas((int32_t*)(ctx->ws + ctx->W.table),
                                 (const int32_t*)(ctx->ws + ctx->W.meta) + 3 * R + 4 * ctx->D.max_tiles + ROPE_INTS,
                                 (int)nd, ctx->pool, ctx->D.page_bytes, st), "apply_deltas");
    return run_forward(ctx, st, P, x_in, y_out);
  }();
  if (r) rollback(ctx, std::move(jr));
  const int rl = leave(ctx, st);
  return r ? r : rl;
}

int logits_check(dory_ctx* ctx, int n, const float* states, float* logits) {
  if (!ctx->vocab_bound) return ctx->fail(DORY_ERR_STATE, "vocabulary not bound");
  if (n < 1 || n > ctx->cfg.max_rows || !states || !logits)
    return ctx->fail(DORY_ERR_INVALID_ARG, "need 1 <= n <= max_rows and non-null states, logits");
  return DORY_OK;
}

// split-K factor of the LM-head GEMM for n rows (1 in fp32 contexts and above the
// split-K sizes)
int logits_splits(const dory_ctx* ctx, int n) {
  if (ctx->cfg.act_dtype == DORY_DTYPE_F32 || n > SKINNY_M) return 1;
  return gemm_pick_splits(n, (int)ctx->vocab.vocab, ctx->D.H, W_BF16);
}

// The LM head: logits = s_z * (states . lm_head) over n rows. bf16 contexts stage the
// states (float copy s_buf, bf16 copy sb_buf, n x H each) and, with splits > 1, take
// fp32 split-K partials in part (splits x n x V) that the logit-scale kernel sums.
int logits_run(dory_ctx* ctx, hipStream_t st, int n, const float* states, float* logits, float* s_buf, void* sb_buf,
               float* part, int splits) {
  const int H = ctx->D.H;
  const int64_t V = ctx->vocab.vocab;
  const bool f32 = ctx->cfg.act_dtype == DORY_DTYPE_F32;
  GemmArgs g;
  g.B = ctx->vocab.lm_head;
  g.M = n;
  g.N = (int)V;
  g.K = H;
  g.lda = H;
  g.C = logits;
  g.ldc = (int)V;
  if (f32) {
    g.A = states;
    g.act = ACT_F32;
    g.wfmt = W_F32;
    g.epi = EPI_F32;
  } else {
    g.A = sb_buf;  // the states in the activation type, as the projections read them
    g.act = ACT_BF16;
    g.wfmt = W_BF16;
    if (n <= SKINNY_M) {  // decode-sized: split-K streaming tiles
      g.epi = EPI_PARTIAL;
      g.splits = splits;
      if (splits > 1) g.C = part;
    } else {
      g.epi = EPI_F32;
    }
    Prof ps(ctx, st, DORY_KC_UPDATE);
    HIPCHK(launch_stage_input(states, s_buf, sb_buf, n, H, ACT_BF16, st), "LM-head input");
    ps.end(0.0, (double)n * H * (4 + 4 + 2));
  }
  {
    Prof pr(ctx, st, DORY_KC_VOCAB);
    HIPCHK(launch_gemm(g, st), "LM-head GEMM");
    pr.end(2.0 * n * (double)V * H, (double)V * H * ctx->D.esz + (double)n * H * ctx->D.esz + 4.0 * n * V * splits);
  }
  Prof pr(ctx, st, DORY_KC_VOCAB);
  HIPCHK(launch_logit_scale(splits > 1 ? part : logits, splits, (size_t)n * V, logits, V, n, V, ctx->vocab.logit_scale,
                            st),
         "logit scale");
  pr.end(0.0, 4.0 * n * V * (splits + 1) + 4.0 * V);
  return DORY_OK;
}

}  // namespace

// ============================================================================ C ABI
extern "C" {

int dory_create(const dory_config* cfg, dory_ctx** out) {
  if (!out) {
    g_create_err = "null output pointer";
    return DORY_ERR_INVALID_ARG;
  }
  *out = nullptr;
  std::string msg;
  const int r = check_config(cfg, msg);
  if (r) {
    g_create_err = msg;
    return r;
  }
  dory_ctx* c = new dory_ctx();
  c->cfg = *cfg;
  c->D = dims_of(*cfg);
  c->W = layout_of(*cfg, c->D);
  c->k = std::min(2, cfg->max_loops);
  c->lw.assign(c->D.L, dory_layer_weights{});
  c->lw_bound.assign(c->D.L, false);
  for (int i = cfg->max_seqs - 1; i >= 0; --i) c->free_slots.push_back(i);
  g_create_err.clear();
  *out = c;
  return DORY_OK;
}

int dory_destroy(dory_ctx* ctx) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  for (auto e : ctx->pev) {
    (void)hipEventSynchronize(e);
    (void)hipEventDestroy(e);
  }
  if (ctx->done_ev) {
    (void)hipEventSynchronize(ctx->done_ev);
    (void)hipEventDestroy(ctx->done_ev);
  }
  for (int i = 0; i < NSTAGE; ++i) {
    if (ctx->ev[i]) {
      (void)hipEventSynchronize(ctx->ev[i]);
      (void)hipEventDestroy(ctx->ev[i]);
    }
    if (ctx->stage[i]) (void)hipHostFree(ctx->stage[i]);
  }
  delete ctx;
  return DORY_OK;
}

const char* dory_last_error(const dory_ctx* ctx) {
  return ctx ? ctx->err.c_str() : g_create_err.c_str();
}

int dory_query_sizes(const dory_config* cfg, size_t* page_bytes, size_t* workspace_bytes) {
  std::string msg;
  const int r = check_config(cfg, msg);
  if (r) {
    g_create_err = msg;
    return r;
  }
  const Dims D = dims_of(*cfg);
  if (page_bytes) *page_bytes = D.page_bytes;
  if (workspace_bytes) *workspace_bytes = layout_of(*cfg, D).total;
  return DORY_OK;
}

int dory_kv_pages_needed(const dory_config* cfg, int mode, int k, int64_t seq_len, int64_t n_seqs,
                         int64_t* pages) {
  std::string msg;
  const int r = check_config(cfg, msg);
  if (r) {
    g_create_err = msg;
    return r;
  }
  if (!pages || (mode != DORY_KV_PER_LOOP && mode != DORY_KV_LAST_LOOP) || k < 1 ||
      k > cfg->max_loops || seq_len < 0 || n_seqs < 0) {
    g_create_err = "bad argument";
    return DORY_ERR_INVALID_ARG;
  }
  const Dims D = dims_of(*cfg);
  int64_t per = 0;
  const int L = D.L;
  for (int l = 0; l < L; ++l) {
    const bool full = l % cfg->full_period == cfg->full_period - 1;
    const bool rec = l >= cfg->n_in && l < cfg->n_in + cfg->n_rec;
    const int slots = rec && mode == DORY_KV_PER_LOOP ? k : 1;
    per += slots * pages_for_stream(seq_len, full, full ? D.tab_len : D.ring_swa);
  }
  *pages = per * n_seqs;
  return DORY_OK;
}

int dory_bind_weights(dory_ctx* ctx, int layer, const dory_layer_weights* w) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (layer < 0 || layer >= ctx->D.L) return ctx->fail(DORY_ERR_INVALID_ARG, "layer %d out of range", layer);
  if (!w || !w->w_qkvg || !w->w_o || !w->w_gu || !w->w_down || !w->alpha_attn || !w->alpha_mlp || !w->s_qk)
    return ctx->fail(DORY_ERR_INVALID_ARG, "null weight pointer");
  if (ctx->cfg.weight_format == DORY_WFMT_MXFP8 && (!w->s_qkvg || !w->s_o || !w->s_gu || !w->s_down))
    return ctx->fail(DORY_ERR_INVALID_ARG, "MXFP8 weights need scale arrays");
  if (ctx->cfg.weight_format == DORY_WFMT_NVFP4 &&
      (!w->s_qkvg || !w->s_o || !w->s_gu || !w->s_down || !w->g_qkvg || !w->g_o || !w->g_gu || !w->g_down))
    return ctx->fail(DORY_ERR_INVALID_ARG, "NVFP4 weights need block and matrix scales");
  const uintptr_t mask = 15;
  if (((uintptr_t)w->w_qkvg | (uintptr_t)w->w_o | (uintptr_t)w->w_gu | (uintptr_t)w->w_down) & mask)
    return ctx->fail(DORY_ERR_INVALID_ARG, "weight matrices must be 16-byte aligned");
  if (((uintptr_t)w->alpha_attn | (uintptr_t)w->alpha_mlp) & mask)
    return ctx->fail(DORY_ERR_INVALID_ARG, "alpha_attn and alpha_mlp must be 16-byte aligned");
  if ((w->f_qkvg || w->f_o || w->f_gu || w->f_down) && ctx->cfg.weight_format != DORY_WFMT_BF16)
    return ctx->fail(DORY_ERR_INVALID_ARG, "fragment-order copies are for bf16 weights");
  if (((uintptr_t)w->f_qkvg | (uintptr_t)w->f_o | (uintptr_t)w->f_gu | (uintptr_t)w->f_down) & mask)
    return ctx->fail(DORY_ERR_INVALID_ARG, "fragment-order copies must be 16-byte aligned");
  ctx->lw[layer] = *w;
  ctx->lw_bound[layer] = true;
  return DORY_OK;
}

int dory_bind_kv_pool(dory_ctx* ctx, void* pool, size_t bytes) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (!ctx->seqs.empty()) return ctx->fail(DORY_ERR_STATE, "sequences are live");
  if (!pool || ((uintptr_t)pool & 255)) return ctx->fail(DORY_ERR_INVALID_ARG, "pool must be non-null, 256-byte aligned");
  const int64_t n = (int64_t)(bytes / ctx->D.page_bytes);
  if (n < 1) return ctx->fail(DORY_ERR_INVALID_ARG, "pool smaller than one page (%zu bytes)", ctx->D.page_bytes);
  if (n > 0x7fffffff) return ctx->fail(DORY_ERR_INVALID_ARG, "too many pages");
  ctx->pool = pool;
  ctx->pool_bytes = bytes;
  ctx->n_pages = n;
  ctx->free_pages.clear();
  for (int64_t i = n - 1; i >= 0; --i) ctx->free_pages.push_back((int32_t)i);
  return DORY_OK;
}

int dory_bind_workspace(dory_ctx* ctx, void* ws, size_t bytes) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (!ctx->seqs.empty()) return ctx->fail(DORY_ERR_STATE, "sequences are live");
  if (!ws || ((uintptr_t)ws & 255)) return ctx->fail(DORY_ERR_INVALID_ARG, "workspace must be non-null, 256-byte aligned");
  if (bytes < ctx->W.total) return ctx->fail(DORY_ERR_INVALID_ARG, "workspace %zu < %zu bytes", bytes, ctx->W.total);
  ctx->ws = (char*)ws;
  ctx->ws_bytes = bytes;
  return DORY_OK;
}

int dory_set_loops(dory_ctx* ctx, int k) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (k < 1 || k > ctx->cfg.max_loops) return ctx->fail(DORY_ERR_INVALID_ARG, "k=%d outside 1..%d", k, ctx->cfg.max_loops);
  ctx->k = k;
  return DORY_OK;
}

int dory_set_seq_loops(dory_ctx* ctx, int32_t seq_id, int k) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  auto it = ctx->seqs.find(seq_id);
  if (it == ctx->seqs.end()) return ctx->fail(DORY_ERR_INVALID_ARG, "unknown sequence %d", seq_id);
  if (k < 0 || k > ctx->cfg.max_loops) return ctx->fail(DORY_ERR_INVALID_ARG, "k=%d outside 0..%d", k, ctx->cfg.max_loops);
  if (ctx->mode == DORY_KV_PER_LOOP && k > it->second.k_built)
    return ctx->fail(DORY_ERR_STATE, "per_loop sequence %d holds KV for k=%d", seq_id, it->second.k_built);
  it->second.k_set = k;
  return DORY_OK;
}

int dory_truncate_seq(dory_ctx* ctx, int32_t seq_id, int64_t len) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  auto it = ctx->seqs.find(seq_id);
  if (it == ctx->seqs.end()) return ctx->fail(DORY_ERR_INVALID_ARG, "unknown sequence %d", seq_id);
  if (len < 1 || len > it->second.len)
    return ctx->fail(DORY_ERR_INVALID_ARG, "length %lld outside 1..%lld", (long long)len, (long long)it->second.len);
  it->second.len = len;  // the pages stay with the sequence; later positions are rewritten before use
  return DORY_OK;
}

int dory_capture_states(dory_ctx* ctx, float* x_out, float* s1_out, int skip_output_block) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (!x_out || !s1_out) return ctx->fail(DORY_ERR_INVALID_ARG, "null capture buffer");
  ctx->cap_x = x_out;
  ctx->cap_s1 = s1_out;
  ctx->cap_skip_out = skip_output_block != 0;
  return DORY_OK;
}

int dory_resume_states(dory_ctx* ctx, const float* x_in, const float* s1_in) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (!x_in || !s1_in) return ctx->fail(DORY_ERR_INVALID_ARG, "null state buffer");
  ctx->res_x = x_in;
  ctx->res_s1 = s1_in;
  return DORY_OK;
}

int dory_spec_accept(void* stream, int n, int gamma, int64_t vocab, const float* draft_logits, int64_t ld_d,
                     const float* target_logits, int64_t ld_t, const int32_t* draft_tokens, float temperature,
                     float top_p, const float* u_accept, const float* u_sample, int32_t* tokens, int32_t* n_out) {
  if (n < 1 || gamma < 1 || gamma > 16 || vocab < 1 || vocab > (1 << 24) || ld_d < vocab || ld_t < vocab ||
      !draft_logits || !target_logits || !draft_tokens || !u_accept || !u_sample || !tokens || !n_out ||
      !(temperature > 0.f) || !std::isfinite(temperature) || !(top_p > 0.f) || !(top_p <= 1.f)) {
    g_create_err = "bad speculative-acceptance argument";
    return DORY_ERR_INVALID_ARG;
  }
  const hipError_t e = launch_spec_accept(n, gamma, vocab, draft_logits, ld_d, target_logits, ld_t, draft_tokens,
                                          temperature, top_p, u_accept, u_sample, tokens, n_out, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_create_err = hipGetErrorString(e);
    return DORY_ERR_HIP;
  }
  return DORY_OK;
}

int dory_seq_loops(const dory_ctx* ctx, int32_t seq_id, int* k) {
  if (!ctx || !k) return DORY_ERR_INVALID_ARG;
  auto it = ctx->seqs.find(seq_id);
  if (it == ctx->seqs.end()) return DORY_ERR_INVALID_ARG;
  *k = loops_of(ctx, it->second);
  return DORY_OK;
}

int dory_get_loops(const dory_ctx* ctx, int* k) {
  if (!ctx || !k) return DORY_ERR_INVALID_ARG;
  *k = ctx->k;
  return DORY_OK;
}

int dory_set_kv_mode(dory_ctx* ctx, int mode) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (mode != DORY_KV_PER_LOOP && mode != DORY_KV_LAST_LOOP) return ctx->fail(DORY_ERR_INVALID_ARG, "bad mode %d", mode);
  if (!ctx->seqs.empty()) return ctx->fail(DORY_ERR_STATE, "sequences are live");
  ctx->mode = mode;
  return DORY_OK;
}

int dory_get_kv_mode(const dory_ctx* ctx, int* mode) {
  if (!ctx || !mode) return DORY_ERR_INVALID_ARG;
  *mode = ctx->mode;
  return DORY_OK;
}

int dory_prefill(dory_ctx* ctx, void* stream, int n_seqs, const int32_t* seq_ids, const int32_t* n_new,
                 const float* x_in, float* y_out) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  return step(ctx, (hipStream_t)stream, n_seqs, seq_ids, n_new, x_in, y_out, false);
}

int dory_decode_step(dory_ctx* ctx, void* stream, int n_seqs, const int32_t* seq_ids, const float* x_in,
                     float* y_out) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  return step(ctx, (hipStream_t)stream, n_seqs, seq_ids, nullptr, x_in, y_out, true);
}

int dory_release_seq(dory_ctx* ctx, int32_t seq_id) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  auto it = ctx->seqs.find(seq_id);
  if (it == ctx->seqs.end()) return ctx->fail(DORY_ERR_INVALID_ARG, "unknown sequence %d", seq_id);
  release(ctx, it->second);
  ctx->seqs.erase(it);
  return DORY_OK;
}

int dory_seq_len(const dory_ctx* ctx, int32_t seq_id, int64_t* len) {
  if (!ctx || !len) return DORY_ERR_INVALID_ARG;
  auto it = ctx->seqs.find(seq_id);
  if (it == ctx->seqs.end()) return DORY_ERR_INVALID_ARG;
  *len = it->second.len;
  return DORY_OK;
}

int dory_live_seqs(const dory_ctx* ctx, int32_t* n) {
  if (!ctx || !n) return DORY_ERR_INVALID_ARG;
  *n = (int32_t)ctx->seqs.size();
  return DORY_OK;
}

int dory_kv_bytes_in_use(const dory_ctx* ctx, size_t* bytes) {
  if (!ctx || !bytes) return DORY_ERR_INVALID_ARG;
  *bytes = (size_t)(ctx->n_pages - (int64_t)ctx->free_pages.size()) * ctx->D.page_bytes;
  return DORY_OK;
}

int dory_last_layer_calls(const dory_ctx* ctx, int64_t* n) {
  if (!ctx || !n) return DORY_ERR_INVALID_ARG;
  *n = ctx->last_calls;
  return DORY_OK;
}

int dory_test_reserve(dory_ctx* ctx, int32_t seq_id, int32_t n_tokens) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (!ctx->pool || !ctx->ws) return ctx->fail(DORY_ERR_STATE, "KV pool and workspace must be bound");
  if (n_tokens < 1) return ctx->fail(DORY_ERR_INVALID_ARG, "n_tokens < 1");
  auto it = ctx->seqs.find(seq_id);
  if (it == ctx->seqs.end() && (int)ctx->seqs.size() >= ctx->cfg.max_seqs)
    return ctx->fail(DORY_ERR_INVALID_ARG, "more than max_seqs live sequences");
  Seq probe;
  if (it != ctx->seqs.end()) probe = it->second;
  else probe.rec_slots = ctx->mode == DORY_KV_PER_LOOP ? ctx->k : 1;

  if (probe.len + n_tokens > ctx->cfg.max_seq_len)
    return ctx->fail(DORY_ERR_INVALID_ARG, "sequence would exceed max_seq_len");
  const int64_t need = pages_to_grow(ctx, probe, probe.len + n_tokens);
  if (need > (int64_t)ctx->free_pages.size())
    return ctx->fail(DORY_ERR_OUT_OF_KV, "need %lld KV pages, %zu free", (long long)need, ctx->free_pages.size());
  if (it == ctx->seqs.end()) {
    Seq q;
    q.id = seq_id;
    q.slot = ctx->free_slots.back();
    ctx->free_slots.pop_back();
    q.k_built = ctx->k;
    q.rec_slots = probe.rec_slots;
    q.pages.assign(ctx->D.n_streams, {});
    it = ctx->seqs.emplace(seq_id, std::move(q)).first;
  }
  grow(ctx, it->second, it->second.len + n_tokens);
  return DORY_OK;
}

int dory_test_inject_failure(dory_ctx* ctx, int at) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (at < -1) return ctx->fail(DORY_ERR_INVALID_ARG, "at must be >= -1");
  ctx->inject_at = at;
  return DORY_OK;
}

int dory_test_fill_kv(dory_ctx* ctx, void* stream, int32_t seq_id, int layer, int slot, int32_t pos0,
                      int32_t n, const void* k, const void* v) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  auto it = ctx->seqs.find(seq_id);
  if (it == ctx->seqs.end()) return ctx->fail(DORY_ERR_INVALID_ARG, "unknown sequence %d", seq_id);
  const Seq& q = it->second;
  if (layer < 0 || layer >= ctx->D.L) return ctx->fail(DORY_ERR_INVALID_ARG, "layer out of range");
  const bool rec = layer >= ctx->cfg.n_in && layer < ctx->cfg.n_in + ctx->cfg.n_rec;
  if (slot < 0 || slot >= (rec ? q.rec_slots : 1)) return ctx->fail(DORY_ERR_INVALID_ARG, "slot out of range");
  if (!k || !v || n < 1 || pos0 < 0 || pos0 + (int64_t)n > q.len)
    return ctx->fail(DORY_ERR_INVALID_ARG, "positions outside the sequence");
  if (!ctx->is_full(layer)) {
    const int64_t last_lp = (q.len - 1) / DORY_PAGE_TOKENS;
    const int64_t first_ok = std::max<int64_t>(0, (last_lp - ctx->D.ring_swa + 1) * DORY_PAGE_TOKENS);
    if (pos0 < first_ok) return ctx->fail(DORY_ERR_INVALID_ARG, "position %d left the sliding-window ring", pos0);
  }
  hipStream_t st = (hipStream_t)stream;
  int r = enter(ctx, st);
  if (r) return r;
  if (!(r = flush_deltas(ctx, st, 0))) {
    const hipError_t e = launch_fill_kv(kv_layout(ctx, layer), q.slot, ctx->stream_of(layer, slot), pos0, n, k, v, st);
    if (e != hipSuccess) r = hip_fail(ctx, e, "fill_kv");
  }
  const int rl = leave(ctx, st);
  return r ? r : rl;
}

int dory_bind_vocab(dory_ctx* ctx, const dory_vocab_weights* v) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (!v || !v->embed || !v->lm_head || !v->logit_scale) return ctx->fail(DORY_ERR_INVALID_ARG, "null vocabulary pointer");
  if (v->vocab < 128 || v->vocab > (1 << 24) || v->vocab % 128)
    return ctx->fail(DORY_ERR_INVALID_ARG, "vocabulary size must be a multiple of 128 in [128, 2^24]");
  if (((uintptr_t)v->embed | (uintptr_t)v->lm_head) & 15)
    return ctx->fail(DORY_ERR_INVALID_ARG, "vocabulary tables must be 16-byte aligned");
  ctx->vocab = *v;
  ctx->vocab_bound = true;
  return DORY_OK;
}

int dory_embed(dory_ctx* ctx, void* stream, int n, const int32_t* ids, float* x_out) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (!ctx->vocab_bound) return ctx->fail(DORY_ERR_STATE, "vocabulary not bound");
  if (n < 1 || n > ctx->cfg.max_rows || !ids || !x_out)
    return ctx->fail(DORY_ERR_INVALID_ARG, "need 1 <= n <= max_rows and non-null ids, x_out");
  hipStream_t st = (hipStream_t)stream;
  Prof pr(ctx, st, DORY_KC_VOCAB);
  HIPCHK(launch_embed(ctx->vocab.embed, ctx->cfg.act_dtype == DORY_DTYPE_BF16, ctx->vocab.vocab, ctx->D.H, ids, n,
                      x_out, st),
         "embedding");
  pr.end(0.0, (double)n * ctx->D.H * (ctx->D.esz + 4) + 4.0 * n);
  return DORY_OK;
}

int dory_logits(dory_ctx* ctx, void* stream, int n, const float* states, float* logits) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  if (!ctx->ws) return ctx->fail(DORY_ERR_STATE, "workspace not bound");
  int r = logits_check(ctx, n, states, logits);
  if (r) return r;
  hipStream_t st = (hipStream_t)stream;
  const int splits = logits_splits(ctx, n);
  if ((size_t)splits * n * ctx->vocab.vocab > ctx->W.part_floats)
    return ctx->fail(DORY_ERR_UNSUPPORTED, "LM-head partials exceed the workspace");
  if ((r = enter(ctx, st))) return r;
  r = logits_run(ctx, st, n, states, logits, (float*)(ctx->ws + ctx->W.s), ctx->ws + ctx->W.sb,
                 (float*)(ctx->ws + ctx->W.part), splits);
  const int rl = leave(ctx, st);
  return r ? r : rl;
}

int dory_logits_noalloc(dory_ctx* ctx, void* stream, int n, const float* states, float* logits) {
  if (!ctx) return DORY_ERR_INVALID_ARG;
  int r = logits_check(ctx, n, states, logits);
  if (r) return r;
  const int splits = logits_splits(ctx, n);
  const bool f32 = ctx->cfg.act_dtype == DORY_DTYPE_F32;
  const size_t rows = f32 ? 0 : (size_t)n * ctx->D.H;
  const size_t o_sb = al(rows * 4), o_part = o_sb + al(rows * 2);
  const size_t need = o_part + (splits > 1 ? (size_t)splits * n * ctx->vocab.vocab * 4 : 0);
  if (need > NOALLOC_SCRATCH_BYTES)
    return ctx->fail(DORY_ERR_INVALID_ARG, "%d rows need %zu bytes of scratch, more than the %zu the library holds", n,
                     need, NOALLOC_SCRATCH_BYTES);
  void* base = nullptr;
  HIPCHK(noalloc_scratch(&base), "scratch address");
  char* b = (char*)base;
  return logits_run(ctx, (hipStream_t)stream, n, states, logits, (float*)b, b + o_sb, (float*)(b + o_part), splits);
}

int dory_sample_top_p(void* stream, int n, int64_t vocab, const float* logits, int64_t ld, float temperature,
                      float top_p, const float* u, int32_t* tokens) {
  if (n < 1 || vocab < 1 || vocab > (1 << 24) || ld < vocab || !logits || !u || !tokens ||
      !(temperature > 0.f) || !std::isfinite(temperature) || !(top_p > 0.f) || !(top_p <= 1.f)) {
    g_create_err = "bad sampling argument (need n >= 1, 1 <= vocab <= 2^24, ld >= vocab, temperature > 0, "
                   "0 < top_p <= 1, non-null pointers)";
    return DORY_ERR_INVALID_ARG;
  }
  const hipError_t e = launch_sample_top_p(logits, ld, n, vocab, temperature, top_p, u, tokens, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_create_err = hipGetErrorString(e);
    return DORY_ERR_HIP;
  }
  return DORY_OK;
}

int dory_test_gemm(void* stream, const void* A, int lda, const void* B, const uint8_t* B_scales,
                   const float* B_gscale, int wfmt, int M, int N, int K, int epi, void* C, int ldc, int* splits,
                   const void* B_frag) {
  const bool mx = wfmt == DORY_WFMT_MXFP8, nv = wfmt == DORY_WFMT_NVFP4;
  const bool ok_fmt = (wfmt == DORY_WFMT_BF16 && !B_scales && !B_gscale) || (mx && B_scales && !B_gscale) ||
                      (nv && B_scales && B_gscale);
  const bool ok_epi = epi == EPI_F32 || epi == EPI_PARTIAL || epi == EPI_STORE_ACT || epi == EPI_SWIGLU;
  if (!A || !B || !splits || !ok_fmt || !ok_epi || M < 1 || N < 64 || K < 64 || K % 64 || N % 64 ||
      (epi == EPI_SWIGLU && N % 128) || lda < K || (C && ldc < (epi == EPI_SWIGLU ? N / 2 : N)) ||
      ((mx || nv) && epi != EPI_PARTIAL) || (nv && N % 128) || (B_frag && (mx || nv || ((uintptr_t)B_frag & 15)))) {
    g_create_err = "bad GEMM argument";
    return DORY_ERR_INVALID_ARG;
  }
  const int wf = mx ? W_MXFP8 : nv ? W_NVFP4 : W_BF16;
  const int S = epi == EPI_PARTIAL ? gemm_pick_splits(M, N, K, wf) : 1;
  *splits = S;
  if (!C) return DORY_OK;
  GemmArgs g;
  g.A = A;
  g.lda = lda;
  g.B = B;
  g.Bs = B_scales;
  g.M = M;
  g.N = N;
  g.K = K;
  g.act = ACT_BF16;
  g.wfmt = wf;
  g.Bg = B_gscale;
  g.epi = epi;
  g.splits = S;
  g.C = C;
  g.ldc = ldc;
  g.n_half = epi == EPI_SWIGLU ? N / 2 : 0;
  g.Bf = epi == EPI_PARTIAL ? B_frag : nullptr;
  const hipError_t e = launch_gemm(g, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_create_err = hipGetErrorString(e);
    return e == hipErrorInvalidValue ? DORY_ERR_INVALID_ARG : DORY_ERR_HIP;
  }
  return DORY_OK;
}

int dory_arrange_weights(void* stream, const void* w, int64_t N, int64_t K, void* out) {
  if (!w || !out || N < 16 || K < 32 || N % 16 || K % 32 || ((uintptr_t)w & 15) || ((uintptr_t)out & 15) ||
      N > (int64_t)1 << 30 || K > (int64_t)1 << 30) {
    g_create_err = "bad arrangement argument (non-null, 16-byte aligned, N % 16 == 0, K % 32 == 0)";
    return DORY_ERR_INVALID_ARG;
  }
  const char* a = (const char*)w;
  const char* b = (const char*)out;
  const size_t bytes = (size_t)N * (size_t)K * 2;
  if (a < b + bytes && b < a + bytes) {
    g_create_err = "arrangement output overlaps its input";
    return DORY_ERR_INVALID_ARG;
  }
  const hipError_t e = launch_arrange_frag(w, N, K, out, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_create_err = hipGetErrorString(e);
    return DORY_ERR_HIP;
  }
  return DORY_OK;
}

int dory_test_mfma_rate(void* stream, int iters, long long* cycles, float* sink, int* n_wg) {
  int dev = 0, cus = 0;
  if (iters < 1 || iters > 1000000 || !cycles || !sink || !n_wg || hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
    g_create_err = "bad MFMA-rate argument (or no device)";
    return DORY_ERR_INVALID_ARG;
  }
  *n_wg = cus;
  const hipError_t e = launch_mfma_rate(iters, cus, cycles, sink, (hipStream_t)stream);
  if (e != hipSuccess) {
    g_create_err = hipGetErrorString(e);
    return DORY_ERR_HIP;
  }
  return DORY_OK;
}

int dory_quantize_mxfp8(void* stream, const void* w, int w_dtype, int64_t rows, int64_t cols,
                        uint8_t* codes, uint8_t* scales) {
  if (!w || !codes || !scales || rows < 0 || cols < 0 || cols % 32 ||
      (w_dtype != DORY_DTYPE_F32 && w_dtype != DORY_DTYPE_BF16)) {
    g_create_err = "bad quantiser argument";
    return DORY_ERR_INVALID_ARG;
  }
  if (rows * (cols / 32) > (int64_t)0x7fffffff * 8) {
    g_create_err = "matrix too large";
    return DORY_ERR_INVALID_ARG;
  }
  const hipError_t e = launch_quantize_mxfp8(w, w_dtype == DORY_DTYPE_BF16, rows, cols, codes, scales,
                                             (hipStream_t)stream);
  if (e != hipSuccess) {
    g_create_err = hipGetErrorString(e);
    return DORY_ERR_HIP;
  }
  return DORY_OK;
}

int dory_quantize_nvfp4(void* stream, const void* w, int w_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                        uint8_t* scales, float* g) {
  if (!w || !codes || !scales || !g || rows < 0 || cols < 0 || cols % 16 ||
      (w_dtype != DORY_DTYPE_F32 && w_dtype != DORY_DTYPE_BF16)) {
    g_create_err = "bad quantiser argument";
    return DORY_ERR_INVALID_ARG;
  }
  if (rows * (cols / 16) > (int64_t)0x7fffffff * 64) {
    g_create_err = "matrix too large";
    return DORY_ERR_INVALID_ARG;
  }
  const hipError_t e = launch_quantize_nvfp4(w, w_dtype == DORY_DTYPE_BF16, rows, cols, codes, scales, g,
                                             (hipStream_t)stream);
  if (e != hipSuccess) {
    g_create_err = hipGetErrorString(e);
    return DORY_ERR_HIP;
  }
  return DORY_OK;
}

int dory_profile_enable(dory_ctx* ctx, int class_mask) {
  if (!ctx || class_mask < 0 || class_mask >= (1 << DORY_KC_COUNT)) return DORY_ERR_INVALID_ARG;
  if (class_mask) {
    for (int i = 0; i < ctx->pev_used; ++i) (void)hipEventSynchronize(ctx->pev[i]);
    ctx->precs.clear();
    ctx->pev_used = 0;
  }
  ctx->prof = class_mask;
  return DORY_OK;
}

int dory_profile_read(dory_ctx* ctx, int kclass, dory_kernel_stats* out) {
  if (!ctx || !out || kclass < 0 || kclass >= DORY_KC_COUNT) return DORY_ERR_INVALID_ARG;
  dory_kernel_stats r{0, 0.0, 0.0, 0.0};
  for (auto& p : ctx->precs) {
    if (p.kc != kclass) continue;
    float ms = 0.f;
    HIPCHK(hipEventSynchronize(ctx->pev[p.ev + 1]), "hipEventSynchronize");
    HIPCHK(hipEventElapsedTime(&ms, ctx->pev[p.ev], ctx->pev[p.ev + 1]), "hipEventElapsedTime");
    r.launches += 1;
    r.ms += ms;
    r.flops += p.flops;
    r.bytes += p.bytes;
  }
  *out = r;
  return DORY_OK;
}

int dory_sync(dory_ctx* ctx, void* stream) {
  const hipError_t e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) {
    if (ctx) ctx->err = hipGetErrorString(e);
    return DORY_ERR_HIP;
  }
  return DORY_OK;
}

}  // extern "C"
