// Host-side launchers of the HIP kernels. Each returns the launch's hipError_t and
// enqueues on `st`; argument shapes are checked by the caller (runtime.cpp) before
// any launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dory {

enum ActType { ACT_F32 = 0, ACT_BF16 = 1 };
enum WFmt { W_F32 = 0, W_BF16 = 1, W_MXFP8 = 2, W_NVFP4 = 3 };

// ---------------------------------------------------------------- GEMM  C = A B^T
enum Epi {
  EPI_F32 = 0,          // C float [M, N] ("partial" with one split)
  EPI_PARTIAL = 1,      // C float [splits][M][N], split-K partial sums
  EPI_STORE_ACT = 2,    // C bf16 [M, N]
  EPI_SWIGLU = 4,       // rows [0, n_half) gate, [n_half, 2 n_half) up: C bf16 [M, n_half]
                        // = SiLU(gate) * up
};

struct GemmArgs {
  const void* A = nullptr;  // [M, K] activations (act type), row stride lda
  int lda = 0;
  const void* B = nullptr;  // [N, K] weights (wfmt), row stride K
  const void* Bf = nullptr; // bf16: the same weights in fragment order (launch_arrange_frag),
                            // read by the decode GEMV when set; else null
  const uint8_t* Bs = nullptr;  // MXFP8 scales [N, K/32]; NVFP4 E4M3 block scales [N, K/16]
  const float* Bg = nullptr;    // NVFP4 matrix scale (one float); B then holds packed codes [N, K/2]
  int M = 0, N = 0, K = 0;
  int act = ACT_BF16;
  int wfmt = W_BF16;
  int epi = EPI_F32;
  int splits = 1;
  void* C = nullptr;
  int ldc = 0;
  int n_half = 0;
};
// out [rows, cols] bf16 = E4M3 code * 2^(E8M0 scale - 127), groups of 32 along a row (exact)
hipError_t launch_expand_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols, void* out,
                               hipStream_t st);
// out [N*K] bf16 = w [N, K] bf16 in fragment order: 1 KiB block (n/16) (K/32) + k/32
// holds rows 16 (n/16) .. + 15 at K 32 (k/32) .. + 31, element (n, k) at 8 (16 ((k %
// 32) / 8) + n % 16) + k % 8 (one 16x16x32 MFMA B operand per block, in lane order)
hipError_t launch_arrange_frag(const void* w, int64_t N, int64_t K, void* out, hipStream_t st);
// Split count the launcher would use for a decode-shaped GEMM (EPI_PARTIAL).
int gemm_pick_splits(int M, int N, int K, int wfmt);
hipError_t launch_gemm(const GemmArgs& g, hipStream_t st);
// n_wg work-groups of 8 waves, each running 8 chains of iters bf16 MFMAs (32x32x16);
// cycles[n_wg] shader-clock cycles, sink[n_wg * 512] results
hipError_t launch_mfma_rate(int iters, int n_wg, long long* cycles, float* sink, hipStream_t st);

// ------------------------------------------------------- nGPT update / loop boundary
enum Boundary {
  BND_NONE = 0,
  BND_SAVE_X = 1,        // x <- s'; s <- N(s' + x)             (end of the input block)
  BND_LOOP_CONTINUE = 2, // s_t = N(s'); s <- N(s_t + x)        (end of loop t < k)
  BND_LOOP_FINAL = 3,    // s <- N(s')                          (end of loop k)
};
struct UpdateArgs {
  const float* y = nullptr;  // [splits][M][H] raw sublayer output (partial sums); any
                             // positive row scale (the pre-projection norms) cancels in N(y)
  int splits = 1;
  int y_bf16 = 0;            // y is one bf16 [M][H] array instead (splits == 1)
  float* s = nullptr;        // [M, H] state, updated in place
  float* s_out = nullptr;    // where the new state goes (== s, or the caller's output)
  void* sb = nullptr;        // [M, H] act-type copy of the new state (GEMM operand)
  float* x = nullptr;        // [M, H] loop input x
  const float* alpha = nullptr;  // [H]
  int M = 0, H = 0;
  int act = ACT_BF16;
  int bnd = BND_NONE;
  int final_from = 0x7fffffff;  // with BND_LOOP_CONTINUE: rows >= this one end their last
                                // loop here and take BND_LOOP_FINAL (mixed loop counts)
  int state_act = 0;  // the state lives in s16 (fp16, read and rewritten in place) beside
                      // its bf16 copy sb; s is not read, and s_out, when set, receives a
                      // float copy of the new state (prefill form only: y_bf16, >= 512
                      // rows, act bf16)
  void* s16 = nullptr;  // [M, H] fp16 state (state_act)
};
hipError_t launch_update(const UpdateArgs& u, hipStream_t st);
// s = x_in; sb = act(x_in); s16 = fp16(x_in) when set; with rows != NULL row r of s is
// row rows[r] of x_in; s may be null
hipError_t launch_stage_input(const float* x_in, float* s, void* sb, int M, int H, int act,
                              hipStream_t st, const int32_t* rows = nullptr, void* s16 = nullptr);
// y[rows[r]] = s[r] for r < M (float rows of H)
hipError_t launch_scatter_rows(const float* s, const int32_t* rows, int M, int H, float* y, hipStream_t st);
// x = x_in, s = N(s1_in + x_in) (and its act copy sb) per row, from the caller's rows
// (rows[r]: caller row of internal row r; null: the same)
hipError_t launch_resume_state(const float* x_in, const float* s1_in, const int32_t* rows, int M, int H, float* x,
                               float* s, void* sb, int act, hipStream_t st);

// ------------------------------------------------------------ RoPE + QK norm + KV write
struct KVLayout {
  void* pool = nullptr;      // page pool base
  int act = ACT_BF16;        // element type of K/V
  int Hkv = 0, d = 0;
  size_t page_elems = 0;     // elements per page (K and V)
  const int32_t* table = nullptr;  // [max_seqs][n_streams][tab_len]
  int n_streams = 0, tab_len = 0;
  int ring = 0;              // ring length (pages) of this stream, tab_len for full layers
};
struct RopeArgs {
  const void* qkvg = nullptr;  // bf16 [M, Nqkvg] or float [splits][M][Nqkvg]
  int in_f32 = 0;
  int splits = 1;
  int M = 0, Hq = 0, Hkv = 0, d = 0, Nqkvg = 0, gate = 0;
  const int32_t* pos = nullptr;      // [M]
  const int32_t* row_seq = nullptr;  // [M] sequence slot
  const double* freq = nullptr;  // [d/2] theta^(-2i/d) for this layer's base
  int qk_norm = 1;
  const float* s_qk = nullptr;  // [d]
  void* q_out = nullptr;        // act [M, Hq*d]
  KVLayout kv;
  int stream_idx = 0;           // (layer, slot) stream within the sequence
  const int32_t* tiles = nullptr;  // prefill tiles [n_tiles][4]: row0, nrows, pos0, seq slot
  int n_tiles = 0;
  const float* cs = nullptr;    // tiled form: this layer's (cos, sin) table (launch_rope_table)
};
hipError_t launch_rope_kv(const RopeArgs& a, hipStream_t st);
// Prefill form over the tiles (bf16 projection output, d in {64, 128, 160}); q_out null:
// only K and V (the MFMA attention rotates q itself).
hipError_t launch_rope_kv_tiles(const RopeArgs& a, hipStream_t st);
// (cos, sin) of p * freq[b][i] for both bases b (0 sliding, 1 full; freq [2][128] doubles,
// angle reduced modulo 2 pi in double, sin/cos in float) for the rows of the prefill
// tiles, one block of 64 rows per tile: row r (position tile.pos0 + r, r < tile.nrows) of
// tile t, pairs 2k and 2k + 1, as 4 floats at cs + b * ld + t * 64 * 2 half + 4 (64 k + r)
// (chunk-major, so that 16-byte reads of consecutive rows are consecutive).
hipError_t launch_rope_table(const int32_t* tiles, int n_tiles, const double* freq, int half, size_t ld, float* cs,
                             hipStream_t st);

// ------------------------------------------------------------------------ attention
struct AttnArgs {
  const void* q = nullptr;        // act [M, Hq*d] (rotated, normalised)
  // MFMA prefill with rope_cs: q is read unrotated from the projection output (row m,
  // head h at q_raw[m * q_ld + h * d], bf16) and rotated by rope_cs (this layer's table
  // of launch_rope_table), normalised and scaled by s_qk (when set) in the kernel; q is
  // then not read
  const void* q_raw = nullptr;
  int q_ld = 0;
  const float* rope_cs = nullptr;
  // gate pre-activation, read where the projection left it: row m, channel c at
  // g[m * g_ld + c] (+ split s at s * g_sstride for float partials, summed over g_splits)
  const void* g = nullptr;        // null: no gate
  int g_f32 = 0, g_ld = 0, g_splits = 1;
  size_t g_sstride = 0;
  int M = 0, Hq = 0, Hkv = 0, d = 0;
  const int32_t* pos = nullptr;
  const int32_t* row_seq = nullptr;
  int window = 0;                 // 0 = full attention
  float scale = 1.f;
  // per-channel query-key scale when q and k were L2-normalised and scaled by it (null
  // otherwise): then every logit is bounded by scale * max s_qk^2
  const float* s_qk = nullptr;
  KVLayout kv;
  int stream_idx = 0;
  int max_pos = 0;                // largest position among the rows (host-known)
  float* part = nullptr;          // [M][Hq][splits][d + 2] split partials (workspace)
  int part_cap = 0;               // capacity of part in floats
  void* o = nullptr;              // act [M, Hq*d]
  // prefill tiles (chunks of consecutive rows of one sequence), MFMA path
  const int32_t* tiles = nullptr; // [n_tiles][4]: row0, nrows, pos0, seq slot
  int n_tiles = 0;
  int max_tile_rows = 0;
  int n_quads = 0;                // sum over tiles of ceil(rows / 4): row-wise kernel by quads
};
// Row-wise paged attention (any row count; split over keys) + combine + gate, in two
// phases launched separately: ATTN_SPLITS (the split-key kernel, writes partials) and
// ATTN_MERGE (combines them, applies the gate, writes o). Both phases pick the same
// split count for the same arguments; *splits_out receives it (may be null).
enum AttnPhase { ATTN_SPLITS = 0, ATTN_MERGE = 1 };
hipError_t launch_attn_rows(const AttnArgs& a, int phase, int* splits_out, hipStream_t st);
// Prefill attention on bf16 with MFMA (query tiles of 64 rows); writes o.
hipError_t launch_attn_prefill(const AttnArgs& a, hipStream_t st);
size_t attn_rows_part_floats(int M, int Hq, int d, int max_pos, int window);

// -------------------------------------------------------------------- SwiGLU reduce
// h = SiLU(sum_s gate) * (sum_s up) from float partials [splits][M][2I]; h act [M, I];
hipError_t launch_swiglu(const float* gu, int splits, int M, int I, void* h, int act,
                         hipStream_t st);

// ------------------------------------------------------------------ page table etc.
// Install page-table entries (pairs of flat table index, page) and zero those pages.
hipError_t launch_apply_deltas(int32_t* table, const int32_t* deltas, int n, void* pool,
                               size_t page_bytes, hipStream_t st);
hipError_t launch_fill_kv(const KVLayout& kv, int seq_slot, int stream_idx, int pos0, int n,
                          const void* k, const void* v, hipStream_t st);
hipError_t launch_quantize_mxfp8(const void* w, int w_bf16, int64_t rows, int64_t cols,
                                 uint8_t* codes, uint8_t* scales, hipStream_t st);

// ------------------------------------------------- vocabulary side (k_vocab.hip)
// x[i] = N(E[ids[i]]) float [n, H]; ids outside [0, V) give zero rows.
hipError_t launch_embed(const void* E, int e_bf16, int64_t V, int H, const int32_t* ids, int n, float* x,
                        hipStream_t st);
// logits[i][v] = sz[v] * sum over splits of part[s][i][v] (row stride ld, split stride
// sstride elements; part may be logits itself for one split).
hipError_t launch_logit_scale(const float* part, int splits, size_t sstride, float* logits, int64_t ld, int n,
                              int64_t V, const float* sz, hipStream_t st);
// Static device scratch for dory_logits_noalloc: NOALLOC_SCRATCH_BYTES per GPU; the
// address on the current device (looked up once per device).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
constexpr int MAX_DEVICES = 64;
hipError_t noalloc_scratch(void** out);
// out[i] = the token u[i] draws from row i of logits under temperature and top-p.
hipError_t launch_sample_top_p(const float* logits, int64_t ld, int n, int64_t V, float temperature, float top_p,
                               const float* u, int32_t* out, hipStream_t st);

// speculative acceptance (k_vocab.hip): per sequence, gamma draft tokens against the
// verifying model's gamma + 1 rows; out [n, gamma + 1] tokens, n_out [n] emitted counts
hipError_t launch_spec_accept(int n, int gamma, int64_t V, const float* draft, int64_t ld_d, const float* target,
                              int64_t ld_t, const int32_t* dtok, float temperature, float top_p, const float* u_acc,
                              const float* u_smp, int32_t* out, int32_t* n_out, hipStream_t st);

// ------------------------------------------------------- NVFP4 weights (k_nvfp4.hip)
// codes [rows, cols/2] (two E2M1 codes a byte, element 2j in the low nibble), E4M3 block
// scales [rows, cols/16], the power-of-two matrix scale g (one float).
hipError_t launch_quantize_nvfp4(const void* w, int w_bf16, int64_t rows, int64_t cols, uint8_t* codes,
                                 uint8_t* scales, float* g, hipStream_t st);
// out [rows, cols] bf16 = e2m1 * e4m3 * g (exact)
hipError_t launch_expand_nvfp4(const uint8_t* codes, const uint8_t* scales, const float* g, int64_t rows,
                               int64_t cols, void* out, hipStream_t st);

}  // namespace dory
