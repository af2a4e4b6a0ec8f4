/*
 * dory.h — C ABI of the MI355X (gfx950) looped normalized-GPT forward pass.
 *
 * The model ("Dory1.0-4B: A Looped Normalized-GPT", arXiv 2611.03998): an input block
 * of layers runs once and yields x; a shared recurrent block runs k times as
 *   s_0 = x,  u_t = N(s_{t-1} + x),  s_t = N(F(u_t))      (paper summary, core method)
 * and an output block runs once. Every sublayer applies the nGPT update
 *   s <- N((1 - a) * s + a * N(sublayer(s)))            (paper summary, nGPT; arXiv §2)
 * with N the row-wise L2 normalisation and a a per-channel rate. A layer is an
 * attention sublayer (GQA, RoPE, sliding-window or full, sigmoid output gate, an L2
 * norm before the output projection) followed by a SwiGLU MLP sublayer (an L2 norm
 * before the down projection) — paper summary "technical novelty", arXiv §2.
 * Recurrent attention layers keep k KV slots per token (per_loop) or one slot
 * overwritten every loop (last_loop) — arXiv §6.1, model-card digest §2.
 *
 * Conventions for every call:
 *  - Return value: DORY_OK or a negative DORY_ERR_* code; dory_last_error() gives a
 *    message. Every error but DORY_ERR_HIP is found before any device work, and the
 *    context is unchanged. After DORY_ERR_HIP (a failed HIP call, possibly reporting
 *    earlier asynchronous work) the context's sequences are as before the call
 *    (lengths, pages, live set, page-table updates still to apply), but device work
 *    enqueued before the failing step may still run: it can write the call's output
 *    rows and cache entries at positions the sequences do not hold yet, which later
 *    calls write again before any call reads them.
 *  - "device" pointers are HIP device memory owned by the caller; the library never
 *    allocates or frees device memory. "host" pointers are read during the call only.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Device
 *    work is enqueued asynchronously on it; results are valid after the stream is
 *    synchronised. Host arrays may be reused as soon as a call returns.
 *  - One context is used from one host thread at a time. Calls on one context may use
 *    different streams: a call whose stream differs from the previous call's first
 *    makes its stream wait for the previous call's device work (the workspace and page
 *    tables are shared), so consecutive calls never overlap on the device.
 *  - Matrices are row-major. A weight W is [N_out, K_in] and a projection is
 *    y = s W^T.
 *  - Tracing: with DORY_TRACE=1 in the environment, dory_prefill and dory_decode_step
 *    open one marker range per call, nested ranges for the input block, each loop and
 *    the output block, and one range per layer call inside those (rocprofv3
 *    --marker-trace records them). The marker library (librocprofiler-sdk-roctx.so.1,
 *    or the file DORY_TRACE_LIB names) is opened on the first traced call; if it
 *    cannot be opened, calls run untraced.
 */
#ifndef DORY_H
#define DORY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes */
#define DORY_OK 0
#define DORY_ERR_INVALID_ARG (-1) /* bad argument: shape, pointer, id, range */
#define DORY_ERR_STATE (-2)       /* call not allowed in the context's state */
#define DORY_ERR_OUT_OF_KV (-3)   /* the bound KV pool has too few free pages */
#define DORY_ERR_UNSUPPORTED (-4) /* valid, but not a shape/format this library runs */
#define DORY_ERR_HIP (-5)         /* a HIP runtime call failed */

/* ---- element types */
#define DORY_DTYPE_F32 0
#define DORY_DTYPE_BF16 1
/* ---- weight formats */
#define DORY_WFMT_F32 0
#define DORY_WFMT_BF16 1
#define DORY_WFMT_MXFP8 2 /* E4M3 codes + one E8M0 scale byte per 32 along K */
#define DORY_WFMT_NVFP4 3 /* packed E2M1 codes + one E4M3 scale byte per 16 along K + a
                             power-of-two float per matrix (dory_quantize_nvfp4) */

/* ---- recurrent KV-cache modes (arXiv §6.1) */
#define DORY_KV_PER_LOOP 0  /* k slots per recurrent attention layer, slot t-1 in loop t */
#define DORY_KV_LAST_LOOP 1 /* one slot, overwritten by every loop */

/* ---- attention output gate (paper summary: input-dependent sigmoid gate) */
#define DORY_GATE_NONE 0
#define DORY_GATE_ELEMENTWISE 1 /* o <- sigmoid(s W_g^T) * concat_h(o_h), width Hq*d */

#define DORY_PAGE_TOKENS 64        /* tokens per KV page */
#define DORY_MAX_POSITIONS 262144  /* max_position_embeddings (MXFP8 article, config) */
#define DORY_MAX_LOOPS 8           /* base model evaluated up to k = 8 (arXiv §3.5) */

typedef struct dory_ctx dory_ctx; /* opaque, library-owned */

/*
 * Model shape and runtime limits. Layer i (global physical index) is full attention
 * iff i % full_period == full_period - 1, else sliding-window (3:1 pattern, MXFP8
 * article "hybrid attention"; full_period = 4). RoPE base theta_full on full layers,
 * theta_swa on sliding layers; window W counts the query itself (keys j with
 * 0 <= p - j < W are visible). With qk_norm the rotated per-head q and k are
 * L2-normalised and multiplied by s_qk (nGPT); attention logits are attn_scale * q.k.
 */
typedef struct dory_config {
  int32_t hidden;        /* H */
  int32_t n_q_heads;     /* Hq */
  int32_t n_kv_heads;    /* Hkv; Hq % Hkv == 0; query head h uses KV head h / (Hq/Hkv) */
  int32_t head_dim;      /* d, even */
  int32_t intermediate;  /* I, SwiGLU width */
  int32_t n_in, n_rec, n_out; /* layers per block, each >= 1 */
  int32_t window;        /* W >= 1 */
  int32_t full_period;   /* >= 1 */
  double theta_swa;
  double theta_full;
  float attn_scale;
  int32_t qk_norm;       /* 0 or 1 */
  int32_t attn_gate;     /* DORY_GATE_* */
  int32_t act_dtype;     /* DORY_DTYPE_*: activations fed to projections and KV cache */
  int32_t weight_format; /* DORY_WFMT_*; F32 needs act F32; BF16/MXFP8/NVFP4 need act BF16 */
  int32_t max_loops;     /* 1..DORY_MAX_LOOPS */
  int32_t max_seqs;      /* live sequences at once */
  int32_t max_seq_len;   /* positions per sequence, <= DORY_MAX_POSITIONS */
  int32_t max_rows;      /* rows per prefill call (sum of n_new) or per decode step */
} dory_config;

/*
 * One physical layer's parameters (device pointers, caller-owned, must stay valid
 * while the context uses them). Weight element type follows weight_format
 * (float, bf16 stored as uint16, or E4M3 bytes).
 *  w_qkvg [Hq*d + 2*Hkv*d + G, H]  rows: q | k | v | gate (G = Hq*d with the gate, else 0)
 *  w_o    [H, Hq*d]
 *  w_gu   [2*I, H]                 rows: SwiGLU gate | up
 *  w_down [H, I]
 *  s_*    MXFP8: E8M0 scale bytes [rows, K/32] of the matching matrix; NVFP4: E4M3
 *         block scale bytes [rows, K/16]; else NULL
 *  g_*    NVFP4 only: the matching matrix's scale (one float, device); else NULL.
 *         NVFP4 matrices hold packed codes [rows, K/2] (element 2j in the low nibble)
 *  alpha_attn, alpha_mlp [H] float, 16-byte aligned: effective per-channel rates
 *         (arXiv §2: 0.05 init)
 *  s_qk   [d] float: effective query-key scale
 *  f_*    bf16 contexts, optional: the matching matrix in fragment order, as written by
 *         dory_arrange_weights (same bytes, another order; 16-byte aligned). When set,
 *         projections of at most 32 rows (decode) read it instead of w_*, with one
 *         contiguous KiB per load instruction; the results are bitwise the same. NULL:
 *         they read w_*.
 */
typedef struct dory_layer_weights {
  const void* w_qkvg;
  const void* w_o;
  const void* w_gu;
  const void* w_down;
  const uint8_t* s_qkvg;
  const uint8_t* s_o;
  const uint8_t* s_gu;
  const uint8_t* s_down;
  const float* alpha_attn;
  const float* alpha_mlp;
  const float* s_qk;
  const float* g_qkvg;
  const float* g_o;
  const float* g_gu;
  const float* g_down;
  const void* f_qkvg;
  const void* f_o;
  const void* f_gu;
  const void* f_down;
} dory_layer_weights;

/* Create a context for cfg. Checks shapes, formats and limits (INVALID_ARG /
 * UNSUPPORTED). Loops default to min(2, max_loops) (MXFP8 article: default 2), mode to
 * per_loop. Makes no HIP call. */
int dory_create(const dory_config* cfg, dory_ctx** out);
int dory_destroy(dory_ctx* ctx);
/* Message of the context's last error ("" if none). ctx may be NULL for create errors
 * (then the thread's last create message is returned). Owned by the library. */
const char* dory_last_error(const dory_ctx* ctx);

/* Sizes the caller allocates: bytes of one KV page (DORY_PAGE_TOKENS tokens of K and V
 * for all KV heads) and the workspace the context needs. */
int dory_query_sizes(const dory_config* cfg, size_t* page_bytes, size_t* workspace_bytes);
/* KV pages that n_seqs sequences of seq_len tokens hold with k loops in `mode`
 * (sliding layers keep a ring of ceil((W + max_rows - 1)/64) + 1 pages). */
int dory_kv_pages_needed(const dory_config* cfg, int mode, int k, int64_t seq_len,
                         int64_t n_seqs, int64_t* pages);

int dory_bind_weights(dory_ctx* ctx, int layer, const dory_layer_weights* w);
/* KV pool: device memory of `bytes` (a whole number of pages used). Only while no
 * sequence is live (STATE). */
int dory_bind_kv_pool(dory_ctx* ctx, void* pool, size_t bytes);
/* Workspace: device memory, >= workspace_bytes, 256-byte aligned. It holds the page
 * tables, so it belongs to the context until destroy or rebind (STATE while live). */
int dory_bind_workspace(dory_ctx* ctx, void* ws, size_t bytes);

/* Loop count k of the context (1..max_loops, else INVALID_ARG), allowed any time. Each
 * sequence runs its own k (the paper summary's elastic depth: k chosen per request):
 * a per_loop sequence the k its KV cache was built for (the context's k when it was
 * created) unless dory_set_seq_loops set a smaller one; a last_loop sequence the k set
 * for it with dory_set_seq_loops, else the context's k at each call. One prefill or decode call may mix sequences of different
 * k: the recurrent block runs max k times, loop t on the rows of the sequences with
 * k >= t. */
int dory_set_loops(dory_ctx* ctx, int k);
int dory_get_loops(const dory_ctx* ctx, int* k);
/* Loop count of live sequence seq_id for its next calls: 1..max_loops, or 0 for its
 * mode's default (per_loop: the k its cache was built for; last_loop: the context's k).
 * per_loop mode: at most the k its cache was built for (STATE otherwise); running fewer
 * loops leaves the cache slots of the skipped loops unwritten for the new positions, so
 * those positions must be truncated away and recomputed at the full k before a call at
 * the full k reads them (self-speculative drafting, arXiv summary §6.2). Unknown id:
 * INVALID_ARG. */
int dory_set_seq_loops(dory_ctx* ctx, int32_t seq_id, int k);
/* The loop count seq_id runs with (INVALID_ARG for an unknown id). */
int dory_seq_loops(const dory_ctx* ctx, int32_t seq_id, int* k);
/* KV mode (DORY_KV_*). STATE while any sequence is live. */
int dory_set_kv_mode(dory_ctx* ctx, int mode);
int dory_get_kv_mode(const dory_ctx* ctx, int* mode);

/*
 * Prefill: the looped forward pass over new tokens (paper summary, core-method equation:
 * input block once giving x, s_0 = x, u_t = N(s_{t-1} + x), s_t = N(F(u_t)) for t = 1..k,
 * output block once; arXiv summary §3.2), writing each attention layer's cache entries
 * for the new positions into the slot the KV mode gives (arXiv summary §6.1).
 * Append n_new[i] tokens to sequence seq_ids[i] for i < n_seqs (host arrays).
 * A new id starts a sequence at position 0; a live id continues it (chunked prefill).
 * x_in  device float [sum n_new, H]: unit-norm input states, rows grouped by sequence
 *       in seq_ids order, positions increasing.
 * y_out device float [sum n_new, H]: final states (output of the output block).
 * x_in and y_out are 16-byte aligned (the update kernels move 16 bytes per access).
 * Errors: INVALID_ARG (ids repeated, n_new < 1, sum n_new > max_rows, position would
 * reach max_seq_len, too many live sequences, null or misaligned pointers), STATE (weights, pool or
 * workspace unbound), OUT_OF_KV (pool too small; nothing reserved), HIP.
 * In last_loop mode results depend on the chunk schedule (earlier chunks' tokens are
 * seen with their final-loop entries).
 */
int dory_prefill(dory_ctx* ctx, void* stream, int n_seqs, const int32_t* seq_ids,
                 const int32_t* n_new, const float* x_in, float* y_out);

/* One decode step: the same looped forward pass (paper summary, core method; arXiv
 * summary §3.2 and §6.1) for one new token of each listed live sequence (a chunk of one
 * row at position = the sequence's length), whose queries read the cached keys and
 * values of all earlier positions (the sliding window's last W on sliding layers).
 * x_in, y_out device float [n_seqs, H], 16-byte aligned. Errors as prefill; unknown id
 * -> INVALID_ARG. */
int dory_decode_step(dory_ctx* ctx, void* stream, int n_seqs, const int32_t* seq_ids,
                     const float* x_in, float* y_out);

int dory_release_seq(dory_ctx* ctx, int32_t seq_id); /* frees its pages */
/* Shorten live sequence seq_id to its first len positions (1 <= len <= its length): the
 * next call continues at position len, rewriting the cache entries of the positions it
 * covers (rejected speculative drafts). Host bookkeeping only; pages stay allocated. */
int dory_truncate_seq(dory_ctx* ctx, int32_t seq_id, int64_t len);
int dory_seq_len(const dory_ctx* ctx, int32_t seq_id, int64_t* len);
int dory_live_seqs(const dory_ctx* ctx, int32_t* n);
/* KV footprint: bytes of pages currently held by live sequences. */
int dory_kv_bytes_in_use(const dory_ctx* ctx, size_t* bytes);
/* Layer calls enqueued by the last prefill/decode call (host counter): E(k) =
 * n_in + n_out + k * n_rec, k the largest loop count of the call's sequences. */
int dory_last_layer_calls(const dory_ctx* ctx, int64_t* n);

/* ---- vocabulary side: token embedding, LM head, top-p sampling
 * The steps on either side of the stack ("Dory1.0-4B" pages: nGPT keeps embeddings on
 * the unit sphere — paper summary, "prerequisites: nGPT"; logit-scale parameters —
 * arXiv summary §2; generation settings temperature 1.0, top_p 0.95 — MXFP8 article,
 * deployment section).
 *  embed       [V, H] input token embedding
 *  lm_head     [V, H] output embedding (may be the same array as embed)
 *  logit_scale [V] float: effective per-token logit scale s_z
 * Tables are float in an F32 context and bf16 (uint16) otherwise (both contexts'
 * activation type: the pages keep embeddings and LM head out of weight quantisation,
 * arXiv summary §5.1); V % 128 == 0, V <= 2^24. Device pointers, caller-owned, valid
 * while the context uses them. */
typedef struct dory_vocab_weights {
  int64_t vocab;
  const void* embed;
  const void* lm_head;
  const float* logit_scale;
} dory_vocab_weights;
/* Errors: INVALID_ARG (null pointers, V out of range or not a multiple of 128). */
int dory_bind_vocab(dory_ctx* ctx, const dory_vocab_weights* v);

/* Input states of tokens: x_out[i] = N(embed[ids[i]]) (device float [n, H]); ids device
 * int32 [n]. An id outside [0, V) yields a zero row (the table is not read). The rows
 * are unit-norm states as dory_prefill / dory_decode_step take them.
 * 1 <= n <= max_rows. Errors: INVALID_ARG, STATE (vocabulary unbound), HIP. */
int dory_embed(dory_ctx* ctx, void* stream, int n, const int32_t* ids, float* x_out);

/* LM head: logits[i][v] = logit_scale[v] * (states[i] . lm_head[v]); states device float
 * [n, H] (final states, e.g. y_out of a decode step), logits device float [n, V] (row
 * stride V). The states enter the product in the context's activation type (bf16 in a
 * bf16 context), as in the projections; float accumulation. Uses the workspace.
 * 1 <= n <= max_rows. Errors: INVALID_ARG, STATE (vocabulary or workspace unbound), HIP. */
int dory_logits(dory_ctx* ctx, void* stream, int n, const float* states, float* logits);

/* dory_logits for callers that cannot allocate device memory or bind a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid allocation): the
 * same result, with the staged states and split-K partials in a scratch array the
 * library holds on each GPU (32 MiB, from the first call on a device until the process
 * ends) instead of the workspace. Needs the vocabulary bound, not the workspace. Limit:
 * n * H * 6 bytes (bf16 contexts; none in fp32 ones), plus splits * n * V * 4 when the
 * LM-head GEMM splits K (small vocabularies only: below 25600 tokens at n <= 128; the
 * 131072-token vocabulary never does), at most 32 MiB (INVALID_ARG beyond, before any
 * device work). Nothing needs clearing between calls: each call writes every scratch
 * byte it reads. Calls no hipMalloc or hipFree.
 * Every call on a GPU uses that GPU's one array: calls that overlap on a GPU (other
 * streams, other contexts, other threads) race, and must be ordered by the caller.
 * Errors as dory_logits, except that no workspace is needed. */
int dory_logits_noalloc(dory_ctx* ctx, void* stream, int n, const float* states, float* logits);

/* Top-p sampling, one token per row: p = softmax(logits[i] / temperature); tokens in
 * order of p, highest first, equal p by lower id; the nucleus is the shortest prefix of
 * that order whose cumulative p reaches top_p; the token is the first of the nucleus
 * whose cumulative p exceeds u[i] times the nucleus mass. logits device float [n, V],
 * row stride ld >= V; u device float [n], each in [0, 1) (the random draws are inputs);
 * tokens device int32 [n]. Probabilities and running sums are float32, summed in a fixed
 * order, so the result is a deterministic function of the inputs; probabilities equal in
 * float32 go by id. Logits must be finite. 1 <= V <= 2^24, temperature > 0,
 * 0 < top_p <= 1. No context: INVALID_ARG before any device work (message in
 * dory_last_error(NULL)), HIP. */
int dory_sample_top_p(void* stream, int n, int64_t vocab, const float* logits, int64_t ld, float temperature,
                      float top_p, const float* u, int32_t* tokens);

/* ---- test and benchmark support: installing a seeded context without computing it */
/* Extend sequence seq_id (created if new) by n_tokens positions and reserve their
 * pages; the entries are undefined until written by dory_test_fill_kv. */
int dory_test_reserve(dory_ctx* ctx, int32_t seq_id, int32_t n_tokens);
/* Write entries pos0..pos0+n-1 of (layer, slot) of sequence seq_id from device arrays
 * k, v [n, Hkv, d] in the act dtype. slot < k for recurrent layers in per_loop mode,
 * else 0. Positions must be below the sequence length and, on sliding layers, inside
 * the window ring. */
int dory_test_fill_kv(dory_ctx* ctx, void* stream, int32_t seq_id, int layer, int slot,
                      int32_t pos0, int32_t n, const void* k, const void* v);

/* Make the next dory_prefill / dory_decode_step on ctx fail with DORY_ERR_HIP after it
 * has committed (sequences created and grown, pages taken) and before the step named by
 * `at` enqueues anything: 0 = the upload of the call's metadata, n >= 1 = layer call n;
 * -1 disarms. Consumed by the next call whatever its outcome. Test support for the error
 * contract above; no device work fails. */
int dory_test_inject_failure(dory_ctx* ctx, int at);

/* One projection GEMM exactly as a layer call launches it (test support for the GEMM
 * kernels): C = A B^T, A [M, K] bf16 device rows with stride lda elements, B [N, K]
 * device weights in format wfmt: DORY_WFMT_BF16; DORY_WFMT_MXFP8 codes with B_scales
 * [N, K/32] E8M0 bytes; or DORY_WFMT_NVFP4 packed codes [N, K/2] with B_scales [N, K/16]
 * E4M3 bytes and B_gscale the matrix scale (one device float). B_scales and B_gscale are
 * NULL when the format has none. epi selects the output the layers use:
 *   0: C float [M, N] (prefill output and down projections);
 *   1: C float split-K partials [splits][M][N] (decode projections), summed by the caller;
 *   2: C bf16 [M, N] ([q|k|v|gate] projection in prefill);
 *   4: SwiGLU: B rows [0, N/2) gate, [N/2, N) up; C bf16 [M, N/2] = SiLU(gate) * up.
 * Quantised formats take epi 1 only (layers expand MXFP8 and NVFP4 matrices to bf16,
 * exactly, for the other epilogues). ldc = row stride of C in elements. The kernel and tile shape are the ones a
 * layer call would pick for these sizes (K % 64 == 0; N % 64 == 0, for epi 4 N % 128 == 0,
 * for NVFP4 N % 128 == 0). *splits receives the split count (1 unless epi 1). B_frag: optional
 * fragment-order copy of a bf16 B (dory_arrange_weights), read where a layer would read
 * it (epi 1, M <= 32). With C == NULL the call only reports *splits. The caller owns every buffer; C must hold
 * splits * M * ldc elements for epi 1. Invalid sizes return DORY_ERR_INVALID_ARG before
 * any device work. */
int dory_test_gemm(void* stream, const void* A, int lda, const void* B, const uint8_t* B_scales,
                   const float* B_gscale, int wfmt, int M, int N, int K, int epi, void* C, int ldc,
                   int* splits, const void* B_frag);

/* Fragment-order copy of a bf16 weight matrix, for the f_* fields of
 * dory_layer_weights: w [N, K] row-major bf16 (device) -> out [N * K] bf16 (device,
 * caller-owned, 16-byte aligned, not overlapping w) as 1 KiB blocks, block
 * (n / 16) * (K / 32) + k / 32 holding rows 16 (n / 16) .. + 15 at columns
 * 32 (k / 32) .. + 31, element (n, k) at position 8 * (16 * ((k % 32) / 8) + n % 16)
 * + k % 8 of its block: each block is one v_mfma_f32_16x16x32_bf16 B operand in lane
 * order. Layout of the library's own making (no page defines it); asynchronous on
 * `stream`. N % 16 == 0 and K % 32 == 0, non-null pointers, else DORY_ERR_INVALID_ARG
 * before any device work. */
int dory_arrange_weights(void* stream, const void* w, int64_t N, int64_t K, void* out);

/* Sustained rate of the bf16 matrix instruction the projection GEMMs run on
 * (v_mfma_f32_32x32x16_bf16, 32768 flops each): one work-group of 8 waves per compute
 * unit, each wave running 8 independent accumulator chains of `iters` instructions on
 * register operands that hold non-zero data (the clock the chip sustains under dense
 * matrix work depends on the data). Measurement support for the roofline's practical
 * ceiling; the caller times the call on `stream`. cycles: device int64 array with one
 * entry per compute unit, receives the shader-clock cycles each work-group spent in its
 * loop; sink: device float array of 512 entries per compute unit (the results, so that
 * no work is elided); *n_wg receives the number of work-groups (the compute-unit count).
 * 1 <= iters <= 1000000, else DORY_ERR_INVALID_ARG before any device work. */
int dory_test_mfma_rate(void* stream, int iters, long long* cycles, float* sink, int* n_wg);

/* MXFP8 quantiser (arXiv §5.2: maximum scaling, group 32): w [rows, cols] device
 * (w_dtype F32 or BF16), cols % 32 == 0 -> codes [rows, cols] E4M3 bytes and scales
 * [rows, cols/32] E8M0 bytes (device). Scale 2^(floor(log2 amax) - 8), elements
 * round-to-nearest-even with saturation at 448, all-zero group -> byte 0. */
int dory_quantize_mxfp8(void* stream, const void* w, int w_dtype, int64_t rows,
                        int64_t cols, uint8_t* codes, uint8_t* scales);

/* Activation reuse for self-speculative decoding (arXiv summary §6.2: verification reuses
 * what the draft computed). Both set one-shot options of the next dory_prefill or
 * dory_decode_step call on ctx (that call consumes them whatever its outcome).
 * dory_capture_states: every sequence of that call must run one loop (INVALID_ARG
 * otherwise); it writes each row's input-block output x and first-loop state s_1 to
 * x_out and s1_out (device float [rows, H], the call's row order); with
 * skip_output_block the output block is not run and y_out is not written.
 * dory_resume_states: every sequence of that call must run two loops or more; the call
 * takes x and s_1 of its rows from x_in and s1_in (device float [rows, H], the call's row
 * order), runs neither the input block nor loop 1 (their cache entries for these
 * positions must already hold what a pass over them wrote: a draft at one loop), and
 * starts at loop 2 from N(s_1 + x); x_in of the call itself is not read. Buffers must
 * stay valid until the call's work on its stream is done. */
int dory_capture_states(dory_ctx* ctx, float* x_out, float* s1_out, int skip_output_block);
int dory_resume_states(dory_ctx* ctx, const float* x_in, const float* s1_in);

/* Self-speculative decoding's acceptance step (paper summary and arXiv summary §6.2: draft
 * gamma tokens with one loop, verify with k loops, rejection sampling keeps the k-loop
 * distribution). n sequences, V = vocab:
 *   draft_logits  [gamma, n, V] position-major, row (j, b) at (j n + b) ld_d: the rows
 *                 draft token j of sequence b was drawn from (one draft step's logits);
 *   target_logits [n, gamma + 1, V] sequence-major, row (b, j) at (b (gamma+1) + j) ld_t:
 *                 the verifying model at the same positions and one more (one chunk);
 *   draft_tokens, u_accept [gamma, n] position-major; u_sample [n];
 *   tokens [n, gamma + 1] out; n_out [n] out.
 * Both rows of a position are processed as top-p sampling processes them (temperature,
 * nucleus renormalised: p and q). Draft j is accepted when u_accept < p(x_j) / q(x_j)
 * (never for an id outside [0, V) or outside q's nucleus); at the first rejection one
 * token is drawn from max(0, p - q) renormalised, by inverse CDF over increasing ids with
 * u_sample (from p if that is empty), and the step ends; if all are accepted, one more
 * token is drawn from the last verifying row by dory_sample_top_p's rule with u_sample.
 * tokens[b, 0 .. n_out[b] - 1] receive the accepted drafts and the drawn token, n_out[b]
 * in 1..gamma+1; entries past n_out[b] are unspecified. Float32 sums in a fixed order:
 * deterministic. 1 <= gamma <= 16; other limits as for dory_sample_top_p. INVALID_ARG
 * before device work (dory_last_error(NULL)), HIP. */
int dory_spec_accept(void* stream, int n, int gamma, int64_t vocab, const float* draft_logits, int64_t ld_d,
                     const float* target_logits, int64_t ld_t, const int32_t* draft_tokens, float temperature,
                     float top_p, const float* u_accept, const float* u_sample, int32_t* tokens, int32_t* n_out);

/* NVFP4 quantiser (W4A16; arXiv summary §5.1-5.2: dynamic MSE scale selection; paper
 * summary: E2M1 elements with E4M3 scale factors): w [rows, cols] device (w_dtype F32 or
 * BF16), cols % 16 == 0 -> codes [rows, cols/2] bytes (two E2M1 codes each, element 2j
 * in the low nibble), scales [rows, cols/16] E4M3 bytes (one per 16 along a row) and
 * g [1] float, the matrix scale 2^ceil(log2(amax / 2688)) (1 for an all-zero matrix).
 * Each block of 16 takes the positive E4M3 scale code whose float32 sum of squared
 * errors (element by element, in order, no fused multiply-add) is smallest, the smaller
 * code on equal sums; elements round to the nearest E2M1 value, ties to even, saturating
 * at 6. A dequantised weight e2m1 * e4m3 * g is exactly a bf16 value. */
int dory_quantize_nvfp4(void* stream, const void* w, int w_dtype, int64_t rows, int64_t cols,
                        uint8_t* codes, uint8_t* scales, float* g);

/* ---- tracing: per-kernel-class launch timing with HIP events on the call's stream */
#define DORY_KC_GEMM 0   /* projections: [q|k|v|gate], output, SwiGLU gate/up, down */
#define DORY_KC_ATTN 1   /* attention over the KV cache: the prefill kernel (with gate), or the
                            split-key kernel of decode and fp32 calls */
#define DORY_KC_ROPE 2   /* RoPE + QK norm + KV-cache write */
#define DORY_KC_UPDATE 3 /* nGPT update / loop boundary, input staging */
#define DORY_KC_SWIGLU 4 /* SwiGLU from split-K partials */
#define DORY_KC_MERGE 5  /* merge of the split-key partials, gate (decode and fp32 calls) */
#define DORY_KC_VOCAB 6  /* vocabulary side: the LM-head GEMM and its logit scale, the embedding
                            lookup (the sampler takes no context and is not recorded) */
#define DORY_KC_COUNT 7
typedef struct dory_kernel_stats {
  int64_t launches; /* kernel launches recorded */
  double ms;        /* summed event time of those launches */
  double flops;     /* algorithmic FLOPs: GEMM 2*M*N*K; attention 4*Hq*d per visible
                       (query, key) pair */
  double bytes;     /* algorithmic HBM bytes: GEMM weights (+ scales) + activations in and
                       out; attention K/V entries read (once per row) + q; merge partials
                       read + gate + o */
} dory_kernel_stats;
#define DORY_KC_ALL ((1 << DORY_KC_COUNT) - 1)
/* Start recording the classes in class_mask (bit 1 << DORY_KC_*; counters cleared), or
 * stop (class_mask 0). Recording brackets each launch of a selected class with a pair of
 * HIP events on the call's stream; it adds no device work beyond the event markers, but
 * each marker costs some launch latency, so time a step with only the classes needed.
 * INVALID_ARG for bits outside DORY_KC_ALL. */
int dory_profile_enable(dory_ctx* ctx, int class_mask);
/* Totals for one class since enabling (waits for the recorded events). */
int dory_profile_read(dory_ctx* ctx, int kclass, dory_kernel_stats* out);

/* Synchronise `stream` and report any pending HIP error (HIP). */
int dory_sync(dory_ctx* ctx, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DORY_H */
