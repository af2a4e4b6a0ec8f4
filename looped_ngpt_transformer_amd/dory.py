"""Thin ctypes binding of the C ABI in include/dory.h.

Functions carry the C names and do argument marshalling only: torch tensors become
device pointers, the current torch stream becomes the hipStream_t, python ints become
host int32 arrays, and a non-zero status raises DoryError with the library's message.
Every step of the forward pass runs in the HIP library; there is no other path, and
loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdory.so")

OK, ERR_INVALID_ARG, ERR_STATE, ERR_OUT_OF_KV, ERR_UNSUPPORTED, ERR_HIP = 0, -1, -2, -3, -4, -5
DTYPE_F32, DTYPE_BF16 = 0, 1
WFMT_F32, WFMT_BF16, WFMT_MXFP8, WFMT_NVFP4 = 0, 1, 2, 3
KV_PER_LOOP, KV_LAST_LOOP = 0, 1
GATE_NONE, GATE_ELEMENTWISE = 0, 1
PAGE_TOKENS = 64
MAX_POSITIONS = 262144
MODES = {"per_loop": KV_PER_LOOP, "last_loop": KV_LAST_LOOP}


class DoryError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"dory error {code}: {msg}")
        self.code = code


class dory_config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("intermediate", C.c_int32), ("n_in", C.c_int32),
                ("n_rec", C.c_int32), ("n_out", C.c_int32), ("window", C.c_int32),
                ("full_period", C.c_int32), ("theta_swa", C.c_double),
                ("theta_full", C.c_double), ("attn_scale", C.c_float), ("qk_norm", C.c_int32),
                ("attn_gate", C.c_int32), ("act_dtype", C.c_int32), ("weight_format", C.c_int32),
                ("max_loops", C.c_int32), ("max_seqs", C.c_int32), ("max_seq_len", C.c_int32),
                ("max_rows", C.c_int32)]


class dory_layer_weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in
                ("w_qkvg", "w_o", "w_gu", "w_down", "s_qkvg", "s_o", "s_gu", "s_down",
                 "alpha_attn", "alpha_mlp", "s_qk", "g_qkvg", "g_o", "g_gu", "g_down",
                 "f_qkvg", "f_o", "f_gu", "f_down")]


class dory_vocab_weights(C.Structure):
    _fields_ = [("vocab", C.c_int64), ("embed", C.c_void_p), ("lm_head", C.c_void_p),
                ("logit_scale", C.c_void_p)]


class dory_kernel_stats(C.Structure):
    _fields_ = [("launches", C.c_int64), ("ms", C.c_double), ("flops", C.c_double),
                ("bytes", C.c_double)]


KC_GEMM, KC_ATTN, KC_ROPE, KC_UPDATE, KC_SWIGLU, KC_MERGE, KC_VOCAB = range(7)
KC_NAMES = {KC_GEMM: "gemm", KC_ATTN: "attention", KC_ROPE: "rope_kv", KC_UPDATE: "update",
            KC_SWIGLU: "swiglu", KC_MERGE: "attn_merge", KC_VOCAB: "vocab"}

_P = C.c_void_p
_I32P = C.POINTER(C.c_int32)
_SIGS = {
    "dory_create": (C.c_int, [C.POINTER(dory_config), C.POINTER(_P)]),
    "dory_destroy": (C.c_int, [_P]),
    "dory_last_error": (C.c_char_p, [_P]),
    "dory_query_sizes": (C.c_int, [C.POINTER(dory_config), C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "dory_kv_pages_needed": (C.c_int, [C.POINTER(dory_config), C.c_int, C.c_int, C.c_int64, C.c_int64,
                                       C.POINTER(C.c_int64)]),
    "dory_bind_weights": (C.c_int, [_P, C.c_int, C.POINTER(dory_layer_weights)]),
    "dory_bind_kv_pool": (C.c_int, [_P, _P, C.c_size_t]),
    "dory_bind_workspace": (C.c_int, [_P, _P, C.c_size_t]),
    "dory_set_loops": (C.c_int, [_P, C.c_int]),
    "dory_get_loops": (C.c_int, [_P, C.POINTER(C.c_int)]),
    "dory_set_seq_loops": (C.c_int, [_P, C.c_int32, C.c_int]),
    "dory_seq_loops": (C.c_int, [_P, C.c_int32, C.POINTER(C.c_int)]),
    "dory_truncate_seq": (C.c_int, [_P, C.c_int32, C.c_int64]),
    "dory_capture_states": (C.c_int, [_P, _P, _P, C.c_int]),
    "dory_resume_states": (C.c_int, [_P, _P, _P]),
    "dory_spec_accept": (C.c_int, [_P, C.c_int, C.c_int, C.c_int64, _P, C.c_int64, _P, C.c_int64, _P, C.c_float,
                                   C.c_float, _P, _P, _P, _P]),
    "dory_set_kv_mode": (C.c_int, [_P, C.c_int]),
    "dory_get_kv_mode": (C.c_int, [_P, C.POINTER(C.c_int)]),
    "dory_prefill": (C.c_int, [_P, _P, C.c_int, _I32P, _I32P, _P, _P]),
    "dory_decode_step": (C.c_int, [_P, _P, C.c_int, _I32P, _P, _P]),
    "dory_release_seq": (C.c_int, [_P, C.c_int32]),
    "dory_seq_len": (C.c_int, [_P, C.c_int32, C.POINTER(C.c_int64)]),
    "dory_live_seqs": (C.c_int, [_P, C.POINTER(C.c_int32)]),
    "dory_kv_bytes_in_use": (C.c_int, [_P, C.POINTER(C.c_size_t)]),
    "dory_last_layer_calls": (C.c_int, [_P, C.POINTER(C.c_int64)]),
    "dory_test_reserve": (C.c_int, [_P, C.c_int32, C.c_int32]),
    "dory_test_fill_kv": (C.c_int, [_P, _P, C.c_int32, C.c_int, C.c_int, C.c_int32, C.c_int32, _P, _P]),
    "dory_test_inject_failure": (C.c_int, [_P, C.c_int]),
    "dory_test_gemm": (C.c_int, [_P, _P, C.c_int, _P, _P, _P, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, _P,
                                 C.c_int, C.POINTER(C.c_int), _P]),
    "dory_arrange_weights": (C.c_int, [_P, _P, C.c_int64, C.c_int64, _P]),
    "dory_test_mfma_rate": (C.c_int, [_P, C.c_int, _P, _P, C.POINTER(C.c_int)]),
    "dory_quantize_mxfp8": (C.c_int, [_P, _P, C.c_int, C.c_int64, C.c_int64, _P, _P]),
    "dory_quantize_nvfp4": (C.c_int, [_P, _P, C.c_int, C.c_int64, C.c_int64, _P, _P, _P]),
    "dory_bind_vocab": (C.c_int, [_P, C.POINTER(dory_vocab_weights)]),
    "dory_embed": (C.c_int, [_P, _P, C.c_int, _P, _P]),
    "dory_logits": (C.c_int, [_P, _P, C.c_int, _P, _P]),
    "dory_logits_noalloc": (C.c_int, [_P, _P, C.c_int, _P, _P]),
    "dory_sample_top_p": (C.c_int, [_P, C.c_int, C.c_int64, _P, C.c_int64, C.c_float, C.c_float, _P, _P]),
    "dory_profile_enable": (C.c_int, [_P, C.c_int]),
    "dory_profile_read": (C.c_int, [_P, C.c_int, C.POINTER(dory_kernel_stats)]),
    "dory_sync": (C.c_int, [_P, _P]),
}

_lib = None


def lib():
    """The loaded libdory.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run looped_ngpt_transformer_amd.build.build()")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, ctx=None):
    if rc != OK:
        msg = lib().dory_last_error(ctx)
        raise DoryError(rc, msg.decode() if msg else "")


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return C.c_void_p(stream)
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _i32(values):
    a = np.ascontiguousarray(np.asarray(values, dtype=np.int32))
    return a, a.ctypes.data_as(_I32P)


_ACT = {"f32": DTYPE_F32, "bf16": DTYPE_BF16}
_WF = {"f32": WFMT_F32, "bf16": WFMT_BF16, "mxfp8": WFMT_MXFP8, "nvfp4": WFMT_NVFP4}


def make_config(d: dict, max_loops=4, max_seqs=1, max_seq_len=4096, max_rows=4096) -> dory_config:
    """dory_config from a shape dict (synth.CONFIGS entry) and runtime limits."""
    return dory_config(
        hidden=d["hidden"], n_q_heads=d["n_q_heads"], n_kv_heads=d["n_kv_heads"],
        head_dim=d["head_dim"], intermediate=d["intermediate"], n_in=d["n_in"], n_rec=d["n_rec"],
        n_out=d["n_out"], window=d["window"], full_period=d.get("full_period", 4),
        theta_swa=d["theta_swa"], theta_full=d["theta_full"], attn_scale=d["attn_scale"],
        qk_norm=d["qk_norm"], attn_gate=d["attn_gate"], act_dtype=_ACT[d["act_dtype"]],
        weight_format=_WF[d["weight_format"]], max_loops=max_loops, max_seqs=max_seqs,
        max_seq_len=max_seq_len, max_rows=max_rows)


# ------------------------------------------------------------------ C-named wrappers
def dory_create(cfg: dory_config):
    h = C.c_void_p()
    _check(lib().dory_create(C.byref(cfg), C.byref(h)))
    return h


def dory_destroy(ctx):
    _check(lib().dory_destroy(ctx))


def dory_last_error(ctx=None) -> str:
    m = lib().dory_last_error(ctx)
    return m.decode() if m else ""


def dory_query_sizes(cfg: dory_config):
    pb, wb = C.c_size_t(), C.c_size_t()
    _check(lib().dory_query_sizes(C.byref(cfg), C.byref(pb), C.byref(wb)))
    return pb.value, wb.value


def dory_kv_pages_needed(cfg: dory_config, mode: int, k: int, seq_len: int, n_seqs: int) -> int:
    p = C.c_int64()
    _check(lib().dory_kv_pages_needed(C.byref(cfg), mode, k, seq_len, n_seqs, C.byref(p)))
    return p.value


def dory_bind_weights(ctx, layer: int, w: dory_layer_weights):
    _check(lib().dory_bind_weights(ctx, layer, C.byref(w)), ctx)


def dory_bind_kv_pool(ctx, pool_ptr: int, nbytes: int):
    _check(lib().dory_bind_kv_pool(ctx, C.c_void_p(pool_ptr), nbytes), ctx)


def dory_bind_workspace(ctx, ws_ptr: int, nbytes: int):
    _check(lib().dory_bind_workspace(ctx, C.c_void_p(ws_ptr), nbytes), ctx)


def dory_set_loops(ctx, k: int):
    _check(lib().dory_set_loops(ctx, k), ctx)


def dory_get_loops(ctx) -> int:
    k = C.c_int()
    _check(lib().dory_get_loops(ctx, C.byref(k)), ctx)
    return k.value


def dory_set_seq_loops(ctx, seq_id: int, k: int):
    _check(lib().dory_set_seq_loops(ctx, seq_id, k), ctx)


def dory_seq_loops(ctx, seq_id: int) -> int:
    k = C.c_int(0)
    _check(lib().dory_seq_loops(ctx, seq_id, C.byref(k)), ctx)
    return k.value


def dory_truncate_seq(ctx, seq_id: int, length: int):
    _check(lib().dory_truncate_seq(ctx, seq_id, length), ctx)


def dory_capture_states(ctx, x_out, s1_out, skip_output_block=False):
    _check(lib().dory_capture_states(ctx, _ptr(x_out), _ptr(s1_out), int(bool(skip_output_block))), ctx)


def dory_resume_states(ctx, x_in, s1_in):
    _check(lib().dory_resume_states(ctx, _ptr(x_in), _ptr(s1_in)), ctx)


def dory_spec_accept(draft_logits, target_logits, draft_tokens, u_accept, u_sample, tokens, n_out,
                     temperature=1.0, top_p=0.95, stream=None):
    """draft_logits [gamma * n, V] and draft_tokens, u_accept [gamma, n] position-major;
    target_logits [n * (gamma + 1), V] sequence-major; tokens [n, gamma + 1], n_out [n]."""
    gamma, n = int(draft_tokens.shape[0]), int(draft_tokens.shape[1])
    _check(lib().dory_spec_accept(_stream(stream), n, gamma, int(draft_logits.shape[1]), _ptr(draft_logits),
                                  int(draft_logits.stride(0)), _ptr(target_logits), int(target_logits.stride(0)),
                                  _ptr(draft_tokens), float(temperature), float(top_p), _ptr(u_accept),
                                  _ptr(u_sample), _ptr(tokens), _ptr(n_out)))


def dory_set_kv_mode(ctx, mode: int):
    _check(lib().dory_set_kv_mode(ctx, mode), ctx)


def dory_get_kv_mode(ctx) -> int:
    m = C.c_int()
    _check(lib().dory_get_kv_mode(ctx, C.byref(m)), ctx)
    return m.value


def dory_prefill(ctx, seq_ids, n_new, x_in, y_out, stream=None):
    ids, idp = _i32(seq_ids)
    nn, nnp = _i32(n_new)
    _check(lib().dory_prefill(ctx, _stream(stream), len(ids), idp, nnp, _ptr(x_in), _ptr(y_out)), ctx)


def dory_decode_step(ctx, seq_ids, x_in, y_out, stream=None):
    ids, idp = _i32(seq_ids)
    _check(lib().dory_decode_step(ctx, _stream(stream), len(ids), idp, _ptr(x_in), _ptr(y_out)), ctx)


def dory_release_seq(ctx, seq_id: int):
    _check(lib().dory_release_seq(ctx, seq_id), ctx)


def dory_seq_len(ctx, seq_id: int) -> int:
    n = C.c_int64()
    _check(lib().dory_seq_len(ctx, seq_id, C.byref(n)), ctx)
    return n.value


def dory_live_seqs(ctx) -> int:
    n = C.c_int32()
    _check(lib().dory_live_seqs(ctx, C.byref(n)), ctx)
    return n.value


def dory_kv_bytes_in_use(ctx) -> int:
    n = C.c_size_t()
    _check(lib().dory_kv_bytes_in_use(ctx, C.byref(n)), ctx)
    return n.value


def dory_last_layer_calls(ctx) -> int:
    n = C.c_int64()
    _check(lib().dory_last_layer_calls(ctx, C.byref(n)), ctx)
    return n.value


def dory_test_reserve(ctx, seq_id: int, n_tokens: int):
    _check(lib().dory_test_reserve(ctx, seq_id, n_tokens), ctx)


def dory_test_fill_kv(ctx, seq_id, layer, slot, pos0, k, v, stream=None):
    n = k.shape[0]
    _check(lib().dory_test_fill_kv(ctx, _stream(stream), seq_id, layer, slot, pos0, n, _ptr(k), _ptr(v)), ctx)


def dory_test_inject_failure(ctx, at: int):
    _check(lib().dory_test_inject_failure(ctx, at), ctx)


EPI_F32, EPI_PARTIAL, EPI_STORE_BF16, EPI_SWIGLU = 0, 1, 2, 4


def dory_test_gemm(A, B, epi, out=None, B_scales=None, stream=None, M=None, N=None, K=None, lda=None,
                   ldc=None, B_gscale=None, B_frag=None):
    """One projection GEMM as a layer launches it: out = A B^T with the layer's epilogue
    (see dory.h). B_scales alone: MXFP8 codes; B_scales and B_gscale: NVFP4 packed codes.
    Returns the split count; with out None only the split count is computed."""
    M = M if M is not None else A.shape[0]
    K = K if K is not None else A.shape[1]
    N = N if N is not None else B.shape[0]
    lda = lda if lda is not None else A.stride(0)
    ldc = ldc if ldc is not None else (out.shape[-1] if out is not None else 0)
    wf = WFMT_NVFP4 if B_gscale is not None else WFMT_MXFP8 if B_scales is not None else WFMT_BF16
    splits = C.c_int(0)
    _check(lib().dory_test_gemm(_stream(stream), _ptr(A), lda, _ptr(B), _ptr(B_scales), _ptr(B_gscale), wf, M, N,
                                K, epi, _ptr(out), ldc, C.byref(splits), _ptr(B_frag)))
    return splits.value


def dory_arrange_weights(w, out, stream=None):
    """Fragment-order copy of the bf16 matrix w [N, K] into out (N * K bf16 elements)
    for the f_* fields of dory_layer_weights (see dory.h)."""
    N, K = w.shape
    _check(lib().dory_arrange_weights(_stream(stream), _ptr(w), N, K, _ptr(out)))


def dory_test_mfma_rate(iters, cycles, sink, stream=None):
    """Sustained bf16 MFMA rate probe (see dory.h): cycles int64 [n_cu], sink float
    [n_cu * 512] device tensors. Returns the number of work-groups launched."""
    n = C.c_int(0)
    _check(lib().dory_test_mfma_rate(_stream(stream), int(iters), _ptr(cycles), _ptr(sink), C.byref(n)))
    return n.value


def dory_quantize_mxfp8(w, codes, scales, stream=None):
    import torch
    wd = DTYPE_BF16 if w.dtype == torch.bfloat16 else DTYPE_F32
    rows, cols = w.shape
    _check(lib().dory_quantize_mxfp8(_stream(stream), _ptr(w), wd, rows, cols, _ptr(codes), _ptr(scales)))


def dory_bind_vocab(ctx, embed, lm_head, logit_scale):
    """Bind the vocabulary tables (device tensors [V, H] in the activation type, and the
    float [V] logit scale); the caller keeps them alive."""
    v = dory_vocab_weights(int(embed.shape[0]), embed.data_ptr(), lm_head.data_ptr(), logit_scale.data_ptr())
    _check(lib().dory_bind_vocab(ctx, C.byref(v)), ctx)


def dory_embed(ctx, ids, x_out, stream=None):
    _check(lib().dory_embed(ctx, _stream(stream), int(ids.shape[0]), _ptr(ids), _ptr(x_out)), ctx)


def dory_logits(ctx, states, logits, stream=None):
    _check(lib().dory_logits(ctx, _stream(stream), int(states.shape[0]), _ptr(states), _ptr(logits)), ctx)


def dory_logits_noalloc(ctx, states, logits, stream=None):
    _check(lib().dory_logits_noalloc(ctx, _stream(stream), int(states.shape[0]), _ptr(states), _ptr(logits)), ctx)


def dory_sample_top_p(logits, u, tokens, temperature=1.0, top_p=0.95, vocab=None, stream=None):
    n, ld = int(logits.shape[0]), int(logits.stride(0))
    vocab = int(logits.shape[1]) if vocab is None else int(vocab)
    _check(lib().dory_sample_top_p(_stream(stream), n, vocab, _ptr(logits), ld, float(temperature),
                                   float(top_p), _ptr(u), _ptr(tokens)))


def dory_quantize_nvfp4(w, codes, scales, g, stream=None):
    wd = DTYPE_BF16 if str(w.dtype) == "torch.bfloat16" else DTYPE_F32
    rows, cols = int(w.shape[0]), int(w.shape[1])
    _check(lib().dory_quantize_nvfp4(_stream(stream), _ptr(w), wd, rows, cols, _ptr(codes), _ptr(scales), _ptr(g)))


def dory_sync(ctx=None, stream=None):
    _check(lib().dory_sync(ctx, _stream(stream)), ctx)


def dory_profile_enable(ctx, classes):
    """classes: True (all), False/None (stop), or an iterable of KC_* class ids."""
    if classes is True:
        mask = (1 << len(KC_NAMES)) - 1
    elif not classes:
        mask = 0
    else:
        mask = 0
        for k in classes:
            mask |= 1 << k
    _check(lib().dory_profile_enable(ctx, mask), ctx)


def dory_profile_read(ctx, kclass: int) -> dict:
    r = dory_kernel_stats()
    _check(lib().dory_profile_read(ctx, kclass, C.byref(r)), ctx)
    return {"launches": r.launches, "ms": r.ms, "flops": r.flops, "bytes": r.bytes}
