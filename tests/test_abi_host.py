"""Host-side checks of the C ABI that need no GPU: the library loads and exports
every declared symbol; argument and state validation; the paged KV allocator's
footprint (per_loop grows with k, last_loop stays at the one-loop size)."""
import re
import os

import pytest

import synth
from looped_ngpt_transformer_amd import dory as D

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_POOL = 0x7F0000000000  # never dereferenced: these calls do host work only
FAKE_WS = 0x7F1000000000


def declared_symbols():
    with open(os.path.join(ROOT, "include", "dory.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(dory_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    L = D.lib()
    names = declared_symbols()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(D._SIGS)


def cfg(name="T", **kw):
    c = synth.config(name)
    lim = dict(max_loops=4, max_seqs=4, max_seq_len=4096, max_rows=256)
    lim.update(kw)
    return D.make_config(c, **lim)


def ctx_with_fakes(c, pages=100000, bind_weights=False):
    ctx = D.dory_create(c)
    pb, wb = D.dory_query_sizes(c)
    D.dory_bind_kv_pool(ctx, FAKE_POOL, pages * pb)
    D.dory_bind_workspace(ctx, FAKE_WS, wb)
    if bind_weights:
        w = D.dory_layer_weights(*[0x7F2000000000 + 256 * i for i in range(11)])
        for l in range(c.n_in + c.n_rec + c.n_out):
            D.dory_bind_weights(ctx, l, w)
    return ctx


def test_create_validation():
    ok = cfg()
    ctx = D.dory_create(ok)
    assert D.dory_get_loops(ctx) == 2 and D.dory_get_kv_mode(ctx) == D.KV_PER_LOOP
    D.dory_destroy(ctx)
    for field, val, code in [("hidden", 0, D.ERR_INVALID_ARG), ("n_kv_heads", 3, D.ERR_INVALID_ARG),
                             ("head_dim", 63, D.ERR_INVALID_ARG), ("n_rec", 0, D.ERR_INVALID_ARG),
                             ("max_loops", 9, D.ERR_INVALID_ARG), ("max_seq_len", 262145, D.ERR_INVALID_ARG),
                             ("weight_format", D.WFMT_BF16, D.ERR_INVALID_ARG),
                             ("head_dim", 264, D.ERR_UNSUPPORTED), ("head_dim", 48, D.ERR_UNSUPPORTED)]:
        c = cfg()
        setattr(c, field, val)
        with pytest.raises(D.DoryError) as e:
            D.dory_create(c)
        assert e.value.code == code, (field, val)
        assert D.dory_last_error(None)


def test_loops_and_mode_setters():
    ctx = D.dory_create(cfg())
    for bad in (0, 5):
        with pytest.raises(D.DoryError) as e:
            D.dory_set_loops(ctx, bad)
        assert e.value.code == D.ERR_INVALID_ARG
    with pytest.raises(D.DoryError) as e:
        D.dory_set_kv_mode(ctx, 7)
    assert e.value.code == D.ERR_INVALID_ARG
    D.dory_set_loops(ctx, 4)
    D.dory_set_kv_mode(ctx, D.KV_LAST_LOOP)
    assert D.dory_get_loops(ctx) == 4 and D.dory_get_kv_mode(ctx) == D.KV_LAST_LOOP
    D.dory_destroy(ctx)


def test_calls_before_binding_are_state_errors():
    ctx = D.dory_create(cfg())
    with pytest.raises(D.DoryError) as e:
        D.lib().dory_prefill(ctx, None, 1, None, None, None, None) and None
        D._check(D.lib().dory_prefill(ctx, None, 1, None, None, None, None), ctx)
    assert e.value.code == D.ERR_STATE
    with pytest.raises(D.DoryError) as e:
        D.dory_test_reserve(ctx, 0, 10)
    assert e.value.code == D.ERR_STATE
    D.dory_destroy(ctx)


def test_prefill_argument_checks_before_device_work():
    c = cfg()
    ctx = ctx_with_fakes(c, bind_weights=True)

    class FakeT:  # only data_ptr() is used by the binding
        def data_ptr(self):
            return 0x7F3000000000
    x = FakeT()
    for ids, nn, code in [([1, 1], [2, 2], D.ERR_INVALID_ARG), ([1], [0], D.ERR_INVALID_ARG),
                          ([1], [257], D.ERR_INVALID_ARG), ([1], [4097], D.ERR_INVALID_ARG)]:
        with pytest.raises(D.DoryError) as e:
            D.dory_prefill(ctx, ids, nn, x, x, stream=0)
        assert e.value.code == code, (ids, nn)
    with pytest.raises(D.DoryError) as e:
        D.dory_decode_step(ctx, [5], x, x, stream=0)
    assert e.value.code == D.ERR_INVALID_ARG                      # unknown sequence
    assert D.dory_live_seqs(ctx) == 0 and D.dory_kv_bytes_in_use(ctx) == 0
    D.dory_destroy(ctx)


@pytest.mark.parametrize("name", ["T", "D"])
def test_last_loop_footprint_is_one_loop_size(name):
    """KV bytes held: last_loop the same at every k; per_loop grows by one slot per
    recurrent attention layer and loop (arXiv §6.1)."""
    sizes = {}
    for mode in ("per_loop", "last_loop"):
        for k in (1, 2, 4):
            c = cfg(name, max_seq_len=8192, max_rows=64)
            ctx = ctx_with_fakes(c)
            D.dory_set_kv_mode(ctx, D.MODES[mode])
            D.dory_set_loops(ctx, k)
            D.dory_test_reserve(ctx, 0, 5000)
            D.dory_test_reserve(ctx, 1, 3000)
            sizes[(mode, k)] = D.dory_kv_bytes_in_use(ctx)
            need = sum(D.dory_kv_pages_needed(c, D.MODES[mode], k, n, 1) for n in (5000, 3000))
            assert sizes[(mode, k)] == need * D.dory_query_sizes(c)[0]
            D.dory_destroy(ctx)
    assert sizes[("last_loop", 1)] == sizes[("last_loop", 2)] == sizes[("last_loop", 4)]
    assert sizes[("per_loop", 1)] == sizes[("last_loop", 1)]
    assert sizes[("per_loop", 1)] < sizes[("per_loop", 2)] < sizes[("per_loop", 4)]


def test_page_counts_by_formula():
    c = cfg("D", max_seq_len=32768, max_rows=32, max_seqs=32)
    pb, _ = D.dory_query_sizes(c)
    assert pb == 2 * 4 * 64 * 160 * 2                 # K and V, 4 KV heads, 64 tokens, bf16
    ring = -(-(1024 + 32 - 1) // 64) + 1               # sliding layers keep a ring
    full = sum(1 for l in range(72) if l % 4 == 3)
    assert full == 18
    n_rec_full = sum(1 for l in range(16, 56) if l % 4 == 3)
    for mode, k in (("last_loop", 4), ("per_loop", 2), ("per_loop", 4)):
        slots_full = 18 + (k - 1) * n_rec_full if mode == "per_loop" else 18
        slots_swa = 54 + (k - 1) * (40 - n_rec_full) if mode == "per_loop" else 54
        want = slots_full * 512 + slots_swa * ring
        assert D.dory_kv_pages_needed(c, D.MODES[mode], k, 32768, 1) == want


def test_mode_and_loop_changes_with_live_sequences():
    c = cfg()
    ctx = ctx_with_fakes(c)
    D.dory_test_reserve(ctx, 3, 100)
    with pytest.raises(D.DoryError) as e:
        D.dory_set_kv_mode(ctx, D.KV_LAST_LOOP)
    assert e.value.code == D.ERR_STATE
    # per_loop: the context's k applies to sequences created later; a live sequence keeps
    # the k its cache was built for (mixed loop counts in one call)
    D.dory_set_loops(ctx, 3)
    D.dory_test_reserve(ctx, 4, 50)
    assert D.dory_seq_loops(ctx, 3) == 2 and D.dory_seq_loops(ctx, 4) == 3
    with pytest.raises(D.DoryError) as e:               # per_loop KV was built for k=2
        D.dory_set_seq_loops(ctx, 3, 4)
    assert e.value.code == D.ERR_STATE
    D.dory_set_seq_loops(ctx, 3, 1)                     # fewer loops (drafting): allowed
    assert D.dory_seq_loops(ctx, 3) == 1
    D.dory_set_seq_loops(ctx, 3, 0)                     # back to the k its cache holds
    assert D.dory_seq_loops(ctx, 3) == 2
    with pytest.raises(D.DoryError) as e:
        D.dory_truncate_seq(ctx, 3, 101)                # longer than the sequence
    assert e.value.code == D.ERR_INVALID_ARG
    D.dory_truncate_seq(ctx, 3, 60)
    assert D.dory_seq_len(ctx, 3) == 60
    with pytest.raises(D.DoryError) as e:
        D.dory_set_seq_loops(ctx, 99, 2)                # unknown sequence
    assert e.value.code == D.ERR_INVALID_ARG
    D.dory_release_seq(ctx, 3)
    D.dory_release_seq(ctx, 4)
    D.dory_set_kv_mode(ctx, D.KV_LAST_LOOP)
    D.dory_test_reserve(ctx, 3, 100)
    D.dory_set_loops(ctx, 4)                            # last_loop: allowed while live
    assert D.dory_seq_loops(ctx, 3) == 4                # follows the context's k ...
    D.dory_set_seq_loops(ctx, 3, 1)                     # ... until set for the sequence
    D.dory_set_loops(ctx, 2)
    assert D.dory_seq_loops(ctx, 3) == 1
    D.dory_set_seq_loops(ctx, 3, 0)                     # 0: back to the context's
    assert D.dory_seq_loops(ctx, 3) == 2
    with pytest.raises(D.DoryError) as e:
        D.dory_set_seq_loops(ctx, 3, 5)                 # max_loops is 4
    assert e.value.code == D.ERR_INVALID_ARG
    D.dory_destroy(ctx)


def test_out_of_kv_leaves_context_unchanged():
    c = cfg()
    need = D.dory_kv_pages_needed(c, D.KV_PER_LOOP, 2, 1000, 1)
    ctx = ctx_with_fakes(c, pages=need + 3)
    D.dory_test_reserve(ctx, 0, 1000)
    used = D.dory_kv_bytes_in_use(ctx)
    with pytest.raises(D.DoryError) as e:
        D.dory_test_reserve(ctx, 1, 1000)
    assert e.value.code == D.ERR_OUT_OF_KV
    assert D.dory_kv_bytes_in_use(ctx) == used and D.dory_live_seqs(ctx) == 1
    with pytest.raises(D.DoryError):
        D.dory_seq_len(ctx, 1)
    D.dory_release_seq(ctx, 0)
    assert D.dory_kv_bytes_in_use(ctx) == 0
    D.dory_test_reserve(ctx, 1, 1000)                   # freed pages are reusable
    assert D.dory_seq_len(ctx, 1) == 1000
    D.dory_destroy(ctx)


def test_sequence_limits():
    c = cfg(max_seqs=2, max_seq_len=300)
    ctx = ctx_with_fakes(c)
    D.dory_test_reserve(ctx, 0, 250)
    with pytest.raises(D.DoryError) as e:
        D.dory_test_reserve(ctx, 0, 51)                 # position 300 >= max_seq_len
    assert e.value.code == D.ERR_INVALID_ARG
    D.dory_test_reserve(ctx, 0, 50)
    D.dory_test_reserve(ctx, 1, 1)
    with pytest.raises(D.DoryError) as e:
        D.dory_test_reserve(ctx, 2, 1)                  # a third live sequence
    assert e.value.code == D.ERR_INVALID_ARG
    assert D.dory_seq_len(ctx, 0) == 300
    D.dory_destroy(ctx)


def test_vocabulary_calls_validate_before_device_work():
    c = cfg()
    ctx = ctx_with_fakes(c, bind_weights=True)
    fake = 0x7F3000000000
    with pytest.raises(D.DoryError) as e:      # vocabulary not bound yet
        D._check(D.lib().dory_embed(ctx, None, 1, D.C.c_void_p(fake), D.C.c_void_p(fake)), ctx)
    assert e.value.code == D.ERR_STATE
    with pytest.raises(D.DoryError) as e:
        D._check(D.lib().dory_logits(ctx, None, 1, D.C.c_void_p(fake), D.C.c_void_p(fake)), ctx)
    assert e.value.code == D.ERR_STATE
    for vocab, ptrs in ((100, (fake, fake, fake)), (0, (fake, fake, fake)), (1 << 25, (fake, fake, fake)),
                        (1024, (0, fake, fake)), (1024, (fake + 8, fake, fake))):
        v = D.dory_vocab_weights(vocab, *ptrs)
        with pytest.raises(D.DoryError) as e:
            D._check(D.lib().dory_bind_vocab(ctx, D.C.byref(v)), ctx)
        assert e.value.code == D.ERR_INVALID_ARG
    D._check(D.lib().dory_bind_vocab(ctx, D.C.byref(D.dory_vocab_weights(1024, fake, fake, fake))), ctx)
    for n in (0, 257):                          # max_rows is 256
        with pytest.raises(D.DoryError) as e:
            D._check(D.lib().dory_logits(ctx, None, n, D.C.c_void_p(fake), D.C.c_void_p(fake)), ctx)
        assert e.value.code == D.ERR_INVALID_ARG
        with pytest.raises(D.DoryError) as e:
            D._check(D.lib().dory_embed(ctx, None, n, D.C.c_void_p(fake), D.C.c_void_p(fake)), ctx)
        assert e.value.code == D.ERR_INVALID_ARG
    D.dory_destroy(ctx)


@pytest.mark.parametrize("n,vocab,ld,temp,top_p", [
    (0, 1000, 1000, 1.0, 0.95), (1, 0, 1000, 1.0, 0.95), (1, 1000, 999, 1.0, 0.95),
    (1, 1000, 1000, 0.0, 0.95), (1, 1000, 1000, float("inf"), 0.95), (1, 1000, 1000, 1.0, 0.0),
    (1, 1000, 1000, 1.0, 1.5), (1, 1000, 1000, 1.0, float("nan")), (1, (1 << 24) + 1, 1 << 25, 1.0, 0.9)])
def test_sampler_rejects_bad_arguments(n, vocab, ld, temp, top_p):
    fake = D.C.c_void_p(0x7F3000000000)
    rc = D.lib().dory_sample_top_p(None, n, vocab, fake, ld, temp, top_p, fake, fake)
    assert rc == D.ERR_INVALID_ARG
    assert "sampling" in D.lib().dory_last_error(None).decode()


def test_capture_and_resume_options():
    """The activation-reuse options are host bookkeeping: null buffers are refused, others
    are taken without touching them, and a call on an unbound context still fails as a
    state error with the options set (that the options are consumed is checked on the GPU)."""
    ctx = D.dory_create(cfg())
    buf = 4096   # an address never dereferenced: no call here reaches device work
    with pytest.raises(D.DoryError) as e:
        D._check(D.lib().dory_capture_states(ctx, None, buf, 0), ctx)
    assert e.value.code == D.ERR_INVALID_ARG
    with pytest.raises(D.DoryError) as e:
        D._check(D.lib().dory_resume_states(ctx, buf, None), ctx)
    assert e.value.code == D.ERR_INVALID_ARG
    D._check(D.lib().dory_capture_states(ctx, buf, buf, 1), ctx)
    D._check(D.lib().dory_resume_states(ctx, buf, buf), ctx)
    with pytest.raises(D.DoryError) as e:
        D._check(D.lib().dory_prefill(ctx, None, 1, None, None, None, None), ctx)
    assert e.value.code == D.ERR_STATE
    D.dory_destroy(ctx)


def test_decode_split_counts():
    """The split-K count a decode-shaped projection takes (host only: with no output the
    call just reports it). bf16 at <= 32 rows: K ranges of 512 where that leaves >= 300
    work-groups, else 256; a matrix whose 64-column tiles fill the device unsplit (the LM
    head over 131072 tokens) takes no split, so its partials stay within the workspace."""
    import torch
    A = torch.zeros((32, 4096), dtype=torch.bfloat16)
    B = torch.zeros((64, 64), dtype=torch.bfloat16)  # never read: no output, no launch
    cases = {(6400, 2560): 5, (8192, 2560): 5, (2560, 2560): 10, (2560, 4096): 8, (131072, 2560): 1}
    for (N, K), want in cases.items():
        assert D.dory_test_gemm(A, B, D.EPI_PARTIAL, None, stream=0, M=32, N=N, K=K) == want, (N, K)


def test_mxfp8_decode_split_counts():
    """MXFP8 projections at 33-128 rows split K into ranges of 2, 4, 5, 8 or 10 chunks of
    128, the fewest splits that give >= 192 work-groups of 64 weight rows; at <= 32 and
    above 128 rows the 128-row tiles keep their own rule (host only, no launch)."""
    import torch
    A = torch.zeros((128, 4096), dtype=torch.bfloat16)
    B = torch.zeros((64, 64), dtype=torch.uint8)
    Bs = torch.zeros((64, 2), dtype=torch.uint8)
    cases = {(128, 6400, 2560): 2, (128, 8192, 2560): 2, (128, 2560, 2560): 5, (128, 2560, 4096): 8,
             (33, 1280, 2560): 10, (40, 12288, 1024): 1, (97, 6144, 1280): 2, (70, 2560, 2560): 5}
    for (M, N, K), want in cases.items():
        got = D.dory_test_gemm(A, B, D.EPI_PARTIAL, None, B_scales=Bs, stream=0, M=M, N=N, K=K)
        assert got == want, (M, N, K, got)
    # outside 33-128 rows: the tile rule (K / 64 even splits, at most 8)
    for M in (32, 129):
        got = D.dory_test_gemm(A, B, D.EPI_PARTIAL, None, B_scales=Bs, stream=0, M=M, N=2560, K=2560)
        assert got in (1, 2, 4, 8), (M, got)


def test_arrange_weights_validates_before_device_work():
    """dory_arrange_weights refuses bad shapes, null pointers and overlap on the host."""
    import torch
    w = torch.zeros((64, 128), dtype=torch.bfloat16)
    out = torch.zeros(64 * 128, dtype=torch.bfloat16)
    for bad in (torch.zeros((60, 128), dtype=torch.bfloat16), torch.zeros((64, 100), dtype=torch.bfloat16)):
        with pytest.raises(D.DoryError):
            D.dory_arrange_weights(bad, out, stream=0)
    with pytest.raises(D.DoryError):
        D.dory_arrange_weights(w, w, stream=0)  # in place: overlaps
    with pytest.raises(D.DoryError):
        D.dory_arrange_weights(w, None, stream=0)
