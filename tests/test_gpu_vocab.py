"""GPU parity of the vocabulary side through the C ABI: token embedding, LM head with
its logit scale, and top-p sampling, against the float64 oracle on the same seeded
tables, states and draws.

Tolerances: embedding rows |d| <= 1e-6 (one float32 norm); logits |d| <= s_z * (2^-9 +
1e-5) in a bf16 context (the states enter the product rounded to bf16: |sum e_c d_c| <=
2^-9 |e| |s| for unit rows and states) and s_z * 1e-5 in an fp32 context. Sampling sums
in float32 where the oracle sums in float64 (per-thread runs of <= 128 positive terms, then
fixed trees: relative error below about 1e-5), so a token is checked for validity: it lies
in the oracle's nucleus, or in one a cut within 5e-5 of top_p gives, and the draw falls
in the token's interval of that renormalised nucleus widened by 5e-5. Where the draw is
further than that from every boundary the token must equal the oracle's."""
import numpy as np
import pytest
import torch

import synth
from looped_ngpt_transformer_amd import dory as D
from looped_ngpt_transformer_amd.runtime import DoryRuntime
from oracle import vocab as OV
from tests.gpu_helpers import check_valid, gpu_weights
from tests.helpers import to_np

pytestmark = pytest.mark.gpu

PSMALL = synth.config("P", n_in=1, n_rec=1, n_out=1, window=64)
TSMALL = synth.config("T")


def runtime(shape, vocab, seed=21, max_rows=256, scale=(15.0, 25.0)):
    rt = DoryRuntime(shape, gpu_weights(shape, 7), max_loops=2, max_seqs=1, max_seq_len=128,
                     max_rows=max_rows, loops=1)
    tables = synth.make_vocab(shape, vocab, seed, "cuda", scale=scale)
    rt.bind_vocab(tables)
    return rt, tables


@pytest.mark.parametrize("shape", [PSMALL, TSMALL], ids=["bf16", "f32"])
def test_embedding(shape):
    rt, tab = runtime(shape, 4096)
    ids = synth.make_ids(200, 4096, 5, "cuda")
    ids[3], ids[7], ids[11], ids[12] = -1, 4096, 0, 4095      # two invalid ids, both ends
    x = rt.embed(ids)
    torch.cuda.synchronize()
    want = OV.embed(to_np(tab["embed"]), ids.cpu().numpy())
    got = x.cpu().double().numpy()
    assert np.abs(got - want).max() <= 1e-6
    assert np.all(got[3] == 0) and np.all(got[7] == 0)
    rt.close()


@pytest.mark.parametrize("n", [1, 32, 200, 300])
def test_logits_bf16(n):
    rt, tab = runtime(PSMALL, 8192, max_rows=320)
    s = synth.make_inputs(n, PSMALL["hidden"], 31, device="cuda")
    lg = rt.logits(s)
    torch.cuda.synchronize()
    sz = to_np(tab["logit_scale"])
    want = OV.logits(to_np(s), to_np(tab["lm_head"]), sz)
    d = np.abs(lg.cpu().double().numpy() - want)
    assert np.all(d <= sz[None, :] * (2.0 ** -9 + 1e-5)), f"max |d| {d.max():.3e}"
    rt.close()


def test_logits_f32():
    rt, tab = runtime(TSMALL, 2048)
    s = synth.make_inputs(50, TSMALL["hidden"], 32, device="cuda")
    lg = rt.logits(s)
    torch.cuda.synchronize()
    sz = to_np(tab["logit_scale"])
    want = OV.logits(to_np(s), to_np(tab["lm_head"]), sz)
    assert np.all(np.abs(lg.cpu().double().numpy() - want) <= sz[None, :] * 1e-5)
    rt.close()


def test_logits_full_vocabulary():
    """The LM head at the tokenizer's 131072 tokens for a decode batch of 32."""
    rt, tab = runtime(PSMALL, synth.VOCAB)
    s = synth.make_inputs(32, PSMALL["hidden"], 33, device="cuda")
    lg = rt.logits(s)
    torch.cuda.synchronize()
    sz = to_np(tab["logit_scale"])
    want = OV.logits(to_np(s), to_np(tab["lm_head"]), sz)
    d = np.abs(lg.cpu().double().numpy() - want)
    assert np.all(d <= sz[None, :] * (2.0 ** -9 + 1e-5)), f"max |d| {d.max():.3e}"
    rt.close()


def sample(lg, u, temperature=1.0, top_p=0.95):
    tok = torch.full((lg.shape[0],), -7, dtype=torch.int32, device="cuda")
    D.dory_sample_top_p(lg, u, tok, temperature=temperature, top_p=top_p)
    torch.cuda.synchronize()
    return tok.cpu().numpy()


@pytest.mark.parametrize("scale,min_exact", [((15.0, 25.0), 0), ((300.0, 500.0), 28)], ids=["flat", "peaked"])
def test_sampling_full_vocabulary(scale, min_exact):
    """Rows of real LM-head logits at 131072 tokens: near-uniform (the nucleus holds most
    of the vocabulary, each token's interval of u is narrower than the tolerance, so only
    validity is checked) and peaked (a few hundred tokens: the draws pick exact tokens)."""
    rt, tab = runtime(PSMALL, synth.VOCAB, scale=scale)
    s = synth.make_inputs(32, PSMALL["hidden"], 34, device="cuda")
    lg = rt.logits(s)
    u = synth.make_draws(32, 35, device="cuda")
    toks = sample(lg, u)
    exact = check_valid(lg.cpu().double().numpy(), u.cpu().numpy(), toks, 1.0, 0.95)
    assert exact >= min_exact
    assert np.array_equal(sample(lg, u), toks)          # deterministic
    rt.close()


@pytest.mark.parametrize("vocab,temperature,top_p", [(1000, 1.0, 0.95), (777, 0.5, 0.9), (5000, 2.0, 0.5),
                                                     (1, 1.0, 0.95), (3000, 1.0, 1.0)])
def test_sampling_small_vocabularies(vocab, temperature, top_p):
    g = torch.Generator().manual_seed(vocab)
    lg = (torch.randn((64, vocab), generator=g) * 3).cuda()
    u = synth.make_draws(64, vocab, device="cuda")
    toks = sample(lg, u, temperature, top_p)
    exact = check_valid(lg.cpu().double().numpy(), u.cpu().numpy(), toks, temperature, top_p)
    assert exact >= 48   # rows whose draw is clear of every boundary (each one compared exactly)


def test_sampling_row_stride_and_greedy():
    g = torch.Generator().manual_seed(3)
    big = (torch.randn((16, 2100), generator=g) * 4).cuda()
    lg = big[:, :2000]                                   # row stride 2100
    u = synth.make_draws(16, 4, device="cuda")
    toks = sample(lg, u, 1.0, 1e-7)                      # nucleus of one token: the argmax
    assert np.array_equal(toks, lg.cpu().numpy().argmax(axis=1))


def test_sampling_equal_logits_go_by_id():
    # 4096 equal logits: every weight is exactly 1, so the float32 running sums are exact;
    # the nucleus is the first 3892 ids (3891 / 4096 < 0.95 <= 3892 / 4096)
    lg = torch.zeros((8, 4096), device="cuda")
    u = torch.tensor([0.0, 0.1, 0.25, 0.5, 0.75, 0.9, 0.99, 0.9999], device="cuda")
    toks = sample(lg, u)
    want = [OV.sample_top_p(np.zeros(4096), 1.0, 0.95, float(x)) for x in u.cpu().numpy()]
    assert list(toks) == want
    assert max(want) < 3892


def test_generation_loop_against_oracle():
    """Three generation steps on the Dory layer shape after a 40-token prompt: decode ->
    LM head -> top-p -> embedding of the sampled token -> next decode input. Each step's
    final states are compared with the oracle's decode of the same input, the logits
    with the oracle's LM head on the GPU's states, the token for validity on the GPU's
    logits, and the next input with the oracle's embedding of that token (which the
    oracle then also takes as its next input)."""
    from oracle import dory_oracle as O
    from tests.gpu_helpers import compare, oracle_model
    S = PSMALL
    k, mode, V = 2, "per_loop", 8192
    w = gpu_weights(S, 11)
    rt = DoryRuntime(S, w, max_loops=2, max_seqs=1, max_seq_len=64, max_rows=64, mode=mode, loops=k)
    tab = synth.make_vocab(S, V, 12, "cuda", scale=(300.0, 500.0))
    rt.bind_vocab(tab)
    cfg, W = oracle_model(S, w)
    seq = O.Sequence(cfg)
    X = synth.make_inputs(40, S["hidden"], 13, device="cuda")
    y = rt.prefill([0], [40], X)
    torch.cuda.synchronize()
    compare(y.cpu().double().numpy(), O.prefill(cfg, W, seq, to_np(X), k, mode), S, "prompt")
    emb, head, sz = to_np(tab["embed"]), to_np(tab["lm_head"]), to_np(tab["logit_scale"])
    x = synth.make_inputs(1, S["hidden"], 14, device="cuda")
    u = synth.make_draws(3, 15, device="cuda")
    tokens = []
    for step in range(3):
        x_np = x.cpu().double().numpy()
        y = rt.decode([0], x)
        lg = rt.logits(y)
        tok = torch.empty((1,), dtype=torch.int32, device="cuda")
        D.dory_sample_top_p(lg, u[step:step + 1], tok)
        x = rt.embed(tok)
        torch.cuda.synchronize()
        y_np = y.cpu().double().numpy()
        compare(y_np, O.prefill(cfg, W, seq, x_np, k, mode), S, f"step {step}")
        lg_np = lg.cpu().double().numpy()
        d = np.abs(lg_np - OV.logits(y_np, head, sz))
        assert np.all(d <= sz[None, :] * (2.0 ** -9 + 1e-5)), f"step {step}: logits max |d| {d.max():.3e}"
        t = tok.cpu().numpy()
        check_valid(lg_np, u[step:step + 1].cpu().numpy(), t, 1.0, 0.95)
        assert np.abs(x.cpu().double().numpy() - OV.embed(emb, t)).max() <= 1e-6
        tokens.append(int(t[0]))
    rt.close()
