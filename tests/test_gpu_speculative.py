"""GPU parity of self-speculative decoding's acceptance step (dory_spec_accept) against
the float64 oracle on the same seeded logits, draft tokens and draws.

The kernel takes each position's decisions in float32 where the oracle takes them in
float64, so a decision is demanded only where it is clear: an acceptance test whose
ratio p(x) / q(x) lies within 1e-4 (relative) of its draw, or a residual draw within
3e-5 of probability mass of a token boundary, accepts either outcome and ends the
comparison of that sequence there. Elsewhere count, accepted tokens and the drawn token
must equal the oracle's. The token after a fully accepted block is the top-p sampler's
(the same kernel path: equal to dory_sample_top_p on that row, bit for bit)."""
import numpy as np
import pytest
import torch

import synth
from looped_ngpt_transformer_amd import dory as D
from oracle import speculative as OS
from oracle import vocab as OV
from tests.gpu_helpers import check_valid

pytestmark = pytest.mark.gpu

TOL_R = 1e-4     # relative band around an acceptance ratio
TOL_M = 3e-5     # probability mass band around a residual boundary


def draft_tokens(draft, gamma, temperature, top_p, seed):
    """Draft tokens [gamma, n] drawn from the draft rows (position-major) by the oracle's
    sampler (the draft model's own choices), so most lie in the draft nucleus."""
    n = draft.shape[0] // gamma
    u = synth.make_draws(n * gamma, seed).numpy()
    d = draft.cpu().double().numpy()
    return np.array([OV.sample_top_p(d[i], temperature, top_p, float(u[i])) for i in range(n * gamma)],
                    dtype=np.int32).reshape(gamma, n)


def run(draft, target, toks, u_acc, u_smp, temperature, top_p):
    gamma, n = toks.shape
    out = torch.full((n, gamma + 1), -9, dtype=torch.int32, device="cuda")
    n_out = torch.full((n,), -9, dtype=torch.int32, device="cuda")
    D.dory_spec_accept(draft, target, torch.from_numpy(toks).cuda(), u_acc, u_smp, out, n_out,
                       temperature=temperature, top_p=top_p)
    torch.cuda.synchronize()
    return out.cpu().numpy(), n_out.cpu().numpy()


def check_sequence(dr, tg, x, ua, us, out, n_out, temperature, top_p):
    """Returns True when every decision of the sequence was clear (and matched)."""
    gamma = len(x)
    assert 1 <= n_out <= gamma + 1
    for j in range(gamma):
        p = OS.processed(tg[j], temperature, top_p)
        q = OS.processed(dr[j], temperature, top_p)
        ratio = p[x[j]] / q[x[j]] if (0 <= x[j] < p.size and q[x[j]] > 0) else 0.0
        if abs(ua[j] - ratio) <= TOL_R * max(ratio, 1e-30):
            assert out[j] == x[j] or n_out == j + 1
            return False
        if ua[j] < ratio:
            assert out[j] == x[j] and n_out > j + 1, f"position {j}: accepted {x[j]}, got {out[j]} n_out {n_out}"
            continue
        assert n_out == j + 1, f"position {j}: rejected, n_out {n_out}"
        r = np.maximum(p - q, 0.0)
        total = r.sum()
        if total <= TOL_M:
            return False                 # residual too small to tell from an empty one
        tok = int(out[j])
        assert 0 <= tok < p.size
        cum = np.cumsum(r)
        lo, hi, target = (cum[tok - 1] if tok else 0.0), cum[tok], us * total
        assert lo - TOL_M <= target <= hi + TOL_M, f"position {j}: residual token {tok}"
        if lo + TOL_M < target < hi - TOL_M:
            assert tok == OS.residual_draw(p, q, us)
            return True
        return False
    assert n_out == gamma + 1
    check_valid(tg[gamma:gamma + 1], np.array([us]), out[gamma:gamma + 1], temperature, top_p)
    return True


@pytest.mark.parametrize("n,gamma,vocab,temperature,top_p,min_clear", [
    (3, 1, 2048, 1.0, 0.95, 2),
    (33, 4, 2048, 1.0, 0.95, 20),
    (8, 7, 4096, 0.7, 0.9, 4),
    (4, 4, synth.VOCAB, 1.0, 0.95, 2),
])
def test_accept_matches_oracle(n, gamma, vocab, temperature, top_p, min_clear):
    draft, target = synth.make_spec_logits(n, gamma, vocab, 61, device="cuda")
    x = draft_tokens(draft, gamma, temperature, top_p, 62)
    x[0, 0] = -1                                  # invalid id: q = 0, always rejected
    u_acc = synth.make_draws(n * gamma, 63, device="cuda")
    u_smp = synth.make_draws(n, 64, device="cuda")
    out, n_out = run(draft, target, x, u_acc, u_smp, temperature, top_p)
    assert n_out[0] == 1
    dr, tg = draft.cpu().double().numpy(), target.cpu().double().numpy()
    dr = dr.reshape(gamma, n, vocab)
    ua, us = u_acc.cpu().numpy().reshape(gamma, n), u_smp.cpu().numpy()
    clear = 0
    for b in range(n):
        clear += check_sequence(dr[:, b], tg[b * (gamma + 1):(b + 1) * (gamma + 1)], x[:, b],
                                ua[:, b], float(us[b]), out[b], int(n_out[b]), temperature, top_p)
    assert clear >= min_clear
    assert 0 < (n_out - 1).sum() < n * gamma      # some drafts accepted, some rejected
    out2, n_out2 = run(draft, target, x, u_acc, u_smp, temperature, top_p)
    assert np.array_equal(n_out2, n_out) and all(np.array_equal(out2[b, :n_out[b]], out[b, :n_out[b]])
                                                 for b in range(n))


def test_same_model_accepts_everything():
    """Draft rows equal to the verifying rows: every draft in the nucleus is accepted and
    the extra token is the sampler's own draw on the last row."""
    n, gamma, vocab = 16, 4, 8192
    _, target = synth.make_spec_logits(n, gamma, vocab, 65, spread=6.0, device="cuda")
    tg = target.view(n, gamma + 1, vocab)
    draft = tg[:, :gamma].transpose(0, 1).contiguous().view(gamma * n, vocab)
    x = draft_tokens(draft, gamma, 1.0, 0.95, 66)
    u_acc = synth.make_draws(n * gamma, 67, device="cuda")
    u_smp = synth.make_draws(n, 68, device="cuda")
    out, n_out = run(draft, target, x, u_acc, u_smp, 1.0, 0.95)
    assert np.all(n_out == gamma + 1)
    assert np.array_equal(out[:, :gamma], x.T)
    last = tg[:, gamma].contiguous()
    want = torch.empty(n, dtype=torch.int32, device="cuda")
    D.dory_sample_top_p(last, u_smp, want, temperature=1.0, top_p=0.95)
    torch.cuda.synchronize()
    assert np.array_equal(out[:, gamma], want.cpu().numpy())


def test_first_token_follows_the_target():
    """Over many draws the first emitted token is distributed as the verifying model's
    processed distribution, whatever the draft (the point of the rejection rule): a
    chi-square statistic over a 24-token vocabulary with 20000 seeded trials."""
    n, gamma, vocab = 20000, 2, 24
    d1, t1 = synth.make_spec_logits(1, gamma, vocab, 69, spread=1.0, noise=1.5)
    draft = d1.view(gamma, 1, vocab).expand(gamma, n, vocab).reshape(gamma * n, vocab).cuda()
    target = t1.repeat(n, 1).cuda()
    q0 = OS.processed(d1[0].double().numpy(), 1.0, 1.0)
    ux = synth.make_draws(n, 70).numpy()
    cq = np.cumsum(q0)
    x = np.zeros((gamma, n), dtype=np.int32)
    x[0] = np.minimum(np.searchsorted(cq, ux * cq[-1], side="right"), vocab - 1)
    x[1] = 3
    u_acc = synth.make_draws(n * gamma, 71, device="cuda")
    u_smp = synth.make_draws(n, 72, device="cuda")
    out, _ = run(draft, target, x, u_acc, u_smp, 1.0, 1.0)
    p0 = OS.processed(t1[0].double().numpy(), 1.0, 1.0)
    counts = np.bincount(out[:, 0], minlength=vocab)
    expect = p0 * n
    keep = expect > 5
    chi2 = float((((counts - expect) ** 2)[keep] / expect[keep]).sum())
    assert chi2 < 60.0, f"chi2 {chi2:.1f} over {int(keep.sum())} cells"   # 23 dof: p < 1e-5 beyond 60


def test_bad_arguments():
    lg = torch.zeros((2, 256), device="cuda")
    x = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
    u = torch.zeros(1, device="cuda")
    out = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    n_out = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(D.DoryError):
        D.dory_spec_accept(lg[:1], lg, x, u, u, out, n_out, temperature=0.0)
    with pytest.raises(D.DoryError):
        D.dory_spec_accept(lg[:1], lg, x, u, u, out, n_out, top_p=1.5)


# End to end the logits differ from the oracle's by the forward's rounding: at most
# LOGIT_TOL, which moves each probability by a factor within exp(+-2 LOGIT_TOL) and so
# every cumulative boundary by less than 2.1 LOGIT_TOL < BAND.
LOGIT_TOL = 6e-4
BAND = 2e-3


def clear_draw(row, u, temperature, top_p):
    """The oracle's top-p token for u, or None when a logit error of the forward's size
    could move the nucleus cut or a boundary of u across."""
    order, _, cum = OV.sorted_order(row, temperature)
    m = OV.nucleus_size(cum, top_p)
    if cum[m - 1] - top_p < BAND or (m > 1 and top_p - cum[m - 2] < BAND):
        return None
    tok = OV.sample_top_p(row, temperature, top_p, u)
    _, _, lo, hi = OV.draw_interval(row, temperature, top_p, tok)
    return tok if lo + BAND < u < hi - BAND else None


def oracle_spec(cfg, W, seq, tab, cur, gamma, ud, ua, us, k, mode, gpu, b, n, T=1.0, top_p=0.95):
    """The step for sequence b on the oracle model, compared with the GPU's as it goes.
    Returns the emitted tokens, or None once a decision is too close to call (the
    sequence is then dropped)."""
    from oracle import dory_oracle as O
    emb, head, sz = tab
    L0, tok, xs, qrows = seq.length, cur, [], []
    for j in range(gamma):
        row = OV.logits(O.prefill(cfg, W, seq, OV.embed(emb, [tok]), 1, mode), head, sz)
        d = np.abs(gpu["draft"][j * n + b] - row[0]).max()
        assert d <= LOGIT_TOL, f"draft row {j}: max |d| {d:.3e}"
        qrows.append(row[0])
        tok = clear_draw(row[0], float(ud[j]), T, top_p)
        if tok is None:
            return None
        assert gpu["drafts"][j, b] == tok, f"draft token {j}"
        xs.append(tok)
    seq.length = L0
    tg = OV.logits(O.prefill(cfg, W, seq, OV.embed(emb, [cur] + xs), k, mode), head, sz)
    d = np.abs(gpu["target"][b * (gamma + 1):(b + 1) * (gamma + 1)] - tg).max()
    assert d <= LOGIT_TOL, f"verifying rows: max |d| {d:.3e}"
    out = []
    for j in range(gamma):
        p = OS.processed(tg[j], T, top_p)
        q = OS.processed(qrows[j], T, top_p)
        ratio = p[xs[j]] / q[xs[j]] if q[xs[j]] > 0 else 0.0
        if abs(ua[j] - ratio) <= BAND * max(ratio, 1e-30) or q[xs[j]] < BAND:
            return None
        if ua[j] < ratio:
            out.append(xs[j])
            continue
        r = np.maximum(p - q, 0.0)
        if r.sum() < 0.05:
            return None
        t = OS.residual_draw(p, q, us)
        c = np.cumsum(r)
        lo, hi = (c[t - 1] if t else 0.0), c[t]
        if not (lo + BAND < us * c[-1] < hi - BAND):
            return None
        out.append(t)
        break
    else:
        t = clear_draw(tg[gamma], us, T, top_p)
        if t is None:
            return None
        out.append(t)
    seq.length = L0 + len(out)
    return out


@pytest.mark.parametrize("reuse", [False, True], ids=["recompute", "reuse"])
@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_spec_step_matches_oracle(mode, reuse):
    """Two speculative steps (gamma = 3, drafts with one loop, verification with two) for
    three sequences of an fp32 stack, against the oracle model run the same way: draft
    rows, draft tokens, verifying rows, accepted count and emitted tokens, and the cache
    left behind (the next step's rows read it). With reuse the verifying chunk starts at
    loop 2 from the drafts' x and s_1; the oracle recomputes everything."""
    from looped_ngpt_transformer_amd.runtime import DoryRuntime
    from tests.gpu_helpers import gpu_weights, oracle_model
    from tests.helpers import to_np
    from oracle import dory_oracle as O
    S, k, V, n, gamma = synth.config("T"), 2, 4096, 3, 3
    w = gpu_weights(S, 81)
    rt = DoryRuntime(S, w, max_loops=2, max_seqs=n, max_seq_len=96, max_rows=64, mode=mode, loops=k)
    tab = synth.make_vocab(S, V, 82, "cuda", scale=(150.0, 250.0))
    rt.bind_vocab(tab)
    cfg, W = oracle_model(S, w)
    otab = (to_np(tab["embed"]), to_np(tab["lm_head"]), to_np(tab["logit_scale"]))
    seqs = [O.Sequence(cfg) for _ in range(n)]
    for b in range(n):
        X = synth.make_inputs(12 + 7 * b, S["hidden"], 83 + b, device="cuda")
        rt.prefill([b], [X.shape[0]], X)
        O.prefill(cfg, W, seqs[b], to_np(X), k, mode)
    cur = synth.make_ids(n, V, 86, "cuda")
    ocur = [int(t) for t in cur.cpu()]
    alive, emitted = set(range(n)), 0
    for step in range(2):
        ud = synth.make_draws(gamma * n, 87, step, device="cuda").view(gamma, n)
        ua = synth.make_draws(gamma * n, 88, step, device="cuda").view(gamma, n)
        us = synth.make_draws(n, 89, step, device="cuda")
        lens = [D.dory_seq_len(rt.ctx, b) for b in range(n)]
        out, n_out, info = rt.spec_step(list(range(n)), cur, gamma, ud, ua, us, reuse=reuse)
        gpu = {"draft": info["draft"].cpu().double().numpy(), "drafts": info["drafts"].cpu().numpy(),
               "target": info["target"].cpu().double().numpy()}
        udn, uan, usn = ud.cpu().numpy(), ua.cpu().numpy(), us.cpu().numpy()
        for b in range(n):
            assert D.dory_seq_len(rt.ctx, b) == lens[b] + n_out[b]
            if b not in alive:
                continue
            want = oracle_spec(cfg, W, seqs[b], otab, ocur[b], gamma, udn[:, b], uan[:, b], float(usn[b]),
                               k, mode, gpu, b, n)
            if want is None:
                alive.discard(b)
                continue
            assert n_out[b] == len(want) and list(out[b, :n_out[b]]) == want, f"step {step} seq {b}"
            emitted += len(want)
            ocur[b] = want[-1]
        cur = torch.tensor([out[b, n_out[b] - 1] for b in range(n)], dtype=torch.int32, device="cuda")
    assert len(alive) >= 2 and emitted >= 6
    rt.close()


def test_truncated_sequence_regrows_into_its_own_pages():
    """A pool sized exactly for 130 positions: a one-loop draft step past a page boundary
    takes the last free pages; after truncation the verifying step must reuse them
    rather than ask the empty pool for more."""
    from looped_ngpt_transformer_amd.runtime import DoryRuntime
    from tests.gpu_helpers import gpu_weights
    S = synth.config("T")
    cfg = D.make_config(S, max_loops=2, max_seqs=1, max_seq_len=130, max_rows=128)
    pages = D.dory_kv_pages_needed(cfg, D.KV_PER_LOOP, 2, 130, 1)
    rt = DoryRuntime(S, gpu_weights(S, 91), max_loops=2, max_seqs=1, max_seq_len=130, max_rows=128,
                     kv_pages=pages, mode="per_loop", loops=2)
    rt.prefill([0], [128], synth.make_inputs(128, S["hidden"], 92, device="cuda"))
    x = synth.make_inputs(2, S["hidden"], 93, device="cuda")
    D.dory_set_seq_loops(rt.ctx, 0, 1)
    rt.decode([0], x[:1])
    assert D.dory_kv_bytes_in_use(rt.ctx) == pages * rt.page_bytes      # every page taken
    D.dory_set_seq_loops(rt.ctx, 0, 0)
    D.dory_truncate_seq(rt.ctx, 0, 128)
    rt.prefill([0], [2], x)
    torch.cuda.synchronize()
    assert D.dory_seq_len(rt.ctx, 0) == 130
    rt.close()


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_drafts_leave_no_trace_bf16(mode):
    check_against_undrafted_context(mode, reuse=False)


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_reused_activations_bf16(mode):
    """The same with the verifying chunk resumed at loop 2 from the drafts' x and s_1: the
    drafts' first-loop states come from one-row decode GEMMs instead of the chunk's, so
    the verifying logits agree with the undrafted context's to bf16 rounding (cosine of
    every row >= 0.9999) rather than bit for bit."""
    check_against_undrafted_context(mode, reuse=True)


def check_against_undrafted_context(mode, reuse):
    """bf16 stack (chunk attention by quads of rows): the verifying rows of a speculative
    step equal, bit for bit, those of a second context that never drafted and prefills
    the same chunk, and after the step both contexts give identical decode rows; so the
    one-loop drafts, truncated away, leave nothing behind that a later call reads."""
    from looped_ngpt_transformer_amd.runtime import DoryRuntime
    from tests.gpu_helpers import gpu_weights
    S = synth.config("P", n_in=1, n_rec=1, n_out=1, window=64)
    k, V, n, gamma = 2, 4096, 2, 3
    w = gpu_weights(S, 95)
    tab = synth.make_vocab(S, V, 96, "cuda")
    rts = []
    for _ in range(2):
        rt = DoryRuntime(S, w, max_loops=2, max_seqs=n, max_seq_len=160, max_rows=96, mode=mode, loops=k)
        rt.bind_vocab(tab)
        for b in range(n):
            rt.prefill([b], [60 + 13 * b], synth.make_inputs(60 + 13 * b, S["hidden"], 97 + b, device="cuda"))
        rts.append(rt)
    a, ref = rts
    cur = synth.make_ids(n, V, 99, "cuda")
    ud = synth.make_draws(gamma * n, 100, device="cuda").view(gamma, n)
    ua = synth.make_draws(gamma * n, 101, device="cuda").view(gamma, n)
    us = synth.make_draws(n, 102, device="cuda")
    out, n_out, info = a.spec_step(list(range(n)), cur, gamma, ud, ua, us, reuse=reuse)
    chunk = torch.cat([cur.view(n, 1), info["drafts"].t()], dim=1).contiguous().view(-1)
    y = ref.prefill(list(range(n)), [gamma + 1] * n, ref.embed(chunk))
    target = ref.logits(y)
    torch.cuda.synchronize()
    if reuse:
        cos = torch.nn.functional.cosine_similarity(target.double(), info["target"].double(), dim=1)
        assert cos.min().item() >= 0.9999, f"min cosine {cos.min().item():.6f}"
        for rt in rts:
            rt.close()
        return
    assert torch.equal(target, info["target"])
    L = [D.dory_seq_len(a.ctx, b) for b in range(n)]
    for b in range(n):
        D.dory_truncate_seq(ref.ctx, b, L[b])
    nxt = torch.tensor([out[b, n_out[b] - 1] for b in range(n)], dtype=torch.int32, device="cuda")
    ya = a.decode(list(range(n)), a.embed(nxt))
    yr = ref.decode(list(range(n)), ref.embed(nxt))
    torch.cuda.synchronize()
    assert torch.equal(ya, yr)
    for rt in rts:
        rt.close()


def test_capture_and_resume_arguments():
    """The one-shot options check the loop counts of the call that consumes them, and are
    consumed even when it fails."""
    from looped_ngpt_transformer_amd.runtime import DoryRuntime
    from tests.gpu_helpers import gpu_weights
    S = synth.config("T")
    rt = DoryRuntime(S, gpu_weights(S, 103), max_loops=2, max_seqs=1, max_seq_len=64, max_rows=32, loops=2)
    X = synth.make_inputs(4, S["hidden"], 104, device="cuda")
    buf = torch.empty_like(X)
    D.dory_capture_states(rt.ctx, buf, buf)
    with pytest.raises(D.DoryError) as e:                 # k = 2: no capture
        rt.prefill([0], [4], X)
    assert e.value.code == D.ERR_INVALID_ARG
    rt.prefill([0], [4], X)                              # option consumed
    D.dory_set_seq_loops(rt.ctx, 0, 1)
    D.dory_resume_states(rt.ctx, X, X)
    with pytest.raises(D.DoryError) as e:                 # k = 1: no resume
        rt.decode([0], X[:1])
    assert e.value.code == D.ERR_INVALID_ARG
    with pytest.raises(D.DoryError):
        D.dory_capture_states(rt.ctx, None, buf)
    rt.close()


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_captured_states_match_the_oracle(mode):
    """dory_capture_states on a one-loop decode of two sequences (fp32 stack): the captured
    x is the oracle's input-block output and s_1 its first-loop state, row by row."""
    from looped_ngpt_transformer_amd.runtime import DoryRuntime
    from oracle import dory_oracle as O
    from tests.gpu_helpers import gpu_weights, oracle_model
    from tests.helpers import to_np
    S = synth.config("T")
    w = gpu_weights(S, 105)
    rt = DoryRuntime(S, w, max_loops=2, max_seqs=2, max_seq_len=64, max_rows=32, mode=mode, loops=2)
    cfg, W = oracle_model(S, w)
    seqs = [O.Sequence(cfg) for _ in range(2)]
    for b in range(2):
        X = synth.make_inputs(9 + 5 * b, S["hidden"], 106 + b, device="cuda")
        rt.prefill([b], [X.shape[0]], X)
        O.prefill(cfg, W, seqs[b], to_np(X), 2, mode)
        D.dory_set_seq_loops(rt.ctx, b, 1)
    x = synth.make_inputs(2, S["hidden"], 108, device="cuda")
    xc, sc = torch.empty_like(x), torch.empty_like(x)
    D.dory_capture_states(rt.ctx, xc, sc)
    y = rt.decode([0, 1], x)
    torch.cuda.synchronize()
    for b in range(2):
        states = []
        pos = np.array([seqs[b].length])
        want_y = O.forward_chunk(cfg, W, to_np(x[b:b + 1]), pos, 1, mode, seqs[b].kv, states=states)
        want_x = [v for tag, l, v in states if tag == "in"][-1]
        want_s1 = [v for tag, t, v in states if tag == "s" and t == 1][0]
        assert np.abs(xc[b].cpu().double().numpy() - want_x[0]).max() <= 1e-5
        assert np.abs(sc[b].cpu().double().numpy() - want_s1[0]).max() <= 1e-5
        assert np.abs(y[b].cpu().double().numpy() - want_y[0]).max() <= 1e-5
    rt.close()
