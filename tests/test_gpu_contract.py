"""The boundary's error and stream contracts on the GPU.

* A prefill or decode call that fails after committing (its sequences created and grown,
  pages taken) leaves the context as it was: the test hook dory_test_inject_failure makes
  the call return DORY_ERR_HIP just before a step enqueues anything (the metadata upload,
  or a layer call), so no device work fails. Afterwards the context computes exactly what
  a context that never saw the failure computes (bitwise).
* Calls on one context from different streams are ordered: the results equal those of
  the same calls on one stream.
* Marker ranges (DORY_TRACE=1) leave the results bitwise unchanged."""
import pytest
import torch

import synth
from looped_ngpt_transformer_amd import dory as D
from looped_ngpt_transformer_amd.runtime import DoryRuntime
from tests.gpu_helpers import gpu_weights

pytestmark = pytest.mark.gpu

S = synth.config("P", n_in=1, n_rec=2, n_out=1, window=64)


def xin(n, seed):
    return synth.make_inputs(n, S["hidden"], seed, device="cuda")


def state(rt, ids):
    live = {i: D.dory_seq_len(rt.ctx, i) for i in ids if _is_live(rt, i)}
    return D.dory_live_seqs(rt.ctx), D.dory_kv_bytes_in_use(rt.ctx), live


def _is_live(rt, i):
    try:
        D.dory_seq_len(rt.ctx, i)
        return True
    except D.DoryError:
        return False


@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
@pytest.mark.parametrize("at", [0, 1, 3, 6])  # the upload; the input layer; a recurrent call; the last call
def test_failure_after_commit_leaves_context_unchanged(at, mode):
    w = gpu_weights(S, 5)
    a, b = [DoryRuntime(S, w, max_loops=2, max_seqs=3, max_seq_len=512, max_rows=160, mode=mode, loops=2)
            for _ in range(2)]
    X = torch.cat([xin(100, 1), xin(30, 2)])
    for rt in (a, b):
        rt.prefill([0, 1], [100, 30], X)
    ids = [0, 1, 2]
    # a chunk that crosses a page boundary of sequence 0 and starts sequence 2
    Xc = torch.cat([xin(40, 3), xin(10, 4)])
    before = state(a, ids)
    D.dory_test_inject_failure(a.ctx, at)
    with pytest.raises(D.DoryError) as e:
        a.prefill([0, 2], [40, 10], Xc)
    assert e.value.code == D.ERR_HIP
    torch.cuda.synchronize()
    assert state(a, ids) == before
    ya, yb = a.prefill([0, 2], [40, 10], Xc), b.prefill([0, 2], [40, 10], Xc)
    torch.cuda.synchronize()
    assert torch.equal(ya, yb)
    # a failing decode step
    before = state(a, ids)
    D.dory_test_inject_failure(a.ctx, at)
    Xd = xin(3, 5)
    with pytest.raises(D.DoryError):
        a.decode(ids, Xd)
    torch.cuda.synchronize()
    assert state(a, ids) == before
    for step in range(2):
        Xd = xin(3, 6 + step)
        ya, yb = a.decode(ids, Xd), b.decode(ids, Xd)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), f"decode {step}"
    a.close()
    b.close()


def test_calls_on_different_streams_are_ordered():
    w = gpu_weights(S, 6)
    a, b = [DoryRuntime(S, w, max_loops=2, max_seqs=2, max_seq_len=512, max_rows=256, loops=2) for _ in range(2)]
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    X = xin(200, 11)
    torch.cuda.synchronize()
    outs = {}
    for name, rt, streams in (("two", a, (s1, s2)), ("one", b, (s1, s1))):
        ys = []
        with torch.cuda.stream(streams[0]):
            ys.append(rt.prefill([0], [200], X))
        for step in range(3):  # no host synchronisation between the calls
            with torch.cuda.stream(streams[(step + 1) % 2]):
                ys.append(rt.decode([0], xin(1, 20 + step)))
        torch.cuda.synchronize()
        outs[name] = ys
    for i, (p, q) in enumerate(zip(outs["two"], outs["one"])):
        assert torch.equal(p, q), f"call {i}"
    a.close()
    b.close()


def test_misaligned_states_are_refused_before_any_work():
    """x_in and y_out must be 16-byte aligned: a call with either off by one float fails
    with DORY_ERR_INVALID_ARG and leaves the context as it was."""
    w = gpu_weights(S, 5)
    rt = DoryRuntime(S, w, max_loops=2, max_seqs=2, max_seq_len=256, max_rows=64, mode="per_loop", loops=2)
    rt.prefill([0], [20], xin(20, 1))
    torch.cuda.synchronize()
    before = state(rt, [0, 1])
    H = S["hidden"]
    xbuf = torch.empty(8 * H + 1, dtype=torch.float32, device="cuda")
    ybuf = torch.empty(8 * H + 1, dtype=torch.float32, device="cuda")
    x_ok, x_off = xbuf[:8 * H].view(8, H), xbuf[1:].view(8, H)
    x_ok.copy_(xin(8, 2))
    x_off.copy_(xin(8, 2))
    y_ok, y_off = ybuf[:8 * H].view(8, H), ybuf[1:].view(8, H)
    for x, y in ((x_off, y_ok), (x_ok, y_off)):
        with pytest.raises(D.DoryError) as e:
            rt.prefill([1], [8], x, y)
        assert e.value.code == D.ERR_INVALID_ARG
        with pytest.raises(D.DoryError) as e:
            rt.decode([0], x[:1], y[:1])
        assert e.value.code == D.ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert state(rt, [0, 1]) == before
    rt.close()


def test_trace_ranges_leave_results_unchanged(monkeypatch):
    """With DORY_TRACE=1 every prefill and decode call pushes and pops marker ranges
    through the platform's marker library; the results are bitwise those of untraced
    calls. The library is loaded the way the runtime loads it."""
    import ctypes
    ctypes.CDLL("librocprofiler-sdk-roctx.so.1")  # the marker library the runtime opens
    w = gpu_weights(S, 5)
    X, xd = xin(300, 6), xin(2, 7)
    out = []
    for traced in (False, True):
        if traced:
            monkeypatch.setenv("DORY_TRACE", "1")
        rt = DoryRuntime(S, w, max_loops=2, max_seqs=2, max_seq_len=512, max_rows=300, mode="per_loop", loops=2)
        y0 = rt.prefill([0, 1], [200, 100], X)
        y1 = rt.decode([0, 1], xd)
        torch.cuda.synchronize()
        out.append((y0.clone(), y1.clone()))
        rt.close()
    monkeypatch.delenv("DORY_TRACE")
    assert torch.equal(out[0][0], out[1][0]) and torch.equal(out[0][1], out[1][1])
