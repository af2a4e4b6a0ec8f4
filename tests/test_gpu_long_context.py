"""GPU parity for the long-context prefill: chunks at positions beyond 65536 (the
131072-token chunked prefill reaches 131071), and long chunks at the real window of
1024 keys. Both on the Dory layer shape (hidden 2560, 16/4 heads of 160, SwiGLU 4096)
with a few layers, so that the float64 oracle can follow every row.

* positions: layers 1 / 3 / 1 (layer 3, full attention, is recurrent: in per_loop
  mode each loop has its own 65536-token cache), a 264-row chunk continuing a seeded
  65536-token context (the MFMA prefill attention reads 1029 KV pages per query tile on
  the full layer; RoPE angles at positions 65536..65799 for both bases), then a decode
  step, k = 2, both KV modes;
* window: layers 1 / 2 / 1, window 1024, a 2600-row prefill (rows past 1024 see a
  window cut inside a page; the [q|k|v|gate] projection takes the 256 x 256 tiles, which
  it uses from 2561 rows on) and a decode step, k = 2, both KV modes.
Each at the configurations' rate (0.05) and with the attention rate 1 on the layer
under test.
Tolerance: cosine >= 0.9995 and max|d| <= 2e-2 per row."""
import gc

import pytest
import torch

import synth
from looped_ngpt_transformer_amd.runtime import DoryRuntime
from oracle import dory_oracle as O
from tests.gpu_helpers import compare, gpu_weights, oracle_model, oracle_schedule, run_schedule, seed_context
from tests.helpers import to_np

pytestmark = pytest.mark.gpu


def _rates(w, shape, rates, sharp_layers):
    """rates "config": 0.05 in every channel (the configurations' rate); "sharp": the
    attention rate 1 on the layers under test, so that the state after their attention
    is the direction of its output and an error there reaches the final states at full
    size (rate 1 on every layer instead compounds bf16 rounding over the undamped calls:
    cosine 0.99945 after eight such calls, whatever the context length)."""
    if rates == "sharp":
        for l in sharp_layers:
            w[l]["alpha_attn"].fill_(1.0)
    return w


def _free(rt):
    rt.close()
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rates", ["config", "sharp"])
@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_chunk_at_positions_beyond_65536(mode, rates):
    S = synth.config("L", n_in=1, n_rec=3, n_out=1)
    k, C, T = 2, 65536, 264
    w = _rates(gpu_weights(S, 51), S, rates, [3])  # layer 3: full attention over 65536+ keys
    rt = DoryRuntime(S, w, max_loops=2, max_seqs=1, max_seq_len=C + T + 64, max_rows=T, mode=mode, loops=k)
    stores = seed_context(rt, S, {0: C}, k, mode, seed=53, extra=T + 8)
    cfg, W = oracle_model(S, w)
    X = synth.make_inputs(T, S["hidden"], 54, device="cuda")
    y = rt.prefill([0], [T], X)
    torch.cuda.synchronize()
    ref = O.prefill(cfg, W, stores[0], to_np(X), k, mode)
    compare(y.cpu().double().numpy(), ref, S, f"chunk at {C}")
    x1 = synth.make_inputs(1, S["hidden"], 55, device="cuda")
    y = rt.decode([0], x1)
    torch.cuda.synchronize()
    compare(y.cpu().double().numpy(), O.prefill(cfg, W, stores[0], to_np(x1), k, mode), S, f"decode at {C + T}")
    _free(rt)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("rates", ["config", "sharp"])
@pytest.mark.parametrize("mode", ["per_loop", "last_loop"])
def test_prefill_2600_rows_window_1024(mode, rates):
    S = synth.config("P", n_in=1, n_rec=2, n_out=1)
    assert S["window"] == 1024
    sched = [("prefill", [(0, synth.make_inputs(2600, S["hidden"], 61, device="cuda"))]),
             ("decode", [(0, synth.make_inputs(1, S["hidden"], 62, device="cuda"))])]
    w = _rates(gpu_weights(S, 63), S, rates, [0])  # layer 0: sliding window
    rt = DoryRuntime(S, w, max_loops=2, max_seqs=1, max_seq_len=2688, max_rows=2600, mode=mode, loops=2)
    got = run_schedule(rt, sched)
    cfg, W = oracle_model(S, w)
    want = oracle_schedule(cfg, W, sched, 2, mode)
    for i, (g, r) in enumerate(zip(got, want)):
        compare(g, r, S, f"call {i}")
    _free(rt)
