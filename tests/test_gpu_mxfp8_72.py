"""GPU parity at the MXFP8 decode shape: 16/40/16 layers of the Dory layer shape with
MXFP8 weights (E4M3 codes, one E8M0 scale per 32 along K, from the library's own
quantiser on the device), bf16 activations, a decode batch of 128 sequences over
seeded 8192-token contexts at k = 4 in last_loop mode. The oracle quantises the same
bf16 values with its own quantiser and recomputes rows 0 and 127 of two steps.

The 72 layers take their matrices from five seeded weight sets (layer l uses set
l % 5, so every set serves sliding and full layers of every block): the oracle's
NumPy quantiser handles about five million weights a second, and 72 distinct layers
would take it over ten minutes. Rates, cache entries and every layer's KV streams are
still per layer; the 72-layer bf16 case draws every layer's weights."""
import gc

import numpy as np
import pytest
import torch

import synth
from looped_ngpt_transformer_amd import dory as D
from looped_ngpt_transformer_amd.runtime import DoryRuntime
from oracle import dory_oracle as O
from tests.gpu_helpers import compare, seed_context
from tests.helpers import oracle_weights, to_np
from tests.mx_pool import dequantised_many

pytestmark = pytest.mark.gpu

SHAPE = synth.config("Q")
BATCH = 128
CTX = 8192
ROWS = (0, BATCH - 1)
SETS = 5
K = 4
MODE = "last_loop"


@pytest.mark.timeout(900)
def test_mxfp8_decode_batch_128_over_8192_tokens_k4_last_loop():
    L = synth.n_layers(SHAPE)
    sets = [synth.make_layer_weights(SHAPE, j, 41, "cuda", alpha="uniform") for j in range(SETS)]
    w = [dict(sets[l % SETS]) for l in range(L)]
    for l in range(L):  # per-layer rates so that a layer mix-up cannot hide
        g = torch.Generator(device="cuda").manual_seed(1000 + l)
        for name in ("alpha_attn", "alpha_mlp"):
            w[l][name] = 0.01 + 0.09 * torch.rand((SHAPE["hidden"],), generator=g, device="cuda")
    # the oracle's own quantisation of the same bf16 values
    names = ("w_qkvg", "w_o", "w_gu", "w_down")
    mats = [sets[j][n].float().cpu().numpy() for j in range(SETS) for n in names]
    deq = dequantised_many(mats)
    cpu_sets = []
    for j in range(SETS):
        cpu_sets.append({n: torch.from_numpy(deq[j * len(names) + i]) for i, n in enumerate(names)})
    packed = []
    for l in range(L):
        d = dict(cpu_sets[l % SETS])
        for name in ("alpha_attn", "alpha_mlp", "s_qk"):
            d[name] = w[l][name].cpu()
        packed.append(d)
    cfg = O.Config.from_dict(SHAPE)
    W = oracle_weights(SHAPE, packed)
    del mats, deq, cpu_sets, packed

    msl = CTX + 64
    c = D.make_config(SHAPE, max_loops=K, max_seqs=BATCH, max_seq_len=msl, max_rows=BATCH)
    pages = D.dory_kv_pages_needed(c, D.MODES[MODE], K, msl, BATCH)
    rt = DoryRuntime(SHAPE, w, max_loops=K, max_seqs=BATCH, max_seq_len=msl, max_rows=BATCH, kv_pages=pages,
                     mode=MODE, loops=K)
    stores = seed_context(rt, SHAPE, {s: CTX for s in range(BATCH)}, K, MODE, keep=ROWS, seed=43)
    ids = list(range(BATCH))
    for step in range(2):
        X = synth.make_inputs(BATCH, SHAPE["hidden"], 500 + step, device="cuda")
        y = rt.decode(ids, X)
        torch.cuda.synchronize()
        assert D.dory_last_layer_calls(rt.ctx) == 32 + 40 * K
        got = y.cpu().double().numpy()
        assert np.all(np.isfinite(got))
        for r in ROWS:
            ref = O.prefill(cfg, W, stores[r], to_np(X[r:r + 1]), K, MODE)
            compare(got[r:r + 1], ref, SHAPE, f"step {step} row {r}")
    rt.close()
    del rt, w, sets
    gc.collect()
    torch.cuda.empty_cache()
