"""GPU parity at the 72-layer decode shape: 16/40/16 layers of the Dory layer shape
(hidden 2560, 16/4 heads of 160, SwiGLU 4096, window 1024, 3:1 sliding/full), bf16
weights drawn per layer, a decode batch of 32 sequences over seeded contexts of 8200
tokens (more than 2048 keys, so the full layers go by the two-register-set split-key
kernel), at k = 1, 2 and 4 in both KV modes. Every row of the batch runs on the GPU;
the oracle (float64) recomputes rows 0 and 31 of two consecutive steps from the same
seeded cache entries. Tolerance: cosine >= 0.9995 and max|d| <= 2e-2 per row."""
import gc

import pytest
import torch

import synth
from looped_ngpt_transformer_amd import dory as D
from looped_ngpt_transformer_amd.runtime import DoryRuntime
from oracle import dory_oracle as O
from tests.gpu_helpers import compare, gpu_weights, oracle_model, seed_context
from tests.helpers import to_np

pytestmark = pytest.mark.gpu

SHAPE = synth.config("D")
BATCH = 32
CTX = 8200
ROWS = (0, BATCH - 1)
STEPS = 2


@pytest.fixture(scope="module")
def model():
    w = gpu_weights(SHAPE, 21)
    cfg, W = oracle_model(SHAPE, w)
    yield w, cfg, W
    del w, W
    gc.collect()
    torch.cuda.empty_cache()


def kv_pages(mode, k, max_seq_len, max_rows):
    c = D.make_config(SHAPE, max_loops=4, max_seqs=BATCH, max_seq_len=max_seq_len, max_rows=max_rows)
    return D.dory_kv_pages_needed(c, D.MODES[mode], k, max_seq_len, BATCH)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("k,mode", [(1, "per_loop"), (2, "per_loop"), (2, "last_loop"), (4, "per_loop"),
                                    (4, "last_loop")])
def test_decode_batch_32_over_8200_tokens(model, k, mode):
    w, cfg, W = model
    msl = CTX + 64
    rt = DoryRuntime(SHAPE, w, max_loops=4, max_seqs=BATCH, max_seq_len=msl, max_rows=BATCH,
                     kv_pages=kv_pages(mode, k, msl, BATCH), mode=mode, loops=k)
    stores = seed_context(rt, SHAPE, {s: CTX for s in range(BATCH)}, k, mode, keep=ROWS, seed=31)
    ids = list(range(BATCH))
    for step in range(STEPS):
        X = synth.make_inputs(BATCH, SHAPE["hidden"], 400 + step, device="cuda")
        y = rt.decode(ids, X)
        torch.cuda.synchronize()
        assert D.dory_last_layer_calls(rt.ctx) == 32 + 40 * k
        got = y.cpu().double().numpy()
        for r in ROWS:
            ref = O.prefill(cfg, W, stores[r], to_np(X[r:r + 1]), k, mode)
            compare(got[r:r + 1], ref, SHAPE, f"k={k} {mode} step {step} row {r}")
    rt.close()
    del rt
    gc.collect()
    torch.cuda.empty_cache()
