"""dory_logits_noalloc, the LM head with its staging and split-K partials in the
library's static device scratch, against dory_logits (the same kernels on the bound
workspace): bitwise equal on two calls in a row, the second with fewer rows, for the
131072-token vocabulary (one split) and a small one (split-K partials in the scratch);
a request beyond the scratch is refused before any device work."""
import pytest
import torch

import synth
from looped_ngpt_transformer_amd import dory as D
from looped_ngpt_transformer_amd.runtime import DoryRuntime
from tests.gpu_helpers import gpu_weights

pytestmark = pytest.mark.gpu

S = synth.config("P", n_in=1, n_rec=1, n_out=1)


@pytest.mark.parametrize("vocab", [131072, 1024])
def test_logits_noalloc_equals_logits(vocab):
    rt = DoryRuntime(S, gpu_weights(S, 3), max_loops=1, max_seqs=1, max_seq_len=64, max_rows=64, loops=1)
    rt.bind_vocab(synth.make_vocab(S, vocab, 7, "cuda"))
    for n, seed in ((48, 1), (5, 2)):
        states = synth.make_inputs(n, S["hidden"], seed, device="cuda")
        ref = torch.empty((n, vocab), dtype=torch.float32, device="cuda")
        got = torch.full((n, vocab), float("nan"), dtype=torch.float32, device="cuda")
        D.dory_logits(rt.ctx, states, ref)
        D.dory_logits_noalloc(rt.ctx, states, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"{n} rows"
    rt.close()


def test_logits_noalloc_refuses_more_than_its_scratch():
    rt = DoryRuntime(S, gpu_weights(S, 3), max_loops=1, max_seqs=1, max_seq_len=64, max_rows=4096, loops=1)
    rt.bind_vocab(synth.make_vocab(S, 1024, 7, "cuda"))
    states = synth.make_inputs(4096, S["hidden"], 3, device="cuda")  # 4096 x 2560 x 6 bytes > 32 MiB
    out = torch.zeros((1, 1024), dtype=torch.float32, device="cuda")
    with pytest.raises(D.DoryError) as e:
        D.dory_logits_noalloc(rt.ctx, states, out)
    assert e.value.code == D.ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert not out.any()
    rt.close()
