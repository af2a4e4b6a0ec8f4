"""Helpers for the GPU parity tests: run a schedule of prefill / decode calls through
the C ABI and through the oracle on the same seeded inputs, and compare."""
import math

import numpy as np
import torch

import synth
from oracle import dory_oracle as O
from oracle import mxfp8 as MX
from oracle import nvfp4 as NV
from oracle import vocab as OV
from tests.helpers import oracle_weights, to_np

BF16_COS = 0.9995
BF16_MAXABS = 2e-2
F32_MAXABS = 1e-4


def gpu_weights(shape, seed, alpha="const"):
    return synth.make_weights(shape, seed, "cuda", alpha=alpha)


_NV_CACHE = {}


def _nvfp4_dequantised(w):
    """The oracle's NVFP4 round trip of a weight matrix, cached by content (the exhaustive
    float32 scale search is slow in NumPy and the tests reuse their seeded weights)."""
    import hashlib
    key = (w.shape, hashlib.sha1(np.ascontiguousarray(w).tobytes()).hexdigest())
    if key not in _NV_CACHE:
        _NV_CACHE[key] = NV.dequantize(*NV.quantize(w))
    return _NV_CACHE[key]


_MX_CACHE = {}


def _mxfp8_dequantised(w):
    """The oracle's MXFP8 round trip of a weight matrix, cached by content (several
    parity cases reuse the same seeded weights)."""
    import hashlib
    key = (w.shape, hashlib.sha1(np.ascontiguousarray(w).tobytes()).hexdigest())
    if key not in _MX_CACHE:
        _MX_CACHE[key] = MX.dequantize(*MX.quantize(w))
    return _MX_CACHE[key]


def oracle_model(shape, w_gpu, rt=None):
    """Oracle weights: the same bf16/fp32 values, or dequantised MXFP8 / NVFP4 codes
    produced by the oracle's own quantisers from the same bf16 values."""
    cfg = O.Config.from_dict(shape)
    cpu = [{k: v.detach().cpu() for k, v in w.items()} for w in w_gpu]
    if shape["weight_format"] == "mxfp8":
        for w in cpu:
            for name in ("w_qkvg", "w_o", "w_gu", "w_down"):
                w[name] = torch.from_numpy(_mxfp8_dequantised(to_np(w[name])))
    if shape["weight_format"] == "nvfp4":
        for w in cpu:
            for name in ("w_qkvg", "w_o", "w_gu", "w_down"):
                w[name] = torch.from_numpy(_nvfp4_dequantised(to_np(w[name])))
    return cfg, oracle_weights(shape, cpu)


def compare(y_gpu, y_ref, shape, what=""):
    g = np.asarray(y_gpu, dtype=np.float64)
    r = np.asarray(y_ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    maxabs = np.abs(g - r).max()
    if shape["act_dtype"] == "f32":
        assert maxabs <= F32_MAXABS, f"{what}: max|d| {maxabs:.3e} > {F32_MAXABS}"
        return maxabs, 1.0
    cos = np.sum(g * r, axis=1) / (np.linalg.norm(g, axis=1) * np.linalg.norm(r, axis=1))
    assert cos.min() >= BF16_COS, f"{what}: min cosine {cos.min():.6f} < {BF16_COS}"
    assert maxabs <= BF16_MAXABS, f"{what}: max|d| {maxabs:.3e} > {BF16_MAXABS}"
    return maxabs, float(cos.min())


def run_schedule(rt, schedule):
    """schedule: list of (kind, [(seq_id, X float32 cuda [n, H])]). Returns the list of
    outputs (numpy) per call."""
    outs = []
    for kind, items in schedule:
        ids = [i for i, _ in items]
        X = torch.cat([x for _, x in items]).contiguous()
        if kind == "prefill":
            y = rt.prefill(ids, [x.shape[0] for _, x in items], X)
        else:
            y = rt.decode(ids, X)
        torch.cuda.synchronize()
        outs.append(y.cpu().double().numpy())
    return outs


def oracle_schedule(cfg, W, schedule, k, mode, seqs=None):
    seqs = {} if seqs is None else seqs
    outs = []
    for kind, items in schedule:
        ys = []
        for sid, x in items:
            if sid not in seqs:
                seqs[sid] = O.Sequence(cfg)
            ys.append(O.prefill(cfg, W, seqs[sid], to_np(x), k, mode))
        outs.append(np.concatenate(ys))
    return outs


# float32 sums of the sampler against the oracle's float64: the width of the band around
# every boundary of u (and of the top_p cut) inside which either side is accepted
TOL_U = 5e-5


def check_valid(lg_np, u_np, toks, temperature, top_p):
    """Every token valid; returns how many rows were far enough from every boundary to
    demand the oracle's exact token (those must match)."""
    exact = 0
    for i in range(lg_np.shape[0]):
        t = int(toks[i])
        assert 0 <= t < lg_np.shape[1], f"row {i}: token {t}"
        order, _, cum = OV.sorted_order(lg_np[i], temperature)
        n = OV.nucleus_size(cum, top_p)
        rank = int(np.nonzero(order == t)[0][0])
        u = float(u_np[i])
        # nucleus sizes a float32 sum may also find: cuts whose running mass is within
        # TOL_U of top_p
        sizes = [m for m in range(max(1, n - 1), min(cum.size, n + 1) + 1)
                 if m == n or abs(cum[m - 1] - top_p) <= TOL_U or (m == n + 1 and abs(cum[n - 1] - top_p) <= TOL_U)]
        ok, clear = False, True
        for m in sizes:
            if rank >= m:
                clear = False
                continue
            lo = (cum[rank - 1] if rank else 0.0) / cum[m - 1]
            hi = cum[rank] / cum[m - 1]
            ok |= lo - TOL_U <= u <= hi + TOL_U
            clear &= lo + TOL_U < u < hi - TOL_U
        assert ok, f"row {i}: token {t} (rank {rank}, nucleus {n}) does not match u {u}"
        if clear:
            assert t == OV.sample_top_p(lg_np[i], temperature, top_p, u), f"row {i}: token {t}"
            exact += 1
    return exact


def seed_context(rt, shape, seqs, k, mode, keep=None, seed=9, swa_tail=None, extra=64):
    """Install a seeded context without computing it: reserve seqs[sid] positions for each
    sequence and write seeded K/V (synth.make_kv, drawn on the device by torch) into every
    cache slot the sequence holds; sliding layers get only their last `swa_tail` positions
    (default window + 64). Returns oracle sequences holding the same entries (float64) for
    the ids in `keep` (default all), with room for `extra` more positions."""
    cfg = O.Config.from_dict(shape)
    L = shape["n_in"] + shape["n_rec"] + shape["n_out"]
    keep = set(seqs) if keep is None else set(keep)
    tail = shape["window"] + 64 if swa_tail is None else swa_tail
    from looped_ngpt_transformer_amd import dory as D
    stores = {}
    for sid, C in seqs.items():
        D.dory_test_reserve(rt.ctx, sid, C)
        seq = None
        if sid in keep:
            seq = O.Sequence(cfg)
            seq.length = C
        for l in range(L):
            rec = shape["n_in"] <= l < shape["n_in"] + shape["n_rec"]
            slots = k if (rec and mode == "per_loop") else 1
            p0 = 0 if O.layer_is_full(cfg, l) else max(0, C - tail)
            for s in range(slots):
                kk, vv = synth.make_kv(shape, seed, sid, l, s, p0, C - p0, device="cuda")
                D.dory_test_fill_kv(rt.ctx, sid, l, s, p0, kk, vv)
                if seq is not None:
                    seq.kv._ensure((l, s), C + extra)   # room for the positions the test appends
                    seq.kv.write(l, s, np.arange(p0, C), to_np(kk), to_np(vv))
        if seq is not None:
            stores[sid] = seq
    torch.cuda.synchronize()
    return stores
