"""Seeded synthetic inputs for the looped nGPT forward pass.

This module is shared by the oracle tests, the GPU parity tests and the benchmark.
It defines the model shapes and produces seeded weights, unit-norm input states and
prefilled KV entries. It holds none of the forward pass's arithmetic: the only
operations here are drawing random numbers, scaling them to the stated
distribution, rounding weights to bf16 (round-to-nearest-even, torch's cast) and
normalising input rows so that they lie on the unit sphere, which is what the
method's inputs are.

Shapes follow the model described on the pages "Dory1.0-4B: A Looped Normalized-GPT"
(config.json fields quoted in the MXFP8 article: hidden 2560, 16 query / 4 KV heads,
sliding window 1024, RoPE bases 1e4 / 1e7; the 16/40/16 block split from the paper
summary's method section and the 8/20/8 split from the model-card digest).
"""
from __future__ import annotations

import math

import torch

# --------------------------------------------------------------------------- shapes
# act/weight formats: "f32", "bf16", "mxfp8", "nvfp4" (the last two for weights only)

_DORY = dict(hidden=2560, n_q_heads=16, n_kv_heads=4, head_dim=160, intermediate=4096,
             window=1024, full_period=4, theta_swa=1e4, theta_full=1e7,
             attn_scale=math.sqrt(160.0), qk_norm=1, attn_gate=1,
             act_dtype="bf16", weight_format="bf16")

CONFIGS = {
    # tiny looped nGPT: fp32 parity configuration
    "T": dict(hidden=256, n_q_heads=4, n_kv_heads=1, head_dim=64, intermediate=1024,
              n_in=2, n_rec=4, n_out=2, window=16, full_period=4, theta_swa=1e4,
              theta_full=1e7, attn_scale=8.0, qk_norm=1, attn_gate=1,
              act_dtype="f32", weight_format="f32"),
    # Dory shape read as 8/20/8 blocks (36 layers), bf16
    "P": dict(_DORY, n_in=8, n_rec=20, n_out=8),
    # Dory shape read as 16/40/16 blocks (72 layers), bf16
    "D": dict(_DORY, n_in=16, n_rec=40, n_out=16),
    "L": dict(_DORY, n_in=16, n_rec=40, n_out=16),
    # 72-layer shape with MXFP8 weights (E4M3 + E8M0 per 32 along K), bf16 activations
    "Q": dict(_DORY, n_in=16, n_rec=40, n_out=16, weight_format="mxfp8"),
    # 72-layer shape with NVFP4 weights (E2M1 + E4M3 per 16 along K + matrix scale)
    "N": dict(_DORY, n_in=16, n_rec=40, n_out=16, weight_format="nvfp4"),
}

WORKLOADS = {
    "T": dict(batch=1, prefill=64, decode_steps=16, loops=(1, 2)),
    "P": dict(batch=1, prefill=4096, loops=(2,)),
    "D": dict(batch=32, context=32768, decode_steps=256, loops=(1, 2, 4)),
    "L": dict(batch=1, prefill=131072, chunk=8192, loops=(2,)),
    "Q": dict(batch=128, context=8192, loops=(4,), kv_mode="last_loop"),
    "N": dict(batch=128, context=8192, loops=(4,), kv_mode="last_loop"),
}

WEIGHT_STD = 0.02
ALPHA = 0.05


def config(name: str, **over) -> dict:
    c = dict(CONFIGS[name])
    c.update(over)
    return c


def n_layers(cfg: dict) -> int:
    return cfg["n_in"] + cfg["n_rec"] + cfg["n_out"]


def qkvg_rows(cfg: dict) -> int:
    qd = cfg["n_q_heads"] * cfg["head_dim"]
    kd = cfg["n_kv_heads"] * cfg["head_dim"]
    return qd + 2 * kd + (qd if cfg["attn_gate"] else 0)


def weight_shapes(cfg: dict) -> dict:
    H, I = cfg["hidden"], cfg["intermediate"]
    qd = cfg["n_q_heads"] * cfg["head_dim"]
    return {
        "w_qkvg": (qkvg_rows(cfg), H),
        "w_o": (H, qd),
        "w_gu": (2 * I, H),      # gate rows, then up rows
        "w_down": (H, I),
    }


def _seed(*parts: int) -> int:
    # fold integers into one 63-bit seed (FNV-1a over the decimal digits)
    h = 0xCBF29CE484222325
    for p in parts:
        for ch in str(int(p)).encode() + b"|":
            h ^= ch
            h = (h * 0x100000001B3) & 0xFFFFFFFFFFFFFFFF
    return h & 0x7FFFFFFFFFFFFFFF


_NAME_ID = {"w_qkvg": 1, "w_o": 2, "w_gu": 3, "w_down": 4, "alpha_attn": 5,
            "alpha_mlp": 6, "s_qk": 7, "x": 8, "k": 9, "v": 10, "embed": 11, "lm_head": 12,
            "logit_scale": 13, "ids": 14, "u": 15, "spec_base": 16, "spec_target": 17,
            "spec_draft": 18}

VOCAB = 131072  # the tokenizer's vocabulary (MXFP8 article, checkpoint notes)


def _gen(device, *parts):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def make_layer_weights(cfg: dict, layer: int, seed: int, device="cpu",
                       alpha: str = "const") -> dict:
    """Weights of one physical layer.

    Matrices are i.i.d. N(0, 0.02^2), drawn in fp32 and stored in the config's
    storage type: fp32 for the fp32 configuration, bf16 (RNE) otherwise. For the
    MXFP8 configuration the bf16 values are returned; quantisation is a step of the
    method and happens on each side. alpha="const" gives 0.05 in every channel;
    alpha="uniform" draws U(0.01, 0.1) per channel. s_qk is 1 (its effective value).
    """
    store = torch.float32 if cfg["weight_format"] == "f32" else torch.bfloat16
    out = {}
    for name, shape in weight_shapes(cfg).items():
        g = _gen(device, seed, layer, _NAME_ID[name])
        w = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * WEIGHT_STD
        out[name] = w.to(store).contiguous()
    H = cfg["hidden"]
    for name in ("alpha_attn", "alpha_mlp"):
        if alpha == "const":
            out[name] = torch.full((H,), ALPHA, device=device, dtype=torch.float32)
        else:
            g = _gen(device, seed, layer, _NAME_ID[name])
            out[name] = (0.01 + 0.09 * torch.rand((H,), generator=g, device=device,
                                                   dtype=torch.float32)).contiguous()
    out["s_qk"] = torch.ones((cfg["head_dim"],), device=device, dtype=torch.float32)
    return out


def make_weights(cfg: dict, seed: int, device="cpu", alpha: str = "const") -> list:
    return [make_layer_weights(cfg, l, seed, device, alpha) for l in range(n_layers(cfg))]


def make_inputs(n: int, hidden: int, seed: int, stream: int = 0, device="cpu") -> torch.Tensor:
    """n seeded unit-norm rows (Gaussian direction), fp32 [n, hidden]."""
    g = _gen(device, seed, stream, _NAME_ID["x"])
    x = torch.randn((n, hidden), generator=g, device=device, dtype=torch.float64)
    x = x / x.norm(dim=1, keepdim=True)
    return x.to(torch.float32).contiguous()


def make_kv(cfg: dict, seed: int, seq: int, layer: int, slot: int, pos0: int, n: int,
            device="cpu") -> tuple:
    """Seeded KV entries for positions [pos0, pos0+n) of one (sequence, layer, slot).

    K rows per head are Gaussian directions (unit norm, as QK-normalised keys with
    s_qk = 1 are); V ~ N(0, 0.02^2), the spread of s W_v^T for unit s. Returned in
    the KV storage type ([n, Hkv, d] each).
    """
    Hkv, d = cfg["n_kv_heads"], cfg["head_dim"]
    store = torch.float32 if cfg["act_dtype"] == "f32" else torch.bfloat16
    gk = _gen(device, seed, seq, layer, slot, pos0, _NAME_ID["k"])
    k = torch.randn((n, Hkv, d), generator=gk, device=device, dtype=torch.float32)
    k = k / k.norm(dim=2, keepdim=True)
    gv = _gen(device, seed, seq, layer, slot, pos0, _NAME_ID["v"])
    v = torch.randn((n, Hkv, d), generator=gv, device=device, dtype=torch.float32) * WEIGHT_STD
    return k.to(store).contiguous(), v.to(store).contiguous()


def make_vocab(cfg: dict, vocab: int, seed: int, device="cpu", scale=(15.0, 25.0)) -> dict:
    """Seeded vocabulary tables: input and output embeddings [vocab, H] whose rows are
    Gaussian directions (unit norm, the sphere nGPT keeps embeddings on) stored in the
    activation type, and a per-token logit scale drawn from U(scale) (the effective
    scale; with unit-norm states and rows, logits span about +-scale / sqrt(H) * 3)."""
    H = cfg["hidden"]
    store = torch.float32 if cfg["act_dtype"] == "f32" else torch.bfloat16
    out = {}
    for name in ("embed", "lm_head"):
        g = _gen(device, seed, vocab, _NAME_ID[name])
        e = torch.randn((vocab, H), generator=g, device=device, dtype=torch.float32)
        out[name] = (e / e.norm(dim=1, keepdim=True)).to(store).contiguous()
    g = _gen(device, seed, vocab, _NAME_ID["logit_scale"])
    lo, hi = scale
    out["logit_scale"] = (lo + (hi - lo) * torch.rand((vocab,), generator=g, device=device,
                                                       dtype=torch.float32)).contiguous()
    return out


def make_ids(n: int, vocab: int, seed: int, device="cpu") -> torch.Tensor:
    """n seeded token ids, uniform over [0, vocab), int32."""
    g = _gen(device, seed, vocab, _NAME_ID["ids"])
    return torch.randint(0, vocab, (n,), generator=g, device=device, dtype=torch.int32)


def make_draws(n: int, seed: int, stream: int = 0, device="cpu") -> torch.Tensor:
    """n seeded uniform draws in [0, 1), float32 (the sampler's random numbers)."""
    g = _gen(device, seed, stream, _NAME_ID["u"])
    return torch.rand((n,), generator=g, device=device, dtype=torch.float32)


def make_spec_logits(n: int, gamma: int, vocab: int, seed: int, spread: float = 3.0, noise: float = 0.5,
                     device="cpu"):
    """Logit rows for a speculative step of n sequences: a shared base row per position
    (Gaussian, std `spread`) plus independent Gaussian noise (std `noise`) for the
    verifying model's gamma + 1 rows and the draft's gamma rows, so the two distributions
    overlap without being equal. Returns (draft [gamma * n, V] position-major, target
    [n * (gamma + 1), V] sequence-major)."""
    g = _gen("cpu", seed, n, gamma, vocab, _NAME_ID["spec_base"])
    base = torch.randn((n, gamma + 1, vocab), generator=g, dtype=torch.float32) * spread
    g = _gen("cpu", seed, n, gamma, vocab, _NAME_ID["spec_target"])
    target = base + torch.randn(base.shape, generator=g, dtype=torch.float32) * noise
    g = _gen("cpu", seed, n, gamma, vocab, _NAME_ID["spec_draft"])
    draft = base[:, :gamma] + torch.randn((n, gamma, vocab), generator=g, dtype=torch.float32) * noise
    return (draft.transpose(0, 1).reshape(gamma * n, vocab).contiguous().to(device),
            target.reshape(n * (gamma + 1), vocab).contiguous().to(device))
