"""Shared test helpers: small configurations and conversions to oracle inputs."""
import math

import numpy as np

import synth
from oracle import dory_oracle as O

# 5 layers: 0,1,2 sliding, 3 full (inside the recurrent block), 4 sliding
TINY = dict(hidden=16, n_q_heads=2, n_kv_heads=1, head_dim=8, intermediate=24,
            n_in=1, n_rec=3, n_out=1, window=3, full_period=4, theta_swa=1e4,
            theta_full=1e7, attn_scale=math.sqrt(8.0), qk_norm=1, attn_gate=1,
            act_dtype="f32", weight_format="f32")

# GQA group of 2, two KV heads
SMALL = dict(hidden=32, n_q_heads=4, n_kv_heads=2, head_dim=8, intermediate=48,
             n_in=2, n_rec=2, n_out=1, window=5, full_period=4, theta_swa=1e4,
             theta_full=1e7, attn_scale=math.sqrt(8.0), qk_norm=1, attn_gate=1,
             act_dtype="f32", weight_format="f32")


def to_np(t):
    return t.detach().cpu().double().numpy()


def oracle_weights(cfg_dict, packed):
    cfg = O.Config.from_dict(cfg_dict)
    return [O.LayerWeights.from_packed(cfg, to_np(w["w_qkvg"]), to_np(w["w_o"]),
                                       to_np(w["w_gu"]), to_np(w["w_down"]),
                                       to_np(w["alpha_attn"]), to_np(w["alpha_mlp"]),
                                       to_np(w["s_qk"])) for w in packed]


def model(cfg_dict, seed=1, alpha="uniform"):
    packed = synth.make_weights(cfg_dict, seed, "cpu", alpha=alpha)
    return O.Config.from_dict(cfg_dict), oracle_weights(cfg_dict, packed), packed


def inputs(cfg_dict, n, seed=2, stream=0):
    return to_np(synth.make_inputs(n, cfg_dict["hidden"], seed, stream))


def rownorms(a):
    return np.sqrt(np.sum(np.asarray(a) ** 2, axis=-1))
