"""Plain float64 CPU oracle for the looped normalized-GPT forward pass.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU
baseline leg may import this module. It shares no code with the HIP library and
imports neither it nor torch: inputs are NumPy arrays, arithmetic is float64.

What it computes, with the passages it follows ("Dory1.0-4B: A Looped
Normalized-GPT"; page names below are those of the five web pages):

* N(v) = v / ||v||_2 row-wise, the unit-sphere projection of nGPT
  (paper summary, "prerequisites: nGPT").
* every sublayer update  s <- N((1 - a) * s + a * N(sublayer(s)))  with a per-channel
  rate a (paper summary, nGPT prerequisite; arXiv summary section 2: the sublayer
  output is normalised before it is blended, and the blend is normalised again).
* attention sublayer: GQA with 16 query / 4 KV heads, RoPE with base 1e4 on
  sliding-window layers and 1e7 on full layers, window 1024, 3 sliding layers then
  one full layer, an input-dependent sigmoid gate on the attention output, an extra
  L2 norm of the gated, concatenated heads before the output projection
  (paper summary, "technical novelty"; arXiv summary section 2; config.json fields
  in the MXFP8 article).
* MLP sublayer: SwiGLU with an extra L2 norm of the activation before the down
  projection (same passages).
* looped stack: input block once -> x; s0 = x; u_t = N(s_{t-1} + x);
  s_t = N(F(u_t)) for t = 1..k with the recurrent weights shared across loops;
  output block once (paper summary, "core method" equation; arXiv summary 3.2).
* KV modes: per_loop keeps one cache slot per loop for each recurrent attention
  layer; last_loop keeps one slot, overwritten every loop, so earlier-loop queries
  see the final-loop entries of prior tokens (arXiv summary 6.1; model-card digest,
  "memory-friendly KV cache").

Arrays keep the type of the inputs: the oracle is float64 (its callers pass float64);
the benchmark also times it once on float32 inputs.

Readings where the pages are silent are listed in the design notes and restated at
each function. No tiling, fusion or reordering: every query's visible keys are marked
explicitly (causal, and the window on sliding layers) and softmax runs over them alone.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

EPS = 1e-12  # N(0) reading: v / max(||v||, 1e-12)


# ----------------------------------------------------------------------------- config
@dataclass
class Config:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    intermediate: int
    n_in: int
    n_rec: int
    n_out: int
    window: int
    full_period: int = 4
    theta_swa: float = 1e4
    theta_full: float = 1e7
    attn_scale: float = 1.0
    qk_norm: int = 1
    attn_gate: int = 1
    # the extra norms before W_o and W_down: True = over the whole row (the reading
    # taken), False = none, "per_head" = the attention output normalised per head (an
    # alternative reading of the same passage; the MLP activation has no heads and keeps
    # the row norm)
    pre_proj_norm: bool | str = True

    @staticmethod
    def from_dict(d: dict) -> "Config":
        names = Config.__dataclass_fields__.keys()
        return Config(**{k: v for k, v in d.items() if k in names})

    @property
    def n_layers(self) -> int:
        return self.n_in + self.n_rec + self.n_out


def layer_is_full(cfg: Config, layer: int) -> bool:
    """3:1 interleave: physical layer i is full attention iff i % 4 == 3.

    The pages give the pattern as three sliding-window groups followed by one full
    group (MXFP8 article, hybrid attention section); the phase is read from the
    first layer of the stack.
    """
    return layer % cfg.full_period == cfg.full_period - 1


def effective_depth(cfg: Config, k: int) -> int:
    """Layers executed per token: L_in + L_out + k * L_rec (paper summary: 32 + 40k)."""
    return cfg.n_in + cfg.n_out + k * cfg.n_rec


def attn_slots(cfg: Config, k: int, mode: str) -> int:
    """Cache slots per token: one per input/output attention layer, and k (per_loop)
    or 1 (last_loop) per recurrent attention layer."""
    rec = k if mode == "per_loop" else 1
    return cfg.n_in + cfg.n_out + rec * cfg.n_rec


# -------------------------------------------------------------------------- primitives
def l2n(v: np.ndarray) -> np.ndarray:
    """N(v): project each row (last axis) onto the unit sphere."""
    n = np.sqrt(np.sum(v * v, axis=-1, keepdims=True))
    return v / np.maximum(n, EPS)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def silu(z):
    """SiLU(z) = z * sigmoid(z), the SwiGLU gate nonlinearity."""
    return z / (1.0 + np.exp(-z))


def softmax(z: np.ndarray) -> np.ndarray:
    """Softmax over the last axis (max-subtracted for range)."""
    m = np.max(z, axis=-1, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def ngpt_update(s: np.ndarray, h: np.ndarray, alpha: np.ndarray) -> np.ndarray:
    """s <- N((1 - alpha) * s + alpha * N(h)); h is the raw sublayer output."""
    return l2n((1.0 - alpha) * s + alpha * l2n(h))


def rope(x: np.ndarray, pos: np.ndarray, theta: float) -> np.ndarray:
    """Rotary embedding on the last axis of x [T, heads, d] at positions pos [T].

    Reading (the pages give only the bases): dimension pairs (i, i + d/2), frequency
    theta^(-2i/d), angle = pos * frequency, all d dimensions rotated, 0-based
    absolute positions, the same position in every loop.
    """
    d = x.shape[-1]
    half = d // 2
    freq = theta ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = pos.astype(np.float64)[:, None] * freq[None, :]          # [T, half]
    c = np.cos(ang).astype(x.dtype)[:, None, :]
    s = np.sin(ang).astype(x.dtype)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x1 * s + x2 * c], axis=-1)


# ----------------------------------------------------------------------------- weights
@dataclass
class LayerWeights:
    """One physical layer, float64. W matrices are [out, in]; y = s @ W.T."""
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wg: np.ndarray | None
    wo: np.ndarray
    wgate: np.ndarray
    wup: np.ndarray
    wdown: np.ndarray
    alpha_attn: np.ndarray
    alpha_mlp: np.ndarray
    s_qk: np.ndarray

    @staticmethod
    def from_packed(cfg: Config, w_qkvg, w_o, w_gu, w_down, alpha_attn, alpha_mlp, s_qk):
        """Split the packed storage: w_qkvg rows are [q | k | v | gate], w_gu rows are
        [gate | up]."""
        f = lambda a: np.asarray(a, dtype=np.float64)
        w_qkvg = f(w_qkvg)
        qd = cfg.n_q_heads * cfg.head_dim
        kd = cfg.n_kv_heads * cfg.head_dim
        wq = w_qkvg[:qd]
        wk = w_qkvg[qd:qd + kd]
        wv = w_qkvg[qd + kd:qd + 2 * kd]
        wg = w_qkvg[qd + 2 * kd:] if cfg.attn_gate else None
        w_gu = f(w_gu)
        I = cfg.intermediate
        return LayerWeights(wq, wk, wv, wg, f(w_o), w_gu[:I], w_gu[I:], f(w_down),
                            f(alpha_attn), f(alpha_mlp), f(s_qk))


# ---------------------------------------------------------------------------- KV store
class KVStore:
    """Per-(layer, slot) key/value entries by absolute position, float64.

    Writes for a chunk's positions happen before that layer's attention reads them.
    A read of a position never written raises, so a wrong visible set cannot pass
    silently.
    """

    def __init__(self, cfg: Config):
        self.cfg = cfg
        self.k: dict = {}
        self.v: dict = {}
        self.valid: dict = {}

    def _ensure(self, key, hi, dtype=np.float64):
        if key not in self.k:
            cap = max(64, hi)
            shp = (cap, self.cfg.n_kv_heads, self.cfg.head_dim)
            self.k[key] = np.zeros(shp, dtype=dtype)
            self.v[key] = np.zeros(shp, dtype=dtype)
            self.valid[key] = np.zeros(cap, dtype=bool)
        cap = self.k[key].shape[0]
        if hi > cap:
            new = max(hi, 2 * cap)
            for d in (self.k, self.v):
                a = np.zeros((new,) + d[key].shape[1:], dtype=d[key].dtype)
                a[:cap] = d[key]
                d[key] = a
            vv = np.zeros(new, dtype=bool)
            vv[:cap] = self.valid[key]
            self.valid[key] = vv

    def write(self, layer: int, slot: int, pos: np.ndarray, k: np.ndarray, v: np.ndarray):
        key = (layer, slot)
        self._ensure(key, int(pos.max()) + 1, k.dtype)
        self.k[key][pos] = k
        self.v[key][pos] = v
        self.valid[key][pos] = True

    def read(self, layer: int, slot: int, lo: int, hi: int):
        """Entries for positions lo..hi inclusive."""
        key = (layer, slot)
        if key not in self.k or hi >= self.k[key].shape[0] or not self.valid[key][lo:hi + 1].all():
            raise KeyError(f"KV read of unwritten entries: layer {layer} slot {slot} [{lo},{hi}]")
        return self.k[key][lo:hi + 1], self.v[key][lo:hi + 1]

    def slots_used(self) -> int:
        return len(self.k)


# --------------------------------------------------------------------------- sublayers
def attention(cfg: Config, lw: LayerWeights, s: np.ndarray, pos: np.ndarray, layer: int,
              kv: KVStore, slot: int) -> np.ndarray:
    """Attention sublayer on rows s [T, H] at positions pos [T] (one sequence).

    Returns the raw projection y = N(o) W_o^T (the caller's nGPT update normalises it).
    Readings: per-head QK normalisation after RoPE times s_qk and logit scale
    attn_scale (sqrt(d) in the nGPT form); the gate is elementwise over the
    concatenated head channels, computed from the sublayer input; window W counts
    the query itself (visible iff 0 <= p - j < W).
    """
    T = s.shape[0]
    Hq, Hkv, d = cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    q = (s @ lw.wq.T).reshape(T, Hq, d)
    k = (s @ lw.wk.T).reshape(T, Hkv, d)
    v = (s @ lw.wv.T).reshape(T, Hkv, d)
    full = layer_is_full(cfg, layer)
    theta = cfg.theta_full if full else cfg.theta_swa
    q = rope(q, pos, theta)
    k = rope(k, pos, theta)
    if cfg.qk_norm:
        q = lw.s_qk * l2n(q)
        k = lw.s_qk * l2n(k)
    kv.write(layer, slot, pos, k, v)

    # Keys any row of the chunk may see: [lo, hi]. Row t sees key j iff j <= p_t and,
    # on sliding layers, p_t - j < W; the other logits of its row are -inf, so softmax
    # gives them weight exactly 0 and runs over the visible set alone.
    p = pos.astype(np.int64)
    lo = 0 if full else max(0, int(p.min()) - cfg.window + 1)
    hi = int(p.max())
    K, V = kv.read(layer, slot, lo, hi)
    j = np.arange(lo, hi + 1)
    visible = j[None, :] <= p[:, None]
    if not full:
        visible &= p[:, None] - j[None, :] < cfg.window
    out = np.zeros((T, Hq, d), dtype=q.dtype)
    for h in range(Hq):
        hk = (h * Hkv) // Hq                          # GQA: query head -> KV head
        logits = cfg.attn_scale * (q[:, h, :] @ K[:, hk, :].T)   # [T, keys]
        a = softmax(np.where(visible, logits, -np.inf))
        out[:, h] = a @ V[:, hk, :]
    o = out.reshape(T, Hq * d)
    if cfg.attn_gate:
        o = sigmoid(s @ lw.wg.T) * o
    if cfg.pre_proj_norm == "per_head":
        o = l2n(o.reshape(T, Hq, d)).reshape(T, Hq * d)
    elif cfg.pre_proj_norm:
        o = l2n(o)
    return o @ lw.wo.T


def mlp(cfg: Config, lw: LayerWeights, s: np.ndarray) -> np.ndarray:
    """SwiGLU sublayer: h = SiLU(s Wg^T) * (s Wu^T); h <- N(h); y = h Wd^T (raw)."""
    h = silu(s @ lw.wgate.T) * (s @ lw.wup.T)
    if cfg.pre_proj_norm:
        h = l2n(h)
    return h @ lw.wdown.T


@dataclass
class Counter:
    layer_calls: int = 0
    trace: list = field(default_factory=list)


def layer(cfg: Config, lw: LayerWeights, s, pos, idx, kv, slot, counter: Counter | None = None):
    """One layer = attention sublayer then MLP sublayer, each with its nGPT update."""
    if counter is not None:
        counter.layer_calls += 1
        counter.trace.append((idx, slot))
    s = ngpt_update(s, attention(cfg, lw, s, pos, idx, kv, slot), lw.alpha_attn)
    s = ngpt_update(s, mlp(cfg, lw, s), lw.alpha_mlp)
    return s


# ------------------------------------------------------------------------ looped stack
def forward_chunk(cfg: Config, weights: list, X: np.ndarray, pos: np.ndarray, k: int,
                  mode: str, kv: KVStore, counter: Counter | None = None,
                  states: list | None = None) -> np.ndarray:
    """Forward one chunk of a single sequence (rows X [T, H] at positions pos).

    Input block once -> x; s = x; for t = 1..k: u = N(s + x), s = N(RecBlock(u)) with
    KV slot t-1 (per_loop) or 0 (last_loop); output block once. Decode is a chunk of
    one row. `states`, when given, collects every intermediate state for the
    unit-norm checks.
    """
    assert mode in ("per_loop", "last_loop") and k >= 1
    s = np.asarray(X)
    s = s.astype(np.result_type(s.dtype, np.float32))  # float64 in, float64 out
    pos = np.asarray(pos)
    rec0 = cfg.n_in
    out0 = cfg.n_in + cfg.n_rec
    for l in range(cfg.n_in):
        s = layer(cfg, weights[l], s, pos, l, kv, 0, counter)
        if states is not None:
            states.append(("in", l, s))
    x = s
    s = x
    for t in range(1, k + 1):
        u = l2n(s + x)
        if states is not None:
            states.append(("u", t, u))
        slot = t - 1 if mode == "per_loop" else 0
        r = u
        for l in range(rec0, out0):
            r = layer(cfg, weights[l], r, pos, l, kv, slot, counter)
            if states is not None:
                states.append(("rec", (t, l), r))
        s = l2n(r)
        if states is not None:
            states.append(("s", t, s))
    for l in range(out0, cfg.n_layers):
        s = layer(cfg, weights[l], s, pos, l, kv, 0, counter)
        if states is not None:
            states.append(("out", l, s))
    return s


def forward_plain(cfg: Config, weights: list, X: np.ndarray, pos: np.ndarray,
                  kv: KVStore) -> np.ndarray:
    """A plain, non-looped stack: every physical layer once, slot 0, no boundary ops."""
    s = np.asarray(X)
    s = s.astype(np.result_type(s.dtype, np.float32))  # float64 in, float64 out
    for l in range(cfg.n_layers):
        s = layer(cfg, weights[l], s, np.asarray(pos), l, kv, 0)
    return s


class Sequence:
    """A sequence being served: its KV store and current length."""

    def __init__(self, cfg: Config):
        self.kv = KVStore(cfg)
        self.length = 0


def prefill(cfg, weights, seq: Sequence, X, k, mode, counter=None):
    """Append X's rows as positions length..length+T-1 (a chunk)."""
    T = X.shape[0]
    pos = np.arange(seq.length, seq.length + T)
    y = forward_chunk(cfg, weights, X, pos, k, mode, seq.kv, counter)
    seq.length += T
    return y


def decode_step(cfg, weights, seq: Sequence, x_row, k, mode, counter=None):
    """One decode step: a chunk of one row at the next position."""
    return prefill(cfg, weights, seq, np.asarray(x_row).reshape(1, -1), k, mode, counter)
