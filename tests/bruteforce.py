"""Pure-Python brute-force looped nGPT for tiny shapes (a pin for the oracle).

Written from the method's definition with explicit loops over scalars (no NumPy
vectorisation, no shared helpers with the oracle): every matrix product, rotation,
softmax and normalisation is spelled out element by element. It keeps its own KV
store: a dict keyed by (layer, slot, position). Only for shapes of a few dozen
channels.
"""
import math


def _norm(v):
    n = math.sqrt(sum(a * a for a in v))
    n = max(n, 1e-12)
    return [a / n for a in v]


def _matvec(W, v):
    # W: list of rows [out][in]
    return [sum(W[o][i] * v[i] for i in range(len(v))) for o in range(len(W))]


def _rot(vec, p, theta):
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for i in range(h):
        ang = p * theta ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = vec[i] * c - vec[i + h] * s
        out[i + h] = vec[i] * s + vec[i + h] * c
    return out


class BruteModel:
    def __init__(self, cfg, weights):
        """cfg: dict of shapes; weights: list per layer of dicts with python lists
        wq, wk, wv, wg (or None), wo, wgate, wup, wdown, aa, am, sqk."""
        self.c = cfg
        self.w = weights
        self.kv = {}

    def _attn(self, l, slot, s_rows, positions):
        c = self.c
        Hq, Hkv, d = c["n_q_heads"], c["n_kv_heads"], c["head_dim"]
        w = self.w[l]
        full = (l % c["full_period"]) == c["full_period"] - 1
        theta = c["theta_full"] if full else c["theta_swa"]
        qs = []
        # project, rotate, normalise and store every row of the chunk first
        for s, p in zip(s_rows, positions):
            q = _matvec(w["wq"], s)
            k = _matvec(w["wk"], s)
            v = _matvec(w["wv"], s)
            qh = []
            for h in range(Hq):
                vec = _rot(q[h * d:(h + 1) * d], p, theta)
                if c["qk_norm"]:
                    vec = [w["sqk"][i] * a for i, a in enumerate(_norm(vec))]
                qh.append(vec)
            for h in range(Hkv):
                vec = _rot(k[h * d:(h + 1) * d], p, theta)
                if c["qk_norm"]:
                    vec = [w["sqk"][i] * a for i, a in enumerate(_norm(vec))]
                self.kv[(l, slot, p, h)] = (vec, v[h * d:(h + 1) * d])
            qs.append(qh)
        outs = []
        for s, p, qh in zip(s_rows, positions, qs):
            cat = []
            for h in range(Hq):
                hk = h // (Hq // Hkv)
                keys = [j for j in range(p + 1) if full or p - j < c["window"]]
                logits = []
                for j in keys:
                    kk, _ = self.kv[(l, slot, j, hk)]
                    logits.append(c["attn_scale"] * sum(a * b for a, b in zip(qh[h], kk)))
                m = max(logits)
                e = [math.exp(x - m) for x in logits]
                z = sum(e)
                o = [0.0] * d
                for wgt, j in zip(e, keys):
                    _, vv = self.kv[(l, slot, j, hk)]
                    for i in range(d):
                        o[i] += wgt / z * vv[i]
                cat.extend(o)
            if c["attn_gate"]:
                g = _matvec(w["wg"], s)
                cat = [a / (1.0 + math.exp(-b)) for a, b in zip(cat, g)]
            cat = _norm(cat)
            outs.append(_matvec(w["wo"], cat))
        return outs

    def _mlp(self, l, s):
        w = self.w[l]
        g = _matvec(w["wgate"], s)
        u = _matvec(w["wup"], s)
        h = [a / (1.0 + math.exp(-a)) * b for a, b in zip(g, u)]
        h = _norm(h)
        return _matvec(w["wdown"], h)

    def _update(self, s, y, alpha):
        yn = _norm(y)
        return _norm([(1 - a) * si + a * yi for si, yi, a in zip(s, yn, alpha)])

    def _layer(self, l, slot, rows, positions):
        att = self._attn(l, slot, rows, positions)
        rows = [self._update(s, y, self.w[l]["aa"]) for s, y in zip(rows, att)]
        rows = [self._update(s, self._mlp(l, s), self.w[l]["am"]) for s in rows]
        return rows

    def chunk(self, rows, positions, k, mode):
        c = self.c
        for l in range(c["n_in"]):
            rows = self._layer(l, 0, rows, positions)
        x = rows
        s = x
        for t in range(1, k + 1):
            u = [_norm([a + b for a, b in zip(si, xi)]) for si, xi in zip(s, x)]
            slot = t - 1 if mode == "per_loop" else 0
            r = u
            for l in range(c["n_in"], c["n_in"] + c["n_rec"]):
                r = self._layer(l, slot, r, positions)
            s = [_norm(ri) for ri in r]
        for l in range(c["n_in"] + c["n_rec"], c["n_in"] + c["n_rec"] + c["n_out"]):
            s = self._layer(l, 0, s, positions)
        return s


def weights_to_lists(cfg, packed):
    """Split packed numpy/torch weights of each layer into python lists."""
    import numpy as np
    out = []
    qd = cfg["n_q_heads"] * cfg["head_dim"]
    kd = cfg["n_kv_heads"] * cfg["head_dim"]
    I = cfg["intermediate"]
    for w in packed:
        f = lambda a: np.asarray(a, dtype=np.float64).tolist()
        qkvg = np.asarray(w["w_qkvg"], dtype=np.float64)
        gu = np.asarray(w["w_gu"], dtype=np.float64)
        out.append(dict(
            wq=qkvg[:qd].tolist(), wk=qkvg[qd:qd + kd].tolist(),
            wv=qkvg[qd + kd:qd + 2 * kd].tolist(),
            wg=qkvg[qd + 2 * kd:].tolist() if cfg["attn_gate"] else None,
            wo=f(w["w_o"]), wgate=gu[:I].tolist(), wup=gu[I:].tolist(),
            wdown=f(w["w_down"]), aa=f(w["alpha_attn"]), am=f(w["alpha_mlp"]),
            sqk=f(w["s_qk"])))
    return out
