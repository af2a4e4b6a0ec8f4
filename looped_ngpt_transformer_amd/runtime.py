"""Device-memory plumbing around the C ABI: allocates the KV pool, workspace and MXFP8
weight codes with torch, binds them to a context and keeps them alive. No arithmetic
of the forward pass happens here (MXFP8 codes come from the library's quantiser)."""
from __future__ import annotations

import torch

from . import dory as D


class DoryRuntime:
    def __init__(self, shape: dict, weights: list, *, max_loops=4, max_seqs=1,
                 max_seq_len=4096, max_rows=4096, kv_pages: int | None = None,
                 mode: str = "per_loop", loops: int = 2, device="cuda", arrange: bool = True):
        """arrange: with bf16 weights, also bind fragment-order copies of the four
        matrices (dory_arrange_weights), which the decode projections read with
        contiguous loads; it doubles the weights' device memory."""
        self.shape = shape
        self.arrange = arrange and shape["weight_format"] == "bf16" and shape.get("act_dtype", "bf16") == "bf16"
        self.device = torch.device(device)
        self.cfg = D.make_config(shape, max_loops=max_loops, max_seqs=max_seqs,
                                 max_seq_len=max_seq_len, max_rows=max_rows)
        self.ctx = D.dory_create(self.cfg)
        self.page_bytes, self.ws_bytes = D.dory_query_sizes(self.cfg)
        if kv_pages is None:
            kv_pages = D.dory_kv_pages_needed(self.cfg, D.KV_PER_LOOP, max_loops, max_seq_len, max_seqs)
        self.kv_pages = kv_pages
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.pool = torch.empty(kv_pages * self.page_bytes, dtype=torch.uint8, device=self.device)
        D.dory_bind_workspace(self.ctx, self.ws.data_ptr(), self.ws_bytes)
        D.dory_bind_kv_pool(self.ctx, self.pool.data_ptr(), kv_pages * self.page_bytes)
        self._keep = []
        self.mx = {}  # (layer, matrix name) -> quantised codes and scales (MXFP8, NVFP4)
        self.bind_weights(weights)
        D.dory_set_kv_mode(self.ctx, D.MODES[mode])
        D.dory_set_loops(self.ctx, loops)

    def bind_weights(self, weights: list):
        mx = self.shape["weight_format"] == "mxfp8"
        nv = self.shape["weight_format"] == "nvfp4"
        for l, w in enumerate(weights):
            lw = D.dory_layer_weights()
            for name in ("w_qkvg", "w_o", "w_gu", "w_down"):
                t = w[name]
                assert t.is_contiguous() and t.device.type == "cuda"
                if nv:
                    codes = torch.empty((t.shape[0], t.shape[1] // 2), dtype=torch.uint8, device=t.device)
                    scales = torch.empty((t.shape[0], t.shape[1] // 16), dtype=torch.uint8, device=t.device)
                    g = torch.empty((1,), dtype=torch.float32, device=t.device)
                    D.dory_quantize_nvfp4(t, codes, scales, g)
                    self.mx[(l, name)] = (codes, scales, g)
                    setattr(lw, name, codes.data_ptr())
                    setattr(lw, "s_" + name[2:], scales.data_ptr())
                    setattr(lw, "g_" + name[2:], g.data_ptr())
                elif mx:
                    codes = torch.empty(t.shape, dtype=torch.uint8, device=t.device)
                    scales = torch.empty((t.shape[0], t.shape[1] // 32), dtype=torch.uint8, device=t.device)
                    D.dory_quantize_mxfp8(t, codes, scales)
                    self.mx[(l, name)] = (codes, scales)
                    setattr(lw, name, codes.data_ptr())
                    setattr(lw, "s_" + name[2:], scales.data_ptr())
                else:
                    self._keep.append(t)
                    setattr(lw, name, t.data_ptr())
                    if self.arrange:
                        f = torch.empty_like(t)
                        D.dory_arrange_weights(t, f)
                        self._keep.append(f)
                        setattr(lw, "f_" + name[2:], f.data_ptr())
            for name in ("alpha_attn", "alpha_mlp", "s_qk"):
                t = w[name].to(self.device, torch.float32).contiguous()
                self._keep.append(t)
                setattr(lw, name, t.data_ptr())
            D.dory_bind_weights(self.ctx, l, lw)
        torch.cuda.synchronize(self.device)

    def prefill(self, seq_ids, n_new, x, y=None):
        if y is None:
            y = torch.empty((x.shape[0], self.shape["hidden"]), dtype=torch.float32, device=self.device)
        D.dory_prefill(self.ctx, seq_ids, n_new, x, y)
        return y

    def decode(self, seq_ids, x, y=None):
        if y is None:
            y = torch.empty((x.shape[0], self.shape["hidden"]), dtype=torch.float32, device=self.device)
        D.dory_decode_step(self.ctx, seq_ids, x, y)
        return y

    def bind_vocab(self, tables: dict):
        """Bind embed / lm_head [V, H] (activation type) and logit_scale [V] (float)."""
        t = {k: v.to(self.device).contiguous() for k, v in tables.items()}
        self._keep.extend(t.values())
        self.vocab = int(t["embed"].shape[0])
        D.dory_bind_vocab(self.ctx, t["embed"], t["lm_head"], t["logit_scale"])

    def embed(self, ids, x=None):
        if x is None:
            x = torch.empty((ids.shape[0], self.shape["hidden"]), dtype=torch.float32, device=self.device)
        D.dory_embed(self.ctx, ids, x)
        return x

    def logits(self, states, out=None):
        if out is None:
            out = torch.empty((states.shape[0], self.vocab), dtype=torch.float32, device=self.device)
        D.dory_logits(self.ctx, states, out)
        return out

    def sample(self, logits, u, tokens=None, temperature=1.0, top_p=0.95):
        if tokens is None:
            tokens = torch.empty((logits.shape[0],), dtype=torch.int32, device=self.device)
        D.dory_sample_top_p(logits, u, tokens, temperature=temperature, top_p=top_p)
        return tokens

    def spec_step(self, seq_ids, cur, gamma, u_draft, u_accept, u_sample, temperature=1.0, top_p=0.95,
                  reuse=False):
        """One self-speculative step for live sequences seq_ids whose next input token is
        cur [n] (int32, device): draft gamma tokens with one loop, truncate the drafts
        away, verify cur and the drafts as one chunk at the sequences' own loop counts,
        accept by rejection sampling, and keep the cache entries of the emitted positions.
        u_draft, u_accept [gamma, n], u_sample [n]: uniform draws (device float).
        reuse: the drafts keep their input-block output and first-loop state, one more
        one-loop pass (no output block) gives them for the last draft token, and the
        verifying chunk starts at loop 2 from them (sequences must verify at k >= 2).
        Returns tokens [n, gamma + 1] and n_out [n] on the host, and the device tensors
        used: draft logits [gamma * n, V], draft tokens [gamma, n], verifying logits
        [n * (gamma + 1), V]."""
        n = len(seq_ids)
        ctx = self.ctx
        L0 = [D.dory_seq_len(ctx, s) for s in seq_ids]
        for s in seq_ids:
            D.dory_set_seq_loops(ctx, s, 1)
        V = self.vocab
        draft = torch.empty((gamma * n, V), dtype=torch.float32, device=self.device)
        xt = torch.empty((gamma, n), dtype=torch.int32, device=self.device)
        H = self.shape["hidden"]
        if reuse:
            XC = torch.empty((gamma + 1, n, H), dtype=torch.float32, device=self.device)
            SC = torch.empty_like(XC)
        tok = cur
        try:
            for j in range(gamma):
                if reuse:
                    D.dory_capture_states(ctx, XC[j], SC[j])
                y = self.decode(seq_ids, self.embed(tok))
                lg = self.logits(y, out=draft[j * n:(j + 1) * n])
                tok = self.sample(lg, u_draft[j], xt[j], temperature, top_p)
            if reuse:  # the last draft token through the input block and loop 1 only
                D.dory_capture_states(ctx, XC[gamma], SC[gamma], skip_output_block=True)
                self.decode(seq_ids, self.embed(tok))
        finally:
            for s, l0 in zip(seq_ids, L0):
                D.dory_set_seq_loops(ctx, s, 0)
                D.dory_truncate_seq(ctx, s, l0)
        if reuse:
            X = XC.transpose(0, 1).contiguous().view(n * (gamma + 1), H)
            S1 = SC.transpose(0, 1).contiguous().view(n * (gamma + 1), H)
            D.dory_resume_states(ctx, X, S1)
            y = self.prefill(seq_ids, [gamma + 1] * n, X)
        else:
            chunk = torch.cat([cur.view(n, 1), xt.t()], dim=1).contiguous().view(-1)
            y = self.prefill(seq_ids, [gamma + 1] * n, self.embed(chunk))
        target = self.logits(y)
        out = torch.empty((n, gamma + 1), dtype=torch.int32, device=self.device)
        n_out = torch.empty((n,), dtype=torch.int32, device=self.device)
        D.dory_spec_accept(draft, target, xt, u_accept, u_sample, out, n_out, temperature=temperature, top_p=top_p)
        out_h, n_h = out.cpu().numpy(), n_out.cpu().numpy()
        for s, l0, m in zip(seq_ids, L0, n_h):
            D.dory_truncate_seq(ctx, s, l0 + int(m))
        return out_h, n_h, {"draft": draft, "drafts": xt, "target": target}

    def close(self):
        if self.ctx is not None:
            torch.cuda.synchronize(self.device)
            D.dory_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
