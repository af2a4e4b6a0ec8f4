"""Throughput of the looped nGPT forward pass on one MI355X.

Default workload (the one the metric is quoted on that fits one GPU): the Dory shape
read as 8/20/8 blocks (36 layers, hidden 2560, 16/4 heads of 160, SwiGLU 4096, window
1024, 3:1 sliding/full), bf16, batch 1, one 4096-token prefill at k = 2 (56 executed
layers). One step = one whole prefill of a fresh sequence through the C ABI. Weights
and inputs are seeded synthetic data resident in HBM before timing starts.

Also: --workload D runs decode steps of the 72-layer shape (batch 32 over a seeded
32768-token KV context) and --workload Q the MXFP8 decode (batch 128, 8192 context,
k = 4, last_loop) and --workload N the same with NVFP4 weights; --ks 1,2,4 measures
several loop counts. --workload G is D with
the vocabulary side in the loop: each step's final states go through the LM head
(131072 tokens), top-p sampling (T 1.0, p 0.95, seeded draws) and the embedding of the
sampled tokens, which is the next step's input.

Prints one JSON line. The roofline object covers the dominant kernel class (the
projection GEMMs for prefill, the split-key attention kernel for decode) from HIP events around each launch
over the timed region; cpu_baseline times the float64 oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E

WORKLOAD_TEXT = {
    "P": "Dory-shape 8/20/8 (36 layers) bf16, batch 1, 4096-token prefill",
    "D": "Full 16/40/16 (72 layers) bf16, decode batch 32 over a seeded 32768-token KV context",
    "Q": "16/40/16 (72 layers) MXFP8 W8A16, decode batch 128 over a seeded 8192-token KV context",
    "N": "16/40/16 (72 layers) NVFP4 W4A16, decode batch 128 over a seeded 8192-token KV context",
    "L": "16/40/16 (72 layers) bf16, batch 1, chunked prefill (chunks of 8192)",
    "T": "tiny looped nGPT fp32, prefill 64",
    "G": "Full 16/40/16 (72 layers) bf16, generation batch 32 over a seeded 32768-token KV context: "
         "decode step, LM head over 131072 tokens, top-p sampling, embedding of the sampled tokens",
    "S": "Full 16/40/16 (72 layers) bf16, self-speculative generation over a seeded per_loop KV context: "
         "gamma tokens drafted with one loop, verified as one chunk with k loops, rejection sampling",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="P", choices=["P", "D", "Q", "N", "L", "T", "G", "S"])
    ap.add_argument("--gamma", type=int, default=4, help="speculative draft length (S)")
    ap.add_argument("--no-reuse", dest="reuse", action="store_false",
                    help="S: recompute the drafted positions' input block and loop 1 in the verifying "
                         "chunk instead of starting at loop 2 from the drafts' activations")
    ap.add_argument("--k", type=int, default=None)
    ap.add_argument("--ks", default=None, help="comma list of loop counts to measure too")
    ap.add_argument("--mode", default=None, choices=["per_loop", "last_loop"])
    ap.add_argument("--mix-k", default=None,
                    help="decode: comma list of loop counts given to the batch's sequences in turn "
                         "(one call mixes them)")
    ap.add_argument("--tokens", type=int, default=None, help="prefill length (P, L)")
    ap.add_argument("--weights", default=None, choices=["bf16", "mxfp8", "nvfp4"],
                    help="prefill (P, L): weight format (default bf16)")
    ap.add_argument("--context", type=int, default=None, help="seeded KV context (D, Q)")
    ap.add_argument("--batch", type=int, default=None, help="decode batch (D, Q)")
    ap.add_argument("--cpu-rows", type=int, default=1024)
    ap.add_argument("--no-decode-leg", action="store_true", help="P: skip the 72-layer decode leg")
    ap.add_argument("--decode-steps", type=int, default=8, help="decode leg: timed steps per k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-context", action="store_true",
                    help="P: skip the sustained-MFMA and platform-BLAS measurements")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run out = src * 1 over 1 GiB first (counter calibration for rocprofv3 --pmc)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest(*names):
    """Digest of kernel sources: measured traffic applies only to the code it came from."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "looped_ngpt_transformer_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key, workload, sources):
    """HBM bytes per launch from the committed counter summary (FETCH_SIZE + WRITE_SIZE,
    scaled by the copy-probe calibration), or None when absent, taken on another
    workload or taken on other code."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)[key]
    except (OSError, KeyError, ValueError):
        return None
    if t.get("bench_workload") != workload or t.get("source_digest") != source_digest(*sources):
        return None
    return t.get("bytes_per_launch")


def kernel_stats(rt, D):
    return {D.KC_NAMES[k]: D.dory_profile_read(rt.ctx, k) for k in D.KC_NAMES}


def roofline_of(stats, kind, workload):
    if kind == "mfma":
        g = stats["gemm"]
        ach = g["flops"] / (g["ms"] / 1e3) / 1e12
        return {"bound": "mfma",
                "kernel": "gemm (bf16 MFMA projections; a launch here is one projection call, the "
                          "[q|k|v|gate] call being two kernels over its column tiles)",
                "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic("prefill_gemm", workload, ["k_gemm.hip", "common.h", "kernels.h"]),
                "launches": g["launches"], "avg_launch_us": round(1e3 * g["ms"] / g["launches"], 2)}
    a = stats["attention"]
    ach = a["bytes"] / (a["ms"] / 1e3) / 1e9
    return {"bound": "hbm", "kernel": "k_attn_decode (split-key decode attention over the paged KV cache)",
            "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("decode_attention", workload, ["k_attn.hip", "common.h", "kernels.h"]),
            "launches": a["launches"], "avg_launch_us": round(1e3 * a["ms"] / a["launches"], 2)}


def lm_head_line(stats, steps):
    """The LM head (logits GEMM over the vocabulary + logit scale + embedding lookup),
    HBM-bound: algorithmic bytes (the [V, H] bf16 table once per step, states, logits)
    over its summed HIP-event time."""
    v = stats["vocab"]
    ach = v["bytes"] / (v["ms"] / 1e3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "launches": v["launches"],
            "ms_per_step": round(v["ms"] / steps, 3)}


def time_prefill(rt, D, torch, X, tokens, steps, warmup, chunk=None):
    """Each step: prefill a fresh sequence (in chunks if given), then release it. The
    timed steps carry no events (wall clock around `steps` steps); the same number of
    steps is then run again with HIP events around the GEMM launches only (the roofline
    of the dominant kernel class), and one more step records every kernel class for the
    per-class breakdown."""
    chunk = chunk or tokens
    Y = torch.empty((chunk, X.shape[1]), dtype=torch.float32, device="cuda")

    def one():
        for c0 in range(0, tokens, chunk):
            n = min(chunk, tokens - c0)
            D.dory_prefill(rt.ctx, [0], [n], X[c0:c0 + n], Y[:n])
        D.dory_release_seq(rt.ctx, 0)

    for _ in range(warmup):
        one()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    D.dory_profile_enable(rt.ctx, [D.KC_GEMM])
    for _ in range(steps):
        one()
    torch.cuda.synchronize()
    D.dory_profile_enable(rt.ctx, False)
    timed = kernel_stats(rt, D)
    D.dory_profile_enable(rt.ctx, True)
    one()
    torch.cuda.synchronize()
    D.dory_profile_enable(rt.ctx, False)
    return (t1 - t0) / steps, timed, kernel_stats(rt, D), Y


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline_prefill(shape, weights, X, k, mode, rows, y_gpu):
    """The float64 oracle on the first `rows` tokens of the prefill (a causal prefix,
    so its outputs are exactly the first rows of the full prefill), with its BLAS
    threads set to the cores this process may run on; then the same prefix with the
    weights and input rows in float32 (a timing variant: NumPy then multiplies in
    float32; the oracle's result is the float64 one)."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import dory_oracle as O
    cores = len(os.sched_getaffinity(0))
    cfg = O.Config.from_dict(shape)
    names = ("w_qkvg", "w_o", "w_gu", "w_down", "alpha_attn", "alpha_mlp", "s_qk")
    W = [O.LayerWeights.from_packed(cfg, *(w[n].cpu().double().numpy() for n in names)) for w in weights]
    Xs = X[:rows].cpu().double().numpy()
    with threadpool_limits(limits=cores):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        t0 = time.perf_counter()
        ref = O.prefill(cfg, W, O.Sequence(cfg), Xs, k, mode)
        dt = time.perf_counter() - t0
        W32 = [O.LayerWeights(*(None if a is None else a.astype(np.float32) for a in
                                (lw.wq, lw.wk, lw.wv, lw.wg, lw.wo, lw.wgate, lw.wup, lw.wdown,
                                 lw.alpha_attn, lw.alpha_mlp, lw.s_qk))) for lw in W]
        t0 = time.perf_counter()
        O.prefill(cfg, W32, O.Sequence(cfg), Xs.astype(np.float32), k, mode)
        dt32 = time.perf_counter() - t0
    g = y_gpu[:rows].cpu().double().numpy()
    cos = np.sum(g * ref, 1) / (np.linalg.norm(g, axis=1) * np.linalg.norm(ref, axis=1))
    return ({"value": round(rows / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
             "sample": f"first {rows} of the 4096 tokens of the prefill (a causal prefix: its attention "
                       f"covers at most {rows} keys, so the rate is higher than the whole prefill's), all "
                       f"{O.effective_depth(cfg, k)} layer calls, float64, {dt:.1f} s",
             "cpu": cpu_model(), "affinity_cores": cores,
             "float32_value": round(rows / dt32, 3), "float32_s": round(dt32, 1)},
            {"rows": rows, "max_abs": float(np.abs(g - ref).max()), "min_cos": float(cos.min())})


def bench_prefill(args, torch, synth, D, DoryRuntime):
    wl = args.workload
    shape = synth.config(wl, **({"weight_format": args.weights} if args.weights else {}))
    k = args.k or 2
    mode = args.mode or "per_loop"
    tokens = args.tokens or (4096 if wl == "P" else 131072 if wl == "L" else 64)
    chunk = 8192 if wl == "L" else None
    default_ks = {1, 2, 4} if wl == "P" else set()
    ks = sorted({k} | ({int(x) for x in args.ks.split(",")} if args.ks else default_ks))
    log(f"[bench] workload {wl}: generating weights")
    weights = synth.make_weights(shape, 1234, "cuda")
    max_rows = min(tokens, chunk or tokens)
    rt = DoryRuntime(shape, weights, max_loops=max(ks + [2]), max_seqs=1, max_seq_len=tokens,
                     max_rows=max_rows, mode=mode, loops=k)
    X = synth.make_inputs(tokens, shape["hidden"], 99, device="cuda")
    results = {}
    for kk in ks:
        D.dory_set_loops(rt.ctx, kk)
        log(f"[bench] k={kk}: warmup {args.warmup}, steps {args.steps}")
        dt, stats, brk, Y = time_prefill(rt, D, torch, X, tokens, args.steps, args.warmup, chunk)
        results[kk] = (dt, stats, Y, brk)
        log(f"[bench] k={kk}: {dt * 1e3:.2f} ms/step, {tokens / dt:.0f} tok/s, "
            f"gemm {stats['gemm']['flops'] / stats['gemm']['ms'] / 1e9:.0f} TFLOP/s")
    dt, stats, Y, brk = results[k]
    out = {
        "metric": "prefill tokens/s (k=%d)" % k, "value": round(tokens / dt, 1),
        "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if shape["act_dtype"] == "bf16" else "f32",
        "data": "synthetic (seeded random weights N(0,0.02) and unit-norm input states)",
        "config": {"workload": WORKLOAD_TEXT[wl] + ("" if shape["weight_format"] == "bf16" else
                                                     ", %s weights" % shape["weight_format"].upper()),
                   "tokens": tokens, "loops": k, "kv_mode": mode,
                   "executed_layers": shape["n_in"] + shape["n_out"] + k * shape["n_rec"],
                   "chunk": chunk or tokens},
        "roofline": roofline_of(stats, "mfma", wl),
        "kernels": {n: {"launches": s["launches"], "ms": round(s["ms"], 3)} for n, s in brk.items()},
    }
    if len(ks) > 1:
        out["by_loops"] = {str(kk): {"tokens_per_s": round(tokens / r[0], 1),
                                     "ms_per_step": round(r[0] * 1e3, 3),
                                     "gemm_tflops": round(r[1]["gemm"]["flops"] / r[1]["gemm"]["ms"] / 1e9, 1),
                                     "gemm_frac": round(r[1]["gemm"]["flops"] / r[1]["gemm"]["ms"] / 1e9
                                                        / PEAK_BF16_TFLOPS, 4)}
                           for kk, r in results.items()}
    rt.close()
    del rt
    torch.cuda.empty_cache()
    if wl == "P" and not args.no_gemm_context:
        out["gemm_context"] = gemm_context(torch, D, shape, tokens)
    if wl == "P" and not args.no_decode_leg:
        out["decode_leg"] = decode_leg(args, torch, synth, D, DoryRuntime)
    if not args.no_cpu_baseline and wl in ("P", "T"):
        log(f"[bench] cpu baseline: oracle on the first {args.cpu_rows} tokens")
        cb, par = cpu_baseline_prefill(shape, weights, X, k, mode, min(args.cpu_rows, tokens), Y)
        out["cpu_baseline"] = cb
        out["parity_prefix"] = par
    return out


def gemm_context(torch, D, shape, M):
    """What bounds the projection GEMMs on this device, measured beside them (context for
    the roofline, not the headline):
      * mfma_sustained: the rate of the bf16 matrix instruction itself, every compute unit
        running independent chains on register operands (dory_test_mfma_rate). Under
        dense matrix work the chip holds a lower clock than the one its 2.5 PFLOP/s is
        quoted at; this is the practical ceiling;
      * the four projection shapes at this prefill's M, each timed alone (50 back-to-back
        launches, HIP events): through dory_test_gemm (this library's tiles), and through
        torch.mm (the platform's BLAS library, hipBLASLt) on the same bf16 operands."""
    log("[bench] gemm context: sustained MFMA rate, projection shapes vs the platform BLAS")
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    cyc = torch.zeros(n_cu, dtype=torch.int64, device="cuda")
    sink = torch.zeros(n_cu * 512, dtype=torch.float32, device="cuda")
    iters = 20000
    D.dory_test_mfma_rate(1000, cyc, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    n_wg = D.dory_test_mfma_rate(iters, cyc, sink)
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3
    mf_tflops = n_wg * 8 * 8 * iters * 32768.0 / t / 1e12
    clock = float(cyc.double().mean()) / t / 1e9
    H, I = shape["hidden"], shape["intermediate"]
    qd, kd = shape["n_q_heads"] * shape["head_dim"], shape["n_kv_heads"] * shape["head_dim"]
    nqkvg = qd + 2 * kd + (qd if shape["attn_gate"] else 0)
    shapes = [("qkvg", nqkvg, H, D.EPI_STORE_BF16), ("o", H, qd, D.EPI_STORE_BF16),
              ("gate_up", 2 * I, H, D.EPI_SWIGLU), ("down", H, I, D.EPI_STORE_BF16)]
    g = torch.Generator(device="cuda").manual_seed(7)

    def timed(fn, reps=50):
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    per, ours_us, blas_us, flops = {}, 0.0, 0.0, 0.0
    for name, N, K, epi in shapes:
        A = (torch.randn((M, K), generator=g, device="cuda") * 0.1).to(torch.bfloat16)
        B = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        C = torch.empty((M, N // 2 if epi == D.EPI_SWIGLU else N), dtype=torch.bfloat16, device="cuda")
        Cb = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        Bt = B.t()
        u_o = timed(lambda: D.dory_test_gemm(A, B, epi, out=C))
        u_b = timed(lambda: torch.mm(A, Bt, out=Cb))
        f = 2.0 * M * N * K
        per[name] = {"M": M, "N": N, "K": K, "us": round(u_o, 1), "blas_us": round(u_b, 1),
                     "frac": round(f / u_o / 1e6 / PEAK_BF16_TFLOPS, 4),
                     "blas_frac": round(f / u_b / 1e6 / PEAK_BF16_TFLOPS, 4)}
        ours_us, blas_us, flops = ours_us + u_o, blas_us + u_b, flops + f
        del A, B, C, Cb
    torch.cuda.empty_cache()
    return {"mfma_sustained": {"tflops": round(mf_tflops, 1), "frac_of_peak": round(mf_tflops / PEAK_BF16_TFLOPS, 4),
                               "clock_ghz": round(clock, 3), "work_groups": n_wg},
            "shapes": per,
            "ours": {"us": round(ours_us, 1), "frac": round(flops / ours_us / 1e6 / PEAK_BF16_TFLOPS, 4),
                     "frac_of_sustained": round(flops / ours_us / 1e6 / mf_tflops, 4)},
            "blas": {"library": "torch.mm (hipBLASLt)", "us": round(blas_us, 1),
                     "frac": round(flops / blas_us / 1e6 / PEAK_BF16_TFLOPS, 4),
                     "frac_of_sustained": round(flops / blas_us / 1e6 / mf_tflops, 4)}}


def decode_step_bytes(shape, k, batch, ctx):
    """Algorithmic HBM bytes of one decode step: every executed layer's weights once, and
    the K and V entries each query row's attention reads (full layers: the whole context;
    sliding layers: the last W positions), once per loop (the same in both KV modes)."""
    H, I = shape["hidden"], shape["intermediate"]
    qd, kd = shape["n_q_heads"] * shape["head_dim"], shape["n_kv_heads"] * shape["head_dim"]
    params = (qd + 2 * kd + (qd if shape["attn_gate"] else 0)) * H + H * qd + 2 * I * H + H * I
    wbytes = {"bf16": 2.0, "mxfp8": 1.0 + 1.0 / 32, "nvfp4": 0.5 + 1.0 / 16}[shape["weight_format"]]
    L = synth_layers(shape)
    kv_tok = 2 * kd * 2  # K and V of one position, bf16
    total_w = total_kv = 0.0
    for l, reps in L:
        total_w += reps(k) * params * wbytes
        full = l % shape["full_period"] == shape["full_period"] - 1
        keys = ctx + 1 if full else min(ctx + 1, shape["window"])
        total_kv += reps(k) * batch * keys * kv_tok
    return total_w, total_kv


def synth_layers(shape):
    """(physical layer, calls as a function of k) for every layer."""
    n_in, n_rec, n_out = shape["n_in"], shape["n_rec"], shape["n_out"]
    out = [(l, lambda k: 1) for l in range(n_in)]
    out += [(l, lambda k: k) for l in range(n_in, n_in + n_rec)]
    out += [(l, lambda k: 1) for l in range(n_in + n_rec, n_in + n_rec + n_out)]
    return out


def decode_leg(args, torch, synth, D, DoryRuntime):
    """The 72-layer decode shape (batch 32 over a seeded 32768-token context) at k = 1, 2
    and 4 in last_loop mode, whose cache holds one slot per layer whatever k is, so one
    seeded context serves every loop count. Per k: wall-clock ms per step (no events),
    the whole step's HBM fraction (weights and KV bytes of the method per step over that
    time, against 8 TB/s), and, from a separate pass with HIP events around its launches,
    the split-key attention kernel's own fraction."""
    shape = synth.config("D")
    batch, ctx_len, mode = 32, 32768, "last_loop"
    ks = [1, 2, 4]
    steps, warm = args.decode_steps, 2
    n_pos = ctx_len + len(ks) * (2 * steps + warm + 1) + 1
    weights = synth.make_weights(shape, 1234, "cuda")
    c = D.make_config(shape, max_loops=max(ks), max_seqs=batch, max_seq_len=n_pos, max_rows=batch)
    pages = D.dory_kv_pages_needed(c, D.MODES[mode], max(ks), n_pos, batch)
    rt = DoryRuntime(shape, weights, max_loops=max(ks), max_seqs=batch, max_seq_len=n_pos, max_rows=batch,
                     kv_pages=pages, mode=mode, loops=2)
    log(f"[bench] decode leg: seeding {ctx_len} tokens x {batch} (last_loop)")
    seed_kv(rt, shape, synth, D, torch, batch, ctx_len, [2] * batch, mode)
    for b in range(batch):
        D.dory_set_seq_loops(rt.ctx, b, 0)  # follow the context's k
    torch.cuda.synchronize()
    X = synth.make_inputs(batch, shape["hidden"], 77, device="cuda")
    Y = torch.empty((batch, shape["hidden"]), dtype=torch.float32, device="cuda")
    ids = list(range(batch))
    res = {}
    for kk in ks:
        D.dory_set_loops(rt.ctx, kk)
        for _ in range(warm):
            D.dory_decode_step(rt.ctx, ids, X, Y)
        torch.cuda.synchronize()
        ctx_now = D.dory_seq_len(rt.ctx, 0)
        t0 = time.perf_counter()
        for _ in range(steps):
            D.dory_decode_step(rt.ctx, ids, X, Y)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        D.dory_profile_enable(rt.ctx, [D.KC_ATTN])
        for _ in range(steps):
            D.dory_decode_step(rt.ctx, ids, X, Y)
        torch.cuda.synchronize()
        D.dory_profile_enable(rt.ctx, False)
        a = D.dory_profile_read(rt.ctx, D.KC_ATTN)
        wb, kvb = decode_step_bytes(shape, kk, batch, ctx_now + steps // 2)
        att = a["bytes"] / (a["ms"] / 1e3) / 1e9
        res[str(kk)] = {"tokens_per_s": round(batch / dt, 1), "ms_per_step": round(dt * 1e3, 3),
                        "step_gb": round((wb + kvb) / 1e9, 2),
                        "step_hbm_frac": round((wb + kvb) / dt / 1e9 / PEAK_HBM_GBS, 4),
                        "attention_hbm_frac": round(att / PEAK_HBM_GBS, 4)}
        log(f"[bench] decode k={kk}: {dt * 1e3:.2f} ms/step, {batch / dt:.0f} tok/s, "
            f"step {res[str(kk)]['step_hbm_frac']:.3f} of HBM")
    rt.close()
    del rt, weights
    torch.cuda.empty_cache()
    hbm = hbm_probe(torch)
    for r in res.values():
        r["step_frac_of_copy"] = round(r["step_hbm_frac"] * PEAK_HBM_GBS / hbm["copy_gbs"], 4)
    return {"workload": WORKLOAD_TEXT["D"] + ", last_loop", "batch": batch, "context": ctx_len,
            "steps": steps, "warmup": warm, "by_loops": res, "hbm_measured": hbm}


def hbm_probe(torch):
    """What HBM delivers to plain kernels on this device, for the decode fractions: a
    1 GiB copy (bytes read + written per second) and row sums over 1 GiB (rows of 4 KiB:
    bytes read per second), each the best of 10 timed launches."""
    n = 2 ** 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)

    def best(fn):
        ts = []
        for i in range(13):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            if i >= 3:
                ts.append(a.elapsed_time(b) / 1e3)
        return min(ts)

    rows = torch.empty(n // 1024, dtype=torch.float32, device="cuda")
    t_copy = best(lambda: dst.copy_(src))
    t_read = best(lambda: torch.sum(src.view(-1, 1024), dim=1, out=rows))
    del src, dst
    torch.cuda.empty_cache()
    return {"copy_gbs": round(2 * 4 * n / t_copy / 1e9, 1), "read_gbs": round(4 * n / t_read / 1e9, 1),
            "peak_gbs": PEAK_HBM_GBS}


def bench_decode(args, torch, synth, D, DoryRuntime):
    wl = args.workload
    gen = wl == "G"
    shape = synth.config("D" if gen else wl)
    dl = wl in ("D", "G")
    batch = args.batch or (32 if dl else 128)
    ctx_len = args.context or (32768 if dl else 8192)
    k = args.k or (2 if dl else 4)
    mode = args.mode or ("per_loop" if dl else "last_loop")
    ks = sorted({k} | ({int(x) for x in args.ks.split(",")} if args.ks else set()))
    mix = [int(x) for x in args.mix_k.split(",")] if args.mix_k else None
    if mix:
        k = max(mix)
        ks = [k]
    log(f"[bench] workload {wl}: weights")
    weights = synth.make_weights(shape, 1234, "cuda")
    cfg_loops = max(ks)
    steps = args.steps
    results = {}
    for kk in ks:
        from looped_ngpt_transformer_amd import dory as DD
        c = DD.make_config(shape, max_loops=cfg_loops, max_seqs=batch, max_seq_len=ctx_len + steps + args.warmup + 1,
                           max_rows=batch)
        pages = DD.dory_kv_pages_needed(c, DD.MODES[mode], kk, ctx_len + steps + args.warmup + 1, batch)
        rt = DoryRuntime(shape, weights, max_loops=cfg_loops, max_seqs=batch,
                         max_seq_len=ctx_len + steps + args.warmup + 1, max_rows=batch,
                         kv_pages=pages, mode=mode, loops=kk)
        log(f"[bench] k={kk} {mode}: KV pool {pages * rt.page_bytes / 1e9:.1f} GB; seeding {ctx_len} tokens x {batch}")
        t0 = time.perf_counter()
        kseq = [mix[b % len(mix)] for b in range(batch)] if mix else [kk] * batch
        seed_kv(rt, shape, synth, D, torch, batch, ctx_len, kseq, mode)
        D.dory_set_loops(rt.ctx, kk)
        torch.cuda.synchronize()
        log(f"[bench] seeded in {time.perf_counter() - t0:.1f} s")
        X = synth.make_inputs(batch * (steps + args.warmup), shape["hidden"], 77, device="cuda")
        Y = torch.empty((batch, shape["hidden"]), dtype=torch.float32, device="cuda")
        ids = list(range(batch))
        if gen:
            rt.bind_vocab(synth.make_vocab(shape, synth.VOCAB, 4321, "cuda"))
            U = synth.make_draws(batch * (steps + args.warmup + 1), 99, device="cuda")
            LG = torch.empty((batch, synth.VOCAB), dtype=torch.float32, device="cuda")
            TOK = torch.empty((batch,), dtype=torch.int32, device="cuda")
            XG = X[:batch].clone()

        def step(s):
            if not gen:
                r = s % (steps + args.warmup)  # the untimed breakdown step reuses the first inputs
                D.dory_decode_step(rt.ctx, ids, X[r * batch:(r + 1) * batch], Y)
                return
            D.dory_decode_step(rt.ctx, ids, XG, Y)
            D.dory_logits(rt.ctx, Y, LG)
            D.dory_sample_top_p(LG, U[s * batch:(s + 1) * batch], TOK, temperature=1.0, top_p=0.95)
            D.dory_embed(rt.ctx, TOK, XG)

        for s in range(args.warmup):
            step(s)
        torch.cuda.synchronize()
        # timed steps: HIP events around the attention launches (and the LM head) only
        D.dory_profile_enable(rt.ctx, [D.KC_ATTN] + ([D.KC_VOCAB] if gen else []))
        t0 = time.perf_counter()
        for s in range(args.warmup, args.warmup + steps):
            step(s)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        D.dory_profile_enable(rt.ctx, False)
        stats = kernel_stats(rt, D)
        kvb = D.dory_kv_bytes_in_use(rt.ctx)
        # one more (untimed) step with every kernel class recorded, for the breakdown
        D.dory_profile_enable(rt.ctx, True)
        step(args.warmup + steps)
        torch.cuda.synchronize()
        D.dory_profile_enable(rt.ctx, False)
        brk = kernel_stats(rt, D)
        results[kk] = (dt, stats, kvb, brk)
        log(f"[bench] k={kk}: {dt * 1e3:.2f} ms/step, {batch / dt:.1f} tok/s")
        rt.close()
        del rt
        torch.cuda.empty_cache()
    dt, stats, kvb, brk = results[k]
    tot_bytes = sum(s["bytes"] for s in brk.values())
    out = {
        "metric": ("generation" if gen else "decode") + " tokens/s (k=%s)" % (args.mix_k if mix else k),
        "value": round(batch / dt, 2),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random weights, seeded KV context, unit-norm inputs)",
        "config": {"workload": WORKLOAD_TEXT[wl], "batch": batch, "context": ctx_len,
                   "loops": ("mixed " + args.mix_k) if mix else k,
                   "kv_mode": mode, "weights": shape["weight_format"],
                   "executed_layers": shape["n_in"] + shape["n_out"] + k * shape["n_rec"]},
        "roofline": roofline_of(stats, "hbm", wl),
        **({"lm_head": lm_head_line(stats, steps)} if gen else {}),
        "step_hbm_gbs": round(tot_bytes / dt / 1e9, 1),
        "kv_bytes_in_use": kvb,
        "kernels": {n: {"launches": s["launches"], "ms": round(s["ms"], 3),
                        "gb": round(s["bytes"] / 1e9, 3)} for n, s in brk.items()},
    }
    if len(ks) > 1:
        out["by_loops"] = {str(kk): {"tokens_per_s": round(batch / r[0], 2), "ms_per_step": round(r[0] * 1e3, 3),
                                     "kv_bytes_in_use": r[2]} for kk, r in results.items()}
    del weights
    torch.cuda.empty_cache()
    out["hbm_measured"] = hbm_probe(torch)
    out["step_frac_of_copy"] = round(out["step_hbm_gbs"] / out["hbm_measured"]["copy_gbs"], 4)
    return out


def bench_spec(args, torch, synth, D, DoryRuntime):
    """Self-speculative generation against plain generation at the verifying loop count,
    same batch, context and weights. A step emits 1..gamma+1 tokens per sequence; value
    is emitted tokens per second. Random weights set the acceptance rate, so the line
    also gives the cost of each part and the acceptance at which the two break even."""
    shape = synth.config("D")
    batch = args.batch or 32
    ctx_len = args.context or 4096
    k = args.k or 4
    gamma = args.gamma
    steps, warm = args.steps, args.warmup
    n_tok = ctx_len + (steps + warm + 2) * (gamma + 1) + 2
    weights = synth.make_weights(shape, 1234, "cuda")
    pages = D.dory_kv_pages_needed(D.make_config(shape, max_loops=k, max_seqs=batch, max_seq_len=n_tok,
                                                 max_rows=batch * (gamma + 1)), D.KV_PER_LOOP, k, n_tok, batch)
    rt = DoryRuntime(shape, weights, max_loops=k, max_seqs=batch, max_seq_len=n_tok,
                     max_rows=batch * (gamma + 1), kv_pages=pages, mode="per_loop", loops=k)
    log(f"[bench] S: KV pool {pages * rt.page_bytes / 1e9:.1f} GB; seeding {ctx_len} tokens x {batch}")
    seed_kv(rt, shape, synth, D, torch, batch, ctx_len, [k] * batch, "per_loop")
    rt.bind_vocab(synth.make_vocab(shape, synth.VOCAB, 4321, "cuda"))
    ids = list(range(batch))
    nd = steps + warm
    UD = synth.make_draws(nd * gamma * batch, 101, device="cuda").view(nd, gamma, batch)
    UA = synth.make_draws(nd * gamma * batch, 102, device="cuda").view(nd, gamma, batch)
    US = synth.make_draws(nd * batch, 103, device="cuda").view(nd, batch)
    cur = synth.make_ids(batch, synth.VOCAB, 104, "cuda")
    emitted, accepted = 0, 0
    for s in range(nd):
        if s == warm:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        out, n_out, _ = rt.spec_step(ids, cur, gamma, UD[s], UA[s], US[s], reuse=args.reuse)
        cur = torch.tensor([int(out[b, n_out[b] - 1]) for b in ids], dtype=torch.int32, device="cuda")
        if s >= warm:
            emitted += int(n_out.sum())
            accepted += int((n_out - 1).sum())
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    log(f"[bench] spec: {dt * 1e3:.2f} ms/step, {emitted / steps / dt:.1f} tok/s")

    # the parts, timed alone on the same context (each restores the lengths it changed)
    lens = [D.dory_seq_len(rt.ctx, b) for b in ids]
    V = synth.VOCAB
    LG = torch.empty((batch, V), dtype=torch.float32, device="cuda")
    TOK = torch.empty((batch,), dtype=torch.int32, device="cuda")
    Y = torch.empty((batch, shape["hidden"]), dtype=torch.float32, device="cuda")

    def gen_step(loops, r):
        for b in ids:
            D.dory_set_seq_loops(rt.ctx, b, loops)
        x = rt.embed(TOK if r else cur)
        D.dory_decode_step(rt.ctx, ids, x, Y)
        D.dory_logits(rt.ctx, Y, LG)
        D.dory_sample_top_p(LG, US[r % nd], TOK)

    def timed(fn, reps):
        fn(0)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for r in range(reps):
            fn(r + 1)
        torch.cuda.synchronize()
        el = (time.perf_counter() - t) / reps
        for b, l0 in zip(ids, lens):
            D.dory_set_seq_loops(rt.ctx, b, 0)
            D.dory_truncate_seq(rt.ctx, b, l0)
        return el

    t_ar = timed(lambda r: gen_step(0, r), gamma)   # plain generation at k loops
    t_draft = timed(lambda r: gen_step(1, r), gamma)  # one draft step at one loop
    XV = synth.make_inputs(batch * (gamma + 1), shape["hidden"], 105, device="cuda")
    YV = torch.empty_like(XV)
    LV = torch.empty((batch * (gamma + 1), V), dtype=torch.float32, device="cuda")

    def verify(r):
        for b, l0 in zip(ids, lens):
            D.dory_truncate_seq(rt.ctx, b, l0)
        D.dory_prefill(rt.ctx, ids, [gamma + 1] * batch, XV, YV)
        D.dory_logits(rt.ctx, YV, LV)

    t_verify = timed(verify, 3)
    D.dory_profile_enable(rt.ctx, True)   # one more verifying chunk, every kernel class timed
    verify(0)
    torch.cuda.synchronize()
    D.dory_profile_enable(rt.ctx, False)
    vbrk = kernel_stats(rt, D)
    for b, l0 in zip(ids, lens):
        D.dory_truncate_seq(rt.ctx, b, l0)
    rt.close()
    ar_tps = batch / t_ar
    spec_tps = emitted / steps / dt
    out = {
        "metric": "self-speculative generation tokens/s (draft 1 loop, verify k=%d, gamma=%d)" % (k, gamma),
        "value": round(spec_tps, 2), "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded random weights, seeded per_loop KV context, seeded draws)",
        "config": {"workload": WORKLOAD_TEXT["S"], "batch": batch, "context": ctx_len, "loops": k,
                   "gamma": gamma, "kv_mode": "per_loop", "weights": shape["weight_format"],
                   "verify": "from loop 2 on the drafts' activations" if args.reuse else "recomputed"},
        "spec": {"accepted_per_step": round(accepted / steps / batch, 3),
                 "emitted_per_step": round(emitted / steps / batch, 3),
                 "autoregressive_k_tokens_per_s": round(ar_tps, 2),
                 "ratio_to_autoregressive": round(spec_tps / ar_tps, 3),
                 "ms_autoregressive_step": round(t_ar * 1e3, 3),
                 "ms_draft_step": round(t_draft * 1e3, 3),
                 "ms_verify_chunk": round(t_verify * 1e3, 3),
                 "breakeven_emitted_per_step": round((gamma * t_draft + t_verify) / t_ar, 3),
                 "verify_kernels": {n: {"launches": v["launches"], "ms": round(v["ms"], 3)} for n, v in vbrk.items()}},
    }
    return out


def seed_kv(rt, shape, synth, D, torch, batch, ctx_len, kseq, mode):
    """Reserve ctx_len positions per sequence and write seeded K/V into every cache slot
    the sequence holds (sliding layers: the last window of positions). Sequence b runs
    kseq[b] loops."""
    L = shape["n_in"] + shape["n_rec"] + shape["n_out"]
    W = shape["window"]
    for b in range(batch):
        k = kseq[b]
        D.dory_set_loops(rt.ctx, k)  # the loop count a new sequence takes
        D.dory_test_reserve(rt.ctx, b, ctx_len)
        if mode == "last_loop":
            D.dory_set_seq_loops(rt.ctx, b, k)
        for l in range(L):
            full = l % shape["full_period"] == shape["full_period"] - 1
            rec = shape["n_in"] <= l < shape["n_in"] + shape["n_rec"]
            slots = k if (rec and mode == "per_loop") else 1
            p0 = 0 if full else max(0, ctx_len - W)
            for s in range(slots):
                kk, vv = synth.make_kv(shape, 555, b, l, s, p0, ctx_len - p0, device="cuda")
                D.dory_test_fill_kv(rt.ctx, b, l, s, p0, kk, vv)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import synth
    from looped_ngpt_transformer_amd import dory as D
    from looped_ngpt_transformer_amd.runtime import DoryRuntime
    torch.cuda.set_device(0)
    if args.copy_probe:  # a plain copy kernel of known size: 1 GiB read, 1 GiB written
        src = torch.ones(2 ** 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if args.workload in ("P", "L", "T"):
        out = bench_prefill(args, torch, synth, D, DoryRuntime)
    elif args.workload == "S":
        out = bench_spec(args, torch, synth, D, DoryRuntime)
    else:
        out = bench_decode(args, torch, synth, D, DoryRuntime)
    out["env"] = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                  "gpu": torch.cuda.get_device_name(0)}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
