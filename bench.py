"""Benchmarks of the activation-sparse gated FFN on one MI355X.

Default workload (the headline): one decode FFN layer at the Llama-2-7B shape
(d_model 4096, d_ff 11008), bf16 weights N(0, 1/d_in), batch 1, ReLU exact
gating with the active fraction a set by the gate offset, 1024 seeded
synthetic tokens resident in HBM.  A step is one layer forward for one token.
Four weight copies rotate so that the 256 MB Infinity Cache cannot hold the
working set.  Reported: microseconds per layer and effective HBM GB/s on the
algorithmic bytes (W_gate in full, 16 KiB per active neuron, the token and
output vectors) for a in {1.0, 0.6, 0.3, 0.1}, the dense baseline, the speed-up
and its ideal 3 / (1 + 2a), the breakeven a (linear fit of sparse time against
a, solved against dense), the roofline of the main kernel (HIP events around
each of its launches) and the CPU oracle timed on the host cores.  `value` is
the effective GB/s at a = 0.1.

Other workloads (same JSON contract, one line each):
  --workload topk      int4 Qwen2.5-3B FFN shape, weight-aware top-k, batch 1 and 8
  --workload schedule  28 layers of 3584 / 18944 bf16 SwiGLU, batch 16, dense /
                       a ~ 0.3 / a ~ 0.13 thresholds, RMSNorm and residual
  --workload prefill   token-selective prefill, d_model 5120, d_ff 25600, L 16384
  --workload experts   adaptive expert top-K by routing mass over 16384 tokens,
                       384 and 256 routed experts, tau 0.5, buckets 3..6
  --workload breakeven batched decode (5 / 8 / 16 tokens): tile path, row gather and
                       the device's automatic choice against the union fraction

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
VALU_FP32_PEAK_TFLOPS = 157.3  # fp32 vector FMA: 256 CU x 128 lanes/clk x 2 flop x 2.4 GHz (unpacked v_fmac reaches it)
METRIC = "µs/layer & effective HBM GB/s (% of peak) vs active fraction a; breakeven a"

# HBM bytes per dispatch of a kernel from two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE in KiB per
# dispatch), FETCH scaled by what the counter reads for a plain 256 MiB copy (1.9998), WRITE by 1.0.
# Each entry is valid only for the kernel sources it was taken on (sha256 prefix over the listed
# files); after any change the figure is reported as null until the counters are taken again.
COUNTER_TRAFFIC = {
    "k_decode_b1": {"sources": ("decode.hip", "dev_common.h", "sffn_internal.h"),
                    "sha256_16": "1949ab87d41eb2f6",
                    "workload": "a = 0.1, bf16 4096 x 11008, batch 1",
                    "fetch_kib": 52955.10, "write_kib": 4171.10, "fetch_factor": 1.9998, "write_factor": 1.0000},
    "k_gu_i4_b1": {"sources": ("decode.hip", "dev_common.h", "sffn_internal.h"),
                   "sha256_16": "1949ab87d41eb2f6",
                   "workload": "int4-g128 2048 x 11008, batch 1, top-k",
                   "fetch_kib": 11517.00, "write_kib": 192.72, "fetch_factor": 1.9998, "write_factor": 1.0000},
    "k_gate_up_dual": {"sources": ("decode.hip", "dev_common.h", "sffn_internal.h"),
                       "sha256_16": "1949ab87d41eb2f6",
                       "workload": "bf16 3584 x 18944, 16 tokens, 28-layer schedule",
                       "fetch_kib": 134503.70, "write_kib": 7104.40, "fetch_factor": 1.9998, "write_factor": 1.0000},
    "k_gemm_big_gate_up": {"sources": ("prefill.hip", "dev_common.h", "sffn_internal.h"),
                           "sha256_16": "42fe0ba510580f94",
                           "workload": "bf16 5120 x 25600, L 16384, mass 0.5 (2674 kept rows)",
                           "fetch_kib": 1260053.50, "write_kib": 133700.00, "fetch_factor": 1.9998,
                           "write_factor": 1.0000},
    "k_expert_select": {"sources": ("experts.hip", "dev_common.h", "sffn_internal.h"),
                        "sha256_16": "7a84aadd75893141",
                        "workload": "16384 tokens x 384 experts, tau 0.5, buckets 3..6",
                        "fetch_kib": 12313.10, "write_kib": 896.00, "fetch_factor": 1.9998, "write_factor": 1.0000},
}


def counter_traffic(name):
    """Measured HBM bytes per dispatch for `name`, or None if its sources changed since."""
    import hashlib
    e = COUNTER_TRAFFIC.get(name)
    if e is None:
        return None
    h = hashlib.sha256()
    for f in e["sources"]:
        with open(os.path.join(ROOT, "activation_sparse_gated_gate_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != e["sha256_16"]:
        return None
    return int(round((e["fetch_kib"] * e["fetch_factor"] + e["write_kib"] * e["write_factor"]) * 1024))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2048)
    p.add_argument("--warmup", type=int, default=128)
    p.add_argument("--workload", default="decode",
                   choices=["decode", "topk", "schedule", "prefill", "experts", "breakeven", "copy", "reorder", "read",
                            "merge"])
    p.add_argument("--a", type=float, nargs="*", default=None,
                   help="decode: active fractions to time (default 1.0 0.6 0.3 0.1)")
    p.add_argument("--copies", type=int, default=4)
    p.add_argument("--tokens", type=int, default=1024)
    p.add_argument("--graph-steps", type=int, default=64, help="steps captured per HIP graph")
    p.add_argument("--cpu-tokens", type=int, default=1024, help="tokens timed on the CPU oracle (0 = skip)")
    p.add_argument("--no-sweep", action="store_true", help="decode: skip the a = 0.50..1.00 sweep (steps of 0.05)")
    p.add_argument("--no-torch", action="store_true", help="decode: skip the torch F.linear dense figure")
    p.add_argument("--no-graph", action="store_true")
    return p.parse_args()


# ---------------------------------------------------------------------------
# shared timing helpers
# ---------------------------------------------------------------------------

def graph_time_us(run, n_steps, graph_steps, n_graph_variants=None, spread=None):
    """Mean microseconds per step over exactly n_steps steps.  run(s0, n)
    launches steps s0 .. s0 + n - 1; the n_steps steps are captured into HIP
    graphs of graph_steps steps (the last one holding the remainder), each graph
    is replayed once untimed, then every graph once in order between two
    synchronisations: that pass is the timed one.  With a dict `spread`, events
    recorded between the replays of the timed pass, and further untimed passes
    until there are at least 16 replays, give the per-replay microseconds per step
    (p10 / median / p90 in spread).  n_graph_variants is accepted for callers that
    cap the number of distinct graphs; the steps of every graph are distinct."""
    import numpy as np
    import torch
    K = max(1, int(n_steps))
    G = max(1, min(int(graph_steps), K))
    sizes = [G] * (K // G) + ([K % G] if K % G else [])
    graphs = []
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        s0 = 0
        for n in sizes:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                run(s0, n)
            graphs.append(g)
            s0 += n
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(graphs) + 1)]
    ev[0].record()
    for i, g in enumerate(graphs):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    total_us = ev[0].elapsed_time(ev[-1]) * 1e3
    if spread is not None:
        per = [ev[i].elapsed_time(ev[i + 1]) * 1e3 / sizes[i] for i in range(len(graphs))]
        while len(per) < 16:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            i = len(per) % len(graphs)
            e0.record()
            graphs[i].replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / sizes[i])
        q = np.percentile(per, [10, 50, 90])
        spread.update(p10=round(float(q[0]), 3), median=round(float(q[1]), 3), p90=round(float(q[2]), 3),
                      replays=len(per), steps_per_replay=G)
    return total_us / K


def eager_time_us(run, n_steps):
    import torch
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    run(0, n_steps)
    en.record()
    torch.cuda.synchronize()
    return st.elapsed_time(en) * 1e3 / n_steps


def _hip():
    """The HIP runtime torch has loaded (same soname), for raw event handles."""
    import ctypes as C
    hip = C.CDLL("libamdhip64.so.7")
    hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
    hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
    hip.hipEventDestroy.argtypes = [C.c_void_p]
    return hip


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


def main_kernel_us(layers, run, nk, hold_ms=100.0):
    """Average duration of the library's main kernel over nk launches, from the
    start / stop events its own dispatch records (sffn_set_kernel_timer, which
    launches it through hipExtLaunchKernel).  The events skip the system-scope
    fence, so they bracket the kernel only.  A spin kernel of hold_ms runs
    first so that the launches queue back to back."""
    import ctypes as C

    import numpy as np
    import torch

    import activation_sparse_gated_gate_amd as sf
    hip = _hip()

    def mk():
        e = C.c_void_p()
        if hip.hipEventCreateWithFlags(C.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e.value
    pairs = [(mk(), mk()) for _ in range(nk)]
    arrays = []
    for i, L in enumerate(layers):
        mine = pairs[i::len(layers)]
        b = (C.c_void_p * len(mine))(*[p[0] for p in mine])
        e = (C.c_void_p * len(mine))(*[p[1] for p in mine])
        arrays.append((b, e))
        if sf.sffn_set_kernel_timer(L.handle, b, e, len(mine)) != 0:
            raise RuntimeError("sffn_set_kernel_timer failed")
    torch.cuda.synchronize()
    torch.cuda._sleep(int(hold_ms * 1e-3 * 2.4e9))
    run(0, nk)
    torch.cuda.synchronize()
    for L in layers:
        sf.sffn_set_kernel_timer(L.handle, None, None, 0)
    us = []
    for b, e in pairs:
        v = C.c_float()
        hip.hipEventElapsedTime(C.byref(v), b, e)
        us.append(v.value * 1e3)
        hip.hipEventDestroy(b)
        hip.hipEventDestroy(e)
    return float(np.mean(us))


def line(metric, value, unit, steps, warmup, ms_per_step, dtype, config, roofline, cpu, higher=True):
    return {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": ms_per_step, "higher_is_better": higher, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype, "data": "synthetic (seeded)", "config": config, "roofline": roofline,
        "cpu_baseline": cpu,
    }


def dev_tensor(a):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to("cuda:0")


def weights_dev(w):
    out = {"w_gate": dev_tensor(w.w_gate), "w_up": dev_tensor(w.w_up), "w_down": dev_tensor(w.w_down)}
    if w.s_gate is not None:
        out.update(s_gate=dev_tensor(w.s_gate), s_up=dev_tensor(w.s_up), s_down=dev_tensor(w.s_down))
    return out


# ---------------------------------------------------------------------------
# decode, Llama-2-7B FFN shape, batch 1 (the headline)
# ---------------------------------------------------------------------------

def torch_dense_us(w, X, copies, steps, warmup, graph_steps):
    """Sanity figure: the same dense ReGLU layer as three torch F.linear calls in
    bf16 (hipBLASLt / rocBLAS GEMV at batch 1), weights rotating over `copies`
    copies like the library's, graph-replayed over exactly `steps` steps."""
    import torch
    import torch.nn.functional as F
    Wg = [dev_tensor(w.w_gate).view(torch.bfloat16) for _ in range(copies)]
    Wu = [dev_tensor(w.w_up).view(torch.bfloat16) for _ in range(copies)]
    Wd = [dev_tensor(w.w_down).view(torch.bfloat16) for _ in range(copies)]
    Xb = dev_tensor(X).to(torch.bfloat16)
    Yb = torch.empty_like(Xb)
    T = X.shape[0]

    def run(s0, n):
        for st in range(s0, s0 + n):
            c, t = st % copies, st % T
            x = Xb[t:t + 1]
            h = torch.relu(F.linear(x, Wg[c])) * F.linear(x, Wu[c])
            Yb[t:t + 1] = F.linear(h, Wd[c])
    run(0, warmup)
    torch.cuda.synchronize()
    us = graph_time_us(run, steps, graph_steps)
    del Wg, Wu, Wd
    return us


def bench_decode(args):
    import numpy as np
    import torch

    import activation_sparse_gated_gate_amd as sf
    import synth

    d, f = 4096, 11008
    t0 = time.time()
    w = synth.cfg2_weights(d, f)
    X = synth.cfg2_tokens(args.tokens, d)
    log("generated inputs in %.1fs" % (time.time() - t0))
    wt = weights_dev(w)
    layers = [sf.Layer(d, f, 1, sf.W_BF16, sf.ACT_RELU, wt) for _ in range(args.copies)]
    del wt
    Xd = dev_tensor(X)
    Yd = torch.empty_like(Xd)
    T = args.tokens
    xs = [Xd[i:i + 1] for i in range(T)]
    ys = [Yd[i:i + 1] for i in range(T)]
    idx_buf = torch.empty(f, dtype=torch.int32, device="cuda:0")
    torch.cuda.synchronize()
    K = args.steps

    def policy(a):
        if a >= 1.0:
            return sf.make_policy("all")
        return sf.make_policy("exact", gate_bias=synth.gate_offset_for_active_fraction(a))

    def runner(pol, counts=None):
        def run(s0, n):
            for s in range(s0, s0 + n):
                L = layers[s % len(layers)]
                if counts is None:
                    L.forward(pol, xs[s % T], ys[s % T])
                else:
                    L.forward(pol, xs[s % T], ys[s % T], idx_out=idx_buf, count_out=counts[s - s0:s - s0 + 1])
        return run

    def time_policy(pol, spread=None):
        run = runner(pol)
        run(0, args.warmup)
        torch.cuda.synchronize()
        if args.no_graph:
            return eager_time_us(run, K)
        return graph_time_us(run, K, args.graph_steps, spread=spread)

    def realized_active(pol, n):
        cnt = torch.zeros(n, dtype=torch.int32, device="cuda:0")
        runner(pol, cnt)(0, n)
        torch.cuda.synchronize()
        return float(cnt.double().mean().item())

    def bytes_alg(n_active):
        # W_gate in full + (W_up row + W_down^T row + index/value) per active
        # neuron + x in and y out (fp32)
        return f * d * 2 + n_active * (2 * d * 2 + 8) + 2 * d * 4

    dense_bytes = 3 * f * d * 2 + 2 * d * 4
    dense_spread = {}
    dense_us = time_policy(sf.make_policy("dense"), dense_spread)
    log("dense (fused streaming kernel, every neuron): %.2f us/layer (%.0f GB/s on %.1f MB)"
        % (dense_us, dense_bytes / dense_us / 1e3, dense_bytes / 1e6))
    torch_us = float("nan")
    if not args.no_torch:
        torch_us = torch_dense_us(w, X, args.copies, K, args.warmup, args.graph_steps)
        log("torch F.linear dense (bf16): %.2f us/layer" % torch_us)
    a_main = [1.0, 0.6, 0.3, 0.1]
    a_list = list(args.a) if args.a else list(a_main)
    if 0.1 not in a_list:
        a_list.append(0.1)
    if not args.no_sweep:
        a_list += [a for a in [round(0.5 + 0.05 * i, 2) for i in range(10)] if a not in a_list]
    rows = {}
    for a in a_list:
        pol = policy(a)
        n_act = realized_active(pol, min(T, 256))
        sp = {}
        us = time_policy(pol, sp)
        rows[a] = dict(a=a, a_realized=round(n_act / f, 4), n_active=round(n_act, 1), us_per_layer=round(us, 3),
                       spread_us=sp, bytes_alg=int(bytes_alg(n_act)))
    # the dense reference: the faster of the dense kernel and the sparse kernels with every neuron
    dense_ref = min(dense_us, rows[1.0]["us_per_layer"]) if 1.0 in rows else dense_us
    for a in a_list:
        r = rows[a]
        us, n_act, B = r["us_per_layer"], r["n_active"], r["bytes_alg"]
        r.update(GBps=round(B / us / 1e3, 1), pct_peak=round(B / us / 1e3 / HBM_PEAK_GBS * 100, 1),
                 speedup_vs_dense=round(dense_ref / us, 3), ideal=round(3.0 / (1.0 + 2.0 * n_act / f), 3))
        r["frac_of_ideal"] = round(r["speedup_vs_dense"] / r["ideal"], 3)
        log("a=%.2f  n_active=%.0f  %.2f us/layer (p10 %.2f, p90 %.2f)  %.0f GB/s (%.1f%% of peak)  speedup %.2fx "
            "(ideal %.2fx)" % (a, n_act, us, r["spread_us"].get("p10", us), r["spread_us"].get("p90", us), r["GBps"],
                              r["pct_peak"], r["speedup_vs_dense"], r["ideal"]))

    # breakeven: the linear fit of sparse time against the realised a over the four main points, solved
    # against the dense reference; a crossing outside [0, 1] is no breakeven.  The sweep gives the
    # smallest measured a at which the sparse layer is no faster than dense.
    fit_a = [a for a in a_main if a in rows]
    breakeven, fit = None, None
    if len(fit_a) >= 2:
        pts = [(rows[a]["a_realized"], rows[a]["us_per_layer"]) for a in fit_a]
        c, t0f = np.polyfit([p[0] for p in pts], [p[1] for p in pts], 1)
        fit = {"t0_us": round(float(t0f), 3), "slope_us": round(float(c), 3)}
        if c > 0:
            x0 = float((dense_ref - t0f) / c)
            breakeven = round(x0, 3) if 0.0 <= x0 <= 1.0 else None
    swept = sorted(a for a in rows)
    sweep_be = next((a for a in swept if rows[a]["us_per_layer"] >= dense_ref), None)

    pol = policy(0.1)
    run = runner(pol)
    run(0, args.warmup)
    torch.cuda.synchronize()
    kus = main_kernel_us(layers, run, min(max(K, 256), 512))
    k_bytes = bytes_alg(rows[0.1]["n_active"])
    achieved = k_bytes / kus / 1e3
    log("main kernel (fused gate/selection/up/down): %.2f us avg, %.0f GB/s" % (kus, achieved))

    cpu = None
    if args.cpu_tokens > 0:
        import oracle
        threads = oracle.default_threads()
        b = synth.gate_offset_for_active_fraction(0.1)
        n = min(args.cpu_tokens, X.shape[0])
        oracle.decode(w, X[:1], mode="exact", bias=b, threads=threads)
        t1 = time.time()
        r = oracle.decode(w, X[:n], mode="exact", bias=b, threads=threads)
        dt = time.time() - t1
        n_act_cpu = float(r["sel"].sum(axis=1).mean())
        us_cpu = dt * 1e6 / n
        cpu = {"value": round(bytes_alg(n_act_cpu) / us_cpu / 1e3, 3), "unit": "GB/s",
               "us_per_layer": round(us_cpu, 1), "cores": threads, "kind": "oracle",
               "sample": "%d tokens of the same workload at a = 0.1 in one oracle call (OpenMP over tokens), "
                         "%.1f s wall" % (n, dt)}
        log("cpu oracle: %.0f us/layer with %d threads" % (us_cpu, threads))

    head = rows[0.1]
    cfg = {"workload": "decode gated-FFN layer, d_model 4096, d_ff 11008, bf16 weights, fp32 accumulate, "
                       "batch 1, ReLU exact gating, a = 0.1 headline",
           "tokens": T, "weight_copies": len(layers),
           "timing": "eager" if args.no_graph else
                     "exactly %d steps per point, HIP graphs of %d steps replayed once each; spread = "
                     "microseconds per step of single graph replays" % (K, min(args.graph_steps, K)),
           "dense_us_per_layer": round(dense_us, 3), "dense_spread_us": dense_spread,
           "dense_kernel": "mode DENSE: the fused streaming kernel over every neuron, no selection",
           "torch_flinear_us_per_layer": None if torch_us != torch_us else round(torch_us, 3),
           "dense_reference_us": round(dense_ref, 3),
           "dense_reference": "min(DENSE, sparse kernels at a = 1.0)",
           "sweep": [rows[a] for a in sorted(rows, reverse=True)],
           "breakeven_a": breakeven,
           "breakeven_note": None if breakeven is not None else
                             "none within [0, 1]: the fit of sparse time against a does not reach the dense "
                             "reference below a = 1",
           "breakeven_fit": fit,
           "sweep_first_a_not_faster_than_dense": sweep_be}
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic("k_decode_b1"),
            "kernel": "k_decode_b1<1,8> (gate GEMV + selection + compaction + up + down partial)",
            "kernel_us": round(kus, 3), "bytes_per_launch": int(k_bytes)}
    out = line(METRIC, head["GBps"], "GB/s", K, args.warmup, round(head["us_per_layer"] / 1e3, 6),
               "bf16", cfg, roof, cpu)
    print(json.dumps(out), flush=True)
    for L in layers:
        L.close()


# ---------------------------------------------------------------------------
# weight-aware top-k, int4 Qwen2.5-3B FFN shape, batch 1 and 8
# ---------------------------------------------------------------------------

def bench_topk(args):
    import numpy as np
    import torch

    import activation_sparse_gated_gate_amd as sf
    import synth

    d, f = 2048, 11008
    w = synth.cfg3_weights(d, f)
    X = synth.cfg3_tokens(args.tokens, d)
    wt = weights_dev(w)
    copies = 16  # 16 x 35 MB rotate past the Infinity Cache
    layers = [sf.Layer(d, f, 8, sf.W_INT4_G128, sf.ACT_SILU, wt) for _ in range(copies)]
    del wt
    Xd = dev_tensor(X)
    Yd = torch.empty_like(Xd)
    T = args.tokens
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    idx = torch.empty(f, dtype=torch.int32, device="cuda:0")
    steps = min(args.steps, 512)
    gate_up_bytes = 2 * (f * d // 2 + f * (d // 128) * 2)

    def bytes_alg(n_union, touched_groups):
        # gate and up read in full (the score needs u), W_down^T rows of the
        # union, the scale rows of touched 128-neuron groups, the column norms
        return gate_up_bytes + n_union * (d // 2) + touched_groups * d * 2 + f * 8

    dense_bytes = 3 * (f * d // 2) + 3 * f * (d // 128) * 2   # every int4 weight and its scales

    def time_pol(pol, B):
        xs = [Xd[i * B:(i + 1) * B] for i in range(T // B)]
        ys = [Yd[i * B:(i + 1) * B] for i in range(T // B)]
        nb = len(xs)

        def run(s0, n):
            for s in range(s0, s0 + n):
                layers[s % copies].forward(pol, xs[s % nb], ys[s % nb])
        run(0, args.warmup)
        torch.cuda.synchronize()
        return eager_time_us(run, steps) if args.no_graph else graph_time_us(run, steps, 32)

    # the dense reference per batch size: the faster of the dense GEMVs (mode DENSE) and every
    # neuron through the sparse kernels (mode ALL: the fixed-order gate, the up rows, the down rows)
    dense = {}
    for B in (1, 8):
        t_dense = time_pol(sf.make_policy("dense"), B)
        t_all = time_pol(sf.make_policy("all", use_union=True), B)
        dense[B] = {"dense_us": round(t_dense, 3), "all_us": round(t_all, 3), "ref_us": round(min(t_dense, t_all), 3)}
        log("int4 dense B=%d: DENSE %.2f us, ALL %.2f us" % (B, t_dense, t_all))

    rows = []
    for B in (1, 8):
        for pct in synth.CFG3_KEEP_PCT:
            k = synth.topk_count(f, pct)
            pol = sf.make_policy("topk", topk_k=k, use_union=B > 1)
            xs = [Xd[i * B:(i + 1) * B] for i in range(T // B)]
            ys = [Yd[i * B:(i + 1) * B] for i in range(T // B)]
            nb = len(xs)
            nu, tg = [], []
            for i in range(min(nb, 32)):  # union size and touched groups (not timed)
                layers[0].forward(pol, xs[i], ys[i], idx_out=idx, count_out=cnt)
                torch.cuda.synchronize()
                n = int(cnt.item())
                sel = idx[:n].cpu().numpy()
                nu.append(n)
                tg.append(len(np.unique(sel // 128)))
            us = time_pol(pol, B)
            Bb = bytes_alg(np.mean(nu), np.mean(tg))
            ideal = dense_bytes / Bb
            r = dict(batch=B, keep_pct=pct, k=k, union=round(float(np.mean(nu)), 1),
                     union_frac=round(float(np.mean(nu)) / f, 4), us_per_step=round(us, 3),
                     us_per_token=round(us / B, 3), bytes_alg=int(Bb), GBps=round(Bb / us / 1e3, 1),
                     speedup_vs_dense=round(dense[B]["ref_us"] / us, 3), ideal=round(ideal, 3),
                     frac_of_ideal=round(dense[B]["ref_us"] / us / ideal, 3))
            rows.append(r)
            log("topk B=%d keep %d%%: union %.0f, %.2f us/step, %.0f GB/s, %.2fx dense (ideal %.2fx)"
                % (B, pct, r["union"], us, r["GBps"], r["speedup_vs_dense"], ideal))
    pol = sf.make_policy("topk", topk_k=synth.topk_count(f, 17))
    xs1 = [Xd[i:i + 1] for i in range(T)]

    def run1(s0, n):
        for s in range(s0, s0 + n):
            layers[s % copies].forward(pol, xs1[s % T], Yd[:1])
    run1(0, 64)
    torch.cuda.synchronize()
    kus = main_kernel_us(layers, run1, 256)
    achieved = gate_up_bytes / kus / 1e3
    cpu = None
    if args.cpu_tokens > 0:
        import oracle
        threads = oracle.default_threads()
        n = min(64, args.cpu_tokens)
        t1 = time.time()
        oracle.decode(w, X[:n], mode="topk", topk_k=synth.topk_count(f, 17), threads=threads)
        dt = time.time() - t1
        cpu = {"value": round(dt * 1e6 / n, 1), "unit": "us/step", "cores": threads, "kind": "oracle",
               "sample": "%d tokens at batch 1, keep 17%%, one oracle call; %.1f s wall" % (n, dt)}
    head = rows[0]
    cfg = {"workload": "weight-aware top-k decode layer, int4-g128 fp16 scales, d_model 2048, d_ff 11008, "
                       "SwiGLU, batch 1 and 8 (union), keep 17/30/50%", "weight_copies": copies,
           "dense": dense, "dense_bytes": dense_bytes,
           "ideal": "dense bytes / the top-k path's algorithmic bytes (gate and up read in full)",
           "results": rows}
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic("k_gu_i4_b1"),
            "kernel": "k_gu_i4_b1<1,8> (int4 gate and up in the fixed order + score keys, batch 1)",
            "kernel_us": round(kus, 3), "bytes_per_launch": gate_up_bytes}
    out = line("µs/step & effective HBM GB/s, weight-aware top-k", head["GBps"], "GB/s", steps, args.warmup,
               round(head["us_per_step"] / 1e3, 6), "int4", cfg, roof, cpu)
    print(json.dumps(out), flush=True)
    for L in layers:
        L.close()


# ---------------------------------------------------------------------------
# 28-layer schedule, batch 16
# ---------------------------------------------------------------------------

def bench_schedule(args):
    import torch

    import activation_sparse_gated_gate_amd as sf
    import synth

    d, f, B, NL = synth.CFG4_D, synth.CFG4_F, synth.CFG4_B, synth.CFG4_LAYERS
    layers, pols = [], []
    t0 = time.time()
    for l in range(NL):
        w = synth.cfg4_layer_weights(l, d, f)
        wt = weights_dev(w)
        layers.append(sf.Layer(d, f, B, sf.W_BF16, sf.ACT_SILU, wt, rmsnorm=True, residual=True,
                               layouts=sf.LAYOUT_DECODE | sf.LAYOUT_BATCH))
        del wt, w
        mode, a = synth.cfg4_schedule(l)
        th = synth.gate_threshold_for_active_fraction(a) if mode == "thresh" else 0.0
        pols.append(sf.make_policy(mode, theta=th, use_union=True))
    log("built 28 layers in %.1fs" % (time.time() - t0))
    xs = [dev_tensor(synth.cfg4_input(B, d))] + [torch.empty(B, d, dtype=torch.float32, device="cuda:0")
                                                for _ in range(NL)]

    def step(s0, n):
        for _ in range(n):
            for l in range(NL):
                layers[l].forward(pols[l], xs[l], xs[l + 1])
    steps = min(args.steps, 64)
    step(0, 2)
    torch.cuda.synchronize()
    us_step = eager_time_us(step, steps) if args.no_graph else graph_time_us(step, steps, 4, 1)
    seg = {}
    for name, l in (("all_0_7", 0), ("a0.3_8_19", 8), ("a0.13_20_27", 20)):
        def one(s0, n, l=l):
            for _ in range(n):
                layers[l].forward(pols[l], xs[l], xs[l + 1])
        seg[name] = round(graph_time_us(one, 64, 16, 1), 3)
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    idx = torch.empty(f, dtype=torch.int32, device="cuda:0")
    dens = []
    for l in range(NL):
        layers[l].forward(pols[l], xs[l], xs[l + 1], idx_out=idx, count_out=cnt)
        torch.cuda.synchronize()
        dens.append(int(cnt.item()) / f)
    mat = f * d * 2
    bytes_step = sum(mat + dn * f * 2 * d * 2 + 3 * B * d * 4 for dn in dens)
    gbps = bytes_step / us_step / 1e3

    def gl(s0, n):
        for _ in range(n):
            layers[8].forward(pols[8], xs[8], xs[9])
    kus = main_kernel_us([layers[8]], gl, 64)
    flops_gate = 2.0 * B * f * d
    # the combined gate + up launch reads W_gate and W_up once each (4 d f bytes) and x_hat
    # (B d fp32), and writes the four gate class partials and the two halves of u (fp32)
    bytes_gu = 4.0 * d * f + 4.0 * B * d + 4.0 * 4 * B * f + 4.0 * 2 * B * f
    achieved = bytes_gu / kus / 1e3
    alu_frac = flops_gate / kus / 1e6 / VALU_FP32_PEAK_TFLOPS
    cpu = None
    if args.cpu_tokens > 0:
        import oracle
        threads = oracle.default_threads()
        w8 = synth.cfg4_layer_weights(8, d, f)
        x8 = xs[8].cpu().numpy()
        t1 = time.time()
        oracle.decode(w8, x8, mode="thresh", theta=synth.gate_threshold_for_active_fraction(0.3), union=True,
                      rmsnorm=True, residual=True, threads=threads)
        dt = time.time() - t1
        cpu = {"value": round(dt * 1e6, 1), "unit": "us/layer", "cores": threads, "kind": "oracle",
               "sample": "one threshold layer (a ~ 0.3, batch 16), %.1f s wall" % dt}
    cfg = {"workload": "28-layer decode schedule, d_model 3584, d_ff 18944, bf16 SwiGLU, batch 16, "
                       "RMSNorm + residual, layers 0-7 all, 8-19 a~0.3, 20-27 a~0.13, union per step",
           "us_per_layer_by_segment": seg, "union_density": [round(v, 4) for v in dens],
           "bytes_per_step": int(bytes_step)}
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": counter_traffic("k_gate_up_dual"),
            "kernel": "k_gate_up_dual<16> (fixed-order class-split gate GEMV on fp32 FMA and MFMA up, one launch, "
                      "16 tokens)",
            "kernel_us": round(kus, 3), "bytes_per_launch": int(bytes_gu), "flops_per_launch": flops_gate,
            "alu_frac": round(alu_frac, 4)}
    out = line("µs per 28-layer step & effective HBM GB/s", round(gbps, 1), "GB/s", steps, 2,
               round(us_step / 1e3, 4), "bf16", cfg, roof, cpu)
    print(json.dumps(out), flush=True)
    for L in layers:
        L.close()


# ---------------------------------------------------------------------------
# token-selective prefill, d_model 5120, d_ff 25600, L 16384
# ---------------------------------------------------------------------------

def bench_prefill(args):
    import numpy as np
    import torch

    import activation_sparse_gated_gate_amd as sf
    import synth

    d, f, L = synth.CFG5_D, synth.CFG5_F, synth.CFG5_L
    w = synth.cfg5_weights(d, f)
    Y, A = synth.cfg5_activations(L, d)
    wt = weights_dev(w)
    layer = sf.Layer(d, f, L, sf.W_BF16, sf.ACT_SILU, wt, layouts=sf.LAYOUT_PREFILL)
    del wt
    Yd, Ad = dev_tensor(Y), dev_tensor(A)
    Xd = Yd.clone()
    keep = torch.empty(L, dtype=torch.int32, device="cuda:0")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    fwd = sf.make_policy("tokens")
    reps = 5
    rows = []
    for mass in synth.CFG5_MASS:
        pol = sf.make_policy("tokens", mass_thresh=mass, recent_n=synth.CFG5_RECENT, min_keep=synth.CFG5_MIN_KEEP)
        layer.select(pol, Ad, keep, cnt)
        torch.cuda.synchronize()
        M = int(cnt.item())
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        t_sel, t_ffn, t_oop = [], [], []
        for _ in range(reps):
            ev[0].record()
            layer.select(pol, Ad, keep, cnt)
            ev[1].record()
            layer.forward(fwd, Xd, Xd, idx_in=keep, count_in=cnt)   # in place: t3 + t4
            ev[2].record()
            layer.forward(fwd, Yd, Xd, idx_in=keep, count_in=cnt)   # out of place: + copy of un-kept rows
            ev[3].record()
            torch.cuda.synchronize()
            t_sel.append(ev[0].elapsed_time(ev[1]) * 1e3)
            t_ffn.append(ev[1].elapsed_time(ev[2]) * 1e3)
            t_oop.append(ev[2].elapsed_time(ev[3]) * 1e3)
        flops = 6.0 * M * d * f
        us_ffn = float(np.median(t_ffn))

        # selection alone: HIP graphs of 8 back-to-back calls (no host launch gaps)
        def sel(s0, n, pol=pol):
            for _ in range(n):
                layer.select(pol, Ad, keep, cnt)
        us_sel = graph_time_us(sel, 32, 8, 1)
        r = dict(mass=mass, kept=M, kept_frac=round(M / L, 4), select_us=round(us_sel, 2),
                 select_us_eager=round(float(np.median(t_sel)), 2),
                 ffn_ms=round(us_ffn / 1e3, 4), ffn_out_of_place_ms=round(float(np.median(t_oop)) / 1e3, 4),
                 tflops=round(flops / us_ffn / 1e6, 1),
                 mfma_frac=round(flops / us_ffn / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4))
        rows.append(r)
        log("mass %.1f: kept %d, select %.1f us, FFN %.3f ms (%.0f TFLOP/s)"
            % (mass, M, r["select_us"], r["ffn_ms"], r["tflops"]))
    dense_ms = rows[-1]["ffn_ms"]
    for r in rows:
        r["speedup_vs_mass1"] = round(dense_ms / r["ffn_ms"], 3)
    # block-granular selection (128-token blocks, kept fraction bounded to
    # [0.10, 0.50]) over the same activations, one sequence and a varlen batch
    cu_sets = {"1 sequence": [0, L], "7 sequences": [0, 8192, 12288, 14336, 15360, 15872, 16383, 16384]}
    brows = []
    for name, cu in cu_sets.items():
        cut = torch.tensor(cu, dtype=torch.int32, device="cuda:0")
        for mass in synth.CFG5_MASS:
            bpol = sf.make_block_policy(mass, 0.10, 0.50, 128, synth.CFG5_RECENT, synth.CFG5_MIN_KEEP)
            layer.select_blocks(bpol, Ad, cut, keep, cnt)
            torch.cuda.synchronize()
            M = int(cnt.item())

            def bsel(s0, n, bpol=bpol, cut=cut):
                for _ in range(n):
                    layer.select_blocks(bpol, Ad, cut, keep, cnt)
            us_bsel = graph_time_us(bsel, 32, 8, 1)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            t_ffn = []
            for _ in range(reps):
                ev[0].record()
                layer.forward(fwd, Xd, Xd, idx_in=keep, count_in=cnt)
                ev[1].record()
                torch.cuda.synchronize()
                t_ffn.append(ev[0].elapsed_time(ev[1]) * 1e3)
            us_ffn = float(np.median(t_ffn))
            br = dict(batch=name, mass=mass, kept=M, kept_frac=round(M / L, 4), select_us=round(us_bsel, 2),
                      ffn_ms=round(us_ffn / 1e3, 4), speedup_vs_mass1=round(dense_ms * 1e3 / us_ffn, 3))
            brows.append(br)
            log("blocks, %s, mass %.1f: kept %d, select %.1f us, FFN %.3f ms"
                % (name, mass, M, br["select_us"], br["ffn_ms"]))
    pol = sf.make_policy("tokens", mass_thresh=0.5, recent_n=synth.CFG5_RECENT, min_keep=1)
    layer.select(pol, Ad, keep, cnt)
    torch.cuda.synchronize()
    M = int(cnt.item())

    def run(s0, n):
        for _ in range(n):
            layer.forward(fwd, Xd, Xd, idx_in=keep, count_in=cnt)
    kus = main_kernel_us([layer], run, 5)
    fl = 2.0 * M * d * 2 * f
    achieved = fl / kus / 1e6
    cpu = None
    if args.cpu_tokens > 0:
        import oracle
        threads = oracle.default_threads()
        t1 = time.time()
        s = oracle.token_norms(A, threads=threads)
        k_ref, _, _ = oracle.token_select(s, 0.5, synth.CFG5_RECENT, 1)
        t_sel = time.time() - t1
        n = 16
        t2 = time.time()
        oracle.prefill_rows(w, Y, k_ref[:n], threads=threads)
        dt = time.time() - t2
        cpu = {"value": round((t_sel + dt / n * k_ref.size) * 1e3, 1), "unit": "ms per layer at mass 0.5",
               "cores": threads, "kind": "oracle",
               "sample": "selection over all %d tokens (%.2f s) + FFN on %d of the %d kept rows (%.1f s), "
                         "scaled to all kept rows" % (L, t_sel, n, k_ref.size, dt)}
    mid = rows[1]
    cfg = {"workload": "token-selective prefill FFN, d_model 5120, d_ff 25600, L 16384, bf16 SwiGLU, "
                       "top-P mass with recent_n 128, min_keep 1; value at mass 0.5", "results": rows,
           "block_selection": brows}
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": counter_traffic("k_gemm_big_gate_up"),
            "kernel": "k_gemm_big<gate_up, 8 waves> (gathered rows x interleaved W_gate/W_up, SwiGLU epilogue)",
            "kernel_us": round(kus, 3), "flops_per_launch": fl}
    out = line("ms per prefill FFN layer & TFLOP/s vs mass", mid["tflops"], "TFLOP/s", reps, 1, mid["ffn_ms"],
               "bf16", cfg, roof, cpu)
    print(json.dumps(out), flush=True)
    layer.close()


def bench_breakeven(args):
    """Batched decode (BATCH layout, 5 / 8 / 16 tokens): the MFMA tile path and
    the row gather forced in turn, and the device's automatic choice, against the
    selected union's fraction of d_ff (THRESH on RMSNorm-ed inputs, union rule)."""
    import numpy as np
    import torch

    import activation_sparse_gated_gate_amd as sf
    import synth
    rows = []
    for (d, f) in ((3584, 18944), (4096, 11008)):
        w = synth.cfg4_layer_weights(8, d, f)
        wt = weights_dev(w)
        layer = sf.Layer(d, f, 16, sf.W_BF16, sf.ACT_SILU, wt, rmsnorm=True, residual=True,
                         layouts=sf.LAYOUT_DECODE | sf.LAYOUT_BATCH)
        del wt
        for B in (5, 8, 16):
            xs = [dev_tensor(synth.cfg4_input(B, d) * np.float32(1 + 0.1 * i)) for i in range(4)]
            ys = [torch.empty_like(x) for x in xs]
            for a in (0.002, 0.01, 0.02, 0.04, 0.07, 0.1, 0.3):
                th = synth.gate_threshold_for_active_fraction(a)
                row = {"d": d, "f": f, "B": B, "a": a}
                for name, bp in (("tiled", 1), ("gather", 2), ("auto", 0)):
                    pol = sf.make_policy("thresh", theta=th, use_union=True, batch_path=bp)

                    def run(s0, n, pol=pol):
                        for i in range(s0, s0 + n):
                            layer.forward(pol, xs[i % 4], ys[i % 4])
                    run(0, 4)
                    torch.cuda.synchronize()
                    row[name + "_us"] = round(graph_time_us(run, 64, 16, 4), 2)
                idx = torch.empty(f, dtype=torch.int32, device="cuda:0")
                cnt = torch.zeros(1, dtype=torch.int32, device="cuda:0")
                layer.select(sf.make_policy("thresh", theta=th, use_union=True), xs[0], idx, cnt)
                torch.cuda.synchronize()
                row["union"] = round(int(cnt.item()) / f, 4)
                row["auto_vs_best"] = round(min(row["tiled_us"], row["gather_us"]) / row["auto_us"], 3)
                rows.append(row)
                log(json.dumps(row))
        layer.close()
    worst = min(r["auto_vs_best"] for r in rows)
    cfg = {"workload": "batched decode layer (3584 x 18944 and 4096 x 11008 bf16 SwiGLU, RMSNorm + residual), "
                       "5 / 8 / 16 tokens, union rule, tile vs gather vs automatic path", "results": rows}
    out = line("worst ratio of the best forced path's time to the automatic choice's", worst, "ratio", 64, 4,
               None, "bf16", cfg, None, None)
    print(json.dumps(out), flush=True)


class _FREE_ENTRY_POINTS:
    """Stands for the library's handle-free entry points in main_kernel_us."""
    handle = None


def bench_experts(args):
    """Adaptive expert top-K: one call ranks the experts of 16384 tokens and picks
    each token's K by routing-probability mass.  Algorithmic bytes per token:
    the E fp32 probabilities read, plus K, kmax indices and kmax probabilities
    written (4 + 8 kmax)."""
    import numpy as np
    import torch

    import activation_sparse_gated_gate_amd as sf
    import synth

    T, tau, kmin, kmax = synth.EXPERT_T, synth.EXPERT_TAU, synth.EXPERT_KMIN, synth.EXPERT_KMAX
    rows = []
    main = None
    for E in synth.EXPERT_E:
        probs = synth.router_probs(T, E, seed=660 + E)
        P0 = dev_tensor(probs)
        # copies rotate so that the 256 MB Infinity Cache cannot hold them all
        ncopy = -(-(320 << 20) // P0.numel() // 4)
        Ps = [P0] + [P0.clone() for _ in range(ncopy - 1)]
        k = torch.empty(T, dtype=torch.int32, device="cuda:0")
        idx = torch.empty((T, kmax), dtype=torch.int32, device="cuda:0")
        w = torch.empty((T, kmax), dtype=torch.float32, device="cuda:0")

        def run(s0, n, Ps=Ps, k=k, idx=idx, w=w):
            for i in range(s0, s0 + n):
                sf.expert_select(Ps[i % len(Ps)], tau, kmin, kmax, k_out=k, idx_out=idx, w_out=w)
        run(0, 8)
        torch.cuda.synchronize()
        us_graph = graph_time_us(run, max(args.steps // 16, 64), 16, 4)
        # per-launch kernel time: start / stop events recorded by the kernel's own
        # dispatch (the handle-free timer of the library)
        kus = main_kernel_us([_FREE_ENTRY_POINTS], run, 32)
        kmean = float(k.float().mean().item())
        bytes_alg = T * (4 * E + 4 + 8 * kmax)
        r = dict(experts=E, copies=ncopy, us_per_call=round(us_graph, 2), kernel_us=round(kus, 2),
                 tokens_per_s=round(T / us_graph * 1e6, 0), gbs=round(bytes_alg / kus / 1e3, 1),
                 mean_k=round(kmean, 4), bucket_counts=np.bincount(k.cpu().numpy(), minlength=kmax + 1)[kmin:].tolist())
        rows.append(r)
        log("E %d: %.2f us per call (%.2f us kernel, %.0f GB/s), mean K %.3f"
            % (E, us_graph, kus, r["gbs"], kmean))
        if main is None:
            main = (r, bytes_alg, kus, probs)
    r, bytes_alg, kus, probs = main
    cpu = None
    if args.cpu_tokens > 0:
        import oracle
        n = T
        t1 = time.time()
        reps = 0
        while True:
            oracle.expert_select(probs[:n], tau, kmin, kmax)
            reps += 1
            if time.time() - t1 > 10.0 or reps >= 32:
                break
        dt = (time.time() - t1) / reps
        cpu = {"value": round(n / dt, 0), "unit": "tokens/s", "cores": 1, "kind": "oracle",
               "sample": "all %d tokens at E = %d, %d oracle call(s), single thread (qsort per token)"
                         % (n, synth.EXPERT_E[0], reps)}
    roof = {"bound": "hbm", "achieved": round(bytes_alg / kus / 1e3, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(bytes_alg / kus / 1e3 / HBM_PEAK_GBS, 4), "traffic": counter_traffic("k_expert_select"),
            "kernel": "k_expert_select<6> (one wave per token)", "kernel_us": round(kus, 3),
            "bytes_per_launch": bytes_alg}
    cfg = {"workload": "adaptive expert top-K by routing mass, 16384 tokens, tau 0.5, buckets 3..6; value at "
                       "384 routed experts", "results": rows}
    out = line("tokens/s of adaptive expert top-K (one call over a 16384-token batch)", r["tokens_per_s"],
               "tokens/s", max(args.steps // 16, 64), 8, round(r["us_per_call"] / 1e3, 5), "f32", cfg, roof, cpu)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# counter calibration: a plain device-to-device copy of known size
# ---------------------------------------------------------------------------

def bench_reorder(args):
    """Neuron order by activation frequency (WiSparse notes, section 5) on a
    4096 x 11008 bf16 ReLU layer whose gate rows have log-normal scales (hot and
    cold neurons): calibrate the counts on 256 tokens, then time the batch-1
    kernel and the 8-token MFMA tile path with the neurons in their original,
    BALANCE and CLUSTER orders (HIP graph replay, 4 rotating weight copies)."""
    import numpy as np
    import torch

    import activation_sparse_gated_gate_amd as sf
    import synth

    d, f, copies = 4096, 11008, 4
    w = synth.skewed_weights(synth.WT_BF16, d, f, synth.ACT_RELU, (1001, 1002, 1003, 1004))
    X = synth.round_to_bf16(synth.normal_f32(1005, (args.tokens, d)))
    b = synth.gate_offset_for_active_fraction(0.1)
    wt = weights_dev(w)
    lay = sf.LAYOUT_DECODE | sf.LAYOUT_BATCH
    plain = [sf.Layer(d, f, 8, sf.W_BF16, sf.ACT_RELU, wt, layouts=lay) for _ in range(copies)]
    Xd = dev_tensor(X)
    pol1 = sf.make_policy("exact", gate_bias=b)
    idx = torch.empty(f, dtype=torch.int32, device="cuda:0")
    cnt = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    counts = torch.zeros(f, dtype=torch.int32, device="cuda:0")
    y1 = torch.empty((1, d), dtype=torch.float32, device="cuda:0")
    for t in range(256):
        plain[0].forward(pol1, Xd[t:t + 1], y1, idx_out=idx, count_out=cnt)
        sf.neuron_counts(idx, cnt, counts)
    torch.cuda.synchronize()
    c = counts.cpu().numpy()
    orders = {"original": np.arange(f, dtype=np.int32),
              "balance": sf.frequency_order(c, sf.ORDER_BALANCE, sf.decode_block_rows(f)),
              "cluster": sf.frequency_order(c, sf.ORDER_CLUSTER)}
    layers = {"original": plain}
    for name in ("balance", "cluster"):
        pt = torch.from_numpy(orders[name]).to("cuda:0")
        layers[name] = [sf.Layer(d, f, 8, sf.W_BF16, sf.ACT_RELU, wt, layouts=lay, perm=pt) for _ in range(copies)]
    del wt
    T = args.tokens
    steps = min(args.steps, 1024)
    Y = torch.empty_like(Xd)
    res = {"calibration_tokens": 256, "mean_active": round(float(c.sum()) / 256 / f, 4),
           "hot_share": round(float(np.sort(c)[::-1][:f // 10].sum()) / max(1, int(c.sum())), 4)}
    rb = sf.decode_block_rows(f)
    for name, ls in layers.items():
        # load per batch-1 workgroup (expected active neurons of its block) and per 16-row tile at 8 tokens
        cc = c[orders[name]].astype(np.float64) / 256
        blk = np.add.reduceat(cc, np.arange(0, f, rb))
        tiles = cc.reshape(-1, 16)
        p_tile = 1.0 - np.prod(1.0 - np.minimum(tiles, 1.0), axis=1) ** 8

        def run1(s0, n, ls=ls):
            for s_ in range(s0, s0 + n):
                ls[s_ % copies].forward(pol1, Xd[s_ % T:s_ % T + 1], Y[:1])
        run1(0, args.warmup)
        torch.cuda.synchronize()
        us1 = graph_time_us(run1, steps, 64, 4)
        out = {"b1_us": round(us1, 3), "b1_max_block_load": round(float(blk.max()), 2),
               "b1_mean_block_load": round(float(blk.mean()), 2),
               "b8_expected_tiles_touched": round(float(p_tile.mean()), 4)}
        for path, key in ((1, "b8_tiles_us"), (0, "b8_auto_us")):
            pol8 = sf.make_policy("exact", gate_bias=b, use_union=True, batch_path=path)

            def run8(s0, n, ls=ls, pol8=pol8):
                for s_ in range(s0, s0 + n):
                    q = (8 * s_) % (T - 8)
                    ls[s_ % copies].forward(pol8, Xd[q:q + 8], Y[q:q + 8])
            run8(0, 8)
            torch.cuda.synchronize()
            out[key] = round(graph_time_us(run8, min(steps, 256), 32, 4), 3)
        res[name] = out
        log("reorder %s: batch 1 %.2f us, 8 tokens tiles %.2f us, auto %.2f us" %
            (name, out["b1_us"], out["b8_tiles_us"], out["b8_auto_us"]))
    cfg = {"workload": "neuron order by activation frequency: 4096 x 11008 bf16 ReLU layer, gate rows scaled by "
                       "exp(0.6 z), exact gating at the offset for a = 0.1; batch 1 and 8 tokens (union)",
           "tokens": T, "weight_copies": copies, "timing": "HIP graph replay", **res}
    out = line("µs/layer, 8-token MFMA tile path, neurons in CLUSTER order", res["cluster"]["b8_tiles_us"], "us",
               steps, args.warmup, round(res["cluster"]["b8_tiles_us"] / 1e3, 6), "bf16", cfg, None, None,
               higher=False)
    print(json.dumps(out), flush=True)


def free_kernel_us(run, nk, hold_ms=100.0):
    """Average duration of nk launches of a handle-free entry point's kernel
    (the read probe) from the start / stop events its own dispatch records
    (sffn_set_kernel_timer with no handle), as main_kernel_us does for a layer."""
    import ctypes as C

    import numpy as np
    import torch

    import activation_sparse_gated_gate_amd as sf
    hip = _hip()

    def mk():
        e = C.c_void_p()
        if hip.hipEventCreateWithFlags(C.byref(e), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        return e.value
    pairs = [(mk(), mk()) for _ in range(nk)]
    b = (C.c_void_p * nk)(*[p[0] for p in pairs])
    e = (C.c_void_p * nk)(*[p[1] for p in pairs])
    if sf.sffn_set_kernel_timer(None, b, e, nk) != 0:
        raise RuntimeError("sffn_set_kernel_timer failed")
    torch.cuda.synchronize()
    torch.cuda._sleep(int(hold_ms * 1e-3 * 2.4e9))
    run(nk)
    torch.cuda.synchronize()
    sf.sffn_set_kernel_timer(None, None, None, 0)
    us = []
    for bb, ee in pairs:
        v = C.c_float()
        hip.hipEventElapsedTime(C.byref(v), bb, ee)
        us.append(v.value * 1e3)
        hip.hipEventDestroy(bb)
        hip.hipEventDestroy(ee)
    return float(np.median(us)), float(np.mean(us))


def bench_read(args):
    """What one launch can read: sffn_read_probe_cfg over four rotating buffers
    (past the 256 MB Infinity Cache together) of 108.2 MB (the batch-1 decode
    kernel's algorithmic bytes at a = 0.1 on the 4096 x 11008 layer) and of
    90.2 MB (its gate matrix alone), for every access pattern, in-flight depth,
    cache policy, workgroup size and grid size the probe offers; kernel-only
    durations from dispatch-recorded events, as for the decode kernel.  Also a
    4 GiB stream (the long-run rate)."""
    import torch

    import activation_sparse_gated_gate_amd as sf
    s = torch.cuda.current_stream().cuda_stream
    out = torch.empty(65536, dtype=torch.int32, device="cuda:0")
    rows = []
    sizes = [("108.2 MB", 108198912), ("90.2 MB", 11008 * 4096 * 2)]
    for name, nb in sizes:
        bufs = [torch.ones(nb // 4, dtype=torch.float32, device="cuda:0") for _ in range(4)]
        for wg in (256, 512):
            for nt in (512, 1024):
                for pat in (0, 1):
                    for inf in (4, 8, 16):
                        for ntp in (1, 0):
                            cfg = sf.ProbeCfg(wg, nt, pat, inf, ntp)

                            def run(n, cfg=cfg, bufs=bufs, nb=nb):
                                for i in range(n):
                                    if sf._lib.sffn_read_probe_cfg(bufs[i % 4].data_ptr(), nb, C_byref(cfg),
                                                                   out.data_ptr(), s) != 0:
                                        raise RuntimeError("sffn_read_probe_cfg failed")
                            run(8)
                            torch.cuda.synchronize()
                            med, mean = free_kernel_us(run, 64)
                            rows.append({"bytes": name, "workgroups": wg, "threads": nt,
                                         "pattern": "per-workgroup block" if pat else "grid-stride",
                                         "in_flight": inf, "nontemporal": ntp, "us_median": round(med, 3),
                                         "us_mean": round(mean, 3), "GBps": round(nb / med / 1e3, 1)})
                            log("read %s wg %d x %d %s if %d nt %d: %.2f us (%.0f GB/s)"
                                % (name, wg, nt, "block" if pat else "stride", inf, ntp, med, nb / med / 1e3))
        del bufs
    big = torch.ones((4 << 30) // 4, dtype=torch.float32, device="cuda:0")
    cfg = sf.ProbeCfg(256, 1024, 0, 8, 1)

    def runb(n):
        for i in range(n):
            sf._lib.sffn_read_probe_cfg(big.data_ptr(), 4 << 30, C_byref(cfg), out.data_ptr(), s)
    runb(2)
    med, _ = free_kernel_us(runb, 8)
    stream_gbps = round((4 << 30) / med / 1e3, 1)
    log("read 4 GiB stream: %.1f us, %.0f GB/s" % (med, stream_gbps))
    best = {n: min((r for r in rows if r["bytes"] == n), key=lambda r: r["us_median"]) for n, _ in sizes}
    cfgd = {"workload": "HBM read ceiling of one launch: 4 rotating buffers of 108.2 MB and of 90.2 MB, every "
                        "probe configuration; kernel-only durations (dispatch-recorded events, median of 64)",
            "best": best, "stream_4GiB_GBps": stream_gbps, "results": rows}
    b108 = best["108.2 MB"]
    out_line = line("HBM read GB/s of one 108.2 MB launch (best probe configuration)", b108["GBps"], "GB/s", 64, 8,
                    round(b108["us_median"] / 1e3, 6), "u32", cfgd,
                    {"bound": "hbm", "achieved": b108["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(b108["GBps"] / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "k_read_probe_cfg", "kernel_us": b108["us_median"], "bytes_per_launch": 108198912},
                    None)
    print(json.dumps(out_line), flush=True)


def C_byref(x):
    import ctypes
    return ctypes.byref(x)


def bench_merge(args):
    """Run merging of the int4 W_down^T row gather (denseflux, section 5.5:
    merge adjacent reads when the gap is below L * B bytes, L and B measured on
    the device).  L: isolated 1 KB row reads at random offsets of a 1 GiB
    buffer (one wave, each read finished before the next); B: the best one-launch
    read rate of the gather's size and the long-stream rate.  Then the config-3
    top-k layer (int4, 2048 x 11008, keep 17 %, batch 1) timed with merge gaps of
    0 (off) up to every row of a share."""
    import numpy as np
    import torch

    import activation_sparse_gated_gate_amd as sf
    import synth

    s = torch.cuda.current_stream().cuda_stream
    # --- L: latency of isolated 1 KB row reads ---
    nbuf = 1 << 30
    buf = torch.ones(nbuf // 4, dtype=torch.float32, device="cuda:0")
    rng = np.random.default_rng(7)
    n = 512
    offs = torch.from_numpy((rng.integers(0, nbuf // 1024, n) * 1024).astype(np.uint64).view(np.int64)).to("cuda:0")
    lat = torch.empty(n + 2, dtype=torch.int64, device="cuda:0")
    for _ in range(2):
        if sf._lib.sffn_read_latency_probe(buf.data_ptr(), nbuf, 1024, offs.data_ptr(), n, lat.data_ptr(), s) != 0:
            raise RuntimeError("sffn_read_latency_probe failed")
    torch.cuda.synchronize()
    lv = lat.cpu().numpy()
    ghz = lv[n] / (lv[n + 1] * 10.0)
    cyc = np.sort(lv[:n])
    L_ns = float(np.median(cyc)) / ghz
    log("isolated 1 KB row read: median %.0f cycles = %.0f ns at %.2f GHz (p10 %.0f, p90 %.0f ns)"
        % (np.median(cyc), L_ns, ghz, np.percentile(cyc, 10) / ghz, np.percentile(cyc, 90) / ghz))
    del buf
    # --- B: one-launch read of the gather's bytes (1871 rows of 1 KB) and the long stream ---
    out = torch.empty(65536, dtype=torch.int32, device="cuda:0")
    rates = {}
    for name, nb in (("gather 1.9 MB", 1871 * 1024), ("stream 4 GiB", 4 << 30)):
        bufs = [torch.ones(nb // 4, dtype=torch.float32, device="cuda:0") for _ in range(1 if nb > (1 << 30) else 16)]
        cfg = sf.ProbeCfg(256, 1024, 0, 8, 1)

        def run(k, bufs=bufs, nb=nb, cfg=cfg):
            for i in range(k):
                sf._lib.sffn_read_probe_cfg(bufs[i % len(bufs)].data_ptr(), nb, C_byref(cfg), out.data_ptr(), s)
        run(4)
        med, _ = free_kernel_us(run, 32 if nb > (1 << 30) else 256)
        rates[name] = nb / med / 1e3
        log("B (%s): %.2f us, %.0f GB/s" % (name, med, rates[name]))
        del bufs
    LB = {k: L_ns * 1e-9 * v * 1e9 for k, v in rates.items()}   # bytes
    # --- the gather with merge gaps ---
    d, f = 2048, 11008
    w = synth.cfg3_weights(d, f)
    X = synth.cfg3_tokens(args.tokens, d)
    wt = weights_dev(w)
    copies = 16
    layers = [sf.Layer(d, f, 1, sf.W_INT4_G128, sf.ACT_SILU, wt) for _ in range(copies)]
    del wt
    Xd = dev_tensor(X)
    Yd = torch.empty_like(Xd)
    T = args.tokens
    k = synth.topk_count(f, 17)
    steps = min(args.steps, 512)
    res = []
    yref = None
    for gap in (0, 1, 2, 4, 8, 16, 64):
        pol = sf.make_policy("topk", topk_k=k, merge_gap=gap)

        def runl(s0, nn, pol=pol):
            for st in range(s0, s0 + nn):
                layers[st % copies].forward(pol, Xd[st % T:st % T + 1], Yd[st % T:st % T + 1])
        runl(0, args.warmup)
        torch.cuda.synchronize()
        y = Yd[:64].clone()
        if yref is None:
            yref = y
        same = bool(torch.equal(y, yref))
        us = graph_time_us(runl, steps, 32)
        # rows read per token with this gap, from the selected sets (shares of R = ceil(f / 256) neurons)
        idx = torch.empty(f, dtype=torch.int32, device="cuda:0")
        cnt = torch.zeros(1, dtype=torch.int32, device="cuda:0")
        rows_read = []
        R = (f + 255) // 256
        for t in range(16):
            layers[0].forward(sf.make_policy("topk", topk_k=k), Xd[t:t + 1], Yd[t:t + 1], idx_out=idx, count_out=cnt)
            torch.cuda.synchronize()
            sel = np.zeros(f, bool)
            sel[idx[:int(cnt.item())].cpu().numpy()] = True
            tot = 0
            for q in range(0, f, R):
                sh = np.flatnonzero(sel[q:q + R])
                tot += sh.size
                if gap > 0 and sh.size > 1:
                    g = np.diff(sh) - 1
                    tot += int(g[g <= gap].sum())
            rows_read.append(tot)
        rr = float(np.mean(rows_read))
        res.append({"merge_gap_rows": gap, "us_per_step": round(us, 3), "rows_read": round(rr, 1),
                    "extra_rows_pct": round(100.0 * (rr / k - 1.0), 1), "same_output": same})
        log("merge gap %d rows: %.2f us/step, %.0f rows read (%.1f%% more), same output %s"
            % (gap, us, rr, 100.0 * (rr / k - 1.0), same))
        Yd.zero_()
    base = res[0]["us_per_step"]
    bestm = min(res, key=lambda r: r["us_per_step"])
    cfg = {"workload": "run merging of the int4 W_down^T gather, config-3 top-k layer (2048 x 11008, keep 17 %, "
                       "batch 1, 16 rotating copies)",
           "L_ns_median": round(L_ns, 1), "clock_GHz": round(float(ghz), 3),
           "B_GBps": {k2: round(v, 1) for k2, v in rates.items()},
           "LxB_bytes": {k2: int(v) for k2, v in LB.items()},
           "LxB_rows_of_1KB": {k2: round(v / 1024, 1) for k2, v in LB.items()},
           "results": res, "best_gap_rows": bestm["merge_gap_rows"],
           "rule_gap_rows": int(LB["gather 1.9 MB"] // 1024)}
    out_line = line("µs/step of the top-k layer vs merge gap (run merging, denseflux §5.5)", base, "us", steps,
                    args.warmup, round(base / 1e3, 6), "int4", cfg, None, None, higher=False)
    print(json.dumps(out_line), flush=True)
    for L in layers:
        L.close()


def bench_copy(args):
    import torch
    n = 256 << 20  # 256 MiB per copy, 8 copies per run
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(8):
        dst.copy_(src)
    torch.cuda.synchronize()
    st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.record()
    for _ in range(8):
        dst.copy_(src)
    en.record()
    torch.cuda.synchronize()
    us = st.elapsed_time(en) * 1e3 / 8
    gbps = 2 * n / us / 1e3
    out = line("device copy GB/s (read + write), counter calibration", round(gbps, 1), "GB/s", 8, 8,
               round(us / 1e3, 4), "f32", {"workload": "torch copy of 256 MiB, read 256 MiB + write 256 MiB per launch"},
               None, None)
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch
    torch.cuda.set_device(0)
    {"decode": bench_decode, "topk": bench_topk, "schedule": bench_schedule,
     "prefill": bench_prefill, "experts": bench_experts, "breakeven": bench_breakeven,
     "copy": bench_copy, "reorder": bench_reorder, "read": bench_read, "merge": bench_merge}[args.workload](args)


if __name__ == "__main__":
    main()
