"""Benchmark of the quantized MoE layer on one MI355X.

Default run (no flags): the four measured workloads in one process, one JSON line.
  * decode (the headline, top-level `value`): one Xing4.0-29B-A4B MoE layer -- hidden 3584,
    64 routed experts top-4 + 1 shared, expert_ffn 1024, sigmoid router, routed_scaling 2.0,
    IQ4_NL experts -- decoding 1000 independent tokens, T=1 per call.  The layer is placed 32
    times in HBM (12.9 GB) and token i uses placement i mod 32, so the 256 MB last-level cache
    cannot serve one token's expert reads from an earlier token's.  A step is the 1000-token
    sweep, captured once as a HIP graph and replayed.
  * prefill (nested object): one T=2048 call of the prefill shape (hidden 2048, 256 experts
    top-8 + 1 shared, ffn 512, Zipf(1.0) popularity), bf16 grouped MFMA; reports TFLOP/s and
    the fraction of bf16 MFMA peak, and the HBM fraction.
  * batch (nested): one T=128 call of the Xing4 layer per step.
  * stack (nested): 38 Xing4 layers resident in HBM, T=1 per step through all of them, each
    layer's input chained from the previous one, by moe_stack_decode (one call: two decode
    launches per layer); the same step as chained per-layer calls timed beside it;
    Zipf(1.1) popularity.
  * variants (nested): the sigmoid-gated shared expert (decode), the W4A8 contract (Q8_0
    activations: T=1, T=128, the T=2048 prefill call), a dense FFN block (hidden 3584,
    FFN 9216, T=1) and the IQ4_XS and packed 3-bit codecs (T=1, T=128), each timed and
    checked against the oracle.
Every leg times its steps with HIP events on the stream it launches on (median and spread
over the steps), runs the CPU oracle on a bounded sample of its own inputs (the cpu_baseline),
compares the GPU rows of those tokens with the oracle's (routing bit-exact, outputs within
max-abs 2e-2 / rel-L2 1e-3) and, on the decode and stack paths, reads the status word.  Any miss makes
the exit status non-zero after the line is printed.

`--workload X` runs one leg alone and prints its line at top level (profiling runs).
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
METRIC = "MoE-layer decode tok/s + achieved HBM GB/s (% peak); prefill TFLOP/s (% MFMA)"
TOL_MAX_ABS, TOL_REL_L2 = 2e-2, 1e-3
N_TOKENS = 1000
PLACEMENTS = 32
CPU_LABEL = "CPU oracle (reference semantics, double-precision sums), not an optimized CPU kernel"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--workload", choices=["all", "decode", "prefill", "stack", "batch", "variants"], default="all",
                   help="all (default): decode line with prefill, batch and stack nested; or one leg alone")
    p.add_argument("--stack-layers", type=int, default=38, help="layers of the stack workload")
    p.add_argument("--stack-distinct", type=int, default=4,
                   help="stack: distinct expert weight sets drawn (placed once per layer at distinct addresses)")
    p.add_argument("--stack-tokens", type=int, default=20,
                   help="distinct tokens captured in the stack graph (steps per replay)")
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--distinct-layers", type=int, default=4,
                   help="decode: distinct seeded layers generated; placements reuse them at distinct addresses")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle legs (and the output checks)")
    p.add_argument("--no-graph", action="store_true", help="decode: replay eagerly instead of through a HIP graph")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="first run one plain device copy of this many MiB (a kernel of known traffic, to scale "
                        "the HBM byte counters of a profiler run)")
    return p.parse_args()


# ---------------------------------------------------------------- helpers

def measured_traffic(record):
    """HBM bytes per launch from the committed counter summary, or None when a source of the counted
    kernels (their .hip files and the headers they include) has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", record)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    for src, sha in zip(rec["kernel_sources"], rec["sha256"]):
        p = os.path.join(ROOT, src)
        if not os.path.exists(p):
            return None
        with open(p, "rb") as f:
            if hashlib.sha256(f.read()).hexdigest() != sha:
                return None
    return int(rec["bytes_per_call"])


def copy_calibration(mib):
    """One elementwise copy kernel that reads and writes exactly mib MiB."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    del src, dst


def stream_gbs(torch):
    """The box's own streaming rates, best of 3: the library's read-only streaming kernel over 4 GiB (more
    than the last-level cache) and a torch 1 GiB device copy (read + write)."""
    import quantized_moe_decode_sigmoid_amd as qm
    nbytes = 4 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    dst = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    read_s, copy_s = [], []
    stream = torch.cuda.current_stream()
    for _ in range(3):
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record(stream)
        qm.moe_stream_read(src, nbytes, sink)
        b.record(stream)
        dst.copy_(src[: 1 << 28])
        c.record(stream)
        torch.cuda.synchronize()
        read_s.append(a.elapsed_time(b) / 1e3)
        copy_s.append(b.elapsed_time(c) / 1e3)
    del src, dst
    return {"read_gbs": round(nbytes / min(read_s) / 1e9, 1), "copy_gbs": round(2 * (1 << 30) / min(copy_s) / 1e9, 1),
            "read_kernel": "moe_stream_read, 4 GiB", "copy": "torch copy_, 1 GiB"}


def log(msg):
    """Progress on stderr (the JSON line is the only thing on stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def spread(ms):
    """Median and spread of per-step times (ms)."""
    a = np.asarray(ms, np.float64)
    return {"median_ms": round(float(np.median(a)), 4), "min_ms": round(float(a.min()), 4),
            "max_ms": round(float(a.max()), 4), "n": int(a.size)}


def timed_steps(torch, stream, fn, steps):
    """Run fn() `steps` times on `stream` with a HIP event between consecutive steps; returns the total
    and the per-step times in ms (events recorded on the launching stream)."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        fn()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return evs[0].elapsed_time(evs[-1]), per


class Check:
    """Collects the output checks of every leg; a miss makes the exit status non-zero."""

    def __init__(self):
        self.failures = []

    def compare(self, leg, got, want, ids=None, rid=None, w=None, rw=None):
        got = np.asarray(got, np.float64)
        want = np.asarray(want, np.float64)
        mae = float(np.max(np.abs(got - want))) if got.size else 0.0
        rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)) if got.size else 0.0
        ok = bool(np.all(np.isfinite(got))) and mae <= TOL_MAX_ABS and rel <= TOL_REL_L2
        res = {"rows": int(got.shape[0]) if got.ndim else 1, "max_abs": float(f"{mae:.3e}"),
               "rel_l2": float(f"{rel:.3e}")}
        if ids is not None:
            same = bool(np.array_equal(ids, rid)) and bool(np.array_equal(
                np.asarray(w, np.float32).view(np.uint32), np.asarray(rw, np.float32).view(np.uint32)))
            res["routing_bit_exact"] = same
            ok = ok and same
        res["ok"] = ok
        if not ok:
            self.failures.append(f"{leg}: {res}")
        return res

    def status(self, leg, word):
        if word != 0:
            self.failures.append(f"{leg}: status word {word} (a decode wait gave up)")
        return int(word)


def status_word(torch, qm, cfg, T, ws):
    st = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    qm.moe_workspace_status(cfg, T, ws, st)
    return int(st[0].item())


def oracle_rate(oracle, n, seconds, threads, sample):
    return {"value": round(n / seconds, 3), "unit": "tok/s", "cores": threads, "kind": "oracle", "label": CPU_LABEL,
            "sample": sample, "seconds": round(seconds, 2), **cpu_info()}


# ---------------------------------------------------------------- decode (headline)

def run_decode(args, check):
    import torch

    import quantized_moe_decode_sigmoid_amd as qm
    import synth

    shape = synth.WORKLOADS["xing4"]
    H, E, K, F = shape.hidden, shape.n_experts, shape.top_k, shape.ffn
    cfg = qm.make_config(H, F, E, K, shape.n_shared, shape.routed_scale)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    eb = qm.moe_expert_bytes(cfg)

    t0 = time.time()
    distinct = max(1, min(args.distinct_layers, PLACEMENTS))
    layers = [synth.layer_inputs(shape, layer=l) for l in range(distinct)]
    x_bits = synth.tokens(shape, N_TOKENS)
    gen_s = time.time() - t0

    # placements: packed arena + shared + router weight at distinct addresses
    arenas, shareds, gates = [], [], []
    staged = []
    for l in layers:
        a = torch.from_numpy(l["arena"]).to(dev)
        s = torch.from_numpy(l["shared"]).to(dev)
        pa, ps = torch.empty_like(a), torch.empty_like(s)
        qm.moe_pack_experts(cfg, E, a, pa)
        qm.moe_pack_experts(cfg, 1, s, ps)
        staged.append((pa, ps, torch.from_numpy(l["gate_w"]).to(dev)))
        del a, s
    for c in range(PLACEMENTS):
        pa, ps, g = staged[c % distinct]
        arenas.append(pa.clone())
        shareds.append(ps.clone())
        gates.append(g.clone())
    del staged
    torch.cuda.synchronize()

    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    out = torch.empty((N_TOKENS, H), dtype=torch.float32, device=dev)
    ids = torch.empty((N_TOKENS, K), dtype=torch.int32, device=dev)
    wts = torch.empty((N_TOKENS, K), dtype=torch.float32, device=dev)
    ws = torch.empty(qm.moe_workspace_bytes(cfg, 1), dtype=torch.uint8, device=dev)
    qm.moe_workspace_init(cfg, 1, ws)

    def sweep():
        for i in range(N_TOKENS):
            c = i % PLACEMENTS
            qm.moe_layer_forward(cfg, 1, x[i:i + 1], gates[c], None, arenas[c], shareds[c], out[i:i + 1],
                                 ids[i:i + 1], wts[i:i + 1], ws)

    stream = torch.cuda.Stream()
    graph = None
    with torch.cuda.stream(stream):
        sweep()  # eager warm-up outside the graph
        torch.cuda.synchronize()
        if not args.no_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                sweep()
        run = graph.replay if graph is not None else sweep
        t_first = time.time()
        run()
        torch.cuda.synchronize()
        first_ms = (time.time() - t_first) * 1e3
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        t_wall = time.time()
        total_ms, per_step = timed_steps(torch, stream, run, args.steps)
        wall_s = time.time() - t_wall

        # kernel timing: HIP events around each token's launch on this stream, queued
        # behind a spin kernel so that the GPU never waits for the host
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(N_TOKENS)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(N_TOKENS)]
        torch.cuda._sleep(400_000_000)
        for i in range(N_TOKENS):
            c = i % PLACEMENTS
            starts[i].record(stream)
            qm.moe_layer_forward(cfg, 1, x[i:i + 1], gates[c], None, arenas[c], shareds[c], out[i:i + 1],
                                 ids[i:i + 1], wts[i:i + 1], ws)
            ends[i].record(stream)
        torch.cuda.synchronize()
        word = status_word(torch, qm, cfg, 1, ws)
    call_ev_us = np.array([s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends)])

    ms_per_step = total_ms / args.steps
    tok_s = N_TOKENS / (ms_per_step / 1e3)
    # algorithmic bytes of one layer launch (T=1): 5 experts, router weight, x, out
    layer_bytes = (K + shape.n_shared) * eb + E * H * 4 + H * 2 + H * 4
    # one layer call's duration over the timed region: the events bracketing the
    # graph replays, divided by the calls they hold
    call_us = ms_per_step * 1e3 / N_TOKENS
    achieved = layer_bytes / (call_us / 1e6) / 1e9

    cpu, parity = None, None
    if not args.no_cpu:
        import oracle
        log("decode: CPU oracle")
        thr = oracle.threads()
        # tokens i < n use distinct layer i % distinct (placement i mod 32): one oracle call per distinct layer
        n = 64 * distinct
        want = np.empty((n, H), np.float32)
        rid = np.empty((n, K), np.int32)
        rw = np.empty((n, K), np.float32)
        c0 = time.time()
        for d in range(distinct):
            rows = np.arange(d, n, distinct)
            l = layers[d]
            want[rows], rid[rows], rw[rows] = oracle.layer(x_bits[rows], l["gate_w"], l["arena"], l["shared"], K, F,
                                                           shape.routed_scale)
        cs = time.time() - c0
        used = min(thr, n // distinct)
        cpu = oracle_rate(oracle, n, cs, used, f"the first {n} of the {N_TOKENS} tokens, one oracle.layer call of "
                                               f"{n // distinct} tokens per distinct layer ({used} threads)")
        # the single-threaded oracle on a few of the same tokens: same bits (tokens are independent and each
        # token's sums run in one fixed order), and its rate
        oracle.set_threads(1)
        n1 = 8
        c0 = time.time()
        one, _, _ = oracle.layer(x_bits[0:n1:distinct], layers[0]["gate_w"], layers[0]["arena"], layers[0]["shared"],
                                 K, F, shape.routed_scale)
        c1 = time.time() - c0
        oracle.set_threads(thr)
        cpu["single_thread"] = {"value": round((n1 // distinct) / c1, 3), "unit": "tok/s", "cores": 1,
                                "sample": f"{n1 // distinct} tokens of distinct layer 0, one call"}
        cpu["single_equals_all_cores"] = bool(np.array_equal(one.view(np.uint32),
                                                             want[0:n1:distinct].view(np.uint32)))
        if not cpu["single_equals_all_cores"]:
            check.failures.append("decode: single-threaded oracle differs from the all-core run")
        got = out[:n].cpu().numpy()
        parity = check.compare("decode", got, want, ids[:n].cpu().numpy(), rid, wts[:n].cpu().numpy(), rw)
    box = stream_gbs(torch)
    parity = parity or {}
    parity["status_word"] = check.status("decode", word)

    return {
        "metric": METRIC,
        "value": round(tok_s, 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "xing4 MoE layer decode, T=1 per call: hidden 3584, 64 experts top-4 + 1 shared, "
                               "ffn 1024, IQ4_NL experts, sigmoid router, scale 2.0; 1000 tokens per step over "
                               f"{PLACEMENTS} placements of {distinct} distinct seeded layers",
                   "tokens_per_step": N_TOKENS, "graph": graph is not None},
        "step_spread": spread(per_step),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode_traffic.json"),
                     "kernel": "moe_layer_forward T=1: k_decode_scores + k_decode_experts (HIP events around the "
                               "timed region of graph replays, divided by the layer calls in it)",
                     "bytes_per_launch": layer_bytes, "avg_us": round(call_us, 3),
                     "per_call_events": {"avg_us": round(float(np.mean(call_ev_us)), 3),
                                         "median_us": round(float(np.median(call_ev_us)), 3),
                                         "note": "eager calls with HIP events around each"},
                     "box_stream": box, "frac_of_box_read": round(achieved / box["read_gbs"], 4)},
        "cpu_baseline": cpu,
        "parity": parity,
        "layer_gbs": round(layer_bytes * tok_s / 1e9, 1),
        "first_step_ms": round(first_ms, 3),
        "wall_s": round(wall_s, 3),
        "setup_s": round(gen_s, 1),
    }


# ---------------------------------------------------------------- prefill

def run_prefill(args, check):
    """One prefill-sized layer call per step: T=2048, H=2048, 256 experts top-8 + 1 shared, ffn 512,
    Zipf(1.0) expert popularity through the selection bias; bf16 grouped MFMA FFN."""
    import torch

    import quantized_moe_decode_sigmoid_amd as qm
    import synth

    shape = synth.WORKLOADS["prefill"]
    T, H, E, K, F = shape.tokens, shape.hidden, shape.n_experts, shape.top_k, shape.ffn
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    lam = synth.zipf_lambda(shape)
    inp = synth.layer_inputs(shape, lam=lam)
    x_bits = synth.tokens(shape, T)
    gen_s = time.time() - t0
    cfg = qm.make_config(H, F, E, K, shape.n_shared, shape.routed_scale)
    prec = qm.moe_resolved_precision(cfg, T)
    dl = qm.DeviceLayer(cfg, inp["gate_w"], inp["bias"], inp["arena"], inp["shared"])
    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    wts = torch.empty((T, K), dtype=torch.float32, device=dev)
    ws = dl.workspace(T)
    steps = max(args.steps, 5)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        def step():
            qm.moe_layer_forward(cfg, T, x, dl.gate_w, dl.bias, dl.arena, dl.shared, out, ids, wts, ws)

        t_first = time.time()
        step()
        torch.cuda.synchronize()
        first_ms = (time.time() - t_first) * 1e3
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        total_ms, per_step = timed_steps(torch, stream, step, steps)
        layer_ms = total_ms / steps
        # the expert FFN alone (bucketing, gate/up, down, combine) on the routing just computed
        def ffn():
            qm.moe_expert_forward(cfg, T, x, ids, wts, dl.arena, dl.shared, out, ws)
        torch.cuda._sleep(50_000_000)
        ffn_total, ffn_per = timed_steps(torch, stream, ffn, steps)
    ffn_us = np.array(ffn_per) * 1e3
    counts = np.bincount(ids.cpu().numpy().reshape(-1), minlength=E)
    flops = 2.0 * 3 * H * F * (T * K + T * shape.n_shared)
    # MFMA rows the 16-row sub-tiles execute per useful row (tiles of 128 routes of one expert)
    rows_useful = T * K + T * shape.n_shared
    rows_run = sum(16 * ((c + 15) // 16) for c in counts.tolist()) + 16 * ((T + 15) // 16) * shape.n_shared
    ffn_avg_us = ffn_total * 1e3 / steps
    ffn_tflops = flops / (ffn_avg_us * 1e-6) / 1e12
    # algorithmic bytes of one moe_expert_forward call: every expert once (routed + shared), x, the
    # routing (ids + weights), the fp32 output
    ebytes = 3 * F * (H // 32) * 18
    ffn_bytes = (E + shape.n_shared) * ebytes + T * H * 2 + T * K * 8 + T * H * 4
    ffn_gbs = ffn_bytes / (ffn_avg_us * 1e-6) / 1e9

    cpu, parity = None, None
    if not args.no_cpu:
        import oracle
        log("prefill: CPU oracle")
        n = 256
        c0 = time.time()
        want, rid, rw = oracle.layer(x_bits[:n], inp["gate_w"], inp["arena"], inp["shared"], K, F,
                                     shape.routed_scale, inp["bias"], oracle.BF16 if prec == qm.PREC_BF16 else
                                     oracle.FP32)
        cs = time.time() - c0
        used = min(oracle.threads(), n)
        cpu = oracle_rate(oracle, n, cs, used, f"the first {n} of the {T} tokens in one oracle.layer call")
        parity = check.compare("prefill", out[:n].cpu().numpy(), want, ids[:n].cpu().numpy(), rid,
                               wts[:n].cpu().numpy(), rw)

    mfma_bound = ffn_bytes / HBM_PEAK_GBS <= flops / 1e3 / MFMA_BF16_PEAK_TFLOPS
    return {
        "metric": METRIC,
        "value": round(flops / (layer_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(layer_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if prec == qm.PREC_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": "prefill MoE layer, T=2048: hidden 2048, 256 experts top-8 + 1 shared, ffn 512, "
                               "IQ4_NL experts, sigmoid router, scale 2.0, Zipf(1.0) expert popularity",
                   "tokens_per_step": T, "zipf_lambda": lam},
        "step_spread": spread(per_step),
        "mfma_tflops": round(ffn_tflops, 2),
        "mfma_frac": round(ffn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "hbm_frac": round(ffn_gbs / HBM_PEAK_GBS, 4),
        # Every expert's weights are read once per call (more bytes than the 256 MB last-level cache), so
        # the FFN's HBM floor (bytes / 8 TB/s) is above its MFMA floor (flops / 2.5 PFLOP/s): HBM-bound.
        "roofline": {"bound": "mfma" if mfma_bound else "hbm",
                     "achieved": round(ffn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ffn_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("prefill_traffic.json"),
                     "kernel": "moe_expert_forward bf16: k_bucket + k_gate_up_bf16 + k_down_bf16 (+ combine) "
                               "(HIP events around each call on its stream)",
                     "bytes_per_launch": ffn_bytes, "flops_per_launch": flops,
                     "mfma_tflops": round(ffn_tflops, 2), "mfma_peak": MFMA_BF16_PEAK_TFLOPS,
                     "mfma_frac": round(ffn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "hbm_floor_us": round(ffn_bytes / HBM_PEAK_GBS / 1e3, 2),
                     "mfma_floor_us": round(flops / 1e6 / MFMA_BF16_PEAK_TFLOPS, 2),
                     "avg_us": round(ffn_avg_us, 3), "ffn_spread_us": spread(ffn_us)},
        "cpu_baseline": cpu,
        "parity": parity,
        "tok_s": round(T / (layer_ms * 1e-3), 1),
        "routes_per_expert": {"max": int(counts.max()), "min": int(counts.min()),
                              "median": float(np.median(counts))},
        "mfma_rows_per_useful_row": round(rows_run / rows_useful, 4),
        "first_step_ms": round(first_ms, 3),
        "setup_s": round(gen_s, 1),
    }


# ---------------------------------------------------------------- batch

def run_batch(args, check):
    """One Xing4 layer call of T=128 tokens per step (zero selection bias), on the multi-kernel exact-weight
    path; four placements of the layer cycled so that consecutive steps do not share cached weights."""
    import torch

    import quantized_moe_decode_sigmoid_amd as qm
    import synth

    shape = synth.WORKLOADS["batch"]
    T, H, E, K, F = shape.tokens, shape.hidden, shape.n_experts, shape.top_k, shape.ffn
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    inp = synth.layer_inputs(shape)
    x_bits = synth.tokens(shape, T)
    gen_s = time.time() - t0
    cfg = qm.make_config(H, F, E, K, shape.n_shared, shape.routed_scale)
    prec = qm.moe_resolved_precision(cfg, T)
    n_place = 4
    dl = qm.DeviceLayer(cfg, inp["gate_w"], None, inp["arena"], inp["shared"])
    places = [(dl.gate_w.clone(), dl.arena.clone(), dl.shared.clone()) for _ in range(n_place)]
    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    wts = torch.empty((T, K), dtype=torch.float32, device=dev)
    ws = dl.workspace(T)
    n_steps = max(args.steps, 2 * n_place)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        it = [0]

        def step():
            g, a, sh = places[it[0] % n_place]
            it[0] += 1
            qm.moe_layer_forward(cfg, T, x, g, None, a, sh, out, ids, wts, ws)

        for _ in range(max(args.warmup, n_place)):
            step()
        torch.cuda.synchronize()
        total_ms, per_step = timed_steps(torch, stream, step, n_steps)
        layer_ms = total_ms / n_steps
    counts = np.bincount(ids.cpu().numpy().reshape(-1), minlength=E)
    touched = int((counts > 0).sum())
    eb = qm.moe_expert_bytes(cfg)
    # algorithmic bytes of one call: each expert the batch routes to once, the shared expert, the router
    # weight, x, the fp32 output
    call_bytes = (touched + shape.n_shared) * eb + E * H * 4 + T * H * 2 + T * H * 4
    gbs = call_bytes / (layer_ms * 1e-3) / 1e9

    cpu, parity = None, None
    if not args.no_cpu:
        import oracle
        c0 = time.time()
        want, rid, rw = oracle.layer(x_bits, inp["gate_w"], inp["arena"], inp["shared"], K, F, shape.routed_scale,
                                     None, oracle.BF16 if prec == qm.PREC_BF16 else oracle.FP32)
        cs = time.time() - c0
        used = min(oracle.threads(), T)
        cpu = oracle_rate(oracle, T, cs, used, f"all {T} tokens of the call in one oracle.layer call")
        parity = check.compare("batch", out.cpu().numpy(), want, ids.cpu().numpy(), rid, wts.cpu().numpy(), rw)

    return {
        "metric": METRIC,
        "value": round(T / (layer_ms * 1e-3), 1),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": n_steps,
        "warmup": max(args.warmup, n_place),
        "ms_per_step": round(layer_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if prec == qm.PREC_BF16 else "f32",
        "data": "synthetic",
        "config": {"workload": "xing4 MoE layer, T=128 per call: hidden 3584, 64 experts top-4 + 1 shared, ffn "
                               "1024, IQ4_NL experts, sigmoid router, scale 2.0, no selection bias; "
                               f"{n_place} placements cycled",
                   "tokens_per_step": T},
        "step_spread": spread(per_step),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("batch_traffic.json"),
                     "kernel": "moe_layer_forward T=128: router, top-k, bucketing, gate/up, down, combine "
                               "(HIP events around the timed region, divided by the calls in it)",
                     "bytes_per_launch": call_bytes, "avg_us": round(layer_ms * 1e3, 3)},
        "cpu_baseline": cpu,
        "parity": parity,
        "experts_touched": touched,
        "routes_per_expert": {"max": int(counts.max()), "min": int(counts.min()),
                              "median": float(np.median(counts))},
        "setup_s": round(gen_s, 1),
    }


# ---------------------------------------------------------------- stack

def run_stack(args, check):
    """38 MoE layers of the Xing4 shape resident in HBM, one token per step (T=1) through all of them,
    each layer's input chained from the previous layer's input and output by bf16(rmsnorm(x + out)):
    moe_stack_decode (one call: per layer the decode plan's two launches, the layer's input formed in the
    first), timed through a HIP graph; the same step as chained moe_layer_forward_chained calls timed beside
    it; Zipf(1.1) expert popularity."""
    import torch

    import quantized_moe_decode_sigmoid_amd as qm
    import synth

    shape = synth.WORKLOADS["stack"]
    H, E, K, F = shape.hidden, shape.n_experts, shape.top_k, shape.ffn
    nl = args.stack_layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    lam = synth.zipf_lambda(shape)
    cfg = qm.make_config(H, F, E, K, shape.n_shared, shape.routed_scale)
    t0 = time.time()
    # Router weights and selection biases are drawn per layer (each layer routes differently); expert
    # weights are drawn for `stack_distinct` layers and placed once per layer at distinct addresses, so
    # a token streams as many distinct HBM bytes as with 38 distinct draws (drawing 15 GB of IQ4_NL
    # experts takes minutes on the host).
    nd = max(1, min(args.stack_distinct, nl))
    packed = []
    for d in range(nd):
        inp = synth.layer_inputs(shape, layer=d, lam=lam)
        packed.append((inp["arena"], inp["shared"],
                       qm.DeviceLayer(cfg, inp["gate_w"], None, inp["arena"], inp["shared"])))
        log(f"stack: expert set {d + 1} of {nd} drawn, {time.time() - t0:.0f} s")
    layers, host = [], []
    for l in range(nl):
        arena_h, shared_h, src = packed[l % nd]
        gate_w = synth.gate_weights(shape, layer=l)
        bias = synth.zipf_bias(shape, lam, layer=l)
        layers.append(qm.DeviceLayer.from_packed(cfg, torch.from_numpy(gate_w).to(dev),
                                                 torch.from_numpy(bias).to(dev), src.arena.clone(),
                                                 src.shared.clone()))
        host.append({"gate_w": gate_w, "bias": bias, "arena": arena_h, "shared": shared_h})
    del packed
    gen_s = time.time() - t0
    S = args.stack_tokens
    x_bits = synth.tokens(shape, S, first=7000)
    x0 = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    arr = qm.stack_layers([(dl.gate_w, dl.bias, dl.arena, dl.shared) for dl in layers])
    sws = torch.empty(qm.moe_stack_workspace_bytes(cfg, nl), dtype=torch.uint8, device=dev)
    xall = torch.empty((S, nl, H), dtype=torch.bfloat16, device=dev)  # every token's input to every layer
    oall = torch.empty((S, nl, H), dtype=torch.float32, device=dev)
    ids = torch.empty((S, nl, K), dtype=torch.int32, device=dev)
    wts = torch.empty((S, nl, K), dtype=torch.float32, device=dev)

    def stack_step(i):
        qm.moe_stack_decode(cfg, nl, arr, x0[i:i + 1], xall[i], oall[i], ids[i], wts[i], sws)

    def steps():
        for i in range(S):
            stack_step(i)

    # the same step as chained layer calls (layer 0 on the token, layers 1.. by moe_layer_forward_chained,
    # the norm inside the router kernel): the path moe_stack_decode replaces, timed for comparison
    ws = torch.empty(qm.moe_workspace_bytes(cfg, 1), dtype=torch.uint8, device=dev)
    qm.moe_workspace_init(cfg, 1, ws)
    outs = torch.empty((nl, H), dtype=torch.float32, device=dev)
    xl = torch.empty((nl, H), dtype=torch.bfloat16, device=dev)
    cids = torch.empty((nl, K), dtype=torch.int32, device=dev)
    cw = torch.empty((nl, K), dtype=torch.float32, device=dev)

    def chained_steps():
        for i in range(S):
            xl[0].copy_(x0[i])
            for l, dl in enumerate(layers):
                if l == 0:
                    qm.moe_layer_forward(cfg, 1, xl[0:1], dl.gate_w, dl.bias, dl.arena, dl.shared, outs[0:1],
                                         cids[0], cw[0], ws)
                else:
                    qm.moe_layer_forward_chained(cfg, 1, xl[l - 1:l], outs[l - 1:l], xl[l:l + 1], dl.gate_w,
                                                 dl.bias, dl.arena, dl.shared, outs[l:l + 1], cids[l], cw[l], ws)

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        steps()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            steps()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        total_ms, per_replay = timed_steps(torch, stream, graph.replay, args.steps)
        st = torch.full((4,), -1, dtype=torch.int32, device=dev)
        qm.moe_stack_status(cfg, nl, sws, st)
        word = int(st[0].item())
        # the calls alone: events around each call of one eager pass over the S tokens, the queue kept busy
        # by a spin kernel so that host launch gaps do not enter
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(S)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(S)]
        torch.cuda._sleep(200_000_000)
        for i in range(S):
            starts[i].record(stream)
            stack_step(i)
            ends[i].record(stream)
        torch.cuda.synchronize()
        # the chained calls, captured and timed the same way
        chained_steps()
        torch.cuda.synchronize()
        cgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cgraph, stream=stream):
            chained_steps()
        for _ in range(args.warmup):
            cgraph.replay()
        torch.cuda.synchronize()
        chained_ms, _ = timed_steps(torch, stream, cgraph.replay, args.steps)
        del cgraph
    n_chk = min(S, 8)
    x_in, o_out = xall[:n_chk], oall[:n_chk]
    ms_per_token = total_ms / (args.steps * S)
    chained_ms_per_token = chained_ms / (args.steps * S)
    moe_ms_per_token = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / S
    eb = qm.moe_expert_bytes(cfg)
    expert_bytes = nl * (K + shape.n_shared) * eb
    router_bytes = nl * E * H * 4
    # rank-frequency: each layer's expert counts sorted (layers rank their experts differently), summed by rank
    ids_h = ids.cpu().numpy()
    by_rank = np.zeros(E, np.int64)
    for l in range(nl):
        by_rank += np.sort(np.bincount(ids_h[:, l, :].reshape(-1), minlength=E))[::-1]
    c = by_rank.astype(np.float64)
    c = c[c > 0]
    slope = float(np.polyfit(np.log(np.arange(1, c.size + 1)), np.log(c), 1)[0]) if c.size > 1 else None
    gbs = (expert_bytes + router_bytes) / (ms_per_token * 1e-3) / 1e9

    cpu, parity = None, None
    if not args.no_cpu:
        import oracle
        # the oracle runs each layer on the GPU's input to that layer (n_chk tokens per call), so its outputs
        # are also the per-layer check of the GPU chain
        xin = x_in.view(torch.int16).cpu().numpy().view(np.uint16)
        got = o_out.cpu().numpy()
        gid, gw = ids_h[:n_chk], wts.cpu().numpy()[:n_chk]
        want = np.empty_like(got)
        rid = np.empty((n_chk, nl, K), np.int32)
        rw = np.empty((n_chk, nl, K), np.float32)
        c0 = time.time()
        for l in range(nl):
            if l % 8 == 0:
                log(f"stack: CPU oracle layer {l} of {nl}, {time.time() - c0:.0f} s")
            inp = host[l]
            want[:, l], rid[:, l], rw[:, l] = oracle.layer(xin[:, l], inp["gate_w"], inp["arena"], inp["shared"],
                                                           K, F, shape.routed_scale, inp["bias"])
        cs = time.time() - c0
        used = min(oracle.threads(), n_chk)
        cpu = oracle_rate(oracle, n_chk, cs, used, f"{n_chk} tokens through all {nl} layers, one oracle.layer call "
                                                   f"of {n_chk} tokens per layer on the GPU chain's inputs")
        parity = check.compare("stack", got.reshape(-1, H), want.reshape(-1, H), gid, rid, gw, rw)
        parity["layers"] = nl
    parity = parity or {}
    parity["status_word"] = check.status("stack", word)
    del layers, host
    return {
        "metric": METRIC,
        "value": round(1e3 / ms_per_token, 2),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps * S,
        "warmup": args.warmup * S,
        "ms_per_step": round(ms_per_token, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{nl}-layer MoE stack decode, T=1: each layer hidden 3584, 64 experts top-4 + 1 "
                               "shared, ffn 1024, IQ4_NL, sigmoid router, scale 2.0; layer input = bf16(rmsnorm("
                               "previous input + previous output)) by one fused kernel; Zipf(1.1) expert popularity",
                   "layers": nl, "distinct_tokens": S, "zipf_lambda": lam, "graph": True,
                   "call": "moe_stack_decode: per layer the router kernel (norm of the previous layer's input "
                           "and output, logits) and the experts kernel",
                   "expert_sets": f"router weights and biases drawn per layer; expert weights drawn for {nd} "
                                  f"layers, each layer's placed at its own address"},
        "step_spread": spread(np.asarray(per_replay) / S),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("stack_traffic.json"),
                     "kernel": "whole step: per layer k_decode_scores_chained + k_decode_experts",
                     "bytes_per_token": expert_bytes + router_bytes},
        "cpu_baseline": cpu,
        "parity": parity,
        "expert_bytes_per_token": expert_bytes,
        "moe_calls_ms_per_token": round(moe_ms_per_token, 4),
        "chained_calls": {"ms_per_token": round(chained_ms_per_token, 4),
                          "value": round(1e3 / chained_ms_per_token, 2), "unit": "tok/s",
                          "path": "per layer moe_layer_forward_chained (k_decode_scores with the norm + "
                                  "k_decode_experts), graph of the same tokens"},
        "moe_calls_gbs": round((expert_bytes + router_bytes) / (moe_ms_per_token * 1e-3) / 1e9, 1),
        "popularity": {"rank_frequency_slope": slope, "routes_by_rank": [int(v) for v in by_rank[:16]],
                       "routes": int(by_rank.sum())},
        "setup_s": round(gen_s, 1),
    }


# ---------------------------------------------------------------- variants of the layer

MFMA_I8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA, vendor figure


def run_variants(args, check):
    """The layer's variants on the Xing4 and prefill shapes, each timed and checked against the oracle:
    the sigmoid-gated shared expert (decode, T=1), the W4A8 contract (Q8_0 activations; T=1, T=128 and the
    T=2048 prefill call), a dense FFN block of the same model (hidden 3584, FFN 9216; T=1) and the Xing4
    layer with IQ4_XS and packed 3-bit experts (T=1, T=128)."""
    import torch

    import quantized_moe_decode_sigmoid_amd as qm
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()
    res = {}
    oracle = None
    if not args.no_cpu:
        import oracle
    n_place, n_tok = 16, 400

    def timed_graph(fn, reps):
        """Capture fn() once, replay it `reps` times with events on the launching stream; ms per replay."""
        with torch.cuda.stream(stream):
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                fn()
            g.replay()
            torch.cuda.synchronize()
            total, per = timed_steps(torch, stream, g.replay, reps)
        return total / reps, per

    t0 = time.time()
    shape = synth.WORKLOADS["xing4"]
    H, E, K, F = shape.hidden, shape.n_experts, shape.top_k, shape.ffn
    inp = synth.layer_inputs(shape)
    row = synth.shared_gate_row(shape)
    x_bits = synth.tokens(shape, n_tok, first=20000)
    x = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    base = qm.DeviceLayer(qm.make_config(H, F, E, K), inp["gate_w"], None, inp["arena"], inp["shared"])
    gw1 = torch.from_numpy(np.concatenate([inp["gate_w"], row[None, :]])).to(dev)
    places = [(gw1.clone(), base.arena.clone(), base.shared.clone()) for _ in range(n_place)]
    eb = qm.moe_expert_bytes(base.cfg)
    log(f"variants: inputs ready, {time.time() - t0:.0f} s")

    def decode_sweep(cfg, out, ids, wts, ws, gate_rows):
        def fn():
            for i in range(n_tok):
                g, a, sh = places[i % n_place]
                qm.moe_layer_forward(cfg, 1, x[i:i + 1], g[:gate_rows], None, a, sh, out[i:i + 1], ids[i:i + 1],
                                     wts[i], ws)
        return fn

    n_chk = 16
    # 1. gated shared expert, decode plan
    cfg = qm.make_config(H, F, E, K, shared_gate=1)
    out = torch.empty((n_tok, H), dtype=torch.float32, device=dev)
    ids = torch.empty((n_tok, K), dtype=torch.int32, device=dev)
    wts = torch.empty((n_tok, 8), dtype=torch.float32, device=dev)  # K + 1 values per token, rows 16-byte aligned
    ws = torch.empty(qm.moe_workspace_bytes(cfg, 1), dtype=torch.uint8, device=dev)
    qm.moe_workspace_init(cfg, 1, ws)
    ms, per = timed_graph(decode_sweep(cfg, out, ids, wts, ws, E + 1), args.steps)
    call_us = ms * 1e3 / n_tok
    nbytes = (K + 1) * eb + (E + 1) * H * 4 + H * 6
    gated = {"workload": "xing4 decode, T=1, shared expert scaled by sigmoid(x . gate_w[E])",
             "tok_s": round(n_tok / (ms * 1e-3), 1), "avg_us": round(call_us, 3), "step_spread": spread(per),
             "roofline": {"bound": "hbm", "achieved": round(nbytes / call_us / 1e3, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(nbytes / call_us / 1e3 / HBM_PEAK_GBS, 4),
                          "bytes_per_launch": nbytes}}
    if oracle is not None:
        want, rid, rw = oracle.layer(x_bits[:n_chk], inp["gate_w"], inp["arena"], inp["shared"], K, F, 2.0,
                                     shared_gate=row)
        gated["parity"] = check.compare("variants.gated", out[:n_chk].cpu().numpy(), want, ids[:n_chk].cpu().numpy(),
                                        rid, wts[:n_chk, :K].cpu().numpy(), rw)
    gated["parity"] = dict(gated.get("parity") or {}, status_word=check.status("variants.gated",
                                                                              status_word(torch, qm, cfg, 1, ws)))
    res["gated_shared_expert"] = gated
    log("variants: gated done")

    # 2. W4A8, T = 1 (multi-kernel plan) and T = 128
    w8 = {}
    cfg = qm.make_config(H, F, E, K, precision=qm.PREC_W4A8)
    wts = torch.empty((n_tok, K), dtype=torch.float32, device=dev)
    ws = torch.empty(qm.moe_workspace_bytes(cfg, 128), dtype=torch.uint8, device=dev)
    ms, per = timed_graph(decode_sweep(cfg, out, ids, wts, ws, E), args.steps)
    call_us = ms * 1e3 / n_tok
    nbytes = (K + 1) * eb + E * H * 4 + H * 6
    w8["decode_t1"] = {"tok_s": round(n_tok / (ms * 1e-3), 1), "avg_us": round(call_us, 3),
                       "step_spread": spread(per),
                       "roofline": {"bound": "hbm", "achieved": round(nbytes / call_us / 1e3, 1),
                                    "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                    "frac": round(nbytes / call_us / 1e3 / HBM_PEAK_GBS, 4)}}
    if oracle is not None:
        want, rid, rw = oracle.layer(x_bits[:n_chk], inp["gate_w"], inp["arena"], inp["shared"], K, F, 2.0,
                                     mode=oracle.W4A8)
        w8["decode_t1"]["parity"] = check.compare("variants.w4a8_t1", out[:n_chk].cpu().numpy(), want,
                                                  ids[:n_chk].cpu().numpy(), rid, wts[:n_chk].cpu().numpy(), rw)
    Tb = 128
    it = [0]

    def batch_call():
        g, a, sh = places[it[0] % n_place]
        it[0] += 1
        qm.moe_layer_forward(cfg, Tb, x[:Tb], g[:E], None, a, sh, out[:Tb], ids[:Tb], wts[:Tb], ws)

    with torch.cuda.stream(stream):
        for _ in range(4):
            batch_call()
        torch.cuda.synchronize()
        total, per = timed_steps(torch, stream, batch_call, max(args.steps, 8))
    call_us = total * 1e3 / max(args.steps, 8)
    touched = int((np.bincount(ids[:Tb].cpu().numpy().reshape(-1), minlength=E) > 0).sum())
    nbytes = (touched + 1) * eb + E * H * 4 + Tb * H * 6
    w8["batch_t128"] = {"tok_s": round(Tb / (call_us * 1e-6), 1), "avg_us": round(call_us, 3),
                        "step_spread": spread(per),
                        "roofline": {"bound": "hbm", "achieved": round(nbytes / call_us / 1e3, 1),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(nbytes / call_us / 1e3 / HBM_PEAK_GBS, 4)}}
    if oracle is not None:
        want, rid, rw = oracle.layer(x_bits[:Tb], inp["gate_w"], inp["arena"], inp["shared"], K, F, 2.0,
                                     mode=oracle.W4A8)
        w8["batch_t128"]["parity"] = check.compare("variants.w4a8_t128", out[:Tb].cpu().numpy(), want,
                                                   ids[:Tb].cpu().numpy(), rid, wts[:Tb].cpu().numpy(), rw)
    del places, base
    torch.cuda.empty_cache()
    log("variants: w4a8 decode and batch done")

    # W4A8 at the prefill shape, T = 2048
    pshape = synth.WORKLOADS["prefill"]
    lam = synth.zipf_lambda(pshape)
    pin = synth.layer_inputs(pshape, lam=lam)
    Tp, Hp, Ep, Kp, Fp = pshape.tokens, pshape.hidden, pshape.n_experts, pshape.top_k, pshape.ffn
    px_bits = synth.tokens(pshape, Tp)
    px = torch.from_numpy(px_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    pcfg = qm.make_config(Hp, Fp, Ep, Kp, precision=qm.PREC_W4A8)
    pdl = qm.DeviceLayer(pcfg, pin["gate_w"], pin["bias"], pin["arena"], pin["shared"])
    pout = torch.empty((Tp, Hp), dtype=torch.float32, device=dev)
    pids = torch.empty((Tp, Kp), dtype=torch.int32, device=dev)
    pw = torch.empty((Tp, Kp), dtype=torch.float32, device=dev)
    pws = pdl.workspace(Tp)
    with torch.cuda.stream(stream):
        qm.moe_layer_forward(pcfg, Tp, px, pdl.gate_w, pdl.bias, pdl.arena, pdl.shared, pout, pids, pw, pws)
        torch.cuda.synchronize()

        def pffn():
            qm.moe_expert_forward(pcfg, Tp, px, pids, pw, pdl.arena, pdl.shared, pout, pws)
        pffn()
        torch.cuda.synchronize()
        total, per = timed_steps(torch, stream, pffn, max(args.steps, 5))
    ffn_us = total * 1e3 / max(args.steps, 5)
    ops = 2.0 * 3 * Hp * Fp * (Tp * Kp + Tp)
    w8["prefill_t2048"] = {"ffn_us": round(ffn_us, 3), "tops": round(ops / (ffn_us * 1e-6) / 1e12, 2),
                           "int8_mfma_frac": round(ops / (ffn_us * 1e-6) / 1e12 / MFMA_I8_PEAK_TOPS, 4),
                           "step_spread": spread(per),
                           "note": "moe_expert_forward W4A8 (quantize x, gate/up, quantize h, down, combine); int8 "
                                   "MFMA peak 5.0 POP/s"}
    if oracle is not None:
        n = 64
        want, rid, rw = oracle.layer(px_bits[:n], pin["gate_w"], pin["arena"], pin["shared"], Kp, Fp, 2.0, pin["bias"],
                                     oracle.W4A8)
        w8["prefill_t2048"]["parity"] = check.compare("variants.w4a8_prefill", pout[:n].cpu().numpy(), want,
                                                      pids[:n].cpu().numpy(), rid, pw[:n].cpu().numpy(), rw)
    res["w4a8"] = w8
    del pdl, pws
    torch.cuda.empty_cache()
    log("variants: w4a8 prefill done")

    # 3. dense FFN block, T = 1 (exact weights, multi-kernel plan)
    dshape = synth.WORKLOADS["dense"]
    dinp = synth.layer_inputs(dshape)
    dcfg = qm.make_config(dshape.hidden, dshape.ffn, 0, 0, 1, 1.0)
    ddl = qm.DeviceLayer(dcfg, None, None, None, dinp["shared"])
    dplaces = [ddl.shared.clone() for _ in range(8)]
    dx_bits = synth.tokens(dshape, 200, first=30000)
    dx = torch.from_numpy(dx_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    dout = torch.empty((200, dshape.hidden), dtype=torch.float32, device=dev)
    dws = ddl.workspace(1)

    def dense_sweep():
        for i in range(200):
            qm.moe_layer_forward(dcfg, 1, dx[i:i + 1], None, None, None, dplaces[i % 8], dout[i:i + 1], ws=dws)

    ms, per = timed_graph(dense_sweep, args.steps)
    call_us = ms * 1e3 / 200
    deb = qm.moe_expert_bytes(dcfg)
    nbytes = deb + dshape.hidden * 6
    dense = {"workload": "dense FFN block, T=1: hidden 3584, FFN 9216, IQ4_NL, 8 placements cycled",
             "tok_s": round(200 / (ms * 1e-3), 1), "avg_us": round(call_us, 3), "step_spread": spread(per),
             "roofline": {"bound": "hbm", "achieved": round(nbytes / call_us / 1e3, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(nbytes / call_us / 1e3 / HBM_PEAK_GBS, 4),
                          "bytes_per_launch": nbytes}}
    if oracle is not None:
        want, _, _ = oracle.layer(dx_bits[:8], np.zeros((0, dshape.hidden), np.float32), None, dinp["shared"], 0,
                                  dshape.ffn, 1.0)
        dense["parity"] = check.compare("variants.dense", dout[:8].cpu().numpy(), want)
    res["dense_ffn"] = dense
    del ddl, dplaces
    torch.cuda.empty_cache()
    log("variants: dense done")

    # 4. the other expert codecs on the Xing4 layer: T = 1 and T = 128 (exact weights, multi-kernel plan)
    codecs = {}
    for name in ("xing4_xs", "xing4_q3"):
        cs = synth.WORKLOADS[name]
        cinp = synth.layer_inputs(cs)
        ccfg = qm.make_config(H, F, E, K, codec=cs.codec)
        cdl = qm.DeviceLayer(ccfg, cinp["gate_w"], None, cinp["arena"], cinp["shared"])
        cplaces = [(cdl.gate_w.clone(), cdl.arena.clone(), cdl.shared.clone()) for _ in range(n_place)]
        cx_bits = synth.tokens(cs, n_tok, first=40000)
        cx = torch.from_numpy(cx_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        cws = torch.empty(qm.moe_workspace_bytes(ccfg, 128), dtype=torch.uint8, device=dev)
        ceb = qm.moe_expert_bytes(ccfg)

        def csweep():
            for i in range(n_tok):
                g, a, sh = cplaces[i % n_place]
                qm.moe_layer_forward(ccfg, 1, cx[i:i + 1], g, None, a, sh, out[i:i + 1], ids[i:i + 1], wts[i:i + 1],
                                     cws)

        ms, per = timed_graph(csweep, args.steps)
        call_us = ms * 1e3 / n_tok
        nbytes = (K + 1) * ceb + E * H * 4 + H * 6
        entry = {"expert_bytes": ceb, "packed_expert_bytes": qm.moe_packed_expert_bytes(ccfg),
                 "decode_t1": {"tok_s": round(n_tok / (ms * 1e-3), 1), "avg_us": round(call_us, 3),
                               "step_spread": spread(per),
                               "roofline": {"bound": "hbm", "achieved": round(nbytes / call_us / 1e3, 1),
                                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                            "frac": round(nbytes / call_us / 1e3 / HBM_PEAK_GBS, 4),
                                            "bytes_per_launch": nbytes}}}
        if oracle is not None:
            want, rid, rw = oracle.layer(cx_bits[:n_chk], cinp["gate_w"], cinp["arena"], cinp["shared"], K, F, 2.0,
                                         codec=cs.codec)
            entry["decode_t1"]["parity"] = check.compare(f"variants.{name}_t1", out[:n_chk].cpu().numpy(), want,
                                                         ids[:n_chk].cpu().numpy(), rid, wts[:n_chk, :K].cpu().numpy(),
                                                         rw)
        itc = [0]

        def cbatch():
            g, a, sh = cplaces[itc[0] % n_place]
            itc[0] += 1
            qm.moe_layer_forward(ccfg, 128, cx[:128], g, None, a, sh, out[:128], ids[:128], wts[:128, :K], cws)

        with torch.cuda.stream(stream):
            for _ in range(4):
                cbatch()
            torch.cuda.synchronize()
            total, per = timed_steps(torch, stream, cbatch, max(args.steps, 8))
        call_us = total * 1e3 / max(args.steps, 8)
        touched = int((np.bincount(ids[:128].cpu().numpy().reshape(-1), minlength=E) > 0).sum())
        nbytes = (touched + 1) * ceb + E * H * 4 + 128 * H * 6
        entry["batch_t128"] = {"tok_s": round(128 / (call_us * 1e-6), 1), "avg_us": round(call_us, 3),
                               "step_spread": spread(per),
                               "roofline": {"bound": "hbm", "achieved": round(nbytes / call_us / 1e3, 1),
                                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                            "frac": round(nbytes / call_us / 1e3 / HBM_PEAK_GBS, 4)}}
        codecs[name] = entry
        del cdl, cplaces
        torch.cuda.empty_cache()
        log(f"variants: {name} done")
    res["codecs"] = codecs
    return res


# ---------------------------------------------------------------- main

LEGS = {"decode": run_decode, "prefill": run_prefill, "batch": run_batch, "stack": run_stack,
        "variants": run_variants}
NESTED = ("prefill", "batch", "stack", "variants")


def brief(line):
    """A nested leg: its own line without the keys the top level already carries."""
    return {k: v for k, v in line.items() if k not in ("metric", "n_gpus", "higher_is_better", "scaling", "data")}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU (every workload here fits one MI355X); "
                                   "--gpus must be 1"}))
        sys.exit(2)
    if args.copy_mb > 0:
        copy_calibration(args.copy_mb)
    check = Check()
    if args.workload == "variants":
        line = {"variants": run_variants(args, check)}
    elif args.workload != "all":
        line = LEGS[args.workload](args, check)
    else:
        import torch
        log("decode")
        line = run_decode(args, check)
        torch.cuda.empty_cache()
        for leg in NESTED:
            log(leg)
            try:
                r = LEGS[leg](args, check)
                line[leg] = r if leg == "variants" else brief(r)
            except Exception as e:  # the line is still printed; the exit status reports it
                line[leg] = {"error": f"{type(e).__name__}: {e}"}
                check.failures.append(f"{leg}: {type(e).__name__}: {e}")
            torch.cuda.empty_cache()
    line["checks"] = {"ok": not check.failures, "failures": check.failures}
    print(json.dumps(line), flush=True)
    if check.failures:
        sys.exit(1)


if __name__ == "__main__":
    main()
