"""Benchmark of the quantized MoE layer on one MI355X.

Workload (the headline decode configuration): one Xing4.0-29B-A4B MoE layer --
hidden 3584, 64 routed experts top-4 + 1 shared, expert_ffn 1024, sigmoid router,
routed_scaling 2.0, IQ4_NL experts -- decoding 1000 independent tokens, T=1 per call.
The layer is placed 32 times in HBM (12.9 GB) and token i uses placement i mod 32, so
the 256 MB last-level cache cannot serve one token's expert reads from an earlier
token's.  A step is the 1000-token sweep, captured once as a HIP graph and replayed.

Printed JSON line: tok/s for the whole sweep; the roofline of one layer call (two
launches per token: k_decode_scores, the router logits and sigmoids, then
k_decode_experts, the selection, the five expert FFNs and the combine) from the HIP
events around the timed region divided by the layer calls in it (HIP events around
each eager call, with the stream kept busy so that host launch time does not enter,
are reported beside it); the CPU oracle timed on a bounded sample of the same tokens.
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
N_TOKENS = 1000
PLACEMENTS = 32


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--workload", choices=["decode", "prefill", "stack", "batch"], default="decode",
                   help="decode: the headline T=1 line (default); prefill: one T=2048 layer call per step; "
                        "stack: 38 chained layers per step, T=1; batch: one T=128 Xing4 layer call per step")
    p.add_argument("--stack-layers", type=int, default=38, help="layers of the stack workload")
    p.add_argument("--stack-tokens", type=int, default=20,
                   help="distinct tokens captured in the stack graph (steps per replay)")
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--distinct-layers", type=int, default=4,
                   help="distinct seeded layers generated; placements reuse them at distinct addresses")
    p.add_argument("--cpu-sample", type=int, default=None,
                   help="tokens the CPU oracle runs (0: skip; default: about 10 s of oracle work, 60 decode tokens, "
                        "400 prefill tokens, the whole 128-token batch)")
    p.add_argument("--no-graph", action="store_true", help="replay eagerly instead of through a HIP graph")
    p.add_argument("--copy-mb", type=int, default=0,
                   help="first run one plain device copy of this many MiB (a kernel of known traffic, to scale "
                        "the HBM byte counters of a profiler run)")
    return p.parse_args()


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure


def measured_traffic(record):
    """HBM bytes per launch from the committed counter summary, or None when the counted kernel source
    has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", record)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    sources = rec["kernel_sources"] if "kernel_sources" in rec else [rec["kernel_source"]]
    hashes = rec["sha256"] if isinstance(rec["sha256"], list) else [rec["sha256"]]
    for src, sha in zip(sources, hashes):
        with open(os.path.join(ROOT, src), "rb") as f:
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
    for _ in range(3):
        a, b, c = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        a.record()
        qm.moe_stream_read(src, nbytes, sink)
        b.record()
        dst.copy_(src[: 1 << 28])
        c.record()
        torch.cuda.synchronize()
        read_s.append(a.elapsed_time(b) / 1e3)
        copy_s.append(b.elapsed_time(c) / 1e3)
    del src, dst
    return {"read_gbs": round(nbytes / min(read_s) / 1e9, 1), "copy_gbs": round(2 * (1 << 30) / min(copy_s) / 1e9, 1),
            "read_kernel": "moe_stream_read, 4 GiB", "copy": "torch copy_, 1 GiB"}


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


CPU_SAMPLE = {"decode": 60, "prefill": 400, "batch": 128, "stack": 0}


def main():
    args = parse()
    if args.cpu_sample is None:
        args.cpu_sample = CPU_SAMPLE[args.workload]
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU; --gpus must be 1"}))
        sys.exit(2)
    if args.copy_mb > 0:
        copy_calibration(args.copy_mb)
    if args.workload == "prefill":
        run_prefill(args)
    elif args.workload == "stack":
        run_stack(args)
    elif args.workload == "batch":
        run_batch(args)
    else:
        run_decode(args)


def run_prefill(args):
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
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        layer_ms = ev0.elapsed_time(ev1) / args.steps
        # the expert FFN alone (bucketing, gate/up, down, combine) on the routing just computed
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda._sleep(50_000_000)
        for i in range(args.steps):
            starts[i].record(stream)
            qm.moe_expert_forward(cfg, T, x, ids, wts, dl.arena, dl.shared, out, ws)
            ends[i].record(stream)
        torch.cuda.synchronize()
    ffn_us = np.array([a.elapsed_time(b) * 1e3 for a, b in zip(starts, ends)])
    counts = np.bincount(ids.cpu().numpy().reshape(-1), minlength=E)
    flops = 2.0 * 3 * H * F * (T * K + T * shape.n_shared)
    # MFMA rows the 16-row sub-tiles execute per useful row (tiles of 128 routes of one expert)
    rows_useful = T * K + T * shape.n_shared
    rows_run = sum(16 * ((c + 15) // 16) for c in counts.tolist()) + 16 * ((T + 15) // 16) * shape.n_shared
    ffn_tflops = flops / (float(np.mean(ffn_us)) * 1e-6) / 1e12
    # algorithmic bytes of one moe_expert_forward call: every expert once (routed + shared), x, the
    # routing (ids + weights), the fp32 output
    ebytes = 3 * F * (H // 32) * 18
    ffn_bytes = (E + shape.n_shared) * ebytes + T * H * 2 + T * K * 8 + T * H * 4
    ffn_gbs = ffn_bytes / (float(np.mean(ffn_us)) * 1e-6) / 1e9

    cpu = None
    if args.cpu_sample > 0:
        import oracle
        n = args.cpu_sample
        c0 = time.time()
        oracle.layer(x_bits[:n], inp["gate_w"], inp["arena"], inp["shared"], K, F, shape.routed_scale, inp["bias"],
                     oracle.BF16 if prec == qm.PREC_BF16 else oracle.FP32)
        cs = time.time() - c0
        cpu = {"value": round(n / cs, 3), "unit": "tok/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"the first {n} of the {T} tokens in one oracle.layer call, {cs:.1f} s", **cpu_info()}

    res = {
        "metric": "MoE-layer decode tok/s + achieved HBM GB/s (% peak); prefill TFLOP/s (% MFMA)",
        "value": round(flops / (layer_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
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
        # The FFN needs every expert's weights once (more bytes than the 256 MB last-level cache), so its
        # HBM floor (bytes / 8 TB/s) is above its MFMA floor (flops / 2.5 PFLOP/s): it is HBM-bound.
        "roofline": {"bound": "hbm" if ffn_bytes / HBM_PEAK_GBS > flops / 1e3 / MFMA_BF16_PEAK_TFLOPS else "mfma",
                     "achieved": round(ffn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ffn_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("prefill_traffic.json"),
                     "kernel": "moe_expert_forward bf16: k_bucket + k_gate_up_bf16 + k_down_bf16 + k_combine "
                               "(events around the call)",
                     "bytes_per_launch": ffn_bytes, "flops_per_launch": flops,
                     "mfma_tflops": round(ffn_tflops, 2), "mfma_frac": round(ffn_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "hbm_floor_us": round(ffn_bytes / HBM_PEAK_GBS / 1e3, 2),
                     "mfma_floor_us": round(flops / 1e6 / MFMA_BF16_PEAK_TFLOPS, 2),
                     "avg_us": round(float(np.mean(ffn_us)), 3)},
        "cpu_baseline": cpu,
        "tok_s": round(T / (layer_ms * 1e-3), 1),
        "routes_per_expert": {"max": int(counts.max()), "min": int(counts.min()),
                              "median": float(np.median(counts))},
        "mfma_rows_per_useful_row": round(rows_run / rows_useful, 4),
        "first_step_ms": round(first_ms, 3),
        "setup_s": round(gen_s, 1),
    }
    print(json.dumps(res), flush=True)


def run_batch(args):
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

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        def step(i):
            g, a, sh = places[i % n_place]
            qm.moe_layer_forward(cfg, T, x, g, None, a, sh, out, ids, wts, ws)

        for i in range(max(args.warmup, n_place)):
            step(i)
        torch.cuda.synchronize()
        n_steps = max(args.steps, n_place)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(n_steps):
            step(i)
        ev1.record(stream)
        torch.cuda.synchronize()
        layer_ms = ev0.elapsed_time(ev1) / n_steps
        # events around each call, queued behind a spin kernel so that host launch time does not enter
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_steps)]
        torch.cuda._sleep(50_000_000)
        for i in range(n_steps):
            starts[i].record(stream)
            step(i)
            ends[i].record(stream)
        torch.cuda.synchronize()
    call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in zip(starts, ends)])
    counts = np.bincount(ids.cpu().numpy().reshape(-1), minlength=E)
    touched = int((counts > 0).sum())
    eb = qm.moe_expert_bytes(cfg)
    # algorithmic bytes of one call: each expert the batch routes to once, the shared expert, the router
    # weight, x, the fp32 output
    call_bytes = (touched + shape.n_shared) * eb + E * H * 4 + T * H * 2 + T * H * 4
    # one call's duration over the timed region (events bracketing the calls, divided by them)
    gbs = call_bytes / (layer_ms * 1e-3) / 1e9

    cpu = None
    if args.cpu_sample > 0:
        import oracle
        n = min(args.cpu_sample, T)
        c0 = time.time()
        oracle.layer(x_bits[:n], inp["gate_w"], inp["arena"], inp["shared"], K, F, shape.routed_scale, None,
                     oracle.BF16 if prec == qm.PREC_BF16 else oracle.FP32)
        cs = time.time() - c0
        cpu = {"value": round(n / cs, 3), "unit": "tok/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"the first {n} of the {T} tokens in one oracle.layer call, {cs:.1f} s", **cpu_info()}

    res = {
        "metric": "MoE-layer decode tok/s + achieved HBM GB/s (% peak); prefill TFLOP/s (% MFMA)",
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
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic("batch_traffic.json"),
                     "kernel": "moe_layer_forward T=128: router, top-k, bucketing, gate/up, down, combine "
                               "(HIP events around the timed region, divided by the calls in it)",
                     "bytes_per_launch": call_bytes, "avg_us": round(layer_ms * 1e3, 3),
                     "per_call_events": {"avg_us": round(float(np.mean(call_us)), 3),
                                         "median_us": round(float(np.median(call_us)), 3),
                                         "note": "calls with HIP events around each"}},
        "cpu_baseline": cpu,
        "experts_touched": touched,
        "routes_per_expert": {"max": int(counts.max()), "min": int(counts.min()),
                              "median": float(np.median(counts))},
        "setup_s": round(gen_s, 1),
    }
    print(json.dumps(res), flush=True)


def chain(qm, x, out, y):
    """Next layer's input into y: bf16(rmsnorm(x + out)), eps 1e-6, no weight (the chaining that stands in for
    the rest of a decoder block; not part of the MoE layer), one fused kernel of the library."""
    qm.moe_residual_rmsnorm(out, x, y, eps=1e-6)
    return y


def run_stack(args):
    """38 MoE layers of the Xing4 shape resident in HBM, one token per step (T=1) through all of them,
    each layer's input chained from the previous layer's output; Zipf(1.1) expert popularity."""
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
    layers = []
    for l in range(nl):
        inp = synth.layer_inputs(shape, layer=l, lam=lam)
        layers.append(qm.DeviceLayer(cfg, inp["gate_w"], inp["bias"], inp["arena"], inp["shared"]))
        del inp
    torch.cuda.synchronize()
    gen_s = time.time() - t0
    S = args.stack_tokens
    x_bits = synth.tokens(shape, S, first=7000)
    x0 = torch.from_numpy(x_bits.view(np.int16).copy()).view(torch.bfloat16).to(dev)
    ws = layers[0].workspace(1)
    outs = [torch.empty((1, H), dtype=torch.float32, device=dev) for _ in range(nl)]
    xs = [torch.empty((1, H), dtype=torch.bfloat16, device=dev) for _ in range(nl)]
    ids = torch.empty((S, nl, K), dtype=torch.int32, device=dev)
    wts = torch.empty((S, nl, K), dtype=torch.float32, device=dev)

    def steps():
        for i in range(S):
            x = x0[i:i + 1]
            for l, dl in enumerate(layers):
                qm.moe_layer_forward(cfg, 1, x, dl.gate_w, dl.bias, dl.arena, dl.shared, outs[l], ids[i, l],
                                     wts[i, l], ws)
                x = chain(qm, x, outs[l], xs[l])

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
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(args.steps):
            graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        # the MoE layer calls alone: events around each call of one eager pass over the S tokens, the
        # queue kept busy by a spin kernel so that host launch gaps do not enter
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(S * nl)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(S * nl)]
        torch.cuda._sleep(200_000_000)
        for i in range(S):
            x = x0[i:i + 1]
            for l, dl in enumerate(layers):
                starts[i * nl + l].record(stream)
                qm.moe_layer_forward(cfg, 1, x, dl.gate_w, dl.bias, dl.arena, dl.shared, outs[l], ids[i, l],
                                     wts[i, l], ws)
                ends[i * nl + l].record(stream)
                x = chain(qm, x, outs[l], xs[l])
        torch.cuda.synchronize()
    ms_per_token = ev0.elapsed_time(ev1) / (args.steps * S)
    moe_ms_per_token = sum(a.elapsed_time(b) for a, b in zip(starts, ends)) / S
    eb = qm.moe_expert_bytes(cfg)
    expert_bytes = nl * (K + shape.n_shared) * eb
    router_bytes = nl * E * H * 4
    # rank-frequency: each layer's expert counts sorted (layers rank their experts differently), summed by rank
    ids_h = ids.cpu().numpy()
    by_rank = np.zeros(E, np.int64)
    for l in range(nl):
        by_rank += np.sort(np.bincount(ids_h[:, l, :].reshape(-1), minlength=E))[::-1]
    counts = by_rank
    c = by_rank.astype(np.float64)
    c = c[c > 0]
    slope = float(np.polyfit(np.log(np.arange(1, c.size + 1)), np.log(c), 1)[0]) if c.size > 1 else None
    gbs = (expert_bytes + router_bytes) / (ms_per_token * 1e-3) / 1e9
    res = {
        "metric": "MoE-layer decode tok/s + achieved HBM GB/s (% peak); prefill TFLOP/s (% MFMA)",
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
                   "layers": nl, "distinct_tokens": S, "zipf_lambda": lam, "graph": True},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "whole step: per layer k_decode_scores + k_decode_experts + k_residual_rmsnorm",
                     "bytes_per_token": expert_bytes + router_bytes},
        "expert_bytes_per_token": expert_bytes,
        "moe_calls_ms_per_token": round(moe_ms_per_token, 4),
        "moe_calls_gbs": round((expert_bytes + router_bytes) / (moe_ms_per_token * 1e-3) / 1e9, 1),
        "popularity": {"rank_frequency_slope": slope, "routes_by_rank": [int(v) for v in by_rank[:16]],
                       "routes": int(by_rank.sum())},
        "setup_s": round(gen_s, 1),
    }
    print(json.dumps(res), flush=True)


def run_decode(args):
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
        sweep()  # eager warm-up outside the graph (also the first-call figure)
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
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t_wall = time.time()
        ev0.record(stream)
        for _ in range(args.steps):
            run()
        ev1.record(stream)
        torch.cuda.synchronize()
        wall_s = time.time() - t_wall
        total_ms = ev0.elapsed_time(ev1)

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
    ffn_us = np.array([s.elapsed_time(e) * 1e3 for s, e in zip(starts, ends)])

    ms_per_step = total_ms / args.steps
    tok_s = N_TOKENS / (ms_per_step / 1e3)
    expert_bytes_per_token = (K + shape.n_shared) * eb
    # algorithmic bytes of one layer launch (T=1): 5 experts, router weight, x, out
    layer_bytes = expert_bytes_per_token + E * H * 4 + H * 2 + H * 4
    # one layer call's duration over the timed region: the events bracketing the
    # graph replays, divided by the calls they hold (the per-call events of the
    # eager leg also hold the gap an event record adds between calls)
    call_us = ms_per_step * 1e3 / N_TOKENS
    achieved = layer_bytes / (call_us / 1e6) / 1e9

    cpu = None
    if args.cpu_sample > 0:
        import oracle
        n = args.cpu_sample
        c0 = time.time()
        for i in range(n):
            l = layers[(i % PLACEMENTS) % distinct]
            oracle.layer(x_bits[i:i + 1], l["gate_w"], l["arena"], l["shared"], K, F, shape.routed_scale)
        cs = time.time() - c0
        cpu = {"value": round(n / cs, 3), "unit": "tok/s", "cores": oracle.threads(), "kind": "oracle",
               "sample": f"{n} of the {N_TOKENS} tokens, one oracle.layer call (T=1) each, {cs:.1f} s", **cpu_info()}
    box = stream_gbs(torch)

    res = {
        "metric": "MoE-layer decode tok/s + achieved HBM GB/s (% peak); prefill TFLOP/s (% MFMA)",
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
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("decode_traffic.json"),
                     "kernel": "moe_layer_forward T=1: k_decode_scores + k_decode_experts (HIP events around the "
                               "timed region of graph replays, divided by the layer calls in it)",
                     "bytes_per_launch": layer_bytes, "avg_us": round(call_us, 3),
                     "per_call_events": {"avg_us": round(float(np.mean(ffn_us)), 3),
                                         "median_us": round(float(np.median(ffn_us)), 3),
                                         "note": "eager calls with HIP events around each"},
                     "box_stream": box, "frac_of_box_read": round(achieved / box["read_gbs"], 4)},
        "cpu_baseline": cpu,
        "layer_gbs": round(layer_bytes * tok_s / 1e9, 1),
        "first_step_ms": round(first_ms, 3),
        "wall_s": round(wall_s, 3),
        "setup_s": round(gen_s, 1),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
