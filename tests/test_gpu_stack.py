"""GPU tests of moe_stack_decode (the whole decode step of a stack of layers in one call: per layer the decode
plan's two launches, the layer's input formed in the first), through the C ABI: bit for bit against the chained per-layer
calls it replaces, against the CPU oracle layer by layer, under graph capture, and with the selection bias
absent or present."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_close, cfg_of, to_dev_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import quantized_moe_decode_sigmoid_amd as qm  # noqa: E402


def log(msg):
    print(f"[case] {msg}", flush=True)


_SETS = {}
_STACK = {}


def expert_sets():
    """The expert weights of 2 drawn layers of the stack workload, host and packed on the device."""
    if not _SETS:
        s = synth.WORKLOADS["stack"]
        lam = synth.zipf_lambda(s)
        cfg = cfg_of(s)
        sets = [synth.layer_inputs(s, layer=d, lam=lam) for d in range(2)]
        packed = [qm.DeviceLayer(cfg, st["gate_w"], None, st["arena"], st["shared"]) for st in sets]
        _SETS.update(lam=lam, sets=sets, packed=packed)
    return _SETS


def stack_layers(nl, with_bias=True):
    """nl layers of the stack workload: router weights and Zipf(1.1) selection bias per layer, the expert
    weights of 2 drawn layers placed per layer (as in bench.py); device layers and host arrays."""
    key = (nl, with_bias)
    if key not in _STACK:
        s = synth.WORKLOADS["stack"]
        cfg = cfg_of(s)
        es = expert_sets()
        layers, host = [], []
        for l in range(nl):
            gw = synth.gate_weights(s, layer=l)
            b = synth.zipf_bias(s, es["lam"], layer=l) if with_bias else None
            src = es["packed"][l % 2]
            layers.append(qm.DeviceLayer.from_packed(cfg, torch.from_numpy(gw).cuda(),
                                                     None if b is None else torch.from_numpy(b).cuda(),
                                                     src.arena, src.shared))
            host.append((gw, b, es["sets"][l % 2]))
        _STACK[key] = (s, cfg, layers, host)
    return _STACK[key]


def run_stack(cfg, layers, x0, nl, ws, s=None):
    s = s or synth.WORKLOADS["stack"]
    xs = torch.full((nl, s.hidden), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    outs = torch.full((nl, s.hidden), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((nl, s.top_k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((nl, s.top_k), float("nan"), dtype=torch.float32, device="cuda")
    arr = qm.stack_layers([(dl.gate_w, dl.bias, dl.arena, dl.shared) for dl in layers])
    qm.moe_stack_decode(cfg, nl, arr, x0, xs, outs, ids, w, ws)
    return xs, outs, ids, w


def run_chained(cfg, layers, x0, nl, s=None):
    s = s or synth.WORKLOADS["stack"]
    xs = torch.empty((nl, s.hidden), dtype=torch.bfloat16, device="cuda")
    outs = torch.empty((nl, s.hidden), dtype=torch.float32, device="cuda")
    kp = (s.top_k + 3) // 4 * 4  # rows 16-byte aligned, as the layer call's routing outputs must be
    ids = torch.empty((nl, kp), dtype=torch.int32, device="cuda")
    w = torch.empty((nl, kp), dtype=torch.float32, device="cuda")
    ws = layers[0].workspace(1)
    xs[0].copy_(x0[0])
    for l, dl in enumerate(layers):
        if l == 0:
            qm.moe_layer_forward(cfg, 1, xs[0:1], dl.gate_w, dl.bias, dl.arena, dl.shared, outs[0:1], ids[0], w[0], ws)
        else:
            qm.moe_layer_forward_chained(cfg, 1, xs[l - 1:l], outs[l - 1:l], xs[l:l + 1], dl.gate_w, dl.bias,
                                         dl.arena, dl.shared, outs[l:l + 1], ids[l], w[l], ws)
    return xs, outs, ids[:, :s.top_k], w[:, :s.top_k]


def stack_ws(cfg, nl):
    return torch.empty(qm.moe_stack_workspace_bytes(cfg, nl), dtype=torch.uint8, device="cuda")


def assert_stack_status_ok(cfg, nl, ws):
    st = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    qm.moe_stack_status(cfg, nl, ws, st)
    assert int(st[0].item()) == 0, "a wait of the stack kernel gave up"


def assert_same(a, b, what):
    for got, want, name in zip(a, b, ("x", "out", "ids", "w")):
        assert torch.equal(got.contiguous().view(torch.int8), want.contiguous().view(torch.int8)), f"{what}: {name}"


@pytest.mark.parametrize("nl,with_bias", [(1, True), (3, False), (38, True)])
def test_stack_decode_equals_chained_calls(nl, with_bias):
    """moe_stack_decode over nl layers against moe_layer_forward (layer 0) + moe_layer_forward_chained
    (layers 1..): every layer's input, output and routing identical bit for bit; the status word 0."""
    s, cfg, layers, _ = stack_layers(max(nl, 3), with_bias)
    layers = layers[:nl]
    for tok in (0, 1):
        x0 = to_dev_bf16(synth.tokens(s, 1, first=7000 + tok))
        ws = stack_ws(cfg, nl)
        log(f"stack decode L={nl} bias={with_bias} token={tok}")
        got = run_stack(cfg, layers, x0, nl, ws)
        want = run_chained(cfg, layers, x0, nl)
        torch.cuda.synchronize()
        assert_stack_status_ok(cfg, nl, ws)
        assert_same(got, want, f"L={nl} token {tok}")


def test_stack_decode_against_oracle():
    """The 38-layer step of the stack workload in one call: every layer's routing equals the oracle's on
    the GPU's input to that layer bit for bit and its output is within tolerance of the oracle's; every
    formed input is within one bf16 step of the oracle's norm of the previous layer's input and output."""
    nl = 38
    s, cfg, layers, host = stack_layers(nl, True)
    x0 = to_dev_bf16(synth.tokens(s, 1, first=9100))
    ws = stack_ws(cfg, nl)
    log("stack decode L=38 against the oracle")
    xs, outs, ids, w = run_stack(cfg, layers, x0, nl, ws)
    torch.cuda.synchronize()
    assert_stack_status_ok(cfg, nl, ws)
    xin = xs.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(xin[0], x0.view(torch.int16).cpu().numpy().view(np.uint16)[0])
    got, gid, gw_ = outs.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    for l in range(nl):
        if l % 8 == 0:
            log(f"stack decode oracle layer {l}")
        gwl, bl, st = host[l]
        ref, rid, rw = oracle.layer(xin[l:l + 1], gwl, st["arena"], st["shared"], s.top_k, s.ffn, s.routed_scale,
                                    bl)
        assert np.array_equal(gid[l:l + 1], rid), l
        assert np.array_equal(gw_[l:l + 1].view(np.uint32), rw.view(np.uint32)), l
        assert_close(got[l:l + 1], ref, f"stack decode layer {l}")
        if l + 1 < nl:
            y = oracle.residual_rmsnorm(xin[l:l + 1], got[l:l + 1])
            diff = np.abs(xin[l + 1:l + 2].astype(np.int32) - y.astype(np.int32))
            assert int(diff.max()) <= 1, l


def test_stack_decode_graph_replay():
    """moe_stack_decode for two tokens captured in one HIP graph, replayed 3 times with eager work in
    between (outputs poisoned before each replay): every replay equals the eager run bit for bit."""
    nl = 38
    s, cfg, layers, _ = stack_layers(nl, True)
    x0 = to_dev_bf16(synth.tokens(s, 2, first=9200))
    arr = qm.stack_layers([(dl.gate_w, dl.bias, dl.arena, dl.shared) for dl in layers])
    ws = stack_ws(cfg, nl)
    xs = torch.empty((2, nl, s.hidden), dtype=torch.bfloat16, device="cuda")
    outs = torch.empty((2, nl, s.hidden), dtype=torch.float32, device="cuda")
    ids = torch.empty((2, nl, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((2, nl, s.top_k), dtype=torch.float32, device="cuda")

    def step():
        for t in range(2):
            qm.moe_stack_decode(cfg, nl, arr, x0[t:t + 1], xs[t], outs[t], ids[t], w[t], ws)

    log("stack decode graph: eager")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step()
        torch.cuda.synchronize()
        eager = [a.clone() for a in (xs, outs, ids, w)]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for rep in range(3):
            log(f"stack decode graph: replay {rep}")
            for a in (xs, outs, w):
                a.fill_(float("nan"))
            ids.fill_(-1)
            graph.replay()
            torch.cuda.synchronize()
            assert_same((xs, outs, ids, w), eager, f"replay {rep}")
            _ = layers[rep].forward(x0[0:1])  # eager work between replays
            torch.cuda.synchronize()
    assert_stack_status_ok(cfg, nl, ws)


@pytest.mark.parametrize("nl", [1, 4])
def test_stack_decode_tiny_shape(nl):
    """The tiny shape (hidden 256, ffn 128, 8 experts top-2 + 1 shared: one 256-element router step, one
    packed down tile per row, 8 router rows in 8 shared workgroups), router weights, experts and Zipf
    selection biases drawn per layer: moe_stack_decode equals the chained calls bit for bit, and every
    layer's routing equals the oracle's on the GPU's input to that layer."""
    s = synth.WORKLOADS["tiny"]
    cfg = cfg_of(s)
    layers, host = [], []
    for l in range(nl):
        inp = synth.layer_inputs(s, layer=l)
        b = synth.zipf_bias(s, 0.05, layer=l)
        layers.append(qm.DeviceLayer(cfg, inp["gate_w"], torch.from_numpy(b).cuda(), inp["arena"], inp["shared"]))
        host.append((inp, b))
    for tok in (0, 1, 2):
        x0 = to_dev_bf16(synth.tokens(s, 1, first=300 + tok))
        ws = stack_ws(cfg, nl)
        log(f"stack decode tiny L={nl} token={tok}")
        got = run_stack(cfg, layers, x0, nl, ws, s)
        want = run_chained(cfg, layers, x0, nl, s)
        torch.cuda.synchronize()
        assert_stack_status_ok(cfg, nl, ws)
        assert_same(got, want, f"tiny L={nl} token {tok}")
        xin = got[0].view(torch.int16).cpu().numpy().view(np.uint16)
        gid = got[2].cpu().numpy()
        for l in range(nl):
            inp, b = host[l]
            _, rid, _ = oracle.layer(xin[l:l + 1], inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn,
                                     s.routed_scale, b)
            assert np.array_equal(gid[l:l + 1], rid), (tok, l)
