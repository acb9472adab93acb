"""moe_layer_forward_noalloc: the layer on the library's own per-GPU scratch, against moe_layer_forward.

Same kernels on the same inputs, so the outputs and the routing must be identical bit for bit; two calls in
a row (the second with fewer tokens) check that nothing left in the shared scratch leaks into the next call;
a call above the scratch limit is refused before anything runs.
"""
import numpy as np
import pytest

import synth
from tests.gpu_util import cfg_of, to_dev_bf16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

import quantized_moe_decode_sigmoid_amd as qm  # noqa: E402


def run_both(dl, s, x_bits):
    T = x_bits.shape[0]
    xd = to_dev_bf16(x_bits)
    outs = []
    for fn in ("ws", "noalloc"):
        out = torch.full((T, s.hidden), float("nan"), dtype=torch.float32, device="cuda")
        ids = torch.full((T, s.top_k), -1, dtype=torch.int32, device="cuda")
        w = torch.full((T, s.top_k), float("nan"), dtype=torch.float32, device="cuda")
        if fn == "ws":
            qm.moe_layer_forward(dl.cfg, T, xd, dl.gate_w, dl.bias, dl.arena, dl.shared, out, ids, w,
                                 ws=dl.workspace(T))
        else:
            qm.moe_layer_forward_noalloc(dl.cfg, T, xd, dl.gate_w, dl.bias, dl.arena, dl.shared, out, ids, w)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()))
    (a, ia, wa), (b, ib, wb) = outs
    assert np.all(np.isfinite(b))
    assert np.array_equal(ia, ib)
    assert np.array_equal(wa.view(np.uint32), wb.view(np.uint32))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("name,sizes", [("xing4", (128, 1)), ("tiny", (37, 4)), ("xing4", (1, 1))])
def test_noalloc_equals_workspace_call_twice(name, sizes):
    """Two calls in a row on one GPU's scratch, the second with fewer tokens (batched FP32 plan then the
    two-launch decode plan on the Xing4 layer; the tiny layer's multi-kernel plan twice; decode twice)."""
    s = synth.WORKLOADS[name]
    inp = synth.layer_inputs(s)
    dl = qm.DeviceLayer(cfg_of(s), inp["gate_w"], None, inp["arena"], inp["shared"])
    for i, T in enumerate(sizes):
        print(f"[case] noalloc {name} call {i} T={T}", flush=True)
        run_both(dl, s, synth.tokens(s, T, first=100 * i + T))


def test_noalloc_bf16_plan_and_refusal_above_the_limit():
    """The BF16 plan (prefill shape, T = 300) through the scratch, then a call whose workspace exceeds the
    64 MiB scratch (T = 2048 of the prefill shape) is refused with MOE_EWORKSPACE and writes nothing."""
    s = synth.WORKLOADS["prefill"]
    inp = synth.layer_inputs(s)
    dl = qm.DeviceLayer(cfg_of(s), inp["gate_w"], None, inp["arena"], inp["shared"])
    print("[case] noalloc prefill T=300", flush=True)
    run_both(dl, s, synth.tokens(s, 300, first=9))
    T = 2048
    assert qm.moe_workspace_bytes(dl.cfg, T) > 64 << 20
    out = torch.full((T, s.hidden), 7.0, dtype=torch.float32, device="cuda")
    x = to_dev_bf16(synth.tokens(s, T))
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_layer_forward_noalloc(dl.cfg, T, x, dl.gate_w, None, dl.arena, dl.shared, out)
    assert ei.value.status == qm.MOE_EWORKSPACE
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
