"""Host-side checks of the C ABI (no GPU needed: validation runs before any launch)."""
import ctypes
import os
import re

import pytest

import quantized_moe_decode_sigmoid_amd as qm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

XING4 = dict(hidden=3584, ffn=1024, n_experts=64, top_k=4, n_shared=1, routed_scale=2.0)
A = 0x10000  # fake, 16-byte aligned device addresses: never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert names == sorted(qm.EXPORTED)
    lib = ctypes.CDLL(qm.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_exports_nothing_else():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", qm.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = sorted({l.split()[-1] for l in out.splitlines() if l.split()[1] == "T"})
    assert exported == declared_functions()


def test_version_and_status_strings():
    assert qm.moe_abi_version() == 4
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert isinstance(qm.status_string(s), str) and qm.status_string(s)


def test_sizes_and_precision_rule():
    cfg = qm.make_config(**XING4)
    assert qm.moe_check_config(cfg) == 0
    assert qm.moe_expert_bytes(cfg) == 6193152  # the model card's per-expert figure
    assert qm.moe_resolved_precision(cfg, 1) == qm.PREC_FP32
    assert qm.moe_resolved_precision(cfg, 128) == qm.PREC_FP32   # 512 routes <= 16 * 64
    assert qm.moe_resolved_precision(cfg, 257) == qm.PREC_BF16
    pre = qm.make_config(2048, 512, 256, 8)
    assert qm.moe_expert_bytes(pre) == 1769472
    assert qm.moe_resolved_precision(pre, 2048) == qm.PREC_BF16
    assert qm.moe_workspace_bytes(cfg, 1) > 0
    assert qm.moe_workspace_bytes(cfg, 128) > qm.moe_workspace_bytes(cfg, 1)
    assert qm.moe_workspace_bytes(cfg, 0) > 0


def test_chained_layer_argument_errors():
    cfg = qm.make_config(**XING4)
    ws = qm.moe_workspace_bytes(cfg, 2)
    H = XING4["hidden"]

    def call(x_prev=A, out_prev=A + 0x100000, x=A + 0x200000, eps=1e-6, wsb=ws):
        with pytest.raises(qm.MoeError) as ei:
            qm.moe_layer_forward_chained(cfg, 2, x_prev, out_prev, x, A, None, A, A, A, ws=A + 0x400000, ws_bytes=wsb,
                                         eps=eps, stream=0)
        return ei.value.status

    assert call(x_prev=None) == qm.MOE_EINVAL
    assert call(out_prev=A + 8) == qm.MOE_EALIGN
    assert call(x=A + 2 * H) == qm.MOE_EINVAL              # overlaps x_prev's second row
    assert call(x=A + 0x100000 + 4 * H) == qm.MOE_EINVAL   # overlaps out_prev
    assert call(eps=-1.0) == qm.MOE_EINVAL
    assert call(eps=float("inf")) == qm.MOE_EINVAL
    assert call(wsb=ws - 1) == qm.MOE_EWORKSPACE


def test_stack_decode_argument_errors():
    """moe_stack_decode: the shapes it covers, its workspace size, and argument errors (all refused before
    any launch)."""
    cfg = qm.make_config(**XING4)
    n1, n38 = qm.moe_stack_workspace_bytes(cfg, 1), qm.moe_stack_workspace_bytes(cfg, 38)
    # one token's decode workspace, reused by every layer, plus every layer's routing outputs
    assert qm.moe_workspace_bytes(cfg, 1) <= n1 < n38 <= n1 + 2 * 38 * 8 * 4 + 512
    for bad, code in [(dict(), None), (dict(n_shared=0), None), (dict(shared_gate=1), None),
                      (dict(ffn=512), qm.MOE_EUNSUPPORTED),  # hidden > 4 ffn: not the decode plan's shape
                      (dict(top_k=5), qm.MOE_EUNSUPPORTED), (dict(hidden=4352), qm.MOE_EUNSUPPORTED),
                      (dict(n_experts=0, top_k=0), qm.MOE_EUNSUPPORTED)]:
        c = qm.make_config(**{**XING4, **bad})
        if code is None:
            assert qm.moe_stack_workspace_bytes(c, 4) > 0, bad
            continue
        with pytest.raises(qm.MoeError) as ei:
            qm.moe_stack_workspace_bytes(c, 4)
        assert ei.value.status == code, bad
    for L in (0, 65):
        with pytest.raises(qm.MoeError) as ei:
            qm.moe_stack_workspace_bytes(cfg, L)
        assert ei.value.status == qm.MOE_EUNSUPPORTED
    H = XING4["hidden"]
    L = 3
    good = qm.stack_layers([(A, None, A, A)] * L)

    def call(layers=good, x0=A, x_all=A + 0x100000, out_all=A + 0x200000, eps=1e-6, wsb=None):
        wsb = qm.moe_stack_workspace_bytes(cfg, L) if wsb is None else wsb
        with pytest.raises(qm.MoeError) as ei:
            qm.moe_stack_decode(cfg, L, layers, x0, x_all, out_all, ws=A + 0x400000, ws_bytes=wsb, eps=eps,
                                stream=0)
        return ei.value.status

    assert call(layers=None) == qm.MOE_EINVAL
    assert call(layers=qm.stack_layers([(A, None, A, A), (A, None, None, A), (A, None, A, A)])) == qm.MOE_EINVAL
    assert call(layers=qm.stack_layers([(A, A + 4, A, A)] * L)) == qm.MOE_EALIGN
    assert call(x0=None) == qm.MOE_EINVAL
    assert call(x_all=A + 0x100008) == qm.MOE_EALIGN
    assert call(x_all=A) == qm.MOE_EINVAL                           # overlaps x0
    assert call(out_all=A + 0x100000 + 2 * H) == qm.MOE_EINVAL     # overlaps x_all
    assert call(eps=float("nan")) == qm.MOE_EINVAL
    assert call(wsb=qm.moe_stack_workspace_bytes(cfg, L) - 1) == qm.MOE_EWORKSPACE


def test_codec_configs_and_sizes():
    """Expert bytes of the three codecs at the Xing4 shape (4.5, 4.25 and 3.5 bits per weight: the packed 3-bit
    expert is 7/9 of the IQ4_NL one), the packed sizes (IQ4_XS tiles repeat a super-block's scale), and the
    rules: the other codecs run the FP32 contract only, IQ4_XS needs ffn % 256."""
    nl = qm.make_config(**XING4)
    xs = qm.make_config(**XING4, codec=qm.CODEC_IQ4_XS)
    q3 = qm.make_config(**XING4, codec=qm.CODEC_Q3_AFFINE)
    assert qm.moe_expert_bytes(nl) == 6193152 == qm.moe_packed_expert_bytes(nl)
    assert qm.moe_expert_bytes(xs) == 3 * 1024 * 3584 // 256 * 136 == 5849088
    assert qm.moe_packed_expert_bytes(xs) == 3 * (1024 // 16) * (3584 // 128) * 1120
    assert qm.moe_expert_bytes(q3) == qm.moe_packed_expert_bytes(q3) == 6193152 * 7 // 9
    for c in (xs, q3):
        assert qm.moe_resolved_precision(c, 1) == qm.PREC_FP32
        assert qm.moe_resolved_precision(c, 5000) == qm.PREC_FP32
    bad = [(dict(codec=3), qm.MOE_EINVAL), (dict(codec=1, ffn=128), qm.MOE_EUNSUPPORTED),
           (dict(codec=2, precision=qm.PREC_BF16), qm.MOE_EUNSUPPORTED),
           (dict(codec=1, precision=qm.PREC_W4A8), qm.MOE_EUNSUPPORTED)]
    for b, code in bad:
        assert qm.moe_check_config(qm.make_config(**{**XING4, **b})) == code, b


def test_dense_and_gated_configs():
    """A dense FFN block (E = 0, K = 0, one always-on expert) and a sigmoid-gated shared expert are valid
    shapes; their neighbours are refused, and the routing-only calls refuse a dense block."""
    dense = qm.make_config(3584, 9216, 0, 0, 1)
    assert qm.moe_check_config(dense) == 0
    assert qm.moe_expert_bytes(dense) == 3 * 9216 * 3584 // 32 * 18
    assert qm.moe_resolved_precision(dense, 16) == qm.PREC_FP32
    assert qm.moe_resolved_precision(dense, 17) == qm.PREC_BF16
    gated = qm.make_config(**XING4, shared_gate=1)
    assert qm.moe_check_config(gated) == 0
    assert qm.moe_workspace_bytes(gated, 4) >= qm.moe_workspace_bytes(qm.make_config(**XING4), 4)
    for bad, code in [(dict(n_experts=0, top_k=0, n_shared=0), qm.MOE_EUNSUPPORTED),
                      (dict(n_experts=0, top_k=2), qm.MOE_EUNSUPPORTED),
                      (dict(n_experts=0, top_k=0, shared_gate=1), qm.MOE_EUNSUPPORTED),
                      (dict(top_k=0), qm.MOE_EINVAL),
                      (dict(n_shared=0, shared_gate=1), qm.MOE_EUNSUPPORTED),
                      (dict(shared_gate=2), qm.MOE_EINVAL)]:
        assert qm.moe_check_config(qm.make_config(**{**XING4, **bad})) == code, bad
    ws = qm.moe_workspace_bytes(dense, 4)
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_route(dense, 4, A, A, None, A, A, A, ws_bytes=ws, stream=0)
    assert ei.value.status == qm.MOE_EINVAL
    with pytest.raises(qm.MoeError) as ei:  # the dense block still needs its expert
        qm.moe_layer_forward(dense, 4, A, None, None, None, None, A, ws=A, ws_bytes=ws, stream=0)
    assert ei.value.status == qm.MOE_EINVAL


@pytest.mark.parametrize("bad,code", [
    (dict(hidden=3584 + 64), qm.MOE_EUNSUPPORTED),
    (dict(hidden=0), qm.MOE_EINVAL),
    (dict(ffn=1000), qm.MOE_EUNSUPPORTED),
    (dict(n_experts=300), qm.MOE_EUNSUPPORTED),
    (dict(top_k=9), qm.MOE_EUNSUPPORTED),
    (dict(n_experts=2, top_k=3), qm.MOE_EUNSUPPORTED),
    (dict(n_shared=2), qm.MOE_EUNSUPPORTED),
    (dict(routed_scale=float("nan")), qm.MOE_EINVAL),
    (dict(precision=5), qm.MOE_EINVAL),
])
def test_bad_configs_are_refused(bad, code):
    cfg = qm.make_config(**{**XING4, **bad})
    assert qm.moe_check_config(cfg) == code
    assert qm.moe_expert_bytes(cfg) == 0
    assert qm.moe_workspace_bytes(cfg, 1) == 0
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_route(cfg, 1, A, A, None, A, A, A, ws_bytes=1 << 30, stream=0)
    assert ei.value.status == code


def test_route_argument_errors():
    cfg = qm.make_config(**XING4)
    ws = qm.moe_workspace_bytes(cfg, 4)

    def call(T=4, x=A, g=A, b=None, ids=A, w=A, wsp=A, wsb=ws):
        with pytest.raises(qm.MoeError) as ei:
            qm.moe_route(cfg, T, x, g, b, ids, w, wsp, ws_bytes=wsb, stream=0)
        return ei.value.status

    assert call(T=-1) == qm.MOE_EUNSUPPORTED
    assert call(T=70000) == qm.MOE_EUNSUPPORTED
    assert call(x=None) == qm.MOE_EINVAL
    assert call(g=None) == qm.MOE_EINVAL
    assert call(ids=None) == qm.MOE_EINVAL
    assert call(w=None) == qm.MOE_EINVAL
    assert call(wsp=None) == qm.MOE_EINVAL
    assert call(x=A + 2) == qm.MOE_EALIGN          # an offset view: the research log's float4 lesson
    assert call(g=A + 4) == qm.MOE_EALIGN
    assert call(b=A + 8) == qm.MOE_EALIGN
    assert call(wsp=A + 8) == qm.MOE_EALIGN
    assert call(wsb=ws - 1) == qm.MOE_EWORKSPACE


def test_expert_forward_and_layer_argument_errors():
    cfg = qm.make_config(**XING4)
    ws = qm.moe_workspace_bytes(cfg, 3)
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_expert_forward(cfg, 3, A, A, A, A, None, A, A, ws_bytes=ws, stream=0)  # shared expert missing
    assert ei.value.status == qm.MOE_EINVAL
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_expert_forward(cfg, 3, A, A, A, A + 1, A, A, A, ws_bytes=ws, stream=0)
    assert ei.value.status == qm.MOE_EALIGN
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_expert_forward(cfg, 3, A, A, A, A, A, A, A, ws_bytes=16, stream=0)
    assert ei.value.status == qm.MOE_EWORKSPACE
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_layer_forward(cfg, 3, A, A, None, A, A, A, A + 4, None, ws=A, ws_bytes=ws, stream=0)
    assert ei.value.status == qm.MOE_EALIGN
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_layer_forward(cfg, 3, A, A, None, A, A, None, None, None, ws=A, ws_bytes=ws, stream=0)
    assert ei.value.status == qm.MOE_EINVAL


def test_bucket_pack_dequant_argument_errors():
    cfg = qm.make_config(**XING4)
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_bucket(cfg, 2, A, A, A, None, stream=0)
    assert ei.value.status == qm.MOE_EINVAL
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_pack_experts(cfg, 2, A, A + 1024, stream=0)  # overlapping ranges
    assert ei.value.status == qm.MOE_EINVAL
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_pack_experts(cfg, -1, A, A, stream=0)
    assert ei.value.status == qm.MOE_EINVAL
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_dequant(cfg, A, 3, qm.PREC_FP32, A, stream=0)
    assert ei.value.status == qm.MOE_EINVAL
    with pytest.raises(qm.MoeError) as ei:
        qm.moe_dequant(cfg, A, 0, qm.PREC_AUTO, A, stream=0)
    assert ei.value.status == qm.MOE_EINVAL


def test_zero_sized_calls_enqueue_nothing():
    cfg = qm.make_config(**XING4)
    qm.moe_pack_experts(cfg, 0, A, A + (1 << 24), stream=0)  # no work, no launch


def test_stream_read_argument_errors():
    def call(src=A, n=1 << 20, sink=A):
        with pytest.raises(qm.MoeError) as ei:
            qm.moe_stream_read(src, n, sink, stream=0)
        return ei.value.status

    assert call(n=(1 << 20) + 8) == qm.MOE_EINVAL
    assert call(src=None) == qm.MOE_EINVAL
    assert call(sink=None) == qm.MOE_EINVAL
    assert call(src=A + 4) == qm.MOE_EALIGN
    assert call(sink=A + 4) == qm.MOE_EALIGN
    qm.moe_stream_read(A, 0, A, stream=0)  # zero bytes: validated, nothing enqueued


def test_residual_rmsnorm_argument_errors():
    assert qm._lib.moe_residual_rmsnorm(A, A, 1, 3584 + 64, 1e-6, A, 0) == qm.MOE_EUNSUPPORTED
    assert qm._lib.moe_residual_rmsnorm(A, A, -1, 3584, 1e-6, A, 0) == qm.MOE_EUNSUPPORTED
    assert qm._lib.moe_residual_rmsnorm(A, A, 1, 3584, float("nan"), A, 0) == qm.MOE_EINVAL
    assert qm._lib.moe_residual_rmsnorm(A, A, 1, 3584, -1.0, A, 0) == qm.MOE_EINVAL
    assert qm._lib.moe_residual_rmsnorm(None, A, 1, 3584, 1e-6, A, 0) == qm.MOE_EINVAL
    assert qm._lib.moe_residual_rmsnorm(A, A + 2, 1, 3584, 1e-6, A, 0) == qm.MOE_EALIGN
    assert qm._lib.moe_residual_rmsnorm(A, A, 1, 3584, 1e-6, A + 8, 0) == qm.MOE_EALIGN
    assert qm._lib.moe_residual_rmsnorm(A, A, 0, 3584, 1e-6, None, 0) == qm.MOE_OK  # T = 0: nothing to do
