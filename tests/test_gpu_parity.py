"""GPU parity: every step of the layer, run through the C ABI, against the CPU oracle.

Integer work (routing ids, bucketing, the dequantized weights) must match bit for bit;
the routing weights too (same fp32 operations in the same order); the FP output must
match within max-abs 2e-2 and rel-L2 1e-3 of the oracle in the matching precision mode.
"""
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

_CACHE = {}


def workload(name, layer=0):
    key = (name, layer)
    if key not in _CACHE:
        s = synth.WORKLOADS[name]
        _CACHE[key] = (s, synth.layer_inputs(s, layer=layer))
    return _CACHE[key]


def device_layer(name, precision=qm.PREC_AUTO, bias=None):
    s, inp = workload(name)
    cfg = cfg_of(s, precision)
    return s, inp, qm.DeviceLayer(cfg, inp["gate_w"], bias, inp["arena"], inp["shared"])


def log(msg):
    print(f"[case] {msg}", flush=True)


def assert_status_ok(cfg, T, ws):
    """The workspace's status word through the C ABI: 0 unless a wait of the decode path gave up."""
    st = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    qm.moe_workspace_status(cfg, T, ws, st)
    assert int(st[0].item()) == 0, "a wait of the decode path gave up"


# ---------------------------------------------------------------- dequant (bit-exact)

@pytest.mark.parametrize("name", ["tiny", "xing4", "prefill"])
@pytest.mark.parametrize("precision", [qm.PREC_FP32, qm.PREC_BF16])
def test_dequant_bit_exact(name, precision):
    s, inp, dl = device_layer(name)
    eb = s.expert_bytes
    mb = eb // 3
    for e in (0, s.n_experts - 1):
        for m, (rows, cols) in enumerate([(s.ffn, s.hidden), (s.ffn, s.hidden), (s.hidden, s.ffn)]):
            log(f"dequant {name} expert={e} matrix={m} precision={precision}")
            out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
            qm.moe_dequant(dl.cfg, dl.arena[e * eb:(e + 1) * eb], m, precision, out)
            want = oracle.dequant(inp["arena"][e * eb + m * mb: e * eb + (m + 1) * mb],
                                  oracle.BF16 if precision == qm.PREC_BF16 else oracle.FP32).reshape(rows, cols)
            got = out.cpu().numpy()
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (name, e, m)


# ---------------------------------------------------------------- router (bit-exact)

def run_route(dl, x_bits, bias_dev=None):
    T = x_bits.shape[0]
    cfg = dl.cfg
    ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
    ws = torch.empty(qm.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    qm.moe_route(cfg, T, to_dev_bf16(x_bits), dl.gate_w, bias_dev, ids, w, ws)
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("name,T", [("tiny", 4), ("tiny", 1), ("tiny", 100), ("xing4", 64), ("batch", 128),
                                     ("xing4", 300), ("xing4", 1000), ("prefill", 300), ("prefill", 2048)])
def test_route_bit_exact(name, T):
    """Every router kernel: one row per wavefront (T < 64), 2 x 2 blocks with resident operands (tiny T=100,
    Xing4 T=64, batch T=128), 4 x 4 blocks (Xing4 T=300), 8 x 8 blocks (prefill T=300, 2048)."""
    s, inp, dl = device_layer(name)
    x = synth.tokens(s, T, first=1000)
    log(f"route {name} T={T}")
    ids, w = run_route(dl, x)
    rid, rw, _, _ = oracle.route(x, inp["gate_w"], s.top_k, s.routed_scale)
    assert np.array_equal(ids, rid)
    assert np.array_equal(w.view(np.uint32), rw.view(np.uint32))


def test_route_with_selection_bias_bit_exact():
    s, inp, dl = device_layer("prefill")
    bias = synth.zipf_bias(s, 0.05)
    x = synth.tokens(s, 257, first=7)
    log("route prefill with zipf bias T=257")
    ids, w = run_route(dl, x, torch.from_numpy(bias).cuda())
    rid, rw, _, _ = oracle.route(x, inp["gate_w"], s.top_k, s.routed_scale, bias)
    assert np.array_equal(ids, rid)
    assert np.array_equal(w.view(np.uint32), rw.view(np.uint32))


def test_route_large_hidden_bit_exact():
    """H = 8192 (above the resident-operand router's limit) at T = 70: 4 x 4 blocks streaming 32 steps."""
    s = EXTRA_SHAPES["h8192_f2048"]
    g = synth.gate_weights(s)
    x = synth.tokens(s, 70, first=5)
    log("route h8192 T=70")
    cfg = cfg_of(s)
    ids = torch.empty((70, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((70, s.top_k), dtype=torch.float32, device="cuda")
    ws = torch.empty(qm.moe_workspace_bytes(cfg, 70), dtype=torch.uint8, device="cuda")
    qm.moe_route(cfg, 70, to_dev_bf16(x), torch.from_numpy(g).cuda(), None, ids, w, ws)
    rid, rw, _, _ = oracle.route(x, g, s.top_k, s.routed_scale)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), rw.view(np.uint32))


def sigmoid_grid(n):
    """n fp32 logits in [-30, 30]: an even grid, plus powers of two and random bit patterns near 0."""
    rng = np.random.default_rng(77)
    k = np.arange(-126, 5, dtype=np.float64)
    special = np.concatenate([2.0 ** k, -(2.0 ** k), [0.0, -0.0, 30.0, -30.0, 1e-45, -1e-45]]).astype(np.float32)
    bits = rng.integers(0x30000000, 0x41F00000, 4096).astype(np.uint32)  # |l| from ~5e-10 to 30
    rnd = bits.view(np.float32) * np.where(rng.integers(0, 2, 4096) > 0, 1.0, -1.0).astype(np.float32)
    base = np.linspace(-30.0, 30.0, n - special.size - rnd.size).astype(np.float32)
    return np.concatenate([base, special, rnd]).astype(np.float32)


@pytest.mark.parametrize("T", [4096, 48])
def test_router_sigmoid_dense_grid_bit_exact(T):
    """The GPU sigmoid against the oracle's on a dense grid of 2^20 fp32 logits in [-30, 30], bit for bit.
    Token t is one-hot at element t (H = 4096), so its logit for expert e is exactly gate_w[e][t]: every
    other product is zero and the fixed-order sum adds only zeros to it.  T = 4096 runs the 8 x 8 tiled
    router kernel over the whole grid, T = 48 the one-row-per-wavefront kernel over its first 48 columns."""
    H, E = 4096, 256
    grid = sigmoid_grid(H * E).reshape(E, H)
    x = np.zeros((T, H), np.uint16)
    x[np.arange(T), np.arange(T)] = 0x3F80  # bf16 1.0
    cfg = qm.make_config(H, 128, E, 8)
    scores = torch.empty((T, E), dtype=torch.float32, device="cuda")
    log(f"sigmoid grid T={T}")
    qm.moe_router_scores(cfg, T, to_dev_bf16(x), torch.from_numpy(grid).cuda(), scores)
    got = scores.cpu().numpy()
    want = oracle.sigmoid_many(np.ascontiguousarray(grid[:, :T].T))
    bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
    assert bad.size == 0, (bad.size, grid[:, :T].T.reshape(-1)[bad[:5]])


def test_router_scores_match_route_scores():
    """moe_router_scores on real weights equals the oracle's scores bit for bit (prefill shape, T = 300)."""
    s, inp, dl = device_layer("prefill")
    x = synth.tokens(s, 300, first=31)
    scores = torch.empty((300, s.n_experts), dtype=torch.float32, device="cuda")
    log("router scores prefill T=300")
    qm.moe_router_scores(dl.cfg, 300, to_dev_bf16(x), dl.gate_w, scores)
    _, _, _, want = oracle.route(x, inp["gate_w"], s.top_k, s.routed_scale)
    assert np.array_equal(scores.cpu().numpy().view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- bucketing (bit-exact)

@pytest.mark.parametrize("T,K,E", [(4, 2, 8), (1, 4, 64), (128, 4, 64), (2048, 8, 256), (1000, 3, 5), (0, 4, 64),
                                   (5000, 8, 256), (65536, 8, 256)])
def test_bucket_bit_exact(T, K, E):
    rng = np.random.default_rng(T * 7 + K)
    ids = np.array([rng.choice(E, K, replace=False) for _ in range(T)], np.int32).reshape(T, K)
    cfg = qm.make_config(256, 128, E, K)
    log(f"bucket T={T} K={K} E={E}")
    dids = torch.from_numpy(ids).cuda()
    counts = torch.full((E,), -1, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -1, dtype=torch.int32, device="cuda")
    perm = torch.full((max(T * K, 1),), -1, dtype=torch.int32, device="cuda")
    pos = torch.full((max(T * K, 1),), -1, dtype=torch.int32, device="cuda")
    qm.moe_bucket(cfg, T, dids, counts, offsets, perm, pos)
    rc, ro, rp, rpos = oracle.bucket(ids, E)
    assert np.array_equal(counts.cpu().numpy(), rc)
    assert np.array_equal(offsets.cpu().numpy(), ro)
    assert np.array_equal(perm.cpu().numpy()[:T * K], rp)
    assert np.array_equal(pos.cpu().numpy()[:T * K], rpos)


# ---------------------------------------------------------------- the whole layer (FP tolerance)

def layer_parity(name, T, first=0, sample=None, bias=None, precision=qm.PREC_AUTO):
    s, inp, dl = device_layer(name, precision, bias)
    x = synth.tokens(s, T, first=first)
    cfg = dl.cfg
    prec = qm.moe_resolved_precision(cfg, T)
    log(f"layer {name} T={T} precision={prec}")
    ids = torch.empty((T, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s.top_k), dtype=torch.float32, device="cuda")
    out = dl.forward(to_dev_bf16(x), topk_ids=ids, topk_w=w).cpu().numpy()
    assert_status_ok(cfg, T, dl.workspace(T))
    rows = np.arange(T) if sample is None else np.asarray(sample)
    mode = {qm.PREC_BF16: oracle.BF16, qm.PREC_W4A8: oracle.W4A8}.get(prec, oracle.FP32)
    ref, rid, rw = oracle.layer(x[rows], inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn,
                                s.routed_scale, bias, mode)
    assert np.array_equal(ids.cpu().numpy()[rows], rid)
    assert np.array_equal(w.cpu().numpy()[rows].view(np.uint32), rw.view(np.uint32))
    assert_close(out[rows], ref, f"{name} T={T} rows={len(rows)}")
    return out


# Shapes off the pages' configurations, for the corners of the supported range: no shared
# expert with an odd K, the largest expert count with a small hidden size, K = 1, and the largest
# hidden size of the decode plan.
EXTRA_SHAPES = {
    "noshared_k3": synth.Shape("noshared_k3", 1, 512, 16, 3, 256, n_shared=0, routed_scale=1.5, seed=21),
    "e256_k4": synth.Shape("e256_k4", 1, 512, 256, 4, 128, seed=22),
    "k1": synth.Shape("k1", 1, 256, 4, 1, 128, routed_scale=1.0, seed=23),
    "h4096": synth.Shape("h4096", 1, 4096, 8, 2, 256, seed=24),
    "h8192_f2048": synth.Shape("h8192_f2048", 1, 8192, 4, 2, 2048, seed=25),
    # 2, 5 and 7 tile columns per gate/up wavefront of the exact-weight kernel (H / 128 / 8)
    "h2048": synth.Shape("h2048", 1, 2048, 8, 2, 256, seed=26),
    "h5120": synth.Shape("h5120", 1, 5120, 8, 2, 256, seed=27),
    "h7168": synth.Shape("h7168", 1, 7168, 8, 2, 256, seed=28),
}


def extra_layer_parity(name, T, first=0, precision=qm.PREC_AUTO):
    s = EXTRA_SHAPES[name]
    key = (name, 0)
    if key not in _CACHE:
        _CACHE[key] = (s, synth.layer_inputs(s))
    inp = _CACHE[key][1]
    dl = qm.DeviceLayer(cfg_of(s, precision), inp["gate_w"], None, inp["arena"], inp["shared"])
    x = synth.tokens(s, T, first=first)
    prec = qm.moe_resolved_precision(dl.cfg, T)
    log(f"layer {name} T={T} precision={prec}")
    ids = torch.empty((T, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s.top_k), dtype=torch.float32, device="cuda")
    out = dl.forward(to_dev_bf16(x), topk_ids=ids, topk_w=w).cpu().numpy()
    assert_status_ok(dl.cfg, T, dl.workspace(T))
    mode = oracle.BF16 if prec == qm.PREC_BF16 else oracle.FP32
    ref, rid, rw = oracle.layer(x, inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn, s.routed_scale,
                                None, mode)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), rw.view(np.uint32))
    assert_close(out, ref, f"{name} T={T}")


@pytest.mark.parametrize("name,T", [("noshared_k3", 1), ("noshared_k3", 40), ("noshared_k3", 300),
                                    ("e256_k4", 1), ("e256_k4", 77), ("e256_k4", 1200),
                                    ("k1", 1), ("k1", 33), ("k1", 600), ("h4096", 1), ("h4096", 19),
                                    ("h8192_f2048", 1), ("h8192_f2048", 19), ("h8192_f2048", 33)])
def test_layer_shape_corners(name, T):
    """Decode plan (T = 1), FP32 and BF16 multi-kernel plans on shapes at the edges of the supported range.

    h8192_f2048 (largest hidden size; above the decode plan's limits, so T = 1 takes the multi-kernel
    FP32 plan): the exact-weight kernels walk their tiles in more than one pass (8 gate/up tiles and
    2 down tiles per wavefront); T = 33 takes the BF16 plan."""
    extra_layer_parity(name, T, first=3 * T)


@pytest.mark.parametrize("name", ["h2048", "h5120", "h7168"])
def test_layer_fp32_column_counts(name):
    """FP32 contract at hidden sizes whose gate/up wavefronts walk 2, 5 and 7 tile columns: the
    double-buffered column loop with an odd last column and loads past the range (zeros)."""
    extra_layer_parity(name, 19, first=5, precision=qm.PREC_FP32)
    extra_layer_parity(name, 1, first=2, precision=qm.PREC_FP32)


def test_layer_tiny():
    layer_parity("tiny", 4)


def test_layer_tiny_ragged_and_single():
    layer_parity("tiny", 1, first=11)
    layer_parity("tiny", 37, first=20)


def test_layer_xing4_decode_tokens():
    for i in range(3):
        layer_parity("xing4", 1, first=500 + i)


def test_layer_xing4_small_batch():
    layer_parity("xing4", 5, first=40)


def test_layer_batch_128_all_rows():
    """The batch workload at its full size (T = 128, Xing4 layer, FP32 contract by AUTO): every row."""
    layer_parity("batch", 128)


@pytest.mark.parametrize("precision", [qm.PREC_AUTO, qm.PREC_FP32])
def test_layer_max_tokens_sampled(precision):
    """T = 65536, the largest call the library accepts, on the Xing4 shape (auto takes the BF16 plan;
    forced FP32 runs the exact-weight kernels over 20k+ chunks); first, last and interior rows."""
    layer_parity("batch", 65536, sample=[0, 1, 4095, 4096, 32767, 65534, 65535], precision=precision)


def test_layer_top8_small_batch_fp32():
    """K = 8 (the largest top-k) on the FP32 multi-kernel plan: the prefill shape at T = 3."""
    layer_parity("prefill", 3, first=11)


def test_layer_many_routes_on_one_expert():
    """A selection bias that sends every token to experts 0..K-1: chunks of 16 per expert, ragged tail."""
    s, _ = workload("tiny")
    bias = np.zeros(s.n_experts, np.float32)
    bias[:s.top_k] = 10.0
    layer_parity("tiny", 45, first=3, bias=bias)


def test_layer_zero_tokens_is_a_no_op():
    s, inp, dl = device_layer("tiny")
    log("layer tiny T=0")
    out = torch.empty((0, s.hidden), dtype=torch.float32, device="cuda")
    x = torch.empty((0, s.hidden), dtype=torch.bfloat16, device="cuda")
    dl.forward(x, out=out)
    torch.cuda.synchronize()


def test_layer_is_deterministic_and_token_order_equivariant():
    s, inp, dl = device_layer("xing4")
    x = synth.tokens(s, 24, first=77)
    log("determinism xing4 T=24")
    a = dl.forward(to_dev_bf16(x)).cpu().numpy()
    b = dl.forward(to_dev_bf16(x)).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    perm = np.random.default_rng(5).permutation(24)
    c = dl.forward(to_dev_bf16(x[perm])).cpu().numpy()
    assert np.array_equal(a[perm].view(np.uint32), c.view(np.uint32))


def test_expert_forward_matches_layer_forward():
    s, inp, dl = device_layer("tiny")
    x = synth.tokens(s, 9, first=50)
    log("expert_forward tiny T=9")
    xd = to_dev_bf16(x)
    rid, rw, _, _ = oracle.route(x, inp["gate_w"], s.top_k, s.routed_scale)
    out = torch.empty((9, s.hidden), dtype=torch.float32, device="cuda")
    qm.moe_expert_forward(dl.cfg, 9, xd, torch.from_numpy(rid).cuda(), torch.from_numpy(rw).cuda(), dl.arena,
                          dl.shared, out, dl.workspace(9))
    full = dl.forward(xd).cpu().numpy()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), full.view(np.uint32))


# ---------------------------------------------------------------- one-launch decode path

def assert_paths_agree(a, b, what):
    """Decode path vs multi-kernel path: same contract, fp32 sums split differently."""
    a = a.astype(np.float64)
    b = b.astype(np.float64)
    r = float(np.linalg.norm(a - b) / np.linalg.norm(b))
    print(f"[parity] decode vs multi-kernel {what}: rel_l2={r:.3e}", flush=True)
    assert r < 1e-5, (what, r)

def multi_kernel_layer(dl, xd, T):
    """moe_route + moe_expert_forward: the multi-kernel composition of the same layer."""
    cfg = dl.cfg
    ids = torch.empty((T, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
    ws = torch.empty(qm.moe_workspace_bytes(cfg, T), dtype=torch.uint8, device="cuda")
    qm.moe_route(cfg, T, xd, dl.gate_w, dl.bias, ids, w, ws)
    qm.moe_expert_forward(cfg, T, xd, ids, w, dl.arena, dl.shared, out, ws)
    return out


@pytest.mark.parametrize("name,T,first", [("xing4", 1, 300), ("xing4", 1, 301), ("tiny", 1, 300), ("tiny", 1, 7)])
def test_decode_path_equals_multi_kernel_path(name, T, first):
    s, inp, dl = device_layer(name)
    x = synth.tokens(s, T, first=first)
    xd = to_dev_bf16(x)
    log(f"decode path vs multi-kernel {name} T={T}")
    a = dl.forward(xd).cpu().numpy()
    b = multi_kernel_layer(dl, xd, T).cpu().numpy()
    assert_paths_agree(a, b, f"{name} T={T}")
    assert_status_ok(dl.cfg, T, dl.workspace(T))


def test_decode_path_many_consecutive_calls_one_workspace():
    s, inp, dl = device_layer("xing4")
    x = synth.tokens(s, 64, first=900)
    xd = to_dev_bf16(x)
    log("decode path, 64 consecutive T=1 calls")
    outs = [dl.forward(xd[i:i + 1]) for i in range(64)]
    got = torch.cat(outs).cpu().numpy()
    assert_status_ok(dl.cfg, 1, dl.workspace(1))
    ref = multi_kernel_layer(dl, xd, 64).cpu().numpy()
    assert_paths_agree(got, ref, "64 consecutive decode calls")


def decode_route(dl, x_bits):
    """The decode path's routing outputs for one token (T = 1)."""
    cfg = dl.cfg
    ids = torch.empty((1, cfg.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((1, cfg.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((1, cfg.hidden), dtype=torch.float32, device="cuda")
    qm.moe_layer_forward(cfg, 1, to_dev_bf16(x_bits), dl.gate_w, dl.bias, dl.arena, dl.shared, out, ids, w,
                         ws=dl.workspace(1))
    return ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("with_bias", [False, True])
def test_decode_route_bit_exact(with_bias):
    s, inp = workload("xing4")
    bias = synth.zipf_bias(s, 0.08) if with_bias else None
    _, _, dl = device_layer("xing4", bias=None if bias is None else torch.from_numpy(bias).cuda())
    x = synth.tokens(s, 24, first=5100)
    log(f"decode route xing4 bias={with_bias}")
    rid, rw, _, _ = oracle.route(x, inp["gate_w"], s.top_k, s.routed_scale, bias)
    for t in range(24):
        ids, w = decode_route(dl, x[t:t + 1])
        assert np.array_equal(ids[0], rid[t]), t
        assert np.array_equal(w[0].view(np.uint32), rw[t].view(np.uint32)), t
    assert_status_ok(dl.cfg, 1, dl.workspace(1))


@pytest.mark.parametrize("path", ["decode", "multi-kernel"])
def test_route_ties_break_by_lower_expert_index(path):
    """Experts 1, 4 and 6 share one router row, so their scores tie exactly; tokens on which that row
    wins must pick them in index order (K = 2 of 8 on the tiny shape: experts 1 and 4)."""
    s, inp = workload("tiny")
    gw = inp["gate_w"].copy()
    gw[4] = gw[1]
    gw[6] = gw[1]
    x = synth.tokens(s, 64, first=900)
    rid, rw, _, _ = oracle.route(x, gw, s.top_k, s.routed_scale)
    tied = [t for t in range(64) if rid[t, 0] == 1]
    assert len(tied) >= 3 and all(rid[t, 1] == 4 for t in tied)
    dl = qm.DeviceLayer(cfg_of(s, qm.PREC_FP32), gw, None, inp["arena"], inp["shared"])
    log(f"route ties {path} on {len(tied)} tokens")
    for t in tied:
        if path == "decode":
            ids, w = decode_route(dl, x[t:t + 1])
        else:
            ids, w = run_route(dl, x[t:t + 1])
        assert np.array_equal(ids[0], rid[t]), t
        assert np.array_equal(w[0].view(np.uint32), rw[t].view(np.uint32)), t


@pytest.mark.parametrize("T", [1, 2])
def test_nan_input_still_routes_to_experts_in_range(T):
    """A NaN in a token's activations makes every router logit NaN.  Every ranking compares order keys
    with the expert index as the tie-break, so the token still takes K distinct experts in range: the
    lowest indices, since all its scores tie, and the same ones in every workgroup.  No kernel then
    streams weights from outside the arena.  T = 1 is the decode plan, T = 2 the multi-kernel plan;
    the other token of T = 2 is finite and routed as the oracle routes it."""
    s, inp, dl = device_layer("xing4")
    cfg = dl.cfg
    x = synth.tokens(s, T, first=77).copy()
    x[0, 5] = 0x7FC0  # bf16 quiet NaN
    log(f"NaN input T={T}")
    ids = torch.full((T, cfg.top_k), -1, dtype=torch.int32, device="cuda")
    w = torch.empty((T, cfg.top_k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, cfg.hidden), dtype=torch.float32, device="cuda")
    qm.moe_layer_forward(cfg, T, to_dev_bf16(x), dl.gate_w, dl.bias, dl.arena, dl.shared, out, ids, w,
                         ws=dl.workspace(T))
    got = ids.cpu().numpy()
    assert got[0].tolist() == list(range(cfg.top_k))
    if T == 1:
        assert_status_ok(cfg, 1, dl.workspace(1))
    else:
        rid, _, _, _ = oracle.route(x[1:2], inp["gate_w"], s.top_k, s.routed_scale)
        assert np.array_equal(got[1], rid[0])
        assert np.isfinite(out[1].cpu().numpy()).all()


def test_decode_state_survives_batched_calls_on_the_same_workspace():
    """Decode calls interleaved with batched calls (FP32 and BF16 contracts) on one workspace: the
    decode path's words at the start of the workspace are not disturbed by the batched calls."""
    s, inp, dl = device_layer("xing4")
    cfg = dl.cfg
    ws = torch.empty(qm.moe_workspace_bytes(cfg, 300), dtype=torch.uint8, device="cuda")
    qm.moe_workspace_init(cfg, 300, ws)
    assert qm.moe_resolved_precision(cfg, 300) == qm.PREC_BF16
    x = synth.tokens(s, 300, first=4200)
    xd = to_dev_bf16(x)
    ref = multi_kernel_layer(dl, xd[:8], 8).cpu().numpy()
    log("decode calls around batched calls on one workspace")
    got = []
    for i in range(8):
        out = torch.empty((1, s.hidden), dtype=torch.float32, device="cuda")
        qm.moe_layer_forward(cfg, 1, xd[i:i + 1], dl.gate_w, None, dl.arena, dl.shared, out, ws=ws)
        got.append(out)
        T = 3 if i % 2 == 0 else 300  # FP32 then BF16 contract in between
        big = torch.empty((T, s.hidden), dtype=torch.float32, device="cuda")
        qm.moe_layer_forward(cfg, T, xd[:T], dl.gate_w, None, dl.arena, dl.shared, big, ws=ws)
    assert_paths_agree(torch.cat(got).cpu().numpy(), ref, "decode calls between batched calls")
    assert_status_ok(cfg, 300, ws)


def test_graph_replay_of_decode_calls():
    """A captured sequence of T=1 calls replayed several times, with eager work between replays."""
    s, inp, dl = device_layer("xing4")
    x = synth.tokens(s, 16, first=1500)
    xd = to_dev_bf16(x)
    out = torch.empty((16, s.hidden), dtype=torch.float32, device="cuda")
    ws = dl.workspace(1)
    eager = torch.cat([dl.forward(xd[i:i + 1]) for i in range(16)]).cpu().numpy()
    log("graph capture of 16 decode calls")
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(16):
                qm.moe_layer_forward(dl.cfg, 1, xd[i:i + 1], dl.gate_w, None, dl.arena, dl.shared,
                                     out[i:i + 1], ws=ws)
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        _ = dl.forward(xd[rep:rep + 1])  # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint32), eager.view(np.uint32)), rep
    assert_status_ok(dl.cfg, 1, ws)


# ---------------------------------------------------------------- bf16 grouped MFMA path

def test_layer_tiny_bf16():
    layer_parity("tiny", 4, precision=qm.PREC_BF16)
    layer_parity("tiny", 1, first=5, precision=qm.PREC_BF16)
    layer_parity("tiny", 37, first=20, precision=qm.PREC_BF16)


def test_layer_bf16_tiles_past_128_rows():
    """Every token on experts 0..K-1: 300 routes per expert and 300 shared rows = tiles of 128, 128, 44."""
    s, _ = workload("tiny")
    bias = np.zeros(s.n_experts, np.float32)
    bias[:s.top_k] = 10.0
    layer_parity("tiny", 300, first=3, bias=bias, precision=qm.PREC_BF16)


def test_layer_batch_128_bf16_all_rows():
    layer_parity("batch", 128, precision=qm.PREC_BF16)


def prefill_bias():
    s, _ = workload("prefill")
    return synth.zipf_bias(s, synth.zipf_lambda(s))


def prefill_rows_checked():
    """Rows of the T = 2048 prefill call compared with the oracle: every token of the last tile of 128
    routes of the most popular expert, every token of the shared expert's last tile (tokens 1920..2047),
    the first and last tokens and a seeded sample (>= 256 rows)."""
    s, inp = workload("prefill")
    x = synth.tokens(s, 2048, first=0)
    rid, _, _, _ = oracle.route(x, inp["gate_w"], s.top_k, s.routed_scale, prefill_bias())
    counts, offsets, perm, _ = oracle.bucket(rid, s.n_experts)
    hot = int(np.argmax(counts))
    last_tile = offsets[hot] + 128 * ((counts[hot] - 1) // 128)
    hot_rows = (perm[last_tile:offsets[hot + 1]] // s.top_k).tolist()
    rows = set(hot_rows) | set(range(1920, 2048)) | {0, 1, 127, 128, 1023}
    rng = np.random.default_rng(11)
    extra = [r for r in rng.permutation(2048).tolist() if r not in rows]
    rows |= set(extra[:max(0, 256 - len(rows))])
    return sorted(rows), hot, counts[hot], len(hot_rows)


def test_layer_prefill_full_size_rows():
    """T=2048, H=2048, 256 experts top-8 + shared, ffn 512, Zipf(1.0) popularity (AUTO -> bf16): the hottest
    expert's last tile, one whole shared-expert tile and a sample, >= 256 rows against the oracle."""
    rows, hot, n_hot, n_tile = prefill_rows_checked()
    log(f"prefill rows: {len(rows)} (expert {hot}: {n_hot} routes, last tile {n_tile} rows)")
    assert len(rows) >= 256
    out = layer_parity("prefill", 2048, first=0, sample=rows, bias=prefill_bias())
    assert np.all(np.isfinite(out))


def test_layer_prefill_deterministic_and_order_equivariant():
    s, inp, dl = device_layer("prefill", bias=prefill_bias())
    x = synth.tokens(s, 2048, first=4096)
    log("determinism prefill T=2048")
    a = dl.forward(to_dev_bf16(x)).cpu().numpy()
    b = dl.forward(to_dev_bf16(x)).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    perm = np.random.default_rng(6).permutation(2048)
    c = dl.forward(to_dev_bf16(x[perm])).cpu().numpy()
    assert np.array_equal(a[perm].view(np.uint32), c.view(np.uint32))


def test_bf16_and_fp32_contracts_agree_on_a_batch():
    """The two FFN contracts differ only by the bf16 roundings of weights and h."""
    s, inp = workload("batch")
    x = synth.tokens(s, 32, first=300)
    outs = {}
    for prec in (qm.PREC_FP32, qm.PREC_BF16):
        _, _, dl = device_layer("batch", prec)
        log(f"batch T=32 precision={prec}")
        outs[prec] = dl.forward(to_dev_bf16(x)).cpu().numpy()
    a, b = outs[qm.PREC_FP32].astype(np.float64), outs[qm.PREC_BF16].astype(np.float64)
    r = np.linalg.norm(a - b) / np.linalg.norm(a)
    print(f"[parity] fp32 vs bf16 contract rel_l2={r:.3e}", flush=True)
    assert 0 < r < 2e-2


# ---------------------------------------------------------------- gated shared expert, dense FFN block

def gated_inputs(name):
    s, inp = workload(name)
    row = synth.shared_gate_row(s)
    return s, inp, np.concatenate([inp["gate_w"], row[None, :]]), row


@pytest.mark.parametrize("name,T,precision", [("tiny", 1, qm.PREC_AUTO), ("tiny", 4, qm.PREC_AUTO),
                                              ("tiny", 37, qm.PREC_BF16), ("tiny", 300, qm.PREC_AUTO),
                                              ("xing4", 1, qm.PREC_AUTO), ("xing4", 5, qm.PREC_AUTO),
                                              ("batch", 128, qm.PREC_BF16)])
def test_layer_gated_shared_expert(name, T, precision):
    """The shared expert scaled by sigmoid(x . gate_w[E]): decode plan (T = 1), FP32 and BF16 multi-kernel
    plans.  Routing bit-exact, the gate value (topk_w[:, K]) bit-exact against the oracle's sigmoid of the
    fixed-order logit, outputs within tolerance."""
    s, inp, gw, row = gated_inputs(name)
    cfg = cfg_of(s, precision)
    cfg.shared_gate = 1
    dl = qm.DeviceLayer(cfg, gw, None, inp["arena"], inp["shared"])
    x = synth.tokens(s, T, first=611)
    prec = qm.moe_resolved_precision(cfg, T)
    log(f"gated {name} T={T} precision={prec}")
    ids = torch.empty((T, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s.top_k + 1), dtype=torch.float32, device="cuda")
    out = dl.forward(to_dev_bf16(x), topk_ids=ids, topk_w=w).cpu().numpy()
    assert_status_ok(cfg, T, dl.workspace(T))
    mode = oracle.BF16 if prec == qm.PREC_BF16 else oracle.FP32
    ref, rid, rw = oracle.layer(x, inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn, s.routed_scale,
                                None, mode, shared_gate=row)
    wg = w.cpu().numpy()
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.array_equal(wg[:, :s.top_k].view(np.uint32), rw.view(np.uint32))
    g = oracle.sigmoid_many(oracle.router_logits(x, row[None, :])[:, 0])
    assert np.array_equal(wg[:, s.top_k].view(np.uint32), g.view(np.uint32))
    assert_close(out, ref, f"gated {name} T={T}")


def test_gated_expert_forward_takes_the_gate_from_the_weights():
    """moe_expert_forward of a gated layer reads the gate from topk_w[:, K]: with the router's own weights
    it equals moe_layer_forward bit for bit; with the gate column zeroed it equals the ungated layer without
    the shared expert's contribution (the oracle with no shared expert)."""
    s, inp, gw, row = gated_inputs("tiny")
    cfg = cfg_of(s)
    cfg.shared_gate = 1
    dl = qm.DeviceLayer(cfg, gw, None, inp["arena"], inp["shared"])
    T = 9
    x = synth.tokens(s, T, first=50)
    xd = to_dev_bf16(x)
    ids = torch.empty((T, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s.top_k + 1), dtype=torch.float32, device="cuda")
    full = dl.forward(xd, topk_ids=ids, topk_w=w).cpu().numpy()
    out = torch.empty((T, s.hidden), dtype=torch.float32, device="cuda")
    log("gated expert_forward tiny T=9")
    qm.moe_expert_forward(cfg, T, xd, ids, w, dl.arena, dl.shared, out, dl.workspace(T))
    assert np.array_equal(out.cpu().numpy().view(np.uint32), full.view(np.uint32))
    w[:, s.top_k] = 0.0
    qm.moe_expert_forward(cfg, T, xd, ids, w, dl.arena, dl.shared, out, dl.workspace(T))
    ref, _, _ = oracle.layer(x, inp["gate_w"], inp["arena"], None, s.top_k, s.ffn, s.routed_scale)
    assert_close(out.cpu().numpy(), ref, "gated, gate column zero")


@pytest.mark.parametrize("name,T,precision", [("tiny", 1, qm.PREC_AUTO), ("tiny", 16, qm.PREC_AUTO),
                                              ("tiny", 37, qm.PREC_AUTO), ("dense", 1, qm.PREC_AUTO),
                                              ("dense", 16, qm.PREC_AUTO), ("dense", 64, qm.PREC_AUTO),
                                              ("dense", 3, qm.PREC_BF16)])
def test_dense_ffn_block(name, T, precision):
    """A dense FFN block (E = 0: the always-on expert alone), the tiny width and the model's dense width
    (H = 3584, F = 9216): FP32 plan for T <= 16 and BF16 tiles above (AUTO), against the oracle."""
    s = synth.WORKLOADS[name]
    if name == "tiny":
        s = synth.Shape("tiny_dense", 1, s.hidden, 0, 0, s.ffn, seed=s.seed)
    key = (s.name, 0)
    if key not in _CACHE:
        _CACHE[key] = (s, synth.layer_inputs(s))
    inp = _CACHE[key][1]
    cfg = qm.make_config(s.hidden, s.ffn, 0, 0, 1, 1.0, precision)
    dl = qm.DeviceLayer(cfg, None, None, None, inp["shared"])
    x = synth.tokens(s, T, first=21)
    prec = qm.moe_resolved_precision(cfg, T)
    log(f"dense {s.name} T={T} precision={prec}")
    out = dl.forward(to_dev_bf16(x)).cpu().numpy()
    mode = oracle.BF16 if prec == qm.PREC_BF16 else oracle.FP32
    ref, _, _ = oracle.layer(x, np.zeros((0, s.hidden), np.float32), None, inp["shared"], 0, s.ffn, 1.0, None, mode)
    assert_close(out, ref, f"dense {s.name} T={T}")


# ---------------------------------------------------------------- W4A8: Q8_0 activations

def test_quantize_q8_0_bit_exact():
    """The Q8_0 quantizer against the oracle's, codes and fp16 scales bit for bit: bf16 activations (x) and fp32
    values (h) of several magnitudes, a zero block, and blocks whose values sit exactly on halfway points."""
    s, _ = workload("xing4")
    x = synth.tokens(s, 7, first=77)
    xd = to_dev_bf16(x)
    q = torch.empty(x.size, dtype=torch.int8, device="cuda")
    d = torch.empty(x.size // 32, dtype=torch.int16, device="cuda")
    log("quantize q8_0 bf16")
    qm.moe_quantize_q8_0(xd, q, d)
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    rq, rd = oracle.quantize_q8_0(xf)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(d.cpu().numpy().view(np.uint16), rd)
    rng = np.random.default_rng(3)
    h = (rng.standard_normal(32 * 4096) * np.repeat(10.0 ** rng.uniform(-6, 3, 4096), 32)).astype(np.float32)
    h[:32] = 0.0
    h[32:64] = np.arange(32) - 15.5  # every value a half-integer: codes of a non-trivial scale
    h[64:96] = 0.0
    h[64] = 127.0
    h[65:69] = (2.5, -2.5, 0.5, -126.5)  # amax 127: x * (1/1) lands exactly on halves
    hd = torch.from_numpy(h).cuda()
    q = torch.empty(h.size, dtype=torch.int8, device="cuda")
    d = torch.empty(h.size // 32, dtype=torch.int16, device="cuda")
    log("quantize q8_0 fp32")
    qm.moe_quantize_q8_0(hd, q, d)
    rq, rd = oracle.quantize_q8_0(h)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(d.cpu().numpy().view(np.uint16), rd)
    assert list(rq[64:69]) == [127, 3, -3, 1, -127]


@pytest.mark.parametrize("name,T", [("tiny", 4), ("tiny", 37), ("xing4", 1), ("xing4", 5), ("batch", 128),
                                    ("prefill", 300)])
def test_layer_w4a8(name, T):
    """The W4A8 contract (Q8_0 x and h, integer block dots on int8 MFMA) against the oracle's W4A8 mode: routing
    bit-exact, outputs within tolerance."""
    layer_parity(name, T, first=40, precision=qm.PREC_W4A8)


def test_layer_w4a8_gated_and_dense():
    s, inp, gw, row = gated_inputs("tiny")
    cfg = cfg_of(s, qm.PREC_W4A8)
    cfg.shared_gate = 1
    dl = qm.DeviceLayer(cfg, gw, None, inp["arena"], inp["shared"])
    x = synth.tokens(s, 20, first=5)
    log("w4a8 gated tiny T=20")
    out = dl.forward(to_dev_bf16(x)).cpu().numpy()
    ref, _, _ = oracle.layer(x, inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn, s.routed_scale, None,
                             oracle.W4A8, shared_gate=row)
    assert_close(out, ref, "w4a8 gated tiny T=20")
    d = synth.WORKLOADS["dense"]
    dinp = synth.layer_inputs(d)
    cfg = qm.make_config(d.hidden, d.ffn, 0, 0, 1, 1.0, qm.PREC_W4A8)
    dl = qm.DeviceLayer(cfg, None, None, None, dinp["shared"])
    x = synth.tokens(d, 3, first=8)
    log("w4a8 dense T=3")
    out = dl.forward(to_dev_bf16(x)).cpu().numpy()
    ref, _, _ = oracle.layer(x, np.zeros((0, d.hidden), np.float32), None, dinp["shared"], 0, d.ffn, 1.0, None,
                             oracle.W4A8)
    assert_close(out, ref, "w4a8 dense T=3")


# ---------------------------------------------------------------- other expert codecs

@pytest.mark.parametrize("name", ["tiny_xs", "tiny_q3", "xing4_xs", "xing4_q3"])
def test_codec_dequant_bit_exact(name):
    """The packed IQ4_XS / 3-bit tiles decoded on the GPU (moe_dequant) against the oracle's reading of the input
    layout, every weight of the first and last expert, bit for bit (both are exact in fp32)."""
    s, inp = workload(name)
    cfg = cfg_of(s)
    cfg.codec = s.codec
    dl = qm.DeviceLayer(cfg, inp["gate_w"], None, inp["arena"], inp["shared"])
    eb, pb = s.expert_bytes, qm.moe_packed_expert_bytes(cfg)
    for e in (0, s.n_experts - 1):
        src = inp["arena"][e * eb:(e + 1) * eb]
        at = 0
        for m, (rows, cols) in enumerate([(s.ffn, s.hidden), (s.ffn, s.hidden), (s.hidden, s.ffn)]):
            log(f"dequant {name} expert={e} matrix={m}")
            out = torch.empty((rows, cols), dtype=torch.float32, device="cuda")
            qm.moe_dequant(cfg, dl.arena[e * pb:(e + 1) * pb], m, qm.PREC_FP32, out)
            rb = oracle.codec_row_bytes(s.codec, cols)
            want = np.stack([oracle.dequant_codec(s.codec, src[at + r * rb: at + (r + 1) * rb], cols)
                             for r in range(rows)]).astype(np.float32)
            at += rows * rb
            assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32)), (name, e, m)


@pytest.mark.parametrize("name,T", [("tiny_xs", 1), ("tiny_xs", 4), ("tiny_xs", 37), ("tiny_q3", 1), ("tiny_q3", 4),
                                    ("tiny_q3", 37), ("xing4_xs", 1), ("xing4_xs", 5), ("xing4_q3", 1),
                                    ("xing4_q3", 5), ("xing4_xs", 128), ("xing4_q3", 128)])
def test_layer_codec(name, T):
    """The layer with IQ4_XS and packed 3-bit experts (exact weights, multi-kernel plan) against the oracle:
    routing bit-exact, outputs within tolerance."""
    s, inp = workload(name)
    cfg = cfg_of(s)
    cfg.codec = s.codec
    dl = qm.DeviceLayer(cfg, inp["gate_w"], None, inp["arena"], inp["shared"])
    x = synth.tokens(s, T, first=60)
    log(f"codec layer {name} T={T}")
    ids = torch.empty((T, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, s.top_k), dtype=torch.float32, device="cuda")
    out = dl.forward(to_dev_bf16(x), topk_ids=ids, topk_w=w).cpu().numpy()
    ref, rid, rw = oracle.layer(x, inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn, s.routed_scale,
                                codec=s.codec)
    assert np.array_equal(ids.cpu().numpy(), rid)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), rw.view(np.uint32))
    assert_close(out, ref, f"codec {name} T={T}")


# ---------------------------------------------------------------- the 38-layer stack workload

def test_stack_layers_chained_with_zipf_bias():
    """Three layers of the stack workload (Zipf(1.1) selection bias), each fed bf16(rmsnorm(x + out)) of the
    previous one as in bench.py: every layer's routing is bit-exact and its output within tolerance of the
    oracle on the same input."""
    s = synth.WORKLOADS["stack"]
    lam = synth.zipf_lambda(s)
    cfg = cfg_of(s)
    x = to_dev_bf16(synth.tokens(s, 1, first=123))
    for layer in range(3):
        inp = synth.layer_inputs(s, layer=layer, lam=lam)
        dl = qm.DeviceLayer(cfg, inp["gate_w"], inp["bias"], inp["arena"], inp["shared"])
        log(f"stack layer {layer}")
        ids = torch.empty((1, s.top_k), dtype=torch.int32, device="cuda")
        w = torch.empty((1, s.top_k), dtype=torch.float32, device="cuda")
        out = dl.forward(x, topk_ids=ids, topk_w=w)
        xb = x.view(torch.int16).cpu().numpy().view(np.uint16)
        ref, rid, rw = oracle.layer(xb, inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn,
                                    s.routed_scale, inp["bias"])
        assert np.array_equal(ids.cpu().numpy(), rid)
        assert np.array_equal(w.cpu().numpy().view(np.uint32), rw.view(np.uint32))
        assert_close(out.cpu().numpy(), ref, f"stack layer {layer}")
        h = x.float() + out
        x = torch.nn.functional.rms_norm(h, (s.hidden,), eps=1e-6).to(torch.bfloat16)


@pytest.mark.parametrize("T", [1, 5])
def test_chained_layer_equals_norm_then_layer(T):
    """moe_layer_forward_chained (the stack's norm folded into the router kernel on the decode plan, T = 1; a
    separate norm kernel on the multi-kernel plan, T = 5) against moe_residual_rmsnorm + moe_layer_forward:
    the formed input, the routing and the output are identical bit for bit."""
    s, inp, dl = device_layer("xing4")
    g = torch.Generator().manual_seed(T)
    x_prev = torch.randn(T, s.hidden, generator=g).to(torch.bfloat16).cuda()
    out_prev = torch.randn(T, s.hidden, generator=g).cuda()
    cfg = dl.cfg
    ws = dl.workspace(T)
    log(f"chained layer xing4 T={T}")
    x_a = torch.empty_like(x_prev)
    out_a = torch.empty((T, s.hidden), dtype=torch.float32, device="cuda")
    ids_a = torch.empty((T, s.top_k), dtype=torch.int32, device="cuda")
    w_a = torch.empty((T, s.top_k), dtype=torch.float32, device="cuda")
    qm.moe_layer_forward_chained(cfg, T, x_prev, out_prev, x_a, dl.gate_w, None, dl.arena, dl.shared, out_a, ids_a,
                                 w_a, ws)
    x_b = torch.empty_like(x_prev)
    qm.moe_residual_rmsnorm(out_prev, x_prev, x_b, eps=1e-6)
    out_b = torch.empty_like(out_a)
    ids_b = torch.empty_like(ids_a)
    w_b = torch.empty_like(w_a)
    qm.moe_layer_forward(cfg, T, x_b, dl.gate_w, None, dl.arena, dl.shared, out_b, ids_b, w_b, ws)
    torch.cuda.synchronize()
    assert torch.equal(x_a.view(torch.int16), x_b.view(torch.int16))
    assert torch.equal(ids_a, ids_b) and torch.equal(w_a.view(torch.int32), w_b.view(torch.int32))
    assert torch.equal(out_a.view(torch.int32), out_b.view(torch.int32))
    assert_status_ok(cfg, T, ws)


def test_stack_38_layers_captured_step():
    """The 38-layer T = 1 step of the stack workload (Zipf(1.1) selection bias, router weights per layer,
    expert weights of 2 drawn layers each placed per layer) captured as one HIP graph of chained layer calls
    for two tokens and replayed 3 times with eager work in between: every replay equals the eager run bit for
    bit; every layer's routing equals the oracle's on the GPU's input to that layer bit for bit, its output is
    within tolerance of the oracle's, and every formed input is within one bf16 step of the oracle's norm of
    the previous layer's input and output."""
    s = synth.WORKLOADS["stack"]
    lam = synth.zipf_lambda(s)
    cfg = cfg_of(s)
    nl, nt = 38, 2
    sets = [synth.layer_inputs(s, layer=d, lam=lam) for d in range(2)]
    packed = [qm.DeviceLayer(cfg, st["gate_w"], None, st["arena"], st["shared"]) for st in sets]
    layers, host = [], []
    for l in range(nl):
        gw, b = synth.gate_weights(s, layer=l), synth.zipf_bias(s, lam, layer=l)
        src = packed[l % 2]
        layers.append(qm.DeviceLayer.from_packed(cfg, torch.from_numpy(gw).cuda(), torch.from_numpy(b).cuda(),
                                                 src.arena.clone(), src.shared.clone()))
        host.append((gw, b, sets[l % 2]))
    x0 = to_dev_bf16(synth.tokens(s, nt, first=9000))
    xs = torch.empty((nt, nl, s.hidden), dtype=torch.bfloat16, device="cuda")
    outs = torch.empty((nt, nl, s.hidden), dtype=torch.float32, device="cuda")
    ids = torch.empty((nt, nl, s.top_k), dtype=torch.int32, device="cuda")
    w = torch.empty((nt, nl, s.top_k), dtype=torch.float32, device="cuda")
    ws = layers[0].workspace(1)

    def step():
        for t in range(nt):
            xs[t, 0].copy_(x0[t])
            for l, dl in enumerate(layers):
                if l == 0:
                    qm.moe_layer_forward(cfg, 1, xs[t, 0:1], dl.gate_w, dl.bias, dl.arena, dl.shared, outs[t, 0:1],
                                         ids[t, 0], w[t, 0], ws)
                else:
                    qm.moe_layer_forward_chained(cfg, 1, xs[t, l - 1:l], outs[t, l - 1:l], xs[t, l:l + 1], dl.gate_w,
                                                 dl.bias, dl.arena, dl.shared, outs[t, l:l + 1], ids[t, l], w[t, l],
                                                 ws)

    log("stack 38 layers: eager")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step()
        torch.cuda.synchronize()
        eager = [a.clone() for a in (xs, outs, ids, w)]
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        for rep in range(3):
            for a in (xs, outs, w):
                a.fill_(float("nan"))
            ids.fill_(-1)
            graph.replay()
            torch.cuda.synchronize()
            for got, want in zip((xs, outs, ids, w), eager):
                assert torch.equal(got.view(torch.int8), want.view(torch.int8)), rep
            _ = layers[rep].forward(x0[0:1])  # eager work between replays
            torch.cuda.synchronize()
    assert_status_ok(cfg, 1, ws)
    xin = xs.view(torch.int16).cpu().numpy().view(np.uint16)
    got, gid, gw_ = outs.cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()
    for l in range(nl):
        if l % 8 == 0:
            log(f"stack 38 layers: oracle layer {l}")
        gwl, bl, st = host[l]
        ref, rid, rw = oracle.layer(xin[:, l], gwl, st["arena"], st["shared"], s.top_k, s.ffn, s.routed_scale, bl)
        assert np.array_equal(gid[:, l], rid), l
        assert np.array_equal(gw_[:, l].view(np.uint32), rw.view(np.uint32)), l
        assert_close(got[:, l], ref, f"stack layer {l}")
        if l + 1 < nl:
            y = oracle.residual_rmsnorm(xin[:, l], got[:, l])
            diff = np.abs(xin[:, l + 1].astype(np.int32) - y.astype(np.int32))
            assert int(diff.max()) <= 1, l


def test_stream_read_reads_and_writes_nothing():
    """The measurement kernel: a zero buffer XORs to zero, so the sink keeps its value; a ragged size
    (not a multiple of the grid's stride) ends without touching memory past the buffer (the buffer sits
    inside a larger allocation whose tail is never read: its words would flip the XOR only if read)."""
    n = (1 << 24) + 16 * 12345
    buf = torch.zeros(n // 4 + 4096, dtype=torch.int32, device="cuda")
    buf[n // 4:] = 0x9E3779B9 - (1 << 32)  # the pattern the kernel stores on; never read when in bounds
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    log("stream_read ragged")
    qm.moe_stream_read(buf, n, sink)
    torch.cuda.synchronize()
    assert sink.cpu().tolist() == [7, 7, 7, 7]


@pytest.mark.parametrize("T,alias", [(1, False), (5, True)])
def test_residual_rmsnorm_matches_torch(T, alias):
    """The stack's chaining kernel against torch's widening + add + rms_norm + bf16 rounding: equal up to one
    bf16 ulp (the fp32 sum of squares is formed in another order), in place (y = x) or not."""
    H = 3584
    g = torch.Generator().manual_seed(5)
    x = torch.randn(T, H, generator=g).to(torch.bfloat16).cuda()
    out = torch.randn(T, H, generator=g).cuda()
    want = torch.nn.functional.rms_norm(x.float() + out, (H,), eps=1e-6).to(torch.bfloat16)
    y = x if alias else torch.empty_like(x)
    log(f"residual_rmsnorm T={T} alias={alias}")
    qm.moe_residual_rmsnorm(out, x, y)
    a = y.view(torch.int16).cpu().numpy().astype(np.int32)
    b = want.view(torch.int16).cpu().numpy().astype(np.int32)
    assert np.max(np.abs(a - b)) <= 1
