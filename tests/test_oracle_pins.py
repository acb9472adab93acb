"""Pins of the CPU oracle to things other than itself (CPU only).

Each test ties one oracle function to a value the pages print, to brute force, to a
closed form, to a textbook bound or to an invariant, chosen so that a plausible slip
(dropped term, wrong sign, swapped index, transposed operand, wrong nibble order,
wrong tie rule) fails at least one of them.
"""
import json
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(12345)


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- helpers (test-side, independent)

def pack_block(d_f16: np.float16, q: np.ndarray) -> np.ndarray:
    """Build an 18-byte IQ4_NL block by hand: fp16 scale, then byte j = q[j] | q[j+16] << 4."""
    q = np.asarray(q, np.uint8)
    assert q.shape == (32,) and q.max() < 16
    out = np.empty(18, np.uint8)
    out[:2] = np.frombuffer(np.float16(d_f16).tobytes(), np.uint8)
    out[2:] = q[:16] | (q[16:] << 4)
    return out


def np_dequant(blocks: np.ndarray) -> np.ndarray:
    """Independent numpy decode of GGUF IQ4_NL blocks to float64 (exact values)."""
    levels = np.array(golden("iq4nl_codebook.json")["levels"], np.float64)
    b = np.asarray(blocks, np.uint8).reshape(-1, 18)
    d = b[:, :2].copy().view(np.float16).astype(np.float64).reshape(-1, 1)
    qs = b[:, 2:]
    idx = np.concatenate([qs & 15, qs >> 4], axis=1)
    return (d * levels[idx]).reshape(-1)


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    return (np.asarray(u16, np.uint32) << 16).view(np.float32).astype(np.float64)


def nearest_bf16_f64(v: float) -> float:
    """Round a float64 that is exactly an fp32 value to the nearest bf16, ties to even, by
    comparing the exact distances to its two bf16 neighbours."""
    f = np.float32(v)
    u = int(np.array([f]).view(np.uint32)[0])
    lo_u = u & 0xFFFF0000
    hi_u = lo_u + 0x10000
    lo = float(np.array([lo_u], np.uint32).view(np.float32)[0])
    hi = float(np.array([hi_u], np.uint32).view(np.float32)[0])
    dl, dh = abs(Fraction(float(f)) - Fraction(lo)), abs(Fraction(hi) - Fraction(float(f)))
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if ((lo_u >> 16) & 1) == 0 else hi


# ---------------------------------------------------------------- codec

def test_codebook_matches_printed_levels():
    g = golden("iq4nl_codebook.json")
    assert oracle.codebook() == g["levels"]
    assert g["block_bytes"] * 8 / g["weights_per_block"] == g["bits_per_weight"]


def test_f16_decode_matches_ieee_binary16_for_every_finite_pattern():
    pats = np.arange(65536, dtype=np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_value(int(p)) for p in pats])
    finite = np.isfinite(ref)
    assert np.array_equal(got[finite], ref[finite])
    assert np.all(np.isinf(got[~finite & ~np.isnan(ref)]))


def test_bf16_round_trip_and_round_to_nearest_even():
    # every bf16 pattern decodes to the upper half of an fp32 and re-encodes to itself
    for b in list(range(0, 65536, 97)) + [0x3F80, 0xBF80, 0x7F7F, 0x0001, 0x8001]:
        v = oracle.bf16_value(b)
        if math.isfinite(v):
            assert oracle.to_bf16(v) == b
    # random fp32 values and exact halfway cases against exact nearest-even rounding
    vals = list(RNG.standard_normal(3000).astype(np.float32))
    for base in (0x3F800000, 0x40490000, 0xC1230000, 0x00810000):
        for low in (0x8000, 0x7FFF, 0x8001, 0x18000, 0x0000):
            vals.append(np.array([base + low], np.uint32).view(np.float32)[0])
    for f in vals:
        want = nearest_bf16_f64(float(f))
        got = float(bf16_bits_to_f64(np.array([oracle.to_bf16(float(f))], np.uint16))[0])
        assert got == want, (float(f), got, want)


def test_dequant_of_hand_built_blocks_nibble_order_and_sign():
    levels = golden("iq4nl_codebook.json")["levels"]
    q = np.array([(7 * j + 3) % 16 for j in range(32)], np.uint8)
    q[0], q[31] = 0, 15  # the extreme levels -127 and 113
    for d in (np.float16(0.0009765625), np.float16(-3.5), np.float16(6.1e-5), np.float16(0.0)):
        blk = pack_block(d, q)
        got = oracle.dequant(blk).astype(np.float64)
        want = np.array([float(d) * levels[int(k)] for k in q])
        assert np.array_equal(got, want), d
    # weight 0 and weight 16 share byte 0: low nibble first
    q2 = np.zeros(32, np.uint8)
    q2[16] = 15
    got = oracle.dequant(pack_block(np.float16(1.0), q2))
    assert got[0] == -127 and got[16] == 113 and got[1] == -127


def test_dequant_is_exact_in_fp32_for_every_finite_scale():
    """fp16 (11 significant bits) times a level (<= 7 bits) is exact in fp32: check all scales."""
    levels = np.array(golden("iq4nl_codebook.json")["levels"], np.float64)
    d = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float64)
    d = d[np.isfinite(d)]
    prod = d[:, None] * levels[None, :]
    assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod)
    # and the oracle's dequant returns exactly that product, on a sample of scales
    sel = d[:: 257]
    blocks = np.concatenate([pack_block(np.float16(s), np.arange(32) % 16) for s in sel])
    got = oracle.dequant(blocks).astype(np.float64)
    want = np.concatenate([s * levels[np.arange(32) % 16] for s in sel])
    assert np.array_equal(got, want)


def test_dequant_bf16_mode_is_nearest_even_bf16_of_the_exact_weight():
    blocks = synth.iq4nl_blocks(7, 1, 64)
    exact = np_dequant(blocks)
    got = oracle.dequant(blocks, oracle.BF16).astype(np.float64)
    want = np.array([nearest_bf16_f64(v) for v in exact])
    assert np.array_equal(got, want)


def test_dequant_matches_independent_numpy_decode_on_generated_weights():
    blocks = synth.iq4nl_blocks(3, 2, 4096)
    assert np.array_equal(oracle.dequant(blocks).astype(np.float64), np_dequant(blocks))


def test_encoder_round_trip_of_exactly_representable_blocks():
    """A block built as d*level (index 0 present) encodes back to the same bytes."""
    levels = np.array(golden("iq4nl_codebook.json")["levels"], np.float64)
    for d in (np.float16(0.00042), np.float16(-0.00031), np.float16(1.5)):
        q = RNG.integers(0, 16, 32).astype(np.uint8)
        q[5] = 0
        w = (float(d) * levels[q]).astype(np.float32)
        blk = synth.encode_iq4nl(w)
        assert np.array_equal(oracle.dequant(blk), w)


# ---------------------------------------------------------------- router

def test_router_logits_within_textbook_bound_of_exact_dot():
    H, E, T = 3584, 8, 3
    x = synth.normal_bf16(1, 9, T * H).reshape(T, H)
    W = synth.normal_f32(1, 10, E * H, 0.0, 0.02).reshape(E, H)
    got = oracle.router_logits(x, W).astype(np.float64)
    xv = bf16_bits_to_f64(x)
    u = 2.0 ** -24
    depth = H // 64 + 6  # longest chain: H/64 fused adds per partial, then 6 pairwise levels
    gamma = depth * u / (1 - depth * u)
    for t in range(T):
        for e in range(E):
            prods = xv[t] * W[e].astype(np.float64)  # exact: 8-bit x 24-bit significands
            exact = math.fsum(prods)
            assert abs(got[t, e] - exact) <= gamma * np.abs(prods).sum()


def test_router_logits_exact_when_every_partial_sum_is_exact():
    """Small integers: every partial sum is representable, so any order gives the exact dot.
    A dropped, duplicated or misplaced term changes the result."""
    H, E = 512, 5
    xi = RNG.integers(-8, 9, (2, H)).astype(np.float32)
    wi = RNG.integers(-8, 9, (E, H)).astype(np.float32)
    x = (xi.view(np.uint32) >> 16).astype(np.uint16)
    got = oracle.router_logits(x, wi)
    assert np.array_equal(got.astype(np.float64), xi.astype(np.float64) @ wi.T.astype(np.float64))


def test_router_logits_order_is_the_stated_one():
    """Terms chosen so that fp32 rounding depends on grouping: a big term in partial 0 then
    small terms in later m steps of the same partial are absorbed one at a time; placing
    them in other partials would keep them.  The value below is computed by hand."""
    H = 512
    xs = np.zeros(H, np.float32)
    W = np.zeros((1, H), np.float32)
    xs[0] = 1.0
    W[0, 0] = 2.0 ** 24           # partial 0, m = 0, c = 0
    xs[1] = 1.0
    W[0, 1] = 1.0                 # partial 0, m = 0, c = 1: 2^24 + 1 -> 2^24 (ties to even)
    xs[256] = 1.0
    W[0, 256] = 1.0               # partial 0, m = 1, c = 0: absorbed again
    xs[4] = 1.0
    W[0, 4] = 1.0                 # partial 1: kept until the pairwise stage
    xs[8] = 1.0
    W[0, 8] = 1.0                 # partial 2
    # partials: p0 = 2^24, p1 = 1, p2 = 1. Pairwise: s=32..4 leave p0..p3 as is in lane 0's
    # chain (others are zero); s=2: p0 + p2 = 2^24 + 1 -> 2^24; s=1: (p0+p2) + (p1+p3) = 2^24 + 1 -> 2^24
    x = (xs.view(np.uint32) >> 16).astype(np.uint16).reshape(1, H)
    assert float(oracle.router_logits(x, W)[0, 0]) == 2.0 ** 24
    # the same terms with the small ones paired first (p1 and p3) sum to 2^24 + 2
    xs2, W2 = xs.copy(), W.copy()
    xs2[8], W2[0, 8] = 0.0, 0.0
    xs2[12], W2[0, 12] = 1.0, 1.0  # partial 3 pairs with partial 1 at s = 2
    x2 = (xs2.view(np.uint32) >> 16).astype(np.uint16).reshape(1, H)
    assert float(oracle.router_logits(x2, W2)[0, 0]) == 2.0 ** 24 + 2


def _exp_exact(y: float) -> Decimal:
    getcontext().prec = 50
    return Decimal(y).exp()


def test_exp_spec_within_one_ulp_of_exact():
    ys = list(np.linspace(-200, 200, 401)) + list(RNG.uniform(-40, 40, 600)) + [0.0, 1.0, -1.0, 1e-300, 0.5 * math.log(2)]
    for y in ys:
        got = oracle.exp_spec(float(y))
        ex = _exp_exact(float(y))
        ulp = math.ulp(float(ex))
        assert abs(Decimal(got) - ex) <= Decimal(ulp), y
    assert oracle.exp_spec(0.0) == 1.0
    assert oracle.exp_spec(201.0) == math.inf and oracle.exp_spec(-201.0) == 0.0


def test_sigmoid_within_one_fp32_ulp_and_monotone():
    getcontext().prec = 50
    ls = np.concatenate([RNG.uniform(-30, 30, 2000), np.linspace(-1, 1, 201), [0.0, 17.0, 88.0, -88.0, -104.0]]).astype(np.float32)
    for l in ls:
        got = oracle.sigmoid(float(l))
        ex = 1 / (1 + Decimal(-float(l)).exp())
        ulp = float(np.spacing(np.float32(abs(float(ex)))))
        assert abs(Decimal(got) - ex) <= Decimal(ulp), l
    assert oracle.sigmoid(0.0) == 0.5
    grid = np.sort(np.concatenate([np.linspace(-20, 20, 20001), RNG.uniform(-20, 20, 5000)]).astype(np.float32))
    vals = np.array([oracle.sigmoid(float(v)) for v in grid])
    assert np.all(np.diff(vals) >= 0)
    assert oracle.sigmoid(200.0) == 1.0 and oracle.sigmoid(-200.0) == 0.0


def _brute_route(scores, bias, K, scale):
    """Full sort by (selection score desc, index asc); weights from unbiased scores."""
    sel = scores + (bias if bias is not None else 0)
    E = scores.shape[0]
    order = sorted(range(E), key=lambda e: (-float(sel[e]), e))
    ids = order[:K]
    S = np.float32(0)
    for e in ids:
        S = np.float32(S + scores[e])
    w = [np.float32(np.float32(scores[e] / S) * np.float32(scale)) for e in ids]
    return ids, w


@pytest.mark.parametrize("K,with_bias", [(2, False), (4, False), (8, True), (1, True)])
def test_route_selection_equals_full_sort(K, with_bias):
    T, H, E = 16, 256, 32
    x = synth.normal_bf16(2, 1, T * H).reshape(T, H)
    W = synth.normal_f32(2, 2, E * H, 0.0, 0.02).reshape(E, H)
    bias = synth.normal_f32(2, 3, E, 0.0, 0.05) if with_bias else None
    ids, w, logits, scores = oracle.route(x, W, K, 2.0, bias)
    assert np.array_equal(scores, np.array([[oracle.sigmoid(float(v)) for v in row] for row in logits], np.float32))
    for t in range(T):
        bids, bw = _brute_route(scores[t], bias, K, 2.0)
        assert list(ids[t]) == bids
        assert np.array_equal(w[t], np.array(bw, np.float32))
        # top-k set equality with a dense argsort
        sel = scores[t] + (bias if bias is not None else 0)
        assert set(ids[t]) == set(np.argsort(-sel, kind="stable")[:K])


def test_route_weights_sum_to_scale_within_bound():
    T, H, E, K = 64, 512, 64, 4
    x = synth.normal_bf16(5, 1, T * H).reshape(T, H)
    W = synth.normal_f32(5, 2, E * H, 0.0, 0.02).reshape(E, H)
    _, w, _, _ = oracle.route(x, W, K, 2.0)
    bound = (2 * K - 1) * 2.0 ** -23 * 2.0
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 2.0) <= bound)
    assert np.all(w > 0)


def test_route_special_cases():
    H = 256
    x = synth.normal_bf16(6, 1, 3 * H).reshape(3, H)
    # one expert, top-1: the weight is exactly the scale
    W1 = synth.normal_f32(6, 2, H, 0.0, 0.02).reshape(1, H)
    ids, w, _, _ = oracle.route(x, W1, 1, 2.0)
    assert np.all(ids == 0) and np.all(w == 2.0)
    # K = E, no bias: every expert, w_e = 2 s_e / sum s (in slot order of descending score)
    E = 6
    W = synth.normal_f32(6, 3, E * H, 0.0, 0.02).reshape(E, H)
    ids, w, _, scores = oracle.route(x, W, E, 2.0)
    for t in range(3):
        assert sorted(ids[t]) == list(range(E))
        ref = 2.0 * scores[t][ids[t]].astype(np.float64) / scores[t].astype(np.float64).sum()
        assert np.allclose(w[t], ref, rtol=4e-7, atol=0)
    # identical router rows tie exactly: the lower expert index is taken first
    Wt = np.repeat(W[:1], 4, axis=0)
    ids, w, _, _ = oracle.route(x, Wt, 2, 2.0)
    assert np.all(ids == [0, 1]) and np.all(w == 1.0)
    # the bias moves selection but not the weights' source
    bias = np.array([0, 0, 0, 10.0], np.float32)
    ids, w, _, scores = oracle.route(x, Wt, 2, 2.0, bias)
    assert np.all(ids == [3, 0]) and np.all(w == 1.0)


# ---------------------------------------------------------------- bucketing

def test_bucket_is_the_stable_sort_by_expert():
    for T, K, E in [(4, 2, 8), (128, 4, 64), (333, 8, 256), (1, 4, 64), (0, 4, 8)]:
        ids = RNG.integers(0, E, (T, K)).astype(np.int32)
        # make duplicates within a token impossible, as routing does
        for t in range(T):
            ids[t] = RNG.choice(E, K, replace=False)
        counts, offsets, perm, pos = oracle.bucket(ids, E)
        flat = ids.reshape(-1)
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts) and offsets[-1] == T * K
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))
        assert np.array_equal(pos[perm], np.arange(T * K))


# ---------------------------------------------------------------- expert FFN and layer

def np_expert(x_bits, blocks, H, F, mode=1):
    """Dense float64 FFN from an independent decode (mode 2 rounds weights and h to bf16)."""
    w = np_dequant(blocks)
    if mode == 2:
        w = np.array([nearest_bf16_f64(v) for v in w]) if w.size < 200000 else _vec_bf16(w)
    Wg = w[: F * H].reshape(F, H)
    Wu = w[F * H: 2 * F * H].reshape(F, H)
    Wd = w[2 * F * H:].reshape(H, F)
    xv = bf16_bits_to_f64(x_bits)
    g, u = Wg @ xv, Wu @ xv
    h = g / (1 + np.exp(-g)) * u
    if mode == 2:
        h = _vec_bf16(h.astype(np.float32).astype(np.float64))
    return Wd @ h


def _vec_bf16(v):
    """Vectorised nearest-even bf16 of fp32-exact float64 values, via the two neighbours."""
    f = np.asarray(v, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lo_u = (u & 0xFFFF0000).astype(np.uint32)
    hi_u = (lo_u.astype(np.uint64) + 0x10000).astype(np.uint32)
    lo = lo_u.view(np.float32).astype(np.float64)
    hi = hi_u.view(np.float32).astype(np.float64)
    fv = f.astype(np.float64)
    dl, dh = np.abs(fv - lo), np.abs(hi - fv)
    even = ((lo_u >> 16) & 1) == 0
    return np.where(dl < dh, lo, np.where(dh < dl, hi, np.where(even, lo, hi)))


def test_expert_matches_dense_numpy_decode():
    H, F = 256, 128
    blocks = synth.iq4nl_blocks(8, 1, 3 * F * H // 32)
    x = synth.normal_bf16(8, 2, H)
    for mode in (1, 2):
        y = oracle.expert(x, blocks, H, F, mode)
        ref = np_expert(x, blocks, H, F, mode)
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-15), mode


def test_expert_closed_form_on_constant_input():
    """x = 1 everywhere and one block per row: g_f = d_f * sum(levels of row f), etc."""
    H, F = 32, 32
    levels = golden("iq4nl_codebook.json")["levels"]
    x = np.full(H, 0x3F80, np.uint16)  # bf16 1.0
    rows = []
    qg = [(f * 5 + np.arange(32)) % 16 for f in range(F)]
    qu = [(f * 3 + 2 * np.arange(32)) % 16 for f in range(F)]
    qd = [(n + np.arange(32) * 7) % 16 for n in range(H)]
    dg, du, dd = np.float16(0.001), np.float16(-0.0005), np.float16(0.002)
    blocks = np.concatenate([pack_block(dg, q) for q in qg] + [pack_block(du, q) for q in qu] +
                            [pack_block(dd, q) for q in qd])
    g = [float(dg) * sum(levels[int(k)] for k in q) for q in qg]
    u = [float(du) * sum(levels[int(k)] for k in q) for q in qu]
    h = [gi / (1 + math.exp(-gi)) * ui for gi, ui in zip(g, u)]
    want = [sum(float(dd) * levels[int(q[f])] * h[f] for f in range(F)) for q in qd]
    got = oracle.expert(x, blocks, H, F)
    assert np.allclose(got, want, rtol=1e-12, atol=0)


def _tiny():
    s = synth.WORKLOADS["tiny"]
    inp = synth.layer_inputs(s)
    x = synth.tokens(s, s.tokens)
    return s, inp, x


@pytest.mark.parametrize("mode", [1, 2])
def test_layer_equals_dense_masked_brute_force(mode):
    """All experts on every token, masked by the routing weights (full-sort routing)."""
    s, inp, x = _tiny()
    out, ids, w = oracle.layer(x, inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn, mode=mode)
    eb = s.expert_bytes
    _, _, _, scores = oracle.route(x, inp["gate_w"], s.top_k)
    for t in range(s.tokens):
        bids, bw = _brute_route(scores[t], None, s.top_k, 2.0)
        mask = np.zeros(s.n_experts)
        mask[bids] = np.array(bw, np.float64)
        dense = sum(mask[e] * np_expert(x[t], inp["arena"][e * eb:(e + 1) * eb], s.hidden, s.ffn, mode)
                    for e in range(s.n_experts))
        dense = dense + np_expert(x[t], inp["shared"], s.hidden, s.ffn, mode)
        assert list(ids[t]) == bids
        assert np.allclose(out[t].astype(np.float64), dense, rtol=2 ** -23, atol=1e-12)


def test_layer_special_cases():
    s, inp, x = _tiny()
    eb = s.expert_bytes
    # identical experts with K = E: sum of weights is 2, so out = 2 * FFN(x) + shared(x)
    E = 4
    one = inp["arena"][:eb]
    arena = np.tile(one, E)
    W = inp["gate_w"][:E]
    out, _, w = oracle.layer(x, W, arena, inp["shared"], E, s.ffn)
    for t in range(s.tokens):
        ref = 2 * np_expert(x[t], one, s.hidden, s.ffn) + np_expert(x[t], inp["shared"], s.hidden, s.ffn)
        assert np.allclose(out[t], ref, rtol=1e-5, atol=1e-7)
    # all scales zero: every weight is zero, so the output is exactly zero
    zero = inp["arena"].copy().reshape(-1, 18)
    zero[:, :2] = 0
    zs = inp["shared"].copy().reshape(-1, 18)
    zs[:, :2] = 0
    out, _, _ = oracle.layer(x, inp["gate_w"], zero.reshape(-1), zs.reshape(-1), s.top_k, s.ffn)
    assert np.all(out == 0)
    # no shared expert: one token, top-1 of one expert gives exactly 2 * FFN(x)
    out, ids, w = oracle.layer(x[:1], inp["gate_w"][:1], inp["arena"][:eb], None, 1, s.ffn)
    ref = 2 * np_expert(x[0], inp["arena"][:eb], s.hidden, s.ffn)
    assert np.allclose(out[0], ref.astype(np.float32), rtol=2 ** -23, atol=0)
    # token order: permuting tokens permutes rows exactly
    perm = np.array([2, 0, 3, 1])
    out1, _, _ = oracle.layer(x, inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn)
    out2, _, _ = oracle.layer(x[perm], inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn)
    assert np.array_equal(out1[perm], out2)


# ---------------------------------------------------------------- size arithmetic printed on the pages

def test_page_size_arithmetic():
    g = golden("page_sizes.json")
    sh = g["xing4_shape"]
    H, F = sh["hidden"], sh["expert_ffn"]
    blk = golden("iq4nl_codebook.json")["block_bytes"]
    matrix = F * H // 32 * blk
    assert matrix == g["matrix_bytes"]["value"]
    assert 3 * matrix == g["routed_expert_bytes"]["value"] == synth.WORKLOADS["xing4"].expert_bytes
    assert round(3 * matrix / 2 ** 20, 3) == g["distinct_expert_fill"]["mib_per_expert"]
    assert round(g["distinct_expert_fill"]["mib_total"] / g["distinct_expert_fill"]["experts"], 3) == 5.906
    ws = g["per_token_working_set_gib"]
    assert ws["experts"] == 38 * sh["top_k"]
    assert round(ws["experts"] * 3 * matrix / 2 ** 30, 3) == ws["value"]
    kv = g["kv_bytes_per_token"]
    assert kv["layers"] * kv["values_per_layer"] * kv["bytes_per_value"] == kv["value"]
    st = g["streamed_expert_bytes_4bit"]
    pre = synth.WORKLOADS["prefill"]
    assert 3 * pre.hidden * pre.ffn == st["params"]
    assert st["params"] * (st["bits"] + st["group_overhead_bits"]) / 8 == pre.expert_bytes
    assert round(pre.expert_bytes / 1e6, 2) == st["mbytes"]


# ---------------------------------------------------------------- stack chaining glue (not the layer)

def _bf16_bits(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_residual_rmsnorm_closed_forms():
    H = 256
    # a constant row normalises to +-1 exactly (eps = 0), from x or from out alike
    for c in (3.0, -0.125, 1e-3):
        x = np.tile(_bf16_bits([c]), (1, H))
        y = oracle.residual_rmsnorm(x, np.zeros((1, H), np.float32), eps=0.0)
        assert np.all(y == _bf16_bits([np.sign(c)])), c
        y2 = oracle.residual_rmsnorm(np.zeros((1, H), np.uint16), np.full((1, H), np.float32(oracle.bf16_value(
            int(_bf16_bits([c])[0])))), eps=0.0)
        assert np.array_equal(y, y2)
    # h = (3, 4, 0, ...): mean square 25/H, so y = (3, 4) * sqrt(H)/5 = (9.6, 12.8) -> nearest bf16 (spacing 1/16 in [8, 16)) 9.625, 12.8125
    out = np.zeros((1, H), np.float32)
    out[0, :2] = (3.0, 4.0)
    y = oracle.residual_rmsnorm(np.zeros((1, H), np.uint16), out, eps=0.0)
    assert oracle.bf16_value(int(y[0, 0])) == 9.625 and oracle.bf16_value(int(y[0, 1])) == 12.8125
    assert np.all(y[0, 2:] == 0)
    # the residual add uses both inputs: x = (3, 0, ...) and out = (0, 4, ...) give the same row
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = _bf16_bits([3.0])[0]
    out = np.zeros((1, H), np.float32)
    out[0, 1] = 4.0
    assert np.array_equal(oracle.residual_rmsnorm(x, out, eps=0.0), y)
    # eps enters under the root: a row of ones with eps = 3 gives 1/sqrt(1 + 3) = 0.5
    y = oracle.residual_rmsnorm(np.tile(_bf16_bits([1.0]), (1, H)), np.zeros((1, H), np.float32), eps=3.0)
    assert np.all(y == _bf16_bits([0.5]))


def test_residual_rmsnorm_scale_invariant_and_rowwise():
    rng = np.random.default_rng(3)
    H = 512
    x = _bf16_bits(rng.standard_normal((3, H)))
    out = rng.standard_normal((3, H)).astype(np.float32)
    y = oracle.residual_rmsnorm(x, out, eps=0.0)
    # scaling a row's inputs by a power of two leaves the normalised row unchanged (eps = 0)
    xs = _bf16_bits(np.array([oracle.bf16_value(int(v)) for v in x[1]], np.float32) * 8.0)
    ys = oracle.residual_rmsnorm(xs[None, :], out[1:2] * 8.0, eps=0.0)
    assert np.array_equal(ys[0], y[1])
    # rows are independent
    assert np.array_equal(oracle.residual_rmsnorm(x[2:3], out[2:3], eps=0.0)[0], y[2])


def test_sigmoid_many_is_sigmoid_elementwise():
    l = np.array([-30.0, -1.5, 0.0, 2.0 ** -20, 7.25, 30.0], np.float32)
    assert np.array_equal(oracle.sigmoid_many(l), np.array([oracle.sigmoid(float(v)) for v in l], np.float32))


# ---------------------------------------------------------------- sigmoid-gated shared expert, dense block

def test_shared_gate_closed_forms():
    """The shared expert scaled by sigmoid(x . g): g = 0 gives exactly 1/2; g = +x gives a logit of about
    +H (sigmoid rounds to 1: the ungated layer, bit for bit); g = -x a logit below -200 (sigmoid is 0: the
    layer without a shared expert, bit for bit); in between, the dense masked brute force with the gate."""
    s, inp, x = _tiny()
    base, ids, w = oracle.layer(x, inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn)
    routed, _, _ = oracle.layer(x, inp["gate_w"], inp["arena"], None, s.top_k, s.ffn)
    for t in range(s.tokens):
        xf = bf16_bits_to_f64(x[t]).astype(np.float32)
        up, _, _ = oracle.layer(x[t:t + 1], inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn,
                                shared_gate=xf)
        assert np.array_equal(up[0].view(np.uint32), base[t].view(np.uint32))
        down, _, _ = oracle.layer(x[t:t + 1], inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn,
                                  shared_gate=-xf)
        assert np.array_equal(down[0].view(np.uint32), routed[t].view(np.uint32))
    half, hid, hw = oracle.layer(x, inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn,
                                 shared_gate=np.zeros(s.hidden, np.float32))
    assert np.array_equal(hid, ids) and np.array_equal(hw, w)  # the gate does not touch the routing
    eb = s.expert_bytes
    rng = np.random.default_rng(8)
    g = (rng.standard_normal(s.hidden) * 0.05).astype(np.float32)
    gated, _, _ = oracle.layer(x, inp["gate_w"], inp["arena"], inp["shared"], s.top_k, s.ffn, shared_gate=g)
    for t in range(s.tokens):
        ysh = np_expert(x[t], inp["shared"], s.hidden, s.ffn)
        yr = sum(float(w[t, k]) * np_expert(x[t], inp["arena"][ids[t, k] * eb:(ids[t, k] + 1) * eb], s.hidden,
                                            s.ffn) for k in range(s.top_k))
        assert np.allclose(half[t], yr + 0.5 * ysh, rtol=2 ** -22, atol=1e-12)
        # the gate logit: the exact dot of the bf16 token with the fp32 row, within the fp32 dot bound
        exact = float(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(bf16_bits_to_f64(x[t]), g)))
        sg = 1.0 / (1.0 + math.exp(-exact))
        assert np.allclose(gated[t], yr + sg * ysh, rtol=1e-6, atol=1e-9)


def test_dense_block_is_the_shared_ffn_alone():
    """E = 0, K = 0, one always-on expert: the dense FFN block, out = FFN(x) per token (the expert FFN
    itself is pinned above against an independent decode and closed forms)."""
    s, inp, x = _tiny()
    out, ids, w = oracle.layer(x, np.zeros((0, s.hidden), np.float32), None, inp["shared"], 0, s.ffn)
    assert ids.shape == (s.tokens, 0)
    for t in range(s.tokens):
        want = oracle.expert(x[t], inp["shared"], s.hidden, s.ffn).astype(np.float32)
        assert np.array_equal(out[t].view(np.uint32), want.view(np.uint32))
    outb, _, _ = oracle.layer(x, np.zeros((0, s.hidden), np.float32), None, inp["shared"], 0, s.ffn,
                              mode=oracle.BF16)
    for t in range(s.tokens):
        want = oracle.expert(x[t], inp["shared"], s.hidden, s.ffn, oracle.BF16).astype(np.float32)
        assert np.array_equal(outb[t].view(np.uint32), want.view(np.uint32))


# ---------------------------------------------------------------- W4A8: fp16 rounding, Q8_0, integer block dots

def test_to_f16_is_numpy_nearest_even():
    """fp32 -> fp16 against numpy's conversion (IEEE round to nearest even) on every binade, subnormals,
    exact halfway points and overflow."""
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f) & (np.abs(f) < 1e6)]
    mids = (np.arange(0, 1 << 15, 37, dtype=np.uint32) << 13 | 0x1000).view(np.float32)  # halfway points
    f = np.concatenate([f, mids[np.isfinite(mids)], np.float32([65504.0, 65519.99, 65520.0, 6.0e-8, 2.0 ** -25,
                                                               3 * 2.0 ** -26, -0.0])])
    with np.errstate(over="ignore"):  # 65520 and above round to infinity, as intended
        want = f.astype(np.float16).view(np.uint16)
    got = np.array([oracle.to_f16(float(v)) for v in f], np.uint16)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, (f[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_q8_0_closed_forms():
    # a zero block: scale 0, codes 0
    q, d = oracle.quantize_q8_0(np.zeros(32, np.float32))
    assert d[0] == 0 and np.all(q == 0)
    # a block that is exactly c * q with max |q| = 127 and c a power of two: lossless
    rng = np.random.default_rng(1)
    for c in (1.0, 2.0 ** -7, 2.0 ** 3):
        qr = rng.integers(-127, 128, 32)
        qr[5] = -127
        q, d = oracle.quantize_q8_0((qr * c).astype(np.float32))
        assert np.array_equal(q, qr.astype(np.int8)) and oracle.f16_value(int(d[0])) == c
    # halves round away from zero: amax 127 gives id = 1, so 2.5 -> 3, -2.5 -> -3, 0.5 -> 1, -1.5 -> -2
    x = np.zeros(32, np.float32)
    x[:5] = (127.0, 2.5, -2.5, 0.5, -1.5)
    q, d = oracle.quantize_q8_0(x)
    assert list(q[:5]) == [127, 3, -3, 1, -2]
    # the scale is stored rounded to fp16; codes stay within +-127 and within half a step of x / d32
    x = (rng.standard_normal(32 * 500) * 3).astype(np.float32)
    q, d = oracle.quantize_q8_0(x)
    xb = x.reshape(-1, 32).astype(np.float64)
    d32 = (np.abs(x.reshape(-1, 32)).max(axis=1) / np.float32(127)).astype(np.float32)
    assert np.array_equal(d, d32.astype(np.float16).view(np.uint16))
    assert np.abs(q).max() <= 127
    assert np.all(np.abs(q.reshape(-1, 32) - xb / d32[:, None].astype(np.float64)) <= 0.5 + 1e-5)


def _expert_blocks(rng, rows, cols):
    """Random IQ4_NL rows: fp16 scales of either sign, random nibbles."""
    blk = rng.integers(0, 256, (rows, cols // 32, 18)).astype(np.uint8)
    d = (rng.standard_normal((rows, cols // 32)) * 0.01).astype(np.float16)
    blk[:, :, :2] = d.view(np.uint8).reshape(rows, cols // 32, 2)
    return blk.reshape(-1)


def test_w4a8_expert_exact_brute_force():
    """A small expert (H = F = 64) in W4A8 mode against exact rational arithmetic: the Q8_0 codes of x (the
    quantizer is pinned above), every block dot as an exact integer times the exact scales, SiLU in double,
    h rounded to fp32 and quantized, the down dots exact."""
    rng = np.random.default_rng(6)
    H = F = 64
    levels = golden("iq4nl_codebook.json")["levels"]
    gate, up, down = _expert_blocks(rng, F, H), _expert_blocks(rng, F, H), _expert_blocks(rng, H, F)
    expert = np.concatenate([gate, up, down])
    x = _bf16_bits(rng.standard_normal(H))
    xf = np.array([oracle.bf16_value(int(v)) for v in x], np.float32)
    xq, xd = oracle.quantize_q8_0(xf)

    def exact_dot(rowblocks, q, dq):
        tot = Fraction(0)
        for b in range(len(dq)):
            blk = rowblocks[18 * b:18 * b + 18]
            dw = Fraction(float(np.frombuffer(blk[:2].tobytes(), np.float16)[0]))
            lv = [levels[(blk[2 + (k & 15)] & 15) if k < 16 else (blk[2 + (k & 15)] >> 4)] for k in range(32)]
            s = sum(lv[k] * int(q[32 * b + k]) for k in range(32))
            tot += dw * Fraction(oracle.f16_value(int(dq[b]))) * s
        return tot

    rb = H // 32 * 18
    h = np.empty(F, np.float32)
    for f in range(F):
        g = float(exact_dot(gate[f * rb:(f + 1) * rb], xq, xd))
        u = float(exact_dot(up[f * rb:(f + 1) * rb], xq, xd))
        h[f] = np.float32(g / (1.0 + math.exp(-g)) * u)
    hq, hd = oracle.quantize_q8_0(h)
    rbd = F // 32 * 18
    want = np.array([float(exact_dot(down[n * rbd:(n + 1) * rbd], hq, hd)) for n in range(H)])
    got = oracle.expert(x, expert, H, F, oracle.W4A8)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-15)


def test_w4a8_residual_matches_the_pages_range():
    """The W4A8 expert against the same expert with bf16 activations kept exact (FP32 mode), on the Xing4 expert
    shape: the model card's single-expert check reports max_rel_err 0.011-0.020 and correlation 0.99994 for its
    Q8_0 path; the synthetic expert lands in the same range (max_rel within a factor ~2, corr >= 0.9999)."""
    g = golden("q8_0_residual.json")
    s = synth.WORKLOADS["xing4"]
    inp = synth.layer_inputs(s)
    eb = s.expert_bytes
    x = synth.tokens(s, 4, first=3)
    lo = min(r["max_rel_err"] for r in g["rows"]) / 3
    hi = max(r["max_rel_err"] for r in g["rows"]) * 2
    for t in range(4):
        a = oracle.expert(x[t], inp["arena"][5 * eb:6 * eb], s.hidden, s.ffn, oracle.W4A8)
        b = oracle.expert(x[t], inp["arena"][5 * eb:6 * eb], s.hidden, s.ffn, oracle.FP32)
        max_rel = float(np.max(np.abs(a - b)) / np.max(np.abs(b)))
        corr = float(np.corrcoef(a, b)[0, 1])
        assert lo <= max_rel <= hi, max_rel
        assert corr >= 0.9999, corr


# ---------------------------------------------------------------- other codecs: IQ4_XS, packed 3-bit affine

def _iq4xs_superblock(d, ls, nib):
    """Build a 136-byte IQ4_XS super-block by hand from the format's description: fp16 d, the high 2 bits of
    each 6-bit sub-block scale at bits 2i of a uint16, the low 4 bits in nibble i%2 of byte i/2, then 8 blocks
    of 16 bytes of indices (IQ4_NL order)."""
    out = np.zeros(136, np.uint8)
    out[:2] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
    sh = sum(((int(v) >> 4) & 3) << (2 * i) for i, v in enumerate(ls))
    out[2:4] = (sh & 255, sh >> 8)
    for i, v in enumerate(ls):
        out[4 + i // 2] |= (int(v) & 15) << (4 * (i % 2))
    for ib in range(8):
        q = np.asarray(nib[ib], np.uint8)
        out[8 + 16 * ib: 24 + 16 * ib] = q[:16] | (q[16:] << 4)
    return out


def test_iq4xs_hand_built_superblock():
    """Eight distinct sub-block scales (each bit of the split 6-bit field used) and known indices: every weight
    is d * (ls - 32) * level, exact in fp32."""
    levels = golden("iq4nl_codebook.json")["levels"]
    rng = np.random.default_rng(9)
    ls = [0, 63, 32, 1, 17, 40, 50, 9]
    nib = [rng.integers(0, 16, 32) for _ in range(8)]
    blk = _iq4xs_superblock(0.5, ls, nib)
    w = oracle.dequant_codec(oracle.IQ4_XS, blk, 256)
    want = np.array([0.5 * (ls[ib] - 32) * levels[nib[ib][j]] for ib in range(8) for j in range(32)])
    assert np.array_equal(w, want)
    assert np.array_equal(w.astype(np.float32).astype(np.float64), w)  # exact in fp32
    # 136 bytes per 256 weights: 4.25 bits per weight
    assert oracle.codec_row_bytes(oracle.IQ4_XS, 256) * 8 / 256 == 4.25


def test_iq4xs_expert_equals_iq4nl_expert_when_scales_coincide():
    """An IQ4_XS expert whose sub-block scales d * (ls - 32) are fp16 values gives exactly the IQ4_NL expert
    with those scales and the same indices (the IQ4_NL expert is pinned above)."""
    rng = np.random.default_rng(10)
    H, F = 256, 256
    x = _bf16_bits(rng.standard_normal(H))

    def rows(n, cols):
        xs, nl = [], []
        for _ in range(n):
            for sb in range(cols // 256):
                ls = rng.integers(20, 45, 8)
                nib = [rng.integers(0, 16, 32) for _ in range(8)]
                d = 2.0 ** -9
                xs.append(_iq4xs_superblock(d, ls, nib))
                for ib in range(8):
                    nl.append(pack_block(np.float16(d * (int(ls[ib]) - 32)), nib[ib]))
        return np.concatenate(xs), np.concatenate(nl)

    gx, gn = rows(F, H)
    ux, un = rows(F, H)
    dx, dn = rows(H, F)
    y_xs = oracle.expert_codec(x, np.concatenate([gx, ux, dx]), H, F, oracle.IQ4_XS)
    y_nl = oracle.expert(x, np.concatenate([gn, un, dn]), H, F)
    assert np.allclose(y_xs, y_nl, rtol=1e-12, atol=1e-15)


def _q3_group(scale, bias, codes):
    """A 28-byte packed 3-bit group: fp16 scale, fp16 bias, the 64 codes as one little-endian bit string."""
    out = np.zeros(28, np.uint8)
    out[:2] = np.frombuffer(np.float16(scale).tobytes(), np.uint8)
    out[2:4] = np.frombuffer(np.float16(bias).tobytes(), np.uint8)
    bits = np.zeros(192, np.uint8)
    for j, c in enumerate(codes):
        bits[3 * j:3 * j + 3] = [(int(c) >> k) & 1 for k in range(3)]
    out[4:] = np.packbits(bits, bitorder="little")
    return out


def test_q3_affine_group_and_size():
    """Hand-built groups (codes in every position and value, both signs of scale and bias): weight =
    scale * q + bias; 28 bytes per 64 weights, and an expert is 7/9 of an IQ4_NL expert -- the SSD streaming
    page's packed-3-bit factor for E = P (b + g) / 8 with b = 3 instead of 4 and g = 0.5."""
    rng = np.random.default_rng(11)
    for scale, bias in ((0.25, -1.0), (-0.0078125, 0.5), (3.0, 0.0)):
        codes = rng.integers(0, 8, 64)
        codes[:8] = np.arange(8)
        w = oracle.dequant_codec(oracle.Q3_AFFINE, _q3_group(scale, bias, codes), 64)
        assert np.array_equal(w, scale * codes.astype(np.float64) + bias)
    assert oracle.codec_row_bytes(oracle.Q3_AFFINE, 64) == 28
    nl = oracle.codec_expert_bytes(oracle.IQ4_NL, 3584, 1024)
    q3 = oracle.codec_expert_bytes(oracle.Q3_AFFINE, 3584, 1024)
    assert Fraction(q3, nl) == Fraction(7, 9)


def test_q3_affine_expert_against_independent_decode():
    """A packed 3-bit expert against a numpy evaluation of the same FFN with weights unpacked here by numpy's
    own bit routine (np.unpackbits, little bit order)."""
    rng = np.random.default_rng(12)
    H, F = 256, 128

    def mat(rows, cols):
        g = []
        for _ in range(rows * cols // 64):
            g.append(_q3_group(float(rng.uniform(0.001, 0.01)), float(rng.uniform(-0.02, 0.02)),
                               rng.integers(0, 8, 64)))
        return np.concatenate(g)

    def unpack(m, rows, cols):
        gr = m.reshape(-1, 28)
        sc = gr[:, :2].copy().view(np.float16).astype(np.float64)
        bi = gr[:, 2:4].copy().view(np.float16).astype(np.float64)
        bits = np.unpackbits(gr[:, 4:], axis=1, bitorder="little").reshape(-1, 64, 3).astype(np.int64)
        q = bits[:, :, 0] + 2 * bits[:, :, 1] + 4 * bits[:, :, 2]
        return (sc * q + bi).reshape(rows, cols)

    gate, up, down = mat(F, H), mat(F, H), mat(H, F)
    x = _bf16_bits(rng.standard_normal(H))
    xv = bf16_bits_to_f64(x)
    g = unpack(gate, F, H) @ xv
    u = unpack(up, F, H) @ xv
    h = g / (1.0 + np.exp(-g)) * u
    want = unpack(down, H, F) @ h
    got = oracle.expert_codec(x, np.concatenate([gate, up, down]), H, F, oracle.Q3_AFFINE)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-13)
