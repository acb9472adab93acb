"""Seeded synthetic inputs for the quantized MoE layer (shared by tests, bench and smoke).

Holds no arithmetic of the layer itself: only counter-based normal variates, their
rounding to bf16 / fp32, and the IQ4_NL *encoding* of N(0, sigma) weight matrices
(``synth.c``).  Both the CPU oracle and the GPU library consume these bytes.

Workloads (shapes from the Xing4.0-29B-A4B model card and design record; the
small case and the prefill case are the method at other sizes):

* ``tiny``     T=4, hidden 256, 8 experts top-2 + 1 shared, ffn 128 (seed 0)
* ``xing4``    T=1 decode, hidden 3584, 64 experts top-4 + 1 shared, ffn 1024 (seed 1)
* ``stack``    38 Xing4 layers, T=1, Zipf(1.1) expert popularity (seed 2)
* ``batch``    T=128 through one Xing4 layer, unbiased routing (seed 3)
* ``prefill``  T=2048, hidden 2048, 256 experts top-8 + 1 shared, ffn 512, Zipf(1.0) (seed 4)

Streams: every tensor is its own stream ``(kind << 40) | (layer << 20) | index`` so
any tensor can be regenerated alone.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

KIND_X, KIND_GATE, KIND_EXPERT, KIND_BIAS = 1, 2, 3, 4
IQ4_NL, IQ4_XS, Q3_AFFINE = 0, 1, 2  # expert codecs
_UNIT = {IQ4_XS: (256, 136), Q3_AFFINE: (64, 28)}  # weights and bytes per super-block / group
WEIGHT_STD = 0.02
BLOCK_BYTES = 18


def build(verbose: bool = False) -> str:
    """Compile libsynth.so with gcc (OpenMP)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           os.path.join(_HERE, "synth.c"), "-o", _LIB_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.synth_normal_f32.argtypes = [u64, u64, i64, dbl, dbl, vp]
    lib.synth_normal_bf16.argtypes = [u64, u64, i64, dbl, dbl, vp]
    lib.synth_iq4nl.argtypes = [u64, u64, i64, dbl, vp]
    lib.synth_encode_iq4nl.argtypes = [vp, i64, vp]
    lib.synth_threads.restype = ctypes.c_int
    lib.synth_codec.argtypes = [ctypes.c_int, u64, u64, i64, dbl, vp]
    _lib = lib
    return lib


def stream_id(kind: int, layer: int = 0, index: int = 0) -> int:
    return (kind << 40) | (layer << 20) | index


def threads() -> int:
    return _load().synth_threads()


def normal_f32(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0,
               out: np.ndarray | None = None) -> np.ndarray:
    out = np.empty(n, np.float32) if out is None else out
    assert out.dtype == np.float32 and out.size == n and out.flags.c_contiguous
    _load().synth_normal_f32(seed, stream, n, mean, std, out.ctypes.data)
    return out


def normal_bf16(seed: int, stream: int, n: int, mean: float = 0.0, std: float = 1.0,
                out: np.ndarray | None = None) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(mean, std) rounded to nearest even."""
    out = np.empty(n, np.uint16) if out is None else out
    assert out.dtype == np.uint16 and out.size == n and out.flags.c_contiguous
    _load().synth_normal_bf16(seed, stream, n, mean, std, out.ctypes.data)
    return out


def iq4nl_blocks(seed: int, stream: int, n_blocks: int, std: float = WEIGHT_STD,
                 out: np.ndarray | None = None) -> np.ndarray:
    out = np.empty(n_blocks * BLOCK_BYTES, np.uint8) if out is None else out
    assert out.dtype == np.uint8 and out.size == n_blocks * BLOCK_BYTES and out.flags.c_contiguous
    _load().synth_iq4nl(seed, stream, n_blocks, std, out.ctypes.data)
    return out


def encode_iq4nl(w: np.ndarray) -> np.ndarray:
    """Encode fp32 weights (a multiple of 32 values, row-major) into IQ4_NL blocks."""
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    assert w.size % 32 == 0
    nb = w.size // 32
    out = np.empty(nb * BLOCK_BYTES, np.uint8)
    _load().synth_encode_iq4nl(w.ctypes.data, nb, out.ctypes.data)
    return out


def codec_blocks(codec: int, seed: int, stream: int, n_weights: int, std: float = WEIGHT_STD,
                 out: np.ndarray | None = None) -> np.ndarray:
    """N(0, std) weights (row-major, rows a multiple of the unit) encoded in an expert codec."""
    if codec == IQ4_NL:
        return iq4nl_blocks(seed, stream, n_weights // 32, std, out)
    unit, nb = _UNIT[codec]
    out = np.empty(n_weights // unit * nb, np.uint8) if out is None else out
    assert out.dtype == np.uint8 and out.size == n_weights // unit * nb and out.flags.c_contiguous
    _load().synth_codec(codec, seed, stream, n_weights // unit, std, out.ctypes.data)
    return out


@dataclass(frozen=True)
class Shape:
    name: str
    tokens: int          # tokens per call
    hidden: int
    n_experts: int
    top_k: int
    ffn: int
    n_shared: int = 1
    routed_scale: float = 2.0
    seed: int = 0
    layers: int = 1      # distinct layers generated for the workload
    zipf_s: float = 0.0  # expert-popularity skew (0 = none)
    codec: int = IQ4_NL  # expert weight codec

    @property
    def blocks_per_matrix(self) -> int:
        return self.ffn * self.hidden // 32

    @property
    def expert_bytes(self) -> int:
        if self.codec == IQ4_NL:
            return 3 * self.blocks_per_matrix * BLOCK_BYTES
        unit, nb = _UNIT[self.codec]
        return 3 * self.ffn * self.hidden // unit * nb


WORKLOADS = {
    "tiny": Shape("tiny", 4, 256, 8, 2, 128, seed=0),
    "xing4": Shape("xing4", 1, 3584, 64, 4, 1024, seed=1, layers=32),
    "stack": Shape("stack", 1, 3584, 64, 4, 1024, seed=2, layers=38, zipf_s=1.1),
    "batch": Shape("batch", 128, 3584, 64, 4, 1024, seed=3),
    "prefill": Shape("prefill", 2048, 2048, 256, 8, 512, seed=4, zipf_s=1.0),
    # a dense FFN block of the same model (no routing: one always-on expert of width 9216)
    "dense": Shape("dense", 1, 3584, 0, 0, 9216, seed=5),
    # the Xing4 layer with experts in the other codecs
    "xing4_xs": Shape("xing4_xs", 1, 3584, 64, 4, 1024, seed=6, codec=IQ4_XS),
    "xing4_q3": Shape("xing4_q3", 1, 3584, 64, 4, 1024, seed=7, codec=Q3_AFFINE),
    "tiny_xs": Shape("tiny_xs", 4, 256, 8, 2, 256, seed=8, codec=IQ4_XS),
    "tiny_q3": Shape("tiny_q3", 4, 256, 8, 2, 128, seed=9, codec=Q3_AFFINE),
}


def tokens(shape: Shape, n: int, first: int = 0, layer: int = 0, seed: int | None = None) -> np.ndarray:
    """Activations x [n, hidden] as bf16 bit patterns, token i = stream index first+i."""
    seed = shape.seed if seed is None else seed
    x = np.empty((n, shape.hidden), np.uint16)
    for i in range(n):
        normal_bf16(seed, stream_id(KIND_X, layer, first + i), shape.hidden, 0.0, 1.0, out=x[i])
    return x


def gate_weights(shape: Shape, layer: int = 0, seed: int | None = None) -> np.ndarray:
    """Router weight [n_experts, hidden] fp32 ~ N(0, 0.02)."""
    seed = shape.seed if seed is None else seed
    g = normal_f32(seed, stream_id(KIND_GATE, layer), shape.n_experts * shape.hidden, 0.0, WEIGHT_STD)
    return g.reshape(shape.n_experts, shape.hidden)


def shared_gate_row(shape: Shape, layer: int = 0, seed: int | None = None) -> np.ndarray:
    """The shared expert's gate row [hidden] fp32 ~ N(0, 0.02) (router row E of a gated layer)."""
    seed = shape.seed if seed is None else seed
    return normal_f32(seed, stream_id(KIND_GATE, layer, 1), shape.hidden, 0.0, WEIGHT_STD)


def expert_arena(shape: Shape, layer: int = 0, seed: int | None = None,
                 out: np.ndarray | None = None) -> np.ndarray:
    """Routed experts in GGUF block order: expert e = [gate F x H | up F x H | down H x F]."""
    seed = shape.seed if seed is None else seed
    eb = shape.expert_bytes
    out = np.empty(shape.n_experts * eb, np.uint8) if out is None else out
    for e in range(shape.n_experts):
        codec_blocks(shape.codec, seed, stream_id(KIND_EXPERT, layer, e), 3 * shape.ffn * shape.hidden,
                     out=out[e * eb:(e + 1) * eb])
    return out


def shared_arena(shape: Shape, layer: int = 0, seed: int | None = None) -> np.ndarray:
    seed = shape.seed if seed is None else seed
    return codec_blocks(shape.codec, seed, stream_id(KIND_EXPERT, layer, shape.n_experts), 3 * shape.ffn * shape.hidden)


def zipf_bias(shape: Shape, lam: float, layer: int = 0, seed: int | None = None) -> np.ndarray:
    """Selection bias b_e = -lam * s * ln(rank_e) with ranks a seeded permutation of the experts.

    The popularity skew enters through the method's own selection-only bias input
    (the model card's ffn_exp_probs_b); lam is calibrated separately.
    """
    seed = shape.seed if seed is None else seed
    keys = normal_f32(seed, stream_id(KIND_BIAS, layer), shape.n_experts)
    rank = np.empty(shape.n_experts, np.int64)
    rank[np.argsort(keys, kind="stable")] = np.arange(1, shape.n_experts + 1)
    return (-lam * shape.zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)


ZIPF_LAMBDA_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "golden",
                                "zipf_lambda.json")


def zipf_lambda(shape: Shape) -> float:
    """The bias strength calibrated for a skewed workload (tests/golden/make_zipf_lambda.py)."""
    import json
    with open(ZIPF_LAMBDA_FILE) as f:
        return float(json.load(f)[shape.name]["lam"])


def layer_inputs(shape: Shape, layer: int = 0, seed: int | None = None, lam: float = 0.0) -> dict:
    """Everything one layer consumes except the activations."""
    bias = zipf_bias(shape, lam, layer, seed) if shape.zipf_s and lam else None
    return {
        "gate_w": gate_weights(shape, layer, seed) if shape.n_experts else None,
        "bias": bias,
        "arena": expert_arena(shape, layer, seed),
        "shared": shared_arena(shape, layer, seed) if shape.n_shared else None,
    }
