"""CPU oracle for the quantized MoE layer -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import this package.  The GPU library never calls it and shares no code with it.

Thin ctypes wrapper over ``moe_oracle.c`` (plain C, ``-O2 -ffp-contract=off
-fno-fast-math``).  What each function computes, and the page passage it follows,
is stated in the C source.  Arrays are numpy; bf16 values travel as uint16 bit
patterns, IQ4_NL weights as uint8 blocks in GGUF order (18 bytes: fp16 scale, then
16 bytes of nibbles).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

FP32, BF16, W4A8 = 1, 2, 3  # precision modes (see moe_oracle.c)
IQ4_NL, IQ4_XS, Q3_AFFINE = 0, 1, 2  # expert codecs

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", os.path.join(_HERE, "moe_oracle.c"), "-o", _LIB_PATH, "-lm"]
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
    i32, i64, f32, f64, vp = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
    lib.oracle_codebook.argtypes = [i32]
    lib.oracle_codebook.restype = i32
    lib.oracle_f16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_value.restype = f64
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = f32
    lib.oracle_to_bf16.argtypes = [f32]
    lib.oracle_to_bf16.restype = ctypes.c_uint16
    lib.oracle_to_f16.argtypes = [f32]
    lib.oracle_to_f16.restype = ctypes.c_uint16
    lib.oracle_quantize_q8_0.argtypes = [i64, vp, vp, vp]
    lib.oracle_dequant.argtypes = [vp, i64, i32, vp]
    lib.oracle_router_logits.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.oracle_exp_spec.argtypes = [f64]
    lib.oracle_exp_spec.restype = f64
    lib.oracle_sigmoid.argtypes = [f32]
    lib.oracle_sigmoid.restype = f32
    lib.oracle_route.argtypes = [i32, i32, i32, i32, f32, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_bucket.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp]
    lib.oracle_expert.argtypes = [i32, i32, vp, vp, i32, vp]
    lib.oracle_layer.argtypes = [i32, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_codec_row_bytes.argtypes = [i32, i32]
    lib.oracle_codec_row_bytes.restype = i64
    lib.oracle_codec_expert_bytes.argtypes = [i32, i32, i32]
    lib.oracle_codec_expert_bytes.restype = i64
    lib.oracle_dequant_codec.argtypes = [i32, vp, i32, vp]
    lib.oracle_expert_codec.argtypes = [i32, i32, i32, vp, vp, vp]
    lib.oracle_layer_codec.argtypes = [i32, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_layer_gated.argtypes = [i32, i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_threads.restype = i32
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_sigmoid_many.argtypes = [i64, vp, vp]
    lib.oracle_residual_rmsnorm.argtypes = [i32, i32, vp, vp, f64, vp]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def threads() -> int:
    return _load().oracle_threads()


def set_threads(n: int) -> None:
    """Threads of the token loop of layer() (n <= 0 leaves the setting unchanged); results do not depend on it."""
    _load().oracle_set_threads(n)


def codebook() -> list[int]:
    lib = _load()
    return [lib.oracle_codebook(i) for i in range(16)]


def f16_value(h: int) -> float:
    return _load().oracle_f16_value(h)


def bf16_value(b: int) -> float:
    return _load().oracle_bf16_value(b)


def to_bf16(f: float) -> int:
    return _load().oracle_to_bf16(f)


def to_f16(f: float) -> int:
    return _load().oracle_to_f16(f)


def quantize_q8_0(x: np.ndarray):
    """fp32 values (a multiple of 32, blocks in order) -> (int8 codes, fp16 scale bits per block)."""
    x = _c(x, np.float32).reshape(-1)
    assert x.size % 32 == 0
    q = np.empty(x.size, np.int8)
    d = np.empty(x.size // 32, np.uint16)
    _load().oracle_quantize_q8_0(x.size // 32, _ptr(x), _ptr(q), _ptr(d))
    return q, d


def exp_spec(y: float) -> float:
    return _load().oracle_exp_spec(y)


def sigmoid(l: float) -> float:
    return _load().oracle_sigmoid(l)


def sigmoid_many(logits: np.ndarray) -> np.ndarray:
    """sigmoid() over an array of fp32 logits."""
    l = _c(logits, np.float32).reshape(-1)
    out = np.empty(l.size, np.float32)
    _load().oracle_sigmoid_many(l.size, _ptr(l), _ptr(out))
    return out.reshape(np.shape(logits))


def residual_rmsnorm(x: np.ndarray, out: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """Stack chaining glue (not the layer): bf16(rmsnorm(x + out)), x bf16 bits [T,H], out fp32 [T,H]."""
    x = _c(x, np.uint16)
    out = _c(out, np.float32)
    T, H = x.shape
    y = np.empty((T, H), np.uint16)
    _load().oracle_residual_rmsnorm(T, H, _ptr(x), _ptr(out), eps, _ptr(y))
    return y


def dequant(blocks: np.ndarray, mode: int = FP32) -> np.ndarray:
    """IQ4_NL blocks (uint8, n*18) -> fp32 weights (n*32)."""
    blocks = _c(blocks, np.uint8).reshape(-1)
    nb = blocks.size // 18
    out = np.empty(nb * 32, np.float32)
    _load().oracle_dequant(_ptr(blocks), nb, mode, _ptr(out))
    return out


def router_logits(x: np.ndarray, gate_w: np.ndarray) -> np.ndarray:
    x = _c(x, np.uint16)
    gate_w = _c(gate_w, np.float32)
    T, H = x.shape
    E = gate_w.shape[0]
    out = np.empty((T, E), np.float32)
    _load().oracle_router_logits(T, H, E, _ptr(x), _ptr(gate_w), _ptr(out))
    return out


def route(x: np.ndarray, gate_w: np.ndarray, top_k: int, scale: float = 2.0,
          bias: np.ndarray | None = None):
    """Returns (ids int32 [T,K], weights fp32 [T,K], logits fp32 [T,E], scores fp32 [T,E])."""
    x = _c(x, np.uint16)
    gate_w = _c(gate_w, np.float32)
    bias = _c(bias, np.float32)
    T, H = x.shape
    E = gate_w.shape[0]
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    logits = np.empty((T, E), np.float32)
    scores = np.empty((T, E), np.float32)
    _load().oracle_route(T, H, E, top_k, scale, _ptr(x), _ptr(gate_w), _ptr(bias), _ptr(ids), _ptr(w),
                         _ptr(logits), _ptr(scores))
    return ids, w, logits, scores


def bucket(ids: np.ndarray, n_experts: int):
    """Returns (counts [E], offsets [E+1], perm [T*K], pos [T*K]) as int32."""
    ids = _c(ids, np.int32)
    T, K = ids.shape
    counts = np.empty(n_experts, np.int32)
    offsets = np.empty(n_experts + 1, np.int32)
    perm = np.empty(T * K, np.int32)
    pos = np.empty(T * K, np.int32)
    _load().oracle_bucket(T, K, n_experts, _ptr(ids), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(pos))
    return counts, offsets, perm, pos


def expert(x_row: np.ndarray, expert_bytes: np.ndarray, hidden: int, ffn: int, mode: int = FP32) -> np.ndarray:
    """One expert FFN on one token -> y [H] float64."""
    x_row = _c(x_row, np.uint16).reshape(-1)
    expert_bytes = _c(expert_bytes, np.uint8)
    assert x_row.size == hidden and expert_bytes.size == 3 * ffn * hidden // 32 * 18
    y = np.empty(hidden, np.float64)
    _load().oracle_expert(hidden, ffn, _ptr(expert_bytes), _ptr(x_row), mode, _ptr(y))
    return y


def codec_row_bytes(codec: int, cols: int) -> int:
    return _load().oracle_codec_row_bytes(codec, cols)


def codec_expert_bytes(codec: int, hidden: int, ffn: int) -> int:
    return _load().oracle_codec_expert_bytes(codec, hidden, ffn)


def dequant_codec(codec: int, row: np.ndarray, cols: int) -> np.ndarray:
    """One row of `cols` weights in a codec -> float64 (exact)."""
    row = _c(row, np.uint8).reshape(-1)
    assert row.size == codec_row_bytes(codec, cols)
    out = np.empty(cols, np.float64)
    _load().oracle_dequant_codec(codec, _ptr(row), cols, _ptr(out))
    return out


def expert_codec(x_row: np.ndarray, expert_bytes: np.ndarray, hidden: int, ffn: int, codec: int) -> np.ndarray:
    x_row = _c(x_row, np.uint16).reshape(-1)
    expert_bytes = _c(expert_bytes, np.uint8)
    assert expert_bytes.size == codec_expert_bytes(codec, hidden, ffn)
    y = np.empty(hidden, np.float64)
    _load().oracle_expert_codec(hidden, ffn, codec, _ptr(expert_bytes), _ptr(x_row), _ptr(y))
    return y


def layer(x: np.ndarray, gate_w: np.ndarray, arena: np.ndarray | None, shared: np.ndarray | None,
          top_k: int, ffn: int, scale: float = 2.0, bias: np.ndarray | None = None, mode: int = FP32,
          shared_gate: np.ndarray | None = None, codec: int = IQ4_NL):
    """Whole MoE layer.  Returns (out fp32 [T,H], ids int32 [T,K], weights fp32 [T,K]).

    gate_w [E,H] (E may be 0 with top_k 0: a dense FFN block, the shared expert alone);
    shared_gate fp32 [H] or None: the shared expert is scaled by sigmoid(x . shared_gate)."""
    x = _c(x, np.uint16)
    T, H = x.shape
    gate_w = _c(gate_w, np.float32).reshape(-1, H)
    arena = _c(arena, np.uint8)
    shared = _c(shared, np.uint8)
    bias = _c(bias, np.float32)
    sg = _c(shared_gate, np.float32)
    E = gate_w.shape[0]
    assert (arena.size if arena is not None else 0) == E * codec_expert_bytes(codec, H, ffn)
    assert sg is None or sg.size == H
    out = np.empty((T, H), np.float32)
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float32)
    if codec != IQ4_NL:
        _load().oracle_layer_codec(T, H, ffn, E, top_k, 1 if shared is not None else 0, scale, codec, _ptr(x),
                                   _ptr(gate_w), _ptr(bias), _ptr(sg), _ptr(arena), _ptr(shared), _ptr(out),
                                   _ptr(ids), _ptr(w))
        return out, ids, w
    _load().oracle_layer_gated(T, H, ffn, E, top_k, 1 if shared is not None else 0, scale, mode, _ptr(x),
                               _ptr(gate_w), _ptr(bias), _ptr(sg), _ptr(arena), _ptr(shared), _ptr(out), _ptr(ids),
                               _ptr(w))
    return out, ids, w
