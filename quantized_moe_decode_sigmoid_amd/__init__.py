"""Python binding of libmoe: one quantized MoE FFN layer on MI355X (gfx950).

Argument marshalling only -- every step of the layer runs in the hand-written HIP
kernels of ``libmoe.so`` (C ABI in ``include/moe.h``); torch provides device memory
and the current HIP stream.  The functions carry the C names; each takes torch
tensors, passes their device pointers and ``torch.cuda.current_stream()``, and raises
``MoeError`` on a non-zero status.  There is no fallback: if the library is missing
the import of this module fails.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EWORKSPACE, MOE_EUNSUPPORTED, MOE_ELAUNCH = 0, -1, -2, -3, -4, -5
PREC_AUTO, PREC_FP32, PREC_BF16, PREC_W4A8 = 0, 1, 2, 3
MATRIX_GATE, MATRIX_UP, MATRIX_DOWN = 0, 1, 2
CODEC_IQ4_NL, CODEC_IQ4_XS, CODEC_Q3_AFFINE = 0, 1, 2


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class moe_config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("ffn", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("routed_scale", ctypes.c_float),
                ("precision", ctypes.c_int32), ("shared_gate", ctypes.c_int32), ("codec", ctypes.c_int32)]


def make_config(hidden: int, ffn: int, n_experts: int, top_k: int, n_shared: int = 1,
                routed_scale: float = 2.0, precision: int = PREC_AUTO, shared_gate: int = 0,
                codec: int = 0) -> moe_config:
    return moe_config(hidden, ffn, n_experts, top_k, n_shared, routed_scale, precision, shared_gate, codec)


def weight_cols(cfg: moe_config) -> int:
    """Values per token row of the routing weights: K, plus the shared expert's gate when it is gated."""
    return cfg.top_k + cfg.shared_gate


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                      "python quantized_moe_decode_sigmoid_amd/build.py")

# torch brings its own HIP runtime (soname libamdhip64.so.7, requested by its
# libraries under another name).  Loading torch first makes libmoe bind to that
# same runtime instead of pulling a second copy into the process.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_cfgp = ctypes.POINTER(moe_config)


class moe_stack_layer(ctypes.Structure):
    """One layer of moe_stack_decode: device pointers of its weights (include/moe.h)."""
    _fields_ = [("gate_w", ctypes.c_void_p), ("sel_bias", ctypes.c_void_p), ("arena", ctypes.c_void_p),
                ("shared", ctypes.c_void_p)]


_stackp = ctypes.POINTER(moe_stack_layer)
_SIGS = {
    "moe_abi_version": ([], _i32),
    "moe_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "moe_check_config": ([_cfgp], _i32),
    "moe_expert_bytes": ([_cfgp], _sz),
    "moe_packed_expert_bytes": ([_cfgp], _sz),
    "moe_resolved_precision": ([_cfgp, _i32], _i32),
    "moe_workspace_bytes": ([_cfgp, _i32], _sz),
    "moe_workspace_init": ([_cfgp, _i32, _vp, _sz, _vp], _i32),
    "moe_workspace_status": ([_cfgp, _i32, _vp, _sz, _vp, _vp], _i32),
    "moe_pack_experts": ([_cfgp, _i32, _vp, _vp, _vp], _i32),
    "moe_dequant": ([_cfgp, _vp, _i32, _i32, _vp, _vp], _i32),
    "moe_router_scores": ([_cfgp, _i32, _vp, _vp, _vp, _vp], _i32),
    "moe_route": ([_cfgp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "moe_bucket": ([_cfgp, _i32, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "moe_expert_forward": ([_cfgp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "moe_layer_forward": ([_cfgp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "moe_layer_forward_chained": ([_cfgp, _i32, _vp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _sz, _vp], _i32),
    "moe_layer_forward_noalloc": ([_cfgp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp], _i32),
    "moe_quantize_q8_0": ([_vp, _i32, ctypes.c_int64, _vp, _vp, _vp], _i32),
    "moe_stream_read": ([_vp, _sz, _vp, _vp], _i32),
    "moe_residual_rmsnorm": ([_vp, _vp, _i32, _i32, ctypes.c_float, _vp, _vp], _i32),
    "moe_stack_workspace_bytes": ([_cfgp, _i32, ctypes.POINTER(_sz)], _i32),
    "moe_stack_decode": ([_cfgp, _i32, _stackp, _vp, ctypes.c_float, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "moe_stack_status": ([_cfgp, _i32, _vp, _sz, _vp, _vp], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res
EXPORTED = tuple(_SIGS)


def _p(t):
    """Device pointer of a tensor (None -> NULL).  Raw integers pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_abi_version() -> int:
    return _lib.moe_abi_version()


def moe_check_config(cfg: moe_config) -> int:
    return _lib.moe_check_config(ctypes.byref(cfg))


def moe_expert_bytes(cfg: moe_config) -> int:
    return _lib.moe_expert_bytes(ctypes.byref(cfg))


def moe_packed_expert_bytes(cfg: moe_config) -> int:
    return _lib.moe_packed_expert_bytes(ctypes.byref(cfg))


def moe_resolved_precision(cfg: moe_config, T: int) -> int:
    return _lib.moe_resolved_precision(ctypes.byref(cfg), T)


def moe_workspace_bytes(cfg: moe_config, T: int) -> int:
    return _lib.moe_workspace_bytes(ctypes.byref(cfg), T)


def moe_workspace_init(cfg, T, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(_lib.moe_workspace_init(ctypes.byref(cfg), T, _p(ws), ws_bytes, _stream(stream)), "moe_workspace_init")


def moe_workspace_status(cfg, T, ws, status, ws_bytes=None, stream=None):
    """Copy the workspace's status word (0 ok, 1 a decode wait gave up) into the device int32 tensor status."""
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(_lib.moe_workspace_status(ctypes.byref(cfg), T, _p(ws), ws_bytes, _p(status), _stream(stream)),
           "moe_workspace_status")


def moe_pack_experts(cfg, n_experts, src, dst, stream=None):
    _check(_lib.moe_pack_experts(ctypes.byref(cfg), n_experts, _p(src), _p(dst), _stream(stream)), "moe_pack_experts")


def moe_quantize_q8_0(src, q, d, stream=None):
    """Q8_0 of a bf16 or fp32 tensor (numel a multiple of 32) into int8 codes q and fp16-bit scales d (int16)."""
    import torch
    bf16 = 1 if src.dtype == torch.bfloat16 else 0
    assert bf16 or src.dtype == torch.float32
    _check(_lib.moe_quantize_q8_0(_p(src), bf16, src.numel(), _p(q), _p(d), _stream(stream)), "moe_quantize_q8_0")


def moe_stream_read(src, nbytes, sink, stream=None):
    """Measurement kernel: read nbytes of src once (no writes); sink is a 16-byte aligned device word."""
    _check(_lib.moe_stream_read(_p(src), nbytes, _p(sink), _stream(stream)), "moe_stream_read")


def moe_residual_rmsnorm(out, x, y, eps=1e-6, stream=None):
    """Chaining between stacked layers: y = bf16(rmsnorm(x + out)), one fused kernel (not part of the layer)."""
    T, H = out.shape
    _check(_lib.moe_residual_rmsnorm(_p(out), _p(x), T, H, eps, _p(y), _stream(stream)), "moe_residual_rmsnorm")


def moe_dequant(cfg, packed_expert, matrix, precision, out, stream=None):
    _check(_lib.moe_dequant(ctypes.byref(cfg), _p(packed_expert), matrix, precision, _p(out), _stream(stream)),
           "moe_dequant")


def moe_router_scores(cfg, T, x, gate_w, scores, stream=None):
    _check(_lib.moe_router_scores(ctypes.byref(cfg), T, _p(x), _p(gate_w), _p(scores), _stream(stream)),
           "moe_router_scores")


def moe_route(cfg, T, x, gate_w, sel_bias, topk_ids, topk_w, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(_lib.moe_route(ctypes.byref(cfg), T, _p(x), _p(gate_w), _p(sel_bias), _p(topk_ids), _p(topk_w), _p(ws),
                          ws_bytes, _stream(stream)), "moe_route")


def moe_bucket(cfg, T, topk_ids, counts, offsets, perm, pos=None, stream=None):
    _check(_lib.moe_bucket(ctypes.byref(cfg), T, _p(topk_ids), _p(counts), _p(offsets), _p(perm), _p(pos),
                           _stream(stream)), "moe_bucket")


def moe_expert_forward(cfg, T, x, topk_ids, topk_w, arena, shared, out, ws, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(_lib.moe_expert_forward(ctypes.byref(cfg), T, _p(x), _p(topk_ids), _p(topk_w), _p(arena), _p(shared),
                                   _p(out), _p(ws), ws_bytes, _stream(stream)), "moe_expert_forward")


def moe_layer_forward(cfg, T, x, gate_w, sel_bias, arena, shared, out, topk_ids=None, topk_w=None, ws=None,
                      ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(_lib.moe_layer_forward(ctypes.byref(cfg), T, _p(x), _p(gate_w), _p(sel_bias), _p(arena), _p(shared),
                                  _p(out), _p(topk_ids), _p(topk_w), _p(ws), ws_bytes, _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_chained(cfg, T, x_prev, out_prev, x, gate_w, sel_bias, arena, shared, out, topk_ids=None,
                              topk_w=None, ws=None, ws_bytes=None, eps=1e-6, stream=None):
    """A stacked layer whose input x = bf16(rmsnorm(x_prev + out_prev)) is formed (and written to x) in the call."""
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(_lib.moe_layer_forward_chained(ctypes.byref(cfg), T, _p(x_prev), _p(out_prev), eps, _p(x), _p(gate_w),
                                          _p(sel_bias), _p(arena), _p(shared), _p(out), _p(topk_ids), _p(topk_w),
                                          _p(ws), ws_bytes, _stream(stream)), "moe_layer_forward_chained")


def moe_layer_forward_noalloc(cfg, T, x, gate_w, sel_bias, arena, shared, out, topk_ids=None, topk_w=None,
                              stream=None):
    """moe_layer_forward on the library's own per-GPU scratch (no workspace argument, no allocation)."""
    _check(_lib.moe_layer_forward_noalloc(ctypes.byref(cfg), T, _p(x), _p(gate_w), _p(sel_bias), _p(arena),
                                          _p(shared), _p(out), _p(topk_ids), _p(topk_w), _stream(stream)),
           "moe_layer_forward_noalloc")


def moe_stack_workspace_bytes(cfg, L):
    n = _sz(0)
    _check(_lib.moe_stack_workspace_bytes(ctypes.byref(cfg), L, ctypes.byref(n)), "moe_stack_workspace_bytes")
    return n.value


def stack_layers(layers):
    """A moe_stack_layer array from (gate_w, sel_bias, arena, shared) tuples of device tensors (or None)."""
    arr = (moe_stack_layer * len(layers))()
    for i, (g, b, a, sh) in enumerate(layers):
        arr[i] = moe_stack_layer(_p(g), _p(b), _p(a), _p(sh))
    return arr


def moe_stack_decode(cfg, L, layers, x0, x_all, out_all, ids_all=None, w_all=None, ws=None, ws_bytes=None, eps=1e-6,
                     stream=None):
    """One decode token through L chained layers in one call, two decode launches per layer (layers: stack_layers(...))."""
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None and ws is not None else (ws_bytes or 0)
    _check(_lib.moe_stack_decode(ctypes.byref(cfg), L, layers, _p(x0), eps, _p(x_all), _p(out_all), _p(ids_all),
                                 _p(w_all), _p(ws), ws_bytes, _stream(stream)), "moe_stack_decode")


def moe_stack_status(cfg, L, ws, status, ws_bytes=None, stream=None):
    ws_bytes = ws.numel() * ws.element_size() if ws_bytes is None else ws_bytes
    _check(_lib.moe_stack_status(ctypes.byref(cfg), L, _p(ws), ws_bytes, _p(status), _stream(stream)),
           "moe_stack_status")


class DeviceLayer:
    """Device copies of one layer's weights, the expert arena packed by moe_pack_experts.

    gate_w fp32 [E + shared_gate, H] (row E: the shared expert's gate), bias fp32 [E] or None,
    arena / shared uint8 in GGUF block order (numpy or torch); a dense block (E = 0) has no
    gate_w, bias or arena (None).  ``forward`` allocates the outputs and workspace with torch
    and calls moe_layer_forward.
    """

    def __init__(self, cfg: moe_config, gate_w, bias, arena, shared, device="cuda"):
        import torch

        def dev(a, dtype):
            t = torch.as_tensor(a)
            return t.to(device=device, dtype=dtype).contiguous()

        self.cfg = cfg
        self.device = device
        self.gate_w = None if gate_w is None or cfg.n_experts == 0 else dev(gate_w, torch.float32)
        if self.gate_w is not None:
            assert self.gate_w.shape[0] == cfg.n_experts + cfg.shared_gate
        self.bias = None if bias is None else dev(bias, torch.float32)
        eb, pb = moe_expert_bytes(cfg), moe_packed_expert_bytes(cfg)
        self.arena = None
        if cfg.n_experts:
            src = dev(arena, torch.uint8)
            assert src.numel() == eb * cfg.n_experts
            self.arena = torch.empty(pb * cfg.n_experts, dtype=torch.uint8, device=device)
            moe_pack_experts(cfg, cfg.n_experts, src, self.arena)
        self.shared = None
        if cfg.n_shared:
            ssrc = dev(shared, torch.uint8)
            assert ssrc.numel() == eb
            self.shared = torch.empty(pb, dtype=torch.uint8, device=device)
            moe_pack_experts(cfg, 1, ssrc, self.shared)
        self._ws = None

    @classmethod
    def from_packed(cls, cfg: moe_config, gate_w, bias, arena, shared, device="cuda"):
        """A layer over device tensors already in packed order (moe_pack_experts), used as given."""
        self = cls.__new__(cls)
        self.cfg, self.device, self._ws = cfg, device, None
        self.gate_w, self.bias, self.arena, self.shared = gate_w, bias, arena, shared
        return self

    def workspace(self, T: int):
        import torch
        need = moe_workspace_bytes(self.cfg, T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
            moe_workspace_init(self.cfg, T, self._ws)
        return self._ws

    def forward(self, x, out=None, topk_ids=None, topk_w=None):
        """x: bf16 [T, H] (torch.bfloat16 or int16/uint16 bit patterns) -> fp32 [T, H]."""
        import torch
        T = x.shape[0]
        if out is None:
            out = torch.empty((T, self.cfg.hidden), dtype=torch.float32, device=self.device)
        ws = self.workspace(T)
        moe_layer_forward(self.cfg, T, x, self.gate_w, self.bias, self.arena, self.shared, out, topk_ids, topk_w, ws)
        return out
