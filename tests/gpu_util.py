"""Helpers for the GPU parity tests: seeded inputs to device, comparison metrics."""
import numpy as np

import synth

TOL_MAX_ABS = 2e-2   # FP output tolerance of the layer: max |gpu - oracle|
TOL_REL_L2 = 1e-3    # and ||gpu - oracle||_2 / ||oracle||_2


def torch_dev():
    import torch
    return torch


def to_dev_bf16(x_bits: np.ndarray):
    """uint16 bf16 bit patterns -> torch.bfloat16 on the GPU (bit-exact)."""
    torch = torch_dev()
    t = torch.from_numpy(x_bits.view(np.int16).copy())
    return t.view(torch.bfloat16).cuda()


def cfg_of(shape: synth.Shape, precision=0):
    import quantized_moe_decode_sigmoid_amd as qm
    return qm.make_config(shape.hidden, shape.ffn, shape.n_experts, shape.top_k, shape.n_shared,
                          shape.routed_scale, precision)


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def assert_close(got, want, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.isfinite(got)), what
    mae = float(np.max(np.abs(got - want))) if got.size else 0.0
    r = rel_l2(got, want) if got.size else 0.0
    print(f"[parity] {what}: max_abs={mae:.3e} rel_l2={r:.3e}", flush=True)
    assert mae <= TOL_MAX_ABS, (what, mae)
    assert r <= TOL_REL_L2, (what, r)
