"""Helpers shared by the GPU tests: moving seeded host arrays to the device,
fp64 shadow copies for the oracle, and the error metrics of the parity bar."""
import numpy as np

import oracle
from hybrid_linear_attention_decode_amd import Layer as GpuLayer
from hybrid_linear_attention_decode_amd import synth


def layers(shape: synth.Shape, **kw):
    """The same layer for the GPU binding and for the oracle."""
    common = dict(n_k_heads=shape.n_k_heads, n_v_heads=shape.n_v_heads, d_k=shape.d_k,
                  d_v=shape.d_v, conv_width=shape.conv_width, gate=shape.gate)
    g = GpuLayer(act_dtype=shape.dtype, **common, **kw)
    okw = {("eps" if k == "l2_eps" else k): v for k, v in kw.items()}
    o = oracle.Layer(**common, **okw)
    return g, o


def dev(a: np.ndarray):
    """Host array (float32, int32, or uint16 bf16 bits) -> contiguous cuda tensor."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t) -> np.ndarray:
    """cuda tensor -> numpy (bf16 comes back as uint16 bits)."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(t) -> np.ndarray:
    """Raw bit pattern of a cuda tensor, for bitwise comparisons (NaN-safe)."""
    import torch
    t = t.detach().contiguous()
    if t.element_size() == 4:
        return t.view(torch.int32).cpu().numpy()
    return t.view(torch.int16).cpu().numpy()


def shadow(pool: synth.Pool):
    """fp64 copies of a seeded pool for the oracle."""
    return oracle.as_f64(pool.ssm).copy(), oracle.as_f64(pool.conv).copy()


def rel_err(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / max |ref| (the parity metric for outputs and states)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(gpu - ref)) / max(np.max(np.abs(ref)), 1e-30))


# The parity bar: outputs max|do|/max|o| <= 2e-3 (bf16 inputs, fp32 state);
# final state relative error <= 1e-4 after 16 fp32 steps.
OUT_TOL = 2e-3
STATE_TOL_16 = 1e-4
