"""fp64 CPU oracle for the gated-delta-rule state step -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  The product (``hybrid_linear_attention_decode_amd``)
never imports it, and it imports nothing from the product.

The arithmetic lives in ``gdn_oracle.c`` (plain fp64 loops, definitions D1-D8
in ``gdn_oracle.h``).  This module only

* builds / loads ``libgdn_oracle.so`` with gcc,
* decodes bf16 bit patterns into fp64 itself (bf16 -> fp64 is exact),
* marshals numpy arrays into the C calls.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (closed forms, special cases, library routines,
brute force on tiny inputs).
"""
from __future__ import annotations

import ctypes as ct
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
# GDN_ORACLE_LIB_PATH names another build of the oracle (e.g. one with
# sanitizers); by default the in-tree libgdn_oracle.so.
_LIB = os.environ.get("GDN_ORACLE_LIB_PATH") or os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fast-math, no FMA contraction)."""
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
           "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ct.CDLL(_LIB)
        P = ct.c_void_p
        i32, i64 = ct.c_int32, ct.c_int64
        lp = ct.POINTER(OrcLayer)
        lib.orc_decode.argtypes = [lp, P, P, i64, P, i32, i32, P, P, P, P, P, P, P, P, i32, i32]
        lib.orc_spec_commit.argtypes = [lp, P, P, i64, P, P, P, i32, P, i32]
        lib.orc_slot_copy.argtypes = [lp, P, P, i64, P, P, i32]
        lib.orc_slot_zero.argtypes = [lp, P, P, i64, P, i32]
        lib.orc_prefill.argtypes = [lp, P, P, i64, P, P, i32, P, P, P, P, P, P, P, i32]
        lib.orc_prefill_chunked.argtypes = [lp, P, P, i64, P, P, i32, P, i32, P, P, P, P, P, P, i32]
        for f in (lib.orc_decode, lib.orc_spec_commit, lib.orc_slot_copy, lib.orc_slot_zero,
                  lib.orc_prefill, lib.orc_prefill_chunked):
            f.restype = ct.c_int
        _lib = lib
    return _lib


class OrcLayer(ct.Structure):
    _fields_ = [("n_k_heads", ct.c_int32), ("n_v_heads", ct.c_int32),
                ("d_k", ct.c_int32), ("d_v", ct.c_int32), ("conv_width", ct.c_int32),
                ("gate", ct.c_int32), ("conv_silu", ct.c_int32), ("l2norm", ct.c_int32),
                ("q_scale", ct.c_double), ("eps", ct.c_double)]


@dataclass
class Layer:
    """Layer shape and switches, as the oracle sees them."""
    n_k_heads: int
    n_v_heads: int
    d_k: int
    d_v: int
    conv_width: int = 4
    gate: str = "scalar"          # "scalar" (GDN) or "channel" (KDA)
    conv_silu: bool = True
    l2norm: bool = True
    q_scale: float | None = None  # default 1/sqrt(d_k)
    eps: float = 1e-6

    @property
    def channels(self) -> int:
        return 2 * self.n_k_heads * self.d_k + self.n_v_heads * self.d_v

    def c_struct(self) -> OrcLayer:
        qs = self.q_scale if self.q_scale is not None else 1.0 / np.sqrt(self.d_k)
        return OrcLayer(self.n_k_heads, self.n_v_heads, self.d_k, self.d_v, self.conv_width,
                        1 if self.gate == "channel" else 0, int(self.conv_silu),
                        int(self.l2norm), float(qs), float(self.eps))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact decoding of bf16 bit patterns (uint16) to fp64."""
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << 16
    with np.errstate(invalid="ignore"):   # NaN patterns widen to NaN
        return b.view(np.float32).astype(np.float64)


def as_f64(a) -> np.ndarray:
    """fp64 view of an input that is fp32, fp64 or bf16 bits (uint16)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_bits_to_f64(a)
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(ct.c_void_p)


def _i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _chk(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def _need_f64(*arrs):
    for a in arrs:
        if a is not None and (a.dtype != np.float64 or not a.flags.c_contiguous):
            raise TypeError("oracle pools must be C-contiguous float64 arrays")


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def decode(layer: Layer, ssm, conv, idx, x, alpha, beta, conv_w, conv_b=None,
           spec_ssm=None, spec_conv=None, T: int | None = None, nthreads: int | None = None):
    """D3-D5.  ssm/conv (fp64 pools) are updated in place unless spec_ssm is
    given (then snapshots go to spec_ssm/spec_conv).  x: [B, T, C]; returns
    out [B, T, H_v, d_v] fp64 (rows of skipped requests stay zero)."""
    _need_f64(ssm, conv, spec_ssm, spec_conv)
    idx = _i32(idx)
    B = idx.shape[0]
    x = as_f64(x)
    if T is None:
        T = x.shape[1] if x.ndim == 3 else x.shape[0] // max(B, 1)
    x = x.reshape(B * T, layer.channels)
    al, be = as_f64(alpha), as_f64(beta)
    w = as_f64(conv_w)
    b = None if conv_b is None else as_f64(conv_b)
    out = np.zeros((B, T, layer.n_v_heads, layer.d_v), dtype=np.float64)
    t_max = 0 if spec_ssm is None else spec_ssm.shape[1]
    L = layer.c_struct()
    rc = _load().orc_decode(ct.byref(L), _p(ssm), _p(conv), ssm.shape[0], _p(idx), B, T,
                            _p(x), _p(al), _p(be), _p(w), _p(b), _p(out), _p(spec_ssm),
                            _p(spec_conv), t_max, nthreads or default_threads())
    _chk(rc, "decode")
    return out


def spec_commit(layer: Layer, ssm, conv, idx, spec_ssm, spec_conv, accepted_len):
    _need_f64(ssm, conv, spec_ssm, spec_conv)
    idx, acc = _i32(idx), _i32(accepted_len)
    L = layer.c_struct()
    rc = _load().orc_spec_commit(ct.byref(L), _p(ssm), _p(conv), ssm.shape[0], _p(idx),
                                 _p(spec_ssm), _p(spec_conv), spec_ssm.shape[1], _p(acc),
                                 idx.shape[0])
    _chk(rc, "spec_commit")


def slot_copy(layer: Layer, ssm, conv, src, dst):
    _need_f64(ssm, conv)
    src, dst = _i32(src), _i32(dst)
    L = layer.c_struct()
    rc = _load().orc_slot_copy(ct.byref(L), _p(ssm), _p(conv), ssm.shape[0], _p(src), _p(dst),
                               src.shape[0])
    _chk(rc, "slot_copy")


def slot_zero(layer: Layer, ssm, conv, idx):
    _need_f64(ssm, conv)
    idx = _i32(idx)
    L = layer.c_struct()
    rc = _load().orc_slot_zero(ct.byref(L), _p(ssm), _p(conv), ssm.shape[0], _p(idx),
                               idx.shape[0])
    _chk(rc, "slot_zero")


def _prefill(fn, layer, ssm, conv, dst, init_slot, cu_seqlens, x, alpha, beta, conv_w,
             conv_b, chunk, nthreads):
    _need_f64(ssm, conv)
    dst, cu = _i32(dst), _i32(cu_seqlens)
    init = _i32(init_slot)
    N = dst.shape[0]
    total = int(cu[-1])
    x = as_f64(x).reshape(total, layer.channels)
    al, be, w = as_f64(alpha), as_f64(beta), as_f64(conv_w)
    b = None if conv_b is None else as_f64(conv_b)
    out = np.zeros((total, layer.n_v_heads, layer.d_v), dtype=np.float64)
    L = layer.c_struct()
    lib = _load()
    if fn == "seq":
        rc = lib.orc_prefill(ct.byref(L), _p(ssm), _p(conv), ssm.shape[0], _p(dst), _p(init),
                             N, _p(cu), _p(x), _p(al), _p(be), _p(w), _p(b), _p(out),
                             nthreads or default_threads())
    else:
        rc = lib.orc_prefill_chunked(ct.byref(L), _p(ssm), _p(conv), ssm.shape[0], _p(dst),
                                     _p(init), N, _p(cu), chunk, _p(x), _p(al), _p(be), _p(w),
                                     _p(b), _p(out), nthreads or default_threads())
    _chk(rc, "prefill")
    return out


def prefill(layer: Layer, ssm, conv, dst, init_slot, cu_seqlens, x, alpha, beta, conv_w,
            conv_b=None, nthreads=None):
    """D7 (the authority): token-by-token recurrence over each sequence."""
    return _prefill("seq", layer, ssm, conv, dst, init_slot, cu_seqlens, x, alpha, beta,
                    conv_w, conv_b, 0, nthreads)


def prefill_chunked(layer: Layer, ssm, conv, dst, init_slot, cu_seqlens, x, alpha, beta,
                    conv_w, conv_b=None, chunk=64, nthreads=None):
    """D8: fp64 chunk (WY/UT) form -- a self-check of the algebra only."""
    return _prefill("chunk", layer, ssm, conv, dst, init_slot, cu_seqlens, x, alpha, beta,
                    conv_w, conv_b, chunk, nthreads)
