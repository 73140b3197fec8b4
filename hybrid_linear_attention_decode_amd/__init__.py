"""Python binding of libgdn (include/gdn.h): argument marshalling only.

Every step of the state path runs in the HIP kernels of ``libgdn.so``; this
module turns torch tensors (device memory) and the current HIP stream into the
plain pointers and sizes of the C ABI, and raises ``GdnError`` on a non-OK
status.  There is no fallback: if the library is not built, every call fails
loudly.  Build it with ``python -m hybrid_linear_attention_decode_amd.build``.

Entry points (same names as the C ABI):
    gdn_decode_step (+ decode_work, a zero work counter for it), gdn_spec_decode_commit,
    gdn_spec_commit_index, gdn_prefill_chunked, gdn_prefill_chunked_static,
    gdn_prefill_workspace_size, gdn_slot_copy, gdn_slot_zero, gdn_slot_bytes, gdn_slot_pack,
    gdn_slot_unpack, gdn_status_string
"""
from __future__ import annotations

import ctypes as ct
import os
from dataclasses import dataclass

# GDN_LIB_PATH names another build of the library to load (e.g. one with
# host-side sanitizers); by default the in-tree libgdn.so.
LIB_PATH = os.environ.get("GDN_LIB_PATH") or \
    os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")

GDN_OK = 0
GDN_ERR_NULL_ARG = 1
GDN_ERR_BAD_SHAPE = 2
GDN_ERR_BAD_DTYPE = 3
GDN_ERR_UNSUPPORTED = 4
GDN_ERR_WORKSPACE = 5
GDN_ERR_LAUNCH = 6
GDN_ERR_PRECONDITION = 7

GDN_F32, GDN_BF16 = 0, 1
GDN_GATE_SCALAR, GDN_GATE_CHANNEL = 0, 1
GDN_F_CONV_SILU, GDN_F_L2NORM_QK = 1, 2

EXPORTED = ("gdn_decode_step", "gdn_spec_decode_commit", "gdn_spec_commit_index",
            "gdn_prefill_chunked", "gdn_prefill_chunked_static", "gdn_prefill_workspace_size",
            "gdn_slot_copy", "gdn_slot_zero", "gdn_slot_bytes", "gdn_slot_pack",
            "gdn_slot_unpack", "gdn_status_string")

GDN_PREFILL_STATIC_BYTES = 64 * 1024 * 1024


class GdnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {gdn_status_string(status)} (status {status})")
        self.status = status


class GdnLayer(ct.Structure):
    _fields_ = [("n_k_heads", ct.c_int32), ("n_v_heads", ct.c_int32), ("d_k", ct.c_int32),
                ("d_v", ct.c_int32), ("conv_width", ct.c_int32), ("gate", ct.c_int32),
                ("act_dtype", ct.c_int32), ("flags", ct.c_uint32), ("q_scale", ct.c_float),
                ("l2_eps", ct.c_float)]


class GdnPool(ct.Structure):
    _fields_ = [("ssm", ct.c_void_p), ("conv", ct.c_void_p), ("num_slots", ct.c_int64)]


class GdnSpecCache(ct.Structure):
    _fields_ = [("ssm", ct.c_void_p), ("conv", ct.c_void_p), ("t_max", ct.c_int32),
                ("slots", ct.c_void_p)]


class GdnPrefillCkpt(ct.Structure):
    _fields_ = [("slots", ct.c_void_p), ("every", ct.c_int32), ("per_seq", ct.c_int32)]


class GdnInputs(ct.Structure):
    _fields_ = [("x", ct.c_void_p), ("alpha", ct.c_void_p), ("beta", ct.c_void_p),
                ("conv_w", ct.c_void_p), ("conv_b", ct.c_void_p)]


_lib = None


def lib() -> ct.CDLL:
    """The loaded libgdn.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libgdn.so is not built ({LIB_PATH}); run "
                               "python -m hybrid_linear_attention_decode_amd.build")
        L = ct.CDLL(LIB_PATH)
        P, i32, i64 = ct.c_void_p, ct.c_int32, ct.c_int64
        lp = ct.POINTER(GdnLayer)
        pp = ct.POINTER(GdnPool)
        sp = ct.POINTER(GdnSpecCache)
        ip = ct.POINTER(GdnInputs)
        L.gdn_decode_step.argtypes = [lp, pp, P, P, i32, i32, ip, P, sp, P, P]
        L.gdn_spec_decode_commit.argtypes = [lp, pp, P, sp, P, i32, P]
        L.gdn_spec_commit_index.argtypes = [pp, sp, P, P, P, i32, P]
        L.gdn_prefill_chunked.argtypes = [lp, pp, P, P, i32, P, i32, i32, i32, ip, P,
                                          ct.POINTER(GdnPrefillCkpt), P, ct.c_size_t, P]
        L.gdn_prefill_chunked_static.argtypes = [lp, pp, P, P, i32, P, i32, i32, i32, ip, P,
                                                 ct.POINTER(GdnPrefillCkpt), P]
        L.gdn_prefill_workspace_size.argtypes = [lp, i32, i32, i32, i32]
        L.gdn_prefill_workspace_size.restype = ct.c_size_t
        L.gdn_slot_copy.argtypes = [lp, pp, P, P, i32, P]
        L.gdn_slot_zero.argtypes = [lp, pp, P, i32, P]
        L.gdn_slot_bytes.argtypes = [lp]
        L.gdn_slot_bytes.restype = ct.c_size_t
        L.gdn_slot_pack.argtypes = [lp, pp, P, i32, P, ct.c_size_t, P]
        L.gdn_slot_unpack.argtypes = [lp, pp, P, ct.c_size_t, P, i32, P]
        L.gdn_status_string.argtypes = [ct.c_int]
        L.gdn_status_string.restype = ct.c_char_p
        for f in ("gdn_decode_step", "gdn_spec_decode_commit", "gdn_spec_commit_index",
                  "gdn_prefill_chunked", "gdn_prefill_chunked_static", "gdn_slot_copy",
                  "gdn_slot_zero", "gdn_slot_pack", "gdn_slot_unpack"):
            getattr(L, f).restype = ct.c_int
        _lib = L
    return _lib


def gdn_status_string(status: int) -> str:
    return lib().gdn_status_string(int(status)).decode()


@dataclass
class Layer:
    """One linear-attention layer (mirrors gdn_layer)."""
    n_k_heads: int
    n_v_heads: int
    d_k: int
    d_v: int
    conv_width: int = 4
    gate: str = "scalar"          # "scalar" (GDN) or "channel" (KDA)
    act_dtype: str = "bf16"       # "bf16" or "f32"
    conv_silu: bool = True
    l2norm: bool = True
    q_scale: float | None = None  # default 1/sqrt(d_k)
    l2_eps: float = 1e-6

    @property
    def channels(self) -> int:
        return 2 * self.n_k_heads * self.d_k + self.n_v_heads * self.d_v

    @property
    def torch_act_dtype(self):
        import torch
        return torch.bfloat16 if self.act_dtype == "bf16" else torch.float32

    def c_struct(self) -> GdnLayer:
        qs = self.q_scale if self.q_scale is not None else self.d_k ** -0.5
        flags = (GDN_F_CONV_SILU if self.conv_silu else 0) | (GDN_F_L2NORM_QK if self.l2norm else 0)
        return GdnLayer(self.n_k_heads, self.n_v_heads, self.d_k, self.d_v, self.conv_width,
                        GDN_GATE_CHANNEL if self.gate == "channel" else GDN_GATE_SCALAR,
                        GDN_BF16 if self.act_dtype == "bf16" else GDN_F32, flags, float(qs),
                        float(self.l2_eps))


def _ptr(t):
    return None if t is None else ct.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ct.c_void_p(s.cuda_stream)


def _on(stream):
    """Context for allocating buffers the library fills on `stream`: the
    caching allocator then hands the block to no other stream's work while
    the call's kernels may still use it."""
    import contextlib
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _dev(*tensors):
    for t in tensors:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("libgdn takes contiguous device tensors")


def _check(status: int, what: str):
    if status != GDN_OK:
        raise GdnError(status, what)


def _pool(ssm, conv) -> GdnPool:
    return GdnPool(_ptr(ssm), _ptr(conv), ssm.shape[0])


def decode_work(device="cuda"):
    """A decode work counter (the `work` argument of gdn_decode_step): one
    zero int32 word.  Calls on one stream may share it; calls that may run at
    the same time need their own.  The library leaves it at zero."""
    import torch
    return torch.zeros(1, dtype=torch.int32, device=device)


def _check_work(work):
    import torch
    if work is not None and (work.dtype != torch.int32 or work.numel() < 1):
        raise ValueError("work must be an int32 tensor of at least one element")


def _check_pool(layer: "Layer", ssm, conv):
    """ssm [slots, H_v, d_v, d_k] fp32; conv [slots, W-1, C] in the layer's
    activation dtype (may be None when W == 1)."""
    import torch
    if ssm is None or ssm.dtype != torch.float32 or ssm.dim() != 4 or \
            tuple(ssm.shape[1:]) != (layer.n_v_heads, layer.d_v, layer.d_k):
        raise ValueError(f"ssm pool must be float32 [slots, {layer.n_v_heads}, {layer.d_v}, "
                         f"{layer.d_k}]")
    if conv is None:
        if layer.conv_width > 1:
            raise ValueError("conv pool missing")
        return
    if conv.dtype != layer.torch_act_dtype or conv.dim() != 3 or conv.shape[0] != ssm.shape[0] \
            or tuple(conv.shape[1:]) != (layer.conv_width - 1, layer.channels):
        raise ValueError(f"conv pool must be {layer.torch_act_dtype} [{ssm.shape[0]}, "
                         f"{layer.conv_width - 1}, {layer.channels}]")


def _check_act(layer: "Layer", what: str, t, numel: int):
    """An activation-dtype input of numel elements (None allowed)."""
    if t is not None and (t.dtype != layer.torch_act_dtype or t.numel() != numel):
        raise ValueError(f"{what} must be {layer.torch_act_dtype} with {numel} elements")


def _check_out(t, shape):
    import torch
    if t is not None and (t.dtype != torch.float32 or tuple(t.shape) != tuple(shape)):
        raise ValueError(f"out must be float32 {list(shape)}")


def _spec(spec_ssm, spec_conv, spec_slots=None):
    if spec_slots is not None:
        return ct.byref(GdnSpecCache(None, None, spec_slots.shape[1], _ptr(spec_slots)))
    if spec_ssm is None:
        return None
    return ct.byref(GdnSpecCache(_ptr(spec_ssm), _ptr(spec_conv), spec_ssm.shape[1], None))


def _i32(t, n, what, required=False):
    """An int32 index array of n entries (the kernels read 32-bit words: an
    int64 tensor would be read as pairs of halves)."""
    import torch
    if t is None:
        if required:
            raise ValueError(f"{what} is required")
        return
    if t.dtype != torch.int32 or (n is not None and t.numel() != n):
        raise ValueError(f"{what} must be int32 [{n if n is not None else 'n'}]")


def _check_inputs(layer: "Layer", rows: int, x, alpha, beta, conv_w, conv_b):
    gates = layer.n_v_heads * (layer.d_k if layer.gate == "channel" else 1)
    _check_act(layer, "x", x, rows * layer.channels)
    _check_act(layer, "alpha", alpha, rows * gates)
    _check_act(layer, "beta", beta, rows * layer.n_v_heads)
    _check_act(layer, "conv_w", conv_w, layer.channels * layer.conv_width)
    _check_act(layer, "conv_b", conv_b, layer.channels)


def gdn_decode_step(layer: Layer, ssm, conv, mamba_pool_indices, x, alpha, beta, conv_w,
                    conv_b=None, out=None, spec_ssm=None, spec_conv=None, init_slot=None,
                    spec_slots=None, work=None, stream=None):
    """x [B, T, C]; returns out [B, T, H_v, d_v] fp32.  init_slot [B] int32:
    fused slot preparation (-1 zero start, s copy-on-write source); spec_slots
    [B, t_max] int32: snapshots into pool slots; work: a decode work counter
    (decode_work()) for the run-time balanced tail.  See include/gdn.h."""
    import torch
    _check_pool(layer, ssm, conv)
    _check_work(work)
    if x.dim() != 3:
        raise ValueError("x must be [B, T, C]")
    B, T = x.shape[0], x.shape[1]
    _check_inputs(layer, B * T, x, alpha, beta, conv_w, conv_b)
    _i32(mamba_pool_indices, B, "mamba_pool_indices", required=True)
    _i32(init_slot, B, "init_slot")
    if spec_slots is not None and (spec_slots.dtype != torch.int32 or spec_slots.dim() != 2
                                   or spec_slots.shape[0] != B):
        raise ValueError("spec_slots must be int32 [B, t_max]")
    if spec_ssm is not None:
        _check_pool(layer, spec_ssm.flatten(0, 1) if spec_ssm.dim() == 5 else spec_ssm,
                    None if spec_conv is None else
                    (spec_conv.flatten(0, 1) if spec_conv.dim() == 4 else spec_conv))
        if spec_ssm.dim() != 5 or spec_ssm.shape[0] != B or \
                (spec_conv is not None and tuple(spec_conv.shape[:2]) != tuple(spec_ssm.shape[:2])):
            raise ValueError("spec_ssm / spec_conv must be [B, t_max, ...]")
    shape = (B, T, layer.n_v_heads, layer.d_v)
    _check_out(out, shape)
    if out is None:
        with _on(stream):
            out = torch.empty(shape, dtype=torch.float32, device=x.device)
    _dev(ssm, conv, mamba_pool_indices, x, alpha, beta, conv_w, conv_b, out, spec_ssm, spec_conv,
         init_slot, spec_slots, work)
    L = layer.c_struct()
    P = _pool(ssm, conv)
    inp = GdnInputs(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(conv_w), _ptr(conv_b))
    st = lib().gdn_decode_step(ct.byref(L), ct.byref(P), _ptr(mamba_pool_indices),
                               _ptr(init_slot), B, T, ct.byref(inp), _ptr(out),
                               _spec(spec_ssm, spec_conv, spec_slots), _ptr(work),
                               _stream(stream))
    _check(st, "gdn_decode_step")
    return out


def gdn_spec_commit_index(ssm, conv, spec_slots, accepted_len, mamba_pool_indices,
                          released=None, stream=None):
    """Commit by index: mamba_pool_indices[b] <- spec_slots[b, L-1] for L =
    accepted_len[b] >= 1; released [B] int32 gets each request's previous slot
    (-1 where unchanged).  See include/gdn.h."""
    import torch
    B = mamba_pool_indices.numel()
    _i32(mamba_pool_indices, B, "mamba_pool_indices", required=True)
    _i32(accepted_len, B, "accepted_len", required=True)
    _i32(released, B, "released")
    if spec_slots.dtype != torch.int32 or spec_slots.dim() != 2 or spec_slots.shape[0] != B:
        raise ValueError("spec_slots must be int32 [B, t_max]")
    _dev(ssm, conv, spec_slots, accepted_len, mamba_pool_indices, released)
    P = _pool(ssm, conv)
    st = lib().gdn_spec_commit_index(ct.byref(P), _spec(None, None, spec_slots),
                                     _ptr(accepted_len), _ptr(mamba_pool_indices),
                                     _ptr(released), B, _stream(stream))
    _check(st, "gdn_spec_commit_index")


def gdn_spec_decode_commit(layer: Layer, ssm, conv, mamba_pool_indices, spec_ssm, spec_conv,
                           accepted_len, stream=None):
    _check_pool(layer, ssm, conv)
    B = mamba_pool_indices.numel()
    _i32(mamba_pool_indices, B, "mamba_pool_indices", required=True)
    _i32(accepted_len, B, "accepted_len", required=True)
    if spec_ssm is None or spec_ssm.dim() != 5 or spec_ssm.shape[0] != B:
        raise ValueError("spec_ssm must be [B, t_max, H_v, d_v, d_k]")
    _check_pool(layer, spec_ssm.flatten(0, 1),
                None if spec_conv is None else spec_conv.flatten(0, 1))
    _dev(ssm, conv, mamba_pool_indices, spec_ssm, spec_conv, accepted_len)
    L = layer.c_struct()
    P = _pool(ssm, conv)
    st = lib().gdn_spec_decode_commit(ct.byref(L), ct.byref(P), _ptr(mamba_pool_indices),
                                      _spec(spec_ssm, spec_conv), _ptr(accepted_len),
                                      B, _stream(stream))
    _check(st, "gdn_spec_decode_commit")


def gdn_slot_copy(layer: Layer, ssm, conv, src, dst, stream=None):
    _check_pool(layer, ssm, conv)
    _i32(src, None, "src", required=True)
    _i32(dst, src.numel(), "dst", required=True)
    _dev(ssm, conv, src, dst)
    L = layer.c_struct()
    P = _pool(ssm, conv)
    st = lib().gdn_slot_copy(ct.byref(L), ct.byref(P), _ptr(src), _ptr(dst), src.numel(),
                             _stream(stream))
    _check(st, "gdn_slot_copy")


def gdn_slot_zero(layer: Layer, ssm, conv, idx, stream=None):
    _check_pool(layer, ssm, conv)
    _i32(idx, None, "idx", required=True)
    _dev(ssm, conv, idx)
    L = layer.c_struct()
    P = _pool(ssm, conv)
    st = lib().gdn_slot_zero(ct.byref(L), ct.byref(P), _ptr(idx), idx.numel(), _stream(stream))
    _check(st, "gdn_slot_zero")


def gdn_slot_bytes(layer: Layer) -> int:
    L = layer.c_struct()
    return int(lib().gdn_slot_bytes(ct.byref(L)))


def gdn_slot_pack(layer: Layer, ssm, conv, idx, buffer=None, stream=None):
    """Slots idx [n] int32 -> a contiguous uint8 buffer of n packed items
    (allocated when not given); returns the buffer.  See include/gdn.h."""
    import torch
    _check_pool(layer, ssm, conv)
    _i32(idx, None, "idx", required=True)
    n = idx.numel()
    if buffer is None:
        with _on(stream):
            buffer = torch.empty(max(n * gdn_slot_bytes(layer), 16), dtype=torch.uint8,
                                 device=ssm.device)
    _dev(ssm, conv, idx, buffer)
    L = layer.c_struct()
    P = _pool(ssm, conv)
    st = lib().gdn_slot_pack(ct.byref(L), ct.byref(P), _ptr(idx), n, _ptr(buffer),
                             buffer.numel() * buffer.element_size(), _stream(stream))
    _check(st, "gdn_slot_pack")
    return buffer


def gdn_slot_unpack(layer: Layer, ssm, conv, buffer, idx, stream=None):
    _check_pool(layer, ssm, conv)
    _i32(idx, None, "idx", required=True)
    _dev(ssm, conv, idx, buffer)
    L = layer.c_struct()
    P = _pool(ssm, conv)
    st = lib().gdn_slot_unpack(ct.byref(L), ct.byref(P), _ptr(buffer),
                               buffer.numel() * buffer.element_size(), _ptr(idx), idx.numel(),
                               _stream(stream))
    _check(st, "gdn_slot_unpack")


def gdn_prefill_workspace_size(layer: Layer, N: int, max_seqlen: int, total_tokens: int,
                               chunk: int = 64) -> int:
    L = layer.c_struct()
    return int(lib().gdn_prefill_workspace_size(ct.byref(L), N, max_seqlen, total_tokens, chunk))


def gdn_prefill_chunked(layer: Layer, ssm, conv, dst_slots, init_slot, cu_seqlens, max_seqlen,
                        x, alpha, beta, conv_w, conv_b=None, out=None, workspace=None,
                        chunk: int = 64, ckpt_slots=None, ckpt_every: int = 128, stream=None):
    """x [total, C]; cu_seqlens [N+1] int32 (device); returns out [total, H_v, d_v] fp32.
    ckpt_slots [N, per_seq] int32: checkpoint k of sequence s (the state after
    (k+1)*ckpt_every tokens) goes to pool slot ckpt_slots[s, k].  A workspace
    allocated here is allocated on `stream` (the current stream if None)."""
    import torch
    _check_pool(layer, ssm, conv)
    N = dst_slots.numel()
    _i32(dst_slots, N, "dst_slots", required=True)
    _i32(init_slot, N, "init_slot")
    _i32(cu_seqlens, N + 1, "cu_seqlens", required=True)
    ck = None
    if ckpt_slots is not None:
        if ckpt_slots.dtype != torch.int32 or ckpt_slots.dim() != 2 or \
                ckpt_slots.shape[0] != N:
            raise ValueError("ckpt_slots must be int32 [N, per_seq]")
        ck = ct.byref(GdnPrefillCkpt(_ptr(ckpt_slots), int(ckpt_every), ckpt_slots.shape[1]))
    if x.dim() != 2:
        raise ValueError("x must be [total, C]")
    total = x.shape[0]
    _check_inputs(layer, total, x, alpha, beta, conv_w, conv_b)
    shape = (total, layer.n_v_heads, layer.d_v)
    _check_out(out, shape)
    need = gdn_prefill_workspace_size(layer, N, max_seqlen, total, chunk)
    with _on(stream):
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=x.device)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    _dev(ssm, conv, dst_slots, init_slot, cu_seqlens, x, alpha, beta, conv_w, conv_b, out,
         workspace, ckpt_slots)
    L = layer.c_struct()
    P = _pool(ssm, conv)
    inp = GdnInputs(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(conv_w), _ptr(conv_b))
    st = lib().gdn_prefill_chunked(ct.byref(L), ct.byref(P), _ptr(dst_slots), _ptr(init_slot),
                                   N, _ptr(cu_seqlens), int(max_seqlen), int(total), int(chunk),
                                   ct.byref(inp), _ptr(out), ck, _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "gdn_prefill_chunked")
    return out


def gdn_prefill_chunked_static(layer: Layer, ssm, conv, dst_slots, init_slot, cu_seqlens,
                               max_seqlen, x, alpha, beta, conv_w, conv_b=None, out=None,
                               chunk: int = 64, ckpt_slots=None, ckpt_every: int = 128,
                               stream=None):
    """gdn_prefill_chunked with the library's own workspace array (nothing is
    allocated by the library; `out` must be given for a call that allocates
    nothing at all).  See include/gdn.h."""
    import torch
    _check_pool(layer, ssm, conv)
    N = dst_slots.numel()
    _i32(dst_slots, N, "dst_slots", required=True)
    _i32(init_slot, N, "init_slot")
    _i32(cu_seqlens, N + 1, "cu_seqlens", required=True)
    ck = None
    if ckpt_slots is not None:
        if ckpt_slots.dtype != torch.int32 or ckpt_slots.dim() != 2 or \
                ckpt_slots.shape[0] != N:
            raise ValueError("ckpt_slots must be int32 [N, per_seq]")
        ck = ct.byref(GdnPrefillCkpt(_ptr(ckpt_slots), int(ckpt_every), ckpt_slots.shape[1]))
    if x.dim() != 2:
        raise ValueError("x must be [total, C]")
    total = x.shape[0]
    _check_inputs(layer, total, x, alpha, beta, conv_w, conv_b)
    shape = (total, layer.n_v_heads, layer.d_v)
    _check_out(out, shape)
    if out is None:
        with _on(stream):
            out = torch.empty(shape, dtype=torch.float32, device=x.device)
    _dev(ssm, conv, dst_slots, init_slot, cu_seqlens, x, alpha, beta, conv_w, conv_b, out,
         ckpt_slots)
    L = layer.c_struct()
    P = _pool(ssm, conv)
    inp = GdnInputs(_ptr(x), _ptr(alpha), _ptr(beta), _ptr(conv_w), _ptr(conv_b))
    st = lib().gdn_prefill_chunked_static(ct.byref(L), ct.byref(P), _ptr(dst_slots),
                                          _ptr(init_slot), N, _ptr(cu_seqlens), int(max_seqlen),
                                          int(total), int(chunk), ct.byref(inp), _ptr(out), ck,
                                          _stream(stream))
    _check(st, "gdn_prefill_chunked_static")
    return out
