"""Seeded synthetic workloads for the GDN / KDA state step.

Shared by the tests, the oracle-side checks and ``bench.py``.  This module
holds none of the method's arithmetic: it only draws random inputs with the
shapes and distributions of the workloads and encodes them (fp32 or bf16 bit
patterns).  Everything is numpy on the host.

Recipe (one ``numpy.random.SeedSequence(seed)`` spawned into independent
streams in a fixed order):

* ``pool_ssm``  live state slots ~ N(0, 1/d_k) in fp32; unused slots hold NaN;
* ``pool_conv`` live conv windows ~ N(0, 1); unused slots NaN;
* ``conv_w``    taps ~ U(-1/sqrt(W), 1/sqrt(W)); no bias;
* ``x``         token activations ~ N(0, 1);
* ``alpha``     exp(-softplus(z)), z ~ N(0, 1) (per value head, or per value
                head and key channel for the KDA gate);
* ``beta``      sigmoid(z'), z' ~ N(0, 1);
* ``indices``   distinct slot indices per call;
* ``accept``    accepted draft lengths, uniform in 0..T;
* ``slot_roles`` which slots are fresh / copied / live.

bf16 values are produced from fp32 by round-to-nearest-even and are carried
as ``uint16`` bit patterns, so the same bits reach the GPU and the oracle.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

STREAMS = ("pool_ssm", "pool_conv", "conv_w", "x", "alpha", "beta", "indices", "accept",
           "slot_roles")

BF16_NAN = np.uint16(0x7FC0)


def streams(seed: int) -> dict:
    """Independent generators, one per named stream, in the fixed order."""
    kids = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(k)) for name, k in zip(STREAMS, kids)}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); NaN stays a quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    return np.where(np.isnan(a), BF16_NAN, r).astype(np.uint16)


def encode(a: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 array -> storage array ('f32': float32, 'bf16': uint16 bits)."""
    if dtype == "f32":
        return np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(a)
    raise ValueError(dtype)


@dataclass
class Shape:
    """One linear-attention layer as the workloads describe it."""
    n_k_heads: int
    n_v_heads: int
    d_k: int
    d_v: int
    conv_width: int = 4
    gate: str = "scalar"   # "scalar" (GDN) or "channel" (KDA)
    dtype: str = "bf16"    # storage of x, alpha, beta, conv_w, conv_state

    @property
    def channels(self) -> int:
        return 2 * self.n_k_heads * self.d_k + self.n_v_heads * self.d_v


# the workloads' layer shapes
TINY = Shape(2, 2, 16, 16, 4, "scalar", "f32")          # 96 channels
QWEN35 = Shape(16, 32, 128, 128, 4, "scalar", "bf16")   # 8192 channels, GQA 2:1
KDA = Shape(32, 32, 128, 128, 4, "channel", "bf16")     # 12288 channels


def _normal(g, shape, scale=1.0):
    return (g.standard_normal(shape, dtype=np.float32) * np.float32(scale)).astype(np.float32)


def _softplus(z):
    return np.logaddexp(np.float32(0), z).astype(np.float32)


@dataclass
class Pool:
    ssm: np.ndarray          # [slots, H_v, d_v, d_k] float32
    conv: np.ndarray         # [slots, W-1, C] float32 or uint16 bits
    live: np.ndarray = field(default_factory=lambda: np.zeros(0, np.int32))


def make_pool(shape: Shape, num_slots: int, live, rs: dict) -> Pool:
    """Pool whose `live` slots (sorted order) hold random state; every other
    slot is NaN."""
    live = np.unique(np.asarray(live, dtype=np.int32))
    W1, C = shape.conv_width - 1, shape.channels
    per_slot = (shape.n_v_heads, shape.d_v, shape.d_k)
    ssm = np.empty((num_slots,) + per_slot, np.float32)
    conv = np.empty((num_slots, W1, C), np.float32)
    scale = np.float32(1.0 / np.sqrt(shape.d_k))
    if live.size == num_slots:   # draw straight into the pool (same values)
        rs["pool_ssm"].standard_normal(dtype=np.float32, out=ssm)
        ssm *= scale
        rs["pool_conv"].standard_normal(dtype=np.float32, out=conv)
    else:
        ssm.fill(np.nan)
        conv.fill(np.nan)
        if live.size:
            ssm[live] = _normal(rs["pool_ssm"], (live.size,) + per_slot, scale)
            conv[live] = _normal(rs["pool_conv"], (live.size, W1, C))
    return Pool(ssm, encode(conv, shape.dtype), live)


def make_conv_w(shape: Shape, rs: dict) -> np.ndarray:
    lim = 1.0 / np.sqrt(shape.conv_width)
    w = rs["conv_w"].uniform(-lim, lim, (shape.channels, shape.conv_width)).astype(np.float32)
    return encode(w, shape.dtype)


def make_tokens(shape: Shape, lead: tuple, rs: dict):
    """x [*lead, C], alpha [*lead, H_v(, d_k)], beta [*lead, H_v]."""
    x = _normal(rs["x"], lead + (shape.channels,))
    ash = lead + ((shape.n_v_heads, shape.d_k) if shape.gate == "channel" else (shape.n_v_heads,))
    alpha = np.exp(-_softplus(_normal(rs["alpha"], ash))).astype(np.float32)
    z = _normal(rs["beta"], lead + (shape.n_v_heads,))
    beta = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    return encode(x, shape.dtype), encode(alpha, shape.dtype), encode(beta, shape.dtype)


def rotating_indices(num_slots: int, B: int, n_calls: int, g) -> np.ndarray:
    """[n_calls, B] distinct indices per call: consecutive B-blocks of a seeded
    permutation of the pool, reshuffled whenever it is used up, so a slot is
    revisited only after about num_slots/B calls."""
    if B > num_slots:
        raise ValueError("more requests than slots")
    per = num_slots // B
    out = np.empty((n_calls, B), np.int32)
    perm = None
    for c in range(n_calls):
        if c % per == 0:
            perm = g.permutation(num_slots).astype(np.int32)
        k = c % per
        out[c] = perm[k * B:(k + 1) * B]
    return out


@dataclass
class DecodeCase:
    shape: Shape
    pool: Pool
    conv_w: np.ndarray
    x: np.ndarray          # [n_calls, B, T, C]
    alpha: np.ndarray      # [n_calls, B, T, H_v(, d_k)]
    beta: np.ndarray       # [n_calls, B, T, H_v]
    indices: np.ndarray    # [n_calls, B] int32


def decode_case(shape: Shape, B: int, T: int, num_slots: int, n_calls: int, seed: int,
                all_live: bool = False, rotate: bool = True) -> DecodeCase:
    """Decode workload: every slot that any call touches is live; the rest of
    the pool is NaN-poisoned unless all_live.  rotate=False keeps one seeded
    draw of B distinct slots for every call."""
    rs = streams(seed)
    if rotate:
        idx = rotating_indices(num_slots, B, n_calls, rs["indices"])
    else:
        one = rs["indices"].permutation(num_slots)[:B].astype(np.int32)
        idx = np.tile(one, (n_calls, 1))
    live = np.arange(num_slots, dtype=np.int32) if all_live else np.unique(idx)
    pool = make_pool(shape, num_slots, live, rs)
    w = make_conv_w(shape, rs)
    x, a, b = make_tokens(shape, (n_calls, B, T), rs)
    return DecodeCase(shape, pool, w, x, a, b, idx)


def accepted_lengths(B: int, T: int, seed: int) -> np.ndarray:
    """Accepted draft lengths, i.i.d. uniform in 0..T."""
    return streams(seed)["accept"].integers(0, T + 1, B).astype(np.int32)


@dataclass
class PrefillCase:
    shape: Shape
    pool: Pool
    conv_w: np.ndarray
    x: np.ndarray          # [total, C]
    alpha: np.ndarray      # [total, H_v(, d_k)]
    beta: np.ndarray       # [total, H_v]
    cu_seqlens: np.ndarray  # [N+1] int32
    dst: np.ndarray        # [N] destination working slots
    init_slot: np.ndarray  # [N]: -1 zero state, else copy-on-write source


def prefill_case(shape: Shape, seqlens, num_slots: int, seed: int) -> PrefillCase:
    """Variable-length prefill: sequence s writes slot dst[s]; it starts from
    zeros (init -1) or from a distinct live checkpoint slot, alternating so
    both kinds occur.  Destination slots start NaN-poisoned (fresh)."""
    rs = streams(seed)
    N = len(seqlens)
    if 2 * N > num_slots:
        raise ValueError("pool too small")
    perm = rs["slot_roles"].permutation(num_slots).astype(np.int32)
    dst, ckpt = perm[:N], perm[N:2 * N]
    init = np.where(np.arange(N) % 2 == 0, -1, ckpt).astype(np.int32)
    pool = make_pool(shape, num_slots, np.sort(ckpt), rs)
    w = make_conv_w(shape, rs)
    cu = np.zeros(N + 1, np.int32)
    cu[1:] = np.cumsum(np.asarray(seqlens, dtype=np.int64))
    x, a, b = make_tokens(shape, (int(cu[-1]),), rs)
    return PrefillCase(shape, pool, w, x, a, b, cu, dst, init)
