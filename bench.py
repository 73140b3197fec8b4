#!/usr/bin/env python3
"""Benchmark of the GDN decode state step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Headline workload (the metric is quoted on it): a Qwen3.5-shaped Gated
DeltaNet layer -- 16 key / 32 value heads, d_k = d_v = 128, conv width 4 over
8192 q|k|v channels, bf16 inputs, fp32 state -- decoding B = 64 requests, one
token each, in place on a pool of 1024 slots.  Slot indices are distinct per
call, taken as consecutive 64-blocks of a seeded permutation of the pool that
is redrawn every 16 calls, so a slot comes back only after ~15 calls (about
1.9 GiB of other state in between, far above the 256 MB Infinity Cache).

A step is one gdn_decode_step call through the C ABI: conv update, head prep
and the gated delta rule for all 64 requests, in one kernel.  W warm-up steps,
then K timed steps between two HIP events on the launch stream.  One JSON line
goes to stdout.  Other paths of the state step are measured the same way and
reported under "paths".
"""
from __future__ import annotations

import argparse
import ctypes as ct
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA peak, TFLOP/s
DECODE_KERNEL = "decode_kernel<128, 32, bf16, false>"


def log(msg: str):
    print(msg, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------
# algorithmic bytes (what the method must move; see the design notes)

def decode_bytes(shape, B: int, T: int = 1, spec: bool = False) -> int:
    """HBM bytes of one decode call: state read + write (or T snapshot writes),
    conv window read + write, x, alpha, beta, taps, out, indices."""
    act = 2 if shape.dtype == "bf16" else 4
    C, W1 = shape.channels, shape.conv_width - 1
    state = shape.n_v_heads * shape.d_v * shape.d_k * 4
    conv = W1 * C * act
    n_state_w = T if spec else 1
    per_req = state * (1 + n_state_w) + conv * (1 + n_state_w)
    per_tok = C * act + shape.n_v_heads * act * (shape.d_k if shape.gate == "channel" else 1) \
        + shape.n_v_heads * act + shape.n_v_heads * shape.d_v * 4
    return B * per_req + B * T * per_tok + C * shape.conv_width * act + B * 4


def source_hash(path: str) -> str:
    """Hash of a kernel source's code: comments and whitespace are dropped,
    so only a change to the code itself retires counters taken on it.  (A
    quote inside a string or character literal is the source's business;
    these kernels have no comment markers inside literals.)"""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = "".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def traffic_from_profile(kernel_src: str):
    """HBM bytes per launch from the committed PMC summary, if it was taken on
    the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "decode_qwen35_b64_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_sha256_16") != source_hash(kernel_src):
        return None
    return d.get("hbm_bytes_per_launch")


# ----------------------------------------------------------------------------

class DecodeBench:
    """Device pools, inputs and pre-built C-ABI argument blocks for
    back-to-back decode calls, so the host loop issues launches far faster
    than the GPU retires them.  The pool holds n_distinct_slots seeded slot
    states replicated over all slots (values do not change the traffic)."""

    def __init__(self, torch, gdn, synth, shape, B, slots, n_calls, seed, n_inputs=64,
                 n_distinct_slots=64, T=1, spec=False, spec_pool=False, with_work=True):
        self.torch = torch
        rs = synth.streams(seed)
        base = synth.make_pool(shape, n_distinct_slots, np.arange(n_distinct_slots), rs)
        self.w_host = synth.make_conv_w(shape, rs)
        x, al, be = synth.make_tokens(shape, (n_inputs, B, T), rs)
        self.idx_host = synth.rotating_indices(slots, B, n_calls, rs["indices"])
        self.inputs_host = (x, al, be)
        self.base = base
        dev = _dev(torch)
        reps = -(-slots // n_distinct_slots)
        self.ssm = dev(base.ssm).repeat(reps, 1, 1, 1)[:slots].contiguous()
        self.conv = dev(base.conv).repeat(reps, 1, 1)[:slots].contiguous()
        self.w = dev(self.w_host)
        self.x, self.al, self.be = dev(x), dev(al), dev(be)
        self.idx = dev(self.idx_host)
        self.out = torch.empty((B, T, shape.n_v_heads, shape.d_v), dtype=torch.float32,
                               device="cuda")
        self.g = gdn.Layer(shape.n_k_heads, shape.n_v_heads, shape.d_k, shape.d_v,
                           shape.conv_width, shape.gate, shape.dtype)
        self.L = self.g.c_struct()
        self.P = gdn.GdnPool(self.ssm.data_ptr(), self.conv.data_ptr(), slots)
        # the work counter of the ticket-balanced tail (zero; each call leaves it at zero)
        self.work = torch.zeros(1, dtype=torch.int32, device="cuda") if with_work else None
        self.work_ptr = ct.c_void_p(self.work.data_ptr()) if with_work else None
        self.fn = gdn.lib().gdn_decode_step
        self.stream = ct.c_void_p(torch.cuda.current_stream().cuda_stream)
        self.B, self.T = B, T
        self.n_inputs = n_inputs
        self.inputs = [gdn.GdnInputs(self.x[i].data_ptr(), self.al[i].data_ptr(),
                                     self.be[i].data_ptr(), self.w.data_ptr(), None)
                       for i in range(n_inputs)]
        self.idx_ptrs = [ct.c_void_p(self.idx[c].data_ptr()) for c in range(n_calls)]
        self.out_ptr = ct.c_void_p(self.out.data_ptr())
        self.Lref, self.Pref = ct.byref(self.L), ct.byref(self.P)
        self.inref = [ct.byref(i) for i in self.inputs]
        self.spec = None
        self.specs = None
        if spec and spec_pool:
            # per call, B*T snapshot slots drawn from the slots no request of
            # that call works on
            g = np.random.default_rng(seed)
            tab = np.empty((n_calls, B, T), np.int32)
            for c in range(n_calls):
                free = np.setdiff1d(np.arange(slots, dtype=np.int32), self.idx_host[c])
                tab[c] = g.permutation(free)[:B * T].reshape(B, T)
            self.spec_slots_host = tab
            self.spec_slots = dev(tab)
            self.S_list = [gdn.GdnSpecCache(None, None, T, self.spec_slots[c].data_ptr())
                           for c in range(n_calls)]
            self.specs = [ct.byref(x) for x in self.S_list]
        elif spec:
            self.spec_ssm = torch.empty((B, T) + tuple(self.ssm.shape[1:]), dtype=torch.float32,
                                        device="cuda")
            self.spec_conv = torch.empty((B, T) + tuple(self.conv.shape[1:]),
                                         dtype=self.conv.dtype, device="cuda")
            self.S = gdn.GdnSpecCache(self.spec_ssm.data_ptr(), self.spec_conv.data_ptr(), T)
            self.spec = ct.byref(self.S)

    def call(self, c: int):
        spec = self.specs[c] if self.specs is not None else self.spec
        st = self.fn(self.Lref, self.Pref, self.idx_ptrs[c], None, self.B, self.T,
                     self.inref[c % self.n_inputs], self.out_ptr, spec, self.work_ptr, self.stream)
        if st != 0:
            raise RuntimeError(f"gdn_decode_step failed with status {st}")


def _dev(torch):
    def dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()
    return dev


def time_calls(torch, fn, first: int, n: int) -> float:
    """Milliseconds for n back-to-back calls fn(first..first+n-1) on the
    current stream, between two HIP events."""
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for c in range(first, first + n):
        fn(c)
    e.record()
    e.synchronize()
    return s.elapsed_time(e)


def cpu_baseline(synth, shape, bench: DecodeBench, budget_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    consecutive calls of the same index stream on fp64 copies of the pool."""
    import oracle
    o = oracle.Layer(shape.n_k_heads, shape.n_v_heads, shape.d_k, shape.d_v, shape.conv_width,
                     shape.gate)
    nthreads = oracle.default_threads()
    n_distinct = bench.base.ssm.shape[0]
    slots = int(bench.ssm.shape[0])
    reps = -(-slots // n_distinct)
    s64 = np.tile(oracle.as_f64(bench.base.ssm), (reps, 1, 1, 1))[:slots].copy()
    c64 = np.tile(oracle.as_f64(bench.base.conv), (reps, 1, 1))[:slots].copy()
    x, al, be = bench.inputs_host
    t0 = time.perf_counter()
    n = 0
    calls = bench.idx_host.shape[0]
    while True:
        i = n % bench.n_inputs
        oracle.decode(o, s64, c64, bench.idx_host[n % calls], x[i], al[i], be[i], bench.w_host,
                      nthreads=nthreads)
        n += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s:
            break
    return {"value": round(bench.B * n / dt, 2), "unit": "tokens/s", "cores": nthreads,
            "kind": "oracle",
            "sample": f"{n} consecutive B={bench.B} decode calls of the headline workload, "
                      f"its index stream repeated past {calls} calls "
                      f"(fp64 oracle, {nthreads} threads, {dt:.1f} s)"}


def _timed(fn, budget_s: float):
    """Calls fn() until about budget_s seconds have passed (at least twice);
    returns (calls, seconds)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        dt = time.perf_counter() - t0
        if n >= 2 and dt >= budget_s:
            return n, dt


def oracle_rates(synth, budget_s: float = 2.0) -> dict:
    """The fp64 oracle, as it stands, on bounded samples of each path's
    workload (same shapes and input recipe, fewer requests or tokens), timed
    on the host cores beside the GPU figures: tokens/s per path, and for the
    headline decode also a one-thread rate on 10 calls."""
    import oracle
    nthreads = oracle.default_threads()
    out = {}

    def olayer(shape):
        return oracle.Layer(shape.n_k_heads, shape.n_v_heads, shape.d_k, shape.d_v,
                            shape.conv_width, shape.gate)

    def decode_sample(shape, B, T, seed, spec=False, threads=nthreads, calls=None):
        case = synth.decode_case(shape, B=B, T=T, num_slots=B, n_calls=1, seed=seed,
                                 rotate=False)
        o = olayer(shape)
        s64, c64 = oracle.as_f64(case.pool.ssm).copy(), oracle.as_f64(case.pool.conv).copy()
        sp = None
        if spec:
            sp = (np.zeros((B, T) + s64.shape[1:]), np.zeros((B, T) + c64.shape[1:]))

        def one():
            oracle.decode(o, s64, c64, case.indices[0], case.x[0], case.alpha[0], case.beta[0],
                          case.conv_w, spec_ssm=None if sp is None else sp[0],
                          spec_conv=None if sp is None else sp[1], nthreads=threads)
        if calls is not None:
            t0 = time.perf_counter()
            for _ in range(calls):
                one()
            return calls, time.perf_counter() - t0
        return _timed(one, budget_s)

    def rec(tok_s, sample, threads=nthreads):
        return {"oracle_tok_s": round(tok_s, 2), "oracle_cores": threads,
                "oracle_sample": sample}

    n, dt = decode_sample(synth.QWEN35, 64, 1, 5, threads=1, calls=10)
    out["headline_one_thread"] = rec(64 * n / dt, f"{n} B=64 decode calls of the headline "
                                                  f"shape, one thread, {dt:.1f} s", 1)
    n, dt = decode_sample(synth.QWEN35, 16, 1, 1)
    out["decode_qwen35_b16"] = rec(16 * n / dt, f"{n} B=16 decode calls, {dt:.1f} s")
    n, dt = decode_sample(synth.QWEN35, 8, 7, 2, spec=True)
    out["spec_draft_qwen35_b64_t7"] = rec(8 * 7 * n / dt, f"{n} drafts of 7 tokens for 8 "
                                                          f"requests (snapshots), {dt:.1f} s")
    n, dt = decode_sample(synth.KDA, 64, 1, 4)
    out["kda_stack_b64_48layers"] = rec(64 * n / (48 * dt), f"{n} B=64 KDA layer calls "
                                                            f"(48 per step), {dt:.1f} s")
    for key, shape in (("prefill_qwen35_4x8192", synth.QWEN35), ("prefill_kda_4x8192", synth.KDA)):
        lens = [256] * 4
        case = synth.prefill_case(shape, lens, 8, seed=17)
        o = olayer(shape)

        def one():
            s64, c64 = oracle.as_f64(case.pool.ssm).copy(), oracle.as_f64(case.pool.conv).copy()
            oracle.prefill(o, s64, c64, case.dst, case.init_slot, case.cu_seqlens, case.x,
                           case.alpha, case.beta, case.conv_w, nthreads=nthreads)
        n, dt = _timed(one, budget_s)
        out[key] = rec(1024 * n / dt, f"{n} sequential prefills of 4 x 256 tokens (the "
                                      f"token-by-token recurrence), {dt:.1f} s")
    return out


def path_record(ms_per_call: float, nbytes: float, tokens: int, what: str) -> dict:
    gbs = nbytes / (ms_per_call * 1e-3) / 1e9
    return {"what": what, "us_per_call": round(ms_per_call * 1e3, 2),
            "tokens_per_s": round(tokens / (ms_per_call * 1e-3), 1),
            "algorithmic_bytes": int(nbytes), "hbm_gbps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def bench_decode_graph(torch, gdn, synth, n_calls=48, replays=20):
    """The headline decode (Qwen3.5 shape, B=64, 1024-slot pool) as a serving
    loop runs it: 48 calls (one per layer of a step, each with its own index
    row) captured in one HIP graph and replayed; the ticket tail keeps its
    caller-owned work counter (one word: the captured calls run in order).
    Returns the graph's per-call record and, for comparison, the same 48
    calls launched eagerly."""
    shape = synth.QWEN35
    b = DecodeBench(torch, gdn, synth, shape, 64, 1024, n_calls, seed=7)
    for c in range(n_calls):
        b.call(c)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    eager_stream = b.stream
    with torch.cuda.graph(graph):
        b.stream = ct.c_void_p(torch.cuda.current_stream().cuda_stream)
        for c in range(n_calls):
            b.call(c)
    b.stream = eager_stream
    for _ in range(2):
        graph.replay()
    torch.cuda.synchronize()
    ms = time_calls(torch, lambda _c: graph.replay(), 0, replays) / (replays * n_calls)
    eager = time_calls(torch, b.call, 0, n_calls) / n_calls
    nbytes = decode_bytes(shape, 64)
    rec = path_record(ms, nbytes, 64, "GDN decode, Qwen3.5 shape, B=64, pool 1024: 48 calls "
                      "captured in one HIP graph, replayed (work counter kept)")
    rec["eager_us_per_call_same_calls"] = round(eager * 1e3, 2)
    return rec


def bench_decode_b16(torch, gdn, synth, K=500, W=50):
    """Qwen3.5-shaped decode at B=16 on a 256-slot pool: indices rotating
    through a seeded permutation (reuse after 15 calls), and the literal
    draw -- 16 distinct slots drawn afresh for every call (reuse distance
    random, the pool's 512 MiB twice the Infinity Cache)."""
    shape = synth.QWEN35
    b = DecodeBench(torch, gdn, synth, shape, 16, 256, W + K, seed=1)
    for c in range(W):
        b.call(c)
    ms = time_calls(torch, b.call, W, K) / K
    rot = path_record(ms, decode_bytes(shape, 16), 16,
                      "GDN decode, Qwen3.5 shape, B=16, T=1, pool 256")
    g = np.random.default_rng(101)
    iid = np.stack([g.choice(256, 16, replace=False) for _ in range(W + K)]).astype(np.int32)
    b.idx.copy_(torch.from_numpy(iid))
    for c in range(W):
        b.call(c)
    ms = time_calls(torch, b.call, W, K) / K
    lit = path_record(ms, decode_bytes(shape, 16), 16,
                      "GDN decode, Qwen3.5 shape, B=16, T=1, pool 256, 16 distinct slots "
                      "drawn independently for every call")
    return rot, lit


def bench_spec(torch, gdn, synth, K=100, W=10):
    """Speculative draft of 7 tokens for B=64 into spec_cache (working slots
    untouched), then the commit of accepted lengths ~ U{0..7}."""
    shape = synth.QWEN35
    B, T = 64, 7
    b = DecodeBench(torch, gdn, synth, shape, B, 1024, W + K, seed=2, n_inputs=8, T=T, spec=True)
    for c in range(W):
        b.call(c)
    ms_draft = time_calls(torch, b.call, W, K) / K
    draft = path_record(ms_draft, decode_bytes(shape, B, T, spec=True), B * T,
                        "speculative draft, Qwen3.5 shape, B=64, 7 tokens, snapshots per token")
    acc_host = synth.accepted_lengths(B, T, seed=2)
    acc = torch.from_numpy(acc_host).cuda()
    fn = gdn.lib().gdn_spec_decode_commit
    acc_ptr = ct.c_void_p(acc.data_ptr())

    def commit(c):
        st = fn(b.Lref, b.Pref, b.idx_ptrs[c], b.spec, acc_ptr, B, b.stream)
        if st != 0:
            raise RuntimeError(f"gdn_spec_decode_commit failed with status {st}")
    for c in range(W):
        commit(c)
    ms_commit = time_calls(torch, commit, W, K) / K
    slot_bytes = shape.n_v_heads * shape.d_v * shape.d_k * 4 + \
        (shape.conv_width - 1) * shape.channels * 2
    commit_bytes = 2 * slot_bytes * int(np.count_nonzero(acc_host)) + 8 * B
    rec = path_record(ms_commit, commit_bytes, int(acc_host.sum()),
                      "commit of accepted lengths ~U{0..7}, B=64 (tokens = accepted)")
    return draft, rec


def bench_spec_pool(torch, gdn, synth, K=100, W=10):
    """The same draft with each snapshot written to a pool slot of its own
    (448 distinct slots per call, none a working slot), then the commit by
    index: the accepted snapshot's slot becomes the request's working slot,
    no state is copied."""
    shape = synth.QWEN35
    B, T = 64, 7
    b = DecodeBench(torch, gdn, synth, shape, B, 1024, W + K, seed=2, n_inputs=8, T=T, spec=True,
                    spec_pool=True)
    for c in range(W):
        b.call(c)
    ms_draft = time_calls(torch, b.call, W, K) / K
    draft = path_record(ms_draft, decode_bytes(shape, B, T, spec=True), B * T,
                        "speculative draft, Qwen3.5 shape, B=64, 7 tokens, snapshots into pool "
                        "slots")
    acc = torch.from_numpy(synth.accepted_lengths(B, T, seed=2)).cuda()
    idx = b.idx[0].clone()
    released = torch.empty_like(idx)
    fn = gdn.lib().gdn_spec_commit_index
    P = ct.byref(b.P)
    args = [(b.specs[c], ct.c_void_p(acc.data_ptr()), ct.c_void_p(idx.data_ptr()),
             ct.c_void_p(released.data_ptr())) for c in range(W + K)]

    def commit(c):
        st = fn(P, *args[c], B, b.stream)
        if st != 0:
            raise RuntimeError(f"gdn_spec_commit_index failed with status {st}")
    for c in range(W):
        commit(c)
    ms_commit = time_calls(torch, commit, W, K) / K
    rec = path_record(ms_commit, 16 * B, int(acc.sum().item()),
                      "commit by index of accepted lengths ~U{0..7}, B=64 (tokens = accepted; "
                      "bytes: indices only)")
    return draft, rec


def bench_slot_pack(torch, gdn, synth, K=50, W=5, n=64):
    """Pack 64 working slots of the Qwen3.5 layer into a contiguous buffer and
    unpack them into 64 other slots (the local half of moving state between
    engines); bytes = 2 x 64 packed items each way."""
    shape = synth.QWEN35
    b = DecodeBench(torch, gdn, synth, shape, n, 1024, 1, seed=6, n_inputs=1)
    g = b.g
    src = torch.arange(0, 2 * n, 2, dtype=torch.int32, device="cuda")
    dst = torch.arange(1, 2 * n, 2, dtype=torch.int32, device="cuda")
    item = gdn.gdn_slot_bytes(g)
    buf = torch.empty(n * item, dtype=torch.uint8, device="cuda")
    lib = gdn.lib()
    ptr = lambda t: ct.c_void_p(t.data_ptr())

    def pack(_c):
        assert lib.gdn_slot_pack(b.Lref, b.Pref, ptr(src), n, ptr(buf), n * item, b.stream) == 0

    def unpack(_c):
        assert lib.gdn_slot_unpack(b.Lref, b.Pref, ptr(buf), n * item, ptr(dst), n,
                                   b.stream) == 0
    out = []
    for fn, what in ((pack, "pack"), (unpack, "unpack")):
        for c in range(W):
            fn(c)
        ms = time_calls(torch, fn, W, K) / K
        rec = path_record(ms, 2 * n * item, n, f"slot {what}: 64 Qwen3.5 working slots "
                                               f"({item} B each) <-> contiguous buffer")
        out.append(rec)
    return out


def bench_kda_stack(torch, gdn, synth, K=20, W=3, layers=48):
    """KDA-style decode (per-channel gate), B=64, 32/32 heads, d=128, 48
    layers each with its own 1024-slot pool.  A step: slot preparation in
    every layer (16 fresh working slots zeroed, 16 copied from distinct
    checkpoint slots), then the 48 decode calls back to back."""
    shape = synth.KDA
    B, slots = 64, 1024
    base = DecodeBench(torch, gdn, synth, shape, B, slots, 1, seed=4, n_inputs=4)
    rs = synth.streams(4)
    roles = [rs["slot_roles"].permutation(slots).astype(np.int32) for _ in range(W + K)]
    dev = _dev(torch)
    idx = dev(np.stack([r[:64] for r in roles]))           # requests' working slots
    fresh = dev(np.stack([r[:16] for r in roles]))
    cow_dst = dev(np.stack([r[16:32] for r in roles]))
    cow_src = dev(np.stack([r[64:80] for r in roles]))     # checkpoints, not in the batch
    pools, convs, ws = [], [], []
    for l in range(layers):
        pools.append(base.ssm.clone())
        convs.append(base.conv.clone())
        ws.append(base.w)
    lib = gdn.lib()
    L = base.L
    P = [gdn.GdnPool(pools[l].data_ptr(), convs[l].data_ptr(), slots) for l in range(layers)]
    work = base.work_ptr
    Pr = [ct.byref(p) for p in P]
    ptr = lambda t: ct.c_void_p(t.data_ptr())
    idx_p = [ptr(idx[c]) for c in range(W + K)]
    fr_p = [ptr(fresh[c]) for c in range(W + K)]
    dst_p = [ptr(cow_dst[c]) for c in range(W + K)]
    src_p = [ptr(cow_src[c]) for c in range(W + K)]
    Lr, stream = ct.byref(L), base.stream

    def step(c):
        for l in range(layers):
            assert lib.gdn_slot_zero(Lr, Pr[l], fr_p[c], 16, stream) == 0
            assert lib.gdn_slot_copy(Lr, Pr[l], src_p[c], dst_p[c], 16, stream) == 0
        for l in range(layers):
            assert lib.gdn_decode_step(Lr, Pr[l], idx_p[c], None, B, 1, base.inref[(c + l) % 4],
                                       base.out_ptr, None, work, stream) == 0
    for c in range(W):
        step(c)
    ms = time_calls(torch, step, W, K) / K
    slot_bytes = shape.n_v_heads * shape.d_v * shape.d_k * 4 + \
        (shape.conv_width - 1) * shape.channels * 2
    prep_bytes = layers * (16 * slot_bytes + 16 * 2 * slot_bytes)
    nbytes = layers * decode_bytes(shape, B) + prep_bytes
    rec = path_record(ms, nbytes, B, "KDA decode stack: B=64, 32/32 heads, d=128, 48 layers, "
                                     "per step 16 zeroed + 16 copied slots per layer")
    rec["ms_per_step"] = rec.pop("us_per_call") / 1e3
    rec["prep_bytes"] = int(prep_bytes)

    # the same step with the preparation fused into the decode call: fresh
    # rows start from zeros (no state or window read), copy-on-write rows read
    # their checkpoint and write their working slot
    init_host = np.stack([r[:64] for r in roles]).copy()
    init_host[:, :16] = -1
    init_host[:, 16:32] = np.stack([r[64:80] for r in roles])
    init = dev(init_host)
    init_p = [ptr(init[c]) for c in range(W + K)]

    def fused(c):
        for l in range(layers):
            assert lib.gdn_decode_step(Lr, Pr[l], idx_p[c], init_p[c], B, 1,
                                       base.inref[(c + l) % 4], base.out_ptr, None, work,
                                       stream) == 0
    for c in range(W):
        fused(c)
    ms_f = time_calls(torch, fused, W, K) / K
    window = (shape.conv_width - 1) * shape.channels * 2
    state = shape.n_v_heads * shape.d_v * shape.d_k * 4
    nbytes_f = layers * (decode_bytes(shape, B) - 16 * (state + window))
    fused_rec = path_record(ms_f, nbytes_f, B, "KDA decode stack as above with the slot "
                                               "preparation fused into each decode call (16 "
                                               "zero starts read nothing, 16 copy-on-write "
                                               "rows read their checkpoint)")
    fused_rec["ms_per_step"] = fused_rec.pop("us_per_call") / 1e3
    del pools, convs
    return rec, fused_rec


def prefill_counts(shape, seqlens):
    """Algorithmic bytes and FLOPs of one chunked prefill call, and the bf16
    MFMA FLOPs the kernels issue.

    bytes: x read, o written (fp32), alpha (per value head, or per value head
    and key channel for the per-channel decay) and beta read, taps, and per
    sequence the final state + conv window written and the initial ones read
    (zero starts read nothing; counted as if every start were a copy).
    flops (dense, per (64-token chunk, value head)): the UT transform
    (K K^T, Q K^T, T V, W = T diag(e^g) K: 5.24 M) and the state pass
    (W S0^T, Q S0^T, P U, U^T K: 6.29 M) -- 11.53 MFLOP at d = 128; the
    per-channel decay changes elementwise factors only.
    issued, scalar decay (32-token blocks): per workgroup (64 value columns)
    and block, 6 Gram tiles and 4 waves of K S0^T, Q S0^T, P U and
    state-update tiles on 16x16x32 MFMAs; on 16x16x16 MFMAs the U solve (3
    block products per wave) and the two diagonal-block inverses (8 products
    each).
    issued, per-channel decay: 12 off-diagonal Gram tiles (the diagonal
    blocks are formed without MFMA), the same K S0^T, Q S0^T and P U tiles,
    and the state update as one 16x16x16 product per 16-token block.  Every
    product runs three times (hi/lo split).  rocprofv3's
    SQ_INSTS_VALU_MFMA_MOPS_BF16 (x 512 FLOP) agrees with the scalar-decay
    count."""
    act = 2 if shape.dtype == "bf16" else 4
    C, Hv, dk, dv = shape.channels, shape.n_v_heads, shape.d_k, shape.d_v
    kda = shape.gate == "channel"
    total = int(sum(seqlens))
    state = Hv * dv * dk * 4 + (shape.conv_width - 1) * C * act
    gate_elems = Hv * dk if kda else Hv
    nbytes = total * (C * act + (gate_elems + Hv) * act + Hv * dv * 4) \
        + C * shape.conv_width * act + 2 * state * len(seqlens)
    chunks = sum(-(-L // 64) for L in seqlens)
    c, dense = 64, 0
    dense += 2 * c * c * dk * 2 + c * c * dv * 2 + c * c * dk * 2     # KK^T, QK^T, TV, TK
    dense += 2 * c * dk * dv * 2 + c * c * dv * 2 + dv * c * dk * 2   # WS, QS, PU, U^T K
    flops = dense * chunks * Hv
    nblk = -(-dv // 64)
    ksl, kdt = dk // 32, dk // 16
    if kda:
        m32 = 12 * ksl * 3 + 4 * (4 * ksl * 2 * 3 + 6 * 3)
        m16 = 4 * 10 * 3 + 4 * kdt * 4 * 3
        steps = chunks
    else:
        m32 = 6 * ksl * 3 + 4 * (2 * ksl * 2 * 3 + 2 * 3 + kdt * 3)
        m16 = 4 * 3 * 3 + 2 * 8 * 3
        steps = sum(-(-L // 32) for L in seqlens)
    issued = (m32 * 16 * 16 * 32 * 2 + m16 * 16 * 16 * 16 * 2) * steps * Hv * nblk
    return nbytes, flops, issued


def bench_prefill(torch, gdn, synth, K=10, W=2, seqlens=(8192,) * 4, shape=None):
    """Chunked prefill, 4 x 8192 tokens, chunk 64, of the Qwen3.5 layer (scalar
    decay) or the KDA layer (per-channel decay): sequences alternate a zero
    start and a copy-on-write start from checkpoint slots."""
    shape = shape or synth.QWEN35
    kda = shape.gate == "channel"
    case = synth.prefill_case(shape, list(seqlens), 64, seed=17)
    dev = _dev(torch)
    g = gdn.Layer(shape.n_k_heads, shape.n_v_heads, shape.d_k, shape.d_v, shape.conv_width,
                  shape.gate, shape.dtype)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    dst, init, cu = dev(case.dst), dev(case.init_slot), dev(case.cu_seqlens)
    x, al, be, w = dev(case.x), dev(case.alpha), dev(case.beta), dev(case.conv_w)
    total = int(case.cu_seqlens[-1])
    out = torch.empty((total, shape.n_v_heads, shape.d_v), dtype=torch.float32, device="cuda")
    need = gdn.gdn_prefill_workspace_size(g, len(seqlens), max(seqlens), total)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")

    def call(_c):
        gdn.gdn_prefill_chunked(g, ssm, conv, dst, init, cu, max(seqlens), x, al, be, w, out=out,
                                workspace=ws)
    for c in range(W):
        call(c)
    ms = time_calls(torch, call, W, K) / K
    nbytes, flops, issued = prefill_counts(shape, seqlens)
    what = ("chunked prefill, KDA layer (32 heads, d=128, per-channel decay)" if kda else
            "chunked prefill, Qwen3.5 shape") + \
        ", 4 x 8192 tokens, chunk 64, zero / copy-on-write starts"
    rec = path_record(ms, nbytes, total, what)
    rec["algorithmic_tflops"] = round(flops / (ms * 1e-3) / 1e12, 1)
    rec["algorithmic_flops"] = int(flops)
    rec["mfma_issued_bf16_flops"] = int(issued)
    rec["mfma_issued_tflops"] = round(issued / (ms * 1e-3) / 1e12, 1)
    rec["mfma_issued_frac_of_bf16_peak"] = round(issued / (ms * 1e-3) / 1e12 /
                                                 MFMA_BF16_PEAK_TFLOPS, 4)
    rec["workspace_bytes"] = int(need)
    return rec


def bench_prefill_ckpt(torch, gdn, synth, K=10, W=2):
    """The agentic path on the Qwen3.5 layer: a 4 x 8192 prefill that also
    emits a checkpoint (state + conv window) every 128 tokens into 256 pool
    slots, and a short append of 4 x 512 tokens that starts from checkpoint
    slots (copy-on-write into fresh working slots)."""
    shape = synth.QWEN35
    seqlens, every = [8192] * 4, 128
    case = synth.prefill_case(shape, seqlens, 272, seed=18)
    dev = _dev(torch)
    g = gdn.Layer(shape.n_k_heads, shape.n_v_heads, shape.d_k, shape.d_v, shape.conv_width,
                  shape.gate, shape.dtype)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    used = set(case.dst.tolist()) | set(case.init_slot[case.init_slot >= 0].tolist())
    spare = np.array([s for s in range(272) if s not in used], np.int32)
    tab = dev(spare[:4 * 64].reshape(4, 64))
    x, al, be, w = dev(case.x), dev(case.alpha), dev(case.beta), dev(case.conv_w)
    dst, init, cu = dev(case.dst), dev(case.init_slot), dev(case.cu_seqlens)
    total = int(case.cu_seqlens[-1])
    out = torch.empty((total, shape.n_v_heads, shape.d_v), dtype=torch.float32, device="cuda")

    def full(_c):
        gdn.gdn_prefill_chunked(g, ssm, conv, dst, init, cu, 8192, x, al, be, w, out=out,
                                ckpt_slots=tab, ckpt_every=every)
    for c in range(W):
        full(c)
    ms = time_calls(torch, full, W, K) / K
    nbytes, flops, _ = prefill_counts(shape, seqlens)
    slot_bytes = shape.n_v_heads * shape.d_v * shape.d_k * 4 + \
        (shape.conv_width - 1) * shape.channels * 2
    ck_bytes = 4 * 64 * slot_bytes
    rec = path_record(ms, nbytes + ck_bytes, total, "chunked prefill, Qwen3.5 shape, 4 x 8192 "
                                                    "tokens, a checkpoint every 128 tokens "
                                                    "(256 slots)")
    rec["checkpoint_bytes"] = int(ck_bytes)
    # append: 4 x 512 tokens from checkpoints 16, 32, 48, 63 of the sequences
    alens = [512] * 4
    acu = dev(np.arange(0, 5 * 512, 512, dtype=np.int32))
    starts = dev(np.array([spare[16], spare[64 + 32], spare[128 + 48], spare[192 + 63]],
                          np.int32))
    adst = dev(spare[4 * 64:4 * 64 + 4].copy())
    ax, aal, abe = x[:2048].contiguous(), al[:2048].contiguous(), be[:2048].contiguous()
    aout = torch.empty((2048, shape.n_v_heads, shape.d_v), dtype=torch.float32, device="cuda")

    def append(_c):
        gdn.gdn_prefill_chunked(g, ssm, conv, adst, starts, acu, 512, ax, aal, abe, w, out=aout)
    for c in range(W):
        append(c)
    ms_a = time_calls(torch, append, W, 5 * K) / (5 * K)
    abytes, _, _ = prefill_counts(shape, alens)
    arec = path_record(ms_a, abytes, 2048, "short append, Qwen3.5 shape, 4 x 512 tokens, each "
                                           "starting from a checkpoint slot")
    return rec, arec


def copy_rate(torch, nbytes: int, reps: int = 200, pairs: int = 4) -> float:
    """GB/s of a plain device copy (torch copy_, read nbytes/2 + write
    nbytes/2 per call) moving the same byte volume as one decode call, over
    `pairs` rotating source / destination buffers so that a buffer comes back
    only after (pairs - 1) * nbytes of other traffic (1.1 GB here, more than
    twice the 256 MB Infinity Cache): the practical streaming ceiling the
    decode kernel is set against."""
    n = nbytes // 2 // 4
    bufs = [(torch.ones(n, device="cuda"), torch.empty(n, device="cuda")) for _ in range(pairs)]

    def one(c):
        src, dst = bufs[c % pairs]
        dst.copy_(src)
    for c in range(20):
        one(c)
    ms = time_calls(torch, one, 0, reps) / reps
    del bufs
    return 2 * n * 4 / (ms * 1e-3) / 1e9


def copy_calibration(torch, mib: int = 256, reps: int = 5):
    """A plain device copy of known size, for scaling the PMC byte counters."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty(n, device="cuda")
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {reps} copies of {mib} MiB (read {mib} MiB + write {mib} MiB each)")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle work for the cpu_baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "decode", "paths", "prefill", "prefill_kda",
                                       "copy"],
                    default="all",
                    help="profiling runs: just the headline decode, the other paths, or a "
                         "plain copy of known size")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the state step shards across GPUs with no "
              "exchange (requests or key-head groups per GPU), so only --gpus 1 is run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import hybrid_linear_attention_decode_amd as gdn
    from hybrid_linear_attention_decode_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gdn.lib()
    if args.only == "copy":
        copy_calibration(torch)
        return
    if args.only == "paths":
        for r in (*bench_decode_b16(torch, gdn, synth), bench_decode_graph(torch, gdn, synth),
                  *bench_spec(torch, gdn, synth),
                  *bench_spec_pool(torch, gdn, synth), *bench_kda_stack(torch, gdn, synth),
                  *bench_slot_pack(torch, gdn, synth),
                  bench_prefill(torch, gdn, synth), *bench_prefill_ckpt(torch, gdn, synth),
                  bench_prefill(torch, gdn, synth, shape=synth.KDA)):
            print(json.dumps(r), flush=True)
        return
    if args.only == "prefill":
        print(json.dumps(bench_prefill(torch, gdn, synth)), flush=True)
        return
    if args.only == "prefill_kda":
        print(json.dumps(bench_prefill(torch, gdn, synth, shape=synth.KDA)), flush=True)
        return

    shape = synth.QWEN35
    B, slots = 64, 1024
    K, W = args.steps, args.warmup
    log(f"bench: generating headline workload (B={B}, pool {slots}, {W}+{K} calls)")
    bench = DecodeBench(torch, gdn, synth, shape, B, slots, W + K, seed=5)
    for c in range(W):
        bench.call(c)
    torch.cuda.synchronize()
    log("bench: warm-up done, timing")
    ms = time_calls(torch, bench.call, W, K)
    ms_step = ms / K
    nbytes = decode_bytes(shape, B)
    achieved = nbytes / (ms_step * 1e-3) / 1e9
    tok_s = B / (ms_step * 1e-3)
    log(f"bench: {ms_step * 1e3:.2f} us/call, {tok_s:.0f} tok/s, {achieved:.0f} GB/s")
    copy_gbs = copy_rate(torch, nbytes)
    log(f"bench: device copy of the same byte volume: {copy_gbs:.0f} GB/s")

    kernel_src = os.path.join(ROOT, "hybrid_linear_attention_decode_amd", "csrc",
                              "gdn_decode.hip")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profile(kernel_src), "kernel": DECODE_KERNEL,
                "algorithmic_bytes_per_launch": nbytes,
                "copy_gbps": round(copy_gbs, 1), "frac_of_copy": round(achieved / copy_gbs, 4)}

    paths = None
    if args.only == "all":
        log("bench: other paths (B=16 decode, B=64 decode replayed from a HIP graph, "
            "speculative draft + commit with snapshots in "
            "spec buffers and in pool slots, KDA 48-layer stack with separate and fused slot "
            "preparation, slot pack / unpack, chunked prefill of both layers, with checkpoints and "
            "the append from them)")
        d16, d16_iid = bench_decode_b16(torch, gdn, synth)
        dgraph = bench_decode_graph(torch, gdn, synth)
        draft, commit = bench_spec(torch, gdn, synth)
        pdraft, pcommit = bench_spec_pool(torch, gdn, synth)
        kda, kda_fused = bench_kda_stack(torch, gdn, synth)
        pack, unpack = bench_slot_pack(torch, gdn, synth)
        pf = bench_prefill(torch, gdn, synth)
        pfc, app = bench_prefill_ckpt(torch, gdn, synth)
        pfk = bench_prefill(torch, gdn, synth, shape=synth.KDA)
        paths = {"decode_qwen35_b16": d16, "decode_qwen35_b16_iid": d16_iid,
                 "decode_qwen35_b64_graph": dgraph,
                 "spec_draft_qwen35_b64_t7": draft,
                 "spec_commit_qwen35_b64": commit,
                 "spec_draft_pool_slots_qwen35_b64_t7": pdraft,
                 "spec_commit_index_b64": pcommit,
                 "kda_stack_b64_48layers": kda, "kda_stack_b64_48layers_fused_prep": kda_fused,
                 "slot_pack_qwen35_64": pack, "slot_unpack_qwen35_64": unpack,
                 "prefill_qwen35_4x8192": pf, "prefill_qwen35_4x8192_ckpt128": pfc,
                 "append_qwen35_4x512_from_ckpt": app, "prefill_kda_4x8192": pfk}

    cpu = None
    if not args.no_cpu_baseline and args.only == "all":
        log("bench: timing the oracle sample")
        cpu = cpu_baseline(synth, shape, bench, args.cpu_budget)
        log("bench: timing the oracle on samples of the other paths")
        rates = oracle_rates(synth)
        cpu["one_thread_value"] = rates.pop("headline_one_thread")["oracle_tok_s"]
        for key, r in rates.items():
            if paths is not None and key in paths:
                paths[key].update(r)

    rec = {
        "metric": "GDN decode tokens/s and achieved HBM GB/s (fraction of peak) at B=64",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "GDN decode, Qwen3.5-shaped layer (16 key / 32 value heads, "
                               "d_k=d_v=128, conv width 4, 8192 channels), B=64, T=1, "
                               "pool 1024, bf16 inputs, fp32 state",
                   "global_batch": B, "tokens_per_request": 1, "pool_slots": slots},
        "hbm_gbps": round(achieved, 1),
        "hbm_frac": round(achieved / HBM_PEAK_GBS, 4),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "paths": paths,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
