"""GPU parity of the decode path, the speculative snapshots/commit and the slot
operations, through the C ABI, against the fp64 oracle on the same seeded
inputs.  Bar: outputs max|do|/max|o| <= 2e-3; final state <= 1e-4 after 16
fp32 steps; slot indexing, copy, zero and rollback bit-exact."""
import numpy as np
import pytest

import oracle
import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import synth
from tests.harness import OUT_TOL, STATE_TOL_16, bits, dev, host, layers, rel_err, shadow

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


class DevCase:
    """Device copies of a seeded decode case; with_work: a work counter is
    passed to every call (the last quarter of the units handed out by
    ticket)."""

    def __init__(self, case: synth.DecodeCase, with_work: bool = False):
        self.ssm = dev(case.pool.ssm)
        self.conv = dev(case.pool.conv)
        self.w = dev(case.conv_w)
        self.case = case
        self.work = gdn.decode_work() if with_work else None

    def call(self, g, c, out=None, spec=None, idx=None):
        cs = self.case
        ix = dev(cs.indices[c] if idx is None else idx)
        spec_ssm, spec_conv = spec if spec is not None else (None, None)
        return gdn.gdn_decode_step(g, self.ssm, self.conv, ix, dev(cs.x[c]), dev(cs.alpha[c]),
                                   dev(cs.beta[c]), self.w, out=out, spec_ssm=spec_ssm,
                                   spec_conv=spec_conv, work=self.work)

    def work_is_zero(self):
        return self.work is None or not bool(self.work.any())


def run_oracle(o, case, s64, c64, calls, T=None):
    outs = []
    for c in calls:
        outs.append(oracle.decode(o, s64, c64, case.indices[c], case.x[c], case.alpha[c],
                                  case.beta[c], case.conv_w))
    return outs


def test_tiny_fp32_16_steps():
    """Tiny GDN decode: B=1, 2/2 heads, d=16, 96 channels, pool 4, 16 steps,
    fp32 throughout.  State within 1e-4 after 16 steps; other slots untouched."""
    torch = _torch()
    case = synth.decode_case(synth.TINY, B=1, T=1, num_slots=4, n_calls=16, seed=0, rotate=False)
    g, o = layers(synth.TINY)
    d = DevCase(case)
    before = bits(d.ssm), bits(d.conv)
    outs = [host(d.call(g, c)) for c in range(16)]
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    refs = run_oracle(o, case, s64, c64, range(16))
    for c in range(16):
        assert rel_err(outs[c], refs[c]) <= OUT_TOL
    slot = int(case.indices[0, 0])
    assert rel_err(host(d.ssm)[slot], s64[slot]) <= STATE_TOL_16
    np.testing.assert_array_equal(host(d.conv)[slot], c64[slot].astype(np.float32))
    others = [s for s in range(4) if s != slot]
    np.testing.assert_array_equal(bits(d.ssm)[others], before[0][others])
    np.testing.assert_array_equal(bits(d.conv)[others], before[1][others])


def test_tiny_multi_token_call_equals_single_steps_bitwise():
    case = synth.decode_case(synth.TINY, B=1, T=1, num_slots=4, n_calls=16, seed=0, rotate=False)
    g, _ = layers(synth.TINY)
    a, b = DevCase(case), DevCase(case)
    outs = [a.call(g, c) for c in range(16)]
    torch = _torch()
    x = dev(case.x[:, 0, 0][None])                       # [1, 16, C]
    al = dev(case.alpha[:, 0, 0][None])
    be = dev(case.beta[:, 0, 0][None])
    o16 = gdn.gdn_decode_step(g, b.ssm, b.conv, dev(case.indices[0]), x, al, be, b.w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o16)[0], np.stack([bits(t)[0, 0] for t in outs]))
    np.testing.assert_array_equal(bits(a.ssm), bits(b.ssm))
    np.testing.assert_array_equal(bits(a.conv), bits(b.conv))


@pytest.mark.parametrize("B,slots,n_calls,seed,with_work",
                         [(16, 256, 1000, 1, True), (64, 1024, 40, 5, True),
                          (64, 1024, 10, 5, False)],
                         ids=["b16_1000_calls", "b64_headline", "b64_no_work_counter"])
def test_qwen35_full_run(B, slots, n_calls, seed, with_work):
    """Qwen3.5-shaped layer, 16/32 heads, d=128, 8192 channels, bf16 inputs,
    fp32 state, rotating distinct indices, T=1, in the launch configuration
    the bench times (a work counter passed: the last quarter of the units by
    ticket): B=16 over a 256-slot pool for 1000 calls, and the headline B=64
    over a 1024-slot pool (seed of the bench) for 40 calls; and without the
    counter (every unit fixed).  Every output of every call against the
    oracle, then the final pool; the counter ends at zero."""
    torch = _torch()
    case = synth.decode_case(synth.QWEN35, B=B, T=1, num_slots=slots, n_calls=n_calls, seed=seed)
    g, o = layers(synth.QWEN35)
    d = DevCase(case, with_work)
    out = torch.empty((n_calls, B, 1, 32, 128), dtype=torch.float32, device="cuda")
    x, al, be, ix = dev(case.x), dev(case.alpha), dev(case.beta), dev(case.indices)
    for c in range(n_calls):
        gdn.gdn_decode_step(g, d.ssm, d.conv, ix[c], x[c], al[c], be[c], d.w, out=out[c],
                            work=d.work)
    torch.cuda.synchronize()
    assert d.work_is_zero()
    got = host(out)
    s64, c64 = shadow(case.pool)
    worst = 0.0
    for c in range(n_calls):
        ref = oracle.decode(o, s64, c64, case.indices[c], case.x[c], case.alpha[c],
                            case.beta[c], case.conv_w)
        worst = max(worst, rel_err(got[c], ref))
    print(f"qwen35 B={B} x {n_calls} calls: worst max|do|/max|o| = {worst:.3e}")
    assert worst <= OUT_TOL
    live = np.unique(case.indices)
    assert rel_err(host(d.ssm)[live], s64[live]) <= OUT_TOL
    np.testing.assert_array_equal(host(d.conv)[live],
                                  synth.f32_to_bf16_bits(c64[live].astype(np.float32)))


@pytest.mark.parametrize("shape,B", [(synth.QWEN35, 64), (synth.TINY, 64)])
def test_spec_draft_commit_equals_recomputation(shape, B):
    """Speculative decode commit: 7 draft tokens per request, snapshots into
    spec_cache, accepted length uniform in 0..7, commit; each working slot is
    bit-exact versus an in-place decode of only the accepted prefix, and the
    draft outputs match the oracle."""
    torch = _torch()
    T, slots = 7, (1024 if shape is synth.QWEN35 else 256)
    case = synth.decode_case(shape, B=B, T=T, num_slots=slots, n_calls=1, seed=2)
    acc = synth.accepted_lengths(B, T, seed=2)
    assert acc.min() == 0 and acc.max() == T
    g, o = layers(shape)
    a, r = DevCase(case), DevCase(case)
    pre_ssm, pre_conv = bits(a.ssm), bits(a.conv)
    sp_ssm = torch.full((B, T) + tuple(a.ssm.shape[1:]), float("nan"), device="cuda")
    sp_conv = torch.zeros((B, T) + tuple(a.conv.shape[1:]), dtype=a.conv.dtype, device="cuda")
    out = a.call(g, 0, spec=(sp_ssm, sp_conv))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(a.ssm), pre_ssm)           # draft leaves the pool
    np.testing.assert_array_equal(bits(a.conv), pre_conv)
    gdn.gdn_spec_decode_commit(g, a.ssm, a.conv, dev(case.indices[0]), sp_ssm, sp_conv, dev(acc))
    # recomputation: requests grouped by accepted length, in-place decode of L tokens
    for L in range(1, T + 1):
        sel = np.nonzero(acc == L)[0]
        if sel.size == 0:
            continue
        o_r = gdn.gdn_decode_step(g, r.ssm, r.conv, dev(case.indices[0][sel]),
                                  dev(case.x[0][sel, :L]), dev(case.alpha[0][sel, :L]),
                                  dev(case.beta[0][sel, :L]), r.w)
        np.testing.assert_array_equal(bits(o_r), bits(out)[sel, :L])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(a.ssm), bits(r.ssm))
    np.testing.assert_array_equal(bits(a.conv), bits(r.conv))
    # draft outputs and snapshots against the oracle
    s64, c64 = shadow(case.pool)
    sp64 = np.zeros((B, T) + s64.shape[1:])
    spc64 = np.zeros((B, T) + c64.shape[1:])
    ref = oracle.decode(o, s64, c64, case.indices[0], case.x[0], case.alpha[0], case.beta[0],
                        case.conv_w, spec_ssm=sp64, spec_conv=spc64)
    assert rel_err(host(out), ref) <= OUT_TOL
    assert rel_err(host(sp_ssm), sp64) <= OUT_TOL
    got_c = host(sp_conv)
    want_c = spc64.astype(np.float32)
    if shape.dtype == "bf16":
        want_c = synth.f32_to_bf16_bits(want_c)
    np.testing.assert_array_equal(got_c, want_c)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("T", [9, 16, 20])
def test_calls_longer_than_one_lds_chunk(gate, T):
    """Calls of more than 8 tokens: the kernel holds the activations of 8
    tokens in LDS at a time and walks the call's tokens in chunks of 8.  In
    place: outputs, states and windows against the oracle.  With snapshots:
    outputs bit for bit equal to the in-place call, the last snapshot equal to
    the in-place state and window, every snapshot against the oracle."""
    torch = _torch()
    shape = synth.Shape(2, 4, 64, 64, 4, gate, "bf16")   # two value heads per key head
    B = 6
    case = synth.decode_case(shape, B=B, T=T, num_slots=16, n_calls=1, seed=40 + T)
    g, o = layers(shape)
    a, b = DevCase(case), DevCase(case)
    out = a.call(g, 0)
    sp_ssm = torch.full((B, T) + tuple(b.ssm.shape[1:]), float("nan"), device="cuda")
    sp_conv = torch.zeros((B, T) + tuple(b.conv.shape[1:]), dtype=b.conv.dtype, device="cuda")
    out_s = b.call(g, 0, spec=(sp_ssm, sp_conv))
    torch.cuda.synchronize()
    idx = case.indices[0]
    s64, c64 = shadow(case.pool)
    ref = oracle.decode(o, s64, c64, idx, case.x[0], case.alpha[0], case.beta[0], case.conv_w)
    assert rel_err(host(out), ref) <= OUT_TOL
    assert rel_err(host(a.ssm)[idx], s64[idx]) <= STATE_TOL_16
    np.testing.assert_array_equal(host(a.conv)[idx],
                                  synth.encode(c64[idx].astype(np.float32), shape.dtype))
    np.testing.assert_array_equal(bits(out_s), bits(out))
    np.testing.assert_array_equal(bits(sp_ssm)[:, T - 1], bits(a.ssm)[idx])
    np.testing.assert_array_equal(bits(sp_conv)[:, T - 1], bits(a.conv)[idx])
    s64, c64 = shadow(case.pool)
    sp64 = np.zeros((B, T) + s64.shape[1:])
    spc64 = np.zeros((B, T) + c64.shape[1:])
    oracle.decode(o, s64, c64, idx, case.x[0], case.alpha[0], case.beta[0], case.conv_w,
                  spec_ssm=sp64, spec_conv=spc64)
    assert rel_err(host(sp_ssm), sp64) <= OUT_TOL
    np.testing.assert_array_equal(host(sp_conv),
                                  synth.encode(spc64.astype(np.float32), shape.dtype))


@pytest.mark.parametrize("shape", [synth.QWEN35, synth.KDA], ids=["qwen35", "kda"])
def test_run_twice_bitwise(shape):
    """The same calls on two copies of the same pool give the same bits: with
    the work counter the tail units go to whichever workgroups draw them, which
    differs from run to run, and nothing of a unit's arithmetic may depend on
    that.  B=64 over a 256-slot pool, 3 calls of T=2."""
    torch = _torch()
    case = synth.decode_case(shape, B=64, T=2, num_slots=256, n_calls=3, seed=44)
    g, _ = layers(shape)
    runs = []
    for _ in range(2):
        d = DevCase(case, with_work=True)
        outs = [bits(d.call(g, c)) for c in range(3)]
        torch.cuda.synchronize()
        assert d.work_is_zero()
        runs.append((outs, bits(d.ssm), bits(d.conv)))
    for c in range(3):
        np.testing.assert_array_equal(runs[0][0][c], runs[1][0][c])
    np.testing.assert_array_equal(runs[0][1], runs[1][1])
    np.testing.assert_array_equal(runs[0][2], runs[1][2])


def test_slot_zero_copy_bitwise_and_isolated():
    torch = _torch()
    shape = synth.QWEN35
    rs = synth.streams(7)
    pool = synth.make_pool(shape, 24, np.arange(24), rs)
    g, _ = layers(shape)
    ssm, conv = dev(pool.ssm), dev(pool.conv)
    s0, c0 = bits(ssm), bits(conv)
    src = np.array([3, 11, 20], np.int32)
    dst = np.array([7, 0, 15], np.int32)
    gdn.gdn_slot_copy(g, ssm, conv, dev(src), dev(dst))
    zi = np.array([5, -1, 23, 999], np.int32)               # pad and out-of-range skipped
    gdn.gdn_slot_zero(g, ssm, conv, dev(zi))
    torch.cuda.synchronize()
    s1, c1 = bits(ssm), bits(conv)
    for a_, b_ in zip(src, dst):
        np.testing.assert_array_equal(s1[b_], s0[a_])
        np.testing.assert_array_equal(c1[b_], c0[a_])
    for z in (5, 23):
        assert not s1[z].any() and not c1[z].any()          # +0.0 bit patterns
    untouched = [k for k in range(24) if k not in (7, 0, 15, 5, 23)]
    np.testing.assert_array_equal(s1[untouched], s0[untouched])
    np.testing.assert_array_equal(c1[untouched], c0[untouched])


def test_beta0_alpha1_state_unchanged_bitwise():
    torch = _torch()
    case = synth.decode_case(synth.QWEN35, B=8, T=3, num_slots=16, n_calls=1, seed=8)
    g, _ = layers(synth.QWEN35)
    d = DevCase(case)
    s0 = bits(d.ssm)
    ones = synth.f32_to_bf16_bits(np.ones(case.alpha.shape[1:], np.float32))
    zeros = synth.f32_to_bf16_bits(np.zeros(case.beta.shape[1:], np.float32))
    gdn.gdn_decode_step(g, d.ssm, d.conv, dev(case.indices[0]), dev(case.x[0]), dev(ones),
                        dev(zeros), d.w)
    torch.cuda.synchronize()
    # equal as values: the fp32 normal draw holds a few exact zeros, and an
    # added signed-zero update may turn -0.0 into +0.0 (still equal)
    live = case.indices[0]
    np.testing.assert_array_equal(host(d.ssm)[live], case.pool.ssm[live])
    nz = case.pool.ssm[live] != 0
    np.testing.assert_array_equal(bits(d.ssm)[live][nz], s0[live][nz])
    rest = np.setdiff1d(np.arange(16), live)
    np.testing.assert_array_equal(bits(d.ssm)[rest], s0[rest])


def test_skipped_rows_and_permutation_bitwise():
    """Negative (pad) and out-of-range indices leave rows untouched; permuting
    requests and their slots permutes the results bit for bit."""
    torch = _torch()
    case = synth.decode_case(synth.QWEN35, B=6, T=2, num_slots=16, n_calls=1, seed=9)
    g, _ = layers(synth.QWEN35)
    idx = case.indices[0].copy()
    idx[1], idx[4] = -1, 16                                 # pad row, out-of-range row
    a, b = DevCase(case), DevCase(case)
    s0 = bits(a.ssm)
    out_a = torch.full((6, 2, 32, 128), 7.0, device="cuda")
    a.call(g, 0, out=out_a, idx=idx)
    p = np.array([3, 5, 0, 2, 1, 4])
    out_b = torch.full((6, 2, 32, 128), 7.0, device="cuda")
    gdn.gdn_decode_step(g, b.ssm, b.conv, dev(idx[p]), dev(case.x[0][p]), dev(case.alpha[0][p]),
                        dev(case.beta[0][p]), b.w, out=out_b)
    torch.cuda.synchronize()
    oa = host(out_a)
    assert (oa[1] == 7.0).all() and (oa[4] == 7.0).all()
    np.testing.assert_array_equal(bits(out_a)[p], bits(out_b))
    np.testing.assert_array_equal(bits(a.ssm), bits(b.ssm))
    np.testing.assert_array_equal(bits(a.conv), bits(b.conv))
    touched = set(int(i) for i in idx if 0 <= i < 16)
    for k in range(16):
        if k not in touched:
            np.testing.assert_array_equal(bits(a.ssm)[k], s0[k])


def test_poisoned_fresh_slots_clean_after_zero_or_cow():
    """NaN-poisoned free slots never leak after explicit zeroing or CoW from a
    clean checkpoint; CoW-then-decode equals decoding the checkpoint's state."""
    torch = _torch()
    shape = synth.QWEN35
    case = synth.decode_case(shape, B=4, T=2, num_slots=12, n_calls=1, seed=10)
    g, o = layers(shape)
    d = DevCase(case)
    live = case.pool.live
    fresh = np.array([s for s in range(12) if s not in set(live.tolist())][:4], np.int32)
    assert np.isnan(host(d.ssm)[fresh]).all()
    gdn.gdn_slot_zero(g, d.ssm, d.conv, dev(fresh[:2]))
    gdn.gdn_slot_copy(g, d.ssm, d.conv, dev(live[:2]), dev(fresh[2:]))
    out = d.call(g, 0, idx=fresh)
    torch.cuda.synchronize()
    assert np.isfinite(host(out)).all()
    assert np.isfinite(host(d.ssm)[fresh]).all()
    s64, c64 = shadow(case.pool)
    s64[fresh[:2]] = 0.0
    c64[fresh[:2]] = 0.0
    s64[fresh[2:]] = s64[live[:2]]
    c64[fresh[2:]] = c64[live[:2]]
    ref = oracle.decode(o, s64, c64, fresh, case.x[0], case.alpha[0], case.beta[0], case.conv_w)
    assert rel_err(host(out), ref) <= OUT_TOL


@pytest.mark.parametrize("kw", [
    dict(shape=synth.Shape(4, 16, 64, 32, 2, "scalar", "f32"), layer=dict(conv_silu=False)),
    dict(shape=synth.Shape(2, 2, 32, 48, 1, "channel", "bf16"), layer=dict(l2norm=False)),
    dict(shape=synth.Shape(1, 4, 16, 64, 3, "channel", "f32"), layer=dict(q_scale=0.5)),
    dict(shape=synth.Shape(8, 8, 128, 256, 4, "scalar", "bf16"), layer=dict()),
    dict(shape=synth.Shape(2, 8, 128, 32, 4, "scalar", "bf16"), layer=dict()),
    dict(shape=synth.Shape(1, 2, 128, 64, 3, "channel", "f32"), layer=dict()),
])
@pytest.mark.parametrize("with_work", [False, True], ids=["fixed", "ticket"])
def test_other_shapes_against_oracle(kw, with_work):
    """d_k in {16, 32, 64, 128}, d_v != d_k, GQA 1:1 / 2:1 / 4:1, conv widths
    1-4, both gates and dtypes, flags off; 5 steps of T=2; without and with a
    work counter."""
    torch = _torch()
    shape = kw["shape"]
    case = synth.decode_case(shape, B=3, T=2, num_slots=8, n_calls=5, seed=11)
    g, o = layers(shape, **kw["layer"])
    d = DevCase(case, with_work)
    outs = [d.call(g, c) for c in range(5)]
    torch.cuda.synchronize()
    assert d.work_is_zero()
    s64, c64 = shadow(case.pool)
    refs = run_oracle(o, case, s64, c64, range(5))
    for c in range(5):
        assert rel_err(host(outs[c]), refs[c]) <= OUT_TOL
    live = case.pool.live
    assert rel_err(host(d.ssm)[live], s64[live]) <= STATE_TOL_16


@pytest.mark.parametrize("shape,B", [(synth.TINY, 9), (synth.Shape(3, 6, 128, 64, 4, "scalar", "bf16"), 5)])
def test_unit_counts_not_a_multiple_of_eight(shape, B):
    """B * H_k = 18 and 15 units, with a work counter: the workgroup -> unit
    order deals blocks of units to the XCDs, leaves the remainder in place and
    hands out the tail by ticket; every unit is run exactly once (outputs and
    states against the oracle, every slot outside the batch bit-identical)."""
    torch = _torch()
    slots = 2 * B + 3
    case = synth.decode_case(shape, B=B, T=1, num_slots=slots, n_calls=3, seed=12)
    g, o = layers(shape)
    d = DevCase(case, with_work=True)
    before = bits(d.ssm), bits(d.conv)
    outs = [d.call(g, c) for c in range(3)]
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    refs = run_oracle(o, case, s64, c64, range(3))
    for c in range(3):
        assert rel_err(host(outs[c]), refs[c]) <= OUT_TOL
    used = np.unique(case.indices[:3])
    assert rel_err(host(d.ssm)[used], s64[used]) <= STATE_TOL_16
    others = np.setdiff1d(np.arange(slots), used)
    np.testing.assert_array_equal(bits(d.ssm)[others], before[0][others])
    np.testing.assert_array_equal(bits(d.conv)[others], before[1][others])


def test_kda_decode_with_slot_prep():
    """KDA-style decode (per-channel gate), 32/32 heads, d=128: a quarter of the
    requests on zeroed fresh slots, a quarter CoW from checkpoints, then decode;
    3 steps against the oracle."""
    torch = _torch()
    shape = synth.KDA
    B, slots = 16, 64
    case = synth.decode_case(shape, B=B, T=1, num_slots=slots, n_calls=3, seed=4,
                             all_live=True, rotate=False)
    g, o = layers(shape)
    d = DevCase(case)
    idx = case.indices[0]
    fresh, cow = idx[:4], idx[4:8]
    ckpt = np.array([s for s in range(slots) if s not in set(idx.tolist())][:4], np.int32)
    # poison the fresh slots first, as a recycled slot would be
    d.ssm[dev(fresh).long()] = float("nan")
    gdn.gdn_slot_zero(g, d.ssm, d.conv, dev(fresh))
    gdn.gdn_slot_copy(g, d.ssm, d.conv, dev(ckpt), dev(cow))
    outs = [d.call(g, c) for c in range(3)]
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    oracle.slot_zero(o, s64, c64, fresh)
    oracle.slot_copy(o, s64, c64, ckpt, cow)
    refs = run_oracle(o, case, s64, c64, range(3))
    for c in range(3):
        assert rel_err(host(outs[c]), refs[c]) <= OUT_TOL
    assert rel_err(host(d.ssm)[idx], s64[idx]) <= OUT_TOL


def test_64bit_offsets_top_slots():
    """A pool above 2 GiB (1100 Qwen3.5 slots, 2.3 GB): the top slots are
    addressed correctly (byte offsets beyond int32)."""
    torch = _torch()
    shape = synth.QWEN35
    n = 1100
    g, o = layers(shape)
    rs = synth.streams(12)
    top = np.array([1099, 1024], np.int32)
    small = synth.make_pool(shape, 2, np.arange(2), rs)
    ssm = torch.zeros((n, 32, 128, 128), dtype=torch.float32, device="cuda")
    conv = torch.zeros((n, 3, shape.channels), dtype=torch.bfloat16, device="cuda")
    ssm[dev(top).long()] = dev(small.ssm)
    conv[dev(top).long()] = dev(small.conv)
    x, al, be = synth.make_tokens(shape, (2, 1), rs)
    w = synth.make_conv_w(shape, rs)
    out = gdn.gdn_decode_step(g, ssm, conv, dev(top), dev(x), dev(al), dev(be), dev(w))
    torch.cuda.synchronize()
    s64, c64 = shadow(small)
    ref = oracle.decode(o, s64, c64, np.array([0, 1], np.int32), x, al, be, w)
    assert rel_err(host(out), ref) <= OUT_TOL
    assert rel_err(host(ssm[dev(top).long()]), s64) <= OUT_TOL
    assert float(ssm[:1024].abs().sum()) == 0.0 and float(ssm[1025:1099].abs().sum()) == 0.0


def test_max_batch_tiny():
    """B = 65535 (the largest the ABI takes) on the tiny shape, one token,
    every request on its own slot of a 65536-slot pool; all outputs and
    states against the oracle, the one unused slot untouched."""
    torch = _torch()
    B, slots = 65535, 65536
    case = synth.decode_case(synth.TINY, B=B, T=1, num_slots=slots, n_calls=1, seed=13)
    g, o = layers(synth.TINY)
    d = DevCase(case)
    before = bits(d.ssm), bits(d.conv)
    out = d.call(g, 0)
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    ref = run_oracle(o, case, s64, c64, range(1))[0]
    assert rel_err(host(out), ref) <= OUT_TOL
    used = case.indices[0]
    assert rel_err(host(d.ssm)[used], s64[used]) <= STATE_TOL_16
    np.testing.assert_array_equal(host(d.conv)[used], c64[used].astype(np.float32))
    spare = np.setdiff1d(np.arange(slots), used)
    assert spare.size == 1
    np.testing.assert_array_equal(bits(d.ssm)[spare], before[0][spare])


def test_graph_capture_and_two_streams():
    """A decode call with a work counter captured into a graph replays
    bit-identical to eager calls (no counter), three replays with eager work
    between them; and two streams decoding disjoint slots of one pool at once,
    each with its own counter, give what one stream gives one call after the
    other.  The counters end at zero."""
    torch = _torch()
    shape = synth.QWEN35
    B = 64
    case = synth.decode_case(shape, B=2 * B, T=1, num_slots=256, n_calls=3, seed=15,
                             rotate=False)
    g, _ = layers(shape)
    idx = dev(case.indices[0])
    ins = [(dev(case.x[c]), dev(case.alpha[c]), dev(case.beta[c])) for c in range(3)]
    w = dev(case.conv_w)

    # eager reference: one stream, calls in order, no counters
    ref_ssm, ref_conv = dev(case.pool.ssm), dev(case.pool.conv)
    ref_out = [gdn.gdn_decode_step(g, ref_ssm, ref_conv, idx, *ins[c], w) for c in range(3)]
    torch.cuda.synchronize()
    ref_bits = bits(ref_ssm), bits(ref_conv)

    # graph: static input buffers refilled before every replay
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    work = gdn.decode_work()
    xs, als, bes = (t.clone() for t in ins[0])
    out = torch.empty_like(ref_out[0])
    gdn.gdn_decode_step(g, ssm, conv, idx, xs, als, bes, w, out=out, work=work)  # warm-up ...
    torch.cuda.synchronize()
    ssm.copy_(dev(case.pool.ssm)); conv.copy_(dev(case.pool.conv))    # ... undone
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gdn.gdn_decode_step(g, ssm, conv, idx, xs, als, bes, w, out=out, work=work)
    torch.cuda.synchronize()
    for c in range(3):
        xs.copy_(ins[c][0]); als.copy_(ins[c][1]); bes.copy_(ins[c][2])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(out), bits(ref_out[c]))
        assert not bool(work.any())
    np.testing.assert_array_equal(bits(ssm), ref_bits[0])
    np.testing.assert_array_equal(bits(conv), ref_bits[1])

    # two streams, disjoint halves of the batch, launched back to back
    ssm2, conv2 = dev(case.pool.ssm), dev(case.pool.conv)
    works = [gdn.decode_work(), gdn.decode_work()]
    halves = [(slice(0, B), torch.cuda.Stream()), (slice(B, 2 * B), torch.cuda.Stream())]
    parts = [[(idx[h].contiguous(), *(t[h].contiguous() for t in ins[c])) for c in range(3)]
             for h, _ in halves]
    outs = [[None] * 3 for _ in halves]
    torch.cuda.synchronize()
    for c in range(3):
        for k, (h, st) in enumerate(halves):
            with torch.cuda.stream(st):
                outs[k][c] = gdn.gdn_decode_step(g, ssm2, conv2, *parts[k][c], w, work=works[k])
    torch.cuda.synchronize()
    for c in range(3):
        got = torch.cat([outs[0][c], outs[1][c]])
        np.testing.assert_array_equal(bits(got), bits(ref_out[c]))
    np.testing.assert_array_equal(bits(ssm2), ref_bits[0])
    np.testing.assert_array_equal(bits(conv2), ref_bits[1])
    assert not any(bool(x.any()) for x in works)


class _PerThreadStream:
    """hipStreamPerThread: one handle value that names a different stream on
    every host thread."""
    cuda_stream = 2


def test_two_host_threads_on_the_per_thread_stream():
    """Two host threads decode disjoint halves of a batch on
    hipStreamPerThread (the same handle value, a different stream on each
    thread), three calls each, sharing one pool, each thread with its own work
    counter; outputs and pools equal, bit for bit, one stream running the
    calls one after the other."""
    import threading
    torch = _torch()
    shape = synth.QWEN35
    B = 32
    case = synth.decode_case(shape, B=2 * B, T=1, num_slots=128, n_calls=3, seed=19,
                             rotate=False)
    g, _ = layers(shape)
    w = dev(case.conv_w)
    ref_ssm, ref_conv = dev(case.pool.ssm), dev(case.pool.conv)
    idx = dev(case.indices[0])
    ref = [gdn.gdn_decode_step(g, ref_ssm, ref_conv, idx, dev(case.x[c]), dev(case.alpha[c]),
                               dev(case.beta[c]), w) for c in range(3)]
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    works = [gdn.decode_work(), gdn.decode_work()]
    halves = [slice(0, B), slice(B, 2 * B)]
    args = [[(dev(case.indices[0][h]), dev(case.x[c][h]), dev(case.alpha[c][h]),
              dev(case.beta[c][h]),
              torch.empty((B, 1, shape.n_v_heads, shape.d_v), device="cuda"))
             for c in range(3)] for h in halves]
    torch.cuda.synchronize()
    errors = []

    def work(k):
        try:
            for c in range(3):
                ix, x, al, be, out = args[k][c]
                gdn.gdn_decode_step(g, ssm, conv, ix, x, al, be, w, out=out, work=works[k],
                                    stream=_PerThreadStream)
        except Exception as e:  # pragma: no cover - reported below
            errors.append(e)
    threads = [threading.Thread(target=work, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for c in range(3):
        got = torch.cat([args[0][c][4], args[1][c][4]])
        np.testing.assert_array_equal(bits(got), bits(ref[c]))
    np.testing.assert_array_equal(bits(ssm), bits(ref_ssm))
    np.testing.assert_array_equal(bits(conv), bits(ref_conv))
    assert not any(bool(x.any()) for x in works)


@pytest.mark.parametrize("shape", [synth.QWEN35, synth.Shape(2, 4, 64, 64, 3, "channel", "f32")],
                         ids=["qwen35_bf16", "kda_f32"])
def test_conv_bias(shape):
    """Decode with a conv bias (bf16 storage on the Qwen3.5 shape, fp32 on a
    per-channel-gate shape): 4 calls of T=2 against the oracle given the same
    bias bits; windows bit-exact (the bias never enters the stored window)."""
    torch = _torch()
    case = synth.decode_case(shape, B=8, T=2, num_slots=24, n_calls=4, seed=16)
    bias = synth.encode(np.random.default_rng(16).standard_normal(shape.channels)
                        .astype(np.float32) * 0.5, shape.dtype)
    g, o = layers(shape)
    d = DevCase(case)
    b_dev = dev(bias)
    outs = [gdn.gdn_decode_step(g, d.ssm, d.conv, dev(case.indices[c]), dev(case.x[c]),
                                dev(case.alpha[c]), dev(case.beta[c]), d.w, conv_b=b_dev)
            for c in range(4)]
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    no_bias = oracle.decode(o, s64.copy(), c64.copy(), case.indices[0], case.x[0],
                            case.alpha[0], case.beta[0], case.conv_w)
    for c in range(4):
        ref = oracle.decode(o, s64, c64, case.indices[c], case.x[c], case.alpha[c],
                            case.beta[c], case.conv_w, conv_b=bias)
        assert rel_err(host(outs[c]), ref) <= OUT_TOL
        if c == 0:   # the bias changes the result (it is not silently dropped)
            assert rel_err(host(outs[0]), no_bias) > 10 * OUT_TOL
    live = case.pool.live
    assert rel_err(host(d.ssm)[live], s64[live]) <= OUT_TOL
    want = c64[live].astype(np.float32)
    if shape.dtype == "bf16":
        want = synth.f32_to_bf16_bits(want)
    np.testing.assert_array_equal(host(d.conv)[live], want)
