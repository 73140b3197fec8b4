"""GPU checks of the slot preparation fused into the decode step (zero start,
copy-on-write source), of speculative snapshots kept in pool slots with the
commit by index, and of slot pack / unpack.  Each is compared bit for bit with the separate-kernel path it
replaces (slot zero / copy, then decode; spec-cache draft, then copy commit),
which the other GPU tests hold against the oracle; outputs are also checked
against the oracle directly."""
import numpy as np
import pytest

import oracle
import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import synth
from tests.harness import OUT_TOL, bits, dev, host, layers, rel_err, shadow

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _pools(case):
    return dev(case.pool.ssm), dev(case.pool.conv)


@pytest.mark.parametrize("shape,B,T", [(synth.QWEN35, 16, 1), (synth.QWEN35, 8, 3),
                                       (synth.KDA, 16, 1), (synth.TINY, 16, 2)])
def test_fused_prep_equals_separate_prep_bitwise(shape, B, T):
    """A quarter of the requests start from zeros (their working slots hold
    NaN, as a recycled slot would), a quarter copy-on-write from checkpoint
    slots, the rest continue in place: one decode call with init_slot equals
    slot_zero + slot_copy + decode, bit for bit, and leaves the checkpoints
    untouched."""
    torch = _torch()
    slots = 64
    case = synth.decode_case(shape, B=B, T=T, num_slots=slots, n_calls=1, seed=31, all_live=True,
                             rotate=False)
    g, o = layers(shape)
    idx = case.indices[0]
    q = B // 4
    fresh, cow = idx[:q], idx[q:2 * q]
    ckpt = np.array([s for s in range(slots) if s not in set(idx.tolist())][:q], np.int32)
    init = idx.copy()
    init[:q] = -1
    init[q:2 * q] = ckpt
    x, al, be, w = dev(case.x[0]), dev(case.alpha[0]), dev(case.beta[0]), dev(case.conv_w)
    # separate preparation
    sa, ca = _pools(case)
    sa[dev(fresh).long()] = float("nan")
    gdn.gdn_slot_zero(g, sa, ca, dev(fresh))
    gdn.gdn_slot_copy(g, sa, ca, dev(ckpt), dev(cow))
    oa = gdn.gdn_decode_step(g, sa, ca, dev(idx), x, al, be, w)
    # fused
    sb, cb = _pools(case)
    sb[dev(fresh).long()] = float("nan")
    cb_ck = bits(cb)[ckpt].copy()
    sb_ck = bits(sb)[ckpt].copy()
    ob = gdn.gdn_decode_step(g, sb, cb, dev(idx), x, al, be, w, init_slot=dev(init))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(oa), bits(ob))
    np.testing.assert_array_equal(bits(sa), bits(sb))
    np.testing.assert_array_equal(bits(ca), bits(cb))
    np.testing.assert_array_equal(bits(sb)[ckpt], sb_ck)
    np.testing.assert_array_equal(bits(cb)[ckpt], cb_ck)
    # and the outputs against the oracle
    s64, c64 = shadow(case.pool)
    oracle.slot_zero(o, s64, c64, fresh)
    oracle.slot_copy(o, s64, c64, ckpt, cow)
    ref = oracle.decode(o, s64, c64, idx, case.x[0], case.alpha[0], case.beta[0], case.conv_w)
    assert rel_err(host(ob), ref) <= OUT_TOL


def test_fused_prep_skip_and_spec_draft():
    """A source slot past the pool skips its row (no output, no write); a
    speculative draft started copy-on-write writes the same snapshots as a
    copy followed by the draft, and leaves both slots alone."""
    torch = _torch()
    shape, B, T, slots = synth.QWEN35, 8, 4, 32
    case = synth.decode_case(shape, B=B, T=T, num_slots=slots, n_calls=1, seed=32, all_live=True,
                             rotate=False)
    g, _ = layers(shape)
    idx = case.indices[0]
    ckpt = np.array([s for s in range(slots) if s not in set(idx.tolist())][:B], np.int32)
    x, al, be, w = dev(case.x[0]), dev(case.alpha[0]), dev(case.beta[0]), dev(case.conv_w)
    # skip: init past the pool for request 0
    s0, c0 = _pools(case)
    before = bits(s0), bits(c0)
    init = idx.copy()
    init[0] = slots + 5
    out = torch.full((B, T, shape.n_v_heads, shape.d_v), float("nan"), device="cuda")
    gdn.gdn_decode_step(g, s0, c0, dev(idx), x, al, be, w, out=out, init_slot=dev(init))
    torch.cuda.synchronize()
    assert np.isnan(host(out)[0]).all() and not np.isnan(host(out)[1:]).any()
    np.testing.assert_array_equal(bits(s0)[idx[0]], before[0][idx[0]])
    np.testing.assert_array_equal(bits(c0)[idx[0]], before[1][idx[0]])
    # spec draft from copy-on-write sources vs copy then draft
    sa, ca = _pools(case)
    sp_a = torch.zeros((B, T) + tuple(sa.shape[1:]), device="cuda")
    spc_a = torch.zeros((B, T) + tuple(ca.shape[1:]), dtype=ca.dtype, device="cuda")
    gdn.gdn_slot_copy(g, sa, ca, dev(ckpt), dev(idx))
    oa = gdn.gdn_decode_step(g, sa, ca, dev(idx), x, al, be, w, spec_ssm=sp_a, spec_conv=spc_a)
    sb, cb = _pools(case)
    before_b = bits(sb), bits(cb)
    sp_b, spc_b = torch.zeros_like(sp_a), torch.zeros_like(spc_a)
    ob = gdn.gdn_decode_step(g, sb, cb, dev(idx), x, al, be, w, spec_ssm=sp_b, spec_conv=spc_b,
                             init_slot=dev(ckpt))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(oa), bits(ob))
    np.testing.assert_array_equal(bits(sp_a), bits(sp_b))
    np.testing.assert_array_equal(bits(spc_a), bits(spc_b))
    np.testing.assert_array_equal(bits(sb), before_b[0])      # the draft writes no pool slot
    np.testing.assert_array_equal(bits(cb), before_b[1])


@pytest.mark.parametrize("shape,B", [(synth.QWEN35, 64), (synth.TINY, 64)])
def test_pool_snapshots_and_commit_by_index(shape, B):
    """7 draft tokens with snapshots into 7B distinct pool slots: each equals
    the spec-cache snapshot bit for bit and nothing else in the pool changes;
    the commit by index then names the accepted snapshot's slot, whose state
    equals the copy commit's working slot; L = 0 and a dropped snapshot (its
    slot outside the pool) leave the index alone."""
    torch = _torch()
    T, slots = 7, 1024
    case = synth.decode_case(shape, B=B, T=T, num_slots=slots, n_calls=1, seed=33)
    acc = synth.accepted_lengths(B, T, seed=33)
    g, o = layers(shape)
    idx = case.indices[0]
    free = np.setdiff1d(np.arange(slots, dtype=np.int32), idx)
    tab = np.random.default_rng(33).permutation(free)[:B * T].reshape(B, T).astype(np.int32)
    drop_b = int(np.nonzero(acc > 0)[0][0])               # this request's accepted snapshot
    tab_dev = tab.copy()
    tab_dev[drop_b, acc[drop_b] - 1] = slots + 1          # is dropped
    x, al, be, w = dev(case.x[0]), dev(case.alpha[0]), dev(case.beta[0]), dev(case.conv_w)
    # reference: spec cache, then copy commit
    sa, ca = _pools(case)
    sp = torch.zeros((B, T) + tuple(sa.shape[1:]), device="cuda")
    spc = torch.zeros((B, T) + tuple(ca.shape[1:]), dtype=ca.dtype, device="cuda")
    oa = gdn.gdn_decode_step(g, sa, ca, dev(idx), x, al, be, w, spec_ssm=sp, spec_conv=spc)
    # snapshots in pool slots
    sb, cb = _pools(case)
    before = bits(sb), bits(cb)
    ob = gdn.gdn_decode_step(g, sb, cb, dev(idx), x, al, be, w, spec_slots=dev(tab_dev))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(oa), bits(ob))
    got_s, got_c = bits(sb), bits(cb)
    want_s, want_c = bits(sp), bits(spc)
    written = np.zeros(slots, bool)
    for b in range(B):
        for t in range(T):
            sl = tab_dev[b, t]
            if sl >= slots:
                continue
            written[sl] = True
            np.testing.assert_array_equal(got_s[sl], want_s[b, t])
            np.testing.assert_array_equal(got_c[sl], want_c[b, t])
    np.testing.assert_array_equal(got_s[~written], before[0][~written])
    np.testing.assert_array_equal(got_c[~written], before[1][~written])
    # commit by index
    ix = dev(idx)
    rel = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    gdn.gdn_spec_commit_index(sb, cb, dev(tab_dev), dev(acc), ix, released=rel)
    gdn.gdn_spec_decode_commit(g, sa, ca, dev(idx), sp, spc, dev(acc))
    torch.cuda.synchronize()
    new_idx, rel_h = host(ix), host(rel)
    for b in range(B):
        L = acc[b]
        if L == 0 or b == drop_b:
            assert new_idx[b] == idx[b] and rel_h[b] == -1
        else:
            assert new_idx[b] == tab[b, L - 1] and rel_h[b] == idx[b]
            np.testing.assert_array_equal(bits(sb)[new_idx[b]], bits(sa)[idx[b]])
            np.testing.assert_array_equal(bits(cb)[new_idx[b]], bits(ca)[idx[b]])
    # draft outputs against the oracle
    s64, c64 = shadow(case.pool)
    ref = oracle.decode(o, s64, c64, idx, case.x[0], case.alpha[0], case.beta[0], case.conv_w,
                        spec_ssm=np.zeros((B, T) + s64.shape[1:]),
                        spec_conv=np.zeros((B, T) + c64.shape[1:]))
    assert rel_err(host(ob), ref) <= OUT_TOL


@pytest.mark.parametrize("shape", [synth.QWEN35, synth.Shape(2, 2, 32, 32, 4, "channel", "f32")])
def test_slot_pack_unpack_bitwise(shape):
    """Packed items are the slots' own bytes (ssm then conv); unpacking them
    into other slots reproduces the slots bit for bit; an index outside the
    pool leaves its buffer item (pack) or nothing (unpack) untouched."""
    torch = _torch()
    slots, n = 48, 6
    case = synth.decode_case(shape, B=n, T=1, num_slots=slots, n_calls=1, seed=34, all_live=True,
                             rotate=False)
    g, _ = layers(shape)
    ssm, conv = _pools(case)
    src = np.array([3, 17, 40, 0, 47, 22], np.int32)
    src_bad = src.copy()
    src_bad[2] = slots + 3
    item = gdn.gdn_slot_bytes(g)
    assert item == ssm[0].numel() * 4 + conv[0].numel() * conv.element_size()
    buf = torch.full((n * item,), 0xA5, dtype=torch.uint8, device="cuda")
    gdn.gdn_slot_pack(g, ssm, conv, dev(src_bad), buffer=buf)
    torch.cuda.synchronize()
    b = host(buf).reshape(n, item)
    s_bytes = host(ssm).view(np.uint8).reshape(slots, -1)
    c_bytes = host(conv).view(np.uint8).reshape(slots, -1)
    for i in range(n):
        if i == 2:
            assert (b[i] == 0xA5).all()
        else:
            np.testing.assert_array_equal(b[i], np.concatenate([s_bytes[src[i]], c_bytes[src[i]]]))
    # full pack, then unpack into fresh slots (one target outside the pool)
    buf = gdn.gdn_slot_pack(g, ssm, conv, dev(src))
    before = bits(ssm), bits(conv)
    dst = np.array([5, 6, 7, 8, 9, slots + 1], np.int32)
    gdn.gdn_slot_unpack(g, ssm, conv, buf, dev(dst))
    torch.cuda.synchronize()
    after = bits(ssm), bits(conv)
    for i in range(5):
        np.testing.assert_array_equal(after[0][dst[i]], before[0][src[i]])
        np.testing.assert_array_equal(after[1][dst[i]], before[1][src[i]])
    others = np.setdiff1d(np.arange(slots), dst[:5])
    np.testing.assert_array_equal(after[0][others], before[0][others])
    np.testing.assert_array_equal(after[1][others], before[1][others])
