"""GPU checks of the GDN_DEBUG mode: with the variable set, every entry point
that takes device index arrays copies them to the host first and refuses a
call whose rows would collide (two rows writing one slot, a row reading a
slot another row writes, snapshot / checkpoint slots that repeat or hit a
row's slots) or whose cu_seqlens break their contract, with
GDN_ERR_PRECONDITION and nothing enqueued; valid calls run unchanged."""
import os

import numpy as np
import pytest

import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import synth
from tests.harness import bits, dev, layers

pytestmark = pytest.mark.gpu

DEC = synth.Shape(2, 4, 32, 32, 4, "scalar", "bf16")


def _torch():
    import torch
    return torch


@pytest.fixture
def debug_env():
    old = os.environ.get("GDN_DEBUG")
    os.environ["GDN_DEBUG"] = "1"
    yield
    if old is None:
        os.environ.pop("GDN_DEBUG", None)
    else:
        os.environ["GDN_DEBUG"] = old


def _refused(fn):
    with pytest.raises(gdn.GdnError) as e:
        fn()
    assert e.value.status == gdn.GDN_ERR_PRECONDITION


def _i32(*v):
    return dev(np.asarray(v, np.int32))


def test_decode_rows_and_snapshots(debug_env):
    torch = _torch()
    case = synth.decode_case(DEC, B=4, T=2, num_slots=16, n_calls=1, seed=31, all_live=True)
    g, _ = layers(DEC)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    x, al, be, w = dev(case.x[0]), dev(case.alpha[0]), dev(case.beta[0]), dev(case.conv_w)
    before = bits(ssm), bits(conv)
    call = lambda idx, **kw: gdn.gdn_decode_step(g, ssm, conv, idx, x, al, be, w, **kw)
    _refused(lambda: call(_i32(1, 2, 1, 3)))                        # two rows write slot 1
    _refused(lambda: call(_i32(1, 2, 3, 4), init_slot=_i32(-1, 5, 1, -1)))  # reads slot 1
    tab = np.array([[5, 6], [7, 8], [9, 10], [11, 12]], np.int32)
    bad = tab.copy(); bad[2, 1] = 6                                  # a snapshot slot twice
    _refused(lambda: call(_i32(1, 2, 3, 4), spec_slots=dev(bad)))
    bad = tab.copy(); bad[0, 0] = 3                                  # a working slot
    _refused(lambda: call(_i32(1, 2, 3, 4), spec_slots=dev(bad)))
    bad = tab.copy(); bad[1, 1] = 13                                 # a copy-on-write source
    _refused(lambda: call(_i32(1, 2, 3, 4), init_slot=_i32(1, 13, 3, 4), spec_slots=dev(bad)))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(ssm), before[0])              # nothing was enqueued
    np.testing.assert_array_equal(bits(conv), before[1])
    # skipped rows may repeat; valid calls match the unchecked ones bit for bit
    o1 = call(_i32(1, -1, 3, -1))
    s1 = bits(ssm)
    ssm.copy_(dev(case.pool.ssm)); conv.copy_(dev(case.pool.conv))
    del os.environ["GDN_DEBUG"]
    o2 = call(_i32(1, -1, 3, -1))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o1)[[0, 2]], bits(o2)[[0, 2]])
    np.testing.assert_array_equal(s1, bits(ssm))
    # without GDN_DEBUG nothing is checked: the colliding call is enqueued
    call(_i32(1, 2, 1, 3))
    torch.cuda.synchronize()


def test_commit_copy_and_unpack(debug_env):
    torch = _torch()
    case = synth.decode_case(DEC, B=4, T=2, num_slots=16, n_calls=1, seed=32, all_live=True)
    g, _ = layers(DEC)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    sp_ssm = torch.zeros((4, 2) + tuple(ssm.shape[1:]), device="cuda")
    sp_conv = torch.zeros((4, 2) + tuple(conv.shape[1:]), dtype=conv.dtype, device="cuda")
    acc = _i32(1, 2, 0, 1)
    _refused(lambda: gdn.gdn_spec_decode_commit(g, ssm, conv, _i32(1, 2, 3, 2), sp_ssm, sp_conv,
                                                acc))
    _refused(lambda: gdn.gdn_slot_copy(g, ssm, conv, _i32(1, 2), _i32(3, 3)))   # dst twice
    _refused(lambda: gdn.gdn_slot_copy(g, ssm, conv, _i32(1, 2), _i32(2, 4)))   # dst is a src
    buf = gdn.gdn_slot_pack(g, ssm, conv, _i32(1, 2))
    _refused(lambda: gdn.gdn_slot_unpack(g, ssm, conv, buf, _i32(5, 5)))
    # valid ones pass; a row whose source is outside the pool is skipped
    gdn.gdn_spec_decode_commit(g, ssm, conv, _i32(1, 2, 3, 4), sp_ssm, sp_conv, acc)
    gdn.gdn_slot_copy(g, ssm, conv, _i32(1, -1), _i32(5, 1))
    gdn.gdn_slot_unpack(g, ssm, conv, buf, _i32(6, 7))
    torch.cuda.synchronize()


def test_prefill_sequences_and_checkpoints(debug_env):
    torch = _torch()
    shape = synth.Shape(2, 2, 32, 32, 4, "scalar", "bf16")
    case = synth.prefill_case(shape, [200, 70], 16, seed=33)
    g, _ = layers(shape)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    x, al, be, w = dev(case.x), dev(case.alpha), dev(case.beta), dev(case.conv_w)
    cu = case.cu_seqlens
    call = lambda dst, init, cus, mx=200, **kw: gdn.gdn_prefill_chunked(
        g, ssm, conv, dst, init, cus, mx, x, al, be, w, **kw)
    free = [s for s in range(16) if s not in set(case.dst.tolist()) |
            set(case.init_slot[case.init_slot >= 0].tolist())]
    d0, d1 = int(case.dst[0]), int(case.dst[1])
    _refused(lambda: call(_i32(d0, d0), _i32(-1, -1), dev(cu)))              # one slot twice
    _refused(lambda: call(_i32(d0, d1), _i32(-1, d0), dev(cu)))              # reads d0
    _refused(lambda: call(_i32(d0, d1), _i32(-1, -1), _i32(0, 200, 260)))    # ends before total
    _refused(lambda: call(_i32(d0, d1), _i32(-1, -1), _i32(0, 271, 270), mx=300))  # decreasing
    _refused(lambda: call(_i32(d0, d1), _i32(-1, -1), dev(cu), mx=150))      # longer than max
    tab = np.array([[free[0], -1], [free[1], free[2]]], np.int32)
    bad = tab.copy(); bad[0, 0] = d1                                         # a destination
    _refused(lambda: call(_i32(d0, d1), _i32(-1, -1), dev(cu), ckpt_slots=dev(bad), ckpt_every=64))
    bad = tab.copy(); bad[0, 1] = free[0]                                    # a checkpoint twice
    _refused(lambda: call(_i32(d0, d1), _i32(-1, -1), dev(cu), ckpt_slots=dev(bad), ckpt_every=64))
    # sequence 1 (70 tokens) has one checkpoint at 64: its second entry is
    # never written, so it may repeat one of sequence 0's
    ok = tab.copy(); ok[1, 1] = free[0]
    call(_i32(d0, d1), _i32(-1, -1), dev(cu), ckpt_slots=dev(ok), ckpt_every=64)
    torch.cuda.synchronize()
