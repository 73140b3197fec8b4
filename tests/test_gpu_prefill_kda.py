"""GPU parity of the chunked prefill with the per-channel (KDA) decay against
the fp64 token-by-token recurrence of the oracle, on the same seeded inputs.

Same bar as the scalar-decay prefill: outputs max|do|/max|o| <= 2e-3, final
state max-normalised error <= 2e-3, destination conv window bit-exact, every
other slot bit-identical."""
import numpy as np
import pytest

import oracle
import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import synth
from tests.harness import OUT_TOL, bits, dev, host, layers, rel_err, shadow
from tests.test_gpu_prefill import STATE_TOL, check, run_case

pytestmark = pytest.mark.gpu

SMALL = synth.Shape(2, 2, 32, 32, 4, "channel", "f32")


def _torch():
    import torch
    return torch


def test_kda_ragged_lengths_small():
    """Lengths on both sides of the 16-token block and 64-token chunk edges;
    zero and copy-on-write starts; fp32 inputs, d_k = d_v = 32."""
    r = run_case(SMALL, [1, 15, 16, 17, 63, 64, 65, 130, 200], seed=21)
    print("kda ragged: out %.2e state %.2e" % check(r))


def test_kda_bf16_gqa_partial_columns():
    """bf16 inputs, two value heads per key head, d_k = 64, d_v = 48 (one
    idle consumer wave)."""
    shape = synth.Shape(2, 4, 64, 48, 4, "channel", "bf16")
    r = run_case(shape, [37, 128, 99], seed=22)
    print("kda gqa: out %.2e state %.2e" % check(r))


@pytest.mark.parametrize("dv", [16, 80, 128])
def test_kda_value_widths(dv):
    shape = synth.Shape(2, 2, 128, dv, 4, "channel", "bf16")
    r = run_case(shape, [150, 64, 3], seed=23 + dv)
    print("kda dv=%d: out %.2e state %.2e" % ((dv,) + check(r)))


def test_kda_extreme_decays():
    """Decays of exactly 0, of 1e-30 and of exactly 1 mixed into the gates:
    the block-relative products stay in range where e^{-g} would not."""
    torch = _torch()
    shape = synth.Shape(2, 2, 64, 32, 4, "channel", "f32")
    case = synth.prefill_case(shape, [200, 77], 4, seed=24)
    rng = np.random.default_rng(24)
    u = rng.random(case.alpha.shape)
    case.alpha[u < 0.05] = 0.0
    case.alpha[(u >= 0.05) & (u < 0.10)] = 1e-30
    case.alpha[u > 0.9] = 1.0
    g, o = layers(shape)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    out = gdn.gdn_prefill_chunked(g, ssm, conv, dev(case.dst), dev(case.init_slot),
                                  dev(case.cu_seqlens), 200, dev(case.x), dev(case.alpha),
                                  dev(case.beta), dev(case.conv_w))
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    ref = oracle.prefill(o, s64, c64, case.dst, case.init_slot, case.cu_seqlens, case.x,
                         case.alpha, case.beta, case.conv_w)
    eo, es = rel_err(host(out), ref), rel_err(host(ssm)[case.dst], s64[case.dst])
    print("kda extreme decays: out %.2e state %.2e" % (eo, es))
    assert eo <= OUT_TOL and es <= STATE_TOL


def test_kda_no_silu_no_norm_with_conv_bias():
    torch = _torch()
    shape = synth.Shape(1, 1, 32, 32, 4, "channel", "f32")
    case = synth.prefill_case(shape, [96, 40], 4, seed=25)
    case.x[:] *= 0.05
    bias = (np.random.default_rng(25).standard_normal(shape.channels) * 0.05).astype(np.float32)
    g, o = layers(shape, conv_silu=False, l2norm=False)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    out = gdn.gdn_prefill_chunked(g, ssm, conv, dev(case.dst), dev(case.init_slot),
                                  dev(case.cu_seqlens), 96, dev(case.x), dev(case.alpha),
                                  dev(case.beta), dev(case.conv_w), conv_b=dev(bias))
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    ref = oracle.prefill(o, s64, c64, case.dst, case.init_slot, case.cu_seqlens, case.x,
                         case.alpha, case.beta, case.conv_w, conv_b=bias)
    assert rel_err(host(out), ref) <= OUT_TOL
    assert rel_err(host(ssm)[case.dst], s64[case.dst]) <= STATE_TOL


def test_kda_empty_skipped_and_in_place():
    torch = _torch()
    shape = synth.Shape(2, 2, 32, 32, 4, "channel", "bf16")
    case = synth.prefill_case(shape, [0, 70, 0, 50, 40], 12, seed=26)
    g, o = layers(shape)
    init = case.init_slot.copy()
    dst = case.dst.copy()
    init[2] = case.init_slot[1]
    live = case.init_slot[3]
    case.pool.ssm[dst[3]] = case.pool.ssm[live]
    case.pool.conv[dst[3]] = case.pool.conv[live]
    init[3] = dst[3]
    dst[1] = -1
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    before = bits(ssm), bits(conv)
    total = int(case.cu_seqlens[-1])
    out = torch.full((total, shape.n_v_heads, shape.d_v), float("nan"), device="cuda")
    gdn.gdn_prefill_chunked(g, ssm, conv, dev(dst), dev(init), dev(case.cu_seqlens), 70,
                            dev(case.x), dev(case.alpha), dev(case.beta), dev(case.conv_w),
                            out=out)
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    ref = oracle.prefill(o, s64, c64, dst, init, case.cu_seqlens, case.x, case.alpha,
                         case.beta, case.conv_w)
    o_h = host(out)
    cu = case.cu_seqlens
    assert np.isnan(o_h[cu[1]:cu[2]]).all()
    assert rel_err(o_h[cu[3]:], ref[cu[3]:]) <= OUT_TOL
    written = dst[dst >= 0]
    assert rel_err(host(ssm)[written], s64[written]) <= STATE_TOL
    for s in (0, 2):
        np.testing.assert_array_equal(host(ssm)[dst[s]], s64[dst[s]].astype(np.float32))
    np.testing.assert_array_equal(oracle.as_f64(host(conv)[written]), c64[written])
    untouched = np.setdiff1d(np.arange(12), written)
    np.testing.assert_array_equal(bits(ssm)[untouched], before[0][untouched])
    np.testing.assert_array_equal(bits(conv)[untouched], before[1][untouched])


def test_kda_4x8192_zero_and_cow():
    """The KDA layer shape (32 heads, d = 128, 12288 channels) over 4 x 8192
    tokens, bf16 inputs; every output and final state element compared."""
    r = run_case(synth.KDA, [8192] * 4, num_slots=64, seed=27)
    print("kda 4x8192: out %.2e state %.2e" % check(r))


def test_kda_split_prefill_equals_one_shot_bitwise():
    torch = _torch()
    shape = synth.KDA
    case = synth.prefill_case(shape, [4096], 8, seed=28)
    g, _ = layers(shape)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    x, al, be, w = dev(case.x), dev(case.alpha), dev(case.beta), dev(case.conv_w)
    one, mid, cow, two = 4, 5, 6, 7
    i32 = lambda *v: dev(np.asarray(v, np.int32))
    o_full = gdn.gdn_prefill_chunked(g, ssm, conv, i32(one), i32(-1), i32(0, 4096), 4096, x, al,
                                     be, w)
    o_a = gdn.gdn_prefill_chunked(g, ssm, conv, i32(mid), i32(-1), i32(0, 2048), 2048,
                                  x[:2048], al[:2048], be[:2048], w)
    gdn.gdn_slot_copy(g, ssm, conv, i32(mid), i32(cow))
    o_b = gdn.gdn_prefill_chunked(g, ssm, conv, i32(two), i32(cow), i32(0, 2048), 2048,
                                  x[2048:].contiguous(), al[2048:].contiguous(),
                                  be[2048:].contiguous(), w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o_full)[:2048], bits(o_a))
    np.testing.assert_array_equal(bits(o_full)[2048:], bits(o_b))
    np.testing.assert_array_equal(bits(ssm)[one], bits(ssm)[two])
    np.testing.assert_array_equal(bits(conv)[one], bits(conv)[two])
