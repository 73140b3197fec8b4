"""A seeded sweep over random layer shapes, beside the hand-picked ones of the
other GPU tests: key heads 1-3, GQA 1:1 / 2:1 / 4:1, d_k in {16, 32, 64,
128}, d_v any multiple of 16 up to 256, conv widths 1-4, both gates and
activation dtypes, ragged lengths and 1-3 decode tokens per call.  Each
prefill is checked against the oracle's token-by-token recurrence (outputs,
final state, conv windows, untouched slots); each decode against the
oracle's steps (outputs, states).  A decode shape that does not fit one
workgroup must be refused, exactly when the rule stated in include/gdn.h
says so."""
import numpy as np
import pytest

import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import synth
from tests.harness import OUT_TOL, STATE_TOL_16, host, layers, rel_err, shadow
from tests.test_gpu_decode import DevCase, run_oracle
from tests.test_gpu_prefill import check, run_case

pytestmark = pytest.mark.gpu

SEEDS = list(range(12))


def draw_shape(rng) -> synth.Shape:
    hk = int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 4]))
    return synth.Shape(hk, hk * g, int(rng.choice([16, 32, 64, 128])),
                       int(16 * rng.integers(1, 17)), int(rng.integers(1, 5)),
                       str(rng.choice(["scalar", "channel"])), str(rng.choice(["f32", "bf16"])))


def decode_fits(s: synth.Shape) -> bool:
    """The decode's shape rule as include/gdn.h states it: the unit's G d_v
    rows over w <= 8 waves of r in {32, 16, 8} rows (r | d_v, r a multiple of
    4 for d_k >= 64 or of 256 / d_k), 64 w threads covering the 2 d_k + G d_v
    conv channels and the gates plus betas."""
    g = s.n_v_heads // s.n_k_heads
    rows = g * s.d_v
    per_pass = 4 if s.d_k >= 64 else 256 // s.d_k
    gates = g * (s.d_k if s.gate == "channel" else 1)
    for r in (32, 16, 8):
        if r % per_pass or s.d_v % r:
            continue
        w = rows // r
        if 1 <= w <= 8 and 64 * w >= 2 * s.d_k + rows and 64 * w >= gates + g:
            return True
    return False


@pytest.mark.parametrize("seed", SEEDS)
def test_prefill_random_shape(seed):
    rng = np.random.default_rng(1000 + seed)
    shape = draw_shape(rng)
    lens = [int(v) for v in rng.integers(1, 160, 3)]
    r = run_case(shape, lens, seed=2000 + seed)
    print(shape, lens, "out %.2e state %.2e" % check(r))


@pytest.mark.parametrize("seed", SEEDS)
def test_decode_random_shape(seed):
    """Shapes are drawn until one fits; the first that does not (if any) must
    be refused, the one that fits must match the oracle."""
    import torch
    rng = np.random.default_rng(3000 + seed)
    refused = None
    for _ in range(100):
        shape = draw_shape(rng)
        if decode_fits(shape):
            break
        refused = refused or shape
    assert decode_fits(shape)
    B, T = int(rng.integers(1, 6)), int(rng.integers(1, 4))
    if refused is not None:
        rc = synth.decode_case(refused, B=B, T=T, num_slots=2 * B + 2, n_calls=1, seed=seed)
        with pytest.raises(gdn.GdnError):
            DevCase(rc).call(layers(refused)[0], 0)
        print(refused, "refused, as the rule says")
    case = synth.decode_case(shape, B=B, T=T, num_slots=2 * B + 2, n_calls=3, seed=4000 + seed)
    g, o = layers(shape)
    d = DevCase(case, with_work=True)
    outs = [d.call(g, c) for c in range(3)]
    torch.cuda.synchronize()
    assert d.work_is_zero()
    s64, c64 = shadow(case.pool)
    refs = run_oracle(o, case, s64, c64, range(3))
    for c in range(3):
        assert rel_err(host(outs[c]), refs[c]) <= OUT_TOL
    live = case.pool.live
    assert rel_err(host(d.ssm)[live], s64[live]) <= STATE_TOL_16
    # conv windows hold raw inputs: bit-exact
    np.testing.assert_array_equal(host(d.conv)[live],
                                  synth.encode(c64[live].astype(np.float32), shape.dtype))
    print(shape, f"B={B} T={T} ok")
