"""The oracle against tests/golden/hand_worked_two_tokens.txt: two decode
tokens of a 2x2 head worked by hand in exact binary fractions, for the scalar
(GDN) and the per-channel (KDA) gate -- in one call, in two calls, as a
two-token prefill (sequential form; the chunked form for the scalar gate),
and through snapshots and a commit.  Every comparison is exact."""
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked_two_tokens.txt")


def _fixture():
    vals = {}
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].split()
        if line:
            vals[line[0]] = np.array([float(v) for v in line[1:]])
    return vals


F = _fixture()


def _layer(gate):
    return oracle.Layer(1, 1, 2, 2, conv_width=2, gate=gate, conv_silu=False, l2norm=False,
                        q_scale=1.0)


def _pool():
    """Slot 0 holds S0 and the window; slot 1 is NaN and must stay so."""
    ssm = np.full((2, 1, 2, 2), np.nan)
    conv = np.full((2, 1, 6), np.nan)
    ssm[0, 0] = F["S0"].reshape(2, 2)
    conv[0, 0] = F["window0"]
    return ssm, conv


def _inputs(gate):
    x = np.stack([F["x1"], F["x2"]])                        # [T=2, C]
    beta = F["beta"].reshape(2, 1)
    alpha = (F["gdn_alpha"].reshape(2, 1) if gate == "scalar"
             else F["kda_alpha"].reshape(2, 1, 2))
    w = np.tile([0.5, 1.0], (6, 1))
    return x, alpha, beta, w


def _expect(gate):
    p = "gdn" if gate == "scalar" else "kda"
    return (F[p + "_S1"].reshape(2, 2), F[p + "_S2"].reshape(2, 2),
            np.stack([F[p + "_o1"], F[p + "_o2"]]))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_one_call_of_two_tokens(gate):
    L, (ssm, conv), (x, al, be, w) = _layer(gate), _pool(), _inputs(gate)
    S1, S2, o = _expect(gate)
    out = oracle.decode(L, ssm, conv, np.array([0], np.int32), x[None], al[None], be[None], w)
    np.testing.assert_array_equal(out[0, :, 0], o)
    np.testing.assert_array_equal(ssm[0, 0], S2)
    np.testing.assert_array_equal(conv[0, 0], F["x2"])
    assert np.isnan(ssm[1]).all() and np.isnan(conv[1]).all()


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_two_calls_of_one_token(gate):
    L, (ssm, conv), (x, al, be, w) = _layer(gate), _pool(), _inputs(gate)
    S1, S2, o = _expect(gate)
    idx = np.array([0], np.int32)
    o1 = oracle.decode(L, ssm, conv, idx, x[None, :1], al[None, :1], be[None, :1], w)
    np.testing.assert_array_equal(ssm[0, 0], S1)
    np.testing.assert_array_equal(conv[0, 0], F["x1"])
    o2 = oracle.decode(L, ssm, conv, idx, x[None, 1:], al[None, 1:], be[None, 1:], w)
    np.testing.assert_array_equal(np.concatenate([o1[0, :, 0], o2[0, :, 0]]), o)
    np.testing.assert_array_equal(ssm[0, 0], S2)


@pytest.mark.parametrize("gate,form", [("scalar", "sequential"), ("channel", "sequential"),
                                       ("scalar", "chunked")])
def test_two_token_prefill(gate, form):
    """The chunked fp64 form (D8) is written for the scalar gate only."""
    L, (ssm, conv), (x, al, be, w) = _layer(gate), _pool(), _inputs(gate)
    S1, S2, o = _expect(gate)
    fn = oracle.prefill if form == "sequential" else oracle.prefill_chunked
    out = fn(L, ssm, conv, np.array([0], np.int32), np.array([0], np.int32),
             np.array([0, 2], np.int32), x, al, be, w)
    np.testing.assert_array_equal(out[:, 0], o)
    np.testing.assert_array_equal(ssm[0, 0], S2)
    np.testing.assert_array_equal(conv[0, 0], F["x2"])


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_snapshots_and_commit(gate):
    L, (ssm, conv), (x, al, be, w) = _layer(gate), _pool(), _inputs(gate)
    S1, S2, o = _expect(gate)
    sp_ssm = np.zeros((1, 2, 1, 2, 2))
    sp_conv = np.zeros((1, 2, 1, 6))
    idx = np.array([0], np.int32)
    out = oracle.decode(L, ssm, conv, idx, x[None], al[None], be[None], w,
                        spec_ssm=sp_ssm, spec_conv=sp_conv)
    np.testing.assert_array_equal(out[0, :, 0], o)
    np.testing.assert_array_equal(sp_ssm[0, 0, 0], S1)
    np.testing.assert_array_equal(sp_ssm[0, 1, 0], S2)
    np.testing.assert_array_equal(sp_conv[0, 0, 0], F["x1"])
    np.testing.assert_array_equal(sp_conv[0, 1, 0], F["x2"])
    np.testing.assert_array_equal(ssm[0, 0], F["S0"].reshape(2, 2))   # working slot untouched
    oracle.spec_commit(L, ssm, conv, idx, sp_ssm, sp_conv, np.array([1], np.int32))
    np.testing.assert_array_equal(ssm[0, 0], S1)
    np.testing.assert_array_equal(conv[0, 0], F["x1"])
    oracle.spec_commit(L, ssm, conv, idx, sp_ssm, sp_conv, np.array([0], np.int32))  # no-op
    np.testing.assert_array_equal(ssm[0, 0], S1)
    oracle.spec_commit(L, ssm, conv, idx, sp_ssm, sp_conv, np.array([2], np.int32))
    np.testing.assert_array_equal(ssm[0, 0], S2)
    np.testing.assert_array_equal(conv[0, 0], F["x2"])
