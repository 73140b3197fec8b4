"""Pins of the fp64 oracle against what the definition and the mathematics fix.

The pages print no worked example, so every pin is definitional: closed forms,
special cases that reduce to a library routine (scipy's FIR filter, numpy's
norm / QR / matmul), exact rational arithmetic on a tiny case, brute force of
the literal O(d^3) matrix form, and algebraic identities between the oracle's
own independent forms (sequential vs chunked).  Shapes use d_k != d_v where a
transposed operand could otherwise hide.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy.signal import lfilter
from scipy.special import expit

import oracle
from oracle import Layer


def pools(L: Layer, slots: int):
    ssm = np.zeros((slots, L.n_v_heads, L.d_v, L.d_k))
    conv = np.zeros((slots, L.conv_width - 1, L.channels))
    return ssm, conv


def ident_taps(L: Layer):
    w = np.zeros((L.channels, L.conv_width))
    w[:, -1] = 1.0
    return w


def chans(L: Layer):
    """(q, k, v) channel index arrays per key head / value head."""
    q = [np.arange(kh * L.d_k, (kh + 1) * L.d_k) for kh in range(L.n_k_heads)]
    k = [L.n_k_heads * L.d_k + qq for qq in q]
    v = [2 * L.n_k_heads * L.d_k + np.arange(h * L.d_v, (h + 1) * L.d_v)
         for h in range(L.n_v_heads)]
    return q, k, v


def relerr(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# --------------------------------------------------------------------------
# D1 / D2: conv and head prep, against scipy's FIR filter and numpy's norm

@pytest.mark.parametrize("silu,l2", [(False, False), (True, False), (True, True)])
def test_conv_and_prep_match_fir_filter(silu, l2):
    L = Layer(2, 4, 8, 8, conv_width=4, conv_silu=silu, l2norm=l2, q_scale=0.37, eps=1e-6)
    C, T = L.channels, 20
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, T, C))
    w = rng.standard_normal((C, 4))
    bias = rng.standard_normal(C)
    ssm, conv = pools(L, 2)
    ssm[1] = np.eye(8)                        # S0 = I, beta = 0, alpha = 1 -> o_t = q^_t
    conv[1] = rng.standard_normal((3, C))
    win0 = conv[1].copy()
    out = oracle.decode(L, ssm, conv, [1], x, np.ones((1, T, 4)), np.zeros((1, T, 4)), w, bias)
    q, _, _ = chans(L)
    for h in range(4):
        kh = h // 2                           # GQA: value head h reads key head h // G
        y = np.stack([lfilter(w[c, ::-1], [1.0], np.concatenate([win0[:, c], x[0, :, c]]))[3:]
                      + bias[c] for c in q[kh]], axis=1)
        a = y * expit(y) if silu else y
        if l2:
            a = a / np.sqrt(np.sum(a * a, axis=1, keepdims=True) + 1e-6)
        assert relerr(out[0, :, h, :], a * 0.37) < 1e-13
    np.testing.assert_array_equal(ssm[1], np.broadcast_to(np.eye(8), (4, 8, 8)))


def test_conv_taps_identity_and_delay():
    """P11: taps [0,0,0,1] pass x through; [1,0,0,0] delay it by three tokens."""
    L = Layer(1, 1, 4, 4, conv_width=4, conv_silu=False, l2norm=False, q_scale=1.0)
    C, T = L.channels, 9
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, T, C))
    for taps, shift in (([0, 0, 0, 1], 0), ([1, 0, 0, 0], 3)):
        ssm, conv = pools(L, 1)
        ssm[0, 0] = np.eye(4)
        conv[0] = rng.standard_normal((3, C))
        hist = np.concatenate([conv[0], x[0]], axis=0)  # z = (window, x_0..)
        w = np.tile(np.array(taps, float), (C, 1))
        out = oracle.decode(L, ssm, conv, [0], x, np.ones((1, T, 1)), np.zeros((1, T, 1)), w)
        expect = hist[3 - shift:3 - shift + T, 0:4]
        np.testing.assert_array_equal(out[0, :, 0, :], expect)
        np.testing.assert_array_equal(conv[0], hist[-3:])   # window = last 3 raw inputs


# --------------------------------------------------------------------------
# D3 / D4: the state step

def test_beta0_alpha1_state_unchanged():
    """P1: beta = 0 and alpha = 1 leave S bit-for-bit unchanged."""
    L = Layer(2, 4, 8, 6)
    rng = np.random.default_rng(3)
    ssm, conv = pools(L, 3)
    ssm[:] = rng.standard_normal(ssm.shape)
    conv[:] = rng.standard_normal(conv.shape)
    before = ssm.copy()
    T = 4
    oracle.decode(L, ssm, conv, [2, 0], rng.standard_normal((2, T, L.channels)),
                  np.ones((2, T, 4)), np.zeros((2, T, 4)), rng.standard_normal((L.channels, 4)))
    np.testing.assert_array_equal(ssm, before)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_delta_rule_writes_v_along_k(gate):
    """P2: with beta = 1 and a unit k^, S_t k^_t = v_t, whatever alpha is."""
    L = Layer(1, 2, 8, 6, conv_silu=False, l2norm=True, eps=0.0, gate=gate)
    rng = np.random.default_rng(4)
    ssm, conv = pools(L, 1)
    ssm[0] = rng.standard_normal(ssm.shape[1:])
    w = ident_taps(L)
    _, k, v = chans(L)
    for t in range(6):
        x = rng.standard_normal((1, 1, L.channels))
        ash = (1, 1, 2, 8) if gate == "channel" else (1, 1, 2)
        alpha = rng.uniform(0.2, 1.0, ash)
        oracle.decode(L, ssm, conv, [0], x, alpha, np.ones((1, 1, 2)), w)
        kh = x[0, 0, k[0]] / np.linalg.norm(x[0, 0, k[0]])
        for h in range(2):
            np.testing.assert_allclose(ssm[0, h] @ kh, x[0, 0, v[h]], rtol=0, atol=1e-13)


def test_orthonormal_keys_closed_form():
    """P3: alpha = beta = 1 and orthonormal k^_1..k^_n give
    S_n = S0 (I - sum k k^T) + sum v k^T."""
    L = Layer(1, 1, 8, 5, conv_silu=False, l2norm=True, eps=0.0)
    rng = np.random.default_rng(5)
    n = 6
    Qm, _ = np.linalg.qr(rng.standard_normal((8, 8)))
    K = Qm[:, :n].T                                  # n orthonormal rows
    V = rng.standard_normal((n, 5))
    ssm, conv = pools(L, 1)
    ssm[0, 0] = rng.standard_normal((5, 8))
    S0 = ssm[0, 0].copy()
    _, k, v = chans(L)
    x = rng.standard_normal((1, n, L.channels))
    x[0, :, k[0]] = K.T
    x[0, :, v[0]] = V.T
    oracle.decode(L, ssm, conv, [0], x, np.ones((1, n, 1)), np.ones((1, n, 1)), ident_taps(L))
    expect = S0 @ (np.eye(8) - K.T @ K) + V.T @ K
    assert relerr(ssm[0, 0], expect) < 1e-12
    np.testing.assert_allclose(ssm[0, 0] @ K.T, V.T, atol=1e-12)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_beta0_pure_decay(gate):
    """P4: beta = 0 gives S_t = (prod alpha) S0 (GDN) or S0 diag(prod alpha_j)
    (KDA, decay along key columns), and o_t = S_t q^_t."""
    L = Layer(1, 2, 6, 4, conv_silu=False, l2norm=False, q_scale=1.0, gate=gate)
    rng = np.random.default_rng(6)
    T = 7
    ssm, conv = pools(L, 2)
    ssm[1] = rng.standard_normal(ssm.shape[1:])
    S0 = ssm[1].copy()
    ash = (1, T, 2, 6) if gate == "channel" else (1, T, 2)
    alpha = rng.uniform(0.3, 1.0, ash)
    x = rng.standard_normal((1, T, L.channels))
    out = oracle.decode(L, ssm, conv, [1], x, alpha, np.zeros((1, T, 2)), ident_taps(L))
    q, _, _ = chans(L)
    for h in range(2):
        S = S0[h].copy()
        for t in range(T):
            if gate == "channel":
                S = S * alpha[0, t, h][None, :]
            else:
                S = S * alpha[0, t, h]
            np.testing.assert_allclose(out[0, t, h], S @ x[0, t, q[0]], rtol=1e-14, atol=1e-15)
        prod = np.prod(alpha[0, :, h], axis=0)
        expect = S0[h] * (prod[None, :] if gate == "channel" else prod)
        assert relerr(ssm[1, h], expect) < 1e-14


def test_scalar_recurrence_d1():
    """P5: d_k = d_v = 1 reduces to s_t = alpha (1 - beta) s + beta v sign(k),
    o_t = s_t sign(q)."""
    L = Layer(1, 1, 1, 1, conv_silu=False, l2norm=True, eps=0.0)
    rng = np.random.default_rng(7)
    T = 50
    x = rng.standard_normal((1, T, 3))
    al = rng.uniform(0.1, 1.0, (1, T, 1))
    be = rng.uniform(0.0, 1.0, (1, T, 1))
    ssm, conv = pools(L, 1)
    ssm[0, 0, 0, 0] = s = 0.7
    out = oracle.decode(L, ssm, conv, [0], x, al, be, ident_taps(L))
    for t in range(T):
        s = al[0, t, 0] * (1 - be[0, t, 0]) * s + be[0, t, 0] * x[0, t, 2] * np.sign(x[0, t, 1])
        assert out[0, t, 0, 0] == pytest.approx(s * np.sign(x[0, t, 0]), rel=1e-13, abs=1e-15)
    assert ssm[0, 0, 0, 0] == pytest.approx(s, rel=1e-13)


def test_exact_rational_worked_example():
    """A tiny case in exact rational arithmetic: dyadic inputs, no SiLU, no
    norm, identity taps; the fp64 oracle must reproduce it exactly."""
    L = Layer(1, 1, 2, 2, conv_silu=False, l2norm=False, q_scale=1.0)
    S = [[Fraction(1, 2), Fraction(-1, 4)], [Fraction(3, 4), Fraction(1, 8)]]
    toks = [  # (q, k, v, alpha, beta)
        ([1, Fraction(1, 2)], [Fraction(1, 2), Fraction(-1, 2)], [2, -1], Fraction(1, 2),
         Fraction(1, 4)),
        ([Fraction(-1, 4), 1], [1, Fraction(1, 4)], [Fraction(1, 2), Fraction(3, 2)],
         Fraction(3, 4), Fraction(1, 2)),
        ([Fraction(1, 8), Fraction(1, 8)], [Fraction(-3, 4), 1], [1, 1], 1, Fraction(1, 8)),
    ]
    ssm, conv = pools(L, 1)
    ssm[0, 0] = np.array(S, dtype=float)
    T = len(toks)
    x = np.zeros((1, T, 6))
    al = np.zeros((1, T, 1))
    be = np.zeros((1, T, 1))
    exp_o = []
    for t, (q, k, v, a, b) in enumerate(toks):
        x[0, t] = [float(z) for z in (*q, *k, *v)]
        al[0, t, 0], be[0, t, 0] = float(a), float(b)
        # literal definition: S <- a S (I - b k k^T) + b v k^T ; o = S q
        M = [[(1 if i == j else 0) - b * k[i] * k[j] for j in range(2)] for i in range(2)]
        S = [[a * sum(S[r][m] * M[m][c] for m in range(2)) + b * v[r] * k[c] for c in range(2)]
             for r in range(2)]
        exp_o.append([sum(S[r][c] * q[c] for c in range(2)) for r in range(2)])
    out = oracle.decode(L, ssm, conv, [0], x, al, be, ident_taps(L))
    for t in range(T):
        assert [Fraction(z) for z in out[0, t, 0]] == exp_o[t]
    assert [[Fraction(z) for z in row] for row in ssm[0, 0]] == S


def _brute_force(L, S0, win0, x, alpha, beta, w, bias):
    """Literal definition on one request: FIR conv (scipy), SiLU (expit), norms
    (numpy), and the O(d^3) matrix update  S <- S D (I - b k k^T) + b v k^T
    with D = alpha I (GDN) or diag(alpha) (KDA);  o = S q."""
    T = x.shape[0]
    q_ch, k_ch, v_ch = chans(L)
    hist = np.concatenate([win0, x], axis=0)
    y = np.stack([lfilter(w[c, ::-1], [1.0], hist[:, c])[L.conv_width - 1:] + bias[c]
                  for c in range(L.channels)], axis=1)
    a = y * expit(y)
    S = S0.copy()
    outs = np.zeros((T, L.n_v_heads, L.d_v))
    G = L.n_v_heads // L.n_k_heads
    for t in range(T):
        for h in range(L.n_v_heads):
            kh = h // G
            q = a[t, q_ch[kh]]
            q = q / np.linalg.norm(np.append(q, np.sqrt(L.eps))) * L.q_scale
            k = a[t, k_ch[kh]]
            k = k / np.linalg.norm(np.append(k, np.sqrt(L.eps)))
            v = a[t, v_ch[h]]
            D = np.diag(alpha[t, h]) if L.gate == "channel" else alpha[t, h] * np.eye(L.d_k)
            b = beta[t, h]
            S[h] = S[h] @ D @ (np.eye(L.d_k) - b * np.outer(k, k)) + b * np.outer(v, k)
            outs[t, h] = S[h] @ q
    return S, outs


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_brute_force_literal_form(gate):
    """P6: the O(d^2) rank-1 oracle equals the literal O(d^3) form."""
    L = Layer(2, 4, 5, 3, conv_width=4, gate=gate, q_scale=0.6)
    rng = np.random.default_rng(8)
    T, B = 6, 2
    ssm, conv = pools(L, 4)
    ssm[:] = rng.standard_normal(ssm.shape)
    conv[:] = rng.standard_normal(conv.shape)
    idx = np.array([3, 0], np.int32)
    x = rng.standard_normal((B, T, L.channels))
    ash = (B, T, 4, 5) if gate == "channel" else (B, T, 4)
    al = rng.uniform(0.2, 1.0, ash)
    be = rng.uniform(0.0, 1.0, (B, T, 4))
    w = rng.standard_normal((L.channels, 4))
    bias = rng.standard_normal(L.channels)
    ref = [_brute_force(L, ssm[s].copy(), conv[s].copy(), x[b], al[b], be[b], w, bias)
           for b, s in enumerate(idx)]
    out = oracle.decode(L, ssm, conv, idx, x, al, be, w, bias)
    for b, s in enumerate(idx):
        assert relerr(ssm[s], ref[b][0]) < 1e-12
        assert relerr(out[b], ref[b][1]) < 1e-12


def test_gqa_equals_duplicated_key_heads():
    """P10: H_k=2/H_v=4 equals H_k=4/H_v=4 with each key head duplicated."""
    La = Layer(2, 4, 6, 5)
    Lb = Layer(4, 4, 6, 5)
    rng = np.random.default_rng(9)
    T = 5
    qa, ka, va = chans(La)
    perm = np.concatenate([qa[0], qa[0], qa[1], qa[1], ka[0], ka[0], ka[1], ka[1],
                           *va])   # channel map b <- a
    xa = rng.standard_normal((1, T, La.channels))
    wa = rng.standard_normal((La.channels, 4))
    ssa, cva = pools(La, 1)
    ssa[:] = rng.standard_normal(ssa.shape)
    cva[:] = rng.standard_normal(cva.shape)
    ssb, cvb = ssa.copy(), cva[:, :, perm].copy()
    al = rng.uniform(0.2, 1, (1, T, 4))
    be = rng.uniform(0, 1, (1, T, 4))
    oa = oracle.decode(La, ssa, cva, [0], xa, al, be, wa)
    ob = oracle.decode(Lb, ssb, cvb, [0], xa[:, :, perm], al, be, wa[perm])
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(ssa, ssb)
    np.testing.assert_array_equal(cva[:, :, perm], cvb)


def test_kda_constant_gate_equals_gdn():
    """P9: the per-channel gate with all channels equal is the scalar gate."""
    Lg = Layer(2, 4, 6, 5, gate="scalar")
    Lk = Layer(2, 4, 6, 5, gate="channel")
    rng = np.random.default_rng(10)
    T = 4
    x = rng.standard_normal((2, T, Lg.channels))
    w = rng.standard_normal((Lg.channels, 4))
    al = rng.uniform(0.2, 1, (2, T, 4))
    be = rng.uniform(0, 1, (2, T, 4))
    s1, c1 = pools(Lg, 3)
    s1[:] = rng.standard_normal(s1.shape)
    c1[:] = rng.standard_normal(c1.shape)
    s2, c2 = s1.copy(), c1.copy()
    o1 = oracle.decode(Lg, s1, c1, [2, 1], x, al, be, w)
    o2 = oracle.decode(Lk, s2, c2, [2, 1], x, np.repeat(al[..., None], 6, axis=-1), be, w)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_power_of_two_homogeneity():
    """P12: scaling S0 and the v inputs by 2^m scales S_t and o_t by 2^m exactly."""
    L = Layer(2, 4, 6, 5, conv_silu=False)
    rng = np.random.default_rng(11)
    T = 6
    _, _, v = chans(L)
    vc = np.concatenate(v)
    x = rng.standard_normal((1, T, L.channels))
    w = rng.standard_normal((L.channels, 4))
    al = rng.uniform(0.2, 1, (1, T, 4))
    be = rng.uniform(0, 1, (1, T, 4))
    s1, c1 = pools(L, 1)
    s1[:] = rng.standard_normal(s1.shape)
    c1[:] = rng.standard_normal(c1.shape)
    s2, c2, x2 = s1 * 8.0, c1.copy(), x.copy()
    c2[:, :, vc] *= 8.0
    x2[:, :, vc] *= 8.0
    o1 = oracle.decode(L, s1, c1, [0], x, al, be, w)
    o2 = oracle.decode(L, s2, c2, [0], x2, al, be, w)
    np.testing.assert_array_equal(o1 * 8.0, o2)
    np.testing.assert_array_equal(s1 * 8.0, s2)


def test_permutation_symmetry():
    """P13: permuting requests and their slots permutes the results."""
    L = Layer(2, 4, 6, 5, gate="channel")
    rng = np.random.default_rng(12)
    B, T = 5, 3
    x = rng.standard_normal((B, T, L.channels))
    w = rng.standard_normal((L.channels, 4))
    al = rng.uniform(0.2, 1, (B, T, 4, 6))
    be = rng.uniform(0, 1, (B, T, 4))
    s1, c1 = pools(L, 8)
    s1[:] = rng.standard_normal(s1.shape)
    c1[:] = rng.standard_normal(c1.shape)
    s2, c2 = s1.copy(), c1.copy()
    idx = np.array([7, 1, 4, 0, 5], np.int32)
    p = np.array([3, 0, 4, 1, 2])
    o1 = oracle.decode(L, s1, c1, idx, x, al, be, w)
    o2 = oracle.decode(L, s2, c2, idx[p], x[p], al[p], be[p], w)
    np.testing.assert_array_equal(o1[p], o2)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)


def test_multi_token_equals_repeated_single_steps_and_skip_rows():
    L = Layer(2, 4, 6, 5)
    rng = np.random.default_rng(13)
    B, T = 3, 5
    x = rng.standard_normal((B, T, L.channels))
    w = rng.standard_normal((L.channels, 4))
    al = rng.uniform(0.2, 1, (B, T, 4))
    be = rng.uniform(0, 1, (B, T, 4))
    s1, c1 = pools(L, 6)
    s1[:] = rng.standard_normal(s1.shape)
    c1[:] = rng.standard_normal(c1.shape)
    s2, c2 = s1.copy(), c1.copy()
    idx = np.array([4, -1, 2], np.int32)
    o1 = oracle.decode(L, s1, c1, idx, x, al, be, w)
    o2 = np.stack([oracle.decode(L, s2, c2, idx, x[:, t:t + 1], al[:, t:t + 1], be[:, t:t + 1],
                                 w)[:, 0] for t in range(T)], axis=1)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)
    assert not np.any(o1[1])                   # skipped row: output untouched
    s3, c3 = pools(L, 6)
    s3[:] = rng.standard_normal(s3.shape)


# --------------------------------------------------------------------------
# D5: speculative drafts and commit

def test_spec_snapshots_and_commit_equal_recomputation():
    """P8: draft T tokens into snapshots, commit L -> the working slot equals a
    plain decode of the first L tokens (bit for bit); L = 0 is a no-op."""
    L = Layer(2, 4, 6, 5)
    rng = np.random.default_rng(14)
    B, T = 4, 5
    x = rng.standard_normal((B, T, L.channels))
    w = rng.standard_normal((L.channels, 4))
    al = rng.uniform(0.2, 1, (B, T, 4))
    be = rng.uniform(0, 1, (B, T, 4))
    s1, c1 = pools(L, 6)
    s1[:] = rng.standard_normal(s1.shape)
    c1[:] = rng.standard_normal(c1.shape)
    s2, c2 = s1.copy(), c1.copy()
    s_before, c_before = s1.copy(), c1.copy()
    idx = np.array([5, 0, 3, 2], np.int32)
    t_max = 7
    sp_s = np.full((B, t_max) + s1.shape[1:], np.nan)
    sp_c = np.full((B, t_max) + c1.shape[1:], np.nan)
    o1 = oracle.decode(L, s1, c1, idx, x, al, be, w, spec_ssm=sp_s, spec_conv=sp_c)
    np.testing.assert_array_equal(s1, s_before)          # working slots untouched
    np.testing.assert_array_equal(c1, c_before)
    for b in range(B):                                   # snapshot windows = raw inputs
        hist = np.concatenate([c_before[idx[b]], x[b]], axis=0)
        for t in range(T):
            np.testing.assert_array_equal(sp_c[b, t], hist[t + 1:t + 4])
    acc = np.array([0, 2, 5, 1], np.int32)
    oracle.spec_commit(L, s1, c1, idx, sp_s, sp_c, acc)
    for b in range(B):
        n = int(acc[b])
        if n == 0:
            continue
        o2 = oracle.decode(L, s2, c2, idx[b:b + 1], x[b:b + 1, :n], al[b:b + 1, :n],
                           be[b:b + 1, :n], w)
        np.testing.assert_array_equal(o1[b, :n], o2[0])
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)


# --------------------------------------------------------------------------
# D6: slot copy / zero and the stale-state rule

def test_slot_copy_zero_exact_and_isolated():
    """P14: exact bytes in the touched slots, every other slot unchanged."""
    L = Layer(2, 4, 6, 5)
    rng = np.random.default_rng(15)
    s, c = pools(L, 8)
    s[:] = rng.standard_normal(s.shape)
    c[:] = rng.standard_normal(c.shape)
    s0, c0 = s.copy(), c.copy()
    oracle.slot_copy(L, s, c, [1, 6], [3, 0])
    oracle.slot_zero(L, s, c, [5, -1])
    np.testing.assert_array_equal(s[3], s0[1])
    np.testing.assert_array_equal(c[0], c0[6])
    assert not np.any(s[5]) and not np.any(c[5])
    assert not np.any(np.signbit(s[5]))
    for k in (1, 2, 4, 6, 7):
        np.testing.assert_array_equal(s[k], s0[k])
        np.testing.assert_array_equal(c[k], c0[k])


def test_poisoned_fresh_slots_are_clean_after_zero_or_cow():
    """P15: NaN-poisoned slots never leak once zeroed or copied from a clean
    checkpoint, and CoW then decode equals decoding the checkpoint itself."""
    L = Layer(2, 4, 6, 5)
    rng = np.random.default_rng(16)
    s, c = pools(L, 4)
    s[:] = np.nan
    c[:] = np.nan
    s[3] = rng.standard_normal(s.shape[1:])
    c[3] = rng.standard_normal(c.shape[1:])
    oracle.slot_zero(L, s, c, [0])
    oracle.slot_copy(L, s, c, [3], [1])
    T = 3
    x = rng.standard_normal((2, T, L.channels))
    w = rng.standard_normal((L.channels, 4))
    al = rng.uniform(0.2, 1, (2, T, 4))
    be = rng.uniform(0, 1, (2, T, 4))
    ref_s, ref_c = s.copy(), c.copy()
    o = oracle.decode(L, s, c, [0, 1], x, al, be, w)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s[:2])) and np.all(np.isfinite(c[:2]))
    o_ref = oracle.decode(L, ref_s, ref_c, [0, 3], x, al, be, w)
    np.testing.assert_array_equal(o, o_ref)
    np.testing.assert_array_equal(s[1], ref_s[3])


# --------------------------------------------------------------------------
# D7 / D8: prefill

def _prefill_inputs(L, seqlens, rng):
    total = int(np.sum(seqlens))
    cu = np.zeros(len(seqlens) + 1, np.int32)
    cu[1:] = np.cumsum(seqlens)
    x = rng.standard_normal((total, L.channels))
    al = np.exp(-np.logaddexp(0, rng.standard_normal((total, L.n_v_heads))))
    be = expit(rng.standard_normal((total, L.n_v_heads)))
    w = rng.uniform(-0.5, 0.5, (L.channels, L.conv_width))
    return cu, x, al, be, w


def test_prefill_equals_decode_of_the_same_tokens():
    """The prefill driver (cu_seqlens, init slots) runs the same recurrence as a
    T-token decode of each sequence."""
    L = Layer(2, 4, 6, 5)
    rng = np.random.default_rng(17)
    lens = [7, 0, 12]
    cu, x, al, be, w = _prefill_inputs(L, lens, rng)
    s, c = pools(L, 8)
    s[:] = rng.standard_normal(s.shape)
    c[:] = rng.standard_normal(c.shape)
    s2, c2 = s.copy(), c.copy()
    dst = np.array([1, 4, 6], np.int32)
    init = np.array([-1, 2, 6], np.int32)     # zero, CoW from 2, continue in place
    o = oracle.prefill(L, s, c, dst, init, cu, x, al, be, w)
    oracle.slot_zero(L, s2, c2, [1])
    oracle.slot_copy(L, s2, c2, [2], [4])
    for i, n in enumerate(lens):
        if n == 0:
            continue
        od = oracle.decode(L, s2, c2, dst[i:i + 1], x[None, cu[i]:cu[i + 1]],
                           al[None, cu[i]:cu[i + 1]], be[None, cu[i]:cu[i + 1]], w)
        np.testing.assert_array_equal(o[cu[i]:cu[i + 1]], od[0])
    np.testing.assert_array_equal(s, s2)
    np.testing.assert_array_equal(c, c2)


@pytest.mark.parametrize("chunk", [1, 3, 16, 64, 256])
def test_chunked_form_equals_sequential(chunk):
    """P7: the WY/UT chunk form (fp64) equals the sequential recurrence."""
    L = Layer(2, 4, 8, 6)
    rng = np.random.default_rng(18)
    lens = [0, 1, 5, 64, 130, 200]
    cu, x, al, be, w = _prefill_inputs(L, lens, rng)
    s, c = pools(L, 12)
    s[:] = rng.standard_normal(s.shape) / np.sqrt(8)
    c[:] = rng.standard_normal(c.shape)
    s2, c2 = s.copy(), c.copy()
    dst = np.arange(6, dtype=np.int32)
    init = np.array([-1, 9, 2, -1, 10, 5], np.int32)
    o1 = oracle.prefill(L, s, c, dst, init, cu, x, al, be, w)
    o2 = oracle.prefill_chunked(L, s2, c2, dst, init, cu, x, al, be, w, chunk=chunk)
    assert relerr(o2, o1) < 1e-10
    assert relerr(s2, s) < 1e-10
    np.testing.assert_array_equal(c2, c)


def test_chunked_form_strong_decay():
    """P7 with gates down to 1e-3 (64-token gate products near 1e-190) and a
    few exact zeros: log-space gates keep the chunk form finite and exact."""
    L = Layer(1, 2, 8, 8)
    rng = np.random.default_rng(19)
    lens = [128]
    cu, x, _, be, w = _prefill_inputs(L, lens, rng)
    al = rng.uniform(1e-3, 0.05, (128, 2))
    s, c = pools(L, 1)
    s2, c2 = s.copy(), c.copy()
    o1 = oracle.prefill(L, s, c, [0], [-1], cu, x, al, be, w)
    o2 = oracle.prefill_chunked(L, s2, c2, [0], [-1], cu, x, al, be, w, chunk=64)
    assert np.all(np.isfinite(o2))
    assert relerr(o2, o1) < 1e-10
    assert relerr(s2, s) < 1e-10


def test_split_prefill_through_checkpoint_equals_one_shot():
    """P16: prefill 96 -> CoW into a fresh slot -> prefill the remaining 64
    equals one-shot prefill of 160 tokens (bit for bit)."""
    L = Layer(2, 4, 6, 5)
    rng = np.random.default_rng(20)
    cu, x, al, be, w = _prefill_inputs(L, [160], rng)
    s, c = pools(L, 4)
    s[:] = np.nan
    c[:] = np.nan
    o1 = oracle.prefill(L, s, c, [0], [-1], cu, x, al, be, w)
    oa = oracle.prefill(L, s, c, [1], [-1], np.array([0, 96], np.int32), x[:96], al[:96],
                        be[:96], w)
    oracle.slot_copy(L, s, c, [1], [2])      # checkpoint 1 -> working slot 2
    ob = oracle.prefill(L, s, c, [3], [2], np.array([0, 64], np.int32), x[96:], al[96:],
                        be[96:], w)
    np.testing.assert_array_equal(np.concatenate([oa, ob]), o1)
    np.testing.assert_array_equal(s[3], s[0])
    np.testing.assert_array_equal(c[3], c[0])


def test_oracle_rejects_bad_arguments():
    L = Layer(2, 4, 6, 5)
    s, c = pools(L, 2)
    x = np.zeros((1, 1, L.channels))
    with pytest.raises(ValueError):
        oracle.decode(L, s, c, [2], x, np.ones((1, 1, 4)), np.zeros((1, 1, 4)), ident_taps(L))
    with pytest.raises(ValueError):
        oracle.decode(Layer(3, 4, 6, 5), *pools(Layer(3, 4, 6, 5), 1), [0],
                      np.zeros((1, 1, Layer(3, 4, 6, 5).channels)), np.ones((1, 1, 4)),
                      np.zeros((1, 1, 4)), ident_taps(Layer(3, 4, 6, 5)))
    with pytest.raises(ValueError):
        oracle.spec_commit(L, s, c, [0], np.zeros((1, 2) + s.shape[1:]),
                           np.zeros((1, 2) + c.shape[1:]), [3])


# --------------------------------------------------------------------------
# the oracle's own bf16 decoding (every bf16 input reaches the oracle through it)

def test_bf16_decoding_all_bit_patterns():
    """oracle.bf16_bits_to_f64 over all 65 536 bf16 bit patterns against torch's
    CPU bfloat16 type widened to float64 (an independent library routine):
    equal values, equal signs of zero, NaN exactly where torch has NaN."""
    import torch
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_bits_to_f64(pats)
    ref = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert got.dtype == np.float64 and got.shape == ref.shape
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 * 127                    # exponent all ones, mantissa != 0
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # as_f64 routes uint16 arrays through the same decoding, shape kept
    np.testing.assert_array_equal(oracle.as_f64(pats.reshape(256, 256)), got.reshape(256, 256))


def test_bf16_decoding_known_values():
    """bf16 is the upper half of an IEEE binary32: a few patterns worked out
    from the format (sign, 8 exponent bits with bias 127, 7 mantissa bits)."""
    cases = {0x0000: 0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0xC040: -3.0,
             0x3FC0: 1.5, 0x3F81: 1.0 + 2.0 ** -7, 0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127,
             0x0080: 2.0 ** -126, 0x0001: 2.0 ** -133, 0x7F80: np.inf, 0xFF80: -np.inf,
             0x3E00: 0.125}
    pats = np.array(list(cases), dtype=np.uint16)
    np.testing.assert_array_equal(oracle.bf16_bits_to_f64(pats), np.array(list(cases.values())))
    assert np.signbit(oracle.bf16_bits_to_f64(np.array([0x8000], np.uint16))[0])
    assert np.isnan(oracle.bf16_bits_to_f64(np.array([0x7FC0, 0xFFC1], np.uint16))).all()
