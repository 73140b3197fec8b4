"""The seeded workload generator: determinism, encoding, structure."""
import numpy as np
import torch

from hybrid_linear_attention_decode_amd import synth


def test_same_seed_same_bytes():
    a = synth.decode_case(synth.TINY, B=1, T=16, num_slots=4, n_calls=3, seed=0)
    b = synth.decode_case(synth.TINY, B=1, T=16, num_slots=4, n_calls=3, seed=0)
    c = synth.decode_case(synth.TINY, B=1, T=16, num_slots=4, n_calls=3, seed=1)
    for f in ("x", "alpha", "beta", "indices", "conv_w"):
        assert getattr(a, f).tobytes() == getattr(b, f).tobytes()
    assert a.pool.ssm.tobytes() == b.pool.ssm.tobytes()
    assert a.x.tobytes() != c.x.tobytes()


def test_bf16_rounding_matches_torch_cast():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 65504.0, 1e-40, -3.4e38, np.inf, -np.inf],
                                 np.float32)])
    ours = synth.f32_to_bf16_bits(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    nan = synth.f32_to_bf16_bits(np.array([np.nan], np.float32))
    assert torch.from_numpy(nan.view(np.int16)).view(torch.bfloat16).isnan().all()


def test_rotating_indices_distinct_and_spread():
    g = synth.streams(5)["indices"]
    idx = synth.rotating_indices(1024, 64, 48, g)
    for row in idx:
        assert len(set(row.tolist())) == 64
    # one full sweep of the pool every 16 calls
    assert sorted(np.concatenate(idx[:16]).tolist()) == list(range(1024))


def test_gate_ranges_and_poison():
    case = synth.decode_case(synth.QWEN35, B=4, T=1, num_slots=16, n_calls=2, seed=3)
    al = (case.alpha.astype(np.uint32) << 16).view(np.float32)
    be = (case.beta.astype(np.uint32) << 16).view(np.float32)
    assert np.all((al > 0) & (al <= 1)) and np.all((be > 0) & (be < 1))
    live = set(np.unique(case.indices).tolist())
    for s in range(16):
        assert np.isnan(case.pool.ssm[s]).all() == (s not in live)


def test_prefill_case_structure():
    p = synth.prefill_case(synth.TINY, [5, 0, 9], num_slots=8, seed=3)
    assert p.cu_seqlens.tolist() == [0, 5, 5, 14]
    assert p.x.shape == (14, 96)
    assert (p.init_slot[0::2] == -1).all() and (p.init_slot[1::2] >= 0).all()
    assert not set(p.dst.tolist()) & set(p.init_slot.tolist())
    for s in p.init_slot[p.init_slot >= 0]:
        assert np.isfinite(p.pool.ssm[s]).all()
