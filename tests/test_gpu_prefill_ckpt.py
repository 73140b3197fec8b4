"""GPU checks of the checkpoints a prefill emits on the way (state and conv
window after every 128 tokens, into pool slots) and of the short append that
starts from one, for the scalar and the per-channel decay:

* against the fp64 oracle: each checkpoint's state equals the sequential
  recurrence over that prefix (max-normalised error <= 2e-3) and its conv
  window is bit-exact; the append's outputs and final state equal the
  oracle's recurrence over the whole sequence (same bar), its window exact;
* bit for bit against the plain GPU prefills they replace (a prefill of the
  prefix alone; the one-shot outputs and final state)."""
import numpy as np
import pytest

import oracle
import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import synth
from tests.harness import OUT_TOL, bits, dev, host, layers, rel_err, shadow

pytestmark = pytest.mark.gpu

STATE_TOL = 2e-3

SHAPES = [synth.Shape(2, 4, 16, 16, 4, "scalar", "bf16"),
          synth.Shape(2, 2, 16, 16, 4, "channel", "bf16"),
          synth.Shape(2, 4, 64, 64, 4, "scalar", "bf16"),
          synth.Shape(2, 2, 64, 64, 4, "channel", "bf16"),
          synth.Shape(2, 4, 128, 128, 4, "scalar", "bf16"),
          synth.Shape(2, 2, 128, 128, 4, "channel", "bf16"),
          # narrower convs: windows of 2 and 1 rows
          synth.Shape(2, 4, 64, 64, 3, "scalar", "f32"),
          synth.Shape(2, 4, 32, 32, 2, "scalar", "bf16"),
          synth.Shape(2, 2, 32, 32, 3, "channel", "bf16")]
IDS = ["scalar_d16", "channel_d16", "scalar_d64", "channel_d64", "scalar_d128", "channel_d128",
       "scalar_d64_w3_f32", "scalar_d32_w2", "channel_d32_w3"]


def _torch():
    import torch
    return torch


def _window_bits(c64_row, dtype):
    """Expected storage bits of an oracle conv window (raw inputs, exact)."""
    w = c64_row.astype(np.float32)
    return synth.f32_to_bf16_bits(w) if dtype == "bf16" else w


@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_checkpoints_and_append(shape):
    torch = _torch()
    lens, every, slots = [600, 300], 128, 40
    case = synth.prefill_case(shape, lens, slots, seed=41)
    g, o = layers(shape)
    x, al, be, w = dev(case.x), dev(case.alpha), dev(case.beta), dev(case.conv_w)
    cu = case.cu_seqlens
    i32 = lambda *v: dev(np.asarray(v, np.int32))
    used = set(case.dst.tolist()) | set(case.init_slot[case.init_slot >= 0].tolist())
    spare = [s for s in range(slots) if s not in used]
    tab = np.array([spare[0:5], spare[5:10]], np.int32)
    tab[1, 1] = -1                                       # no slot for this one
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    before = bits(ssm), bits(conv)
    out = gdn.gdn_prefill_chunked(g, ssm, conv, dev(case.dst), dev(case.init_slot), dev(cu),
                                  max(lens), x, al, be, w, ckpt_slots=dev(tab), ckpt_every=every)
    torch.cuda.synchronize()
    after = bits(ssm), bits(conv)
    ssm_h = host(ssm)

    # every written checkpoint: against the oracle's recurrence over that
    # prefix, and bit for bit against a GPU prefill of the prefix alone
    written, worst = [], 0.0
    for s, T in enumerate(lens):
        t0 = int(cu[s])
        for k in range(tab.shape[1]):
            n = (k + 1) * every
            sl = tab[s, k]
            if n > T or sl < 0:
                continue
            written.append(sl)
            s64, c64 = shadow(case.pool)
            oracle.prefill(o, s64, c64, [sl], [case.init_slot[s]], np.array([0, n], np.int32),
                           case.x[t0:t0 + n], case.alpha[t0:t0 + n], case.beta[t0:t0 + n],
                           case.conv_w)
            err = rel_err(ssm_h[sl], s64[sl])
            worst = max(worst, err)
            assert err <= STATE_TOL, f"checkpoint {s}/{k}: state error {err:.3e}"
            np.testing.assert_array_equal(host(conv)[sl], _window_bits(c64[sl], shape.dtype))

            ref_s, ref_c = dev(case.pool.ssm), dev(case.pool.conv)
            ref_dst = spare[12]
            gdn.gdn_prefill_chunked(g, ref_s, ref_c, i32(ref_dst), i32(case.init_slot[s]),
                                    i32(0, n), n, x[t0:t0 + n].contiguous(),
                                    al[t0:t0 + n].contiguous(), be[t0:t0 + n].contiguous(), w)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(after[0][sl], bits(ref_s)[ref_dst])
            np.testing.assert_array_equal(after[1][sl], bits(ref_c)[ref_dst])
    assert len(written) == 4 + 1
    print(f"{shape.gate} d={shape.d_k}: worst checkpoint state error {worst:.2e}")
    untouched = np.setdiff1d(np.arange(slots), np.concatenate([case.dst, written]))
    np.testing.assert_array_equal(after[0][untouched], before[0][untouched])
    np.testing.assert_array_equal(after[1][untouched], before[1][untouched])

    # append: tokens 384..599 of sequence 0 from its checkpoint after 384
    start = 3 * every
    t0, T = int(cu[0]), lens[0]
    app_dst = spare[13]
    o_app = gdn.gdn_prefill_chunked(g, ssm, conv, i32(app_dst), i32(tab[0, 2]),
                                    i32(0, T - start), T - start,
                                    x[t0 + start:t0 + T].contiguous(),
                                    al[t0 + start:t0 + T].contiguous(),
                                    be[t0 + start:t0 + T].contiguous(), w)
    torch.cuda.synchronize()
    # the oracle: the whole sequence token by token from its initial slot
    s64, c64 = shadow(case.pool)
    ref = oracle.prefill(o, s64, c64, [app_dst], [case.init_slot[0]],
                         np.array([0, T], np.int32), case.x[t0:t0 + T], case.alpha[t0:t0 + T],
                         case.beta[t0:t0 + T], case.conv_w)
    out_err = rel_err(host(o_app), ref[start:])
    st_err = rel_err(host(ssm)[app_dst], s64[app_dst])
    print(f"{shape.gate} d={shape.d_k}: append out {out_err:.2e} state {st_err:.2e}")
    assert out_err <= OUT_TOL and st_err <= STATE_TOL
    np.testing.assert_array_equal(host(conv)[app_dst], _window_bits(c64[app_dst], shape.dtype))
    # ... and bit for bit the tail of the one-shot prefill
    np.testing.assert_array_equal(bits(o_app), bits(out)[t0 + start:t0 + T])
    np.testing.assert_array_equal(bits(ssm)[app_dst], after[0][case.dst[0]])
    np.testing.assert_array_equal(bits(conv)[app_dst], after[1][case.dst[0]])
