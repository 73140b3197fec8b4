"""GPU checks of the checkpoints a prefill emits on the way (state and conv
window after every 128 tokens, into pool slots) and of the short append that
starts from one: both bit-identical to the plain prefills they replace, for
the scalar and the per-channel decay."""
import numpy as np
import pytest

import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import synth
from tests.harness import bits, dev, layers

pytestmark = pytest.mark.gpu

SHAPES = [synth.Shape(2, 4, 64, 64, 4, "scalar", "bf16"),
          synth.Shape(2, 2, 64, 64, 4, "channel", "bf16")]


def _torch():
    import torch
    return torch


@pytest.mark.parametrize("shape", SHAPES, ids=["scalar", "channel"])
def test_checkpoints_and_append_bitwise(shape):
    torch = _torch()
    lens, every, slots = [600, 300], 128, 40
    case = synth.prefill_case(shape, lens, slots, seed=41)
    g, _ = layers(shape)
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
    # every written checkpoint equals a prefill of that prefix alone
    written = []
    for s, T in enumerate(lens):
        for k in range(tab.shape[1]):
            n = (k + 1) * every
            sl = tab[s, k]
            if n > T or sl < 0:
                continue
            written.append(sl)
            ref_s, ref_c = dev(case.pool.ssm), dev(case.pool.conv)
            t0 = int(cu[s])
            ref_dst = spare[12]
            gdn.gdn_prefill_chunked(g, ref_s, ref_c, i32(ref_dst), i32(case.init_slot[s]),
                                    i32(0, n), n, x[t0:t0 + n].contiguous(),
                                    al[t0:t0 + n].contiguous(), be[t0:t0 + n].contiguous(), w)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(after[0][sl], bits(ref_s)[ref_dst])
            np.testing.assert_array_equal(after[1][sl], bits(ref_c)[ref_dst])
    assert len(written) == 4 + 1
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
    np.testing.assert_array_equal(bits(o_app), bits(out)[t0 + start:t0 + T])
    np.testing.assert_array_equal(bits(ssm)[app_dst], after[0][case.dst[0]])
    np.testing.assert_array_equal(bits(conv)[app_dst], after[1][case.dst[0]])
