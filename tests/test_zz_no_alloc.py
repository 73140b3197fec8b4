"""The allocation-free prefill entry point (gdn_prefill_chunked_static, for
callers that cannot allocate) against the prefill with a caller workspace
(gdn_prefill_chunked): the same kernels, so outputs, pools and checkpoints
must match bit for bit.  Two calls in a row, the second smaller (the shared
library array keeps the first call's contents), for both decay kinds; a
call needing more workspace than the array holds is refused with nothing
enqueued."""
import numpy as np
import pytest

import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import synth
from tests.harness import bits, dev, layers

pytestmark = pytest.mark.gpu

SHAPES = [synth.QWEN35, synth.Shape(8, 8, 128, 128, 4, "channel", "bf16")]


def _torch():
    import torch
    return torch


@pytest.mark.parametrize("shape", SHAPES, ids=["scalar_qwen35", "channel_8heads"])
def test_static_prefill_equals_workspace_prefill_bitwise(shape):
    torch = _torch()
    g, _ = layers(shape)
    for call, (lens, seed) in enumerate((([1500, 900, 600], 51), ([300, 77], 52))):
        case = synth.prefill_case(shape, lens, 24, seed=seed)
        total = int(case.cu_seqlens[-1])
        need = gdn.gdn_prefill_workspace_size(g, len(lens), max(lens), total)
        assert 0 < need <= gdn.GDN_PREFILL_STATIC_BYTES
        used = set(case.dst.tolist()) | set(case.init_slot[case.init_slot >= 0].tolist())
        spare = [s for s in range(24) if s not in used]
        tab = dev(np.array([spare[3 * i:3 * i + 3] for i in range(len(lens))], np.int32))
        results = []
        for static in (False, True):
            ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
            out = torch.full((total, shape.n_v_heads, shape.d_v), float("nan"), device="cuda")
            args = (g, ssm, conv, dev(case.dst), dev(case.init_slot), dev(case.cu_seqlens),
                    max(lens), dev(case.x), dev(case.alpha), dev(case.beta), dev(case.conv_w))
            if static:
                gdn.gdn_prefill_chunked_static(*args, out=out, ckpt_slots=tab, ckpt_every=256)
            else:
                gdn.gdn_prefill_chunked(*args, out=out, ckpt_slots=tab, ckpt_every=256)
            torch.cuda.synchronize()
            results.append((bits(out), bits(ssm), bits(conv)))
        for a, b in zip(*results):
            np.testing.assert_array_equal(a, b)
        print(f"{shape.gate} call {call}: {total} tokens, workspace {need} B, bitwise equal")


def test_static_prefill_refuses_too_large_a_call():
    torch = _torch()
    shape = synth.QWEN35
    g, _ = layers(shape)
    lens = [4200]                                   # 4200 * 16 KiB > 64 MiB
    case = synth.prefill_case(shape, lens, 4, seed=53)
    assert gdn.gdn_prefill_workspace_size(g, 1, 4200, 4200) > gdn.GDN_PREFILL_STATIC_BYTES
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    before = bits(ssm), bits(conv)
    with pytest.raises(gdn.GdnError) as err:
        gdn.gdn_prefill_chunked_static(g, ssm, conv, dev(case.dst), dev(case.init_slot),
                                       dev(case.cu_seqlens), 4200, dev(case.x),
                                       dev(case.alpha), dev(case.beta), dev(case.conv_w))
    assert err.value.status == gdn.GDN_ERR_WORKSPACE
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(ssm), before[0])
    np.testing.assert_array_equal(bits(conv), before[1])
