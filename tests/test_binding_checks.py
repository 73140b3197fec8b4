"""The Python binding refuses, before any pointer reaches the C ABI, index
arrays that are not int32 of the right length (the kernels read 32-bit words,
so an int64 tensor would be read as pairs of halves and, e.g., zero slot 0),
pools whose dtype or per-slot shape differs from the layer's, and inputs or
outputs of the wrong dtype or size.  CPU tensors only: every case raises
during validation, and well-formed host tensors are refused as not on the
device."""
import pytest
import torch

import hybrid_linear_attention_decode_amd as gdn

L = gdn.Layer(2, 4, 16, 32, conv_width=4)           # C = 2*2*16 + 4*32 = 192


def pool(slots=8, ssm_dtype=torch.float32, conv_dtype=torch.bfloat16, d_v=32):
    return (torch.zeros(slots, 4, d_v, 16, dtype=ssm_dtype),
            torch.zeros(slots, 3, L.channels, dtype=conv_dtype))


def tokens(B=2, T=1, dtype=torch.bfloat16):
    return (torch.zeros(B, T, L.channels, dtype=dtype), torch.zeros(B, T, 4, dtype=dtype),
            torch.zeros(B, T, 4, dtype=dtype), torch.zeros(L.channels, 4, dtype=dtype))


I32 = lambda *v: torch.tensor(v, dtype=torch.int32)
I64 = lambda *v: torch.tensor(v, dtype=torch.int64)


def test_int64_indices_refused_everywhere():
    ssm, conv = pool()
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_slot_zero(L, ssm, conv, I64(5, 9))
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_slot_copy(L, ssm, conv, I64(1, 2), I32(3, 4))
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_slot_copy(L, ssm, conv, I32(1, 2), I64(3, 4))
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_slot_pack(L, ssm, conv, I64(1))
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_slot_unpack(L, ssm, conv, torch.zeros(1 << 16, dtype=torch.uint8), I64(1))
    x, al, be, w = tokens()
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_decode_step(L, ssm, conv, I64(0, 1), x, al, be, w)
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_decode_step(L, ssm, conv, I32(0, 1), x, al, be, w, init_slot=I64(-1, 3))
    sp = torch.zeros(2, 3, 4, 32, 16)
    spc = torch.zeros(2, 3, 3, L.channels, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_spec_decode_commit(L, ssm, conv, I32(0, 1), sp, spc, I64(1, 2))
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_spec_commit_index(ssm, conv, torch.zeros(2, 3, dtype=torch.int32), I64(1, 2),
                                  I32(0, 1))
    xp = torch.zeros(10, L.channels, dtype=torch.bfloat16)
    alp, bep = torch.zeros(10, 4, dtype=torch.bfloat16), torch.zeros(10, 4, dtype=torch.bfloat16)
    for bad in (dict(dst=I64(0, 1)), dict(init=I64(-1, 2)), dict(cu=I64(0, 4, 10))):
        args = dict(dst=I32(0, 1), init=I32(-1, 2), cu=I32(0, 4, 10))
        args.update(bad)
        with pytest.raises(ValueError, match="int32"):
            gdn.gdn_prefill_chunked(L, ssm, conv, args["dst"], args["init"], args["cu"], 6,
                                    xp, alp, bep, w)
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_prefill_chunked(L, ssm, conv, I32(0, 1), None, I32(0, 4, 10), 6, xp, alp, bep,
                                w, ckpt_slots=torch.zeros(2, 1, dtype=torch.int64))


def test_index_lengths_checked():
    ssm, conv = pool()
    x, al, be, w = tokens(B=2)
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_decode_step(L, ssm, conv, I32(0, 1, 2), x, al, be, w)
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_slot_copy(L, ssm, conv, I32(1, 2), I32(3))
    xp = torch.zeros(10, L.channels, dtype=torch.bfloat16)
    alp, bep = torch.zeros(10, 4, dtype=torch.bfloat16), torch.zeros(10, 4, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="int32"):
        gdn.gdn_prefill_chunked(L, ssm, conv, I32(0, 1), None, I32(0, 10), 10, xp, alp, bep, w)


def test_pool_dtype_and_slot_shape_checked():
    x, al, be, w = tokens()
    for ssm, conv in (pool(ssm_dtype=torch.float64), pool(conv_dtype=torch.float32),
                      pool(d_v=16)):
        with pytest.raises(ValueError, match="pool"):
            gdn.gdn_decode_step(L, ssm, conv, I32(0, 1), x, al, be, w)
        with pytest.raises(ValueError, match="pool"):
            gdn.gdn_slot_zero(L, ssm, conv, I32(0))
    ssm, conv = pool()
    with pytest.raises(ValueError, match="pool"):
        gdn.gdn_slot_copy(L, ssm, conv[:4], I32(0), I32(1))   # pools of different slot counts
    with pytest.raises(ValueError, match="pool"):
        gdn.gdn_slot_zero(L, ssm, None, I32(0))               # conv pool missing (W = 4)


def test_inputs_and_outputs_checked():
    ssm, conv = pool()
    x, al, be, w = tokens()
    with pytest.raises(ValueError, match="x must"):
        gdn.gdn_decode_step(L, ssm, conv, I32(0, 1), x.float(), al, be, w)
    with pytest.raises(ValueError, match="alpha must"):
        gdn.gdn_decode_step(L, ssm, conv, I32(0, 1), x, al[:, :, :2], be, w)
    with pytest.raises(ValueError, match="conv_b must"):
        gdn.gdn_decode_step(L, ssm, conv, I32(0, 1), x, al, be, w,
                            conv_b=torch.zeros(5, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must"):
        gdn.gdn_decode_step(L, ssm, conv, I32(0, 1), x, al, be, w,
                            out=torch.zeros(2, 1, 4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="x must"):
        gdn.gdn_decode_step(L, ssm, conv, I32(0, 1), x[0], al, be, w)


def test_well_formed_host_tensors_refused_as_not_on_device():
    ssm, conv = pool()
    x, al, be, w = tokens()
    with pytest.raises(ValueError, match="device"):
        gdn.gdn_decode_step(L, ssm, conv, I32(0, 1), x, al, be, w,
                            out=torch.zeros(2, 1, 4, 32))
    with pytest.raises(ValueError, match="device"):
        gdn.gdn_slot_zero(L, ssm, conv, I32(0))
