"""GPU parity of the KDA-style decode stack at its own size: per-channel gate,
B = 64, 32/32 heads, d_k = d_v = 128, 12 288 channels, bf16 inputs, fp32
state; every layer has its own 1024-slot pool, taps and inputs, and the
layers run back to back on one stream.  Each step re-purposes slots the way
a serving loop does: 16 fresh working slots (NaN-poisoned first, as a
recycled slot would be, then zeroed), 16 copy-on-write from distinct clean
checkpoint slots, 32 continuing in place.

Two device copies of the stack run the same steps: one with the separate
slot kernels (gdn_slot_zero / gdn_slot_copy, then the decode), one with the
preparation fused into the decode call (init_slot: -1 zero start, else the
checkpoint) and a work counter passed (the last quarter of the units handed
out by ticket, as the bench runs it).  Both are checked: every output
and every working slot against the fp64 oracle (max-normalised error <= 2e-3,
conv windows exact), the two bit for bit against each other over the whole
pools, and every slot no step wrote bit-identical to its initial contents."""
import numpy as np
import pytest

import oracle
import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import synth
from tests.harness import OUT_TOL, dev, host, layers, rel_err

pytestmark = pytest.mark.gpu

SHAPE = synth.KDA
B, SLOTS, LAYERS, STEPS, DISTINCT = 64, 1024, 3, 2, 64


def _torch():
    import torch
    return torch


def _ints(t):
    import torch
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def test_kda_stack_b64_pool1024_fused_and_separate_prep():
    torch = _torch()
    g, o = layers(SHAPE)
    rs = synth.streams(4)
    base = synth.make_pool(SHAPE, DISTINCT, np.arange(DISTINCT), rs)   # slot s holds base[s % 64]
    reps = SLOTS // DISTINCT
    base_ssm, base_conv = dev(base.ssm), dev(base.conv)
    roles = [rs["slot_roles"].permutation(SLOTS).astype(np.int32) for _ in range(STEPS)]

    per_layer = []
    for l in range(LAYERS):
        lrs = synth.streams(100 + l)
        w = synth.make_conv_w(SHAPE, lrs)
        x, al, be = synth.make_tokens(SHAPE, (STEPS, B, 1), lrs)
        pools = {}
        for kind in ("separate", "fused"):
            pools[kind] = (base_ssm.repeat(reps, 1, 1, 1).contiguous(),
                           base_conv.repeat(reps, 1, 1).contiguous())
        per_layer.append(dict(w=w, x=x, al=al, be=be, w_d=dev(w), x_d=dev(x), al_d=dev(al),
                              be_d=dev(be), pools=pools))

    outs = {k: torch.empty((LAYERS, STEPS, B, 1, 32, 128), device="cuda")
            for k in ("separate", "fused")}
    work = gdn.decode_work()
    nan = float("nan")
    for c, r in enumerate(roles):
        idx, fresh, cow_dst, cow_src = r[:B], r[:16], r[16:32], r[B:B + 16]
        init = idx.copy()
        init[:16] = -1
        init[16:32] = cow_src
        idx_d, fresh_d, dst_d, src_d, init_d = (dev(a.copy()) for a in
                                                (idx, fresh, cow_dst, cow_src, init))
        fresh_l = fresh_d.long()
        # slot preparation for every layer, then the decode calls back to back
        for L in per_layer:
            for kind in ("separate", "fused"):
                ssm, conv = L["pools"][kind]
                ssm[fresh_l] = nan
                conv[fresh_l] = nan
            ssm, conv = L["pools"]["separate"]
            gdn.gdn_slot_zero(g, ssm, conv, fresh_d)
            gdn.gdn_slot_copy(g, ssm, conv, src_d, dst_d)
        for l, L in enumerate(per_layer):
            ssm, conv = L["pools"]["separate"]
            gdn.gdn_decode_step(g, ssm, conv, idx_d, L["x_d"][c], L["al_d"][c], L["be_d"][c],
                                L["w_d"], out=outs["separate"][l, c])
        for l, L in enumerate(per_layer):
            ssm, conv = L["pools"]["fused"]
            gdn.gdn_decode_step(g, ssm, conv, idx_d, L["x_d"][c], L["al_d"][c], L["be_d"][c],
                                L["w_d"], out=outs["fused"][l, c], init_slot=init_d,
                                work=work)
    torch.cuda.synchronize()
    assert not bool(work.any())

    # fused == separate, bit for bit: outputs and the whole pools
    assert torch.equal(_ints(outs["separate"]), _ints(outs["fused"]))
    for L in per_layer:
        for a, b in zip(L["pools"]["separate"], L["pools"]["fused"]):
            assert torch.equal(_ints(a), _ints(b))

    # against the oracle, layer by layer, on the slots the steps touch (the
    # fp64 shadow pool holds only those, renumbered; results do not depend on
    # slot numbers)
    touched = np.unique(np.concatenate([r[:B + 16] for r in roles]))
    pos = {int(s): i for i, s in enumerate(touched)}
    remap = lambda a: np.array([pos[int(s)] for s in a], np.int32)
    written = np.unique(np.concatenate([r[:B] for r in roles]))
    worst_o = worst_s = 0.0
    out_sep = host(outs["separate"])
    for l, L in enumerate(per_layer):
        s64 = oracle.as_f64(base.ssm[touched % DISTINCT]).copy()
        c64 = oracle.as_f64(base.conv[touched % DISTINCT]).copy()
        for c, r in enumerate(roles):
            oracle.slot_zero(o, s64, c64, remap(r[:16]))
            oracle.slot_copy(o, s64, c64, remap(r[B:B + 16]), remap(r[16:32]))
            ref = oracle.decode(o, s64, c64, remap(r[:B]), L["x"][c], L["al"][c], L["be"][c],
                                L["w"])
            err = rel_err(out_sep[l, c], ref)
            worst_o = max(worst_o, err)
            assert err <= OUT_TOL, f"layer {l} step {c}: output error {err:.3e}"
        ssm, conv = L["pools"]["separate"]
        wi = dev(written).long()
        got_s, got_c = host(ssm[wi]), host(conv[wi])
        err = rel_err(got_s, s64[remap(written)])
        worst_s = max(worst_s, err)
        assert err <= OUT_TOL, f"layer {l}: state error {err:.3e}"
        np.testing.assert_array_equal(
            got_c, synth.f32_to_bf16_bits(c64[remap(written)].astype(np.float32)))
        # every slot no step wrote (checkpoint sources included) is unchanged
        keep = np.setdiff1d(np.arange(SLOTS), written)
        ki = dev(keep.astype(np.int32)).long()
        src_i = dev((keep % DISTINCT).astype(np.int32)).long()
        assert torch.equal(_ints(ssm[ki]), _ints(base_ssm[src_i]))
        assert torch.equal(_ints(conv[ki]), _ints(base_conv[src_i]))
    print(f"KDA stack B={B}, pool {SLOTS}, {LAYERS} layers x {STEPS} steps: worst output "
          f"error {worst_o:.2e}, worst state error {worst_s:.2e}")
