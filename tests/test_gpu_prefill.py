"""GPU parity of the chunked prefill (gdn_prefill_chunked) against the fp64
sequential recurrence of the oracle, on the same seeded inputs.

Bar (the pages give no number for prefill; the decode bar is reused):
outputs max|do|/max|o| <= 2e-3 and final state max-normalised error <= 2e-3
against the token-by-token recurrence; the destination conv window is
bit-exact (it is a copy of raw inputs); slots other than the destinations
and sequences that are skipped stay bit-identical."""
import numpy as np
import pytest

import oracle
import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import synth
from tests.harness import OUT_TOL, bits, dev, host, layers, rel_err, shadow

pytestmark = pytest.mark.gpu

STATE_TOL = 2e-3


def _torch():
    import torch
    return torch


def run_case(shape, seqlens, num_slots=None, seed=0, **layer_kw):
    """Runs one seeded prefill case on the GPU and on the oracle; returns the
    pieces the tests compare."""
    torch = _torch()
    N = len(seqlens)
    case = synth.prefill_case(shape, seqlens, num_slots or max(4, 2 * N), seed)
    init = case.init_slot
    g, o = layers(shape, **layer_kw)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    before = bits(ssm), bits(conv)
    total = int(case.cu_seqlens[-1])
    out = torch.full((total, shape.n_v_heads, shape.d_v), float("nan"), device="cuda")
    gdn.gdn_prefill_chunked(g, ssm, conv, dev(case.dst), dev(init), dev(case.cu_seqlens),
                            max(seqlens) if seqlens else 0, dev(case.x), dev(case.alpha),
                            dev(case.beta), dev(case.conv_w), out=out)
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    ref = oracle.prefill(o, s64, c64, case.dst, init, case.cu_seqlens, case.x, case.alpha,
                         case.beta, case.conv_w)
    return dict(case=case, init=init, out=host(out), ref=ref, ssm=host(ssm), conv=host(conv),
                s64=s64, c64=c64, before=before, ssm_t=ssm, conv_t=conv)


def check(r, out_tol=OUT_TOL, state_tol=STATE_TOL):
    case = r["case"]
    dst = case.dst
    out_err = rel_err(r["out"], r["ref"]) if r["ref"].size else 0.0
    st_err = rel_err(r["ssm"][dst], r["s64"][dst]) if dst.size else 0.0
    assert out_err <= out_tol, f"output error {out_err:.3e}"
    assert st_err <= state_tol, f"state error {st_err:.3e}"
    np.testing.assert_array_equal(oracle.as_f64(r["conv"][dst]), r["c64"][dst])
    others = np.setdiff1d(np.arange(case.pool.ssm.shape[0]), dst)
    np.testing.assert_array_equal(bits(r["ssm_t"])[others], r["before"][0][others])
    np.testing.assert_array_equal(bits(r["conv_t"])[others], r["before"][1][others])
    return out_err, st_err


SMALL = synth.Shape(2, 4, 32, 32, 4, "scalar", "bf16")


def test_ragged_lengths_small_heads():
    """Lengths around the chunk edges (1, 63, 64, 65, 130, 200), zero and CoW
    starts, d_k = d_v = 32, GQA 2:1, bf16 inputs."""
    r = run_case(SMALL, [1, 63, 64, 65, 130, 200], seed=1)
    print("ragged small: out %.2e state %.2e" % check(r))


def test_fp32_inputs_short_window():
    """fp32 inputs, conv width 2, d_k = 64 and d_v = 48 (a partly idle
    column block)."""
    shape = synth.Shape(1, 2, 64, 48, 2, "scalar", "f32")
    r = run_case(shape, [37, 128, 99], seed=2)
    print("fp32 W=2: out %.2e state %.2e" % check(r))


@pytest.mark.parametrize("dv", [16, 80, 128])
def test_value_widths(dv):
    """d_v not a multiple of 64 spreads one head over partly used blocks."""
    shape = synth.Shape(2, 2, 128, dv, 4, "scalar", "bf16")
    r = run_case(shape, [150, 64, 3], seed=3 + dv)
    print("dv=%d: out %.2e state %.2e" % ((dv,) + check(r)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_silu_no_norm_with_conv_bias(dtype):
    """SiLU and L2 norm switched off, conv bias on (small inputs keep the
    un-normalised state bounded); fp32 and bf16 storage."""
    shape = synth.Shape(1, 1, 32, 32, 4, "scalar", dtype)
    case = synth.prefill_case(shape, [96, 40], 4, seed=5)
    case.x[:] = synth.encode((oracle.as_f64(case.x) * 0.05).astype(np.float32), dtype)
    bias = synth.encode(np.random.default_rng(5).standard_normal(shape.channels) * 0.05, dtype)
    g, o = layers(shape, conv_silu=False, l2norm=False)
    torch = _torch()
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


def test_empty_skipped_and_in_place():
    """Length-0 sequences copy (or zero) the initial state into the
    destination; dst < 0 skips a sequence and leaves its output rows alone;
    init == dst continues a live slot in place."""
    torch = _torch()
    shape = SMALL
    case = synth.prefill_case(shape, [0, 70, 0, 50, 40], 12, seed=7)
    g, o = layers(shape)
    init = case.init_slot.copy()
    dst = case.dst.copy()
    init[2] = case.init_slot[1]        # empty sequence, copy-on-write start
    live = case.init_slot[3]           # sequence 3 continues its own (live) slot
    case.pool.ssm[dst[3]] = case.pool.ssm[live]
    case.pool.conv[dst[3]] = case.pool.conv[live]
    init[3] = dst[3]
    dst[1] = -1                        # skipped
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
    assert np.isnan(o_h[cu[1]:cu[2]]).all()          # skipped rows untouched
    assert rel_err(o_h[cu[3]:], ref[cu[3]:]) <= OUT_TOL
    written = dst[dst >= 0]
    assert rel_err(host(ssm)[written], s64[written]) <= STATE_TOL
    for s in (0, 2):                                 # empty: exact copies (or zeros)
        np.testing.assert_array_equal(host(ssm)[dst[s]], s64[dst[s]].astype(np.float32))
    np.testing.assert_array_equal(oracle.as_f64(host(conv)[written]), c64[written])
    untouched = np.setdiff1d(np.arange(12), written)
    np.testing.assert_array_equal(bits(ssm)[untouched], before[0][untouched])
    np.testing.assert_array_equal(bits(conv)[untouched], before[1][untouched])


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("width,dtype", [(4, "bf16"), (3, "bf16"), (4, "f32")])
def test_short_sequences_continue_their_own_slot(gate, width, dtype):
    """Every sequence continues its own live slot (init == dst), with lengths
    0 .. W-1 among them: the new conv window then takes rows of the old one
    from the slot it overwrites.  Windows bit-exact against the oracle,
    outputs and states to the usual bar, other slots untouched."""
    torch = _torch()
    shape = synth.Shape(2, 4, 32, 32, width, gate, dtype)
    lens = [0, 1, 2, 3, 5, 40, 70]
    case = synth.prefill_case(shape, lens, 16, seed=31)
    g, o = layers(shape)
    dst = case.dst.copy()
    for s in range(len(lens)):                # each destination holds a live state
        src = case.init_slot[s] if case.init_slot[s] >= 0 else case.init_slot[1]
        case.pool.ssm[dst[s]] = case.pool.ssm[src]
        case.pool.conv[dst[s]] = case.pool.conv[src]
    init = dst.copy()
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    before = bits(ssm), bits(conv)
    total = int(case.cu_seqlens[-1])
    out = gdn.gdn_prefill_chunked(g, ssm, conv, dev(dst), dev(init), dev(case.cu_seqlens),
                                  max(lens), dev(case.x), dev(case.alpha), dev(case.beta),
                                  dev(case.conv_w))
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    ref = oracle.prefill(o, s64, c64, dst, init, case.cu_seqlens, case.x, case.alpha,
                         case.beta, case.conv_w)
    assert rel_err(host(out), ref) <= OUT_TOL
    assert rel_err(host(ssm)[dst], s64[dst]) <= STATE_TOL
    np.testing.assert_array_equal(oracle.as_f64(host(conv)[dst]), c64[dst])
    untouched = np.setdiff1d(np.arange(16), dst)
    np.testing.assert_array_equal(bits(ssm)[untouched], before[0][untouched])
    np.testing.assert_array_equal(bits(conv)[untouched], before[1][untouched])
    print(f"{gate} W={width} {dtype}: {total} tokens, windows bit-exact")


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_run_twice_bitwise(gate):
    """The same prefill on two copies of the same pool gives the same bits
    (outputs, final states, windows, checkpoints)."""
    torch = _torch()
    shape = synth.Shape(4, 8, 128, 128, 4, gate, "bf16")
    lens = [700, 64, 333, 1]
    case = synth.prefill_case(shape, lens, 20, seed=45)
    g, _ = layers(shape)
    used = set(case.dst.tolist()) | set(case.init_slot[case.init_slot >= 0].tolist())
    spare = [s for s in range(20) if s not in used]
    tab = dev(np.array([spare[3 * i:3 * i + 3] for i in range(len(lens))], np.int32))
    runs = []
    for _ in range(2):
        ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
        out = gdn.gdn_prefill_chunked(g, ssm, conv, dev(case.dst), dev(case.init_slot),
                                      dev(case.cu_seqlens), max(lens), dev(case.x),
                                      dev(case.alpha), dev(case.beta), dev(case.conv_w),
                                      ckpt_slots=tab, ckpt_every=128)
        torch.cuda.synchronize()
        runs.append((bits(out), bits(ssm), bits(conv)))
    for a, b in zip(*runs):
        np.testing.assert_array_equal(a, b)


def test_qwen35_4x8192_zero_and_cow():
    """The full workload: 4 x 8192 tokens, 16/32 heads, d = 128, chunk 64,
    bf16 inputs; sequences alternate zero start and copy-on-write from a
    checkpoint slot.  Every output and final state element is compared."""
    r = run_case(synth.QWEN35, [8192] * 4, num_slots=64, seed=11)
    print("qwen35 4x8192: out %.2e state %.2e" % check(r))


def test_split_prefill_equals_one_shot_bitwise():
    """Prefill 4096 tokens, copy the slot to a fresh one (CoW), prefill the
    next 4096 from it: bit-identical to one 8192-token prefill (the carry is
    fp32 in both, and the split is chunk-aligned)."""
    torch = _torch()
    shape = synth.QWEN35
    case = synth.prefill_case(shape, [8192], 8, seed=13)
    g, _ = layers(shape)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    x, al, be, w = dev(case.x), dev(case.alpha), dev(case.beta), dev(case.conv_w)
    one, mid, cow, two = 4, 5, 6, 7
    i32 = lambda *v: dev(np.asarray(v, np.int32))
    o_full = gdn.gdn_prefill_chunked(g, ssm, conv, i32(one), i32(-1), i32(0, 8192), 8192, x, al,
                                     be, w)
    o_a = gdn.gdn_prefill_chunked(g, ssm, conv, i32(mid), i32(-1), i32(0, 4096), 4096,
                                  x[:4096], al[:4096], be[:4096], w)
    gdn.gdn_slot_copy(g, ssm, conv, i32(mid), i32(cow))
    o_b = gdn.gdn_prefill_chunked(g, ssm, conv, i32(two), i32(cow), i32(0, 4096), 4096,
                                  x[4096:].contiguous(), al[4096:].contiguous(),
                                  be[4096:].contiguous(), w)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(o_full)[:4096], bits(o_a))
    np.testing.assert_array_equal(bits(o_full)[4096:], bits(o_b))
    np.testing.assert_array_equal(bits(ssm)[one], bits(ssm)[two])
    np.testing.assert_array_equal(bits(conv)[one], bits(conv)[two])


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dk16(gate, dtype):
    """d_k = 16 (the tiny decode shape's heads), run in the d_k = 32 layout
    with the upper channels as zero padding: ragged lengths around the
    16-token block and chunk edges, zero and copy-on-write starts, against
    the oracle; slots hold d_k = 16 rows, untouched slots stay bit-equal."""
    shape = synth.Shape(2, 2, 16, 16, 4, gate, dtype)
    r = run_case(shape, [1, 15, 17, 63, 64, 65, 130, 200], seed=31)
    print("d_k=16 %s %s: out %.2e state %.2e" % ((gate, dtype) + check(r)))


def test_dk16_gqa_with_conv_bias():
    """d_k = 16 with two value heads per key head, d_v = 32 and a conv bias
    (the padded channels must take no bias), bf16 inputs."""
    torch = _torch()
    shape = synth.Shape(2, 4, 16, 32, 4, "scalar", "bf16")
    case = synth.prefill_case(shape, [70, 33, 128], 8, seed=32)
    bias = synth.encode(np.random.default_rng(32).standard_normal(shape.channels) * 0.3, "bf16")
    g, o = layers(shape)
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    out = gdn.gdn_prefill_chunked(g, ssm, conv, dev(case.dst), dev(case.init_slot),
                                  dev(case.cu_seqlens), 128, dev(case.x), dev(case.alpha),
                                  dev(case.beta), dev(case.conv_w), conv_b=dev(bias))
    torch.cuda.synchronize()
    s64, c64 = shadow(case.pool)
    ref = oracle.prefill(o, s64, c64, case.dst, case.init_slot, case.cu_seqlens, case.x,
                         case.alpha, case.beta, case.conv_w, conv_b=bias)
    assert rel_err(host(out), ref) <= OUT_TOL
    assert rel_err(host(ssm)[case.dst], s64[case.dst]) <= STATE_TOL
    np.testing.assert_array_equal(oracle.as_f64(host(conv)[case.dst]), c64[case.dst])


def test_unsupported_shapes_raise():
    torch = _torch()
    case = synth.prefill_case(SMALL, [64], 4, seed=0)
    g, _ = layers(SMALL)
    with pytest.raises(gdn.GdnError):
        gdn.gdn_prefill_chunked(g, dev(case.pool.ssm), dev(case.pool.conv), dev(case.dst),
                                dev(case.init_slot), dev(case.cu_seqlens), 64, dev(case.x),
                                dev(case.alpha), dev(case.beta), dev(case.conv_w), chunk=32)
    torch.cuda.synchronize()


def test_max_sequences_short():
    """N = 65535 sequences (the largest the ABI takes) of 1-3 tokens each,
    half from zero and half copy-on-write; every output, final state and
    window against the oracle, every other slot untouched."""
    shape = synth.Shape(1, 1, 32, 32, 4, "scalar", "bf16")
    lens = (np.arange(65535) % 3 + 1).tolist()
    r = run_case(shape, lens, num_slots=2 * 65535, seed=14)
    print("65535 sequences: out %.2e state %.2e" % check(r))



@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_small_max_seqlen_bitwise(gate):
    """max_seqlen only sizes launch grids: a value below the longest sequence
    (outside the contract, which GDN_DEBUG enforces) still gives the same bits
    for outputs, final states and windows as the true one."""
    torch = _torch()
    shape = synth.Shape(2, 4, 32, 32, 4, gate, "bf16")
    seqlens = [200, 70, 33, 129]
    case = synth.prefill_case(shape, seqlens, 12, seed=21)
    g, _ = layers(shape)
    res = []
    for mx in (max(seqlens), 40):
        ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
        out = gdn.gdn_prefill_chunked(g, ssm, conv, dev(case.dst), dev(case.init_slot),
                                      dev(case.cu_seqlens), mx, dev(case.x), dev(case.alpha),
                                      dev(case.beta), dev(case.conv_w))
        torch.cuda.synchronize()
        res.append((bits(out), bits(ssm), bits(conv)))
    for a, b in zip(*res):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_graph_capture_bitwise(gate):
    """A prefill call -- every kernel it enqueues -- captured into a graph
    replays bit-identical to the eager call: three replays, the pool restored
    and the output poisoned by eager work between them (zero and
    copy-on-write starts, so a replay reads nothing a replay wrote)."""
    torch = _torch()
    shape = synth.Shape(2, 4, 64, 64, 4, gate, "bf16")
    seqlens = [150, 64, 33, 200]
    case = synth.prefill_case(shape, seqlens, 12, seed=23)
    g, _ = layers(shape)
    mx, total = max(seqlens), sum(seqlens)
    dst, init, cu = dev(case.dst), dev(case.init_slot), dev(case.cu_seqlens)
    x, al, be, w = dev(case.x), dev(case.alpha), dev(case.beta), dev(case.conv_w)
    need = gdn.gdn_prefill_workspace_size(g, len(seqlens), mx, total)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    rs, rc = dev(case.pool.ssm), dev(case.pool.conv)
    rout = gdn.gdn_prefill_chunked(g, rs, rc, dst, init, cu, mx, x, al, be, w, workspace=ws)
    torch.cuda.synchronize()
    ref = bits(rout), bits(rs), bits(rc)

    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    out = torch.empty_like(rout)
    call = lambda: gdn.gdn_prefill_chunked(g, ssm, conv, dst, init, cu, mx, x, al, be, w,
                                           out=out, workspace=ws)
    call()                      # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for _ in range(3):
        out.fill_(float("nan"))
        ssm.copy_(dev(case.pool.ssm))
        conv.copy_(dev(case.pool.conv))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((bits(out), bits(ssm), bits(conv)), ref):
            np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("width", [1, 3])
def test_conv_widths(gate, width):
    """Convs narrower than 4 -- width 1 keeps no conv state at all -- against
    the oracle: taps left-padded in the kernels, windows of width - 1 rows,
    both decay kinds."""
    shape = synth.Shape(2, 4, 32, 32, width, gate, "bf16")
    r = run_case(shape, [100, 37, 64], seed=24)
    print("width %d %s: out %.2e state %.2e" % ((width, gate) + check(r)))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_fp32_activations_dk128(gate):
    """fp32 inputs at d_k = 128 (the preparation pass's 16-byte fp32 row and
    tap loads), ragged lengths across block boundaries, both decay kinds."""
    shape = synth.Shape(2, 4, 128, 64, 4, gate, "f32")
    r = run_case(shape, [97, 32, 160, 1], seed=25)
    print("fp32 d_k=128 %s: out %.2e state %.2e" % ((gate,) + check(r)))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_on_a_non_current_stream(gate):
    """The binding allocates the workspace and the output on the call's stream:
    a prefill launched on a side stream, followed at once (no sync) by
    allocations and writes on the current stream, gives the bits of the same
    prefill run alone."""
    torch = _torch()
    shape = synth.Shape(2, 4, 64, 64, 4, gate, "bf16")
    case = synth.prefill_case(shape, [700, 333, 64], 8, seed=43)
    g, _ = layers(shape)
    args = lambda: (dev(case.dst), dev(case.init_slot), dev(case.cu_seqlens), 700, dev(case.x),
                    dev(case.alpha), dev(case.beta), dev(case.conv_w))
    ref_s, ref_c = dev(case.pool.ssm), dev(case.pool.conv)
    ref = gdn.gdn_prefill_chunked(g, ref_s, ref_c, *args())
    torch.cuda.synchronize()
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    a = args()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ws_bytes = gdn.gdn_prefill_workspace_size(g, 3, 700, int(case.cu_seqlens[-1]))
    out = gdn.gdn_prefill_chunked(g, ssm, conv, *a, stream=side)
    # the current stream allocates and scribbles over fresh blocks of the
    # same sizes while the side stream may still run
    junk = [torch.full((ws_bytes,), 255, dtype=torch.uint8, device="cuda") for _ in range(3)]
    junk += [torch.full(tuple(ref.shape), float("nan"), device="cuda") for _ in range(3)]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(ref))
    np.testing.assert_array_equal(bits(ssm), bits(ref_s))
    np.testing.assert_array_equal(bits(conv), bits(ref_c))
    del junk


def test_decode_on_a_non_current_stream():
    """The same for the decode's output buffer."""
    torch = _torch()
    shape = synth.QWEN35
    case = synth.decode_case(shape, B=16, T=2, num_slots=32, n_calls=1, seed=44)
    g, _ = layers(shape)
    ins = lambda: (dev(case.indices[0]), dev(case.x[0]), dev(case.alpha[0]), dev(case.beta[0]),
                   dev(case.conv_w))
    r_s, r_c = dev(case.pool.ssm), dev(case.pool.conv)
    ref = gdn.gdn_decode_step(g, r_s, r_c, *ins())
    torch.cuda.synchronize()
    ssm, conv = dev(case.pool.ssm), dev(case.pool.conv)
    a = ins()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = gdn.gdn_decode_step(g, ssm, conv, *a, stream=side)
    junk = [torch.full(tuple(ref.shape), float("nan"), device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(out), bits(ref))
    np.testing.assert_array_equal(bits(ssm), bits(r_s))
    del junk
