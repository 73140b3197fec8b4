"""libgdn loads without a GPU, exports every symbol include/gdn.h declares,
and rejects bad arguments on the host before anything is enqueued.  No call
here reaches a HIP API: every case returns during validation (or is B = 0)."""
import ctypes as ct
import os
import re

import pytest

import hybrid_linear_attention_decode_amd as gdn
from hybrid_linear_attention_decode_amd import GdnInputs, GdnLayer, GdnPool, GdnSpecCache

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "gdn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdn_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    syms = declared_symbols()
    assert set(syms) == set(gdn.EXPORTED)
    L = gdn.lib()
    for s in syms:
        assert hasattr(L, s), s


def test_status_strings():
    for st in range(8):
        assert gdn.gdn_status_string(st)
    assert "precondition" in gdn.gdn_status_string(gdn.GDN_ERR_PRECONDITION)
    assert gdn.gdn_status_string(99) == "unknown status"


FAKE = ct.c_void_p(0x10000)  # never dereferenced: every call below fails validation


def qwen_layer(**kw):
    d = dict(n_k_heads=16, n_v_heads=32, d_k=128, d_v=128, conv_width=4)
    d.update(kw)
    return gdn.Layer(**d).c_struct()


def decode(L, pool=None, idx=FAKE, B=4, T=1, inp=None, out=FAKE, spec=None):
    pool = pool or GdnPool(FAKE, FAKE, 8)
    inp = inp or GdnInputs(FAKE, FAKE, FAKE, FAKE, None)
    return gdn.lib().gdn_decode_step(ct.byref(L), ct.byref(pool), idx, None, B, T,
                                     ct.byref(inp), out, spec, None, None)


@pytest.mark.parametrize("field,value,status", [
    ("n_v_heads", 24, gdn.GDN_ERR_BAD_SHAPE),      # 24 % 16 != 0
    ("n_k_heads", 0, gdn.GDN_ERR_BAD_SHAPE),
    ("d_k", 96, gdn.GDN_ERR_UNSUPPORTED),
    ("d_v", 40, gdn.GDN_ERR_UNSUPPORTED),
    ("d_v", 512, gdn.GDN_ERR_UNSUPPORTED),
    ("conv_width", 0, gdn.GDN_ERR_BAD_SHAPE),
    ("conv_width", 5, gdn.GDN_ERR_UNSUPPORTED),
    ("gate", 7, gdn.GDN_ERR_BAD_DTYPE),
    ("act_dtype", 3, gdn.GDN_ERR_BAD_DTYPE),
    ("flags", 8, gdn.GDN_ERR_BAD_SHAPE),
])
def test_bad_layer(field, value, status):
    L = qwen_layer()
    setattr(L, field, value)
    assert decode(L) == status


def test_bad_decode_arguments():
    L = qwen_layer()
    assert gdn.lib().gdn_decode_step(None, None, FAKE, None, 1, 1, None, FAKE, None, None,
                                     None) == \
        gdn.GDN_ERR_NULL_ARG
    assert decode(L, pool=GdnPool(None, FAKE, 8)) == gdn.GDN_ERR_NULL_ARG
    assert decode(L, pool=GdnPool(FAKE, None, 8)) == gdn.GDN_ERR_NULL_ARG
    assert decode(L, idx=None) == gdn.GDN_ERR_NULL_ARG
    assert decode(L, out=None) == gdn.GDN_ERR_NULL_ARG
    assert decode(L, inp=GdnInputs(FAKE, None, FAKE, FAKE, None)) == gdn.GDN_ERR_NULL_ARG
    assert decode(L, T=0) == gdn.GDN_ERR_BAD_SHAPE
    # a misaligned work counter word
    assert gdn.lib().gdn_decode_step(ct.byref(L), ct.byref(GdnPool(FAKE, FAKE, 8)), FAKE, None,
                                     4, 1, ct.byref(GdnInputs(FAKE, FAKE, FAKE, FAKE, None)),
                                     FAKE, None, ct.c_void_p(0x10002), None) == \
        gdn.GDN_ERR_BAD_SHAPE
    assert decode(L, B=-1) == gdn.GDN_ERR_BAD_SHAPE
    assert decode(L, B=70000) == gdn.GDN_ERR_BAD_SHAPE
    assert decode(L, pool=GdnPool(ct.c_void_p(0x10004), FAKE, 8)) == gdn.GDN_ERR_BAD_SHAPE
    spec = GdnSpecCache(FAKE, FAKE, 3)
    assert decode(L, T=4, spec=ct.byref(spec)) == gdn.GDN_ERR_BAD_SHAPE   # T > t_max
    spec0 = GdnSpecCache(None, FAKE, 7)
    assert decode(L, T=4, spec=ct.byref(spec0)) == gdn.GDN_ERR_NULL_ARG
    # snapshots in pool slots need no spec buffers, but t_max still bounds T
    pooled = GdnSpecCache(None, None, 3, FAKE)
    assert decode(L, T=4, spec=ct.byref(pooled)) == gdn.GDN_ERR_BAD_SHAPE
    assert decode(L, T=2, spec=ct.byref(pooled), B=0) == gdn.GDN_OK
    # a conv-less layer (W = 1) needs no conv pool; B = 0 enqueues nothing
    L1 = qwen_layer(conv_width=1)
    assert decode(L1, pool=GdnPool(FAKE, None, 8), B=0) == gdn.GDN_OK


def test_decode_shapes_that_do_not_fit_one_workgroup():
    """The decode needs a key head's value rows, conv channels and gates in one
    workgroup of at most 8 waves (include/gdn.h); other shapes are refused
    before anything is enqueued."""
    # 4 value heads of 128 rows per key head: 512 rows > 8 waves x 32
    assert decode(qwen_layer(n_k_heads=8, n_v_heads=32, d_v=128)) == gdn.GDN_ERR_UNSUPPORTED
    # 16 rows but 2 x 128 + 16 conv channels: more than two waves' threads
    assert decode(qwen_layer(n_k_heads=16, n_v_heads=16, d_v=16)) == gdn.GDN_ERR_UNSUPPORTED
    # 4 value heads of 64 rows: 256 rows in 8 waves of 32 -- taken
    assert decode(qwen_layer(n_k_heads=8, n_v_heads=32, d_v=64), B=0) == gdn.GDN_OK


def test_sizes_past_32_bit_offsets_are_refused():
    """Conv channels C and H_v d_k are at most 2^22 for every entry point, and a
    decode's T C, T H_v d_v and T H_v d_k at most 2^31 - 1 (include/gdn.h): the
    kernels address a token's row, and a request's or a chunk's rows, with
    32-bit offsets."""
    # 16 key heads of d_k = 128 and 16384 value heads of d_v = 256: C > 2^22
    big = qwen_layer(n_k_heads=16, n_v_heads=16384, d_v=256)
    assert decode(big, B=0) == gdn.GDN_ERR_BAD_SHAPE
    assert gdn.lib().gdn_slot_bytes(ct.byref(big)) == 0
    # C = 2^22 exactly is taken
    edge = qwen_layer(n_k_heads=8192, n_v_heads=8192, d_k=128, d_v=256)
    assert 2 * 8192 * 128 + 8192 * 256 == 1 << 22
    assert gdn.lib().gdn_slot_bytes(ct.byref(edge)) > 0
    # H_v d_k = 2^23 with C about 2^20: the per-channel decays of one token
    kda = qwen_layer(gate="channel", n_k_heads=1, n_v_heads=65536, d_k=128, d_v=16)
    assert gdn.lib().gdn_slot_bytes(ct.byref(kda)) == 0
    # Qwen3.5 shape, C = 8192: T up to (2^31 - 1) / 8192 tokens per request
    L = qwen_layer()
    assert decode(L, B=0, T=(2**31 - 1) // 8192) == gdn.GDN_OK
    assert decode(L, B=0, T=(2**31 - 1) // 8192 + 1) == gdn.GDN_ERR_BAD_SHAPE


def test_bad_commit_index_arguments():
    pool = GdnPool(FAKE, FAKE, 8)
    lib = gdn.lib()
    pooled = GdnSpecCache(None, None, 7, FAKE)
    assert lib.gdn_spec_commit_index(ct.byref(pool), ct.byref(pooled), None, FAKE, None, 4,
                                     None) == gdn.GDN_ERR_NULL_ARG
    assert lib.gdn_spec_commit_index(ct.byref(pool), ct.byref(pooled), FAKE, None, None, 4,
                                     None) == gdn.GDN_ERR_NULL_ARG
    buffers = GdnSpecCache(FAKE, FAKE, 7, None)     # snapshots not in pool slots
    assert lib.gdn_spec_commit_index(ct.byref(pool), ct.byref(buffers), FAKE, FAKE, None, 4,
                                     None) == gdn.GDN_ERR_NULL_ARG
    assert lib.gdn_spec_commit_index(ct.byref(pool), ct.byref(GdnSpecCache(None, None, 0, FAKE)),
                                     FAKE, FAKE, None, 4, None) == gdn.GDN_ERR_BAD_SHAPE
    assert lib.gdn_spec_commit_index(ct.byref(pool), ct.byref(pooled), FAKE, FAKE, None, -1,
                                     None) == gdn.GDN_ERR_BAD_SHAPE
    assert lib.gdn_spec_commit_index(ct.byref(pool), ct.byref(pooled), FAKE, FAKE, None, 0,
                                     None) == gdn.GDN_OK
    # the copy commit refuses snapshots kept in pool slots
    L = qwen_layer()
    assert lib.gdn_spec_decode_commit(ct.byref(L), ct.byref(pool), FAKE, ct.byref(pooled), FAKE,
                                      4, None) == gdn.GDN_ERR_BAD_SHAPE


def test_slot_pack_arguments():
    """Packed slot size and the refusals of pack / unpack (nothing enqueued)."""
    lib = gdn.lib()
    L = qwen_layer()
    item = 32 * 128 * 128 * 4 + 3 * 8192 * 2          # ssm slot + bf16 conv window
    assert lib.gdn_slot_bytes(ct.byref(L)) == item
    K = qwen_layer(gate="channel", n_k_heads=32, n_v_heads=32, act_dtype="f32")
    assert lib.gdn_slot_bytes(ct.byref(K)) == 32 * 128 * 128 * 4 + 3 * 12288 * 4
    bad = qwen_layer(d_k=96)
    assert lib.gdn_slot_bytes(ct.byref(bad)) == 0
    pool = GdnPool(FAKE, FAKE, 8)
    for fn, args in ((lib.gdn_slot_pack, lambda n, buf, nb, idx: (idx, n, buf, nb)),
                     (lib.gdn_slot_unpack, lambda n, buf, nb, idx: (buf, nb, idx, n))):
        call = lambda n, buf=FAKE, nb=4 * item, idx=FAKE: fn(ct.byref(L), ct.byref(pool),
                                                            *args(n, buf, nb, idx), None)
        assert call(4, nb=4 * item - 1) == gdn.GDN_ERR_BAD_SHAPE     # buffer too small
        assert call(4, buf=ct.c_void_p(0x10008)) == gdn.GDN_ERR_BAD_SHAPE
        assert call(4, buf=None) == gdn.GDN_ERR_NULL_ARG
        assert call(4, idx=None) == gdn.GDN_ERR_NULL_ARG
        assert call(-1) == gdn.GDN_ERR_BAD_SHAPE
        assert call(0, buf=None, idx=None) == gdn.GDN_OK


def test_bad_slot_and_commit_arguments():
    L = qwen_layer()
    pool = GdnPool(FAKE, FAKE, 8)
    lib = gdn.lib()
    assert lib.gdn_slot_copy(ct.byref(L), ct.byref(pool), None, FAKE, 2, None) == \
        gdn.GDN_ERR_NULL_ARG
    assert lib.gdn_slot_copy(ct.byref(L), ct.byref(pool), FAKE, FAKE, -1, None) == \
        gdn.GDN_ERR_BAD_SHAPE
    assert lib.gdn_slot_zero(ct.byref(L), ct.byref(pool), None, 3, None) == gdn.GDN_ERR_NULL_ARG
    assert lib.gdn_slot_zero(ct.byref(L), ct.byref(pool), None, 0, None) == gdn.GDN_OK
    assert lib.gdn_spec_decode_commit(ct.byref(L), ct.byref(pool), FAKE, None, FAKE, 4,
                                      None) == gdn.GDN_ERR_NULL_ARG
    bad_spec = GdnSpecCache(FAKE, FAKE, 0)
    assert lib.gdn_spec_decode_commit(ct.byref(L), ct.byref(pool), FAKE, ct.byref(bad_spec),
                                      FAKE, 4, None) == gdn.GDN_ERR_BAD_SHAPE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        gdn.lib()


def prefill(L, N=2, dst=FAKE, init=None, cu=FAKE, max_len=64, total=128, chunk=64, inp=None,
            out=FAKE, ws=None, ws_bytes=0, ckpt=None):
    pool = GdnPool(FAKE, FAKE, 8)
    inp = inp or GdnInputs(FAKE, FAKE, FAKE, FAKE, None)
    return gdn.lib().gdn_prefill_chunked(ct.byref(L), ct.byref(pool), dst, init, N, cu,
                                         max_len, total, chunk, ct.byref(inp), out,
                                         None if ckpt is None else ct.byref(ckpt), ws,
                                         ws_bytes, None)


def test_bad_prefill_arguments():
    L = qwen_layer()
    assert prefill(L, N=-1) == gdn.GDN_ERR_BAD_SHAPE
    assert prefill(L, max_len=-1) == gdn.GDN_ERR_BAD_SHAPE
    assert prefill(L, chunk=32) == gdn.GDN_ERR_UNSUPPORTED
    assert prefill(qwen_layer(n_k_heads=2, n_v_heads=2, d_k=48, d_v=16)) == \
        gdn.GDN_ERR_UNSUPPORTED
    # d_k = 16 is taken (it runs in the d_k = 32 layout)
    assert prefill(qwen_layer(n_k_heads=2, n_v_heads=2, d_k=16, d_v=16), N=0) == gdn.GDN_OK
    assert prefill(L, dst=None) == gdn.GDN_ERR_NULL_ARG
    assert prefill(L, cu=None) == gdn.GDN_ERR_NULL_ARG
    assert prefill(L, inp=GdnInputs(None, FAKE, FAKE, FAKE, None)) == gdn.GDN_ERR_NULL_ARG
    assert prefill(L, out=None) == gdn.GDN_ERR_NULL_ARG
    misaligned = GdnInputs(ct.c_void_p(0x10002), FAKE, FAKE, FAKE, None)
    assert prefill(L, inp=misaligned) == gdn.GDN_ERR_BAD_SHAPE
    assert prefill(L, N=0) == gdn.GDN_OK                  # nothing to do, nothing enqueued
    # checkpoints: a chunk-multiple interval, a slot table when any are asked for
    Ck = gdn.GdnPrefillCkpt
    assert prefill(L, N=0, ckpt=Ck(FAKE, 96, 4)) == gdn.GDN_ERR_BAD_SHAPE
    assert prefill(L, N=0, ckpt=Ck(FAKE, 0, 4)) == gdn.GDN_ERR_BAD_SHAPE
    assert prefill(L, N=0, ckpt=Ck(FAKE, 128, -1)) == gdn.GDN_ERR_BAD_SHAPE
    assert prefill(L, N=0, ckpt=Ck(None, 128, 4)) == gdn.GDN_ERR_NULL_ARG
    assert prefill(L, N=0, ckpt=Ck(None, 128, 0)) == gdn.GDN_OK
    # the scalar-decay prefill stores the prepared q / k rows: 8 bytes per
    # (token, key head, key channel); missing, short or misaligned is refused
    size = gdn.lib().gdn_prefill_workspace_size
    assert size(ct.byref(L), 4, 8192, 32768, 64) == 32768 * 16 * 128 * 8
    assert size(ct.byref(L), 0, 0, 0, 64) == 0
    need = size(ct.byref(L), 2, 64, 128, 64)
    assert need == 128 * 16 * 128 * 8
    assert prefill(L) == gdn.GDN_ERR_WORKSPACE
    assert prefill(L, ws=FAKE, ws_bytes=need - 1) == gdn.GDN_ERR_WORKSPACE
    assert prefill(L, ws=ct.c_void_p(0x10080), ws_bytes=need) == gdn.GDN_ERR_WORKSPACE
    # d_k = 16 keeps its rows at the d_k = 32 layout's width
    L16 = qwen_layer(n_k_heads=2, n_v_heads=2, d_k=16, d_v=16)
    assert size(ct.byref(L16), 2, 64, 128, 64) == 128 * 2 * 32 * 8


def test_per_channel_prefill_workspace():
    """The per-channel-decay prefill stores one 2 KiB record per (16-token
    block, value head): floor(total / 16) + 4 min(N, total) blocks."""
    K = qwen_layer(gate="channel", n_k_heads=32, n_v_heads=32)
    size = gdn.lib().gdn_prefill_workspace_size
    assert size(ct.byref(K), 4, 8192, 32768, 64) == (2048 + 16) * 32 * 2048
    assert size(ct.byref(K), 3, 100, 130, 64) == (8 + 12) * 32 * 2048
    assert size(ct.byref(K), 1000, 1, 5, 64) == (0 + 20) * 32 * 2048   # empty sequences cost nothing
    assert size(ct.byref(K), 0, 0, 0, 64) == 0
    assert size(ct.byref(K), 4, 8192, 32768, 32) == 0                   # bad chunk
    assert size(ct.byref(K), -1, 8192, 32768, 64) == 0
    need = size(ct.byref(K), 2, 64, 128, 64)
    # missing, short or misaligned workspace is refused before any launch
    assert prefill(K) == gdn.GDN_ERR_WORKSPACE
    assert prefill(K, ws=FAKE, ws_bytes=need - 1) == gdn.GDN_ERR_WORKSPACE
    assert prefill(K, ws=ct.c_void_p(0x10080), ws_bytes=need) == gdn.GDN_ERR_WORKSPACE
    assert prefill(K, N=0) == gdn.GDN_OK
    assert prefill(K, chunk=32) == gdn.GDN_ERR_UNSUPPORTED


def test_static_prefill_refuses_oversized_calls_on_the_host():
    """gdn_prefill_chunked_static: a call whose workspace would exceed the
    library's array is refused before any HIP call (no device needed)."""
    L = qwen_layer()
    cu = FAKE
    inp = GdnInputs(FAKE, FAKE, FAKE, FAKE, None)
    st = gdn.lib().gdn_prefill_chunked_static(ct.byref(L), ct.byref(GdnPool(FAKE, FAKE, 8)),
                                             FAKE, None, 1, cu, 8192, 8192, 64, ct.byref(inp),
                                             FAKE, None, None)
    assert st == gdn.GDN_ERR_WORKSPACE
    need = gdn.gdn_prefill_workspace_size(gdn.Layer(16, 32, 128, 128), 1, 8192, 8192)
    assert need > gdn.GDN_PREFILL_STATIC_BYTES
