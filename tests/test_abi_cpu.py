"""The C-ABI library loads, exports every declared entry point, and rejects bad
arguments on the host (CPU only: rejected calls make no HIP call)."""
import ctypes
import os
import re

import pytest

from sequence_decode_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "seqdecode.h")

SD_OK, SD_EINVAL, SD_EUNSUPPORTED, SD_EALIGN, SD_EWORKSPACE = 0, -1, -2, -3, -4
FAKE = ctypes.c_void_p(0x10000)        # never dereferenced: validation fails first
ODD = ctypes.c_void_p(0x10002)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sd_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libseqdecode.so not built (run __graft_entry__.build())")
    return _lib.load()


def test_every_declared_symbol_is_exported_and_bound(L):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"
    assert set(_lib.SIGNATURES) == set(names)


def test_version_and_status_strings(L):
    assert L.sd_abi_version() == 10
    for code in (0, -1, -2, -3, -4, -5):
        assert L.sd_status_string(code).startswith(b"SD_")
    assert L.sd_status_string(7) == b"unknown sd_status"


def test_gemv_rejections(L):
    g = L.sd_qgemv_q8_0_batch
    assert g(None, 64, 256, FAKE, FAKE, 1, None, FAKE, 64, None) == SD_EINVAL
    assert g(FAKE, 64, 256, FAKE, FAKE, 0, None, FAKE, 64, None) == SD_EINVAL
    assert g(FAKE, 64, 256, FAKE, FAKE, 17, None, FAKE, 64, None) == SD_EINVAL
    assert g(FAKE, 64, 128, FAKE, FAKE, 1, None, FAKE, 64, None) == SD_EUNSUPPORTED
    assert g(FAKE, 64, 4000, FAKE, FAKE, 1, None, FAKE, 64, None) == SD_EUNSUPPORTED
    assert g(FAKE, 64, 256, FAKE, FAKE, 1, None, FAKE, 63, None) == SD_EINVAL
    assert g(ODD, 64, 256, FAKE, FAKE, 1, None, FAKE, 64, None) == SD_EALIGN
    assert g(FAKE, 64, 256, ODD, FAKE, 1, None, FAKE, 64, None) == SD_EALIGN
    assert g(FAKE, 0, 14336, FAKE, FAKE, 16, None, FAKE, 64, None) == SD_EINVAL


def test_gemv_path_rejections(L):
    g = L.sd_qgemv_q8_0_batch_path
    for path in (-1, 3, 99):
        assert g(FAKE, 64, 256, FAKE, FAKE, 1, None, FAKE, 64, path, None) == SD_EINVAL
    for path in (0, 1, 2):
        assert g(FAKE, 64, 256, FAKE, FAKE, 17, None, FAKE, 64, path, None) == SD_EINVAL
        assert g(FAKE, 64, 4000, FAKE, FAKE, 1, None, FAKE, 64, path, None) == SD_EUNSUPPORTED
        assert g(ODD, 64, 256, FAKE, FAKE, 1, None, FAKE, 64, path, None) == SD_EALIGN


def test_gemv_swiglu_rejections(L):
    f = L.sd_qgemv_q8_0_swiglu_q8
    assert f(None, 64, 256, FAKE, FAKE, 1, FAKE, FAKE, None) == SD_EINVAL
    assert f(FAKE, 64, 256, FAKE, FAKE, 0, FAKE, FAKE, None) == SD_EINVAL
    assert f(FAKE, 64, 256, FAKE, FAKE, 1, None, FAKE, None) == SD_EINVAL
    assert f(FAKE, 16, 256, FAKE, FAKE, 1, FAKE, FAKE, None) == SD_EINVAL
    assert f(FAKE, 48, 256, FAKE, FAKE, 1, FAKE, FAKE, None) == SD_EUNSUPPORTED    # F % 32
    assert f(FAKE, 64, 4000, FAKE, FAKE, 1, FAKE, FAKE, None) == SD_EUNSUPPORTED   # K % 256
    assert f(FAKE, 64, 8192, FAKE, FAKE, 4, FAKE, FAKE, None) == SD_EUNSUPPORTED   # two chunks
    assert f(FAKE, 64, 4096, FAKE, FAKE, 9, FAKE, FAKE, None) == SD_EUNSUPPORTED   # > 8 tokens
    assert f(ODD, 64, 256, FAKE, FAKE, 1, FAKE, FAKE, None) == SD_EALIGN
    assert f(FAKE, 64, 256, ODD, FAKE, 1, FAKE, FAKE, None) == SD_EALIGN


def test_stream_read_rejections(L):
    r = L.sd_hbm_stream_read
    assert r(None, 64, FAKE, None) == SD_EINVAL
    assert r(FAKE, 0, FAKE, None) == SD_EINVAL
    assert r(FAKE, 40, FAKE, None) == SD_EINVAL
    assert r(FAKE, 64, None, None) == SD_EINVAL
    assert r(ctypes.c_void_p(0x10008), 64, FAKE, None) == SD_EALIGN


def test_quantize_rejections(L):
    q = L.sd_quantize_q8_act
    assert q(FAKE, 64, 1, 48, FAKE, FAKE, None) == SD_EUNSUPPORTED
    assert q(FAKE, 16, 1, 32, FAKE, FAKE, None) == SD_EINVAL
    assert q(FAKE, 64, 17, 64, FAKE, FAKE, None) == SD_EINVAL
    assert q(FAKE, 64, 1, 64, ODD, FAKE, None) == SD_EALIGN


def _view(ctx, cap, k=FAKE, ld_tok=1024, ld_head=128):
    return _lib.SeqView(k.value, FAKE.value, ctx, cap, ld_tok, ld_head)


def test_attention_rejections(L):
    a = L.sd_decode_attn_multiseq
    views5 = (_lib.SeqView * 5)(*[_view(10, 16) for _ in range(5)])
    assert a(FAKE, 4096, views5, 5, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 20, None) == SD_EINVAL
    v1 = (_lib.SeqView * 1)(_view(10, 16))
    assert a(FAKE, 4096, v1, 0, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 20, None) == SD_EINVAL
    assert a(FAKE, 4096, v1, 1, 32, 8, 64, 0.088, FAKE, FAKE, 1 << 20, None) == SD_EUNSUPPORTED
    # any H_q / H_kv is accepted (two query heads per KV head here); a workspace
    # too small is refused before any HIP call
    assert a(FAKE, 4096, v1, 1, 32, 16, 128, 0.088, FAKE, FAKE, 16, None) == SD_EWORKSPACE
    assert a(FAKE, 4096, v1, 1, 32, 32, 128, 0.088, FAKE, FAKE, 16, None) == SD_EWORKSPACE
    assert a(FAKE, 4096, v1, 1, 30, 8, 128, 0.088, FAKE, FAKE, 1 << 20, None) == SD_EINVAL
    over = (_lib.SeqView * 1)(_view(17, 16))
    assert a(FAKE, 4096, over, 1, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 20, None) == SD_EINVAL
    zero = (_lib.SeqView * 1)(_view(0, 16))
    assert a(FAKE, 4096, zero, 1, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 20, None) == SD_EINVAL
    mis = (_lib.SeqView * 1)(_view(10, 16, k=ctypes.c_void_p(0x10008)))
    assert a(FAKE, 4096, mis, 1, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 20, None) == SD_EALIGN
    need = L.sd_decode_attn_workspace_bytes(v1, 1, 32, 128)
    assert need == 1 * 32 * 132 * 4      # one chunk per head for ctx 10
    assert a(FAKE, 4096, v1, 1, 32, 8, 128, 0.088, FAKE, FAKE, need - 4, None) == SD_EWORKSPACE
    v2 = (_lib.SeqView * 2)(_view(2050, 4096), _view(32768, 32768))
    # chunks: 64 keys below position 2048, 256 beyond -> 32 + 1 and 32 + 120
    assert L.sd_decode_attn_workspace_bytes(v2, 2, 32, 128) == (33 + 152) * 32 * 132 * 4


def test_noalloc_attention_rejections(L):
    """The allocation-free attention entry point validates like the workspace
    one, and refuses partials beyond its 16 MiB scratch array before any HIP
    call (so this runs without a GPU)."""
    a = L.sd_decode_attn_multiseq_noalloc
    views5 = (_lib.SeqView * 5)(*[_view(10, 16) for _ in range(5)])
    assert a(FAKE, 4096, views5, 5, 32, 8, 128, 0.088, FAKE, None) == SD_EINVAL
    v1 = (_lib.SeqView * 1)(_view(10, 16))
    assert a(None, 4096, v1, 1, 32, 8, 128, 0.088, FAKE, None) == SD_EINVAL
    assert a(FAKE, 4096, v1, 1, 32, 8, 64, 0.088, FAKE, None) == SD_EUNSUPPORTED
    assert a(ODD, 4096, v1, 1, 32, 8, 128, 0.088, FAKE, None) == SD_EALIGN
    big = (_lib.SeqView * 4)(*[_view(65536, 65536) for _ in range(4)])
    need = L.sd_decode_attn_workspace_bytes(big, 4, 32, 128)
    assert need == 4 * (32 + 248) * 32 * 132 * 4 > (16 << 20)
    assert a(FAKE, 4096, big, 4, 32, 8, 128, 0.088, FAKE, None) == SD_EWORKSPACE


def test_verify_attention_rejections_and_workspace(L):
    a = L.sd_decode_attn_verify
    v2 = (_lib.SeqView * 2)(_view(258, 300), _view(3, 16))
    nn = (ctypes.c_int32 * 2)(4, 3)
    need = L.sd_decode_attn_verify_workspace_bytes(v2, nn, 2, 32, 128)
    assert need == (5 * 4 + 1 * 3) * 32 * 132 * 4  # chunks x tokens x heads partials
    assert L.sd_decode_attn_verify_workspace_bytes(v2, None, 2, 32, 128) == \
        L.sd_decode_attn_workspace_bytes(v2, 2, 32, 128)
    for bad in ((0, 1), (5, 1), (4, 4)):   # 0 tokens, more than 4, more than ctx_len
        b = (ctypes.c_int32 * 2)(*bad)
        assert a(FAKE, 4096, v2, b, 2, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 30, None) == SD_EINVAL
        assert L.sd_decode_attn_verify_workspace_bytes(v2, b, 2, 32, 128) == 0
    assert a(FAKE, 4096, v2, None, 2, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 30, None) == SD_EINVAL
    assert a(FAKE, 4096, v2, nn, 2, 32, 8, 128, 0.088, FAKE, FAKE, need - 4, None) == SD_EWORKSPACE


def test_window_and_ring_rejections(L):
    a = L.sd_decode_attn_multiseq
    def view(ctx, cap, window, ring):
        return (_lib.SeqView * 1)(_lib.SeqView(FAKE.value, FAKE.value, ctx, cap, 1024, 128, window, ring))
    ok = view(5000, 300, 256, 1)          # ring: 256 positions in use fit 300 rows
    assert a(FAKE, 4096, ok, 1, 32, 8, 128, 0.088, FAKE, FAKE, 0, None) == SD_EWORKSPACE
    need = L.sd_decode_attn_workspace_bytes(ok, 1, 32, 128)
    assert need == 2 * 32 * 132 * 4       # positions 4744..4999 touch chunks 42 and 43
    for bad in (view(5000, 300, 0, 1),    # a ring needs a window
                view(5000, 200, 256, 1),  # the window does not fit the ring
                view(10, 16, -1, 0),      # negative window
                view(10, 16, 0, 2),       # unknown ring flag
                view(17, 16, 4, 0)):      # a plain view still needs ctx_len <= capacity
        assert a(FAKE, 4096, bad, 1, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 30, None) == SD_EINVAL
        assert L.sd_decode_attn_workspace_bytes(bad, 1, 32, 128) == 0
    nn = (ctypes.c_int32 * 1)(4)          # a burst of 4 needs window + 3 rows in the ring
    assert L.sd_decode_attn_verify(FAKE, 4096, view(5000, 258, 256, 1), nn, 1, 32, 8, 128, 0.088,
                                   FAKE, FAKE, 1 << 30, None) == SD_EINVAL
    assert L.sd_decode_attn_verify_workspace_bytes(view(5000, 259, 256, 1), nn, 1, 32, 128) > 0
    huge = view(1 << 30, 1 << 20, 0, 0)
    assert L.sd_decode_attn_workspace_bytes(huge, 1, 32, 128) == 0


def test_paged_rejections(L):
    a = L.sd_decode_attn_multiseq
    def view(ctx, cap, bs, table=FAKE, ring=0, window=0):
        return (_lib.SeqView * 1)(_lib.SeqView(FAKE.value, FAKE.value, ctx, cap, 1024, 128, window,
                                               ring, table.value, bs, 0))
    for bs in (64, 128, 256):
        ok = view(5000, 1024, bs)         # a paged context may exceed the pool (shared blocks)
        need = L.sd_decode_attn_workspace_bytes(ok, 1, 32, 128)
        assert need == (32 + 12) * 32 * 132 * 4
        assert a(FAKE, 4096, ok, 1, 32, 8, 128, 0.088, FAKE, FAKE, need - 4, None) == SD_EWORKSPACE
    for bad in (view(100, 1024, 32),      # blocks of 64, 128 or 256 rows only
                view(100, 1024, 100),
                view(100, 1024, 0),
                view(100, 1000, 64),      # the pool holds whole blocks
                view(100, 1024, 64, ring=1, window=50)):  # not combined with a ring
        assert a(FAKE, 4096, bad, 1, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 30, None) == SD_EINVAL
        assert L.sd_decode_attn_workspace_bytes(bad, 1, 32, 128) == 0
    assert a(FAKE, 4096, view(100, 1024, 64, table=ODD), 1, 32, 8, 128, 0.088, FAKE, FAKE,
             1 << 30, None) == SD_EALIGN
    kv = L.sd_kv_append_f16
    assert kv(FAKE, FAKE, 1024, view(100, 1000, 64), 1, 8, 128, None) == SD_EINVAL


def test_q8_0_view_rejections(L):
    a = L.sd_decode_attn_multiseq
    def view(ctx=100, cap=128, kq=FAKE, kd=FAKE, ld_tok=1024, kv_type=1):
        return _lib.SeqView(0, 0, ctx, cap, ld_tok, 128, 0, 0, None, 0, kv_type,
                            kq.value, FAKE.value, kd.value, FAKE.value)
    one = lambda v: (_lib.SeqView * 1)(v)
    ok = one(view())
    need = L.sd_decode_attn_workspace_bytes(ok, 1, 32, 128)
    assert need == 2 * 32 * 132 * 4       # 100 keys: two 64-key chunks
    assert a(FAKE, 4096, ok, 1, 32, 8, 128, 0.088, FAKE, FAKE, need - 4, None) == SD_EWORKSPACE
    for bad, rc in ((view(kq=ctypes.c_void_p(0)), SD_EINVAL),     # missing codes
                    (view(kd=ctypes.c_void_p(0)), SD_EINVAL),     # missing scales
                    (view(kv_type=5), SD_EINVAL),                 # unknown type
                    (view(kv_type=-1), SD_EINVAL),
                    (view(kq=ODD), SD_EALIGN),
                    (view(kd=ctypes.c_void_p(0x10004)), SD_EALIGN),  # scales need 8 bytes
                    (view(ld_tok=1056), SD_EALIGN)):              # strides: multiples of 128
        assert a(FAKE, 4096, one(bad), 1, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 30, None) == rc
    # one kv_type per call
    mixed = (_lib.SeqView * 2)(view(), _lib.SeqView(FAKE.value, FAKE.value, 100, 128, 1024, 128))
    assert a(FAKE, 4096, mixed, 2, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 30, None) == SD_EUNSUPPORTED
    # each append takes its own type
    kv8, kv16 = L.sd_kv_append_q8_0, L.sd_kv_append_f16
    assert kv16(FAKE, FAKE, 1024, ok, 1, 8, 128, None) == SD_EINVAL
    plain = one(_lib.SeqView(FAKE.value, FAKE.value, 100, 128, 1024, 128))
    assert kv8(FAKE, FAKE, 1024, plain, 1, 8, 128, None) == SD_EINVAL
    assert kv8(FAKE, FAKE, 1024, ok, 1, 8, 100, None) == SD_EINVAL        # D % 32
    assert kv8(FAKE, FAKE, 1024, one(view(ld_tok=1040)), 1, 8, 128, None) == SD_EALIGN


def test_q4_and_mixed_view_rejections_and_workspace(L):
    """q4_0 and the mixed Q4/Q8, Q8/Q4 views take the q8_0 view's checks; their
    workspace is that of any view of the same contexts; one kv_type per call."""
    a = L.sd_decode_attn_multiseq
    def view(kv_type, ctx=100, kq=FAKE, kd=FAKE, ld_tok=1024):
        return _lib.SeqView(0, 0, ctx, 128, ld_tok, 128, 0, 0, None, 0, kv_type,
                            kq.value, FAKE.value, kd.value, FAKE.value)
    one = lambda v: (_lib.SeqView * 1)(v)
    for t in (2, 3, 4):
        ok = one(view(t))
        need = L.sd_decode_attn_workspace_bytes(ok, 1, 32, 128)
        assert need == 2 * 32 * 132 * 4
        assert a(FAKE, 4096, ok, 1, 32, 8, 128, 0.088, FAKE, FAKE, need - 4, None) == SD_EWORKSPACE
        for bad, rc in ((view(t, kq=ctypes.c_void_p(0)), SD_EINVAL),
                        (view(t, kd=ctypes.c_void_p(0)), SD_EINVAL),
                        (view(t, kq=ODD), SD_EALIGN),
                        (view(t, ld_tok=1056), SD_EALIGN)):
            assert a(FAKE, 4096, one(bad), 1, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 30, None) == rc
        for u in (1, 2, 3, 4):
            if u != t:
                pair = (_lib.SeqView * 2)(view(t), view(u))
                assert a(FAKE, 4096, pair, 2, 32, 8, 128, 0.088, FAKE, FAKE, 1 << 30, None) == SD_EUNSUPPORTED
        # the quantized append takes every quantized type, one per call
        kv8 = L.sd_kv_append_q8_0
        assert kv8(FAKE, FAKE, 1024, ok, 1, 8, 100, None) == SD_EINVAL      # D % 32
        assert L.sd_kv_append_f16(FAKE, FAKE, 1024, ok, 1, 8, 128, None) == SD_EINVAL
        pair = (_lib.SeqView * 2)(view(t), view(1))
        assert kv8(FAKE, FAKE, 1024, pair, 2, 8, 128, None) == SD_EUNSUPPORTED


def test_rope_kv_and_glue_rejections(L):
    r = L.sd_rope_posvec
    assert r(FAKE, 4, 32, 128, 4096, 128, FAKE, 1e6, 127, None) == SD_EINVAL
    assert r(FAKE, 4, 32, 128, 4096, 128, FAKE, 1e6, 130, None) == SD_EINVAL
    assert r(FAKE, 4, 32, 128, 4096, 128, FAKE, -1.0, 128, None) == SD_EINVAL
    assert r(ODD, 4, 32, 128, 4096, 128, FAKE, 1e6, 128, None) == SD_EALIGN
    v1 = (_lib.SeqView * 1)(_view(3, 2))
    assert L.sd_kv_append_f16(FAKE, FAKE, 1024, v1, 1, 8, 128, None) == SD_EINVAL
    assert L.sd_rmsnorm_q8(FAKE, 100, 1, 100, FAKE, 1e-6, FAKE, FAKE, None, None) == SD_EUNSUPPORTED
    assert L.sd_rmsnorm_q8(FAKE, 128, 1, 128, FAKE, -1.0, FAKE, FAKE, None, None) == SD_EINVAL
    assert L.sd_swiglu_q8(FAKE, 100, 1, 64, FAKE, FAKE, None, None) == SD_EINVAL
    assert L.sd_argmax_rows(FAKE, 10, 1, 11, FAKE, FAKE, 64, None) == SD_EINVAL
    assert L.sd_argmax_workspace_bytes(4, 151936) == 4 * 19 * 8
    assert L.sd_argmax_rows(FAKE, 151936, 4, 151936, FAKE, FAKE, 4 * 19 * 8 - 1, None) == SD_EWORKSPACE
    assert L.sd_embed_f16(FAKE, 0, 16, FAKE, 1, FAKE, None) == SD_EINVAL


def test_step_rejections(L):
    lw = (_lib.LayerWeights * 1)(_lib.LayerWeights(*([FAKE.value] * 6)))
    m = _lib.Model(1, 4096, 32, 8, 128, 14336, 1000, 1e-6, 1e6, FAKE.value, FAKE.value,
                   FAKE.value, ctypes.cast(lw, ctypes.c_void_p))
    need = L.sd_decode_step_workspace_bytes(ctypes.byref(m), 4, 32768)
    assert need > 0
    assert L.sd_decode_step_workspace_bytes(ctypes.byref(m), 17, 32768) == 0   # rows <= 16
    assert L.sd_decode_step_workspace_bytes(ctypes.byref(m), 16, 32768) > need
    bad = _lib.Model(1, 4096, 32, 8, 64, 14336, 1000, 1e-6, 1e6, FAKE.value, FAKE.value,
                     FAKE.value, ctypes.cast(lw, ctypes.c_void_p))
    assert L.sd_decode_step_workspace_bytes(ctypes.byref(bad), 1, 16) == 0
    seqs = (_lib.StepSeq * 1)(_lib.StepSeq(FAKE.value, FAKE.value, 16, 16))   # pos == capacity
    io = _lib.StepIO(1, ctypes.cast(seqs, ctypes.c_void_p), FAKE.value, FAKE.value, FAKE.value,
                     FAKE.value, 0x100000, 1 << 30)
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io), None) == SD_EINVAL
    assert L.sd_decode_step(ctypes.byref(bad), ctypes.byref(io), None) == SD_EUNSUPPORTED
    seqs[0].pos = 13
    seqs[0].n_new = 4                 # positions 13..16 do not fit capacity 16
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io), None) == SD_EINVAL
    seqs[0].n_new = 5                 # more than SD_ATTN_MAX_NEW
    seqs[0].pos = 3
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io), None) == SD_EINVAL
    seqs[0].n_new = 4
    io.ws_bytes = 16
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io), None) == SD_EWORKSPACE
    paged = (_lib.StepSeq * 1)(_lib.StepSeq(FAKE.value, FAKE.value, 256, 1000, 4, 0, FAKE.value, 64))
    iop = _lib.StepIO(1, ctypes.cast(paged, ctypes.c_void_p), FAKE.value, FAKE.value, FAKE.value,
                      FAKE.value, 0x100000, 16)
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(iop), None) == SD_EWORKSPACE  # pos past pool ok
    for bs, cap, ring, table, rc in ((48, 256, 0, FAKE, SD_EINVAL), (64, 200, 0, FAKE, SD_EINVAL),
                                     (64, 256, 1, FAKE, SD_EINVAL), (64, 256, 0, ODD, SD_EALIGN)):
        paged[0].block_size, paged[0].capacity, paged[0].ring = bs, cap, ring
        paged[0].block_table = table.value
        assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(iop), None) == rc
    q8 = (_lib.StepSeq * 2)(_lib.StepSeq(0, 0, 256, 10, 1, 0, None, 0, 1, FAKE.value, FAKE.value,
                                         FAKE.value, FAKE.value),
                            _lib.StepSeq(0, 0, 256, 10, 1, 0, None, 0, 1, FAKE.value, FAKE.value,
                                         FAKE.value, FAKE.value))
    io8 = _lib.StepIO(2, ctypes.cast(q8, ctypes.c_void_p), FAKE.value, FAKE.value, FAKE.value,
                      FAKE.value, 0x100000, 16)
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io8), None) == SD_EWORKSPACE
    q8[1].kv_type = 0                 # one kv_type per step
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io8), None) == SD_EUNSUPPORTED
    q8[1].kv_type = 3                 # Q4/Q8 beside Q8/Q8
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io8), None) == SD_EUNSUPPORTED
    q8[1].kv_type = 5                 # unknown type
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io8), None) == SD_EINVAL
    q8[1].kv_type = 1
    q8[1].k_d = 0x10004               # scales need 8-byte alignment
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io8), None) == SD_EALIGN
    q8[1].k_d = 0
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io8), None) == SD_EINVAL
    five = (_lib.StepSeq * 5)(*[_lib.StepSeq(FAKE.value, FAKE.value, 64, 3, 4) for _ in range(5)])
    io5 = _lib.StepIO(5, ctypes.cast(five, ctypes.c_void_p), FAKE.value, FAKE.value, FAKE.value,
                      FAKE.value, 0x100000, 1 << 30)
    assert L.sd_decode_step(ctypes.byref(m), ctypes.byref(io5), None) == SD_EINVAL
