"""The C ABI: libmbd loads, exports every function include/mbd.h declares, and
rejects bad arguments with the documented status before touching a GPU (every
call here fails validation on the host, so no device work is ever enqueued)."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
mbd = pytest.importorskip("memory_bound_decode_amd")


@pytest.fixture(scope="module")
def L():
    try:
        return mbd.lib()
    except ImportError as e:                         # pragma: no cover
        pytest.skip(str(e))


def _declared():
    src = open(os.path.join(ROOT, "include", "mbd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mbd_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    from memory_bound_decode_amd import _native
    assert set(names) == set(_native.SIGNATURES)


def test_status_strings(L):
    for s in range(8):
        assert L.mbd_status_str(s)
    assert L.mbd_status_str(99) == b"unknown status"


def _pack_raw(L, fmt, w, M, K, norm=None):
    h = ctypes.c_void_p()
    st = L.mbd_pack(fmt, None if w is None else w.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
                    M, K, None if norm is None else norm.ctypes.data, None, ctypes.byref(h))
    if h.value:
        L.mbd_packed_free(h)
    return st


def test_pack_errors(L):
    w = np.zeros((4, 128), np.uint16)
    assert _pack_raw(L, mbd.MBD_INT4_G128, None, 4, 128) == mbd.MBD_EINVAL
    assert _pack_raw(L, 99, w, 4, 128) == mbd.MBD_EINVAL
    assert _pack_raw(L, mbd.MBD_INT4_G128, w, 4, 100) == mbd.MBD_ESHAPE
    assert _pack_raw(L, mbd.MBD_INT4_G128, w, 0, 128) == mbd.MBD_ESHAPE
    assert _pack_raw(L, mbd.MBD_MX32, np.zeros((2, 96), np.uint16), 2, 96) == mbd.MBD_OK
    assert _pack_raw(L, mbd.MBD_CASSANDRA, w, 4, 128) == mbd.MBD_EINVAL        # no act_norm
    bad = w.copy()
    bad[1, 7] = 0x7F80                                                          # +Inf
    assert _pack_raw(L, mbd.MBD_TERNARY_B128, bad, 4, 128) == mbd.MBD_ERANGE
    assert _pack_raw(L, mbd.MBD_MX32, bad, 4, 128) == mbd.MBD_ERANGE
    big = np.full((1, 128), 0x7F00, np.uint16)                                  # 2^127: scale overflows fp16
    assert _pack_raw(L, mbd.MBD_INT4_G128, big, 1, 128) == mbd.MBD_ERANGE
    nrm = np.ones(128, np.float32)
    nrm[3] = np.nan
    assert _pack_raw(L, mbd.MBD_CASSANDRA, w, 4, 128, nrm) == mbd.MBD_ERANGE
    assert L.mbd_last_error()


def test_validate_detects_corruption(L):
    w = np.zeros((2, 256), np.uint16)
    p = mbd.mbd_pack(mbd.MBD_TERNARY_B128, w)
    p.validate()
    secs = (mbd.MbdSection * 4)()
    n = ctypes.c_int32()
    assert L.mbd_packed_sections(p._h, secs, 4, ctypes.byref(n)) == mbd.MBD_OK
    codes = (ctypes.c_uint32 * 1).from_address(secs[0].data)
    codes[0] = 0xFFFFFFFF                                                       # code 3 is invalid
    with pytest.raises(mbd.MbdError) as e:
        p.validate()
    assert e.value.status == mbd.MBD_EFORMAT

    rng = np.random.default_rng(0)
    wc = synth_w = (rng.standard_normal((2, 256)) * 0.02).astype(np.float32)
    import synth
    wc = synth.f32_to_bf16_bits(synth_w)
    pc = mbd.mbd_pack(mbd.MBD_CASSANDRA, wc, np.ones(256, np.float32))
    pc.validate()
    secs = (mbd.MbdSection * 8)()
    assert L.mbd_packed_sections(pc._h, secs, 8, ctypes.byref(n)) == mbd.MBD_OK
    kp = (ctypes.c_uint32 * 2).from_address(secs[5].data)
    kp[1] += 1                                                                  # kept prefix off by one
    with pytest.raises(mbd.MbdError) as e:
        pc.validate()
    assert e.value.status == mbd.MBD_EFORMAT

    ws = synth.f32_to_bf16_bits((rng.standard_normal((20, 384)) * 0.02).astype(np.float32))
    ws[3, 128:256] = 0                                                          # one all-zero block
    ps = mbd.mbd_pack(mbd.MBD_TERNARY_SKIP, ws)
    ps.validate()
    secs = (mbd.MbdSection * 4)()
    assert L.mbd_packed_sections(ps._h, secs, 4, ctypes.byref(n)) == mbd.MBD_OK
    assert secs[0].bytes == 32 * (20 * 3 - 1)
    slabs = (ctypes.c_uint32 * 6).from_address(secs[2].data)
    assert slabs[1] & 0xFFFF == 0xFFFF & ~(1 << 3)
    slabs[1] |= 1 << 3                                                          # flag says stored, table disagrees
    with pytest.raises(mbd.MbdError) as e:
        ps.validate()
    assert e.value.status == mbd.MBD_EFORMAT


def _desc(fmt, M, K, n_sym=0, ptr=0x1000, n_mats=1):
    d = mbd.MbdDWeights()
    d.fmt, d.M, d.K, d.n_sym, d.n_mats = fmt, M, K, n_sym, n_mats
    for i in range(mbd._native.MBD_MAX_SECTIONS):
        d.sec[i] = ptr
    return d


P16 = ctypes.c_void_p(0x10000)     # fake, never dereferenced: validation fails first


def test_gemv_argument_errors(L):
    d = _desc(mbd.MBD_INT4_G128, 16, 256)
    assert L.mbd_gemv(None, P16, 1, P16, None) == mbd.MBD_EINVAL
    assert L.mbd_gemv(ctypes.byref(d), None, 1, P16, None) == mbd.MBD_EINVAL
    assert L.mbd_gemv(ctypes.byref(d), P16, 0, P16, None) == mbd.MBD_ESHAPE
    assert L.mbd_gemv(ctypes.byref(d), P16, 17, P16, None) == mbd.MBD_ESHAPE
    assert L.mbd_gemv(ctypes.byref(d), ctypes.c_void_p(0x10008), 1, P16, None) == mbd.MBD_EALIGN
    d.K = 200
    assert L.mbd_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_ESHAPE
    d.K = 256
    d.fmt = 42
    assert L.mbd_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_EINVAL
    d = _desc(mbd.MBD_INT4_G128, 16, 256, ptr=0x10004)
    assert L.mbd_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_EALIGN
    d = _desc(mbd.MBD_MX32, 16, 48)
    assert L.mbd_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_ESHAPE
    # codes addressed with 32-bit byte offsets: a matrix whose codes reach 4 GiB is refused
    for fmt, M in ((mbd.MBD_INT4_G128, 1 << 20), (mbd.MBD_TERNARY_B128, 1 << 21)):
        for B in (1, 8):
            d = _desc(fmt, M, 8192)
            assert L.mbd_gemv(ctypes.byref(d), P16, B, P16, None) == mbd.MBD_ESHAPE
            assert b"4 GiB" in L.mbd_last_error()
    # batch 5..16 addresses the activations with 32-bit element offsets: B K >= 2^32 is refused
    for fmt in (mbd.MBD_INT4_G128, mbd.MBD_TERNARY_B128):
        d = _desc(fmt, 16, 1 << 28)
        assert L.mbd_gemv(ctypes.byref(d), P16, 16, P16, None) == mbd.MBD_ESHAPE
        assert b"2^32" in L.mbd_last_error()


def test_skip_format_argument_errors(L):
    d = _desc(mbd.MBD_TERNARY_SKIP, 16, 256, ptr=0x10000)
    d.n_mats = 2
    assert L.mbd_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_EINVAL    # one matrix only
    d.n_mats = 1
    d.sec[3] = None
    assert L.mbd_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_EINVAL    # tile_base missing
    assert L.mbd_dequant(ctypes.byref(d), P16, None) == mbd.MBD_EINVAL
    d.sec[3] = 0x10000
    d.sec[2] = 0x10002
    assert L.mbd_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_EALIGN    # slabs 4-byte aligned
    d.sec[2] = 0x10000
    d.K = 128 * 4097
    assert L.mbd_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_ESHAPE    # 16-bit in-tile offset
    d.K = 200
    assert L.mbd_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_ESHAPE
    e = _desc(mbd.MBD_TERNARY_SKIP, 64, 256)
    assert L.mbd_moe_gemv(ctypes.byref(e), P16, 1, 1, P16, 0, P16, P16, 1 << 20, None) == mbd.MBD_EINVAL


def test_cassandra_mx_argument_errors(L):
    d = _desc(mbd.MBD_CASSANDRA_MX, 16, 256, ptr=0x10000)
    assert L.mbd_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_EINVAL    # speculation data only
    assert L.mbd_spec_gemv(ctypes.byref(d), P16, 17, P16, None) == mbd.MBD_ESHAPE
    d.sec[4] = None
    assert L.mbd_spec_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_EINVAL  # kprefix missing
    assert L.mbd_spec_decode(ctypes.byref(d), P16, None) == mbd.MBD_EINVAL
    d.sec[4] = 0x10008
    assert L.mbd_spec_gemv(ctypes.byref(d), P16, 1, P16, None) == mbd.MBD_EALIGN
    d.sec[4] = 0x10000
    d.K = 200
    assert L.mbd_spec_decode(ctypes.byref(d), P16, None) == mbd.MBD_ESHAPE


def test_encoder_argument_errors(L):
    n = ctypes.c_uint64()
    assert L.mbd_encode_workspace_bytes(0, ctypes.byref(n)) == mbd.MBD_ESHAPE
    assert L.mbd_encode_workspace_bytes(8, ctypes.byref(n)) == mbd.MBD_OK and n.value >= 8 * 8
    plan = mbd.MbdEncodePlan()
    args = lambda M, K, ws, wsb, w=P16: L.mbd_encode_plan(w, P16, M, K, 3, 10, ws, wsb, ctypes.byref(plan), None)
    assert args(8, 256, P16, n.value, w=None) == mbd.MBD_EINVAL
    assert args(8, 200, P16, n.value) == mbd.MBD_ESHAPE                             # K % 128
    assert args(8, 256, P16, 16) == mbd.MBD_EINVAL                                  # workspace too small
    assert args(8, 256, ctypes.c_void_p(0x10008), n.value) == mbd.MBD_EALIGN
    assert L.mbd_encode_plan(P16, P16, 8, 256, 3, 10, P16, n.value, None, None) == mbd.MBD_EINVAL
    # every call below fails validation before anything is enqueued (fake pointers)
    secs = (ctypes.c_void_p * 8)(*([0x10000] * 8))
    plan.n_kept, plan.n_tiles = 8 * 76 + 1, 1                                       # a plan of another shape
    assert L.mbd_encode_cassandra(P16, P16, 8, 256, 3, 10, ctypes.byref(plan), secs, P16, n.value, None) == mbd.MBD_EINVAL
    plan.n_kept = 8 * 76
    secs[2] = None                                                                  # unary buffer missing
    assert L.mbd_encode_cassandra(P16, P16, 8, 256, 3, 10, ctypes.byref(plan), secs, P16, n.value, None) == mbd.MBD_EINVAL
    secs[2] = 0x10008
    assert L.mbd_encode_cassandra(P16, P16, 8, 256, 3, 10, ctypes.byref(plan), secs, P16, n.value, None) == mbd.MBD_EALIGN


def test_cassandra_and_moe_argument_errors(L):
    d = _desc(mbd.MBD_CASSANDRA, 16, 256, n_sym=0)
    d.n_kept = 5
    assert L.mbd_spec_decode(ctypes.byref(d), P16, None) == mbd.MBD_EINVAL      # kept values, no codebook
    d.n_sym = 300
    assert L.mbd_spec_decode(ctypes.byref(d), P16, None) == mbd.MBD_EINVAL
    d.n_sym = 12
    d.sec[2] = None
    assert L.mbd_spec_decode(ctypes.byref(d), P16, None) == mbd.MBD_EINVAL
    d.sec[2] = 0x10000
    assert L.mbd_spec_gemv(ctypes.byref(d), P16, 20, P16, None) == mbd.MBD_ESHAPE
    d.sec[7] = None                                                             # verification data missing
    assert L.mbd_verify_restore(ctypes.byref(d), P16, None) == mbd.MBD_EINVAL
    d = _desc(mbd.MBD_CASSANDRA, 16, 1536, n_sym=12)
    assert L.mbd_gemv(ctypes.byref(d), P16, 16, P16, None) == mbd.MBD_ESHAPE    # K % 4096 != 0
    e = _desc(mbd.MBD_TERNARY_B128, 64, 256, n_mats=8)
    need = ctypes.c_uint64()
    assert L.mbd_moe_workspace_bytes(8, 2, 4, ctypes.byref(need)) == mbd.MBD_OK and need.value > 0
    assert L.mbd_moe_workspace_bytes(0, 2, 4, ctypes.byref(need)) == mbd.MBD_ESHAPE
    assert L.mbd_moe_gemv(ctypes.byref(e), P16, 2, 4, P16, 0, P16, P16, 1, None) == mbd.MBD_EINVAL  # ws too small
    e.fmt = mbd.MBD_CASSANDRA
    assert L.mbd_moe_gemv(ctypes.byref(e), P16, 2, 4, P16, 0, P16, P16, need.value, None) == mbd.MBD_EINVAL


def test_moe_noalloc_argument_errors(L):
    """The allocation-free expert GEMV refuses routes whose grouping tables exceed its
    1 MiB static scratch, and NULL arguments, before any HIP call."""
    e = _desc(mbd.MBD_TERNARY_B128, 64, 256, n_mats=64)
    assert L.mbd_moe_gemv_noalloc(None, P16, 2, 4, P16, 0, P16, None) == mbd.MBD_EINVAL
    assert L.mbd_moe_gemv_noalloc(ctypes.byref(e), None, 2, 4, P16, 0, P16, None) == mbd.MBD_EINVAL
    need = ctypes.c_uint64()
    T_ok, T_big = 1024, 8192                          # 8192 pairs fit; 65536 pairs need about 2.3 MiB
    assert L.mbd_moe_workspace_bytes(64, T_ok, 8, ctypes.byref(need)) == mbd.MBD_OK and need.value <= 1 << 20
    assert L.mbd_moe_workspace_bytes(64, T_big, 8, ctypes.byref(need)) == mbd.MBD_OK and need.value > 1 << 20
    assert L.mbd_moe_gemv_noalloc(ctypes.byref(e), P16, T_big, 8, P16, 0, P16, None) == mbd.MBD_ESHAPE
    assert b"scratch" in L.mbd_last_error()
    assert L.mbd_moe_gemv_noalloc(ctypes.byref(e), P16, 2, 0, P16, 0, P16, None) == mbd.MBD_ESHAPE   # k = 0
    # one expert matrix's codes and scales are addressed with 32-bit offsets: 4 GiB of
    # codes per matrix is refused, on both entry points
    big = _desc(mbd.MBD_INT4_G128, 1 << 20, 8192, n_mats=2)
    assert L.mbd_moe_gemv_noalloc(ctypes.byref(big), P16, 1, 2, P16, 0, P16, None) == mbd.MBD_ESHAPE
    assert b"4 GiB" in L.mbd_last_error()
    assert L.mbd_moe_gemv(ctypes.byref(big), P16, 1, 2, P16, 0, P16, P16, 1 << 20, None) == mbd.MBD_ESHAPE
    assert b"4 GiB" in L.mbd_last_error()
    # with T > 1 the activations are addressed with 32-bit element offsets: x's rows
    # (T k with x_per_pair) times K of 2^32 or more is refused, on both entry points
    wide = _desc(mbd.MBD_TERNARY_B128, 1, 1 << 30, n_mats=2)
    assert L.mbd_moe_gemv(ctypes.byref(wide), P16, 2, 2, P16, 1, P16, P16, 1 << 20, None) == mbd.MBD_ESHAPE
    assert b"2^32" in L.mbd_last_error()
    assert L.mbd_moe_gemv_noalloc(ctypes.byref(wide), P16, 2, 2, P16, 1, P16, None) == mbd.MBD_ESHAPE
    assert b"2^32" in L.mbd_last_error()
