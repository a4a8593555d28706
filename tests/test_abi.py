"""CPU-side checks of the C ABI: exports, the host codebook and QJL matrix
against the reference, argument validation and workspace sizing. None of
these calls reaches the GPU (every path returns before a HIP call)."""

import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O
from tests.conftest import ROOT

tq = pytest.importorskip("kv_cache_vector_07_amd.tq")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(tq._LIB_PATH):
        from kv_cache_vector_07_amd import build
        build.build()
    return tq.lib()


def _header_functions():
    with open(os.path.join(ROOT, "include", "tq.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char \*)\s*(tq_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol(L):
    declared = _header_functions()
    assert set(declared) == set(tq.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_page_bytes(L):
    for d in (128, 256):
        assert tq.tq_k_page_bytes(d) == O.k_page_bytes(d, 256)
        assert tq.tq_v_page_bytes(d) == O.v_page_bytes(d, 256)
        assert tq.tq_k_page_bytes(d) % 256 == 0 and tq.tq_v_page_bytes(d) % 256 == 0
    assert L.tq_k_page_bytes(100, 256) == 0


@pytest.mark.parametrize("d", [8, 128, 256])
def test_host_codebook_matches_reference_bitwise(L, d):
    levels, thr, S = tq.tq_build_codebook(d, 3, 12345)
    cb = O.codebook(d)
    assert np.array_equal(levels.astype(np.float64), cb.levels)
    assert np.array_equal(thr.astype(np.float64), cb.thresholds)
    assert np.array_equal(S, O.qjl_matrix(d, 12345))


def test_codebook_errors(L):
    lv, th = np.zeros(16, np.float32), np.zeros(15, np.float32)
    assert L.tq_build_codebook(128, 5, 1, lv.ctypes.data, th.ctypes.data, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_build_codebook(128, 1, 1, lv.ctypes.data, th.ctypes.data, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_build_codebook(100, 3, 1, lv.ctypes.data, th.ctypes.data, None) == tq.TQ_EINVAL
    assert L.tq_build_codebook(128, 3, 1, None, th.ctypes.data, None) == tq.TQ_EINVAL
    assert L.tq_status_string(tq.TQ_EWORKSPACE) == b"workspace too small"


def _desc(d=128, H=2, P=256, pages=4, k=0x100000, v=0x200000, s=0x300000):
    levels, thr, _ = tq.tq_build_codebook(d if d in (128, 256) else 128, 3, 1, with_qjl=False)
    return tq.TqCacheDesc(d, H, P, pages, k, v, s, (C.c_float * 8)(*levels.tolist()),
                          (C.c_float * 7)(*thr.tolist()))


FAKE = 0x400000  # 256-aligned non-null host address, never dereferenced on these paths


def test_encode_validation(L):
    dsc = _desc()
    r = C.byref(dsc)
    assert L.tq_encode_k(None, FAKE, 0, FAKE, 4, None) == tq.TQ_EINVAL
    assert L.tq_encode_k(r, FAKE, 0, FAKE, -1, None) == tq.TQ_EINVAL
    assert L.tq_encode_k(r, FAKE, 7, FAKE, 4, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_encode_k(r, FAKE, 0, FAKE, 0, None) == tq.TQ_OK          # empty: no-op
    assert L.tq_encode_k(r, None, 0, FAKE, 4, None) == tq.TQ_EINVAL
    assert L.tq_encode_k(r, FAKE + 4, 0, FAKE, 4, None) == tq.TQ_EALIGN
    assert L.tq_encode_v(r, FAKE, 1, None, 4, None) == tq.TQ_EINVAL
    for bad in (_desc(d=64), _desc(P=128)):
        assert L.tq_encode_v(C.byref(bad), FAKE, 0, FAKE, 4, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_encode_v(C.byref(_desc(k=0x100010)), FAKE, 0, FAKE, 4, None) == tq.TQ_EALIGN
    assert L.tq_encode_v(C.byref(_desc(H=0)), FAKE, 0, FAKE, 4, None) == tq.TQ_EINVAL
    assert L.tq_encode_k(C.byref(_desc(s=0)), FAKE, 0, FAKE, 4, None) == tq.TQ_EINVAL


def test_dequant_and_prepare_validation(L):
    r = C.byref(_desc())
    assert L.tq_dequant(r, 2, 0, FAKE, 4, FAKE, None) == tq.TQ_EINVAL
    assert L.tq_dequant(r, 0, 3, FAKE, 4, FAKE, None) == tq.TQ_EINVAL
    assert L.tq_dequant(r, 1, 0, FAKE, 0, FAKE, None) == tq.TQ_OK
    assert L.tq_dequant(r, 1, 0, FAKE, 4, FAKE + 8, None) == tq.TQ_EALIGN
    sz = C.c_size_t(0)
    assert L.tq_query_prepare(r, FAKE, 0, 2, 1, 8, None, C.byref(sz), None) == tq.TQ_OK
    need = sz.value
    # rows of (Pi q, S Pi q) plus the packed operands of the 2 x 2 (sequence, KV head)
    # groups: 5 scoring MFMAs per 128 coordinates, each with 32 query bytes and a
    # scale word per lane, then 4 x 4 row constants
    grp = 5 * (64 * 32 + 64 * 4) + 64
    assert need >= 2 * 8 * 2 * 128 * 4 + 4 * grp
    sz = C.c_size_t(need - 1)
    assert L.tq_query_prepare(r, FAKE, 0, 2, 1, 8, FAKE, C.byref(sz), None) == tq.TQ_EWORKSPACE
    assert sz.value == need
    sz = C.c_size_t(need)
    assert L.tq_query_prepare(r, FAKE, 5, 2, 1, 8, FAKE, C.byref(sz), None) == tq.TQ_EUNSUPPORTED
    assert L.tq_query_prepare(r, None, 0, 2, 1, 8, FAKE, C.byref(sz), None) == tq.TQ_EINVAL
    assert L.tq_query_prepare(r, FAKE, 0, 2, 1, 7, FAKE, C.byref(sz), None) == tq.TQ_EINVAL
    assert L.tq_query_prepare(r, FAKE, 0, 2, 1, 8, FAKE + 16, C.byref(sz), None) == tq.TQ_EALIGN
    assert L.tq_query_prepare(r, FAKE, 0, 2, 1, 8, FAKE, None, None) == tq.TQ_EINVAL
    # 16 rows per KV head (3-bit K and V): one wide query group per (sequence, KV
    # head), whose operand holds each of the 5 scoring MFMAs once per fp6 limb
    # (4 x 5 operands, 32 query bytes and a scale word per lane each), then 16 x 2
    # row constants
    sz16 = C.c_size_t(0)
    assert L.tq_query_prepare(r, FAKE, 0, 2, 2, 16, None, C.byref(sz16), None) == tq.TQ_OK
    wide = 4 * 5 * (64 * 32 + 64 * 4) + 16 * 2 * 4
    assert sz16.value == 2 * 2 * 16 * 2 * 128 * 4 + (2 * 2 * 1 * wide + 255) // 256 * 256


def _decode(L, dsc, ws=None, size=None, B=2, nq=1, Hq=8, maxp=16, causal=0, q=FAKE):
    sz = C.c_size_t(0 if size is None else size)
    st = L.tq_attn_decode(C.byref(dsc), q, 1, B, nq, Hq, FAKE, maxp, FAKE, causal, 0.1, FAKE,
                          ws, C.byref(sz), None)
    return st, sz.value


def test_decode_validation_and_workspace(L):
    dsc = _desc(H=2)
    st, need = _decode(L, dsc)
    assert st == tq.TQ_OK and need > 0 and need % 256 == 0
    st2, need2 = _decode(L, dsc, ws=FAKE, size=need - 1)
    assert st2 == tq.TQ_EWORKSPACE and need2 == need
    # prepared variant needs no query region
    sz = C.c_size_t(0)
    assert L.tq_attn_decode_prepared(C.byref(dsc), FAKE, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, FAKE,
                                     None, C.byref(sz), None) == tq.TQ_OK
    assert 0 < sz.value < need
    assert _decode(L, dsc, Hq=7)[0] == tq.TQ_EINVAL                # Hq not a multiple of Hkv
    assert _decode(L, dsc, Hq=8, nq=1025)[0] == tq.TQ_EUNSUPPORTED   # 4 * 1025 rows > 4096
    assert _decode(L, dsc, Hq=8, nq=1024)[0] == tq.TQ_OK
    # batch x workgroups per sequence must fit the third grid dimension (65535):
    # 4096 rows per KV head are 256 wide groups of 16 rows
    assert _decode(L, dsc, B=255, Hq=8, nq=1024)[0] == tq.TQ_OK
    assert _decode(L, dsc, B=256, Hq=8, nq=1024)[0] == tq.TQ_EUNSUPPORTED
    assert _decode(L, dsc, causal=2)[0] == tq.TQ_EINVAL
    assert _decode(L, dsc, B=0)[0] == tq.TQ_EINVAL
    assert _decode(L, dsc, maxp=0)[0] == tq.TQ_EINVAL
    sz = C.c_size_t(0)
    assert L.tq_attn_decode(C.byref(dsc), FAKE, 1, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, FAKE, None,
                            None, None) == tq.TQ_EINVAL
    st, _ = _decode(L, dsc, ws=FAKE + 16, size=need)
    assert st == tq.TQ_EALIGN


def test_split_and_merge_validation(L):
    dsc = _desc(H=2)
    r = C.byref(dsc)
    sz = C.c_size_t(0)
    assert L.tq_attn_decode_split(r, FAKE, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, None, C.byref(sz),
                                  None) == tq.TQ_OK
    need = sz.value
    sz2 = C.c_size_t(0)
    assert L.tq_attn_decode_prepared(r, FAKE, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, FAKE, None,
                                     C.byref(sz2), None) == tq.TQ_OK
    assert need == sz2.value
    small = C.c_size_t(need - 256)
    assert L.tq_attn_decode_split(r, FAKE, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, FAKE, C.byref(small),
                                  None) == tq.TQ_EWORKSPACE
    assert L.tq_attn_decode_merge(r, 2, 1, 8, 16, FAKE, FAKE, need - 256, None) == tq.TQ_EWORKSPACE
    assert L.tq_attn_decode_merge(r, 2, 1, 8, 16, None, FAKE, need, None) == tq.TQ_EINVAL
    assert L.tq_attn_decode_merge(r, 2, 1, 7, 16, FAKE, FAKE, need, None) == tq.TQ_EINVAL
    assert L.tq_attn_decode_merge(r, 2, 1, 8, 16, FAKE + 4, FAKE, need, None) == tq.TQ_EALIGN


def test_append_decode_validation(L):
    dsc = _desc(H=2)
    r = C.byref(dsc)
    args = lambda ws, n_new=4, kdt=1, qdt=1, k=FAKE, q=FAKE: (
        r, k, FAKE, kdt, FAKE, n_new, q, qdt, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, FAKE, ws)
    sz = C.c_size_t(0)
    assert L.tq_append_decode(*args(None), C.byref(sz), None) == tq.TQ_OK
    need = sz.value
    sz2 = C.c_size_t(0)
    assert L.tq_attn_decode(r, FAKE, 1, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, FAKE, None, C.byref(sz2),
                            None) == tq.TQ_OK
    assert need == sz2.value
    small = C.c_size_t(need - 256)
    assert L.tq_append_decode(*args(FAKE), C.byref(small), None) == tq.TQ_EWORKSPACE
    ok = C.c_size_t(need)
    assert L.tq_append_decode(*args(FAKE, kdt=3), C.byref(ok), None) == tq.TQ_EUNSUPPORTED
    assert L.tq_append_decode(*args(FAKE, n_new=-1), C.byref(ok), None) == tq.TQ_EINVAL
    assert L.tq_append_decode(*args(FAKE, k=None), C.byref(ok), None) == tq.TQ_EINVAL
    assert L.tq_append_decode(*args(FAKE, q=None), C.byref(ok), None) == tq.TQ_EINVAL
    assert L.tq_append_decode(*args(FAKE, k=FAKE + 4), C.byref(ok), None) == tq.TQ_EALIGN
    assert L.tq_append_decode(*args(FAKE + 16), C.byref(ok), None) == tq.TQ_EALIGN


def test_window_decode_validation(L):
    dsc = _desc(H=2)
    _, need = _decode(L, dsc)
    sz = C.c_size_t(0)
    # the window variant needs the same workspace as the plain call
    assert L.tq_attn_decode_window(C.byref(dsc), FAKE, 1, 2, 1, 8, FAKE, 16, FAKE, FAKE, 0, 0.1,
                                   FAKE, None, C.byref(sz), None) == tq.TQ_OK
    assert sz.value == need
    assert L.tq_attn_decode_window(C.byref(dsc), FAKE, 1, 2, 1, 8, FAKE, 16, FAKE, None, 0, 0.1,
                                   FAKE, None, C.byref(sz), None) == tq.TQ_EINVAL
    sz = C.c_size_t(need)
    assert L.tq_attn_decode_window(C.byref(dsc), FAKE, 1, 2, 1, 8, FAKE, 16, FAKE, FAKE + 2, 0,
                                   0.1, FAKE, FAKE, C.byref(sz), None) == tq.TQ_EALIGN


@pytest.mark.parametrize("d", [4, 8, 128, 256])
def test_host_sphere_codebook_matches_reference_bitwise(L, d):
    levels, thr, S = tq.tq_build_codebook(d, 3, 777, density="sphere")
    cb = O.codebook(d, density="sphere")
    assert np.array_equal(levels.astype(np.float64), cb.levels)
    assert np.array_equal(thr.astype(np.float64), cb.thresholds)
    assert np.array_equal(S, O.qjl_matrix(d, 777))
    lv, th = np.zeros(16, np.float32), np.zeros(15, np.float32)
    assert L.tq_build_codebook_sphere(2, 3, 1, lv.ctypes.data, th.ctypes.data, None) == tq.TQ_EINVAL
    assert L.tq_build_codebook_sphere(128, 5, 1, lv.ctypes.data, th.ctypes.data, None) == tq.TQ_EUNSUPPORTED
    assert L.tq_build_codebook_sphere(96, 3, 1, lv.ctypes.data, th.ctypes.data, None) == tq.TQ_EINVAL


def test_mse_only_keys_validation(L):
    """k_mse_only = 1 needs no QJL matrix; other values are rejected; tq_dequant
    refuses the QJL term on such a cache."""
    dsc = _desc(H=2)
    dsc.qjl = None
    sz = C.c_size_t(0)
    decode = lambda: L.tq_attn_decode(C.byref(dsc), FAKE, 1, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, FAKE,
                                      None, C.byref(sz), None)
    assert decode() == tq.TQ_EINVAL                                      # S needed
    assert L.tq_encode_k(C.byref(dsc), FAKE, 1, FAKE, 4, None) == tq.TQ_EINVAL
    dsc.k_mse_only = 1
    assert decode() == tq.TQ_OK                                          # workspace query
    assert L.tq_dequant(C.byref(dsc), 0, 1, FAKE, 4, FAKE, None) == tq.TQ_EINVAL
    dsc.k_mse_only = 2
    assert L.tq_encode_v(C.byref(dsc), FAKE, 1, FAKE, 4, None) == tq.TQ_EINVAL
    prep = C.c_size_t(0)
    assert L.tq_query_prepare(C.byref(dsc), FAKE, 0, 2, 1, 8, None, C.byref(prep), None) == tq.TQ_EINVAL


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("density", ["gaussian", "sphere"])
def test_host_codebooks_of_other_widths_match_reference(L, bits, density):
    for d in (128, 256):
        levels, thr, _ = tq.tq_build_codebook(d, bits, 1, with_qjl=False, density=density)
        cb = O.codebook(d, bits, density=density)
        assert len(levels) == 1 << bits
        assert np.array_equal(levels.astype(np.float64), cb.levels)
        assert np.array_equal(thr.astype(np.float64), cb.thresholds)


def test_v_widths_page_bytes_and_validation(L):
    for d in (128, 256):
        for b in (2, 3, 4):
            assert tq.tq_v_page_bytes(d, bits=b) == O.v_page_bytes(d, 256, b)
        assert L.tq_v_page_bytes_bits(d, 256, 5) == 0 and L.tq_v_page_bytes_bits(d, 256, 1) == 0
    assert tq.tq_v_page_bytes(128) == L.tq_v_page_bytes(128, 256)
    dsc = _desc(H=2)
    sz = C.c_size_t(0)
    decode = lambda: L.tq_attn_decode(C.byref(dsc), FAKE, 1, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, FAKE,
                                      None, C.byref(sz), None)
    assert decode() == tq.TQ_OK
    dsc.v_bits = 5
    assert decode() == tq.TQ_EINVAL
    dsc.v_bits = 2                                   # v_levels still zero: not increasing
    assert decode() == tq.TQ_EINVAL
    lv, th, _ = tq.tq_build_codebook(128, 2, 1, with_qjl=False)
    for k in range(4):
        dsc.v_levels[k] = float(lv[k])
    assert decode() == tq.TQ_EINVAL                  # v_thresholds still zero: not ascending
    for k in range(3):
        dsc.v_thresholds[k] = float(th[k])
    assert decode() == tq.TQ_OK
    dsc.v_levels[0] = float(lv[0]) * 1.01           # no longer odd
    assert decode() == tq.TQ_EINVAL


def test_k_widths_page_bytes_validation_and_operand_size(L):
    for d in (128, 256):
        for b in (2, 3, 4):
            assert tq.tq_k_page_bytes(d, bits=b) == O.k_page_bytes(d, 256, b)
        assert L.tq_k_page_bytes_bits(d, 256, 5) == 0
    assert tq.tq_k_page_bytes(128) == L.tq_k_page_bytes(128, 256)
    dsc = _desc(H=2)
    sz = C.c_size_t(0)
    decode = lambda: L.tq_attn_decode(C.byref(dsc), FAKE, 1, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, FAKE,
                                      None, C.byref(sz), None)
    assert decode() == tq.TQ_OK
    base = sz.value
    dsc.k_bits = 1
    assert decode() == tq.TQ_EINVAL
    dsc.k_bits = 4                                   # k_levels still zero: not increasing
    assert decode() == tq.TQ_EINVAL
    lv, th, _ = tq.tq_build_codebook(128, 4, 1, with_qjl=False)
    for k in range(16):
        dsc.k_levels[k] = float(lv[k])
    assert decode() == tq.TQ_EINVAL                  # k_thresholds still zero: not ascending
    for k in range(15):
        dsc.k_thresholds[k] = float(th[k])
    assert decode() == tq.TQ_OK
    # the packed scoring operand has 9 MFMA operands per 128 coordinates instead of 5
    grp3 = 5 * (64 * 32 + 64 * 4) + 64
    grp4 = 9 * (64 * 32 + 64 * 4) + 64
    assert sz.value - base == (2 * 2 * 1 * grp4 + 255) // 256 * 256 - (2 * 2 * 1 * grp3 + 255) // 256 * 256


def test_prepare_validates_code_widths_and_codebooks(L):
    """tq_query_prepare checks the descriptor's code widths and codebooks as every
    decode call does: a K width or codebook the kernels cannot take is rejected
    instead of being prepared as 3-bit."""
    dsc = _desc(H=2)
    prep = C.c_size_t(0)
    prepare = lambda: L.tq_query_prepare(C.byref(dsc), FAKE, 0, 2, 1, 8, None, C.byref(prep), None)
    assert prepare() == tq.TQ_OK
    dsc.k_bits = 5
    assert prepare() == tq.TQ_EINVAL
    dsc.k_bits = 4                                   # k_levels still zero: not increasing
    assert prepare() == tq.TQ_EINVAL
    dsc.k_bits = 3
    dsc.levels[0] = dsc.levels[0] * 1.01             # 3-bit codebook no longer odd
    assert prepare() == tq.TQ_EINVAL
    dsc = _desc(H=2)
    dsc.v_bits = 7
    assert prepare() == tq.TQ_EINVAL


def test_static_scratch_entry_rejects_what_the_buffer_cannot_hold(L):
    """tq_append_decode_static returns TQ_ESCRATCH, before any HIP call, when the
    workspace tq_append_decode would need exceeds TQ_STATIC_SCRATCH_BYTES (here a
    1024-token chunk: 4096 query rows per KV head); argument errors come first."""
    dsc = _desc(H=8)
    sz = C.c_size_t(0)
    args = (C.byref(dsc), FAKE, FAKE, 1, FAKE, 1024, FAKE, 1, 1, 1024, 32, FAKE, 16, FAKE, 1, 0.1, FAKE)
    assert L.tq_append_decode(*args, None, C.byref(sz), None) == tq.TQ_OK
    assert sz.value > tq.TQ_STATIC_SCRATCH_BYTES
    assert L.tq_append_decode_static(*args, None) == tq.TQ_ESCRATCH
    assert tq.status_string(tq.TQ_ESCRATCH).startswith("needs more than the static scratch")
    bad = (C.byref(dsc), FAKE, FAKE, 1, FAKE, 1, FAKE, 1, 1, 1, 30, FAKE, 16, FAKE, 0, 0.1, FAKE)
    assert L.tq_append_decode_static(*bad, None) == tq.TQ_EINVAL        # 30 % 8 != 0


def test_thresholds_must_ascend(L):
    """The encoders find a code by binary search over the thresholds, so a
    descriptor whose thresholds do not strictly ascend is rejected."""
    dsc = _desc(H=2)
    sz = C.c_size_t(0)
    decode = lambda: L.tq_attn_decode(C.byref(dsc), FAKE, 1, 2, 1, 8, FAKE, 16, FAKE, 0, 0.1, FAKE,
                                      None, C.byref(sz), None)
    assert decode() == tq.TQ_OK
    t1, t2 = dsc.thresholds[1], dsc.thresholds[2]
    dsc.thresholds[1], dsc.thresholds[2] = t2, t1
    assert decode() == tq.TQ_EINVAL
    assert L.tq_encode_k(C.byref(dsc), FAKE, 1, FAKE, 4, None) == tq.TQ_EINVAL
