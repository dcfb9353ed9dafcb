"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/bsattn.h declares, and rejects bad arguments on the host (before any
HIP call) with the documented error codes."""
import ctypes
import os
import re

import pytest

from block_sparse_attention_mask_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "bsattn.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_attention_mask_amd import build
        build.build()
    return _lib.load()


def declared():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsa_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(L):
    names = declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert sorted(names) == sorted(_lib.EXPORTS)


def test_version_and_strerror(L):
    assert L.bsa_version() >= 1
    for code in (0, -1, -2, -3, -4, -99):
        assert L.bsa_strerror(code)


FAKE = ctypes.c_void_p(4096)   # never dereferenced: the calls fail argument checks first


def test_csr_argument_errors(L):
    n = _lib.I64(0)
    # neither and both sources
    assert L.bsa_csr_count(None, None, 0.5, 4, 2, 2, 1, FAKE, ctypes.byref(n), None) == _lib.BSA_ERR_ARG
    assert L.bsa_csr_count(FAKE, FAKE, 0.5, 4, 2, 2, 1, FAKE, ctypes.byref(n), None) == _lib.BSA_ERR_ARG
    assert L.bsa_csr_count(FAKE, None, 0.5, -1, 2, 2, 1, FAKE, ctypes.byref(n), None) == _lib.BSA_ERR_ARG
    assert L.bsa_csr_count(FAKE, None, 0.5, 4, 2, 2, 1, None, ctypes.byref(n), None) == _lib.BSA_ERR_ARG
    assert L.bsa_csr_count(FAKE, None, 0.5, 1 << 30, 4, 4, 1, FAKE, ctypes.byref(n), None) == \
        _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_csr_count(FAKE, None, 0.5, 4, 3, 2, 1, FAKE, ctypes.byref(n), None) == \
        _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_csr_fill(FAKE, None, 0.5, None, 4, 2, 2, 1, FAKE, FAKE, None, -1, None) == _lib.BSA_ERR_ARG
    assert L.bsa_csr_fill(FAKE, None, 0.5, None, 4, 2, 2, 1, FAKE, None, None, 5, None) == _lib.BSA_ERR_ARG


def test_perm_argument_errors(L):
    assert L.bsa_perm_from_labels(None, 2, 10, 4, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_perm_from_labels(FAKE, 2, 10, 0, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_perm_from_labels(FAKE, 2, 10, 5000, FAKE, None) == _lib.BSA_ERR_UNSUPPORTED
    st = _lib.I64x3(1024, 128, 8)
    bad = _lib.I64x3(1024, 128, 3)
    assert L.bsa_permute_rows(FAKE, ctypes.c_void_p(8192), FAKE, 1, 1, 8, 96, st, st, None) == \
        _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_permute_rows(FAKE, ctypes.c_void_p(8192), FAKE, 1, 1, 8, 128, bad, st, None) == \
        _lib.BSA_ERR_ARG
    assert L.bsa_permute_rows(ctypes.c_void_p(4100), ctypes.c_void_p(8192), FAKE, 1, 1, 8, 128, st, st,
                              None) == _lib.BSA_ERR_ARG
    assert L.bsa_unpermute_rows(FAKE, FAKE, FAKE, 1, 1, 8, 128, st, st, None) == _lib.BSA_ERR_ARG
    dst = _lib.I64x3(128 * 64, 128 * 64, 64)
    D2 = ctypes.c_void_p(1 << 20)
    assert L.bsa_transpose_rows(FAKE, D2, None, 1, 1, 60, 128, 56, st, dst, None) == _lib.BSA_ERR_ARG   # ld < N
    assert L.bsa_transpose_rows(FAKE, D2, None, 1, 1, 60, 128, 62, st, dst, None) == _lib.BSA_ERR_ARG   # ld % 8
    assert L.bsa_transpose_rows(FAKE, D2, None, 1, 1, 60, 128, 128, st, dst, None) == _lib.BSA_ERR_ARG  # ld > row
    assert L.bsa_transpose_rows(FAKE, D2, None, 1, 1, 60, 96, 64, st, dst, None) == _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_transpose_rows(FAKE, FAKE, None, 1, 1, 60, 128, 64, st, dst, None) == _lib.BSA_ERR_ARG


def test_schedule_argument_errors(L):
    assert L.bsa_schedule(None, None, 1, 4, 4, 8, 16, 8, None, 1, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_schedule(FAKE, None, 1, 6, 4, 8, 16, 8, None, 1, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_schedule(FAKE, None, 1, 4, 4, 8, 4096, 8, FAKE, 1, FAKE, None) == _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_schedule(FAKE, None, 1, 4, 4, 8, -1, 8, None, 1, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_schedule(FAKE, None, 1, 4, 4, 8, 16, 8, None, 3, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_schedule(FAKE, None, 1, 4, 4, 8, 16, 8, None, 2, FAKE, None) == _lib.BSA_ERR_ARG   # G = 1
    assert L.bsa_schedule(FAKE, None, 1, 6, 2, 8, 16, 8, None, 2, FAKE, None) == _lib.BSA_ERR_ARG   # G = 3


def test_schedule_pairs_argument_errors(L):
    f = L.bsa_schedule_pairs
    ok = [FAKE, FAKE, None, 1, 4, 4, 8, 0, 8, None, FAKE, FAKE, None]
    for i, bad, code in [(0, None, _lib.BSA_ERR_ARG), (1, None, _lib.BSA_ERR_ARG), (10, None, _lib.BSA_ERR_ARG),
                         (11, None, _lib.BSA_ERR_ARG), (3, 0, _lib.BSA_ERR_ARG), (4, 6, _lib.BSA_ERR_ARG),
                         (7, -1, _lib.BSA_ERR_ARG), (8, 65, _lib.BSA_ERR_ARG), (7, 4096, _lib.BSA_ERR_UNSUPPORTED)]:
        a = list(ok)
        a[i] = bad
        assert f(*a) == code, (i, bad)
    a = list(ok)
    a[4], a[5] = 2048, 1                                   # 2048 query heads per KV head
    assert f(*a) == _lib.BSA_ERR_UNSUPPORTED


def test_pair_rows_equal_argument_errors(L):
    f = L.bsa_pair_rows_equal
    assert f(None, FAKE, None, 1, 4, 2, 8, FAKE, None) == _lib.BSA_ERR_ARG
    assert f(FAKE, None, None, 1, 4, 2, 8, FAKE, None) == _lib.BSA_ERR_ARG
    assert f(FAKE, FAKE, None, 1, 4, 2, 8, None, None) == _lib.BSA_ERR_ARG
    assert f(FAKE, FAKE, None, 1, 4, 2, 0, FAKE, None) == _lib.BSA_ERR_ARG
    assert f(FAKE, FAKE, None, 1, 6, 4, 8, FAKE, None) == _lib.BSA_ERR_ARG            # Hq % Hkv
    assert f(FAKE, FAKE, None, 1, 6, 2, 8, FAKE, None) == _lib.BSA_ERR_UNSUPPORTED    # G = 3


def test_spectral_order_argument_errors(L):
    assert L.bsa_spectral_order(None, FAKE, 4, 100, 100, 10, FAKE, None, None, None) == _lib.BSA_ERR_ARG
    assert L.bsa_spectral_order(FAKE, FAKE, 4, 100, 100, 0, FAKE, None, None, None) == _lib.BSA_ERR_ARG
    assert L.bsa_spectral_order(FAKE, FAKE, 4, 100, 100, 10, None, None, None, None) == _lib.BSA_ERR_ARG
    assert L.bsa_spectral_order(FAKE, FAKE, 0, 100, 100, 10, FAKE, None, None, None) == _lib.BSA_ERR_ARG
    assert L.bsa_spectral_order(FAKE, FAKE, 4, 1025, 100, 10, FAKE, None, None, None) == _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_spectral_order(FAKE, FAKE, 4, 1024, 1024, 10, FAKE, None, None, None) == _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_spectral_order(FAKE, FAKE, 4, 700, 700, 10, FAKE, None, None, None) == _lib.BSA_ERR_UNSUPPORTED


def test_clock_probe_argument_errors(L):
    assert L.bsa_clock_probe(4, 100, 0, None, None) == _lib.BSA_ERR_ARG
    assert L.bsa_clock_probe(0, 100, 1, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_clock_probe(4, 0, 0, FAKE, None) == _lib.BSA_ERR_ARG


def test_crm_argument_errors(L):
    n = _lib.I64(0)
    assert L.bsa_crm_build(None, None, 0.5, 4, 2, 2, 1, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_crm_build(FAKE, FAKE, 0.5, 4, 2, 2, 1, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_crm_build(FAKE, None, 0.5, 4, 2, 2, 1, None, None) == _lib.BSA_ERR_ARG
    assert L.bsa_crm_build(FAKE, None, 0.5, 4, 2, 0, 1, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_crm_build(FAKE, None, 0.5, 1 << 30, 4, 4, 1, FAKE, None) == _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_crm_row_ptr(FAKE, 4, 40, None, ctypes.byref(n), None) == _lib.BSA_ERR_ARG
    assert L.bsa_crm_row_ptr(None, 4, 40, FAKE, ctypes.byref(n), None) == _lib.BSA_ERR_ARG
    assert L.bsa_crm_row_ptr(FAKE, -1, 40, FAKE, ctypes.byref(n), None) == _lib.BSA_ERR_ARG
    assert L.bsa_crm_row_ptr(FAKE, 1 << 30, 40, FAKE, ctypes.byref(n), None) == _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_crm_to_csr(FAKE, 4, 40, FAKE, None, 3, None) == _lib.BSA_ERR_ARG
    assert L.bsa_crm_to_csr(FAKE, 4, 40, FAKE, FAKE, -1, None) == _lib.BSA_ERR_ARG
    assert L.bsa_crm_to_csr(FAKE, 4, 0, FAKE, FAKE, 3, None) == _lib.BSA_ERR_ARG


def test_sampler_argument_errors(L):
    st = _lib.I64x3(1024, 128, 8)
    assert L.bsa_segment_offsets(None, 2, 10, 4, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_segment_offsets(FAKE, 2, 10, 0, FAKE, None) == _lib.BSA_ERR_ARG
    assert L.bsa_segment_offsets(FAKE, 2, 10, 9000, FAKE, None) == _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_segment_means(FAKE, st, 1, 1, 10, 8, None, 0, 0, FAKE, None) == _lib.BSA_ERR_ARG       # no seg_len
    assert L.bsa_segment_means(FAKE, st, 1, 1, 10, 12, None, 0, 4, FAKE, None) == _lib.BSA_ERR_UNSUPPORTED
    assert L.bsa_segment_means(FAKE, _lib.I64x3(1024, 128, 4), 1, 1, 10, 8, None, 0, 4, FAKE, None) == \
        _lib.BSA_ERR_ARG
    assert L.bsa_segment_means(ctypes.c_void_p(4100), st, 1, 1, 10, 8, None, 0, 4, FAKE, None) == \
        _lib.BSA_ERR_UNSUPPORTED
    args = [FAKE, FAKE, FAKE, FAKE, 1, 4, 2, 8, 1000, 64, 128, 2, 3, 0.0, FAKE, FAKE, None, None]
    bad = list(args); bad[0] = None
    assert L.bsa_is_sample(*bad) == _lib.BSA_ERR_ARG
    bad = list(args); bad[5] = 3                   # Hq % Hkv
    assert L.bsa_is_sample(*bad) == _lib.BSA_ERR_ARG
    bad = list(args); bad[12] = -1                 # m_sample < 0
    assert L.bsa_is_sample(*bad) == _lib.BSA_ERR_ARG
    bad = list(args); bad[8] = 64 * 1025           # more than 1024 tiles
    assert L.bsa_is_sample(*bad) == _lib.BSA_ERR_UNSUPPORTED
    bad = list(args); bad[10] = 512                # d > 256
    assert L.bsa_is_sample(*bad) == _lib.BSA_ERR_UNSUPPORTED


def _tok_args(**kw):
    a = _lib.TokArgs()
    a.q, a.k, a.v, a.o = FAKE, ctypes.c_void_p(8192), ctypes.c_void_p(16384), ctypes.c_void_p(32768)
    a.B, a.Hq, a.Hkv, a.d, a.N = 1, 4, 2, 128, 1000
    st = _lib.I64x3(4 * 1000 * 128, 1000 * 128, 128)
    a.q_str = a.k_str = a.v_str = a.o_str = st
    a.n_sets, a.set_size = 4, 64
    a.q_idx, a.kv_ptr, a.kv_idx = FAKE, FAKE, FAKE
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.BSA_ERR_ARG),
    (dict(q_idx=None), _lib.BSA_ERR_ARG),
    (dict(kv_ptr=None), _lib.BSA_ERR_ARG),
    (dict(d=64), _lib.BSA_ERR_UNSUPPORTED),
    (dict(set_size=32), _lib.BSA_ERR_UNSUPPORTED),
    (dict(Hq=3), _lib.BSA_ERR_ARG),
    (dict(N=0), _lib.BSA_ERR_ARG),
    (dict(q=ctypes.c_void_p(4104)), _lib.BSA_ERR_ARG),
    (dict(k_str=_lib.I64x3(4 * 1000 * 128, 1000 * 128, 130)), _lib.BSA_ERR_ARG),
    (dict(o=FAKE), _lib.BSA_ERR_ARG),
    (dict(N=1 << 23), _lib.BSA_ERR_UNSUPPORTED),
    (dict(kv_idx=None), _lib.BSA_ERR_ARG),
    (dict(kv_share=1), _lib.BSA_ERR_ARG),
    (dict(kv_share=2, set_size=128), _lib.BSA_ERR_UNSUPPORTED),
    (dict(kv_share=2, Hkv=4), _lib.BSA_ERR_UNSUPPORTED),                                   # G = 1: no pairs
    (dict(kv_share=3), _lib.BSA_ERR_ARG),
    (dict(kv_share=4), _lib.BSA_ERR_UNSUPPORTED),                                          # G = 2: no quads
    (dict(kv_share=4, Hq=8, Hkv=2, set_size=128), _lib.BSA_ERR_UNSUPPORTED),
])
def test_attn_tok_argument_errors(L, kw, code):
    a = _tok_args(**kw)
    assert L.bsa_attn_tok_fwd(ctypes.byref(a), None) == code
    assert L.bsa_attn_tok_fwd(None, None) == _lib.BSA_ERR_ARG


def _mass_args(**kw):
    a = _lib.MassArgs()
    a.q, a.k, a.lse, a.mass = FAKE, ctypes.c_void_p(8192), ctypes.c_void_p(16384), ctypes.c_void_p(32768)
    a.B, a.Hq, a.Hkv, a.d, a.N = 1, 4, 2, 128, 1000
    a.q_str = a.k_str = _lib.I64x3(4 * 1000 * 128, 1000 * 128, 128)
    a.n_sets, a.set_size = 4, 128
    a.q_idx = FAKE
    a.k0, a.k1 = 0, 1000
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.BSA_ERR_ARG),
    (dict(lse=None), _lib.BSA_ERR_ARG),
    (dict(mass=None), _lib.BSA_ERR_ARG),
    (dict(q_idx=None), _lib.BSA_ERR_ARG),
    (dict(d=64), _lib.BSA_ERR_UNSUPPORTED),
    (dict(set_size=32), _lib.BSA_ERR_UNSUPPORTED),
    (dict(Hq=3), _lib.BSA_ERR_ARG),
    (dict(N=0), _lib.BSA_ERR_ARG),
    (dict(k0=-1), _lib.BSA_ERR_ARG),
    (dict(k1=1001), _lib.BSA_ERR_ARG),
    (dict(k0=600, k1=500), _lib.BSA_ERR_ARG),
    (dict(q=ctypes.c_void_p(4104)), _lib.BSA_ERR_ARG),
    (dict(k_str=_lib.I64x3(4 * 1000 * 128, 1000 * 128, 130)), _lib.BSA_ERR_ARG),
    (dict(N=1 << 23, k1=1 << 23), _lib.BSA_ERR_UNSUPPORTED),
    (dict(k0=500, k1=500), _lib.BSA_OK),       # empty key range: nothing enqueued
    (dict(n_sets=0), _lib.BSA_OK),             # no set: nothing enqueued
])
def test_group_mass_argument_errors(L, kw, code):
    a = _mass_args(**kw)
    assert L.bsa_group_mass(ctypes.byref(a), None) == code
    assert L.bsa_group_mass(None, None) == _lib.BSA_ERR_ARG


def test_topk_rows_argument_errors(L):
    f = L.bsa_topk_rows
    assert f(None, 4, 100, 100, 10, FAKE, None) == _lib.BSA_ERR_ARG
    assert f(FAKE, 4, 100, 100, 10, None, None) == _lib.BSA_ERR_ARG
    assert f(FAKE, -1, 100, 100, 10, FAKE, None) == _lib.BSA_ERR_ARG
    assert f(FAKE, 4, 0, 100, 10, FAKE, None) == _lib.BSA_ERR_ARG
    assert f(FAKE, 4, 100, 99, 10, FAKE, None) == _lib.BSA_ERR_ARG     # ld < n
    assert f(FAKE, 4, 100, 100, -1, FAKE, None) == _lib.BSA_ERR_ARG
    assert f(FAKE, 4, 77825, 77825, 10, FAKE, None) == _lib.BSA_ERR_UNSUPPORTED
    assert f(FAKE, 0, 100, 100, 10, FAKE, None) == _lib.BSA_OK          # nothing enqueued
    assert f(FAKE, 4, 100, 100, 0, FAKE, None) == _lib.BSA_OK


def _args(**kw):
    a = _lib.AttnArgs()
    a.q, a.k, a.v, a.o = FAKE, ctypes.c_void_p(8192), ctypes.c_void_p(16384), ctypes.c_void_p(32768)
    a.B, a.Hq, a.Hkv, a.d, a.block, a.N = 1, 4, 2, 128, 128, 1000
    st = _lib.I64x3(4 * 1000 * 128, 1000 * 128, 128)
    a.q_str = a.k_str = a.v_str = a.o_str = st
    a.row_ptr, a.col = FAKE, FAKE
    for k_, v_ in kw.items():
        setattr(a, k_, v_)
    return a


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.BSA_ERR_ARG),
    (dict(row_ptr=None), _lib.BSA_ERR_ARG),
    (dict(d=96), _lib.BSA_ERR_UNSUPPORTED),
    (dict(block=32), _lib.BSA_ERR_UNSUPPORTED),
    (dict(Hq=3), _lib.BSA_ERR_ARG),
    (dict(N=0), _lib.BSA_ERR_ARG),
    (dict(causal=1, scatter_perm_q=FAKE), _lib.BSA_ERR_UNSUPPORTED),
    (dict(causal=1, gather_perm_q=FAKE), _lib.BSA_ERR_UNSUPPORTED),
    (dict(q=ctypes.c_void_p(4104)), _lib.BSA_ERR_ARG),
    (dict(q_str=_lib.I64x3(4 * 1000 * 128, 1000 * 128, 130)), _lib.BSA_ERR_ARG),
    (dict(o=FAKE), _lib.BSA_ERR_ARG),
    (dict(order=FAKE, n_order=10 ** 6), _lib.BSA_ERR_ARG),
    (dict(N=1 << 40), _lib.BSA_ERR_UNSUPPORTED),
    (dict(v_layout=2), _lib.BSA_ERR_ARG),
    (dict(v_layout=1, v_str=_lib.I64x3(128 * 1000, 128 * 1000, 1000)), _lib.BSA_ERR_ARG),   # rows < 1024 keys
    (dict(v_layout=1, N=1 << 20, q_str=_lib.I64x3(0, 0, 1024), v_str=_lib.I64x3(0, 0, 1 << 20)),
     _lib.BSA_ERR_UNSUPPORTED),                                                              # 32-bit offsets
    (dict(crm=FAKE, lw=FAKE, v_layout=1, v_str=_lib.I64x3(128 * 1024, 128 * 1024, 1024)),
     _lib.BSA_ERR_UNSUPPORTED),                                                              # CRM has no weights
    (dict(crm=FAKE), _lib.BSA_ERR_UNSUPPORTED),                                              # CRM: dim-major V only
    (dict(crm=None, col=None), _lib.BSA_ERR_ARG),
    (dict(kv_share=1), _lib.BSA_ERR_ARG),
    (dict(kv_share=2, v_layout=1, v_str=_lib.I64x3(128 * 1024, 128 * 1024, 1024), Hkv=4),
     _lib.BSA_ERR_UNSUPPORTED),                                                              # G = 1: no pairs
    (dict(kv_share=2), _lib.BSA_ERR_UNSUPPORTED),                                            # token-major V
    (dict(kv_share=2, v_layout=1, v_str=_lib.I64x3(128 * 1024, 128 * 1024, 1024), block=64),
     _lib.BSA_ERR_UNSUPPORTED),
    (dict(kv_share=2, v_layout=1, v_str=_lib.I64x3(128 * 1024, 128 * 1024, 1024), order=FAKE, n_order=17),
     _lib.BSA_ERR_ARG),                                                                      # > R / 2 launches
    (dict(order2=FAKE, v_layout=1, v_str=_lib.I64x3(128 * 1024, 128 * 1024, 1024)),
     _lib.BSA_ERR_ARG),                                                                      # order2 without order
    (dict(order2=FAKE, order=FAKE), _lib.BSA_ERR_UNSUPPORTED),                                # token-major V
    (dict(order2=FAKE, order=FAKE, v_layout=1, v_str=_lib.I64x3(128 * 1024, 128 * 1024, 1024), block=64),
     _lib.BSA_ERR_UNSUPPORTED),
    (dict(order2=FAKE, order=FAKE, v_layout=1, v_str=_lib.I64x3(128 * 1024, 128 * 1024, 1024), kv_share=2),
     _lib.BSA_ERR_UNSUPPORTED),
])
def test_attn_argument_errors(L, kw, code):
    a = _args(**kw)
    assert L.bsa_attn_fwd(ctypes.byref(a), None) == code
    assert L.bsa_attn_fwd(None, None) == _lib.BSA_ERR_ARG


def test_stage1_decide_argument_errors(L):
    ok = (FAKE, FAKE, 4, 100, 100, 12800, 128, 128, 10, 256, None, FAKE, None, None)
    for i, bad in [(0, None), (1, None), (11, None), (2, 0), (3, 0), (4, 0), (5, 0), (6, 0), (7, 0), (8, 0),
                   (9, 0)]:
        a = list(ok)
        a[i] = bad
        assert L.bsa_stage1_decide(*a) == _lib.BSA_ERR_ARG, i
    assert L.bsa_stage1_decide(FAKE, FAKE, 1 << 16, 1 << 15, 100, 12800, 128, 128, 10, 256, None, FAKE, None,
                               None) == _lib.BSA_ERR_UNSUPPORTED


def test_stage1_default_params(L):
    p = _lib.Stage1Params()
    L.bsa_stage1_default_params(ctypes.byref(p))
    import oracle
    assert (p.gamma, p.tile_ms, p.row_ms, p.nnz_ms, p.density_min, p.l2_bytes) == oracle.STAGE1_DEFAULTS
