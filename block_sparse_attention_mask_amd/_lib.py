"""ctypes declarations for libbsattn.so (the C ABI in include/bsattn.h)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libbsattn.so")

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
I64x3 = ctypes.c_int64 * 3

BSA_OK = 0
BSA_ERR_ARG = -1
BSA_ERR_UNSUPPORTED = -2
BSA_ERR_HIP = -4
BSA_V_TOKEN_MAJOR = 0
BSA_V_DIM_MAJOR = 1

# Every symbol include/bsattn.h declares.
EXPORTS = ("bsa_version", "bsa_strerror", "bsa_csr_count", "bsa_csr_fill", "bsa_crm_build", "bsa_crm_row_ptr",
           "bsa_crm_to_csr", "bsa_segment_offsets", "bsa_segment_means", "bsa_is_sample", "bsa_perm_from_labels",
           "bsa_permute_rows", "bsa_unpermute_rows", "bsa_transpose_rows", "bsa_spectral_order", "bsa_schedule",
           "bsa_attn_fwd", "bsa_attn_tok_fwd", "bsa_group_mass", "bsa_topk_rows", "bsa_stage1_decide",
           "bsa_stage1_default_params", "bsa_pair_rows_equal", "bsa_schedule_pairs",
           "bsa_device_cus", "bsa_device_clock_khz", "bsa_clock_probe")


class AttnArgs(ctypes.Structure):
    _fields_ = [
        ("q", P), ("k", P), ("v", P), ("o", P), ("lse", P),
        ("B", I32), ("Hq", I32), ("Hkv", I32), ("d", I32), ("block", I32),
        ("N", I64),
        ("q_str", I64x3), ("k_str", I64x3), ("v_str", I64x3), ("o_str", I64x3),
        ("row_ptr", P), ("col", P), ("lw", P), ("order", P),
        ("n_order", I64),
        ("scatter_perm_q", P),
        ("scale", ctypes.c_float),
        ("causal", I32),
        ("v_layout", I32),
        ("crm", P),
        ("gather_perm_q", P),
        ("kv_share", I32),
        ("order2", P),
    ]


class Stage1Params(ctypes.Structure):
    _fields_ = [("gamma", ctypes.c_double), ("tile_ms", ctypes.c_double), ("row_ms", ctypes.c_double),
                ("nnz_ms", ctypes.c_double), ("density_min", ctypes.c_double), ("l2_bytes", ctypes.c_double)]


class TokArgs(ctypes.Structure):
    _fields_ = [
        ("q", P), ("k", P), ("v", P), ("o", P), ("lse", P),
        ("B", I32), ("Hq", I32), ("Hkv", I32), ("d", I32),
        ("N", I64),
        ("q_str", I64x3), ("k_str", I64x3), ("v_str", I64x3), ("o_str", I64x3),
        ("n_sets", I32), ("set_size", I32),
        ("q_idx", P), ("kv_ptr", P), ("kv_idx", P),
        ("scale", ctypes.c_float),
        ("causal", I32),
        ("kv_share", I32),
    ]


class MassArgs(ctypes.Structure):
    _fields_ = [
        ("q", P), ("k", P), ("lse", P), ("mass", P),
        ("B", I32), ("Hq", I32), ("Hkv", I32), ("d", I32),
        ("N", I64),
        ("q_str", I64x3), ("k_str", I64x3),
        ("n_sets", I32), ("set_size", I32),
        ("q_idx", P),
        ("k0", I64), ("k1", I64),
        ("scale", ctypes.c_float),
        ("causal", I32),
    ]


_lib = None


class BsaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        msg = load().bsa_strerror(code).decode() if _lib is not None else str(code)
        super().__init__("%s failed: %s (%d)" % (fn, msg, code))
        self.code = code


def load():
    """Load the in-tree HIP library; there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libbsattn.so is not built (run __graft_entry__.build() or "
                               "python block_sparse_attention_mask_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)   # unresolved symbols fail here
        L.bsa_version.restype = ctypes.c_int
        L.bsa_version.argtypes = []
        L.bsa_strerror.restype = ctypes.c_char_p
        L.bsa_strerror.argtypes = [ctypes.c_int]
        L.bsa_csr_count.restype = ctypes.c_int
        L.bsa_csr_count.argtypes = [P, P, ctypes.c_float, I64, I32, I32, ctypes.c_int, P,
                                    ctypes.POINTER(I64), P]
        L.bsa_csr_fill.restype = ctypes.c_int
        L.bsa_csr_fill.argtypes = [P, P, ctypes.c_float, P, I64, I32, I32, ctypes.c_int, P, P, P,
                                   I64, P]
        L.bsa_crm_build.restype = ctypes.c_int
        L.bsa_crm_build.argtypes = [P, P, ctypes.c_float, I64, I32, I32, ctypes.c_int, P, P]
        L.bsa_crm_row_ptr.restype = ctypes.c_int
        L.bsa_crm_row_ptr.argtypes = [P, I64, I32, P, ctypes.POINTER(I64), P]
        L.bsa_crm_to_csr.restype = ctypes.c_int
        L.bsa_crm_to_csr.argtypes = [P, I64, I32, P, P, I64, P]
        L.bsa_segment_offsets.restype = ctypes.c_int
        L.bsa_segment_offsets.argtypes = [P, I64, I64, I32, P, P]
        L.bsa_segment_means.restype = ctypes.c_int
        L.bsa_segment_means.argtypes = [P, I64x3, I32, I32, I64, I32, P, I32, I32, P, P]
        L.bsa_is_sample.restype = ctypes.c_int
        L.bsa_is_sample.argtypes = [P, P, P, P, I32, I32, I32, I32, I64, I32, I32, I32, I32, ctypes.c_float,
                                    P, P, P, P]
        L.bsa_perm_from_labels.restype = ctypes.c_int
        L.bsa_perm_from_labels.argtypes = [P, I64, I64, I32, P, P]
        for fn in (L.bsa_permute_rows, L.bsa_unpermute_rows):
            fn.restype = ctypes.c_int
            fn.argtypes = [P, P, P, I32, I32, I64, I32, P, P, P]
        L.bsa_transpose_rows.restype = ctypes.c_int
        L.bsa_transpose_rows.argtypes = [P, P, P, I32, I32, I64, I32, I64, P, P, P]
        L.bsa_schedule.restype = ctypes.c_int
        L.bsa_schedule.argtypes = [P, P, I32, I32, I32, I32, I32, I32, P, I32, P, P]
        L.bsa_schedule_pairs.restype = ctypes.c_int
        L.bsa_schedule_pairs.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, P, P, P, P]
        L.bsa_pair_rows_equal.restype = ctypes.c_int
        L.bsa_pair_rows_equal.argtypes = [P, P, P, I32, I32, I32, I32, P, P]
        L.bsa_spectral_order.restype = ctypes.c_int
        L.bsa_spectral_order.argtypes = [P, P, I32, I32, I32, I32, P, P, P, P]
        L.bsa_stage1_default_params.restype = None
        L.bsa_stage1_default_params.argtypes = [ctypes.POINTER(Stage1Params)]
        L.bsa_stage1_decide.restype = ctypes.c_int
        L.bsa_stage1_decide.argtypes = [P, P, I32, I32, I32, I64, I32, I32, I32, I32,
                                        ctypes.POINTER(Stage1Params), P, P, P]
        L.bsa_attn_fwd.restype = ctypes.c_int
        L.bsa_attn_fwd.argtypes = [ctypes.POINTER(AttnArgs), P]
        L.bsa_clock_probe.restype = ctypes.c_int
        L.bsa_clock_probe.argtypes = [I32, I32, I32, P, P]
        L.bsa_attn_tok_fwd.restype = ctypes.c_int
        L.bsa_attn_tok_fwd.argtypes = [ctypes.POINTER(TokArgs), P]
        L.bsa_group_mass.restype = ctypes.c_int
        L.bsa_group_mass.argtypes = [ctypes.POINTER(MassArgs), P]
        L.bsa_topk_rows.restype = ctypes.c_int
        L.bsa_topk_rows.argtypes = [P, I64, I64, I64, I32, P, P]
        L.bsa_device_cus.restype = ctypes.c_int
        L.bsa_device_cus.argtypes = []
        L.bsa_device_clock_khz.restype = ctypes.c_int
        L.bsa_device_clock_khz.argtypes = []
        _lib = L
    return _lib


def check(fn: str, rc: int) -> None:
    if rc != BSA_OK:
        raise BsaError(fn, rc)
