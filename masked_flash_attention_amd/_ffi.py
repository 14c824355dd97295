"""ctypes view of libmfa's C ABI (include/mfa.h). Argument marshalling only."""

from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmfa.so")

MFA_OK = 0
STATUS_NAMES = {0: "MFA_OK", 1: "MFA_E_ARG", 2: "MFA_E_SHAPE", 3: "MFA_E_DTYPE", 4: "MFA_E_UNSUPPORTED",
                5: "MFA_E_NOT_DEVICE", 6: "MFA_E_NONCANONICAL", 7: "MFA_E_HIP", 8: "MFA_E_NO_DEVICE"}

MFA_BF16, MFA_F32 = 0, 1
MASK_NONE, MASK_BLOCKID, MASK_TILES, MASK_BSR, MASK_VARLEN = 0, 1, 2, 3, 4

vp = C.c_void_p
i64x3 = C.c_int64 * 3


class AttnArgs(C.Structure):
    _fields_ = [("dtype", C.c_int), ("B", C.c_int), ("Sq", C.c_int), ("Sk", C.c_int), ("Hq", C.c_int),
                ("Hkv", C.c_int), ("D", C.c_int), ("q", vp), ("k", vp), ("v", vp), ("out", vp), ("lse", vp),
                ("q_stride", i64x3), ("k_stride", i64x3), ("v_stride", i64x3), ("o_stride", i64x3),
                ("alibi_slopes", vp), ("softcap", C.c_float)]


class Mask(C.Structure):
    _fields_ = [("kind", C.c_int),
                ("q_blk", vp), ("k_blk", vp), ("q_valid", vp), ("k_valid", vp), ("qsum", vp), ("ksum", vp),
                ("kv_bits", vp),
                ("tile_kind", vp), ("fine_bits", vp), ("row_ptr", vp), ("col_idx", vp), ("col_kind", vp),
                ("indptr", vp), ("indices", vp), ("bsr_kind", vp), ("csc_ptr", vp), ("csc_idx", vp),
                ("q_block", C.c_int), ("kv_block", C.c_int),
                ("cu_q", vp), ("cu_k", vp), ("work", vp), ("work_cap", C.c_int), ("max_q", C.c_int),
                ("max_k", C.c_int), ("err", vp),
                ("causal", C.c_int), ("win_left", C.c_int), ("win_right", C.c_int), ("nseq", C.c_int),
                ("seqused_k", vp), ("block_table", vp), ("max_pages", C.c_int), ("page_size", C.c_int),
                ("n_pages", C.c_int), ("tile_m", C.c_int)]


class BwdArgs(C.Structure):
    _fields_ = [("fwd", AttnArgs), ("dout", vp), ("dq", vp), ("dk", vp), ("dv", vp), ("delta", vp),
                ("do_stride", i64x3), ("dq_stride", i64x3), ("dk_stride", i64x3), ("dv_stride", i64x3),
                ("workspace", vp), ("workspace_bytes", C.c_int64)]


PRED_MAX_TERMS = 4
PRED_MAX_ATOMS = 4


class PredAtom(C.Structure):
    _fields_ = [("a", C.c_int64), ("b", C.c_int64), ("c", C.c_int64)]


class Predicate(C.Structure):
    _fields_ = [("n_terms", C.c_int), ("n_atoms", C.c_int * PRED_MAX_TERMS),
                ("atoms", (PredAtom * PRED_MAX_ATOMS) * PRED_MAX_TERMS)]


# name -> argument types (restype is int status except where noted)
SIGNATURES = {
    "mfa_is_available": ([], C.c_int),
    "mfa_last_error": ([], C.c_char_p),
    "mfa_status_name": ([C.c_int], C.c_char_p),
    "mfa_make_block_ids": ([vp, vp, C.c_int, C.c_int, C.c_int, vp, vp, vp, vp, vp, vp], C.c_int),
    "mfa_blockid_tile_summary": ([vp, vp, vp, vp, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, vp, vp, vp, vp],
                                 C.c_int),
    "mfa_compact_dense_mask": ([vp, C.c_int, C.c_int, C.c_int, C.c_int, vp, vp, vp, vp, vp, vp], C.c_int),
    "mfa_tile_map_coarsen": ([vp, C.c_int, C.c_int, vp, vp, vp, vp, vp], C.c_int),
    "mfa_tile_counts": ([vp, C.c_int64, vp, vp], C.c_int),
    "mfa_model_tile_time": ([C.POINTER(C.c_int64), C.c_int, C.c_int, C.c_int], C.c_double),
    "mfa_choose_tile_m": ([C.POINTER(C.c_int64), C.POINTER(C.c_int64), C.c_int, C.c_int], C.c_int),
    "mfa_predicate_tiles": ([C.POINTER(Predicate), C.c_int, C.c_int, vp, vp, vp, vp, vp, vp], C.c_int),
    "mfa_bsr_validate": ([vp, vp, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64, C.POINTER(C.c_int), vp], C.c_int),
    "mfa_bsr_prepare": ([vp, vp, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int64, C.c_int, C.c_int, C.c_int,
                         C.c_int, C.c_int, vp, vp, vp, vp, vp], C.c_int),
    "mfa_bsr_from_bitmask": ([vp, C.c_int, C.c_int, C.c_int, C.c_int, vp, vp, C.c_int64, vp], C.c_int),
    "mfa_varlen_schedule": ([vp, vp, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, C.c_int, vp, vp, vp, vp,
                             C.c_int, vp, vp], C.c_int),
    "mfa_attn_fwd": ([C.POINTER(AttnArgs), C.POINTER(Mask), C.c_float, vp], C.c_int),
    "mfa_attn_bwd_preprocess": ([C.POINTER(BwdArgs), vp], C.c_int),
    "mfa_attn_bwd_dkdv": ([C.POINTER(BwdArgs), C.POINTER(Mask), C.c_float, vp], C.c_int),
    "mfa_attn_bwd_dq": ([C.POINTER(BwdArgs), C.POINTER(Mask), C.c_float, vp], C.c_int),
    "mfa_attn_bwd_dkdv_workspace": ([C.POINTER(BwdArgs), C.POINTER(Mask), C.POINTER(C.c_int64),
                                     C.POINTER(C.c_int)], C.c_int),
    "mfa_choose_dkdv_split": ([C.c_int64, C.c_int, C.c_int, C.c_int], C.c_int),
    "mfa_attn_bwd_dkdv_noalloc": ([C.POINTER(BwdArgs), C.POINTER(Mask), C.c_float, vp], C.c_int),
    "mfa_bwd_scratch_bytes": ([], C.c_int64),
}

_lib = None
_load_error = None


class MfaError(RuntimeError):
    def __init__(self, status, message):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


def load():
    """Load libmfa.so; raise ImportError naming the build command if it is missing."""
    global _lib, _load_error
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        _load_error = f"{LIB_PATH} is not built; run `python -m masked_flash_attention_amd.build`"
        raise ImportError(_load_error)
    try:
        lib = C.CDLL(LIB_PATH)
    except OSError as e:
        _load_error = str(e)
        raise ImportError(f"cannot load {LIB_PATH}: {e}") from e
    for name, (argtypes, restype) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = argtypes
        fn.restype = restype
    _lib = lib
    return lib


def load_error():
    return _load_error


def check(status):
    if status != MFA_OK:
        msg = load().mfa_last_error()
        raise MfaError(status, msg.decode() if msg else "")
