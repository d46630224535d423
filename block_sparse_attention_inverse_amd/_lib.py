"""ctypes loader for ``libbsa.so`` — argument marshalling only.

The library must have been built (``python -m block_sparse_attention_inverse_amd.build``
or ``__graft_entry__.build()``); there is no fallback of any kind: a missing
library raises at first use.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbsa.so")

BSA_OK, BSA_EINVAL, BSA_EUNSUPPORTED, BSA_ECAPACITY, BSA_EHIP = 0, -1, -2, -3, -4
BSA_F32, BSA_BF16, BSA_I8 = 0, 1, 2

_P = ctypes.c_void_p
_I = ctypes.c_int32
_L = ctypes.c_int64
_F = ctypes.c_float


class MaskParams(ctypes.Structure):
    """Mirror of ``bsa_mask_params`` in include/bsa.h."""

    _fields_ = [
        ("Bq", ctypes.c_int32), ("Bk", ctypes.c_int32), ("score", ctypes.c_int32),
        ("rho_num", ctypes.c_int32), ("rho_den", ctypes.c_int32),
        ("force_diag", ctypes.c_int32), ("win_T", ctypes.c_int32), ("win_r0", ctypes.c_int32),
    ]


# name -> (restype, argtypes); the complete exported surface of bsa.h
SIGNATURES = {
    "bsa_abi_version": (_I, []),
    "bsa_last_error": (ctypes.c_char_p, []),
    "bsa_permute": (_I, [_I, _P, _I, _P, _I, _L, _L, _I, _I, _I, _I, _I, _P, _P]),
    "bsa_mask_capacity": (_L, [_I, _I, _I, _I, ctypes.POINTER(MaskParams)]),
    "bsa_mask_workspace": (_L, [_I, _I, _I, _I, _I, ctypes.POINTER(MaskParams)]),
    "bsa_build_mask": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, ctypes.POINTER(MaskParams), _P, _P,
                            _L, _P, _P, _L, _P]),
    "bsa_build_mask_pooled": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, ctypes.POINTER(MaskParams), _P,
                                   _P, _L, _P, _P, _L, _P]),
    "bsa_fo_workspace": (_L, [_I, _I, _I, _I, _I]),
    "bsa_fo_compensate": (_I, [_P, _P, _P, _P, _P, _L, _I, _P, _I, _I, _I, _P, _L, _L, _P, _I, _I,
                               _I, _I, _F, _P, _L, _P]),
    "bsa_build_mask_pooled_noalloc": (_I, [_P, _P, _I, _I, _I, _I, _I, _P,
                                           ctypes.POINTER(MaskParams), _P, _P, _L, _P, _P]),
    "bsa_permute_pool": (_I, [_P, _I, _P, _L, _L, _I, _I, _I, _I, _I, _P, _I, _P, _P, _P, _P]),
    "bsa_order_workspace": (_L, [_I, _I, _I, _I, _I]),
    "bsa_order_scores": (_I, [_P, _I, _L, _L, _I, _I, _I, _I, _I, _I, _P, _P, _L, _P]),
    "bsa_select_orders": (_I, [_P, _P, _I, _P, _P]),
    "bsa_quantize_int8": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "bsa_forward": (_I, [_P, _P, _P, _P, _P, _L, _I, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "bsa_forward_int8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _L, _I, _P, _P, _I, _I, _I, _I, _I,
                              _F, _P]),
    "bsa_debug_int8_qk": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _P]),
    "bsa_debug_int8_pv": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _P]),
    "bsa_attn_block_stats": (_I, [_P, _P, _I, _I, _I, _I, _F, _F, _P, _P, _P, _P]),
    "bsa_paro_metric": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P, _P]),
    "bsa_paro_select": (_I, [_P, _I, _P, _P]),
    "bsa_mask_sums_workspace": (_L, [_I, _I, _I, _I]),
    "bsa_mask_from_block_sums": (_I, [_P, _I, _I, _I, _I, _F, _I, _P, _P, _L, _P, _P, _L, _P]),
    "bsa_mask_bits_workspace": (_L, [_I]),
    "bsa_mask_from_bits": (_I, [_P, _I, _I, _P, _P, _L, _P, _P, _L, _P]),
    "bsa_forward_natural": (_I, [_P, _P, _P, _P, _P, _L, _I, _P, _I, _I, _I, _P, _L, _L, _P, _I, _I,
                                 _I, _I, _F, _P]),
    "bsa_forward_int8_natural": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _L, _I, _P, _I, _I, _I, _P, _L,
                                      _L, _P, _I, _I, _I, _I, _F, _P]),
    "bsa_block_scores": (_I, [_P, _P, _I, _I, _I, _I, _I, ctypes.POINTER(MaskParams), _P, _P, _L,
                              _P]),
    "bsa_scores_select_workspace": (_L, [_I, _I, _I, _I, _I, _I]),
    "bsa_mask_from_scores": (_I, [_P, _P, _F, _I, _I, _I, _I, _P, ctypes.POINTER(MaskParams), _I,
                                  _F, _F, _P, _P, _L, _P, _P, _L, _P]),
}

_lib = None


class BsaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"bsa error {code}: {msg}")
        self.code = code


def load():
    """Load libbsa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} not found: build it with `python -m block_sparse_attention_inverse_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(rc):
    if rc != BSA_OK:
        msg = load().bsa_last_error()
        raise BsaError(int(rc), msg.decode() if msg else "")
    return rc
