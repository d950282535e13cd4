"""ctypes binding of libsdm.so (include/sdm.h).  Argument marshalling only.

The library is loaded from this package's directory; if it has not been built
the import fails loudly -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsdm.so")

SDM_OK, SDM_ERR_ARG, SDM_ERR_STATE, SDM_ERR_CAPACITY, SDM_ERR_DEVICE, SDM_ERR_UNSUPPORTED = 0, -1, -2, -3, -4, -5
STATUS_NAMES = {0: "OK", -1: "ERR_ARG", -2: "ERR_STATE", -3: "ERR_CAPACITY", -4: "ERR_DEVICE", -5: "ERR_UNSUPPORTED"}
SDM_F32, SDM_BF16 = 0, 1
SDM_WEIGHTS_BF16, SDM_WEIGHTS_INT4 = 0, 1
SDM_CAUSAL, SDM_BIDIR = 0, 1
SDM_PACK_PLAIN, SDM_PACK_QKV, SDM_PACK_GATE_UP = 0, 1, 2
KERNEL_CLASSES = {"qkv": 0, "attn": 1, "attn_combine": 2, "o": 3, "gate_up": 4, "down": 5, "lm_head": 6,
                  "norm": 7, "finish": 8, "forward": 9}


class SdmError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class SdmConfig(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_q_heads", c_int32), ("n_kv_heads", c_int32),
                ("head_dim", c_int32), ("ffn_dim", c_int32), ("vocab", c_int32), ("mask_id", c_int32),
                ("rope_base", c_float), ("rms_eps", c_float), ("dtype", c_int32),
                ("page_tokens", c_int32), ("max_seqs", c_int32), ("max_block", c_int32),
                ("max_context", c_int32), ("max_rows", c_int32), ("weight_format", c_int32)]


class SdmWeights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("final_norm", c_void_p), ("lm_head", c_void_p),
                ("attn_norm", POINTER(c_void_p)), ("w_qkv", POINTER(c_void_p)), ("w_o", POINTER(c_void_p)),
                ("ffn_norm", POINTER(c_void_p)), ("w_gate_up", POINTER(c_void_p)), ("w_down", POINTER(c_void_p))]


# name -> (restype, argtypes); every name is declared in include/sdm.h
SIGNATURES = {
    "sdm_workspace_bytes": (c_size_t, [POINTER(SdmConfig)]),
    "sdm_kv_page_bytes": (c_size_t, [POINTER(SdmConfig)]),
    "sdm_packed_bytes": (c_size_t, [POINTER(SdmConfig), c_int64, c_int64]),
    "sdm_pack_matrix": (c_int32, [POINTER(SdmConfig), c_int32, c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                  c_void_p]),
    "sdm_packed_bytes_int4": (c_size_t, [POINTER(SdmConfig), c_int64, c_int64]),
    "sdm_pack_matrix_int4": (c_int32, [POINTER(SdmConfig), c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                       c_int64, c_int64, c_void_p]),
    "sdm_init_model": (c_int32, [POINTER(SdmConfig), POINTER(SdmWeights), c_void_p, c_int64, c_void_p, c_size_t,
                                 c_void_p, POINTER(c_void_p)]),
    "sdm_prefill": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p]),
    "sdm_diffuse_step": (c_int32, [c_void_p, c_int32, POINTER(c_int32), c_void_p, c_int32, c_float, c_int32,
                                   c_void_p, c_void_p, c_void_p]),
    "sdm_diffuse_step_revise": (c_int32, [c_void_p, c_int32, POINTER(c_int32), c_void_p, c_int32, c_float, c_float,
                                          c_int32, c_void_p, c_void_p, c_void_p, c_void_p]),
    "sdm_prefill_sample": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_float, c_uint64, c_void_p, c_void_p]),
    "sdm_decode_ar_sample": (c_int32, [c_void_p, c_int32, c_void_p, c_float, c_uint64, c_void_p, c_void_p]),
    "sdm_draft_block_sample": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_float, c_uint64, c_void_p,
                                         c_void_p, c_void_p]),
    "sdm_verify_block_sample": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_float, c_uint64, c_void_p,
                                          c_void_p, c_void_p, c_void_p, c_void_p]),
    "sdm_draft_block": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p]),
    "sdm_verify_block_quadratic": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                             c_void_p]),
    "sdm_verify_block": (c_int32, [c_void_p, c_int32, POINTER(c_int32), c_void_p, c_int32, c_void_p, c_void_p,
                                   c_void_p]),
    "sdm_commit_kv": (c_int32, [c_void_p, c_int32, c_int32]),
    "sdm_decode_ar": (c_int32, [c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "sdm_row_stats": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p]),
    "sdm_seq_reset": (c_int32, [c_void_p, c_int32]),
    "sdm_seq_length": (c_int32, [c_void_p, c_int32, POINTER(c_int32)]),
    "sdm_free_pages": (c_int64, [c_void_p]),
    "sdm_shuffle_free_pages": (c_int32, [c_void_p, c_uint64]),
    "sdm_free_model": (c_int32, [c_void_p]),
    "sdm_last_error": (ctypes.c_char_p, []),
    "sdm_timing_start": (c_int32, [c_void_p, c_int32, c_int32]),
    "sdm_timing_stop": (c_int32, [c_void_p, POINTER(c_int64), POINTER(ctypes.c_double), POINTER(ctypes.c_double),
                                  POINTER(ctypes.c_double)]),
    "sdm_attn_pool_bytes": (c_size_t, [c_int32, c_int32, c_int32]),
    "sdm_attn_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32]),
    "sdm_attn_pack_kv": (c_int32, [c_int32, c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]),
    "sdm_attention": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                c_void_p, c_void_p, c_size_t, c_void_p]),
    "sdm_attention_scratch_max_bytes": (c_size_t, []),
    "sdm_attention_noalloc": (c_int32, [c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                                        c_int32, c_void_p, c_void_p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m self_speculative_amd.build` "
                              "(the HIP library is required; there is no fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != SDM_OK:
        raise SdmError(status, lib().sdm_last_error().decode(errors="replace"))


def ptr(t) -> int | None:
    """Device address of a torch tensor (None for None)."""
    return None if t is None else t.data_ptr()
