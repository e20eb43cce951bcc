"""ctypes binding of libmsa.so (the C ABI declared in include/msa.h).

Argument marshalling only: every step of the hot path runs in the library's
HIP kernels.  torch supplies device memory and the current stream.  There is
no fallback: if the library is missing, loading fails with an error that says
how to build it.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_HIP, MSA_ERR_WORKSPACE = range(5)
MSA_BF16, MSA_F32 = 0, 1

# Every symbol include/msa.h declares.
ABI_VERSION = 4        # include/msa.h MSA_ABI_VERSION; msa_config / msa_layout below
EXPORTS = ("msa_abi_version", "msa_status_string", "msa_last_error", "msa_get_layout",
           "msa_proxy_scores", "msa_select_blocks", "msa_select_blocks_noalloc",
           "msa_select_blocks_noalloc_max_bytes", "msa_fwd", "msa_bwd", "msa_kernel_count",
           "msa_kernel_info", "msa_profile_enable", "msa_profile_collect", "msa_profile_entry")


class MsaConfig(ctypes.Structure):
    _fields_ = [("heads_q", c_int32), ("heads_kv", c_int32), ("head_dim", c_int32),
                ("proxy_dim", c_int32), ("kv_block", c_int32), ("q_block", c_int32),
                ("topk", c_int32), ("local_window", c_int32), ("softmax_scale", c_float),
                ("proxy_scale", c_float), ("proxy_loss_weight", c_float), ("dtype", c_int32),
                ("dilation", c_int32), ("proxy_heads", c_int32)]


class MsaVarlen(ctypes.Structure):
    _fields_ = [("cu_seqlens", c_void_p), ("cu_seqlens_host", POINTER(c_int32)),
                ("batch", c_int32), ("total_tokens", c_int32)]


class MsaLayout(ctypes.Structure):
    _fields_ = [("total_qblocks", c_int64), ("total_kvblocks", c_int64), ("score_elems", c_int64),
                ("sel_stride", c_int64), ("k2q_capacity", c_int64), ("scored_pairs", c_int64),
                ("max_qblocks_doc", c_int64), ("workspace_bytes", c_int64), ("proxy_heads", c_int64)]

    def as_dict(self):
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


class MsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load():
    """Load libmsa.so once; raise a clear error if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m block_sparse_attention_proxy_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    pc, pv, pl = POINTER(MsaConfig), POINTER(MsaVarlen), POINTER(MsaLayout)
    pi = POINTER(c_int32)
    lib.msa_abi_version.restype = c_int32
    if lib.msa_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.msa_abi_version()}, this binding expects "
                          f"{ABI_VERSION}: rebuild it with `python -m block_sparse_attention_proxy_amd.build`")
    lib.msa_status_string.restype = c_char_p
    lib.msa_status_string.argtypes = [c_int32]
    lib.msa_last_error.restype = c_char_p
    lib.msa_get_layout.restype = c_int32
    lib.msa_get_layout.argtypes = [pc, pv, pl]
    lib.msa_proxy_scores.restype = c_int32
    lib.msa_proxy_scores.argtypes = [pc, pv, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
    lib.msa_select_blocks.restype = c_int32
    lib.msa_select_blocks.argtypes = [pc, pv, c_void_p] + [c_void_p] * 4 + [c_void_p, c_size_t, c_void_p]
    lib.msa_select_blocks_noalloc.restype = c_int32
    lib.msa_select_blocks_noalloc.argtypes = [pc, pv, c_void_p] + [c_void_p] * 4 + [c_void_p]
    lib.msa_select_blocks_noalloc_max_bytes.restype = c_int64
    lib.msa_select_blocks_noalloc_max_bytes.argtypes = []
    lib.msa_fwd.restype = c_int32
    lib.msa_fwd.argtypes = [pc, pv] + [c_void_p] * 10 + [c_void_p, c_size_t, c_void_p]
    lib.msa_bwd.restype = c_int32
    lib.msa_bwd.argtypes = [pc, pv] + [c_void_p] * 18 + [c_void_p, c_size_t, c_void_p]
    lib.msa_kernel_count.restype = c_int32
    lib.msa_kernel_info.restype = c_int32
    lib.msa_kernel_info.argtypes = [c_int32, c_char_p, c_size_t, pi, pi, pi, pi]
    lib.msa_profile_enable.restype = c_int32
    lib.msa_profile_enable.argtypes = [c_int32]
    lib.msa_profile_collect.restype = c_int32
    lib.msa_profile_entry.restype = c_int32
    lib.msa_profile_entry.argtypes = [c_int32, c_char_p, c_size_t, POINTER(ctypes.c_double),
                                      POINTER(c_int64)]
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != MSA_OK:
        lib = load()
        msg = lib.msa_last_error().decode() or lib.msa_status_string(status).decode()
        raise MsaError(status, msg)
