"""ctypes view of the C ABI declared in include/mla_decode.h.

Marshalling only: every step of the decode path runs in the HIP library.
Loading fails loudly if the library is missing; there is no fallback.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmla_decode.so")

ABI_VERSION = 6   # MLA_DECODE_ABI_VERSION of the header this binding mirrors
MLA_OK = 0
STATUS_NAMES = {0: "MLA_OK", 1: "MLA_ERR_INVALID_ARG", 2: "MLA_ERR_UNSUPPORTED", 3: "MLA_ERR_WORKSPACE_TOO_SMALL",
                4: "MLA_ERR_METADATA_MISMATCH", 5: "MLA_ERR_HIP"}
KV_BF16_576 = 0
KV_FP8_656 = 1
KV_FP8_528 = 2
KV_FP4_288 = 3
OUT_BF16 = 0
OUT_FP32 = 1

EXPORTED = ("mla_abi_version", "mla_status_string", "mla_plan", "mla_workspace_bytes",
            "mla_get_decode_metadata", "mla_decode_fwd", "mla_sparse_decode_fwd", "mla_sparse_prefill_fwd",
            "mla_combine",
            "mla_debug_gather_rows", "mla_debug_decode_partial", "mla_check_inputs",
            "mla_decode_step", "mla_decode_step_noalloc")


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "s_q", "h_q", "h_kv", "d_qk", "d_v", "block_size", "num_blocks", "max_blocks_per_seq",
        "topk", "causal", "kv_format", "out_dtype")] + [("softmax_scale", ctypes.c_float),
                                                         ("rescale_threshold", ctypes.c_float)]


class Metadata(ctypes.Structure):
    _fields_ = [("sig", Problem), ("num_partitions", ctypes.c_int32), ("num_head_blocks", ctypes.c_int32),
                ("fixed_overhead", ctypes.c_int32), ("max_splits", ctypes.c_int32),
                ("dev", ctypes.c_void_p), ("bytes", ctypes.c_size_t)]


class MlaError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


_lib = None


def load():
    """Load libmla_decode.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with `python -m mla_decode_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.mla_abi_version.restype = i32
    lib.mla_abi_version.argtypes = []
    if lib.mla_abi_version() != ABI_VERSION:
        raise ImportError(f"{LIB_PATH} has ABI version {lib.mla_abi_version()}, this binding expects "
                          f"{ABI_VERSION}; rebuild it with `python -m mla_decode_amd.build`")
    lib.mla_status_string.restype = ctypes.c_char_p
    lib.mla_status_string.argtypes = [ctypes.c_int]
    lib.mla_plan.restype = ctypes.c_int
    lib.mla_plan.argtypes = [P(Problem), i32, P(Metadata)]
    lib.mla_workspace_bytes.restype = ctypes.c_size_t
    lib.mla_workspace_bytes.argtypes = [P(Metadata)]
    lib.mla_get_decode_metadata.restype = ctypes.c_int
    lib.mla_get_decode_metadata.argtypes = [P(Problem), vp, vp, P(Metadata), vp]
    lib.mla_decode_fwd.restype = ctypes.c_int
    lib.mla_decode_fwd.argtypes = [P(Problem), vp, vp, vp, vp, vp, P(Metadata), vp, ctypes.c_size_t, vp, vp, vp]
    lib.mla_sparse_decode_fwd.restype = ctypes.c_int
    lib.mla_sparse_decode_fwd.argtypes = [P(Problem), vp, vp, vp, vp, vp, P(Metadata), vp, ctypes.c_size_t, vp, vp,
                                          vp]
    lib.mla_sparse_prefill_fwd.restype = ctypes.c_int
    lib.mla_sparse_prefill_fwd.argtypes = [P(Problem), i32, vp, vp, vp, vp, vp, P(Metadata), vp, ctypes.c_size_t,
                                           vp, vp, vp]
    lib.mla_combine.restype = ctypes.c_int
    lib.mla_combine.argtypes = [i32, i32, i32, vp, vp, vp, vp, i32, vp, vp, vp]
    lib.mla_debug_gather_rows.restype = ctypes.c_int
    lib.mla_debug_gather_rows.argtypes = [P(Problem), vp, vp, vp, vp, vp]
    lib.mla_debug_decode_partial.restype = ctypes.c_int
    lib.mla_debug_decode_partial.argtypes = [P(Problem), vp, vp, vp, vp, vp, vp, P(Metadata), vp, ctypes.c_size_t,
                                             vp, vp, i32, vp]
    lib.mla_check_inputs.restype = ctypes.c_int
    lib.mla_check_inputs.argtypes = [P(Problem), P(Metadata), vp, vp, vp, vp, ctypes.c_int64, ctypes.c_char_p,
                                     ctypes.c_size_t]
    lib.mla_decode_step.restype = ctypes.c_int
    lib.mla_decode_step.argtypes = [P(Problem), vp, vp, vp, vp, vp, vp, P(Metadata), vp, ctypes.c_size_t, vp, vp,
                                    vp]
    lib.mla_decode_step_noalloc.restype = ctypes.c_int
    lib.mla_decode_step_noalloc.argtypes = [P(Problem), i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    _lib = lib
    return lib


def check(fn, status):
    if status != MLA_OK:
        lib = load()
        raise MlaError(fn, status, lib.mla_status_string(status).decode())
