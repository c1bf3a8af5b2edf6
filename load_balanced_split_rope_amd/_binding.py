"""ctypes binding of liblbsr (include/lbsr.h): argument marshalling only.

Every step of the decode path runs in the library's HIP kernels; this module
checks tensor dtypes, devices and sizes, builds the C structs, and passes raw
device pointers and the current torch stream.  If the library has not been
built, every call raises ``LibraryNotBuilt`` -- there is no fallback.
"""

import ctypes
import os
import threading

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# LBSR_LIB may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("LBSR_LIB") or os.path.join(HERE, "liblbsr.so")

ABI_VERSION = 7
HEAD_DIM = 128
PAGE_SIZE = 64
TILE_ELEMS = HEAD_DIM * PAGE_SIZE
NUM_XCDS = 8
NOALLOC_SCRATCH_BYTES = 32 << 20   # LBSR_NOALLOC_SCRATCH_BYTES
MAX_XCD_WEIGHT = 65536

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_HIP = range(5)
KV_BF16, KV_FP8_E4M3 = 0, 1
SCHED_DYNAMIC, SCHED_STATIC = 0, 1
SCHED_FOLD_MERGE = 1           # lbsr_sched_cfg.flags: merge inside the split launch
OUT_BF16, OUT_FP8_E4M3 = 0, 1
QK_BF16, QK_FP8_E4M3 = 0, 1
DEV_ERR_SEQ_LEN, DEV_ERR_PAGE, DEV_ERR_POSITION, DEV_ERR_QUERY_START = 1, 2, 4, 8

# Every symbol include/lbsr.h declares.
EXPORTS = (
    "lbsr_abi_version", "lbsr_status_string", "lbsr_last_error", "lbsr_device_workers",
    "lbsr_workspace_layout", "lbsr_workspace_size", "lbsr_rope_norm_kv_write", "lbsr_plan",
    "lbsr_attention", "lbsr_decode_step", "lbsr_decode_step_timed", "lbsr_prefill_attention",
    "lbsr_prefill_step", "lbsr_prefill_attention_varlen", "lbsr_prefill_step_varlen",
    "lbsr_prefill_workspace_size", "lbsr_read_plan", "lbsr_read_device_error",
    "lbsr_stream_read", "lbsr_decode_step_noalloc", "lbsr_pack_cache", "lbsr_unpack_cache",
)


class LibraryNotBuilt(RuntimeError):
    pass


class LbsrError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_STATUS_NAMES = {OK: "LBSR_OK", E_INVALID: "LBSR_E_INVALID", E_UNSUPPORTED: "LBSR_E_UNSUPPORTED",
                 E_WORKSPACE: "LBSR_E_WORKSPACE", E_HIP: "LBSR_E_HIP"}


class Shape(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("tokens_per_seq", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("num_pages", ctypes.c_int64), ("page_stride", ctypes.c_int64),
                ("head_stride", ctypes.c_int64)]


class Params(ctypes.Structure):
    _fields_ = [("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_float),
                ("norm_before_rope", ctypes.c_int32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("sm_scale", ctypes.c_float),
                ("out_dtype", ctypes.c_int32), ("out_scale", ctypes.c_float),
                ("qk_dtype", ctypes.c_int32), ("q_scale", ctypes.c_float)]


class SchedCfg(ctypes.Structure):
    _fields_ = [("sched", ctypes.c_int32), ("num_workers", ctypes.c_int32),
                ("static_splits", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("xcd_weight", ctypes.c_int32 * NUM_XCDS)]


class WsLayout(ctypes.Structure):
    _fields_ = [("error_word", ctypes.c_size_t), ("cu_tiles", ctypes.c_size_t),
                ("worker_chunk", ctypes.c_size_t), ("chunks", ctypes.c_size_t),
                ("seq_chunk", ctypes.c_size_t), ("seq_len_eff", ctypes.c_size_t),
                ("token_status", ctypes.c_size_t), ("partial_o", ctypes.c_size_t), ("partial_lse", ctypes.c_size_t),
                ("arrivals", ctypes.c_size_t), ("total", ctypes.c_size_t), ("num_workers", ctypes.c_int32),
                ("max_chunks", ctypes.c_int32), ("static_splits", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class PlanHost(ctypes.Structure):
    _fields_ = [("cu_tiles", ctypes.c_void_p), ("worker_chunk", ctypes.c_void_p),
                ("chunks", ctypes.c_void_p), ("seq_chunk", ctypes.c_void_p),
                ("seq_len_eff", ctypes.c_void_p)]


_lib = None
_lib_lock = threading.Lock()

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


def _declare(lib):
    st = ctypes.c_int
    sig = {
        "lbsr_abi_version": (_I32, []),
        "lbsr_status_string": (ctypes.c_char_p, [st]),
        "lbsr_last_error": (ctypes.c_char_p, []),
        "lbsr_device_workers": (st, [ctypes.c_int, ctypes.POINTER(_I32)]),
        "lbsr_workspace_layout": (st, [ctypes.POINTER(Shape), _I32, ctypes.POINTER(SchedCfg),
                                       ctypes.POINTER(WsLayout)]),
        "lbsr_workspace_size": (st, [ctypes.POINTER(Shape), _I32, ctypes.POINTER(SchedCfg),
                                     ctypes.POINTER(ctypes.c_size_t)]),
        "lbsr_rope_norm_kv_write": (st, [ctypes.POINTER(Shape), ctypes.POINTER(Params), _I32]
                                    + [_P] * 11 + [_P]),
        "lbsr_plan": (st, [ctypes.POINTER(Shape), _I32, _P, ctypes.POINTER(SchedCfg), _P,
                           ctypes.c_size_t, _P]),
        "lbsr_attention": (st, [ctypes.POINTER(Shape), ctypes.POINTER(Params), _I32, _P, _P, _P,
                                _P, ctypes.POINTER(SchedCfg), _P, ctypes.c_size_t, _P, _P, _P]),
        "lbsr_decode_step": (st, [ctypes.POINTER(Shape), ctypes.POINTER(Params), _I32]
                             + [_P] * 11 + [ctypes.POINTER(SchedCfg), _P, ctypes.c_size_t, _P,
                                            _P, _P]),
        "lbsr_prefill_attention": (st, [ctypes.POINTER(Shape), ctypes.POINTER(Params), _I32]
                                   + [_P] * 6 + [ctypes.c_size_t] + [_P] * 4),
        "lbsr_prefill_step": (st, [ctypes.POINTER(Shape), ctypes.POINTER(Params), _I32]
                              + [_P] * 12 + [ctypes.c_size_t] + [_P] * 4),
        "lbsr_prefill_attention_varlen": (st, [ctypes.POINTER(Shape), ctypes.POINTER(Params),
                                               _I32, _I32] + [_P] * 7 + [ctypes.c_size_t]
                                              + [_P] * 4),
        "lbsr_prefill_step_varlen": (st, [ctypes.POINTER(Shape), ctypes.POINTER(Params), _I32,
                                          _I32] + [_P] * 13 + [ctypes.c_size_t] + [_P] * 4),
        "lbsr_prefill_workspace_size": (st, [ctypes.POINTER(Shape), _I32, _I32,
                                             ctypes.POINTER(ctypes.c_size_t)]),
        "lbsr_decode_step_timed": (st, [ctypes.POINTER(Shape), ctypes.POINTER(Params), _I32]
                                   + [_P] * 11 + [ctypes.POINTER(SchedCfg), _P, ctypes.c_size_t,
                                                  _P, _P, _P, ctypes.POINTER(ctypes.c_float), _P]),
        "lbsr_read_plan": (st, [ctypes.POINTER(Shape), _I32, ctypes.POINTER(SchedCfg), _P,
                                ctypes.c_size_t, ctypes.POINTER(PlanHost), ctypes.POINTER(_I32),
                                _P]),
        "lbsr_read_device_error": (st, [_P, ctypes.POINTER(_I32), _P]),
        "lbsr_stream_read": (st, [_P, ctypes.c_size_t, _I32, _I32, _P, _P]),
        "lbsr_decode_step_noalloc": (st, [ctypes.POINTER(Shape), ctypes.POINTER(Params), _I32]
                                     + [_P] * 11 + [ctypes.POINTER(SchedCfg), _P, _P, _P]),
        "lbsr_pack_cache": (st, [ctypes.POINTER(Shape), _I32, _P, ctypes.c_int64,
                                 ctypes.c_int64, ctypes.c_int64, _P, _P]),
        "lbsr_unpack_cache": (st, [ctypes.POINTER(Shape), _I32, _P, _P, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, _P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def lib():
    """The loaded library; raises LibraryNotBuilt if it is missing."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise LibraryNotBuilt(
                        f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                        "(hipcc, gfx950); there is no fallback implementation")
                handle = ctypes.CDLL(LIB_PATH)
                _declare(handle)
                got = handle.lbsr_abi_version()
                if got != ABI_VERSION:
                    raise LibraryNotBuilt(
                        f"{LIB_PATH} has ABI version {got}, this binding needs {ABI_VERSION}: "
                        "rebuild it with __graft_entry__.build()")
                _lib = handle
    return _lib


def _check(status):
    if status != OK:
        raise LbsrError(status, lib().lbsr_last_error().decode())


def _ptr(t):
    # every entry point declares its pointer arguments as c_void_p, so a plain
    # int (or None for NULL) is passed as is
    return None if t is None else t.data_ptr()


def _stream(stream):
    """The HIP stream handle: `stream`'s, or torch's current stream on the current device."""
    if stream is None:
        return torch._C._cuda_getCurrentRawStream(torch._C._cuda_getDevice())
    return stream.cuda_stream
