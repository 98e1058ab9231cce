"""ctypes declarations of libbpw's C ABI (include/bpw.h). Loading fails loudly if the library
is not built: there is no Python or CPU fallback for any entry point."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbpw.so")

# bpw_status
OK, E_INVAL, E_SIZE, E_P1_BOTH_BITS, E_P2_PADDING, E_NOT_VALIDATED, E_ARCH, E_HIP, E_UNSUPPORTED, E_FORMAT = range(10)
# bpw_kernel
KERNEL_AUTO, KERNEL_BITSERIAL, KERNEL_BYTELANE, KERNEL_MFMA = 0, 1, 2, 3
ABI_VERSION = 1


class BpwErr(ctypes.Structure):
    _fields_ = [("code", ctypes.c_int32), ("row", ctypes.c_int64), ("beat", ctypes.c_int64),
                ("col", ctypes.c_int64)]


class BpwTritErr(ctypes.Structure):
    _fields_ = [("code", ctypes.c_int32), ("check", ctypes.c_int32), ("offset", ctypes.c_int64),
                ("tensor", ctypes.c_int64), ("row", ctypes.c_int64), ("beat", ctypes.c_int64), ("col", ctypes.c_int64)]


class BpwTritTensor(ctypes.Structure):
    _fields_ = [("name", ctypes.c_void_p), ("name_len", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("dims", ctypes.c_uint32 * 4), ("scale", ctypes.c_float),
                ("reserved", ctypes.c_uint32), ("offset", ctypes.c_uint64), ("byte_len", ctypes.c_uint64),
                ("data", ctypes.c_void_p)]


class BpwTritTensorIn(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("name_len", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("ndim", ctypes.c_int32), ("dims", ctypes.c_uint32 * 4), ("scale", ctypes.c_float),
                ("reserved", ctypes.c_uint32), ("data", ctypes.c_void_p), ("byte_len", ctypes.c_uint64)]


class BpwDevMat(ctypes.Structure):
    _fields_ = [("d_planes", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("bpr", ctypes.c_int64), ("w_scale", ctypes.c_float), ("reserved", ctypes.c_uint32),
                ("seal", ctypes.c_uint64)]


class BpwGemvJob(ctypes.Structure):
    _fields_ = [("m", BpwDevMat), ("d_x", ctypes.c_void_p), ("x_len", ctypes.c_int64),
                ("x_scale", ctypes.c_float), ("reserved", ctypes.c_uint32),
                ("d_out_i32", ctypes.c_void_p), ("d_out_f32", ctypes.c_void_p), ("d_x_scale", ctypes.c_void_p)]


class BpwIntMlpJob(ctypes.Structure):
    _fields_ = [("gate", BpwDevMat), ("up", BpwDevMat), ("d_x", ctypes.c_void_p), ("x_len", ctypes.c_int64),
                ("x_scale", ctypes.c_float), ("reserved", ctypes.c_uint32), ("d_x_scale", ctypes.c_void_p),
                ("d_t", ctypes.c_void_p), ("d_k", ctypes.c_void_p), ("d_gate_i32", ctypes.c_void_p),
                ("d_up_i32", ctypes.c_void_p)]


class BpwSbJob(ctypes.Structure):
    _fields_ = [("m", BpwDevMat), ("d_X", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("x_scales", ctypes.c_void_p),
                ("d_out_i32", ctypes.c_void_p), ("d_out_f32", ctypes.c_void_p)]


class BpwDevBitcos(ctypes.Structure):
    _fields_ = [("d_base", ctypes.c_void_p), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("bpr", ctypes.c_int64), ("sign_words", ctypes.c_int64), ("row_start_off", ctypes.c_uint64),
                ("signs_off", ctypes.c_uint64), ("w_scale", ctypes.c_float), ("reserved", ctypes.c_uint32),
                ("seal", ctypes.c_uint64)]


class BpwBitcosJob(ctypes.Structure):
    _fields_ = [("m", BpwDevBitcos), ("d_x", ctypes.c_void_p), ("x_len", ctypes.c_int64),
                ("x_scale", ctypes.c_float), ("reserved", ctypes.c_uint32),
                ("d_out_i32", ctypes.c_void_p), ("d_out_f32", ctypes.c_void_p)]


class BpwQuantJob(ctypes.Structure):
    _fields_ = [("d_h", ctypes.c_void_p), ("d_g", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("d_q", ctypes.c_void_p), ("q_len", ctypes.c_int64), ("d_scale", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("reserved", ctypes.c_uint32)]


class BpwError(RuntimeError):
    """A non-OK bpw_status, with the library's reason and (for validation) the offending position."""

    def __init__(self, status: int, reason: str, row: int = -1, beat: int = -1, col: int = -1):
        self.status, self.reason, self.row, self.beat, self.col = status, reason, row, beat, col
        where = f" (row {row}, beat {beat}, col {col})" if row >= 0 else ""
        super().__init__(f"{_status_name(status)}: {reason}{where}")


_lib = None


def _status_name(s: int) -> str:
    if _lib is None:
        return str(s)
    return _lib.bpw_status_string(s).decode()


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
    E = ctypes.POINTER(BpwErr)
    M = ctypes.POINTER(BpwDevMat)
    J = ctypes.POINTER(BpwGemvJob)
    Q = ctypes.POINTER(BpwQuantJob)
    sig = {
        "bpw_abi_version": (i32, []),
        "bpw_status_string": (ctypes.c_char_p, [i32]),
        "bpw_last_error": (ctypes.c_char_p, []),
        "bpw_device_check": (i32, []),
        "bpw_pack_i8": (i32, [vp, i64, i64, vp, sz, E]),
        "bpw_validate": (i32, [vp, sz, i64, i64, E]),
        "bpw_load": (i32, [vp, sz, i64, i64, f32, ctypes.POINTER(vp), E]),
        "bpw_host_mat_free": (None, [vp]),
        "bpw_host_mat_bytes": (sz, [vp]),
        "bpw_upload": (i32, [vp, vp, sz, vp, M]),
        "bpw_gemv_workspace_bytes": (sz, [J, i32]),
        "bpw_gemv": (i32, [J, i32, i32, vp, sz, vp]),
        "bpw_gemv_noalloc": (i32, [J, i32, i32, vp]),
        "bpw_gemv_plan_create": (i32, [J, i32, i32, vp, sz, vp, ctypes.POINTER(vp)]),
        "bpw_gemv_intmlp_workspace_bytes": (sz, [J, i32, ctypes.POINTER(BpwIntMlpJob), i32]),
        "bpw_gemv_intmlp_plan_create": (i32, [J, i32, ctypes.POINTER(BpwIntMlpJob), i32, i32, vp, sz, vp,
                                              ctypes.POINTER(vp)]),
        "bpw_gemv_plan_run": (i32, [vp, vp]),
        "bpw_gemv_plan_free": (None, [vp]),
        "bpw_gemm_small_batch": (i32, [M, vp, i32, i64, vp, vp, vp, i32, vp]),
        "bpw_gemm_small_batch_workspace_bytes": (sz, [ctypes.POINTER(BpwSbJob), i32, i32]),
        "bpw_gemm_small_batch_plan_create": (i32, [ctypes.POINTER(BpwSbJob), i32, i32, i32, vp, sz, vp,
                                                   ctypes.POINTER(vp)]),
        "bpw_gemm_small_batch_plan_run": (i32, [vp, vp]),
        "bpw_gemm_small_batch_plan_free": (None, [vp]),
        "bpw_quantize_workspace_bytes": (sz, [i32]),
        "bpw_quantize": (i32, [Q, i32, vp, sz, vp]),
        "bpw_quant_plan_create": (i32, [Q, i32, vp, sz, vp, ctypes.POINTER(vp)]),
        "bpw_quant_plan_run": (i32, [vp, vp]),
        "bpw_quant_plan_free": (None, [vp]),
        "bpw_dense_head_gemv": (i32, [vp, i64, i64, vp, vp, vp]),
        "bpw_stream_read_probe": (i32, [vp, sz, vp, vp]),
        "bpw_stream_read_probe_shape": (i32, [vp, sz, vp, i32, vp]),
        "bpw_trit_open": (i32, [vp, sz, ctypes.POINTER(vp), ctypes.POINTER(BpwTritErr)]),
        "bpw_trit_verify": (i32, [vp, i32, ctypes.POINTER(BpwTritErr)]),
        "bpw_trit_close": (None, [vp]),
        "bpw_trit_tensor_count": (i64, [vp]),
        "bpw_trit_tensor_info": (i32, [vp, i64, ctypes.POINTER(BpwTritTensor)]),
        "bpw_trit_find": (i64, [vp, ctypes.c_char_p, sz]),
        "bpw_trit_config": (i32, [vp, ctypes.POINTER(vp), ctypes.POINTER(sz)]),
        "bpw_trit_stored_hash": (ctypes.c_uint64, [vp]),
        "bpw_fnv1a64": (ctypes.c_uint64, [vp, sz]),
        "bpw_trit_load": (i32, [vp, i64, ctypes.POINTER(vp), ctypes.POINTER(BpwErr)]),
        "bpw_trit_write_size": (i32, [ctypes.POINTER(BpwTritTensorIn), i64, sz, ctypes.POINTER(ctypes.c_uint64),
                                      ctypes.POINTER(BpwTritErr)]),
        "bpw_trit_write": (i32, [ctypes.POINTER(BpwTritTensorIn), i64, ctypes.c_char_p, sz, i32, vp, sz,
                                 ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(BpwTritErr)]),
        "bpw_cache_flush": (i32, [vp, sz, vp]),
        "bpw_bitcos_pack_i8": (i32, [vp, i64, i64, f32, ctypes.POINTER(vp), E]),
        "bpw_bitcos_from_planes": (i32, [vp, ctypes.POINTER(vp)]),
        "bpw_bitcos_free": (None, [vp]),
        "bpw_bitcos_arrays": (i32, [vp, ctypes.POINTER(vp), ctypes.POINTER(vp), ctypes.POINTER(vp),
                                    ctypes.POINTER(i64), ctypes.POINTER(i64)]),
        "bpw_bitcos_device_bytes": (sz, [vp]),
        "bpw_bitcos_upload": (i32, [vp, vp, sz, vp, ctypes.POINTER(BpwDevBitcos)]),
        "bpw_bitcos_workspace_bytes": (sz, [ctypes.POINTER(BpwBitcosJob), i32]),
        "bpw_bitcos_plan_create": (i32, [ctypes.POINTER(BpwBitcosJob), i32, vp, sz, vp, ctypes.POINTER(vp)]),
        "bpw_bitcos_plan_run": (i32, [vp, vp]),
        "bpw_bitcos_plan_free": (None, [vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    if L.bpw_abi_version() != ABI_VERSION:
        raise ImportError(f"libbpw ABI {L.bpw_abi_version()} != expected {ABI_VERSION}")
    _lib = L
    return L


def check(status: int, err: BpwErr | None = None) -> None:
    if status != OK:
        reason = lib().bpw_last_error().decode()
        if err is not None and err.row >= 0:
            raise BpwError(status, reason, err.row, err.beat, err.col)
        raise BpwError(status, reason)
