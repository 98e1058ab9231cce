"""CPU oracle for the ternary bit-plane GEMV - TEST INFRASTRUCTURE ONLY.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The product path (``bit_plane_weight_amd``)
never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, one weight at a time, int64 sums,
float64 beside the fp32 dequantisation). This module only compiles it with gcc and
marshals numpy arrays. See ``oracle.c`` for the passages each function follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.c")

OK, E_INVAL, E_SIZE, E_P1, E_P2, E_RANGE = 0, 1, 2, 3, 4, 5


class OracleError(Exception):
    def __init__(self, code: int, row: int, beat: int, col: int):
        super().__init__(f"oracle error {code} at row={row} beat={beat} col={col}")
        self.code, self.row, self.beat, self.col = code, row, beat, col


class _Err(ctypes.Structure):
    _fields_ = [("code", ctypes.c_int32), ("row", ctypes.c_int64),
                ("beat", ctypes.c_int64), ("col", ctypes.c_int64)]


def build(force: bool = True) -> str:
    """Compile liboracle.so: -O2, OpenMP for the independent row loop, strict IEEE float."""
    if force or not os.path.exists(_SO):
        tmp = _SO + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
             "-fno-fast-math", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build(force=False)
        lib = ctypes.CDLL(_SO)
        i64, vp, f32, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int
        ep = ctypes.POINTER(_Err)
        lib.oracle_beats_per_row.argtypes = [i64]
        lib.oracle_beats_per_row.restype = i64
        lib.oracle_byte_len.argtypes = [i64, i64]
        lib.oracle_byte_len.restype = i64
        lib.oracle_tail_mask.argtypes = [i64]
        lib.oracle_tail_mask.restype = ctypes.c_uint64
        lib.oracle_pack.argtypes = [vp, i64, i64, vp, i64, ep]
        lib.oracle_validate.argtypes = [vp, i64, i64, i64, ep]
        lib.oracle_unpack.argtypes = [vp, i64, i64, i64, vp, ep]
        lib.oracle_gemv.argtypes = [vp, i64, i64, i64, vp, i64, f32, f32, vp, vp, vp, ci, ep]
        lib.oracle_gemv_bitserial.argtypes = [vp, i64, i64, i64, vp, i64, vp, ci, ep]
        lib.oracle_gemm_small_batch.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, f32, vp, vp, vp, ci, ep]
        lib.oracle_dense_head.argtypes = [vp, i64, i64, vp, vp, vp, ci]
        lib.oracle_quantize.argtypes = [vp, vp, i64, f32, ci, vp, vp]
        lib.oracle_intmlp.argtypes = [vp, vp, i64, i64, i64, vp, i64, f32, f32, f32, vp, vp, vp, vp, ci, ep]
        lib.oracle_bitcos_pack_flat.argtypes = [vp, i64, vp, vp, vp]
        lib.oracle_bitcos_unpack_flat.argtypes = [vp, i64, vp, i64, i64, vp]
        lib.oracle_bitcos_pack_rows.argtypes = [vp, i64, i64, vp, vp, vp]
        lib.oracle_bitcos_gemv.argtypes = [vp, vp, vp, i64, i64, vp, f32, f32, vp, vp, vp, ci]
        for f in ("oracle_pack", "oracle_validate", "oracle_unpack", "oracle_gemv",
                  "oracle_gemv_bitserial", "oracle_gemm_small_batch", "oracle_dense_head", "oracle_quantize",
                  "oracle_intmlp", "oracle_bitcos_pack_flat", "oracle_bitcos_unpack_flat",
                  "oracle_bitcos_pack_rows", "oracle_bitcos_gemv"):
            getattr(lib, f).restype = ci
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _check(rc: int, err: _Err):
    if rc != OK:
        raise OracleError(rc, err.row, err.beat, err.col)


def beats_per_row(cols: int) -> int:
    return int(_load().oracle_beats_per_row(cols))


def byte_len(rows: int, cols: int) -> int:
    return int(_load().oracle_byte_len(rows, cols))


def tail_mask(cols: int) -> int:
    return int(_load().oracle_tail_mask(cols))


def pack(w: np.ndarray) -> np.ndarray:
    """int8 [rows, cols] trits -> .trit v1 plane bytes uint8 [rows * bpr * 16]."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    rows, cols = w.shape
    out = np.zeros(byte_len(rows, cols), dtype=np.uint8)
    err = _Err()
    _check(_load().oracle_pack(_p(w), rows, cols, _p(out), out.size, ctypes.byref(err)), err)
    return out


def validate(planes: np.ndarray, rows: int, cols: int) -> None:
    planes = np.ascontiguousarray(planes, dtype=np.uint8)
    err = _Err()
    _check(_load().oracle_validate(_p(planes), planes.size, rows, cols, ctypes.byref(err)), err)


def unpack(planes: np.ndarray, rows: int, cols: int) -> np.ndarray:
    planes = np.ascontiguousarray(planes, dtype=np.uint8)
    out = np.empty((rows, cols), dtype=np.int8)
    err = _Err()
    _check(_load().oracle_unpack(_p(planes), planes.size, rows, cols, _p(out), ctypes.byref(err)), err)
    return out


def gemv(planes, rows, cols, x, x_scale=1.0, w_scale=1.0, nthreads=1):
    """Returns (acc int32[rows], y fp32[rows] (scales in turn), y float64[rows])."""
    planes = np.ascontiguousarray(planes, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.int8)
    acc = np.empty(rows, dtype=np.int32)
    y32 = np.empty(rows, dtype=np.float32)
    y64 = np.empty(rows, dtype=np.float64)
    err = _Err()
    rc = _load().oracle_gemv(_p(planes), planes.size, rows, cols, _p(x), x.size, float(x_scale),
                             float(w_scale), _p(acc), _p(y32), _p(y64), int(nthreads), ctypes.byref(err))
    _check(rc, err)
    return acc, y32, y64


def gemv_bitserial(planes, rows, cols, x, nthreads=1):
    planes = np.ascontiguousarray(planes, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.int8)
    acc = np.empty(rows, dtype=np.int32)
    err = _Err()
    rc = _load().oracle_gemv_bitserial(_p(planes), planes.size, rows, cols, _p(x), x.size, _p(acc),
                                       int(nthreads), ctypes.byref(err))
    _check(rc, err)
    return acc


def gemm_small_batch(planes, rows, cols, X, x_scales, w_scale=1.0, nthreads=1):
    """X int8 [batch, ldx]; returns (acc int32[batch, rows], y32, y64)."""
    planes = np.ascontiguousarray(planes, dtype=np.uint8)
    X = np.ascontiguousarray(X, dtype=np.int8)
    batch, ldx = X.shape
    xs = np.ascontiguousarray(x_scales, dtype=np.float32)
    acc = np.empty((batch, rows), dtype=np.int32)
    y32 = np.empty((batch, rows), dtype=np.float32)
    y64 = np.empty((batch, rows), dtype=np.float64)
    err = _Err()
    rc = _load().oracle_gemm_small_batch(_p(planes), planes.size, rows, cols, _p(X), batch, ldx, _p(xs),
                                         float(w_scale), _p(acc), _p(y32), _p(y64), int(nthreads),
                                         ctypes.byref(err))
    _check(rc, err)
    return acc, y32, y64


def dense_head(w_bf16: np.ndarray, x_bf16: np.ndarray, nthreads=1):
    """bf16 bit patterns (uint16) W [rows, cols], x [cols] -> (y float64[rows], sum|w*x| float64[rows])."""
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = w.shape
    assert x.size >= cols
    y = np.empty(rows, dtype=np.float64)
    s = np.empty(rows, dtype=np.float64)
    rc = _load().oracle_dense_head(_p(w), rows, cols, _p(x), _p(y), _p(s), int(nthreads))
    if rc != OK:
        raise OracleError(rc, -1, -1, -1)
    return y, s


def quantize(h: np.ndarray, g: np.ndarray, eps: float, folded: bool) -> tuple[np.ndarray, float]:
    """Activation codes and scale of the Reference (folded=False) or Folded (folded=True) mode:
    int8[n] codes and the float32 scale (see oracle_quantize in oracle.c)."""
    h = np.ascontiguousarray(h, dtype=np.float32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    assert h.shape == g.shape and h.ndim == 1
    q = np.empty(h.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    rc = _load().oracle_quantize(_p(h), _p(g), h.size, float(eps), int(bool(folded)), _p(q), _p(s))
    if rc != OK:
        raise OracleError(rc, -1, -1, -1)
    return q, float(s[0])


def intmlp(gate_planes, up_planes, rows, cols, x, x_scale, w_gate, w_up, nthreads=1):
    """IntMlp epilogue of a gate/up pair sharing x (see oracle_intmlp in oracle.c): returns
    (t int64[rows] = relu(a_g)^2 * a_u, K float64 = S_g^2 * S_u, a_g int32[rows], a_u int32[rows])."""
    g = np.ascontiguousarray(gate_planes, dtype=np.uint8)
    u = np.ascontiguousarray(up_planes, dtype=np.uint8)
    x = np.ascontiguousarray(x, dtype=np.int8)
    if g.size != u.size:
        raise OracleError(E_SIZE, -1, -1, -1)
    t = np.empty(max(rows, 1), dtype=np.int64)[:rows]
    k = np.zeros(1, dtype=np.float64)
    ag = np.empty(max(rows, 1), dtype=np.int32)[:rows]
    au = np.empty(max(rows, 1), dtype=np.int32)[:rows]
    err = _Err()
    rc = _load().oracle_intmlp(_p(g), _p(u), g.size, rows, cols, _p(x), x.size, float(x_scale), float(w_gate),
                               float(w_up), _p(t), _p(k), _p(ag), _p(au), int(nthreads), ctypes.byref(err))
    _check(rc, err)
    return t, float(k[0]), ag, au


def bitcos_pack_flat(w):
    """Flat BITCOS of a ternary array (any shape, flattened): (bitmap bytes, sign bytes, nnz)."""
    w = np.ascontiguousarray(w, dtype=np.int8).reshape(-1)
    n = w.size
    bitmap = np.zeros(max((n + 7) // 8, 1), np.uint8)
    signs = np.zeros(max((n + 7) // 8, 1), np.uint8)
    nnz = np.zeros(1, np.int64)
    rc = _load().oracle_bitcos_pack_flat(_p(w), n, _p(bitmap), _p(signs), _p(nnz))
    if rc != OK:
        raise OracleError(rc, -1, -1, -1)
    k = int(nnz[0])
    return bitmap[: (n + 7) // 8].tobytes(), signs[: (k + 7) // 8].tobytes(), k


def bitcos_unpack_flat(bitmap: bytes, signs: bytes, n: int) -> np.ndarray:
    """n weights from a flat bitmap and sign vector; OracleError(SIZE) when the bitmap has more set
    bits than the sign bytes hold."""
    b = np.frombuffer(bitmap, np.uint8).copy() if bitmap else np.zeros(1, np.uint8)
    s = np.frombuffer(signs, np.uint8).copy() if signs else np.zeros(1, np.uint8)
    w = np.zeros(max(n, 1), np.int8)
    rc = _load().oracle_bitcos_unpack_flat(_p(b), len(bitmap), _p(s), len(signs), n, _p(w))
    if rc != OK:
        raise OracleError(rc, -1, -1, -1)
    return w[:n]


def bitcos_pack_rows(w):
    """Row-form BITCOS of a [rows, cols] ternary matrix: (presence u64[rows*bpr], sign words u32,
    row_start u32[rows+1])."""
    w = np.ascontiguousarray(w, dtype=np.int8)
    rows, cols = w.shape
    bpr = (cols + 63) // 64
    row_start = np.zeros(rows + 1, np.uint32)
    rc = _load().oracle_bitcos_pack_rows(_p(w), rows, cols, None, None, _p(row_start))
    if rc != OK:
        raise OracleError(rc, -1, -1, -1)
    presence = np.zeros(max(rows * bpr, 1), np.uint64)
    signs = np.zeros(max(int(row_start[rows]), 1), np.uint32)
    rc = _load().oracle_bitcos_pack_rows(_p(w), rows, cols, _p(presence), _p(signs), _p(row_start))
    if rc != OK:
        raise OracleError(rc, -1, -1, -1)
    return presence[: rows * bpr], signs[: int(row_start[rows])], row_start


def bitcos_gemv(presence, signs, row_start, rows, cols, x, x_scale=1.0, w_scale=1.0, nthreads=1):
    """Returns (acc int32[rows], y fp32[rows], y float64[rows]) from the row form."""
    presence = np.ascontiguousarray(presence, dtype=np.uint64)
    signs = np.ascontiguousarray(signs, dtype=np.uint32)
    row_start = np.ascontiguousarray(row_start, dtype=np.uint32)
    x = np.ascontiguousarray(x, dtype=np.int8)
    acc = np.empty(max(rows, 1), np.int32)
    y32 = np.empty(max(rows, 1), np.float32)
    y64 = np.empty(max(rows, 1), np.float64)
    rc = _load().oracle_bitcos_gemv(_p(presence) if presence.size else None, _p(signs) if signs.size else None,
                                    _p(row_start), rows, cols, _p(x), float(x_scale), float(w_scale), _p(acc),
                                    _p(y32), _p(y64), int(nthreads))
    if rc != OK:
        raise OracleError(rc, -1, -1, -1)
    return acc[:rows], y32[:rows], y64[:rows]
