"""bit_plane_weight_amd - ternary bit-plane (.trit v1) GEMV on AMD Instinct MI355X (gfx950).

A thin binding over libbpw's C ABI (include/bpw.h) with the same entry-point names. Every step
of the computation runs in libbpw's HIP kernels; this module only marshals arguments. PyTorch
is used for device memory (tensors passed by data_ptr()) and streams. Host buffers are numpy
arrays.
"""
from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from ._lib import (BpwDevMat, BpwError, BpwGemvJob, BpwQuantJob, KERNEL_AUTO, KERNEL_BITSERIAL,  # noqa: F401
                   KERNEL_BYTELANE, KERNEL_MFMA)

__all__ = [
    "BpwError", "KERNEL_AUTO", "KERNEL_BITSERIAL", "KERNEL_BYTELANE", "KERNEL_MFMA",
    "bpw_abi_version", "bpw_status_string", "bpw_last_error", "bpw_device_check",
    "bpw_pack_i8", "bpw_validate", "bpw_load", "HostMat", "bpw_upload", "DevMat",
    "gemv_job", "bpw_gemv_workspace_bytes", "bpw_gemv", "bpw_gemv_noalloc", "GemvPlan",
    "intmlp_job", "bpw_gemv_intmlp_workspace_bytes",
    "bpw_gemm_small_batch", "sb_job", "bpw_gemm_small_batch_workspace_bytes", "SmallBatchPlan", "quant_job", "bpw_quantize_workspace_bytes", "bpw_quantize", "QuantPlan",
    "bpw_dense_head_gemv", "bpw_stream_read_probe", "PROBE_SHAPES", "bpw_cache_flush",
    "TritFile", "TritFormatError", "TritTensor", "bpw_fnv1a64", "trit_write", "TRIT_F32", "TRIT_TERNARY", "TRIT_BF16",
    "BitcosHost", "bpw_bitcos_pack_i8", "bpw_bitcos_from_planes", "DevBitcos", "bpw_bitcos_upload", "bitcos_job",
    "bpw_bitcos_workspace_bytes", "BitcosPlan",
]


def _np(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _dptr(t) -> int | None:
    """Device address of a torch tensor (None stays NULL)."""
    if t is None:
        return None
    if not getattr(t, "is_cuda", False):
        raise TypeError("expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError("GPU tensor must be contiguous")
    return t.data_ptr()


def _checked(t, dtype: str, n: int, what: str) -> int | None:
    """Device address of a tensor the kernels read or write, after checking its element type and
    that it holds at least n elements (None stays NULL). The C ABI carries no lengths for outputs,
    so this is where an undersized or mistyped buffer is refused, before anything is launched."""
    if t is None:
        return None
    import torch
    want = getattr(torch, dtype)
    if t.dtype != want:
        raise TypeError(f"{what} must be {want}, got {t.dtype}")
    if t.numel() < n:
        raise ValueError(f"{what} holds {t.numel()} elements, needs at least {n}")
    return _dptr(t)


def _bytes_of(t, what: str) -> int:
    """Byte length of a one-byte-element tensor (int8 codes, uint8 planes)."""
    if t.element_size() != 1:
        raise TypeError(f"{what} must have one-byte elements (int8 or uint8), got {t.dtype}")
    return t.numel()


class _Job:
    """One job of a grouped call: the ctypes record the C ABI reads (``c``) plus every object whose
    device memory that record names (the matrix and its plane buffer, activations, scales, outputs).
    Plans hold their jobs, so those buffers live as long as the plan that launches on them."""

    def __init__(self, c, keep):
        object.__setattr__(self, "c", c)
        object.__setattr__(self, "_keep", keep)

    # the record's fields read and write through the job (job.d_x, job.m.rows, ...)
    def __getattr__(self, name):
        return getattr(self.c, name)

    def __setattr__(self, name, value):
        setattr(self.c, name, value)


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


# ------------------------------------------------------------------------------ library


def bpw_abi_version() -> int:
    return _lib.lib().bpw_abi_version()


def bpw_status_string(status: int) -> str:
    return _lib.lib().bpw_status_string(status).decode()


def bpw_last_error() -> str:
    return _lib.lib().bpw_last_error().decode()


def bpw_device_check() -> None:
    _lib.check(_lib.lib().bpw_device_check())


# ------------------------------------------------------------------------------ host side


def bpw_pack_i8(w: np.ndarray) -> np.ndarray:
    """int8 [rows, cols] in {-1, 0, +1} -> .trit v1 plane bytes (uint8 [rows * bpr * 16])."""
    w = _np(w, np.int8)
    rows, cols = w.shape
    out = np.empty(rows * ((cols + 63) // 64) * 16, dtype=np.uint8)
    err = _lib.BpwErr()
    _lib.check(_lib.lib().bpw_pack_i8(w.ctypes.data, rows, cols, out.ctypes.data, out.size, ctypes.byref(err)),
               err)
    return out


def bpw_validate(planes: np.ndarray, rows: int, cols: int) -> None:
    planes = _np(planes, np.uint8)
    err = _lib.BpwErr()
    _lib.check(_lib.lib().bpw_validate(planes.ctypes.data, planes.size, rows, cols, ctypes.byref(err)), err)


class HostMat:
    """A validated, library-owned host copy of one matrix's planes (bpw_host_mat)."""

    def __init__(self, handle: int, rows: int, cols: int, w_scale: float):
        self._h = ctypes.c_void_p(handle)
        self.rows, self.cols, self.w_scale = rows, cols, w_scale

    @property
    def nbytes(self) -> int:
        return _lib.lib().bpw_host_mat_bytes(self._h)

    def free(self) -> None:
        if self._h:
            _lib.lib().bpw_host_mat_free(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def bpw_load(planes: np.ndarray, rows: int, cols: int, w_scale: float) -> HostMat:
    planes = _np(planes, np.uint8)
    h = ctypes.c_void_p()
    err = _lib.BpwErr()
    _lib.check(_lib.lib().bpw_load(planes.ctypes.data, planes.size, rows, cols, float(w_scale), ctypes.byref(h),
                                   ctypes.byref(err)), err)
    return HostMat(h.value, rows, cols, w_scale)


class DevMat:
    """A matrix resident on the GPU (bpw_dev_mat) plus the tensor that holds its planes."""

    def __init__(self, desc: BpwDevMat, buf):
        self.desc, self.buf = desc, buf

    @property
    def rows(self) -> int:
        return self.desc.rows

    @property
    def cols(self) -> int:
        return self.desc.cols

    @property
    def bpr(self) -> int:
        return self.desc.bpr


def bpw_upload(m: HostMat, d_buf, stream=None) -> DevMat:
    """Copy m's planes into the uint8 GPU tensor d_buf (>= m.nbytes, 256-byte aligned)."""
    desc = BpwDevMat()
    nbytes = d_buf.numel() * d_buf.element_size()
    _lib.check(_lib.lib().bpw_upload(m._h, _dptr(d_buf), nbytes, _stream(stream), ctypes.byref(desc)))
    return DevMat(desc, d_buf)


# ------------------------------------------------------------------------------ batch-1 GEMV


def gemv_job(m: DevMat, x, x_scale: float, out_i32, out_f32=None, x_scale_dev=None) -> _Job:
    """One bpw_gemv_job: x int8 GPU tensor (>= bpr * 64 bytes), outputs int32 / float32 [rows].
    x_scale_dev (a float32 GPU tensor of one element) makes the kernel read the scale there. The
    returned job keeps m, x, the outputs and x_scale_dev alive."""
    j = BpwGemvJob()
    j.m = m.desc
    j.x_len = _bytes_of(x, "x")
    j.d_x = _dptr(x)
    j.x_scale = float(x_scale)
    if out_i32 is None:
        raise ValueError("out_i32 is required")
    j.d_out_i32 = _checked(out_i32, "int32", m.rows, "out_i32")
    j.d_out_f32 = _checked(out_f32, "float32", m.rows, "out_f32")
    j.d_x_scale = _checked(x_scale_dev, "float32", 1, "x_scale_dev")
    return _Job(j, (m, x, out_i32, out_f32, x_scale_dev))


def _records(jobs, ctype):
    """ctypes array of the jobs' records (a _Job's ``c``, or a bare record)."""
    recs = [j.c if isinstance(j, _Job) else j for j in jobs]
    return (ctype * max(1, len(recs)))(*recs), len(recs)


def _jobs_array(jobs):
    return _records(jobs, BpwGemvJob)


def bpw_gemv_workspace_bytes(jobs) -> int:
    arr, n = _jobs_array(jobs)
    return _lib.lib().bpw_gemv_workspace_bytes(arr, n)


def intmlp_job(gate: DevMat, up: DevMat, x, x_scale: float, t_out, k_out, gate_i32=None, up_i32=None,
               x_scale_dev=None) -> _Job:
    """One bpw_intmlp_job: gate and up (same shape) read the int8 GPU tensor x; t_out int64 [rows]
    receives relu(a_g)^2 * a_u, k_out float64 [1] receives K; gate_i32 / up_i32 optional int32 [rows]."""
    j = _lib.BpwIntMlpJob()
    j.gate = gate.desc
    j.up = up.desc
    j.x_len = _bytes_of(x, "x")
    j.d_x = _dptr(x)
    j.x_scale = float(x_scale)
    j.d_x_scale = _checked(x_scale_dev, "float32", 1, "x_scale_dev")
    if t_out is None or k_out is None:
        raise ValueError("t_out and k_out are required")
    j.d_t = _checked(t_out, "int64", gate.rows, "t_out")
    j.d_k = _checked(k_out, "float64", 1, "k_out")
    j.d_gate_i32 = _checked(gate_i32, "int32", gate.rows, "gate_i32")
    j.d_up_i32 = _checked(up_i32, "int32", gate.rows, "up_i32")
    return _Job(j, (gate, up, x, x_scale_dev, t_out, k_out, gate_i32, up_i32))


def _mlp_array(mlp):
    return _records(list(mlp or []), _lib.BpwIntMlpJob)


def bpw_gemv_intmlp_workspace_bytes(jobs, mlp) -> int:
    arr, n = _jobs_array(jobs)
    marr, nm = _mlp_array(mlp)
    return _lib.lib().bpw_gemv_intmlp_workspace_bytes(arr, n, marr, nm)


def bpw_gemv(jobs, d_ws, kernel: int = KERNEL_AUTO, stream=None) -> None:
    arr, n = _jobs_array(jobs)
    ws_len = 0 if d_ws is None else d_ws.numel() * d_ws.element_size()
    _lib.check(_lib.lib().bpw_gemv(arr, n, kernel, _dptr(d_ws), ws_len, _stream(stream)))


def bpw_gemv_noalloc(jobs, kernel: int = KERNEL_AUTO, stream=None) -> None:
    """bpw_gemv with the library's fixed device scratch in place of a workspace (allocates nothing)."""
    arr, n = _jobs_array(jobs)
    _lib.check(_lib.lib().bpw_gemv_noalloc(arr, n, kernel, _stream(stream)))


class GemvPlan:
    """bpw_gemv_plan: the job table written once into d_ws; run() queues the one launch. With mlp
    (a list of intmlp_job) the plan is made by bpw_gemv_intmlp_plan_create."""

    def __init__(self, jobs, d_ws, kernel: int = KERNEL_AUTO, stream=None, mlp=None):
        arr, n = _jobs_array(jobs)
        ws_len = 0 if d_ws is None else d_ws.numel() * d_ws.element_size()
        h = ctypes.c_void_p()
        if mlp is None:
            _lib.check(_lib.lib().bpw_gemv_plan_create(arr, n, kernel, _dptr(d_ws), ws_len, _stream(stream),
                                                       ctypes.byref(h)))
        else:
            marr, nm = _mlp_array(mlp)
            _lib.check(_lib.lib().bpw_gemv_intmlp_plan_create(arr, n, marr, nm, kernel, _dptr(d_ws), ws_len,
                                                              _stream(stream), ctypes.byref(h)))
        self._h, self._keep = h, (jobs, mlp, d_ws)

    def run(self, stream=None) -> None:
        _lib.check(_lib.lib().bpw_gemv_plan_run(self._h, _stream(stream)))

    def free(self) -> None:
        if self._h:
            _lib.lib().bpw_gemv_plan_free(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


# ------------------------------------------------------------------------------ quantiser


def quant_job(h, g, q, scale, eps: float) -> _Job:
    """One bpw_quant_job: h, g float32 GPU tensors [n]; q int8 GPU tensor (>= n); scale float32 [1]."""
    j = BpwQuantJob()
    j.n = h.numel()
    if g.numel() != j.n:
        raise ValueError("h and g must have the same length")
    j.d_h, j.d_g = _checked(h, "float32", j.n, "h"), _checked(g, "float32", j.n, "g")
    j.q_len = _bytes_of(q, "q")
    j.d_q = _dptr(q)
    if scale is None:
        raise ValueError("scale is required")
    j.d_scale = _checked(scale, "float32", 1, "scale")
    j.eps = float(eps)
    return _Job(j, (h, g, q, scale))


def _quant_array(jobs):
    return _records(jobs, BpwQuantJob)


def bpw_quantize_workspace_bytes(n_jobs: int) -> int:
    return _lib.lib().bpw_quantize_workspace_bytes(n_jobs)


def bpw_quantize(jobs, d_ws, stream=None) -> None:
    arr, n = _quant_array(jobs)
    ws_len = 0 if d_ws is None else d_ws.numel() * d_ws.element_size()
    _lib.check(_lib.lib().bpw_quantize(arr, n, _dptr(d_ws), ws_len, _stream(stream)))


class QuantPlan:
    """bpw_quant_plan: the quantiser's job table written once into d_ws; run() queues one launch."""

    def __init__(self, jobs, d_ws, stream=None):
        arr, n = _quant_array(jobs)
        ws_len = 0 if d_ws is None else d_ws.numel() * d_ws.element_size()
        h = ctypes.c_void_p()
        _lib.check(_lib.lib().bpw_quant_plan_create(arr, n, _dptr(d_ws), ws_len, _stream(stream), ctypes.byref(h)))
        self._h, self._keep = h, (jobs, d_ws)

    def run(self, stream=None) -> None:
        _lib.check(_lib.lib().bpw_quant_plan_run(self._h, _stream(stream)))

    def free(self) -> None:
        if self._h:
            _lib.lib().bpw_quant_plan_free(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


# ------------------------------------------------------------------------------ small batch


def bpw_gemm_small_batch(m: DevMat, X, x_scales, out_i32, out_f32, kernel: int = KERNEL_AUTO, stream=None) -> None:
    """X int8 GPU tensor [batch, ldx]; x_scales host float32 [batch]; outputs [batch, rows]."""
    batch, ldx = X.shape
    _bytes_of(X, "X")
    xs = np.ascontiguousarray(np.asarray(x_scales, dtype=np.float32))
    if xs.shape != (batch,):
        raise ValueError(f"x_scales must hold {batch} values")
    if out_i32 is None:
        raise ValueError("out_i32 is required")
    oi = _checked(out_i32, "int32", batch * m.rows, "out_i32")
    of = _checked(out_f32, "float32", batch * m.rows, "out_f32")
    _lib.check(_lib.lib().bpw_gemm_small_batch(ctypes.byref(m.desc), _dptr(X), batch, ldx, xs.ctypes.data,
                                               oi, of, kernel, _stream(stream)))


class _SbJob:
    """One grouped small-batch job; keeps its host scales alive until the plan has copied them, and
    its device tensors as long as the job (the plan reads X and writes the outputs at every run)."""

    def __init__(self, m: DevMat, X, x_scales, out_i32, out_f32=None):
        batch, ldx = X.shape
        self.batch = batch
        self.scales = np.ascontiguousarray(np.asarray(x_scales, dtype=np.float32))
        if self.scales.shape != (batch,):
            raise ValueError(f"x_scales must hold {batch} values")
        _bytes_of(X, "X")
        if out_i32 is None:
            raise ValueError("out_i32 is required")
        j = _lib.BpwSbJob()
        j.m = m.desc
        j.d_X = _dptr(X)
        j.ldx = ldx
        j.x_scales = self.scales.ctypes.data
        j.d_out_i32 = _checked(out_i32, "int32", batch * m.rows, "out_i32")
        j.d_out_f32 = _checked(out_f32, "float32", batch * m.rows, "out_f32")
        self.c = j
        self._keep = (m, X, out_i32, out_f32)


def sb_job(m: DevMat, X, x_scales, out_i32, out_f32=None) -> _SbJob:
    """One job of a grouped small-batch plan: X int8 GPU tensor [batch, ldx], x_scales host [batch],
    outputs [batch, rows]."""
    return _SbJob(m, X, x_scales, out_i32, out_f32)


def _sb_array(jobs):
    arr = (_lib.BpwSbJob * max(1, len(jobs)))(*[j.c for j in jobs])
    return arr, len(jobs)


def bpw_gemm_small_batch_workspace_bytes(jobs, batch: int) -> int:
    arr, n = _sb_array(jobs)
    return _lib.lib().bpw_gemm_small_batch_workspace_bytes(arr, n, batch)


class SmallBatchPlan:
    """bpw_sb_plan: several small-batch calls with one batch size, one launch per run()."""

    def __init__(self, jobs, batch: int, d_ws, kernel: int = KERNEL_AUTO, stream=None):
        if any(j.batch != batch for j in jobs):
            raise ValueError(f"every job's X must hold batch = {batch} rows")
        arr, n = _sb_array(jobs)
        ws_len = 0 if d_ws is None else d_ws.numel() * d_ws.element_size()
        h = ctypes.c_void_p()
        _lib.check(_lib.lib().bpw_gemm_small_batch_plan_create(arr, n, batch, kernel, _dptr(d_ws), ws_len,
                                                               _stream(stream), ctypes.byref(h)))
        self._h, self._keep = h, (jobs, d_ws)

    def run(self, stream=None) -> None:
        _lib.check(_lib.lib().bpw_gemm_small_batch_plan_run(self._h, _stream(stream)))

    def free(self) -> None:
        if self._h:
            _lib.lib().bpw_gemm_small_batch_plan_free(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


# ------------------------------------------------------------------------------ .trit v1 container

TRIT_F32, TRIT_TERNARY, TRIT_BF16 = 0, 1, 2


class TritFormatError(BpwError):
    """A failed container check: check is its number in the format page's section 4 (1..19)."""

    def __init__(self, status: int, reason: str, e):
        super().__init__(status, reason, e.row, e.beat, e.col)
        self.check, self.offset, self.tensor = e.check, e.offset, e.tensor


class TritTensor:
    def __init__(self, t, index: int):
        self.index = index
        self.name = ctypes.string_at(t.name, t.name_len).decode("utf-8")
        self.dtype, self.dims = t.dtype, list(t.dims[: t.ndim])
        self.scale, self.offset, self.byte_len = t.scale, t.offset, t.byte_len
        self._data = t.data

    def bytes(self) -> bytes:
        return ctypes.string_at(self._data, self.byte_len) if self.byte_len else b""


def bpw_fnv1a64(data) -> int:
    buf = np.frombuffer(memoryview(data), dtype=np.uint8)
    return _lib.lib().bpw_fnv1a64(buf.ctypes.data if buf.size else None, buf.size)


def trit_write(tensors, config: bytes = b"", with_hash: bool = True) -> bytes:
    """bpw_trit_write: a .trit v1 container from [(name, dtype, dims, scale, data)] (name str, dtype one of
    TRIT_F32 / TRIT_TERNARY / TRIT_BF16, dims a sequence of 1..4 ints, data a bytes-like payload: .trit
    planes for a ternary tensor, little-endian elements otherwise). Records come out sorted by name;
    the same tensors in any order give the same bytes. Raises TritFormatError naming the check a reader
    would fail."""
    arr = (_lib.BpwTritTensorIn * max(1, len(tensors)))()
    keep = []
    for k, (name, dtype, dims, scale, data) in enumerate(tensors):
        nb = name.encode("utf-8") if isinstance(name, str) else bytes(name)
        buf = np.frombuffer(memoryview(data), dtype=np.uint8)
        keep += [nb, buf]
        e = arr[k]
        e.name, e.name_len, e.dtype, e.ndim = nb, len(nb), int(dtype), len(dims)
        if len(dims) > 4:
            raise ValueError(f"tensor {k}: {len(dims)} dims (at most 4)")
        for j, d in enumerate(dims):
            e.dims[j] = int(d)
        e.scale = float(scale)
        e.data = buf.ctypes.data if buf.size else None
        e.byte_len = buf.size
    cfg = bytes(config)
    err = _lib.BpwTritErr()
    need = ctypes.c_uint64()
    st = _lib.lib().bpw_trit_write_size(arr, len(tensors), len(cfg), ctypes.byref(need), ctypes.byref(err))
    if st != _lib.OK:
        raise TritFormatError(st, _lib.lib().bpw_last_error().decode(), err)
    out = np.empty(max(1, need.value), dtype=np.uint8)
    written = ctypes.c_uint64()
    st = _lib.lib().bpw_trit_write(arr, len(tensors), cfg, len(cfg), int(bool(with_hash)), out.ctypes.data,
                                   need.value, ctypes.byref(written), ctypes.byref(err))
    if st != _lib.OK:
        raise TritFormatError(st, _lib.lib().bpw_last_error().decode(), err)
    return out[: written.value].tobytes()


class TritFile:
    """bpw_trit_file: a .trit v1 container in host memory (bytes, bytearray, mmap, numpy uint8), opened
    with checks 1-16; verify() runs checks 17-19. The object keeps the buffer alive."""

    def __init__(self, data):
        self._buf = np.frombuffer(memoryview(data), dtype=np.uint8)
        self._h = ctypes.c_void_p()
        err = _lib.BpwTritErr()
        st = _lib.lib().bpw_trit_open(self._buf.ctypes.data if self._buf.size else None, self._buf.size,
                                      ctypes.byref(self._h), ctypes.byref(err))
        if st != _lib.OK:
            raise TritFormatError(st, _lib.lib().bpw_last_error().decode(), err)

    def verify(self, check_hash: bool = True) -> None:
        err = _lib.BpwTritErr()
        st = _lib.lib().bpw_trit_verify(self._h, int(bool(check_hash)), ctypes.byref(err))
        if st != _lib.OK:
            raise TritFormatError(st, _lib.lib().bpw_last_error().decode(), err)

    def __len__(self) -> int:
        return _lib.lib().bpw_trit_tensor_count(self._h)

    def tensor(self, index: int) -> TritTensor:
        t = _lib.BpwTritTensor()
        _lib.check(_lib.lib().bpw_trit_tensor_info(self._h, index, ctypes.byref(t)))
        return TritTensor(t, index)

    @property
    def tensors(self) -> list:
        return [self.tensor(i) for i in range(len(self))]

    def find(self, name: str) -> int:
        nb = name.encode("utf-8")
        return _lib.lib().bpw_trit_find(self._h, nb, len(nb))

    @property
    def config(self) -> bytes:
        p, n = ctypes.c_void_p(), ctypes.c_size_t()
        _lib.check(_lib.lib().bpw_trit_config(self._h, ctypes.byref(p), ctypes.byref(n)))
        return ctypes.string_at(p, n.value) if n.value else b""

    @property
    def stored_hash(self) -> int:
        return _lib.lib().bpw_trit_stored_hash(self._h)

    def load(self, index: int) -> HostMat:
        """A ternary tensor as a validated host matrix (for bpw_upload)."""
        t = self.tensor(index)
        h = ctypes.c_void_p()
        err = _lib.BpwErr()
        _lib.check(_lib.lib().bpw_trit_load(self._h, index, ctypes.byref(h), ctypes.byref(err)), err)
        return HostMat(h.value, t.dims[0], t.dims[1], t.scale)

    def close(self) -> None:
        if self._h:
            _lib.lib().bpw_trit_close(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ------------------------------------------------------------------------------ dense head


def bpw_dense_head_gemv(w_bf16, x_bf16, y, stream=None) -> None:
    """w_bf16 [rows, cols] and x_bf16 [cols] GPU tensors of bf16 bits (int16/uint16/bfloat16); y float32."""
    rows, cols = w_bf16.shape
    for t, what in ((w_bf16, "w_bf16"), (x_bf16, "x_bf16")):
        if t.element_size() != 2:
            raise TypeError(f"{what} must hold 16-bit elements (bf16 bit patterns), got {t.dtype}")
    if x_bf16.numel() < cols:
        raise ValueError(f"x_bf16 holds {x_bf16.numel()} elements, needs at least {cols}")
    _lib.check(_lib.lib().bpw_dense_head_gemv(_dptr(w_bf16), rows, cols, _dptr(x_bf16),
                                              _checked(y, "float32", rows, "y"), _stream(stream)))


# ------------------------------------------------------------------------------ measurement


PROBE_SHAPES = 5


def bpw_stream_read_probe(d_buf, d_sink, stream=None, shape: int = 0) -> None:
    if d_sink is None or d_sink.element_size() != 4 or d_sink.numel() < 1:
        raise ValueError("d_sink must be a 4-byte-element tensor of at least one element")
    _lib.check(_lib.lib().bpw_stream_read_probe_shape(_dptr(d_buf), d_buf.numel() * d_buf.element_size(),
                                                      _dptr(d_sink), int(shape), _stream(stream)))


def bpw_cache_flush(d_buf, stream=None) -> None:
    _lib.check(_lib.lib().bpw_cache_flush(_dptr(d_buf), d_buf.numel() * d_buf.element_size(), _stream(stream)))


# ------------------------------------------------------------------------------ BITCOS


class BitcosHost:
    """A library-owned BITCOS matrix on the host (bpw_bitcos_host)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)

    def arrays(self):
        """(presence uint64 [rows * bpr], signs uint32 [sign_words], row_start uint32 [rows + 1], nnz),
        copied out of the library's arrays."""
        p, s, r = ctypes.c_void_p(), ctypes.c_void_p(), ctypes.c_void_p()
        nw, nnz = ctypes.c_int64(), ctypes.c_int64()
        _lib.check(_lib.lib().bpw_bitcos_arrays(self._h, ctypes.byref(p), ctypes.byref(s), ctypes.byref(r),
                                                ctypes.byref(nw), ctypes.byref(nnz)))
        rows = self.rows

        def view(ptr, n, ct, dt):
            if n == 0:
                return np.zeros(0, dt)
            return np.ctypeslib.as_array(ctypes.cast(ptr, ctypes.POINTER(ct)), shape=(n,)).copy()

        return (view(p, rows * self.bpr, ctypes.c_uint64, np.uint64), view(s, nw.value, ctypes.c_uint32, np.uint32),
                view(r, rows + 1, ctypes.c_uint32, np.uint32), nnz.value)

    @property
    def device_bytes(self) -> int:
        return _lib.lib().bpw_bitcos_device_bytes(self._h)

    def free(self) -> None:
        if self._h:
            _lib.lib().bpw_bitcos_free(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def bpw_bitcos_pack_i8(w: np.ndarray, w_scale: float) -> BitcosHost:
    """int8 [rows, cols] in {-1, 0, +1} -> a BITCOS matrix."""
    w = _np(w, np.int8)
    rows, cols = w.shape
    h = ctypes.c_void_p()
    err = _lib.BpwErr()
    _lib.check(_lib.lib().bpw_bitcos_pack_i8(w.ctypes.data, rows, cols, float(w_scale), ctypes.byref(h),
                                             ctypes.byref(err)), err)
    out = BitcosHost(h.value)
    out.rows, out.cols, out.bpr, out.w_scale = rows, cols, (cols + 63) // 64, w_scale
    return out


def bpw_bitcos_from_planes(m: HostMat) -> BitcosHost:
    """The same matrix as a validated .trit host matrix, re-encoded."""
    h = ctypes.c_void_p()
    _lib.check(_lib.lib().bpw_bitcos_from_planes(m._h, ctypes.byref(h)))
    out = BitcosHost(h.value)
    out.rows, out.cols, out.bpr, out.w_scale = m.rows, m.cols, (m.cols + 63) // 64, m.w_scale
    return out


class DevBitcos:
    """A BITCOS matrix resident on the GPU (bpw_dev_bitcos) plus the tensor that holds it."""

    def __init__(self, desc: _lib.BpwDevBitcos, buf):
        self.desc, self.buf = desc, buf

    @property
    def rows(self) -> int:
        return self.desc.rows

    @property
    def cols(self) -> int:
        return self.desc.cols

    @property
    def bpr(self) -> int:
        return self.desc.bpr


def bpw_bitcos_upload(h: BitcosHost, d_buf, stream=None) -> DevBitcos:
    """Copy h into the uint8 GPU tensor d_buf (>= h.device_bytes, 256-byte aligned)."""
    desc = _lib.BpwDevBitcos()
    nbytes = d_buf.numel() * d_buf.element_size()
    _lib.check(_lib.lib().bpw_bitcos_upload(h._h, _dptr(d_buf), nbytes, _stream(stream), ctypes.byref(desc)))
    return DevBitcos(desc, d_buf)


def bitcos_job(m: DevBitcos, x, x_scale: float, out_i32, out_f32=None) -> _Job:
    """One bpw_bitcos_job (outputs int32 / float32 [rows]); the job keeps m, x and the outputs alive."""
    j = _lib.BpwBitcosJob()
    j.m = m.desc
    j.x_len = _bytes_of(x, "x")
    j.d_x = _dptr(x)
    j.x_scale = float(x_scale)
    if out_i32 is None:
        raise ValueError("out_i32 is required")
    j.d_out_i32 = _checked(out_i32, "int32", m.rows, "out_i32")
    j.d_out_f32 = _checked(out_f32, "float32", m.rows, "out_f32")
    return _Job(j, (m, x, out_i32, out_f32))


def _bitcos_array(jobs):
    return _records(list(jobs), _lib.BpwBitcosJob)


def bpw_bitcos_workspace_bytes(jobs) -> int:
    arr, n = _bitcos_array(jobs)
    return _lib.lib().bpw_bitcos_workspace_bytes(arr, n)


class BitcosPlan:
    """bpw_bitcos_plan: job and tile tables written once into d_ws; run() queues the one launch."""

    def __init__(self, jobs, d_ws, stream=None):
        arr, n = _bitcos_array(jobs)
        ws_len = 0 if d_ws is None else d_ws.numel() * d_ws.element_size()
        h = ctypes.c_void_p()
        _lib.check(_lib.lib().bpw_bitcos_plan_create(arr, n, _dptr(d_ws), ws_len, _stream(stream), ctypes.byref(h)))
        self._h, self._keep = h, (jobs, d_ws)

    def run(self, stream=None) -> None:
        _lib.check(_lib.lib().bpw_bitcos_plan_run(self._h, _stream(stream)))

    def free(self) -> None:
        if self._h:
            _lib.lib().bpw_bitcos_plan_free(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass
