"""The C-ABI library on the host (no GPU): it loads, exports every declared symbol, and its host
logic - packing, validation, loading, argument checks that run before any device work - agrees
with the CPU oracle. No kernel is launched here."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import oracle
import synth
from conftest import ROOT, read_worked_example

bpw = pytest.importorskip("bit_plane_weight_amd")
from bit_plane_weight_amd import _lib  # noqa: E402


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \*]*?\b(bpw_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    names = declared_functions()
    assert set(names) >= {"bpw_pack_i8", "bpw_validate", "bpw_load", "bpw_upload", "bpw_gemv", "bpw_gemv_plan_create",
                          "bpw_gemv_plan_run", "bpw_gemm_small_batch", "bpw_dense_head_gemv",
                          "bpw_quantize", "bpw_gemv_intmlp_plan_create"}, names
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert L.bpw_abi_version() == _lib.ABI_VERSION
    assert bpw.bpw_status_string(0) == "BPW_OK"
    assert bpw.bpw_status_string(3) == "BPW_E_P1_BOTH_BITS"
    assert bpw.bpw_status_string(99) == "unknown status"


def test_pack_matches_oracle_bit_for_bit():
    _, _, _, w, payload = read_worked_example()
    assert bpw.bpw_pack_i8(np.array(w, np.int8)).tobytes() == payload
    for rows in (1, 3, 17):
        for cols in (1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 2560, 6912):
            w = synth.trits(rows * 7919 + cols, rows, cols, (0.0, 0.42, 1.0)[cols % 3])
            assert np.array_equal(bpw.bpw_pack_i8(w), oracle.pack(w))
    for z in synth.P_ZERO_SWEEP:
        w = synth.trits(17, 640, 2560, z)
        assert np.array_equal(bpw.bpw_pack_i8(w), oracle.pack(w))


def test_pack_rejects_bad_values_like_oracle():
    for cols, r, c in ((70, 2, 66), (200, 0, 5), (64, 1, 63), (3, 0, 2)):
        w = np.zeros((3, cols), np.int8)
        w[r, c] = 5 if c % 2 else -2
        with pytest.raises(bpw.BpwError) as ei:
            bpw.bpw_pack_i8(w)
        with pytest.raises(oracle.OracleError) as eo:
            oracle.pack(w)
        assert ei.value.status == _lib.E_INVAL
        assert (ei.value.row, ei.value.beat, ei.value.col) == (eo.value.row, eo.value.beat, eo.value.col)


def _corrupt(planes, rows, bpr, r, b, plane, k):
    p = planes.copy().reshape(rows, bpr, 2, 8)
    word = int.from_bytes(p[r, b, plane].tobytes(), "little") | (1 << k)
    p[r, b, plane] = np.frombuffer(word.to_bytes(8, "little"), np.uint8)
    return p.reshape(-1)


@pytest.mark.parametrize("cols", (1, 31, 32, 33, 63, 64, 65, 127, 200))
def test_validate_agrees_with_oracle(cols):
    rows = 4
    bpr = (cols + 63) // 64
    w = synth.trits(cols, rows, cols)
    base = oracle.pack(w)
    bpw.bpw_validate(base, rows, cols)
    rng = np.random.default_rng(cols)
    for _ in range(60):
        p = base
        for _ in range(int(rng.integers(1, 3))):
            p = _corrupt(p, rows, bpr, int(rng.integers(rows)), int(rng.integers(bpr)), int(rng.integers(2)),
                         int(rng.integers(64)))
        try:
            oracle.validate(p, rows, cols)
            o = None
        except oracle.OracleError as e:
            o = e
        try:
            bpw.bpw_validate(p, rows, cols)
            g = None
        except bpw.BpwError as e:
            g = e
        if o is None:
            assert g is None
        else:
            assert g is not None
            code = {oracle.E_P1: _lib.E_P1_BOTH_BITS, oracle.E_P2: _lib.E_P2_PADDING}[o.code]
            assert (g.status, g.row, g.beat, g.col) == (code, o.row, o.beat, o.col)
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_validate(base[:-1], rows, cols)
    assert ei.value.status == _lib.E_SIZE


def test_load_copies_validates_and_checks_scale():
    w = synth.trits(1, 8, 300)
    planes = oracle.pack(w)
    hm = bpw.bpw_load(planes, 8, 300, 0.75)
    assert hm.nbytes == planes.size
    planes[:] = 0xFF  # the library holds its own validated copy
    hm.free()
    bad = _corrupt(oracle.pack(w), 8, 5, 3, 2, 0, 0)
    bad = _corrupt(bad, 8, 5, 3, 2, 1, 0)
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_load(bad, 8, 300, 1.0)
    assert (ei.value.status, ei.value.row, ei.value.beat, ei.value.col) == (_lib.E_P1_BOTH_BITS, 3, 2, 128)
    for s in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(bpw.BpwError) as ei:
            bpw.bpw_load(oracle.pack(w), 8, 300, s)
        assert ei.value.status == _lib.E_INVAL


def test_forged_descriptor_is_refused_before_any_device_work():
    L = _lib.lib()
    d = _lib.BpwDevMat()
    d.d_planes = 0x10000
    d.rows, d.cols, d.bpr, d.w_scale = 4, 64, 1, 1.0
    d.seal = 0x1234
    j = _lib.BpwGemvJob()
    j.m = d
    j.d_x = 0x20000
    j.x_len = 64
    j.d_out_i32 = 0x30000
    arr = (_lib.BpwGemvJob * 1)(j)
    st = L.bpw_gemv(arr, 1, 0, ctypes.c_void_p(0x40000), 1 << 20, None)
    assert st == _lib.E_NOT_VALIDATED
    assert "bpw_upload" in bpw.bpw_last_error()
    st = L.bpw_gemm_small_batch(ctypes.byref(d), ctypes.c_void_p(0x20000), 2, 64,
                                (ctypes.c_float * 2)(1, 1), ctypes.c_void_p(0x30000), None, 0, None)
    assert st == _lib.E_NOT_VALIDATED


def test_forged_intmlp_pair_is_refused_and_bytelane_cannot_serve_pairs():
    L = _lib.lib()
    d = _lib.BpwDevMat()
    d.d_planes = 0x10000
    d.rows, d.cols, d.bpr, d.w_scale = 4, 64, 1, 1.0
    d.seal = 0x1234
    p = _lib.BpwIntMlpJob()
    p.gate = d
    p.up = d
    p.d_x = 0x20000
    p.x_len = 64
    p.d_t = 0x30000
    p.d_k = 0x38000
    arr = (_lib.BpwIntMlpJob * 1)(p)
    h = ctypes.c_void_p()
    assert L.bpw_gemv_intmlp_plan_create(None, 0, arr, 1, 0, ctypes.c_void_p(0x40000), 1 << 20, None,
                                         ctypes.byref(h)) == _lib.E_NOT_VALIDATED
    assert "pair 0 gate" in bpw.bpw_last_error()
    assert L.bpw_gemv_intmlp_plan_create(None, 0, arr, 1, 2, ctypes.c_void_p(0x40000), 1 << 20, None,
                                         ctypes.byref(h)) == _lib.E_UNSUPPORTED
    assert L.bpw_gemv_intmlp_plan_create(None, 0, None, 1, 0, None, 0, None, ctypes.byref(h)) == _lib.E_INVAL
    assert L.bpw_gemv_intmlp_workspace_bytes(None, 0, None, 0) == 0


def test_empty_and_bad_arguments():
    L = _lib.lib()
    assert L.bpw_gemv(None, 0, 0, None, 0, None) == _lib.OK
    assert L.bpw_gemv_workspace_bytes(None, 0) == 0
    j = (_lib.BpwGemvJob * 1)()
    h = ctypes.c_void_p()
    assert L.bpw_gemv_plan_create(j, 1, 7, None, 0, None, ctypes.byref(h)) == _lib.E_UNSUPPORTED
    assert L.bpw_dense_head_gemv(None, 10, 12, None, None, None) == _lib.E_INVAL
    assert L.bpw_stream_read_probe(None, 16, None, None) == _lib.E_INVAL
    for shape in (-1, 5, 99):  # checked before any device call
        assert L.bpw_stream_read_probe_shape(256, 16, 512, shape, None) == _lib.E_INVAL


def test_device_check_without_gpu_is_an_error_not_a_fallback():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; covered by the GPU tests")
    st = _lib.lib().bpw_device_check()
    assert st in (_lib.E_HIP, _lib.E_ARCH)
