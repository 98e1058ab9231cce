"""libbpw's BITCOS packers on the host (no GPU): bpw_bitcos_pack_i8 and bpw_bitcos_from_planes give
the oracle's row form ("BITCOS: Intel's Ternary LLM Weight Format Goes Below 1.58 Bits", "A bitmap
and a sign") array for array, over ragged shapes and the zero-density range; errors carry the
position; limits are refused before anything is built."""
import numpy as np
import pytest

import oracle
import synth

bpw = pytest.importorskip("bit_plane_weight_amd")
from bit_plane_weight_amd import _lib  # noqa: E402

SHAPES = ((1, 1), (3, 63), (5, 64), (7, 65), (17, 200), (9, 2560), (4, 6912), (3, 8192), (0, 100), (5, 0), (0, 0))


def same_as_oracle(h, w):
    p, s, r, nnz = h.arrays()
    P, S, R = oracle.bitcos_pack_rows(w)
    assert np.array_equal(p, P) and np.array_equal(s, S) and np.array_equal(r, R)
    assert nnz == int(np.count_nonzero(w))
    return p, s, r


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_pack_i8_equals_oracle(rows, cols):
    w = synth.trits(rows * 7 + cols, rows, cols)
    h = bpw.bpw_bitcos_pack_i8(w, 0.75)
    same_as_oracle(h, w)
    h.free()


@pytest.mark.parametrize("z", (0.0, 0.2966, 0.5148, 0.95, 1.0))
def test_pack_i8_zero_density_range(z):
    w = synth.trits(33, 40, 2500, min(z, 0.9999)) if z < 1 else np.zeros((40, 2500), np.int8)
    if z == 0.0:
        w = np.where(synth.trits(34, 40, 2500, 0.5) < 0, -1, 1).astype(np.int8)  # no zeros at all
    h = bpw.bpw_bitcos_pack_i8(w, 1.0)
    p, s, r = same_as_oracle(h, w)
    bpr = (2500 + 63) // 64
    assert p.size == 40 * bpr and r[-1] == s.size
    # per row (k + 31) // 32 words; with no zeros every row has 2500 nonzeros
    if z == 0.0:
        assert np.all(np.diff(r.astype(np.int64)) == (2500 + 31) // 32)
    if z == 1.0:
        assert s.size == 0 and np.all(p == 0)


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_from_planes_equals_pack_i8(rows, cols):
    w = synth.trits(rows * 11 + cols + 1, rows, cols)
    hm = bpw.bpw_load(bpw.bpw_pack_i8(w), rows, cols, 2.0)
    h = bpw.bpw_bitcos_from_planes(hm)
    same_as_oracle(h, w)
    g = bpw.bpw_bitcos_pack_i8(w, 2.0)
    assert h.device_bytes == g.device_bytes
    hm.free()


def test_device_bytes_layout():
    # presence, row_start and signs (+ four zero words) each start at a 256-byte boundary
    w = synth.trits(5, 17, 200)
    h = bpw.bpw_bitcos_pack_i8(w, 1.0)
    p, s, r, _ = h.arrays()
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    assert h.device_bytes == up(p.size * 8) + up(r.size * 4) + up((s.size + 4) * 4)


def test_errors():
    w = np.zeros((3, 70), np.int8)
    w[2, 66] = 2
    with pytest.raises(bpw.BpwError) as e:
        bpw.bpw_bitcos_pack_i8(w, 1.0)
    assert (e.value.status, e.value.row, e.value.beat, e.value.col) == (_lib.E_INVAL, 2, 1, 66)
    with pytest.raises(bpw.BpwError) as e:
        bpw.bpw_bitcos_pack_i8(np.zeros((2, 8193), np.int8), 1.0)
    assert e.value.status == _lib.E_UNSUPPORTED and "8192" in e.value.reason
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        with pytest.raises(bpw.BpwError) as e:
            bpw.bpw_bitcos_pack_i8(np.zeros((2, 8), np.int8), bad)
        assert e.value.status == _lib.E_INVAL
    hm = bpw.bpw_load(bpw.bpw_pack_i8(np.zeros((1, 8193), np.int8)), 1, 8193, 1.0)
    with pytest.raises(bpw.BpwError) as e:
        bpw.bpw_bitcos_from_planes(hm)
    assert e.value.status == _lib.E_UNSUPPORTED
    L = _lib.lib()
    assert L.bpw_bitcos_device_bytes(None) == 0
    assert L.bpw_bitcos_workspace_bytes(None, 0) == 0
    assert L.bpw_bitcos_arrays(None, None, None, None, None, None) == _lib.E_INVAL


def test_forged_descriptor_refused_without_gpu():
    """A descriptor not made by bpw_bitcos_upload fails its seal before any device call."""
    d = _lib.BpwDevBitcos()
    d.rows, d.cols, d.bpr, d.w_scale, d.seal = 8, 64, 1, 1.0, 12345
    j = _lib.BpwBitcosJob()
    j.m = d
    j.d_x, j.x_len, j.x_scale, j.d_out_i32 = 16, 64, 1.0, 16
    arr = (_lib.BpwBitcosJob * 1)(j)
    import ctypes
    h = ctypes.c_void_p()
    assert _lib.lib().bpw_bitcos_plan_create(arr, 1, 256, 1 << 20, None, ctypes.byref(h)) == _lib.E_NOT_VALIDATED
