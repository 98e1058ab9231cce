"""The Python binding's own checks, on the CPU: outputs of the wrong element type or too few elements
are refused before anything reaches the C ABI (which carries no output lengths), and grouped jobs and
plans keep every buffer their records name alive. A stand-in object plays the device tensor (type,
element count, address), and a stub library answers the plan calls, so no GPU is needed."""
import gc
import weakref

import numpy as np
import pytest
import torch

import bit_plane_weight_amd as bpw
from bit_plane_weight_amd import _lib


class FakeDev:
    """A contiguous device tensor as the binding sees one: dtype, numel, element size, address."""
    _next = 0x10000000

    def __init__(self, dtype, n):
        self.dtype, self._n, self.is_cuda = dtype, n, True
        FakeDev._next += 1 << 20
        self._addr = FakeDev._next

    def numel(self):
        return self._n

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return self._addr


def devmat(rows, cols):
    d = _lib.BpwDevMat()
    d.rows, d.cols, d.bpr = rows, cols, (cols + 63) // 64
    return bpw.DevMat(d, FakeDev(torch.uint8, rows * d.bpr * 16))


def test_gemv_job_checks_outputs():
    m = devmat(100, 2560)
    x = FakeDev(torch.int8, 2560)
    ok_i, ok_f = FakeDev(torch.int32, 100), FakeDev(torch.float32, 100)
    j = bpw.gemv_job(m, x, 0.5, ok_i, ok_f)
    assert (j.d_x, j.x_len, j.d_out_i32, j.d_out_f32) == (x.data_ptr(), 2560, ok_i.data_ptr(), ok_f.data_ptr())
    with pytest.raises(TypeError, match="out_i32"):
        bpw.gemv_job(m, x, 0.5, FakeDev(torch.float32, 100))
    with pytest.raises(ValueError, match="out_i32"):
        bpw.gemv_job(m, x, 0.5, FakeDev(torch.int32, 99))
    with pytest.raises(TypeError, match="out_f32"):
        bpw.gemv_job(m, x, 0.5, ok_i, FakeDev(torch.float64, 100))
    with pytest.raises(ValueError, match="out_f32"):
        bpw.gemv_job(m, x, 0.5, ok_i, FakeDev(torch.float32, 50))
    with pytest.raises(TypeError, match="x_scale_dev"):
        bpw.gemv_job(m, x, 0.5, ok_i, x_scale_dev=FakeDev(torch.float64, 1))
    with pytest.raises(TypeError, match="x"):
        bpw.gemv_job(m, FakeDev(torch.int16, 2560), 0.5, ok_i)
    with pytest.raises(ValueError, match="out_i32"):
        bpw.gemv_job(m, x, 0.5, None)
    # a real host tensor is refused as a device buffer (after passing the type and size checks)
    with pytest.raises(TypeError, match="GPU"):
        bpw.gemv_job(m, x, 0.5, torch.empty(100, dtype=torch.int32))


def test_intmlp_small_batch_quant_bitcos_head_checks():
    g, u = devmat(64, 2560), devmat(64, 2560)
    x = FakeDev(torch.int8, 2560)
    t, k = FakeDev(torch.int64, 64), FakeDev(torch.float64, 1)
    bpw.intmlp_job(g, u, x, 1.0, t, k, FakeDev(torch.int32, 64), FakeDev(torch.int32, 64))
    with pytest.raises(TypeError, match="t_out"):
        bpw.intmlp_job(g, u, x, 1.0, FakeDev(torch.int32, 64), k)
    with pytest.raises(ValueError, match="t_out"):
        bpw.intmlp_job(g, u, x, 1.0, FakeDev(torch.int64, 63), k)
    with pytest.raises(TypeError, match="k_out"):
        bpw.intmlp_job(g, u, x, 1.0, t, FakeDev(torch.float32, 1))
    with pytest.raises(ValueError, match="up_i32"):
        bpw.intmlp_job(g, u, x, 1.0, t, k, up_i32=FakeDev(torch.int32, 10))

    m = devmat(30, 200)
    X = FakeDev(torch.int8, 4 * 256)
    X.shape = (4, 256)
    bpw.sb_job(m, X, np.ones(4, np.float32), FakeDev(torch.int32, 120), FakeDev(torch.float32, 120))
    with pytest.raises(ValueError, match="out_i32"):
        bpw.sb_job(m, X, np.ones(4, np.float32), FakeDev(torch.int32, 119))
    with pytest.raises(ValueError, match="out_f32"):
        bpw.sb_job(m, X, np.ones(4, np.float32), FakeDev(torch.int32, 120), FakeDev(torch.float32, 30))

    h, gg = FakeDev(torch.float32, 300), FakeDev(torch.float32, 300)
    bpw.quant_job(h, gg, FakeDev(torch.int8, 320), FakeDev(torch.float32, 1), 1e-5)
    with pytest.raises(TypeError, match="h"):
        bpw.quant_job(FakeDev(torch.float64, 300), gg, FakeDev(torch.int8, 320), FakeDev(torch.float32, 1), 1e-5)
    with pytest.raises(TypeError, match="scale"):
        bpw.quant_job(h, gg, FakeDev(torch.int8, 320), FakeDev(torch.float16, 1), 1e-5)
    with pytest.raises(TypeError, match="q"):
        bpw.quant_job(h, gg, FakeDev(torch.int32, 320), FakeDev(torch.float32, 1), 1e-5)

    d = _lib.BpwDevBitcos()
    d.rows, d.cols, d.bpr = 16, 200, 4
    bm = bpw.DevBitcos(d, FakeDev(torch.uint8, 4096))
    bpw.bitcos_job(bm, FakeDev(torch.int8, 256), 1.0, FakeDev(torch.int32, 16))
    with pytest.raises(ValueError, match="out_i32"):
        bpw.bitcos_job(bm, FakeDev(torch.int8, 256), 1.0, FakeDev(torch.int32, 15))

    w = FakeDev(torch.int16, 1000 * 256)
    w.shape = (1000, 256)
    with pytest.raises(ValueError, match="y"):
        bpw.bpw_dense_head_gemv(w, FakeDev(torch.int16, 256), FakeDev(torch.float32, 999))
    with pytest.raises(TypeError, match="y"):
        bpw.bpw_dense_head_gemv(w, FakeDev(torch.int16, 256), FakeDev(torch.float64, 1000))
    with pytest.raises(ValueError, match="x_bf16"):
        bpw.bpw_dense_head_gemv(w, FakeDev(torch.int16, 255), FakeDev(torch.float32, 1000))
    w8 = FakeDev(torch.int8, 1000 * 256)
    w8.shape = (1000, 256)
    with pytest.raises(TypeError, match="w_bf16"):
        bpw.bpw_dense_head_gemv(w8, FakeDev(torch.int16, 256), FakeDev(torch.float32, 1000))


class StubLib:
    """Answers the plan calls with success and records nothing: stands in for libbpw on a machine
    with no GPU, so the binding's own object lifetimes can be checked."""

    def __getattr__(self, name):
        if name.endswith("_workspace_bytes"):
            return lambda *a: 256
        return lambda *a: _lib.OK


def test_jobs_and_plans_keep_their_buffers_alive(monkeypatch):
    monkeypatch.setattr(_lib, "lib", lambda: StubLib())

    def build():
        m = devmat(100, 2560)
        x, oi, of, sd = (FakeDev(torch.int8, 2560), FakeDev(torch.int32, 100), FakeDev(torch.float32, 100),
                         FakeDev(torch.float32, 1))
        j = bpw.gemv_job(m, x, 0.0, oi, of, x_scale_dev=sd)
        t, k = FakeDev(torch.int64, 100), FakeDev(torch.float64, 1)
        p = bpw.intmlp_job(m, m, x, 1.0, t, k)
        refs = [weakref.ref(o) for o in (m, m.buf, x, oi, of, sd, t, k)]
        plan = bpw.GemvPlan([j], FakeDev(torch.uint8, 256), mlp=[p], stream=0)
        return plan, refs

    plan, refs = build()  # the caller holds only the plan
    gc.collect()
    assert all(r() is not None for r in refs), "a plan let go of a buffer its jobs name"
    del plan
    gc.collect()
    assert all(r() is None for r in refs)

    def build_bitcos():
        d = _lib.BpwDevBitcos()
        d.rows, d.cols, d.bpr = 16, 200, 4
        bm = bpw.DevBitcos(d, FakeDev(torch.uint8, 4096))
        x, oi = FakeDev(torch.int8, 256), FakeDev(torch.int32, 16)
        refs = [weakref.ref(o) for o in (bm, bm.buf, x, oi)]
        return bpw.BitcosPlan([bpw.bitcos_job(bm, x, 1.0, oi)], FakeDev(torch.uint8, 256), stream=0), refs

    plan, refs = build_bitcos()
    gc.collect()
    assert all(r() is not None for r in refs)

    def build_quant():
        h, g, q, s = (FakeDev(torch.float32, 64), FakeDev(torch.float32, 64), FakeDev(torch.int8, 64),
                      FakeDev(torch.float32, 1))
        refs = [weakref.ref(o) for o in (h, g, q, s)]
        return bpw.QuantPlan([bpw.quant_job(h, g, q, s, 1e-5)], FakeDev(torch.uint8, 256), stream=0), refs

    plan, refs = build_quant()
    gc.collect()
    assert all(r() is not None for r in refs)

    def build_sb():
        m = devmat(30, 200)
        X = FakeDev(torch.int8, 2 * 256)
        X.shape = (2, 256)
        oi = FakeDev(torch.int32, 60)
        refs = [weakref.ref(o) for o in (m, m.buf, X, oi)]
        return (bpw.SmallBatchPlan([bpw.sb_job(m, X, np.ones(2, np.float32), oi)], 2, FakeDev(torch.uint8, 256),
                                   stream=0), refs)

    plan, refs = build_sb()
    gc.collect()
    assert all(r() is not None for r in refs)


def test_job_fields_read_and_write_through():
    m = devmat(8, 64)
    j = bpw.gemv_job(m, FakeDev(torch.int8, 64), 2.0, FakeDev(torch.int32, 8))
    j.x_len = 7
    assert j.c.x_len == 7 and j.x_scale == 2.0 and j.m.rows == 8
