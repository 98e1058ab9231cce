"""GPU parity: libbpw's HIP kernels, called through the C ABI, against the CPU oracle.

Integers must be bit-identical. The ternary fp32 output must lie within rel 1e-6 of the
oracle's float64 value (and, since both sides apply the scales in turn with the same two
binary32 roundings, equal the oracle's fp32 bits). The bf16 head must satisfy
|err| <= 1e-3 * sum|w*x| + 1e-5 per element. Inputs come from the seeded generator only;
the oracle packs its own planes from the same trits.
"""
import ctypes
import os
import sys

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
import bit_plane_weight_amd as bpw  # noqa: E402
from bit_plane_weight_amd import _lib  # noqa: E402

pytestmark = pytest.mark.gpu
NT = min(16, len(os.sched_getaffinity(0)))


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU (they fail rather than skip)"
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    bpw.bpw_device_check()
    return d


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Uploaded:
    """One ternary case resident on the GPU: packed by the library, loaded, uploaded."""

    def __init__(self, case, dev, tail_junk=False):
        self.case = case
        planes = bpw.bpw_pack_i8(case.w)
        hm = bpw.bpw_load(planes, case.rows, case.cols, case.w_scale)
        self.buf = torch.empty(max(hm.nbytes, 1), dtype=torch.uint8, device=dev)
        self.m = bpw.bpw_upload(hm, self.buf)
        hm.free()
        bpr = (case.cols + 63) // 64
        xh = np.zeros(max(bpr * 64, 16), np.int8)
        if tail_junk:  # codes past cols are never used (P2 keeps those weights zero)
            xh[:] = synth.u64(case.cols + 5, xh.size).astype(np.uint8).view(np.int8)
        xh[: case.cols] = case.x
        self.x = torch.from_numpy(xh).to(dev)
        self.oi = torch.full((max(case.rows, 1),), 0x7EADBEEF, dtype=torch.int32, device=dev)
        self.of = torch.full((max(case.rows, 1),), float("nan"), dtype=torch.float32, device=dev)

    def job(self):
        return bpw.gemv_job(self.m, self.x, self.case.x_scale, self.oi, self.of)


def oracle_ref(case):
    return oracle.gemv(oracle.pack(case.w), case.rows, case.cols, case.x, case.x_scale, case.w_scale, nthreads=NT)


def check_case(u, ref, what):
    acc, y32, y64 = ref
    rows = u.case.rows
    gi = u.oi.cpu().numpy()[:rows]
    gf = u.of.cpu().numpy()[:rows]
    bad = np.nonzero(gi != acc)[0]
    assert bad.size == 0, f"{what}: int32 differs at rows {bad[:8].tolist()} (got {gi[bad[:4]]}, want {acc[bad[:4]]})"
    err = np.abs(gf.astype(np.float64) - y64)
    assert np.all(err <= 1e-6 * np.abs(y64)), f"{what}: fp32 outside rel 1e-6 (max rel {np.max(err / np.maximum(np.abs(y64), 1e-300))})"
    assert np.array_equal(gf.view(np.uint32), y32.view(np.uint32)), f"{what}: fp32 bits differ from scales-in-turn"


def run_grouped(cases, dev, kernel=bpw.KERNEL_AUTO, tail_junk=False):
    ups = [Uploaded(c, dev, tail_junk) for c in cases]
    jobs = [u.job() for u in ups]
    ws = torch.empty(max(bpw.bpw_gemv_workspace_bytes(jobs), 256), dtype=torch.uint8, device=dev)
    bpw.bpw_gemv(jobs, ws, kernel)
    torch.cuda.synchronize()
    return ups


KERNELS = [bpw.KERNEL_BITSERIAL, bpw.KERNEL_BYTELANE]


# ----------------------------------------------------------------------------- configs


@pytest.mark.parametrize("kernel", KERNELS)
def test_single_kproj_640x2560(dev, kernel):
    log(f"case: single k_proj 640x2560 kernel={kernel}")
    case = synth.ternary_case(101, 0, 1, 640, 2560)
    (u,) = run_grouped([case], dev, kernel)
    check_case(u, oracle_ref(case), "k_proj")


@pytest.mark.parametrize("kernel", KERNELS)
def test_one_layer_seven_projections_grouped(dev, kernel):
    log(f"case: one layer, 7 projections grouped, kernel={kernel}")
    cases = synth.layer_cases(202, 3)
    ups = run_grouped(cases, dev, kernel)
    for u in ups:
        check_case(u, oracle_ref(u.case), u.case.name)


def test_decode_step_210_matrices_full(dev):
    """All 210 matrices of a decode step in one grouped plan launch, every output checked."""
    log("case: decode step, 210 matrices, plan + run (the benchmark's launch)")
    ups = []
    for layer in range(synth.N_LAYERS):
        for c in synth.layer_cases(303, layer):
            ups.append(Uploaded(c, dev))
    jobs = [u.job() for u in ups]
    ws = torch.empty(bpw.bpw_gemv_workspace_bytes(jobs), dtype=torch.uint8, device=dev)
    plan = bpw.GemvPlan(jobs, ws)
    plan.run()
    plan.run()  # a second run over the same tables must give the same results
    torch.cuda.synchronize()
    log("  GPU done; oracle over 210 matrices")
    for u in ups:
        check_case(u, oracle_ref(u.case), u.case.name)
    plan.free()


@pytest.mark.parametrize("z", synth.P_ZERO_SWEEP)
def test_zero_density_sweep_layer(dev, z):
    log(f"case: layer at P(0)={z}")
    cases = synth.layer_cases(404, 0, p_zero=z)
    for u in run_grouped(cases, dev):
        check_case(u, oracle_ref(u.case), f"{u.case.name} z={z}")


SB_KERNELS = (bpw.KERNEL_BITSERIAL, bpw.KERNEL_MFMA)


@pytest.mark.parametrize("kernel", SB_KERNELS)
@pytest.mark.parametrize("batch", (1, 2, 3, 4, 8, 16))
@pytest.mark.parametrize("shape", ((6912, 2560), (2560, 6912)))
def test_small_batch(dev, shape, batch, kernel):
    rows, cols = shape
    log(f"case: small batch {rows}x{cols} B={batch} kernel={kernel}")
    case = synth.ternary_case(505, 0, 4 if rows == 6912 else 6, rows, cols)
    u = Uploaded(case, dev)
    bpr = (cols + 63) // 64
    X, sc = synth.small_batch_x(506 + batch, batch, cols)
    ldx = bpr * 64 + (64 if batch % 2 else 0)
    Xh = np.full((batch, ldx), 77, np.int8)
    Xh[:, :cols] = X
    Xd = torch.from_numpy(Xh).to(dev)
    oi = torch.empty((batch, rows), dtype=torch.int32, device=dev)
    of = torch.empty((batch, rows), dtype=torch.float32, device=dev)
    bpw.bpw_gemm_small_batch(u.m, Xd, sc, oi, of, kernel)
    torch.cuda.synchronize()
    acc, y32, y64 = oracle.gemm_small_batch(oracle.pack(case.w), rows, cols, Xh, sc, case.w_scale, nthreads=NT)
    assert np.array_equal(oi.cpu().numpy(), acc)
    gf = of.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(gf - y64) <= 1e-6 * np.abs(y64))
    assert np.array_equal(of.cpu().numpy().view(np.uint32), y32.view(np.uint32))
    if batch == 1:  # batch 1 equals the GEMV bit for bit
        case1 = synth.TernaryCase("b1", case.w, X[0], float(sc[0]), case.w_scale)
        (g,) = run_grouped([case1], dev)
        assert np.array_equal(g.oi.cpu().numpy(), oi.cpu().numpy()[0])
        assert np.array_equal(g.of.cpu().numpy().view(np.uint32), of.cpu().numpy()[0].view(np.uint32))


@pytest.mark.parametrize("kernel", SB_KERNELS + (bpw.KERNEL_AUTO,))
@pytest.mark.parametrize("rows,cols,batch", ((1, 1, 1), (7, 65, 3), (65, 129, 17), (129, 2500, 64), (33, 8193, 5),
                                             (1025, 448, 16), (5, 0, 4), (2560, 6912, 40), (17, 320, 33)))
def test_small_batch_ragged_and_wide(dev, rows, cols, batch, kernel):
    """Ragged column tails, rows wider than one LDS pass, no columns, and batches split into several
    token groups; ldx larger than the row and junk past cols."""
    log(f"case: small batch {rows}x{cols} B={batch} kernel={kernel}")
    case = synth.ternary_case(515, rows % 7, cols % 7, rows, cols)
    u = Uploaded(case, dev)
    bpr = (cols + 63) // 64
    X, sc = synth.small_batch_x(516 + batch, batch, max(cols, 1))
    ldx = bpr * 64 + 48
    Xh = synth.u64(517, batch * ldx).astype(np.uint8).view(np.int8).reshape(batch, ldx).copy()
    Xh[:, :cols] = X[:, :cols]
    Xd = torch.from_numpy(Xh).to(dev)
    oi = torch.full((batch, rows), -7, dtype=torch.int32, device=dev)
    of = torch.full((batch, rows), -7.0, dtype=torch.float32, device=dev)
    bpw.bpw_gemm_small_batch(u.m, Xd, sc, oi, of, kernel)
    torch.cuda.synchronize()
    acc, y32, y64 = oracle.gemm_small_batch(oracle.pack(case.w), rows, cols, Xh, sc, case.w_scale, nthreads=NT)
    assert np.array_equal(oi.cpu().numpy(), acc)
    assert np.array_equal(of.cpu().numpy().view(np.uint32), y32.view(np.uint32))


def test_dense_head_full_128256x2560(dev):
    log("case: dense bf16 head 128256x2560")
    w, x = synth.head_case(606)
    wd = torch.from_numpy(w.view(np.int16)).to(dev)
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    y = torch.empty(w.shape[0], dtype=torch.float32, device=dev)
    bpw.bpw_dense_head_gemv(wd, xd, y)
    torch.cuda.synchronize()
    ry, rs = oracle.dense_head(w, x, nthreads=NT)
    err = np.abs(y.cpu().numpy().astype(np.float64) - ry)
    assert np.all(err <= 1e-3 * rs + 1e-5), f"max err/bound {np.max(err / (1e-3 * rs + 1e-5))}"


@pytest.mark.parametrize("rows,cols", ((1, 8), (3, 64), (17, 136), (1000, 2560), (9, 2560), (129, 32768), (64, 1024),
                                       (5, 40008)))
def test_dense_head_shapes(dev, rows, cols):
    log(f"case: dense head {rows}x{cols}")
    w, x = synth.head_case(rows * 7 + cols, rows=rows, cols=cols)
    wd = torch.from_numpy(w.view(np.int16)).to(dev)
    xd = torch.from_numpy(x.view(np.int16)).to(dev)
    y = torch.empty(rows, dtype=torch.float32, device=dev)
    bpw.bpw_dense_head_gemv(wd, xd, y)
    torch.cuda.synchronize()
    ry, rs = oracle.dense_head(w, x)
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - ry) <= 1e-3 * rs + 1e-5)


# ----------------------------------------------------------------------------- edge cases

RAGGED_ROWS = (1, 7, 63, 64, 65, 129, 1025)
RAGGED_COLS = (1, 63, 64, 65, 127, 129, 448, 2500, 7169, 8193)


@pytest.mark.parametrize("kernel", KERNELS)
def test_ragged_shapes_grouped(dev, kernel):
    log(f"case: ragged rows x cols grid, kernel={kernel}")
    cases = []
    i = 0
    for r in RAGGED_ROWS:
        for c in RAGGED_COLS:
            cases.append(synth.ternary_case(707, i // 7, i % 7, r, c, name=f"{r}x{c}"))
            i += 1
    ups = run_grouped(cases, dev, kernel, tail_junk=True)
    for u in ups:
        check_case(u, oracle_ref(u.case), u.case.name)


@pytest.mark.parametrize("kernel", KERNELS)
def test_wide_rows_multi_pass(dev, kernel):
    """Rows wider than one pass of register-resident blocks (bpr > 7 * 64) take several passes."""
    log(f"case: wide rows (several passes), kernel={kernel}")
    cases = [synth.ternary_case(808, 0, 0, 33, 28673, name="33x28673"),
             synth.ternary_case(808, 0, 1, 5, 65536, name="5x65536"),
             synth.ternary_case(808, 0, 2, 200, 40000, name="200x40000")]
    for u in run_grouped(cases, dev, kernel, tail_junk=True):
        check_case(u, oracle_ref(u.case), u.case.name)


def test_empty_rows_and_cols_and_zero_jobs(dev):
    log("case: empty matrices")
    cases = [synth.ternary_case(909, 0, 0, 5, 0, name="5x0"), synth.ternary_case(909, 0, 1, 0, 100, name="0x100"),
             synth.ternary_case(909, 0, 2, 40, 64, name="40x64")]
    ups = run_grouped(cases, dev)
    assert np.all(ups[0].oi.cpu().numpy()[:5] == 0)
    assert np.all(ups[0].of.cpu().numpy()[:5] == 0.0)
    check_case(ups[2], oracle_ref(cases[2]), "40x64")
    bpw.bpw_gemv([], None)


@pytest.mark.parametrize("kernel", KERNELS)
def test_extremes_minus128(dev, kernel):
    """6912 columns of -1 (and of +1) against x = -128: +-884736, the widening case."""
    log(f"case: -128 extremes, kernel={kernel}")
    cols = 6912
    w = np.stack([-np.ones(cols, np.int8), np.ones(cols, np.int8), np.zeros(cols, np.int8),
                  synth.trits(1, 1, cols)[0]])
    cases = [synth.TernaryCase("ext", w, np.full(cols, -128, np.int8), 1.0, 1.0),
             synth.TernaryCase("ext127", w, np.full(cols, 127, np.int8), 0.5, 2.0),
             synth.TernaryCase("mix", w, synth.u64(9, cols).astype(np.uint8).view(np.int8), 0.01, 1.5)]
    ups = run_grouped(cases, dev, kernel)
    assert ups[0].oi.cpu().numpy()[:3].tolist() == [884736, -884736, 0]
    for u in ups:
        check_case(u, oracle_ref(u.case), u.case.name)


def test_kernels_agree_and_runs_are_deterministic(dev):
    log("case: bit-serial == byte-lane, repeated runs identical")
    cases = synth.layer_cases(1111, 0)
    a = [u.oi.cpu().numpy().copy() for u in run_grouped(cases, dev, bpw.KERNEL_BITSERIAL)]
    b = [u.oi.cpu().numpy().copy() for u in run_grouped(cases, dev, bpw.KERNEL_BYTELANE)]
    c = [u.oi.cpu().numpy().copy() for u in run_grouped(cases, dev, bpw.KERNEL_AUTO)]
    for x, y, z in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, z)


def test_plan_reads_current_activation_contents(dev):
    log("case: plan reuse with new activations")
    cases = synth.layer_cases(1212, 0)[:3]
    ups = [Uploaded(c, dev) for c in cases]
    jobs = [u.job() for u in ups]
    ws = torch.empty(bpw.bpw_gemv_workspace_bytes(jobs), dtype=torch.uint8, device=dev)
    plan = bpw.GemvPlan(jobs, ws)
    for rep in range(3):
        for u in ups:
            x, xs = synth.activation(5000 + rep, u.case.cols)
            u.case.x, u.case.x_scale = x, xs
            u.x[: u.case.cols] = torch.from_numpy(x).to(dev)
        # x_scale lives in the plan's table: keep the scale of the plan, check the integers
        plan.run()
        torch.cuda.synchronize()
        for u in ups:
            acc = oracle.gemv(oracle.pack(u.case.w), u.case.rows, u.case.cols, u.case.x, nthreads=NT)[0]
            assert np.array_equal(u.oi.cpu().numpy(), acc)
    plan.free()


# ----------------------------------------------------------------------------- errors from the host


def test_argument_errors_on_gpu(dev):
    log("case: argument errors")
    case = synth.ternary_case(1313, 0, 0, 64, 256)
    u = Uploaded(case, dev)
    ws = torch.empty(bpw.bpw_gemv_workspace_bytes([u.job()]), dtype=torch.uint8, device=dev)
    short = torch.zeros(200, dtype=torch.int8, device=dev)
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_gemv([bpw.gemv_job(u.m, short, 1.0, u.oi)], ws)
    assert ei.value.status == _lib.E_INVAL
    big = torch.zeros(1024, dtype=torch.int8, device=dev)
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_gemv([bpw.gemv_job(u.m, big[1:257], 1.0, u.oi)], ws)
    assert ei.value.status == _lib.E_INVAL  # misaligned activation
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_gemv([u.job()], ws[:16])
    assert ei.value.status == _lib.E_SIZE
    forged = bpw.DevMat(_lib.BpwDevMat.from_buffer_copy(u.m.desc), u.buf)
    forged.desc.rows = 63  # (fewer rows than the output holds, so only the seal can refuse it)
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_gemv([bpw.gemv_job(forged, u.x, 1.0, u.oi)], ws)
    assert ei.value.status == _lib.E_NOT_VALIDATED
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_gemv([u.job()], ws, kernel=9)
    assert ei.value.status == _lib.E_UNSUPPORTED
    os.environ["BPW_FORCE_ARCH_MISMATCH"] = "1"
    try:
        with pytest.raises(bpw.BpwError) as ei:
            bpw.bpw_gemv([u.job()], ws)
        assert ei.value.status == _lib.E_ARCH
    finally:
        del os.environ["BPW_FORCE_ARCH_MISMATCH"]
    bpw.bpw_gemv([u.job()], ws)  # and the same call succeeds again
    torch.cuda.synchronize()
    check_case(u, oracle_ref(case), "after errors")


def test_probe_and_flush_run(dev):
    log("case: probe (every shape, a length that ends inside a chunk) and flush")
    buf = torch.zeros((64 << 20) + 48, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for shape in range(bpw.PROBE_SHAPES):
        bpw.bpw_stream_read_probe(buf, sink, shape=shape)
    bpw.bpw_stream_read_probe(buf, sink)
    bpw.bpw_cache_flush(buf)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    assert int(buf.sum().item()) == 0


# ----------------------------------------------------------------------------- Folded quantiser


def _hg(seed, n, spread):
    h = (synth.normal_f32(seed, n) * np.float32(spread)).astype(np.float32)
    g = (np.float32(0.5) + synth.uniform(seed + 1, n).astype(np.float32)).astype(np.float32)
    return h, g


@pytest.mark.parametrize("n,spread", ((1, 1.0), (7, 1e-3), (64, 10.0), (2560, 1.0), (2560, 1e4), (6912, 0.5),
                                      (8193, 3.0), (100000, 1.0)))
def test_quantize_folded_parity(dev, n, spread):
    log(f"case: quantiser n={n} spread={spread}")
    h, g = _hg(3131 + n, n, spread)
    q_len = ((n + 63) // 64) * 64 + 64
    hd, gd = torch.from_numpy(h).to(dev), torch.from_numpy(g).to(dev)
    qd = torch.full((q_len,), 55, dtype=torch.int8, device=dev)
    sd = torch.full((1,), -1.0, dtype=torch.float32, device=dev)
    ws = torch.empty(max(bpw.bpw_quantize_workspace_bytes(1), 1), dtype=torch.uint8, device=dev)
    bpw.bpw_quantize([bpw.quant_job(hd, gd, qd, sd, 1e-5)], ws)
    torch.cuda.synchronize()
    q, s = oracle.quantize(h, g, 1e-5, folded=True)
    got = qd.cpu().numpy()
    assert np.array_equal(got[:n], q)
    assert not got[n:].any()
    gs = float(sd.item())
    assert abs(gs - s) <= abs(s) * 2.0 ** -23  # the float64 sum of squares may differ in its last bits


@pytest.mark.parametrize("n", (64, 2560, 9000))
def test_quantize_non_finite_inputs(dev, n):
    """Non-finite residuals and gains: both sides give NaN codes the value 0 and let NaN never raise the
    absmax, so the codes agree bit for bit; the scale is NaN or infinite on both sides alike."""
    log(f"case: quantiser non-finite inputs n={n}")
    for what in ("nan_h", "nan_g", "inf_h"):
        h, g = _hg(4242 + n, n, 2.0)
        if what == "nan_h":
            h[[3, n // 2]] = np.nan
        elif what == "nan_g":
            g[[5, n - 1]] = np.nan
        else:
            h[n // 3] = np.inf
        hd, gd = torch.from_numpy(h).to(dev), torch.from_numpy(g).to(dev)
        qd = torch.full((n,), 55, dtype=torch.int8, device=dev)
        sd = torch.full((1,), -1.0, dtype=torch.float32, device=dev)
        ws = torch.empty(bpw.bpw_quantize_workspace_bytes(1), dtype=torch.uint8, device=dev)
        bpw.bpw_quantize([bpw.quant_job(hd, gd, qd, sd, 1e-5)], ws)
        torch.cuda.synchronize()
        q, s = oracle.quantize(h, g, 1e-5, folded=True)
        assert np.array_equal(qd.cpu().numpy(), q), what
        gs = float(sd.item())
        if np.isfinite(s):
            assert abs(gs - s) <= abs(s) * 2.0 ** -23, what
        else:
            assert (np.isnan(s) and np.isnan(gs)) or gs == s, (what, gs, s)


def test_quantize_zero_and_errors(dev):
    log("case: quantiser zeros and argument errors")
    n = 300
    hd = torch.zeros(n, dtype=torch.float32, device=dev)
    gd = torch.ones(n, dtype=torch.float32, device=dev)
    qd = torch.full((n,), 9, dtype=torch.int8, device=dev)
    sd = torch.full((1,), 1.0, dtype=torch.float32, device=dev)
    ws = torch.empty(bpw.bpw_quantize_workspace_bytes(1), dtype=torch.uint8, device=dev)
    bpw.bpw_quantize([bpw.quant_job(hd, gd, qd, sd, 1e-5)], ws)
    torch.cuda.synchronize()
    assert not qd.cpu().numpy().any() and float(sd.item()) == 0.0
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_quantize([bpw.quant_job(hd, gd, qd[:10], sd, 1e-5)], ws)
    assert ei.value.status == _lib.E_INVAL
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_quantize([bpw.quant_job(hd, gd, qd, sd, float("nan"))], ws)
    assert ei.value.status == _lib.E_INVAL
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_quantize([bpw.quant_job(hd, gd, qd, sd, 1e-5)], ws[:8])
    assert ei.value.status == _lib.E_SIZE


@pytest.mark.parametrize("kernel", KERNELS)
def test_quantise_then_gemv_layer(dev, kernel):
    """A layer's seven projections fed by the Folded quantiser: codes and scales stay on the device
    (the GEMV reads each scale when it runs); two runs of the plans with new residuals."""
    log(f"case: quantiser -> grouped GEMV, kernel={kernel}")
    cases = synth.layer_cases(4242, 0)
    ups, qjobs, keep = [], [], []
    for i, c in enumerate(cases):
        u = Uploaded(c, dev)
        sd = torch.zeros(1, dtype=torch.float32, device=dev)
        hd = torch.empty(c.cols, dtype=torch.float32, device=dev)
        gd = torch.empty(c.cols, dtype=torch.float32, device=dev)
        u.sd, u.hd, u.gd = sd, hd, gd
        qjobs.append(bpw.quant_job(hd, gd, u.x, sd, 1e-5))
        ups.append(u)
    qws = torch.empty(bpw.bpw_quantize_workspace_bytes(len(qjobs)), dtype=torch.uint8, device=dev)
    qplan = bpw.QuantPlan(qjobs, qws)
    jobs = [bpw.gemv_job(u.m, u.x, 0.0, u.oi, u.of, x_scale_dev=u.sd) for u in ups]
    ws = torch.empty(bpw.bpw_gemv_workspace_bytes(jobs), dtype=torch.uint8, device=dev)
    plan = bpw.GemvPlan(jobs, ws, kernel)
    for rep in range(2):
        hs = []
        for i, u in enumerate(ups):
            h, g = _hg(5000 + 10 * rep + i, u.case.cols, 2.0 + rep)
            u.hd.copy_(torch.from_numpy(h))
            u.gd.copy_(torch.from_numpy(g))
            hs.append((h, g))
        qplan.run()
        plan.run()
        torch.cuda.synchronize()
        for u, (h, g) in zip(ups, hs):
            q, s = oracle.quantize(h, g, 1e-5, folded=True)
            acc, y32, y64 = oracle.gemv(oracle.pack(u.case.w), u.case.rows, u.case.cols, q, s, u.case.w_scale,
                                        nthreads=NT)
            assert np.array_equal(u.oi.cpu().numpy(), acc)
            gf = u.of.cpu().numpy().astype(np.float64)
            assert np.all(np.abs(gf - y64) <= 1e-6 * np.abs(y64))
    plan.free()
    qplan.free()


# ----------------------------------------------------------------------------- IntMlp gate/up pairs


class UploadedPair:
    """A gate/up pair sharing one activation, resident on the GPU, with sentinel-filled outputs."""

    def __init__(self, wg, wu, x, x_scale, sg, su, dev, want_i32=True):
        self.wg, self.wu, self.x_np, self.xs, self.sg, self.su = wg, wu, x, x_scale, sg, su
        rows, cols = wg.shape
        self.rows, self.cols = rows, cols
        self.bufs = []
        self.g = self._up(wg, sg, dev)
        self.u = self._up(wu, su, dev)
        bpr = (cols + 63) // 64
        xh = np.zeros(max(bpr * 64, 16), np.int8)
        xh[:cols] = x
        self.x = torch.from_numpy(xh).to(dev)
        n = max(rows, 1)
        self.t = torch.full((n,), 0x5A5A5A5A5A5A5A5A, dtype=torch.int64, device=dev)
        self.k = torch.full((1,), float("nan"), dtype=torch.float64, device=dev)
        self.gi = torch.full((n,), 0x7EADBEEF, dtype=torch.int32, device=dev) if want_i32 else None
        self.ui = torch.full((n,), 0x7EADBEEF, dtype=torch.int32, device=dev) if want_i32 else None

    def _up(self, w, s, dev):
        hm = bpw.bpw_load(bpw.bpw_pack_i8(w), w.shape[0], w.shape[1], s)
        buf = torch.empty(max(hm.nbytes, 1), dtype=torch.uint8, device=dev)
        m = bpw.bpw_upload(hm, buf)
        hm.free()
        self.bufs.append(buf)
        return m

    def job(self, x_scale_dev=None):
        return bpw.intmlp_job(self.g, self.u, self.x, self.xs, self.t, self.k, self.gi, self.ui,
                              x_scale_dev=x_scale_dev)

    def check(self, what, x_scale=None):
        xs = self.xs if x_scale is None else x_scale
        t, k, ag, au = oracle.intmlp(oracle.pack(self.wg), oracle.pack(self.wu), self.rows, self.cols, self.x_np,
                                     xs, self.sg, self.su, nthreads=NT)
        gt = self.t.cpu().numpy()[: self.rows]
        bad = np.nonzero(gt != t)[0]
        assert bad.size == 0, f"{what}: t differs at rows {bad[:8].tolist()} (got {gt[bad[:4]]}, want {t[bad[:4]]})"
        gk = float(self.k.item())
        assert np.float64(gk).view(np.uint64) == np.float64(k).view(np.uint64), f"{what}: K {gk!r} != {k!r}"
        if self.gi is not None:
            assert np.array_equal(self.gi.cpu().numpy()[: self.rows], ag), f"{what}: gate sums"
            assert np.array_equal(self.ui.cpu().numpy()[: self.rows], au), f"{what}: up sums"


def _pair_inputs(seed, rows, cols):
    wg = synth.trits(seed, rows, cols)
    wu = synth.trits(seed + 1, rows, cols)
    x, xs = synth.activation(seed + 2, cols)
    return wg, wu, x, xs, synth.weight_scale(seed + 3), synth.weight_scale(seed + 4)


def _run_plan(jobs, pairs, dev, kernel=bpw.KERNEL_AUTO, reps=1):
    ws = torch.empty(max(bpw.bpw_gemv_intmlp_workspace_bytes(jobs, pairs), 256), dtype=torch.uint8, device=dev)
    plan = bpw.GemvPlan(jobs, ws, kernel, mlp=pairs)
    for _ in range(reps):
        plan.run()
    torch.cuda.synchronize()
    plan.free()


@pytest.mark.parametrize("kernel", (bpw.KERNEL_AUTO, bpw.KERNEL_BITSERIAL))
@pytest.mark.parametrize("want_i32", (True, False))
def test_intmlp_gate_up_6912x2560(dev, kernel, want_i32):
    log(f"case: IntMlp pair 6912x2560 kernel={kernel} i32={want_i32}")
    p = UploadedPair(*_pair_inputs(8801, 6912, 2560), dev, want_i32=want_i32)
    _run_plan([], [p.job()], dev, kernel, reps=2)
    p.check("gate/up 6912x2560")


@pytest.mark.parametrize("rows", (1, 7, 65, 129, 1025))
def test_intmlp_ragged_pairs_beside_plain_jobs(dev, rows):
    """Pairs of every column geometry (generic K = 1 and 2, one and several LDS passes, both model
    widths) in one launch with plain jobs; every output checked."""
    colss = (1, 63, 64, 65, 127, 129, 448, 2500, 2560, 6912, 8193, 16383)
    log(f"case: IntMlp ragged pairs rows={rows} cols={colss}")
    pairs = [UploadedPair(*_pair_inputs(9000 + 37 * rows + c, rows, c), dev) for c in colss]
    plain = [Uploaded(synth.ternary_case(9100 + rows, 0, i, rows, c), dev) for i, c in enumerate((65, 2560, 6912))]
    _run_plan([u.job() for u in plain], [p.job() for p in pairs], dev)
    for p in pairs:
        p.check(f"pair {rows}x{p.cols}")
    for u in plain:
        check_case(u, oracle_ref(u.case), f"plain {rows}x{u.case.cols} beside pairs")


@pytest.mark.parametrize("cols", (2560, 16383))
def test_intmlp_extremes(dev, cols):
    """x = -128, gate all -1, up all +1: t = -(128 cols)^3, the largest |t| of the width."""
    log(f"case: IntMlp extremes cols={cols}")
    rows = 70
    x = np.full(cols, -128, np.int8)
    p = UploadedPair(np.full((rows, cols), -1, np.int8), np.full((rows, cols), 1, np.int8), x, 0.25, 1.0, 1.0, dev)
    _run_plan([], [p.job()], dev)
    p.check(f"extremes {cols}")
    assert int(p.t[0].item()) == -((128 * cols) ** 3)


def test_intmlp_empty_pairs(dev):
    log("case: IntMlp pairs with no columns / no rows")
    p0 = UploadedPair(np.zeros((70, 0), np.int8), np.zeros((70, 0), np.int8), np.zeros(0, np.int8), 0.5, 1.5, 2.0, dev)
    pr = UploadedPair(np.zeros((0, 64), np.int8), np.zeros((0, 64), np.int8), np.zeros(64, np.int8), 0.5, 1.5, 2.0, dev)
    _run_plan([], [p0.job(), pr.job()], dev)
    p0.check("no columns")
    assert not p0.t.cpu().numpy().any()
    assert np.isnan(pr.k.item()) and int(pr.t[0].item()) == 0x5A5A5A5A5A5A5A5A  # no rows: nothing written


def test_intmlp_scale_from_quantiser(dev):
    """Folded quantiser -> IntMlp pair: the codes and the device-resident scale feed both projections."""
    log("case: quantiser -> IntMlp pair 6912x2560")
    wg, wu, _, _, sg, su = _pair_inputs(8901, 6912, 2560)
    h, g = _hg(8902, 2560, 3.0)
    q, s = oracle.quantize(h, g, 1e-5, folded=True)
    p = UploadedPair(wg, wu, q, 0.0, sg, su, dev)
    sd = torch.zeros(1, dtype=torch.float32, device=dev)
    hd, gd = torch.from_numpy(h).to(dev), torch.from_numpy(g).to(dev)
    qws = torch.empty(bpw.bpw_quantize_workspace_bytes(1), dtype=torch.uint8, device=dev)
    p.x.fill_(99)  # overwritten by the quantiser (codes, then zeros up to the buffer's end)
    bpw.bpw_quantize([bpw.quant_job(hd, gd, p.x, sd, 1e-5)], qws)
    _run_plan([], [p.job(x_scale_dev=sd)], dev)
    assert float(sd.item()) == s
    p.check("quantiser -> pair", x_scale=s)


def test_decode_step_with_intmlp_pairs(dev):
    """A decode step with the MLP's squared-ReLU stage fused: per layer q, k, v, o, down as plain
    jobs and gate/up as one pair sharing x, all 30 layers in one launch, run twice."""
    log("case: decode step, 150 plain jobs + 30 IntMlp pairs")
    plain, pairs = [], []
    for layer in range(30):
        cs = synth.layer_cases(777, layer)
        for i in (0, 1, 2, 3, 6):
            plain.append(Uploaded(cs[i], dev))
        gc, uc = cs[4], cs[5]
        pairs.append(UploadedPair(gc.w, uc.w, gc.x, gc.x_scale, gc.w_scale, uc.w_scale, dev, want_i32=(layer % 2 == 0)))
    _run_plan([u.job() for u in plain], [p.job() for p in pairs], dev, reps=2)
    for p in pairs:
        p.check("decode-step pair")
    for u in plain:
        check_case(u, oracle_ref(u.case), u.case.name)


def test_intmlp_argument_errors(dev):
    log("case: IntMlp argument errors")
    wg, wu, x, xs, sg, su = _pair_inputs(8701, 64, 128)
    p = UploadedPair(wg, wu, x, xs, sg, su, dev)
    q = UploadedPair(wg[:32], wu[:32], x, xs, sg, su, dev)
    ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    bad = bpw.intmlp_job(p.g, q.u, p.x, xs, p.t, p.k)  # shapes differ
    with pytest.raises(bpw.BpwError) as ei:
        bpw.GemvPlan([], ws, mlp=[bad])
    assert ei.value.status == _lib.E_INVAL
    with pytest.raises(bpw.BpwError) as ei:
        bpw.GemvPlan([], ws, bpw.KERNEL_BYTELANE, mlp=[p.job()])
    assert ei.value.status == _lib.E_UNSUPPORTED
    j = p.job()
    j.d_t += 4  # misaligned
    with pytest.raises(bpw.BpwError) as ei:
        bpw.GemvPlan([], ws, mlp=[j])
    assert ei.value.status == _lib.E_INVAL
    with pytest.raises(bpw.BpwError) as ei:
        bpw.GemvPlan([], ws[:64], mlp=[p.job()])
    assert ei.value.status == _lib.E_SIZE
    wide = UploadedPair(np.zeros((2, 16384), np.int8), np.zeros((2, 16384), np.int8), np.zeros(16384, np.int8),
                        1.0, 1.0, 1.0, dev)
    with pytest.raises(bpw.BpwError) as ei:
        bpw.GemvPlan([], ws, mlp=[wide.job()])
    assert ei.value.status == _lib.E_UNSUPPORTED
    _run_plan([], [p.job()], dev)  # and a good pair still runs
    p.check("after errors")


# ----------------------------------------------------------------------------- grouped small batch

GROUPED_SHAPES = ((6912, 2560), (2560, 6912), (640, 2560), (1, 1), (7, 65), (65, 129), (33, 8193), (129, 2500), (5, 0))


def _sb_inputs(dev, seed, rows, cols, batch):
    case = synth.ternary_case(seed, rows % 7, cols % 7, rows, cols)
    u = Uploaded(case, dev)
    bpr = (cols + 63) // 64
    X, sc = synth.small_batch_x(seed + 1, batch, max(cols, 1))
    ldx = bpr * 64 + 48
    Xh = synth.u64(seed + 2, batch * ldx).astype(np.uint8).view(np.int8).reshape(batch, ldx).copy()
    Xh[:, :cols] = X[:, :cols]
    Xd = torch.from_numpy(Xh).to(dev)
    oi = torch.full((batch, rows), -7, dtype=torch.int32, device=dev)
    of = torch.full((batch, rows), -7.0, dtype=torch.float32, device=dev)
    return case, u, Xh, Xd, sc, oi, of


@pytest.mark.parametrize("kernel", (bpw.KERNEL_AUTO, bpw.KERNEL_MFMA))
@pytest.mark.parametrize("batch", (1, 3, 16, 17, 64))
def test_small_batch_grouped(dev, batch, kernel):
    """Every shape (model widths, ragged tails, wide rows, no columns) as jobs of one grouped launch,
    run twice; each job equals the oracle and the single-call matrix-core kernel bit for bit. (AUTO at
    batch 1 runs the batch-1 GEMV.)"""
    log(f"case: grouped small batch B={batch} kernel={kernel}, {len(GROUPED_SHAPES)} jobs")
    sets = [_sb_inputs(dev, 900 + 11 * i + batch, r, c, batch) for i, (r, c) in enumerate(GROUPED_SHAPES)]
    jobs = [bpw.sb_job(u.m, Xd, sc, oi, of) for (case, u, Xh, Xd, sc, oi, of) in sets]
    ws = torch.empty(max(bpw.bpw_gemm_small_batch_workspace_bytes(jobs, batch), 256), dtype=torch.uint8, device=dev)
    plan = bpw.SmallBatchPlan(jobs, batch, ws, kernel)
    plan.run()
    plan.run()
    torch.cuda.synchronize()
    for (case, u, Xh, Xd, sc, oi, of) in sets:
        acc, y32, y64 = oracle.gemm_small_batch(oracle.pack(case.w), case.rows, case.cols, Xh, sc, case.w_scale,
                                                nthreads=NT)
        assert np.array_equal(oi.cpu().numpy(), acc), f"{case.rows}x{case.cols}"
        assert np.array_equal(of.cpu().numpy().view(np.uint32), y32.view(np.uint32)), f"{case.rows}x{case.cols}"
        oi2 = torch.empty_like(oi)
        of2 = torch.empty_like(of)
        bpw.bpw_gemm_small_batch(u.m, Xd, sc, oi2, of2, bpw.KERNEL_MFMA)
        torch.cuda.synchronize()
        assert torch.equal(oi2, oi) and torch.equal(of2.view(torch.int32), of.view(torch.int32))
    plan.free()


@pytest.mark.parametrize("batch", (4, 16))
def test_small_batch_grouped_unaligned_outputs(dev, batch):
    """Outputs 4 bytes past a 16-byte boundary, rows a multiple of 4: the grouped matrix-core kernel
    stores word by word there (16-byte stores only with 16-byte aligned outputs). Bit-exact against the
    oracle, and the guard words on both sides of each output stay untouched."""
    log(f"case: grouped small batch, unaligned outputs, B={batch}")
    sets = []
    for i, (r, c) in enumerate(((640, 2560), (256, 6912), (12, 130))):
        case, u, Xh, Xd, sc, _, _ = _sb_inputs(dev, 950 + 7 * i + batch, r, c, batch)
        bi = torch.full((batch * r + 2,), -7, dtype=torch.int32, device=dev)
        bf = torch.full((batch * r + 2,), -7.0, dtype=torch.float32, device=dev)
        oi, of = bi[1:1 + batch * r].view(batch, r), bf[1:1 + batch * r].view(batch, r)
        assert oi.data_ptr() % 16 == 4 and of.data_ptr() % 16 == 4
        sets.append((case, u, Xh, Xd, sc, oi, of, bi, bf))
    jobs = [bpw.sb_job(u.m, Xd, sc, oi, of) for (case, u, Xh, Xd, sc, oi, of, bi, bf) in sets]
    ws = torch.empty(bpw.bpw_gemm_small_batch_workspace_bytes(jobs, batch), dtype=torch.uint8, device=dev)
    plan = bpw.SmallBatchPlan(jobs, batch, ws, bpw.KERNEL_MFMA)
    plan.run()
    torch.cuda.synchronize()
    for (case, u, Xh, Xd, sc, oi, of, bi, bf) in sets:
        acc, y32, y64 = oracle.gemm_small_batch(oracle.pack(case.w), case.rows, case.cols, Xh, sc, case.w_scale,
                                                nthreads=NT)
        assert np.array_equal(oi.cpu().numpy(), acc), f"{case.rows}x{case.cols}"
        assert np.array_equal(of.cpu().numpy().view(np.uint32), y32.view(np.uint32)), f"{case.rows}x{case.cols}"
        assert bi[0].item() == -7 and bi[-1].item() == -7 and bf[0].item() == -7.0 and bf[-1].item() == -7.0
    plan.free()


TOKEN_SHAPES = ((6912, 2560), (2560, 6912), (640, 2560), (1, 2560), (7, 2500), (65, 6850), (129, 6900),
                (1025, 2560), (3, 6912))


@pytest.mark.parametrize("kernel", (bpw.KERNEL_AUTO, bpw.KERNEL_BITSERIAL))
@pytest.mark.parametrize("batch", (2, 3, 4))
def test_small_batch_grouped_tokens(dev, batch, kernel):
    """2 to 4 tokens over the two model row widths (with ragged rows, ragged columns and junk past
    cols in X): the bit-serial token kernel (pinned) and AUTO (the matrix cores) equal the oracle and
    the single-call matrix-core kernel bit for bit, on two runs of one plan."""
    log(f"case: grouped small batch, bit-serial tokens, B={batch} kernel={kernel}")
    sets = [_sb_inputs(dev, 1200 + 13 * i + batch, r, c, batch) for i, (r, c) in enumerate(TOKEN_SHAPES)]
    jobs = [bpw.sb_job(u.m, Xd, sc, oi, of) for (case, u, Xh, Xd, sc, oi, of) in sets]
    ws = torch.empty(max(bpw.bpw_gemm_small_batch_workspace_bytes(jobs, batch), 256), dtype=torch.uint8, device=dev)
    plan = bpw.SmallBatchPlan(jobs, batch, ws, kernel)
    plan.run()
    plan.run()
    torch.cuda.synchronize()
    for (case, u, Xh, Xd, sc, oi, of) in sets:
        if case.rows == 0:
            continue
        acc, y32, y64 = oracle.gemm_small_batch(oracle.pack(case.w), case.rows, case.cols, Xh, sc, case.w_scale,
                                                nthreads=NT)
        assert np.array_equal(oi.cpu().numpy(), acc), f"{case.rows}x{case.cols}"
        assert np.array_equal(of.cpu().numpy().view(np.uint32), y32.view(np.uint32)), f"{case.rows}x{case.cols}"
        oi2 = torch.empty_like(oi)
        of2 = torch.empty_like(of)
        bpw.bpw_gemm_small_batch(u.m, Xd, sc, oi2, of2, bpw.KERNEL_MFMA)
        torch.cuda.synchronize()
        assert torch.equal(oi2, oi) and torch.equal(of2.view(torch.int32), of.view(torch.int32))
    plan.free()


@pytest.mark.parametrize("batch,kernel", ((2, bpw.KERNEL_BITSERIAL), (4, bpw.KERNEL_AUTO), (16, bpw.KERNEL_AUTO)))
def test_small_batch_grouped_decode_step(dev, batch, kernel):
    """The 210 matrices of a decode step in one launch: at B = 2 on the bit-serial token kernel, at B = 4
    and 16 on the matrix cores (AUTO; the benchmark's launches). Every output against the oracle."""
    log(f"case: grouped small batch, decode step, B={batch} kernel={kernel}")
    sets, jobs = [], []
    for layer in range(synth.N_LAYERS):
        for c in synth.layer_cases(707, layer):
            u = Uploaded(c, dev)
            X, sc = synth.small_batch_x(7000 + 7 * layer + len(sets), batch, c.cols)
            Xd = torch.from_numpy(np.ascontiguousarray(X)).to(dev)
            oi = torch.full((batch, c.rows), -7, dtype=torch.int32, device=dev)
            of = torch.full((batch, c.rows), -7.0, dtype=torch.float32, device=dev)
            sets.append((c, u, X, Xd, sc, oi, of))
            jobs.append(bpw.sb_job(u.m, Xd, sc, oi, of))
    ws = torch.empty(bpw.bpw_gemm_small_batch_workspace_bytes(jobs, batch), dtype=torch.uint8, device=dev)
    plan = bpw.SmallBatchPlan(jobs, batch, ws, kernel)
    plan.run()
    torch.cuda.synchronize()
    log(f"  GPU done; oracle over 210 matrices x {batch} tokens")
    for (c, u, X, Xd, sc, oi, of) in sets:
        acc, y32, _ = oracle.gemm_small_batch(oracle.pack(c.w), c.rows, c.cols, X, sc, c.w_scale, nthreads=NT)
        assert np.array_equal(oi.cpu().numpy(), acc), c.name
        assert np.array_equal(of.cpu().numpy().view(np.uint32), y32.view(np.uint32)), c.name
    plan.free()


def test_small_batch_grouped_new_inputs_and_errors(dev):
    log("case: grouped small batch plan reuse and argument errors")
    batch = 4
    case, u, Xh, Xd, sc, oi, of = _sb_inputs(dev, 950, 6912, 2560, batch)
    jobs = [bpw.sb_job(u.m, Xd, sc, oi, of)]
    ws = torch.empty(bpw.bpw_gemm_small_batch_workspace_bytes(jobs, batch), dtype=torch.uint8, device=dev)
    plan = bpw.SmallBatchPlan(jobs, batch, ws)
    plan.run()
    X2, _ = synth.small_batch_x(951, batch, 2560)
    Xh2 = Xh.copy()
    Xh2[:, :2560] = X2
    Xd.copy_(torch.from_numpy(Xh2))
    plan.run()  # reads the new contents, keeps the scales given at creation
    torch.cuda.synchronize()
    acc, y32, _ = oracle.gemm_small_batch(oracle.pack(case.w), 6912, 2560, Xh2, sc, case.w_scale, nthreads=NT)
    assert np.array_equal(oi.cpu().numpy(), acc)
    assert np.array_equal(of.cpu().numpy().view(np.uint32), y32.view(np.uint32))
    plan.free()
    with pytest.raises(bpw.BpwError) as ei:
        bpw.SmallBatchPlan(jobs, batch, ws, bpw.KERNEL_BYTELANE)
    assert ei.value.status == _lib.E_UNSUPPORTED
    # the bit-serial token kernel: at most 4 tokens, model row widths only
    case5, u5, _, Xd5, sc5, oi5, of5 = _sb_inputs(dev, 952, 64, 2560, 5)
    j5 = [bpw.sb_job(u5.m, Xd5, sc5, oi5, of5)]
    ws5 = torch.empty(bpw.bpw_gemm_small_batch_workspace_bytes(j5, 5), dtype=torch.uint8, device=dev)
    with pytest.raises(bpw.BpwError) as ei:
        bpw.SmallBatchPlan(j5, 5, ws5, bpw.KERNEL_BITSERIAL)
    assert ei.value.status == _lib.E_UNSUPPORTED
    case3, u3, _, Xd3, sc3, oi3, of3 = _sb_inputs(dev, 953, 64, 2000, 3)
    j3 = [bpw.sb_job(u3.m, Xd3, sc3, oi3, of3)]
    ws3 = torch.empty(max(bpw.bpw_gemm_small_batch_workspace_bytes(j3, 3), 256), dtype=torch.uint8, device=dev)
    with pytest.raises(bpw.BpwError) as ei:
        bpw.SmallBatchPlan(j3, 3, ws3, bpw.KERNEL_BITSERIAL)
    assert ei.value.status == _lib.E_UNSUPPORTED
    with pytest.raises(bpw.BpwError) as ei:
        bpw.SmallBatchPlan(jobs, batch, ws[:256])
    assert ei.value.status == _lib.E_SIZE
    with pytest.raises(ValueError):
        bpw.SmallBatchPlan(jobs, batch + 1, ws)  # X holds fewer rows than the plan's batch
    arr = (_lib.BpwSbJob * 1)(jobs[0].c)
    h = ctypes.c_void_p()
    assert _lib.lib().bpw_gemm_small_batch_plan_create(arr, 1, 65, 0, ws.data_ptr(), ws.numel(), None,
                                                       ctypes.byref(h)) == _lib.E_INVAL


# ----------------------------------------------------------------------------- .trit container -> GPU


@pytest.mark.parametrize("writer", ("oracle", "library"))
def test_container_to_grouped_gemv(dev, writer):
    """One layer's seven projections written into a .trit v1 container, opened and verified by the
    library, loaded, uploaded and run as one grouped GEMV: equal to the oracle on the same trits, bit
    for bit. Written by the oracle's writer from the oracle's packing, or by the library's packer and
    writer (the whole product path from int8 trits to outputs)."""
    from oracle import trit_container as tc
    log(f"case: .trit container ({writer} writer) -> load -> upload -> grouped GEMV")
    cases = synth.layer_cases(31337, 0)
    if writer == "oracle":
        data = tc.write(b'{"hidden_size": 2560}', [(c.name, tc.TRIT, [c.rows, c.cols], c.w_scale,
                                                    oracle.pack(c.w).tobytes()) for c in cases], with_hash=False)
    else:
        data = bpw.trit_write([(c.name, bpw.TRIT_TERNARY, [c.rows, c.cols], c.w_scale, bpw.bpw_pack_i8(c.w))
                               for c in cases], b'{"hidden_size": 2560}')
    f = bpw.TritFile(data)
    f.verify()
    ups = []
    for c in cases:
        i = f.find(c.name)
        assert i >= 0
        hm = f.load(i)
        u = Uploaded(c, dev)
        buf = torch.empty(max(hm.nbytes, 1), dtype=torch.uint8, device=dev)
        u.m, u.buf = bpw.bpw_upload(hm, buf), buf  # the container's planes, not the packer's
        hm.free()
        ups.append(u)
    jobs = [u.job() for u in ups]
    ws = torch.empty(bpw.bpw_gemv_workspace_bytes(jobs), dtype=torch.uint8, device=dev)
    bpw.bpw_gemv(jobs, ws)
    torch.cuda.synchronize()
    for u in ups:
        check_case(u, oracle_ref(u.case), f"container {u.case.name}")
    f.close()
