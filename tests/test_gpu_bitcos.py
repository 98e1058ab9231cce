"""BITCOS GEMV on the GPU ("BITCOS: Intel's Ternary LLM Weight Format Goes Below 1.58 Bits", "A
bitmap and a sign") against the oracle, through the C ABI: the library packs (or re-encodes .trit
planes), uploads and runs one grouped plan; the oracle packs the same trits itself and computes the
GEMV from its own row form. int32 sums bit-exact, fp32 outputs bit-exact to the scales-in-turn
product (and within 1e-6 relative of the float64 one)."""
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


class BcUploaded:
    def __init__(self, case, dev, from_planes=False, tail_junk=False):
        self.case = case
        if from_planes:
            hm = bpw.bpw_load(bpw.bpw_pack_i8(case.w), case.rows, case.cols, case.w_scale)
            h = bpw.bpw_bitcos_from_planes(hm)
            hm.free()
        else:
            h = bpw.bpw_bitcos_pack_i8(case.w, case.w_scale)
        self.buf = torch.empty(h.device_bytes, dtype=torch.uint8, device=dev)
        self.m = bpw.bpw_bitcos_upload(h, self.buf)
        h.free()
        bpr = (case.cols + 63) // 64
        xh = np.zeros(max(bpr * 64, 16), np.int8)
        if tail_junk:
            xh[:] = synth.u64(case.cols + 9, xh.size).astype(np.uint8).view(np.int8)
        xh[: case.cols] = case.x
        self.x = torch.from_numpy(xh).to(dev)
        self.oi = torch.full((max(case.rows, 1),), 0x7EADBEEF, dtype=torch.int32, device=dev)
        self.of = torch.full((max(case.rows, 1),), float("nan"), dtype=torch.float32, device=dev)

    def job(self, with_f32=True):
        return bpw.bitcos_job(self.m, self.x, self.case.x_scale, self.oi, self.of if with_f32 else None)


def bitcos_ref(case):
    P, S, R = oracle.bitcos_pack_rows(case.w)
    return oracle.bitcos_gemv(P, S, R, case.rows, case.cols, case.x, case.x_scale, case.w_scale)


def trit_ref(case):
    return oracle.gemv(oracle.pack(case.w), case.rows, case.cols, case.x, case.x_scale, case.w_scale, nthreads=NT)


def check(u, ref, what, with_f32=True):
    acc, y32, y64 = ref
    rows = u.case.rows
    gi = u.oi.cpu().numpy()[:rows]
    bad = np.nonzero(gi != acc)[0]
    assert bad.size == 0, f"{what}: int32 differs at rows {bad[:8].tolist()} (got {gi[bad[:4]]}, want {acc[bad[:4]]})"
    if not with_f32:
        assert np.all(np.isnan(u.of.cpu().numpy()[:rows])), f"{what}: fp32 written without d_out_f32"
        return
    gf = u.of.cpu().numpy()[:rows]
    err = np.abs(gf.astype(np.float64) - y64)
    assert np.all(err <= 1e-6 * np.abs(y64)), f"{what}: fp32 outside rel 1e-6"
    assert np.array_equal(gf.view(np.uint32), y32.view(np.uint32)), f"{what}: fp32 bits differ from scales-in-turn"


def run(ups, dev, with_f32=True, reps=1):
    jobs = [u.job(with_f32) for u in ups]
    ws = torch.empty(max(bpw.bpw_bitcos_workspace_bytes(jobs), 256), dtype=torch.uint8, device=dev)
    plan = bpw.BitcosPlan(jobs, ws)
    for _ in range(reps):
        plan.run()
    torch.cuda.synchronize()
    plan.free()


def test_one_layer_seven_projections(dev):
    log("case: BITCOS one layer, 7 projections grouped")
    cases = synth.layer_cases(5151, 2)
    ups = [BcUploaded(c, dev) for c in cases]
    run(ups, dev, reps=2)
    for u in ups:
        check(u, bitcos_ref(u.case), u.case.name)


@pytest.mark.parametrize("z", synth.P_ZERO_SWEEP)
def test_zero_density_sweep_layer(dev, z):
    log(f"case: BITCOS layer at P(0)={z}")
    cases = synth.layer_cases(5252, 1, p_zero=z)
    ups = [BcUploaded(c, dev) for c in cases]
    run(ups, dev)
    for u in ups:
        check(u, bitcos_ref(u.case), f"{u.case.name} z={z}")


RAGGED = ((1, 1), (3, 63), (5, 64), (7, 65), (17, 200), (9, 2560), (33, 6912), (129, 8192), (1, 4096), (8, 640),
          (65, 3000), (31, 4000), (70, 1025), (3, 7000),
          (130, 127), (1025, 2560), (0, 100), (5, 0))


@pytest.mark.parametrize("from_planes", (False, True))
def test_ragged_shapes_grouped(dev, from_planes):
    log(f"case: BITCOS ragged shapes grouped, from_planes={from_planes}")
    cases = [synth.ternary_case(5353, 0, i, r, c, name=f"{r}x{c}") for i, (r, c) in enumerate(RAGGED)]
    ups = [BcUploaded(c, dev, from_planes, tail_junk=True) for c in cases]
    run(ups, dev)
    for u in ups:
        if u.case.rows == 0:
            continue
        if u.case.cols == 0:
            assert np.all(u.oi.cpu().numpy()[: u.case.rows] == 0)
            assert np.all(u.of.cpu().numpy()[: u.case.rows] == 0.0)
            continue
        check(u, bitcos_ref(u.case), u.case.name)


def test_extremes_and_no_f32(dev):
    """Every weight -1 (every sign word full) or +1 against x = -128 everywhere: the largest sums; zero
    density 1 and 0 on one matrix each; a job without d_out_f32."""
    log("case: BITCOS extremes")
    cases = []
    for i, (r, c, v) in enumerate(((64, 8192, -1), (64, 8192, 1), (40, 6912, 0), (3, 2560, -1))):
        cs = synth.ternary_case(5454, 0, i, r, c, name=f"{r}x{c}:{v}")
        cs.w = np.full((r, c), v, np.int8)
        cs.x = np.full(c, -128, np.int8)
        cases.append(cs)
    ups = [BcUploaded(c, dev) for c in cases]
    run(ups[:3], dev)
    run(ups[3:], dev, with_f32=False)
    for u in ups[:3]:
        check(u, bitcos_ref(u.case), u.case.name)
    assert ups[0].oi.cpu().numpy()[0] == 128 * 8192
    check(ups[3], bitcos_ref(ups[3].case), ups[3].case.name, with_f32=False)


def test_decode_step_210_matrices_full(dev):
    """All 210 matrices of a decode step as BITCOS in one plan launch (the benchmark's), every output
    checked against the .trit oracle on the same trits (the BITCOS oracle equals it: pinned on the CPU)."""
    log("case: BITCOS decode step, 210 matrices")
    ups = []
    for layer in range(synth.N_LAYERS):
        for c in synth.layer_cases(303, layer):
            ups.append(BcUploaded(c, dev))
    run(ups, dev, reps=2)
    log("  GPU done; oracle over 210 matrices")
    for u in ups:
        check(u, trit_ref(u.case), u.case.name)


def test_bitcos_equals_trit_gemv_on_gpu(dev):
    """The BITCOS plan and the .trit bit-serial plan give identical outputs on one layer."""
    log("case: BITCOS vs .trit GEMV on the GPU")
    cases = synth.layer_cases(5555, 4)
    ups = [BcUploaded(c, dev) for c in cases]
    run(ups, dev)
    for u in ups:
        planes = bpw.bpw_pack_i8(u.case.w)
        hm = bpw.bpw_load(planes, u.case.rows, u.case.cols, u.case.w_scale)
        buf = torch.empty(hm.nbytes, dtype=torch.uint8, device=dev)
        m = bpw.bpw_upload(hm, buf)
        oi = torch.zeros(u.case.rows, dtype=torch.int32, device=dev)
        of = torch.zeros(u.case.rows, dtype=torch.float32, device=dev)
        j = bpw.gemv_job(m, u.x, u.case.x_scale, oi, of)
        ws = torch.empty(bpw.bpw_gemv_workspace_bytes([j]), dtype=torch.uint8, device=dev)
        bpw.bpw_gemv([j], ws)
        torch.cuda.synchronize()
        assert torch.equal(oi, u.oi) and torch.equal(of.view(torch.int32), u.of.view(torch.int32)), u.case.name
        hm.free()


def test_argument_errors(dev):
    log("case: BITCOS argument errors")
    c = synth.ternary_case(5656, 0, 0, 16, 200)
    u = BcUploaded(c, dev)
    j = u.job()
    ws = torch.empty(max(bpw.bpw_bitcos_workspace_bytes([j]), 256), dtype=torch.uint8, device=dev)
    # a modified descriptor
    j2 = u.job()
    j2.m.rows = 17
    with pytest.raises(bpw.BpwError) as e:
        bpw.BitcosPlan([j2], ws)
    assert e.value.status == _lib.E_NOT_VALIDATED
    # short x, NULL output, workspace too small, unaligned workspace, unaligned d_x
    j3 = u.job()
    j3.x_len = 64 * 3
    with pytest.raises(bpw.BpwError) as e:
        bpw.BitcosPlan([j3], ws)
    assert e.value.status == _lib.E_INVAL
    j4 = u.job()
    j4.d_out_i32 = None
    with pytest.raises(bpw.BpwError) as e:
        bpw.BitcosPlan([j4], ws)
    assert e.value.status == _lib.E_INVAL
    with pytest.raises(bpw.BpwError) as e:
        bpw.BitcosPlan([j], ws[:16])
    assert e.value.status == _lib.E_SIZE
    ws2 = torch.empty(ws.numel() + 256, dtype=torch.uint8, device=dev)
    with pytest.raises(bpw.BpwError) as e:
        bpw.BitcosPlan([j], ws2[1:])
    assert e.value.status == _lib.E_INVAL and "aligned" in e.value.reason
    j5 = u.job()
    j5.d_x = u.x.data_ptr() + 1
    with pytest.raises(bpw.BpwError) as e:
        bpw.BitcosPlan([j5], ws)
    assert e.value.status == _lib.E_INVAL
    # upload into a short or unaligned buffer
    h = bpw.bpw_bitcos_pack_i8(c.w, c.w_scale)
    with pytest.raises(bpw.BpwError) as e:
        bpw.bpw_bitcos_upload(h, u.buf[: h.device_bytes - 1])
    assert e.value.status == _lib.E_SIZE
    big = torch.empty(h.device_bytes + 256, dtype=torch.uint8, device=dev)
    with pytest.raises(bpw.BpwError) as e:
        bpw.bpw_bitcos_upload(h, big[1:])
    assert e.value.status == _lib.E_INVAL
    # a plan of no jobs runs and does nothing
    p = bpw.BitcosPlan([], None)
    p.run()
    p.free()
    # the untouched job still runs correctly after the refusals
    run([u], dev)
    check(u, bitcos_ref(c), "after errors")
