"""bpw_gemv_noalloc (the grouped GEMV with the library's fixed device scratch in place of a caller
workspace) against bpw_gemv with a workspace, through the C ABI: the same int32 sums and fp32 bits on
two calls in a row, the second over a smaller job list, and the oracle's sums on both. Jobs whose
tables exceed the scratch are refused before anything is launched."""
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


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU (they fail rather than skip)"
    d = torch.device("cuda:0")
    torch.cuda.set_device(d)
    bpw.bpw_device_check()
    return d


class Two:
    """One ternary case on the GPU with two sets of outputs: one per entry point."""

    def __init__(self, case, dev):
        self.case = case
        hm = bpw.bpw_load(bpw.bpw_pack_i8(case.w), case.rows, case.cols, case.w_scale)
        self.buf = torch.empty(max(hm.nbytes, 1), dtype=torch.uint8, device=dev)
        self.m = bpw.bpw_upload(hm, self.buf)
        hm.free()
        bpr = (case.cols + 63) // 64
        xh = np.zeros(max(bpr * 64, 16), np.int8)
        xh[: case.cols] = case.x
        self.x = torch.from_numpy(xh).to(dev)
        n = max(case.rows, 1)
        self.out = [(torch.full((n,), 0x7EADBEEF, dtype=torch.int32, device=dev),
                     torch.full((n,), float("nan"), dtype=torch.float32, device=dev)) for _ in range(2)]

    def job(self, k):
        oi, of = self.out[k]
        return bpw.gemv_job(self.m, self.x, self.case.x_scale, oi, of)


def compare(items, what):
    for t in items:
        rows = t.case.rows
        (ai, af), (bi, bf) = [(oi.cpu().numpy()[:rows], of.cpu().numpy()[:rows]) for oi, of in t.out]
        assert np.array_equal(ai, bi), f"{what}: int32 differs from bpw_gemv on {rows}x{t.case.cols}"
        assert np.array_equal(af.view(np.uint32), bf.view(np.uint32)), f"{what}: fp32 bits differ on {rows}x{t.case.cols}"
        acc, y32, _ = oracle.gemv(oracle.pack(t.case.w), rows, t.case.cols, t.case.x, t.case.x_scale, t.case.w_scale,
                                  nthreads=NT)
        assert np.array_equal(bi, acc), f"{what}: int32 differs from the oracle on {rows}x{t.case.cols}"
        assert np.array_equal(bf.view(np.uint32), y32.view(np.uint32)), f"{what}: fp32 differs from the oracle"


def run_both(items, dev):
    jobs_ws = [t.job(0) for t in items]
    ws = torch.empty(bpw.bpw_gemv_workspace_bytes(jobs_ws), dtype=torch.uint8, device=dev)
    bpw.bpw_gemv(jobs_ws, ws)
    bpw.bpw_gemv_noalloc([t.job(1) for t in items])
    torch.cuda.synchronize()


def test_noalloc_matches_workspace_entry_point_on_two_calls(dev):
    log("case: bpw_gemv_noalloc, call 1: one layer's seven projections and a ragged matrix")
    first = [Two(synth.ternary_case(4100, 0, proj, rows, cols), dev)
             for proj, (name, rows, cols) in enumerate(synth.PROJECTIONS)]
    first.append(Two(synth.ternary_case(4101, 0, 0, 70, 6900), dev))
    run_both(first, dev)
    compare(first, "call 1")
    log("case: bpw_gemv_noalloc, call 2: two smaller matrices")
    second = [Two(synth.ternary_case(4200, 1, 1, 640, 2560), dev), Two(synth.ternary_case(4201, 1, 0, 33, 129), dev)]
    run_both(second, dev)
    compare(second, "call 2")


def test_noalloc_refuses_tables_beyond_its_scratch(dev):
    log("case: bpw_gemv_noalloc refuses 5000 jobs (tables beyond 1 MiB)")
    t = Two(synth.ternary_case(4300, 0, 1, 640, 2560), dev)
    jobs = [t.job(1)] * 5000
    assert bpw.bpw_gemv_workspace_bytes(jobs) > (1 << 20)
    before = t.out[1][0].clone()
    with pytest.raises(bpw.BpwError) as ei:
        bpw.bpw_gemv_noalloc(jobs)
    assert ei.value.status == _lib.E_SIZE and "static scratch" in ei.value.reason
    torch.cuda.synchronize()
    assert torch.equal(t.out[1][0], before)  # nothing was launched
    run_both([t], dev)  # and the entry point still serves a list that fits
    compare([t], "after the refusal")
