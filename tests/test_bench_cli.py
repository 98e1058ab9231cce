"""bench.py's command line on the host (no GPU): more than one GPU is refused with a message before
anything touches a device, and the committed counter records name the kernel sources they hash."""
import json
import os
import subprocess
import sys

from conftest import ROOT


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", n], capture_output=True,
                           text=True, timeout=120)
        assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_counter_records_name_existing_sources():
    for name in ("gemv_bitserial_decode_step_traffic.json", "gemv_bitcos_decode_step_counters.json"):
        with open(os.path.join(ROOT, "profiles", name)) as f:
            rec = json.load(f)
        assert len(rec["kernel_source_sha256"]) == 64
        for src in rec["kernel_sources"]:
            assert os.path.exists(os.path.join(ROOT, src)), src


def _fake_run(path, rows):
    import csv
    os.makedirs(path, exist_ok=True)
    cols = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    with open(os.path.join(path, "p_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(cols, r)))


def test_counter_records_from_rocprof_csv(tmp_path):
    """The record writer scales byte counters by the copy calibration and takes medians per dispatch."""
    import bench
    step = 11712 * 256
    fetch = [(1, "bpw::stream_probe_kernel<10, 256, true>(...)", 1, "FETCH_SIZE", 524288.0),
             (2, "bpw::stream_probe_kernel<10, 256, true>(...)", 1, "FETCH_SIZE", 524288.0),
             (3, "bpw::gemv_bitserial_kernel(...)", step, "FETCH_SIZE", 254000.0),
             (4, "bpw::gemv_bitserial_kernel(...)", step, "FETCH_SIZE", 256000.0),
             (5, "bpw::gemv_bitserial_kernel(...)", 4096, "FETCH_SIZE", 10.0),  # another plan: ignored
             (6, "bpw::gemv_bitcos_kernel(...)", 1, "FETCH_SIZE", 200000.0)]
    write = [(1, "bpw::flush_kernel(...)", 1, "WRITE_SIZE", 1048576.0),
             (3, "bpw::gemv_bitserial_kernel(...)", step, "WRITE_SIZE", 5000.0),
             (6, "bpw::gemv_bitcos_kernel(...)", 1, "WRITE_SIZE", 5000.0)]
    sq = [(6, "bpw::gemv_bitcos_kernel(...)", 1, c, v) for c, v in
          (("SQ_INSTS_VALU", 5e7), ("SQ_INSTS_LDS", 6e6), ("SQ_LDS_BANK_CONFLICT", 2e7), ("SQ_WAVES", 28800))]
    for name, rows in (("f", fetch), ("w", write), ("s", sq)):
        _fake_run(str(tmp_path / name), rows)
    out_g, out_b = str(tmp_path / "g.json"), str(tmp_path / "b.json")
    bench.write_counter_records(str(tmp_path / "f"), str(tmp_path / "w"), str(tmp_path / "s"), out_g, out_b)
    g, b = json.load(open(out_g)), json.load(open(out_b))
    assert g["fetch_scale"] == 2.0 and g["write_scale"] == 1.0
    assert g["fetch_size_kib_per_dispatch"] == 255000.0
    assert g["traffic_bytes_per_launch"] == (255000 * 2 + 5000) * 1024
    assert g["kernel_source_sha256"] == bench.kernel_source_hash()
    assert b["sq_insts_valu_per_launch"] == 50000000 and b["traffic_bytes_per_launch"] == (200000 * 2 + 5000) * 1024


def test_kernel_hash_covers_the_build_flags(monkeypatch):
    """A counter record names the kernel by its sources and its compiler flags: the same sources built
    with other flags are another kernel, and its traffic is not reported from the record."""
    import bench
    from bit_plane_weight_amd import build as bpw_build
    h = bench.kernel_source_hash()
    base = bpw_build.flags_for
    monkeypatch.setattr(bpw_build, "flags_for", lambda src: [f for f in base(src) if "preload" not in f])
    assert bench.kernel_source_hash() != h
    monkeypatch.setattr(bpw_build, "flags_for", base)
    assert bench.kernel_source_hash() == h
