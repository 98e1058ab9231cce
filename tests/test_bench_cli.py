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
