"""libbpw's untrusted-input host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The container reader and writer, the plane packer / validator / loader and the BITCOS packers are
compiled from the library's own host sources with clang's -fsanitize=address,undefined
(tests/sanitize holds the driver; the GPU launchers and HIP calls are stubs that abort if reached)
and run over the same suites as the ctypes tests: every truncation of the format page's complete
file and of a multi-tensor file, the 3,000 random header mutations, payload bit flips, the
validator's corruption suites with hostile lengths and shapes, the packers over ragged shapes, bad
values and the zero-density range, and the container writer rewriting every file of the container
suites. Every result line is compared with the oracle, and any sanitizer report fails the run."""
import os
import shutil
import struct
import subprocess

import numpy as np
import pytest

import oracle
import synth
from conftest import ROOT
from oracle import trit_container as tc
from test_trit_container_pins import CHECK_CASES, PAGE, header_mutations, patched, payload_bit_flips, sample_file

CSRC = os.path.join(ROOT, "bit_plane_weight_amd", "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("bpw_trit.cpp", "bpw_host.cpp", "bpw_bitcos_host.cpp")]
DRIVER = os.path.join(ROOT, "tests", "sanitize", "bpw_host_driver.cpp")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]

E_INVAL, E_SIZE, E_P1, E_P2, E_UNSUPPORTED = 1, 2, 3, 4, 8


def _clang():
    for c in ("/opt/rocm/lib/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    return None


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = _clang()
    if cxx is None:
        pytest.skip("clang++ not found")
    out = tmp_path_factory.mktemp("sanitize")
    objs = []
    procs = []
    for src in SOURCES + [DRIVER]:
        obj = str(out / (os.path.basename(src) + ".o"))
        cmd = [cxx, "-std=c++17", "-O1", "-g", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-c", src,
               "-o", obj]
        procs.append((subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT), cmd))
        objs.append(obj)
    for p, cmd in procs:
        log = p.communicate()[0].decode()
        assert p.returncode == 0, (cmd, log)
    exe = str(out / "bpw_host_driver")
    r = subprocess.run([cxx, *SAN, *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def run_cases(exe, tmp_path, records):
    """records: (op, flags, rows, cols, bytes) -> the driver's output lines."""
    path = tmp_path / "cases.bin"
    with open(path, "wb") as f:
        for op, flags, rows, cols, data in records:
            f.write(struct.pack("<IIqqQ", op, flags, rows, cols, len(data)))
            f.write(data)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:halt_on_error=1:abort_on_error=0:exitcode=99"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=98"
    r = subprocess.run([exe, str(path)], capture_output=True, text=True, env=env, timeout=600)
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    lines = r.stdout.splitlines()
    assert len(lines) == len(records)
    return lines


# ---------------------------------------------------------------- expected lines, from the oracle


def container_expected(data: bytes, flags: int) -> str:
    try:
        g = tc.TritFile(data)
    except tc.TritError as e:
        return f"{e.check} {e.tensor} {e.row} {e.beat} {e.col}"
    head = "0 -1 -1 -1 -1"
    if flags & 1:
        try:
            g.verify(bool(flags & 2))
        except tc.TritError as e:
            head = f"{e.check} {e.tensor} {e.row} {e.beat} {e.col}"
    parts = [f"{head} | {len(g.tensors)} {g.payload_hash} {len(g.config)}"]
    for i, t in enumerate(g.tensors):
        if t.dtype != tc.TRIT:
            parts.append(f"{t.dtype}:{i}:{E_INVAL}:-1:-1:-1")
            continue
        try:
            oracle.validate(np.frombuffer(g.payload(i), np.uint8), t.dims[0], t.dims[1])
            parts.append(f"{t.dtype}:{i}:0:-1:-1:-1")
        except oracle.OracleError as e:
            parts.append(f"{t.dtype}:{i}:{e.code}:{e.row}:{e.beat}:{e.col}")
    return " ".join(parts)


def rewrite_expected(data: bytes, flags: int) -> str:
    """The library writer, given an opened file's tensors in record order and its config, refuses what the
    oracle's verify refuses (P1 / P2: check, tensor, row, beat, column) and otherwise writes exactly the
    oracle writer's bytes for the same tensors."""
    try:
        g = tc.TritFile(data)
    except tc.TritError as e:
        return f"open {e.check} {e.tensor}"
    try:
        g.verify(False)
    except tc.TritError as e:
        return f"{e.check} {e.tensor} {e.row} {e.beat} {e.col}"
    ts = [(t.name.decode("utf-8"), t.dtype, t.dims, t.scale, g.payload(i)) for i, t in enumerate(g.tensors)]
    out = tc.write(g.config, ts, with_hash=bool(flags & 1))
    return f"0 | {len(out)} {tc.fnv1a64(out)}"


def lib_shape_ok(rows: int, cols: int) -> bool:
    """The library's documented shape limits: rows <= INT32_MAX, cols <= 2^40, plane bytes < 2^63."""
    if rows < 0 or cols < 0 or rows > 2**31 - 1 or cols > 2**40:
        return False
    return rows * ((cols + 63) // 64) * 16 < 2**63


def planes_expected(planes: bytes, rows: int, cols: int) -> str:
    if not lib_shape_ok(rows, cols):
        return f"{E_INVAL} -1 -1 -1 {E_INVAL}"
    if len(planes) != rows * ((cols + 63) // 64) * 16:
        return f"{E_SIZE} -1 -1 -1 {E_SIZE}"
    try:
        oracle.validate(np.frombuffer(planes, np.uint8), rows, cols)
    except oracle.OracleError as e:
        return f"{e.code} {e.row} {e.beat} {e.col} {e.code}"
    return "0 -1 -1 -1 0"


def _up(v):
    return (v + 255) // 256 * 256


def bitcos_expected(w) -> str:
    P, S, R = oracle.bitcos_pack_rows(w)
    dev = _up(P.size * 8) + _up(R.size * 4) + _up((S.size + 4) * 4)
    return (f"{tc.fnv1a64(P.tobytes())} {tc.fnv1a64(S.tobytes())} {tc.fnv1a64(R.tobytes())} "
            f"{int(np.count_nonzero(w))} {S.size} {dev}")


def trits_expected(w) -> str:
    rows, cols = w.shape
    try:
        planes = oracle.pack(w)
        bad = None
    except oracle.OracleError as e:
        bad = f"{e.row} {e.beat} {e.col}"
    out = f"0 -1 -1 -1 {tc.fnv1a64(planes.tobytes())}" if bad is None else f"{E_INVAL} {bad} 0"
    if cols > 8192:  # the BITCOS kernel's limit, checked before the values
        out += f" / {E_UNSUPPORTED} -1 -1 -1"
    else:
        out += f" / {E_INVAL} {bad}" if bad is not None else " / 0 -1 -1 -1 " + bitcos_expected(w)
    if bad is None:
        out += f" / {E_UNSUPPORTED}" if cols > 8192 else " / " + bitcos_expected(w)
    return out


# ---------------------------------------------------------------- suites


def container_records():
    recs = []
    valid = [PAGE, sample_file(1), sample_file(2, n=1), sample_file(3), tc.write(b"", [])]
    for data in valid:
        for flags in (0, 1, 3):
            recs.append((1, flags, 0, 0, data))
    for off, new, _ in CHECK_CASES:
        for flags in (0, 3):
            recs.append((1, flags, 0, 0, patched(PAGE, off, new)))
    for data in (PAGE, sample_file(3)):  # the truncation suite
        recs += [(1, 3, 0, 0, data[:n]) for n in range(len(data))]
    recs += [(1, 3, 0, 0, d) for d in header_mutations(sample_file(4))]
    recs += [(1, 1, 0, 0, d) for d in payload_bit_flips(sample_file(5, hashed=False))]
    bad = bytearray(sample_file(6))
    bad[-1] ^= 0x10
    recs += [(1, 3, 0, 0, bytes(bad)), (1, 1, 0, 0, bytes(bad))]
    return recs


def _corrupt(planes, rows, bpr, r, b, plane, k):
    p = planes.copy().reshape(rows, bpr, 2, 8)
    word = int.from_bytes(p[r, b, plane].tobytes(), "little") | (1 << k)
    p[r, b, plane] = np.frombuffer(word.to_bytes(8, "little"), np.uint8)
    return p.reshape(-1)


def planes_records():
    recs = []
    for cols in (1, 31, 32, 33, 63, 64, 65, 127, 200, 2560, 8193):
        rows = 4
        bpr = (cols + 63) // 64
        base = oracle.pack(synth.trits(cols, rows, cols))
        rng = np.random.default_rng(cols)
        recs.append((2, 0, rows, cols, base.tobytes()))
        for _ in range(60):
            p = base
            for _ in range(int(rng.integers(1, 3))):
                p = _corrupt(p, rows, bpr, int(rng.integers(rows)), int(rng.integers(bpr)), int(rng.integers(2)),
                             int(rng.integers(64)))
            recs.append((2, 0, rows, cols, p.tobytes()))
        # lengths that do not match the shape, and shapes that do not match the length
        for data in (base[:-1], base[:-16], np.concatenate([base, base[:16]]), base[:0]):
            recs.append((2, 0, rows, cols, data.tobytes()))
        recs += [(2, 0, rows + 1, cols, base.tobytes()), (2, 0, rows, cols + 64, base.tobytes())]
    # empty matrices and hostile shapes: negative, beyond the limits, and rows * bpr * 16 past 2^64,
    # where (2^60 + 1) * 16 = 16 modulo 2^64 would match a 16-byte buffer if the count wrapped
    for rows, cols in ((0, 0), (0, 100), (5, 0), (-1, 64), (4, -1), (2**31, 64), (1, 2**40 + 1),
                       (2**31 - 1, 2**40), (17 * 241 * 61681, 4562284561 * 64)):
        recs.append((2, 0, rows, cols, b""))
        recs.append((2, 0, rows, cols, bytes(16)))
    return recs


def trits_records():
    shapes = ((1, 1), (3, 63), (5, 64), (7, 65), (17, 200), (9, 2560), (4, 6912), (3, 8192), (2, 8193),
              (0, 100), (5, 0), (0, 0), (17, 129))
    ws = [synth.trits(rows * 7 + cols, rows, cols) for rows, cols in shapes]
    for z in (0.2966, 0.5148, 0.95):
        ws.append(synth.trits(33, 40, 2500, z))
    ws.append(np.where(synth.trits(34, 40, 2500, 0.5) < 0, -1, 1).astype(np.int8))
    ws.append(np.zeros((40, 2500), np.int8))
    for cols, r, c, v in ((70, 2, 66, 2), (200, 0, 5, 5), (64, 1, 63, -2), (3, 0, 2, 127), (8193, 1, 8192, -128)):
        w = synth.trits(cols + r, 3, cols)
        w[r, c] = v
        ws.append(w)
    return [(3, 0, w.shape[0], w.shape[1], np.ascontiguousarray(w).tobytes()) for w in ws], ws


def test_container_suites_under_sanitizers(driver, tmp_path):
    recs = container_records()
    assert len(recs) > 4500
    lines = run_cases(driver, tmp_path, recs)
    for k, ((_, flags, _, _, data), line) in enumerate(zip(recs, lines)):
        assert line == container_expected(data, flags), (k, len(data), line)


def test_writer_rewrites_under_sanitizers(driver, tmp_path):
    """bpw_trit_write over every container of the suites above (written back from the opened tensors,
    with and without the payload hash): byte for byte the oracle writer's output, or the same P1 / P2
    refusal as the oracle's verify; every written file reopens and verifies."""
    recs = [(4, flags & 1, 0, 0, data) for _, flags, _, _, data in container_records()]
    lines = run_cases(driver, tmp_path, recs)
    kinds = set()
    for k, ((_, flags, _, _, data), line) in enumerate(zip(recs, lines)):
        assert line == rewrite_expected(data, flags), (k, len(data), line)
        kinds.add(line.split()[0])
    assert {"0", "open", "17", "18"} <= kinds, kinds


def test_validator_suites_under_sanitizers(driver, tmp_path):
    recs = planes_records()
    lines = run_cases(driver, tmp_path, recs)
    codes = set()
    for k, ((_, _, rows, cols, data), line) in enumerate(zip(recs, lines)):
        assert line == planes_expected(data, rows, cols), (k, rows, cols, len(data), line)
        codes.add(int(line.split()[0]))
    assert codes == {0, E_INVAL, E_SIZE, E_P1, E_P2}


def test_packers_under_sanitizers(driver, tmp_path):
    recs, ws = trits_records()
    lines = run_cases(driver, tmp_path, recs)
    for k, (w, line) in enumerate(zip(ws, lines)):
        assert line == trits_expected(w), (k, w.shape, line)
