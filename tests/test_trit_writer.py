"""bpw_trit_write, the library's .trit v1 writer (no GPU), against the oracle's writer and reader.

- Byte for byte the oracle writer's output ("The .trit format, version 1", sections 2-2.4: header,
  records sorted by name, 64-byte aligned payloads, the file ending with the last tensor) over random
  containers: names with multi-byte UTF-8, all three dtypes, empty tensors, empty and non-empty
  configs, with and without the payload hash, the input in shuffled order.
- The page's worked file, except the hash bytes (the printed hash agrees with FNV-1a-64 in its low 40
  bits only; the stored one is FNV-1a-64 of the payload).
- Every refusal carries the number of the section 4 check that the oracle's reader reports on the same
  tensors written without checks (and P1 / P2 with their row, beat and column).
- The output-size contract of the C call."""
import ctypes
import random
import struct

import numpy as np
import pytest

import bit_plane_weight_amd as bpw
import oracle
import synth
from bit_plane_weight_amd import _lib
from oracle import trit_container as tc
from test_trit_container_pins import PAGE, read_worked_example

NAME_PARTS = ("w", "model.layers.0.q", "é", "日本", "ß", "\U0001F600", "a.b", "z", "norm", "x" * 40)


def random_tensors(seed: int, n: int):
    rng = np.random.default_rng(seed)
    names, tensors = set(), []
    while len(tensors) < n:
        name = "".join(rng.choice(NAME_PARTS) for _ in range(int(rng.integers(1, 4))))
        if name in names:
            continue
        names.add(name)
        dtype = int(rng.integers(0, 3))
        scale = float(np.float32(rng.uniform(0.01, 4.0)))
        if dtype == tc.TRIT:
            rows, cols = int(rng.integers(0, 6)), int(rng.integers(0, 200))
            w = synth.trits(seed * 131 + len(tensors), rows, cols) if rows and cols else np.zeros((rows, cols), np.int8)
            data = oracle.pack(w).tobytes() if rows and cols else bytes(rows * ((cols + 63) // 64) * 16)
            tensors.append((name, dtype, [rows, cols], scale, data))
        else:
            dims = [int(rng.integers(0, 6)) for _ in range(int(rng.integers(1, 5)))]
            count = int(np.prod(dims)) * (4 if dtype == tc.F32 else 2)
            data = rng.integers(0, 256, size=count, dtype=np.uint8).tobytes()
            tensors.append((name, dtype, dims, 1.0 if rng.random() < 0.5 else scale, data))
    return tensors


@pytest.mark.parametrize("seed", range(24))
def test_matches_oracle_writer(seed):
    ts = random_tensors(seed, seed % 9)
    cfg = b"" if seed % 3 == 0 else ('{"seed": %d, "name": "tést"}' % seed).encode()
    shuffled = ts[:]
    random.Random(seed).shuffle(shuffled)
    for with_hash in (True, False):
        ref = tc.write(cfg, ts, with_hash=with_hash)
        out = bpw.trit_write(shuffled, cfg, with_hash)
        assert out == ref
        f = bpw.TritFile(out)
        f.verify()
        assert f.config == cfg and len(f) == len(ts)
        start = tc.TritFile(out).payload_start
        assert f.stored_hash == (tc.fnv1a64(out[start:]) if with_hash else 0)
        for name, dtype, dims, scale, data in ts:
            t = f.tensor(f.find(name))
            assert (t.dtype, t.dims, t.scale) == (dtype, dims, scale) and t.bytes() == data


def test_page_file_except_hash():
    rows, cols, scale, w, payload = read_worked_example()
    out = bpw.trit_write([("w", tc.TRIT, [2, 3], 0.5, payload)], b'{"hidden_size":3}')
    assert len(out) == len(PAGE)
    assert out[:12] == PAGE[:12] and out[20:] == PAGE[20:]
    assert struct.unpack("<Q", out[12:20])[0] == tc.fnv1a64(payload)
    plain = bpw.trit_write([("w", tc.TRIT, [2, 3], 0.5, payload)], b'{"hidden_size":3}', with_hash=False)
    assert plain[12:20] == bytes(8) and plain[:12] + plain[20:] == out[:12] + out[20:]


def reader_verdict(cfg: bytes, tensors) -> tuple:
    """The oracle reader's first failure on the tensors written without any check."""
    data = tc.write(cfg, tensors)
    try:
        g = tc.TritFile(data)
        g.verify(False)
    except tc.TritError as e:
        return e.check, e.row, e.beat, e.col
    return 0, -1, -1, -1


def corrupted(rows, cols, r, b, plane, bit, seed=5):
    p = oracle.pack(synth.trits(seed, rows, cols)).reshape(rows, (cols + 63) // 64, 2, 8).copy()
    word = int.from_bytes(p[r, b, plane].tobytes(), "little") | (1 << bit)
    p[r, b, plane] = np.frombuffer(word.to_bytes(8, "little"), np.uint8)
    return p.reshape(-1).tobytes()


GOOD = ("g", tc.F32, [2], 1.0, bytes(8))
REFUSALS = [
    ("config not UTF-8", b"\xff\xfe", [GOOD]),
    ("empty name", b"{}", [("", tc.F32, [1], 1.0, bytes(4))]),
    ("name of 1025 bytes", b"{}", [("n" * 1025, tc.F32, [1], 1.0, bytes(4))]),
    ("duplicate name", b"{}", [GOOD, ("g", tc.BF16, [1], 1.0, bytes(2))]),
    ("unknown dtype", b"{}", [("d", 3, [1], 1.0, bytes(4))]),
    ("no dims", b"{}", [("d", tc.F32, [], 1.0, bytes(4))]),
    ("shape product past 2^64", b"{}", [("d", tc.F32, [2**32 - 1] * 3, 1.0, bytes(4))]),
    ("zero scale", b"{}", [("d", tc.F32, [1], 0.0, bytes(4))]),
    ("negative scale", b"{}", [("d", tc.F32, [1], -1.0, bytes(4))]),
    ("NaN scale", b"{}", [("d", tc.F32, [1], float("nan"), bytes(4))]),
    ("infinite scale", b"{}", [("d", tc.TRIT, [1, 64], float("inf"), bytes(16))]),
    ("ternary with one dim", b"{}", [("t", tc.TRIT, [64], 1.0, bytes(16))]),
    ("ternary with three dims", b"{}", [("t", tc.TRIT, [1, 1, 64], 1.0, bytes(16))]),
    ("ternary byte_len", b"{}", [("t", tc.TRIT, [2, 65], 1.0, bytes(48))]),
    ("dense byte_len", b"{}", [("d", tc.BF16, [3, 3], 1.0, bytes(16))]),
    ("P1 both bits", b"{}", [GOOD, ("t", tc.TRIT, [3, 130], 1.0, corrupted(3, 130, 2, 1, 0, 5))]),
    ("P2 padding bit", b"{}", [("t", tc.TRIT, [3, 130], 1.0, corrupted(3, 130, 1, 2, 1, 63)), GOOD]),
]


@pytest.mark.parametrize("what,cfg,tensors", REFUSALS, ids=[r[0] for r in REFUSALS])
def test_refusals_carry_the_readers_check(what, cfg, tensors):
    check, row, beat, col = reader_verdict(cfg, tensors)
    assert check > 0, what
    with pytest.raises(bpw.TritFormatError) as ei:
        bpw.trit_write(tensors, cfg)
    assert ei.value.check == check, (what, ei.value.check, check)
    if check in (17, 18):
        assert (ei.value.row, ei.value.beat, ei.value.col) == (row, beat, col)
        assert ei.value.status == (_lib.E_P1_BOTH_BITS if check == 17 else _lib.E_P2_PADDING)
    else:
        assert ei.value.status == _lib.E_FORMAT


def test_name_not_utf8_is_check_7():
    with pytest.raises(bpw.TritFormatError) as ei:
        bpw.trit_write([(b"\xc0\x80", tc.F32, [1], 1.0, bytes(4))])
    assert ei.value.check == 7


def _one(dtype=tc.F32, dims=(1,), data=bytes(4), reserved=0, name=b"a"):
    t = _lib.BpwTritTensorIn()
    t.name, t.name_len, t.dtype, t.ndim = name, len(name), dtype, len(dims)
    for j, d in enumerate(dims):
        t.dims[j] = d
    t.scale, t.reserved = 1.0, reserved
    buf = ctypes.create_string_buffer(data, len(data)) if data else None
    t.data = ctypes.cast(buf, ctypes.c_void_p) if buf is not None else None
    t.byte_len = len(data)
    return t, buf


def test_output_size_contract():
    t, keep = _one()
    L = _lib.lib()
    need, written, err = ctypes.c_uint64(), ctypes.c_uint64(), _lib.BpwTritErr()
    assert L.bpw_trit_write_size(ctypes.byref(t), 1, 2, ctypes.byref(need), ctypes.byref(err)) == _lib.OK
    assert need.value == len(tc.write(b"{}", [("a", tc.F32, [1], 1.0, bytes(4))]))
    out = (ctypes.c_uint8 * need.value)(*([0xAB] * need.value))
    st = L.bpw_trit_write(ctypes.byref(t), 1, b"{}", 2, 1, out, need.value - 1, ctypes.byref(written), ctypes.byref(err))
    assert st == _lib.E_SIZE and written.value == need.value and bytes(out) == b"\xab" * need.value
    st = L.bpw_trit_write(ctypes.byref(t), 1, b"{}", 2, 1, out, need.value, ctypes.byref(written), ctypes.byref(err))
    assert st == _lib.OK and written.value == need.value
    assert bytes(out) == tc.write(b"{}", [("a", tc.F32, [1], 1.0, bytes(4))])
    # an empty container: header and config only, the payload starting (and the file ending) at 64
    assert L.bpw_trit_write_size(None, 0, 0, ctypes.byref(need), ctypes.byref(err)) == _lib.OK
    assert need.value == len(tc.write(b"", [])) == 64


def test_reserved_and_null_data_refused():
    L = _lib.lib()
    need, err = ctypes.c_uint64(), _lib.BpwTritErr()
    t, keep = _one(reserved=1)
    assert L.bpw_trit_write_size(ctypes.byref(t), 1, 0, ctypes.byref(need), ctypes.byref(err)) == _lib.E_FORMAT
    assert err.check == 8 and err.tensor == 0 and need.value == 0
    t, keep = _one()
    t.data = None
    assert L.bpw_trit_write_size(ctypes.byref(t), 1, 0, ctypes.byref(need), ctypes.byref(err)) == _lib.E_INVAL
    assert L.bpw_trit_write_size(None, 1, 0, ctypes.byref(need), ctypes.byref(err)) == _lib.E_INVAL
    assert L.bpw_trit_write_size(None, -1, 0, ctypes.byref(need), ctypes.byref(err)) == _lib.E_INVAL
    assert L.bpw_trit_write_size(None, 0, 16 * 1024 * 1024 + 1, ctypes.byref(need), ctypes.byref(err)) == _lib.E_FORMAT
    assert err.check == 6
