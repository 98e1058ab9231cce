"""Pins of the oracle's .trit v1 container reader and writer ("The .trit format, version 1") to the
page itself: the complete file printed in section 3, the check list of section 4 (each check fired by
one crafted change, with the page's number), the truncation suite of section 4, and the published
FNV-1a-64 test vectors. No GPU and no libbpw here."""
import math
import os
import random
import struct

import numpy as np
import pytest

import oracle
from conftest import GOLDEN, read_worked_example
from oracle import trit_container as tc


def read_complete_file() -> bytes:
    out = bytearray()
    with open(os.path.join(GOLDEN, "trit_v1_complete_file.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            off, *vals = line.split()
            assert int(off, 16) == len(out)
            out += bytes(int(v, 16) for v in vals)
    return bytes(out)


PAGE = read_complete_file()


def patched(data: bytes, off: int, new: bytes) -> bytes:
    return data[:off] + new + data[off + len(new):]


def sample_file(seed: int = 1, n: int = 6, hashed: bool = True) -> bytes:
    rng = np.random.default_rng(seed)
    tensors = []
    for i in range(n):
        rows, cols = int(rng.integers(1, 6)), int(rng.integers(1, 150))
        w = rng.integers(-1, 2, size=(rows, cols)).astype(np.int8)
        tensors.append((f"layer.{i}.w", tc.TRIT, [rows, cols], 0.25 * (i + 1), oracle.pack(w).tobytes()))
    tensors.append(("norm", tc.F32, [7], 1.0, np.arange(7, dtype=np.float32).tobytes()))
    tensors.append(("head", tc.BF16, [3, 4], 1.0, bytes(24)))
    return tc.write('{"model": "tést"}'.encode(), tensors, with_hash=hashed)


def header_mutations(base: bytes, count: int = 3000, seed: int = 11):
    """Random changes of one to three header bytes (to 0, 1, 0xFF, 0x80, 0x40 or a random value) of a
    valid file, every fifth one also truncated at a random length."""
    start = tc.TritFile(base).payload_start
    rnd = random.Random(seed)
    for k in range(count):
        data = bytearray(base)
        for _ in range(rnd.randint(1, 3)):
            p = rnd.randrange(start)
            data[p] = rnd.choice((0, 1, 0xFF, 0x80, 0x40, rnd.randrange(256)))
        if k % 5 == 0:
            data = data[: rnd.randrange(len(data))]
        yield bytes(data)


def payload_bit_flips(base: bytes, count: int = 300, seed: int = 3):
    """One set bit in the planes of a random ternary tensor of a valid file, per case."""
    g = tc.TritFile(base)
    rnd = random.Random(seed)
    for _ in range(count):
        i = rnd.choice([j for j, t in enumerate(g.tensors) if t.dtype == tc.TRIT])
        t = g.tensors[i]
        o = g.payload_start + t.offset + rnd.randrange(t.byte_len)
        data = bytearray(base)
        data[o] |= 1 << rnd.randrange(8)
        yield bytes(data)


def check_of(data: bytes, verify: bool = False, check_hash: bool = True) -> int:
    try:
        f = tc.TritFile(data)
        if verify:
            f.verify(check_hash)
    except tc.TritError as e:
        return e.check
    return 0


# ----------------------------------------------------------------------------- the page's file

def test_page_file_fields():
    f = tc.TritFile(PAGE)
    assert len(PAGE) == 160 and f.payload_start == 128
    assert f.config == b'{"hidden_size":3}'
    (t,) = f.tensors
    assert (t.name, t.dtype, t.dims, t.scale, t.offset, t.byte_len) == (b"w", tc.TRIT, [2, 3], 0.5, 0, 32)
    rows, cols, scale, w, payload = read_worked_example()
    assert f.payload(0) == payload and (rows, cols, scale) == (2, 3, 0.5)
    assert f.payload(0) == oracle.pack(np.array(w, np.int8)).tobytes()
    f.verify(check_hash=False)


def test_writer_reproduces_page_file_except_hash():
    """The writer lays out header, record, padding and payload exactly as the page prints them; only
    the eight payload_hash bytes differ (the printed value agrees with standard FNV-1a-64 in its low
    40 bits only)."""
    rows, cols, scale, w, payload = read_worked_example()
    out = tc.write(b'{"hidden_size":3}', [("w", tc.TRIT, [2, 3], 0.5, payload)])
    assert len(out) == len(PAGE)
    assert out[:12] == PAGE[:12] and out[20:] == PAGE[20:]
    printed = struct.unpack("<Q", PAGE[12:20])[0]
    ours = tc.fnv1a64(payload)
    assert struct.unpack("<Q", out[12:20])[0] == ours
    assert ours & ((1 << 40) - 1) == printed & ((1 << 40) - 1) and ours != printed


def test_fnv1a64_published_vectors():
    assert tc.fnv1a64(b"") == 0xCBF29CE484222325
    assert tc.fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert tc.fnv1a64(b"foobar") == 0x85944171F73967E8


# ----------------------------------------------------------------------------- checks 1-16
# Offsets in the page's file: version 4, header_flags 8, payload_hash 12, config_len 20, config 24,
# tensor_count 41, record 45: name_len 45, name 47, dtype 48, ndim 49, reserved0 50, reserved1 51,
# dims 52..59, scale 60, flags 64, offset 68, byte_len 76; payload 128.

CHECK_CASES = [
    (0, b"TRIX", 1),
    (4, struct.pack("<I", 0), 2),
    (4, struct.pack("<I", 2), 3),
    (8, struct.pack("<I", 1), 4),
    (20, struct.pack("<I", 16 * 1024 * 1024 + 1), 6),
    (30, b"\xff", 6),
    (41, struct.pack("<I", 1048577), 7),
    (45, struct.pack("<H", 0), 7),
    (45, struct.pack("<H", 1025), 7),
    (47, b"\xff", 7),
    (48, bytes([3]), 8),
    (49, bytes([0]), 8),
    (49, bytes([5]), 8),
    (50, bytes([1]), 8),
    (51, bytes([1]), 8),
    (60, struct.pack("<f", math.nan), 10),
    (60, struct.pack("<f", math.inf), 10),
    (60, struct.pack("<f", 0.0), 10),
    (60, struct.pack("<f", -0.5), 10),
    (64, struct.pack("<I", 1), 8),
    (68, struct.pack("<Q", 32), 11),
    (68, struct.pack("<Q", 64), 12),
    (76, struct.pack("<Q", 48), 15),
]


@pytest.mark.parametrize("off,new,check", CHECK_CASES)
def test_each_check_fires_on_page_file(off, new, check):
    assert check_of(PAGE) == 0
    assert check_of(patched(PAGE, off, new)) == check


def test_checks_needing_other_shapes():
    # 9: shape product overflow (four dims of 2^32 - 1, dense)
    d = tc.write(b"{}", [("a", tc.F32, [2, 2, 2, 2], 1.0, bytes(64))])
    rec = 4 + 4 + 4 + 8 + 4 + 2 + 4 + 2 + 1  # name_len at 30, name "a", dtype at 33
    dims_off = rec + 1 + 1 + 1 + 1 + 1 - 1
    assert d[dims_off - 4:dims_off - 2] == bytes([tc.F32, 4])
    assert check_of(patched(d, dims_off, struct.pack("<IIII", *[0xFFFFFFFF] * 4))) == 9
    # 14: a ternary tensor of three dims
    d = tc.write(b"{}", [("t", tc.TRIT, [1, 2, 64], 1.0, bytes(32))])
    assert check_of(d) == 14
    # 16: dense byte_len that does not match
    d = tc.write(b"{}", [("f", tc.F32, [3], 1.0, bytes(8))])
    assert check_of(d) == 16
    d = tc.write(b"{}", [("h", tc.BF16, [3, 5], 1.0, bytes(30))])
    assert check_of(d) == 0
    # 7: duplicate names
    d = tc.write(b"{}", [("a", tc.F32, [1], 1.0, bytes(4)), ("b", tc.F32, [1], 1.0, bytes(4))])
    i = d.index(b"\x01\x00b")
    assert check_of(patched(d, i + 2, b"a")) == 7
    # 13: two extents overlap
    off_b = i + 3 + 4 + 4 + 4 + 4
    assert struct.unpack("<Q", d[off_b:off_b + 8])[0] == 64
    assert check_of(patched(d, off_b, struct.pack("<Q", 0))) == 13


def test_truncation_suite():
    """Every prefix of the page's file is refused: up to the end of the header region (payload_start)
    as truncated (5), inside the payload as an extent past the end (12)."""
    for n in range(len(PAGE)):
        c = check_of(PAGE[:n])
        assert c == (5 if n < 128 else 12), (n, c)


# ----------------------------------------------------------------------------- checks 17-19

def test_p1_p2_and_hash_on_request():
    rows, cols, scale, w, payload = read_worked_example()
    good = tc.write(b"{}", [("w", tc.TRIT, [2, 3], 0.5, payload), ("g", tc.F32, [3], 1.0, struct.pack("<3f", 1, 2, 3))])
    f = tc.TritFile(good)
    f.verify()
    start = f.payload_start + f.tensors[[t.name for t in f.tensors].index(b"w")].offset
    # P1: row 1, column 2 both +1 and -1 (neg byte 8 of beat 1 gets bit 2)
    bad = patched(good, start + 16 + 8, bytes([0x04]))
    e = pytest.raises(tc.TritError, tc.TritFile(bad).verify, False).value
    assert (e.check, e.row, e.beat, e.col) == (17, 1, 0, 2)
    # P2: row 0, padding column 5 set in the pos plane
    bad = patched(good, start, bytes([0x01 | 0x20]))
    e = pytest.raises(tc.TritError, tc.TritFile(bad).verify, False).value
    assert (e.check, e.row, e.beat, e.col) == (18, 0, 0, 5)
    # 19: one bit of the dense tensor changes; checked only on request and only with a stored hash
    gstart = f.payload_start + f.tensors[[t.name for t in f.tensors].index(b"g")].offset
    bad = patched(good, gstart, bytes([good[gstart] ^ 1]))
    assert check_of(bad, verify=True) == 19
    assert check_of(bad, verify=True, check_hash=False) == 0
    nohash = patched(bad, 12, bytes(8))
    assert check_of(nohash, verify=True) == 0


def test_round_trip_many_tensors():
    rng = np.random.default_rng(5)
    tensors = []
    for i in range(9):
        rows, cols = int(rng.integers(1, 9)), int(rng.integers(1, 200))
        w = rng.integers(-1, 2, size=(rows, cols)).astype(np.int8)
        tensors.append((f"t{i:02d}", tc.TRIT, [rows, cols], float(i + 1) / 4, oracle.pack(w).tobytes()))
    tensors.append(("dense.f32", tc.F32, [3, 7], 1.0, rng.standard_normal(21).astype(np.float32).tobytes()))
    tensors.append(("dense.bf16", tc.BF16, [5], 1.0, bytes(10)))
    data = tc.write(b'{"n": 11}', tensors)
    f = tc.TritFile(data)
    f.verify()
    assert [t.name for t in f.tensors] == sorted(t[0].encode() for t in tensors)
    by = {t[0].encode(): t for t in tensors}
    for i, t in enumerate(f.tensors):
        src = by[t.name]
        assert (t.dtype, t.dims, t.scale) == (src[1], src[2], src[3])
        assert f.payload(i) == src[4] and t.offset % 64 == 0
    assert f.payload_start % 64 == 0
