"""libbpw's .trit v1 container reader (bpw_trit_*) against the oracle's reader, on the host (no GPU):
the same fields on valid files, the same check number (and tensor, and P1/P2 position) on every
crafted change, every truncation and a few thousand random header mutations."""
import struct

import numpy as np
import pytest

import oracle
from oracle import trit_container as tc
from test_trit_container_pins import CHECK_CASES, PAGE, header_mutations, patched, payload_bit_flips, sample_file

bpw = pytest.importorskip("bit_plane_weight_amd")
from bit_plane_weight_amd import _lib  # noqa: E402

CASES = CHECK_CASES


def lib_check(data: bytes, verify: bool = False, check_hash: bool = True):
    """(check, tensor, row, beat, col) of the library; check 0 when the file is accepted."""
    try:
        f = bpw.TritFile(data)
        if verify:
            f.verify(check_hash)
    except bpw.TritFormatError as e:
        return (e.check, e.tensor, e.row, e.beat, e.col)
    return (0, -1, -1, -1, -1)


def oracle_check(data: bytes, verify: bool = False, check_hash: bool = True):
    try:
        f = tc.TritFile(data)
        if verify:
            f.verify(check_hash)
    except tc.TritError as e:
        return (e.check, e.tensor, e.row, e.beat, e.col)
    return (0, -1, -1, -1, -1)


def test_fields_agree_with_oracle():
    for data in (PAGE, sample_file(1), sample_file(2, n=1), tc.write(b"", [])):
        f, g = bpw.TritFile(data), tc.TritFile(data)
        assert len(f) == len(g.tensors) and f.config == g.config and f.stored_hash == g.payload_hash
        for i, (a, b) in enumerate(zip(f.tensors, g.tensors)):
            assert a.name.encode() == b.name and a.dtype == b.dtype and a.dims == b.dims
            assert np.float32(a.scale) == np.float32(b.scale) and a.offset == b.offset and a.byte_len == b.byte_len
            assert a.bytes() == g.payload(i)
            assert f.find(a.name) == i
        assert f.find("no such tensor") == -1


@pytest.mark.parametrize("off,new,check", CASES)
def test_crafted_changes_agree(off, new, check):
    data = patched(PAGE, off, new)
    assert lib_check(data) == oracle_check(data) and lib_check(data)[0] == check


def test_truncation_suite_agrees():
    for data in (PAGE, sample_file(3)):
        for n in range(len(data)):
            assert lib_check(data[:n]) == oracle_check(data[:n]), n
            assert lib_check(data[:n])[0] != 0


def test_random_header_mutations_agree():
    """Random byte changes in the header region (one to three bytes), and random truncations, of a
    multi-tensor file: the library and the oracle accept the same files and report the same check,
    tensor and P1/P2 position; never a crash."""
    seen = set()
    for k, data in enumerate(header_mutations(sample_file(4))):
        a, b = lib_check(data, verify=True), oracle_check(data, verify=True)
        assert a == b, (k, a, b)
        seen.add(a[0])
    assert len(seen) >= 10, seen  # the mutations reach many different checks


def test_verify_positions_agree():
    for k, data in enumerate(payload_bit_flips(sample_file(5, hashed=False))):
        assert lib_check(data, verify=True) == oracle_check(data, verify=True), k


def test_hash_on_request_agrees():
    data = sample_file(6)
    f = bpw.TritFile(data)
    f.verify()
    assert f.stored_hash == tc.fnv1a64(data[tc.TritFile(data).payload_start:])
    bad = bytearray(data)
    bad[-1] ^= 0x10  # inside the last (dense) tensor
    assert lib_check(bytes(bad), verify=True)[0] == 19 == oracle_check(bytes(bad), verify=True)[0]
    assert lib_check(bytes(bad), verify=True, check_hash=False)[0] == 0


def test_fnv1a64_vectors_and_random():
    assert bpw.bpw_fnv1a64(b"") == 0xCBF29CE484222325
    assert bpw.bpw_fnv1a64(b"a") == 0xAF63DC4C8601EC8C
    assert bpw.bpw_fnv1a64(b"foobar") == 0x85944171F73967E8
    rnd = np.random.default_rng(9)
    for n in (1, 7, 64, 1000):
        b = rnd.integers(0, 256, n, dtype=np.uint8).tobytes()
        assert bpw.bpw_fnv1a64(b) == tc.fnv1a64(b)


def test_load_ternary_tensor_matches_planes():
    data = sample_file(7)
    f, g = bpw.TritFile(data), tc.TritFile(data)
    for i, t in enumerate(f.tensors):
        if t.dtype == bpw.TRIT_TERNARY:
            hm = f.load(i)
            assert hm.nbytes == t.byte_len and (hm.rows, hm.cols) == tuple(t.dims)
            hm.free()
        else:
            with pytest.raises(bpw.BpwError) as ei:
                f.load(i)
            assert ei.value.status == _lib.E_INVAL
    # a P1 violation is refused at load time as well (bpw_load validates the copy)
    t = [t for t in g.tensors if t.dtype == tc.TRIT][0]
    i = g.tensors.index(t)
    o = g.payload_start + t.offset
    bad = patched(data, o + 8, bytes([data[o] | 1]))
    bad = patched(bad, o, bytes([data[o] | 1]))
    with pytest.raises(bpw.BpwError) as ei:
        bpw.TritFile(bad).load(i)
    assert ei.value.status == _lib.E_P1_BOTH_BITS
