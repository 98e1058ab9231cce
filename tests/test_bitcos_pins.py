"""Pins of the oracle's BITCOS ("BITCOS: Intel's Ternary LLM Weight Format Goes Below 1.58 Bits",
"A bitmap and a sign") to the page and to plain mathematics: a small hand-worked case, an
independent numpy formulation of the flat packer (numpy.packbits), round trips, the n + nnz bit
count and the page's two measured tensors (sizes and bits per weight), and the row form's GEMV
against a dense integer product and the .trit oracle. No GPU."""
import math

import numpy as np
import pytest

import oracle
import synth


def test_hand_worked_case():
    # w = [+1, -1, 0, +1, 0, 0, -1, +1]: nonzero at 0, 1, 3, 6, 7; their signs (1 = -1): 0, 1, 0, 1, 0
    w = np.array([1, -1, 0, 1, 0, 0, -1, 1], np.int8)
    bitmap, signs, nnz = oracle.bitcos_pack_flat(w)
    assert (bitmap, signs, nnz) == (bytes([0b11001011]), bytes([0b01010]), 5)
    presence, words, start = oracle.bitcos_pack_rows(w.reshape(2, 4))
    assert presence.tolist() == [0b1011, 0b1100] and words.tolist() == [0b010, 0b01] and start.tolist() == [0, 1, 2]


@pytest.mark.parametrize("z", (0.0, 0.2966, 0.4219, 0.5148, 0.95, 1.0))
def test_flat_packer_equals_numpy_packbits(z):
    w = synth.trits(int(z * 1e4) + 1, 1, 5003, min(z, 0.9999))[0] if z < 1 else np.zeros(5003, np.int8)
    bitmap, signs, nnz = oracle.bitcos_pack_flat(w)
    assert bitmap == np.packbits(w != 0, bitorder="little").tobytes()
    assert signs == np.packbits(w[w != 0] < 0, bitorder="little").tobytes()
    assert nnz == int(np.count_nonzero(w))
    assert len(bitmap) + len(signs) == math.ceil(w.size / 8) + math.ceil(nnz / 8)
    assert np.array_equal(oracle.bitcos_unpack_flat(bitmap, signs, w.size), w)


def test_unpack_refuses_more_nonzeros_than_sign_bits():
    """A bitmap whose set bits outnumber the sign bits is refused, not read past the signs: 9 set
    presence bits need 2 sign bytes; one byte is short by a bit."""
    w = np.array([1, -1, 1, 1, -1, 1, 1, 1, -1, 0, 0], np.int8)
    bitmap, signs, nnz = oracle.bitcos_pack_flat(w)
    assert nnz == 9 and len(signs) == 2
    assert np.array_equal(oracle.bitcos_unpack_flat(bitmap, signs, w.size), w)
    with pytest.raises(oracle.OracleError) as e:
        oracle.bitcos_unpack_flat(bitmap, signs[:1], w.size)
    assert e.value.code == oracle.E_SIZE
    # eight nonzeros fit exactly in one sign byte
    assert np.array_equal(oracle.bitcos_unpack_flat(bitmap, signs[:1], 8), w[:8])


def test_page_table_sizes():
    """The two tensors of the page's table: n weights at zero density z take ceil(n/8) + ceil(nnz/8)
    bytes, printed as 1.222 MB (1.4917 bits/w) and 3.571 MB (1.6146 bits/w); 2 - z at 0.5148 is
    1.4852 and the break-even against 1.625-bit packing is z = 0.375."""
    for n, z, mb, bits in ((6_553_600, 0.5083, 1.222, 1.4917), (17_694_720, 0.3854, 3.571, 1.6146)):
        nnz = round(n * (1 - z))
        size = math.ceil(n / 8) + math.ceil(nnz / 8)
        assert round(size / 1e6, 3) == mb
        assert round(8 * size / n, 4) == bits
    assert round(2 - 0.5148, 4) == 1.4852
    n = 1 << 20
    assert (math.ceil(n / 8) + math.ceil(0.625 * n / 8)) * 8 / n == 1.625  # z = 0.375 exactly at the line


def test_flat_size_is_two_minus_z_on_synthetic_tensors():
    for z in synth.P_ZERO_SWEEP:
        w = synth.trits(77, 640, 2560, z)
        bitmap, signs, nnz = oracle.bitcos_pack_flat(w)
        zz = 1 - nnz / w.size
        assert abs(8 * (len(bitmap) + len(signs)) / w.size - (2 - zz)) < 1e-5
        assert abs(zz - z) < 0.005


@pytest.mark.parametrize("rows,cols", ((1, 1), (3, 63), (5, 64), (7, 65), (17, 200), (640, 2560), (4, 6912)))
def test_row_form_round_trip_and_gemv(rows, cols):
    w = synth.trits(rows * 31 + cols, rows, cols)
    x, xs = synth.activation(rows + cols, cols)
    presence, words, start = oracle.bitcos_pack_rows(w)
    bpr = (cols + 63) // 64
    # each row's presence and signs are the flat form of that row, word-aligned per row
    for r in range(min(rows, 9)):
        bm, sg, k = oracle.bitcos_pack_flat(w[r])
        pw = np.frombuffer(bm + bytes(-len(bm) % 8), np.uint64)
        assert np.array_equal(presence[r * bpr:(r + 1) * bpr], pw)
        sw = np.frombuffer(sg + bytes(-len(sg) % 4), np.uint32) if k else np.zeros(0, np.uint32)
        assert np.array_equal(words[start[r]:start[r + 1]], sw) and start[r + 1] - start[r] == (k + 31) // 32
    acc, y32, y64 = oracle.bitcos_gemv(presence, words, start, rows, cols, x, xs, 1.25)
    dense = w.astype(np.int64) @ x.astype(np.int64)
    assert np.array_equal(acc, dense)
    acc2, y32b, _ = oracle.gemv(oracle.pack(w), rows, cols, x, xs, 1.25)
    assert np.array_equal(acc, acc2) and np.array_equal(y32.view(np.uint32), y32b.view(np.uint32))
