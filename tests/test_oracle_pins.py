"""Pins of the CPU oracle to things other than itself (no GPU needed).

Each test fixes the oracle against something the pages or plain mathematics decide:
the worked-example bytes of "The .trit format, version 1" (section 3), numpy's own bit
packing and integer matrix product (library routines), exhaustive brute force on tiny
shapes, closed-form invariants of Equations 2-3 of the Tritium paper's introduction,
the -128 extremes case of its "The hardware core" section, exact rational arithmetic
for the dequantisation, and the byte counts both pages print for BitNet b1.58 2B4T.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from conftest import read_worked_example


# ----------------------------------------------------------------------------- helpers

def np_pack(w: np.ndarray) -> np.ndarray:
    """Independent packer built on numpy.packbits(bitorder='little'): bit k of byte i is element 8i+k."""
    rows, cols = w.shape
    bpr = (cols + 63) // 64
    pad = np.zeros((rows, bpr * 64), dtype=np.int8)
    pad[:, :cols] = w
    pos = np.packbits(pad == 1, axis=1, bitorder="little").reshape(rows, bpr, 8)
    neg = np.packbits(pad == -1, axis=1, bitorder="little").reshape(rows, bpr, 8)
    return np.concatenate([pos, neg], axis=2).reshape(-1)


def dense_acc(w: np.ndarray, x: np.ndarray) -> np.ndarray:
    """The plain definition through numpy's integer matrix product (int64)."""
    return w.astype(np.int64) @ x[: w.shape[1]].astype(np.int64)


def swap_planes(planes: np.ndarray) -> np.ndarray:
    b = planes.reshape(-1, 2, 8)
    return b[:, ::-1, :].reshape(-1).copy()


def all_rows(cols: int) -> np.ndarray:
    return np.array(list(itertools.product((-1, 0, 1), repeat=cols)), dtype=np.int8).reshape(-1, cols)


# ----------------------------------------------------------------------------- worked example

def test_worked_example_payload_bytes():
    rows, cols, scale, w, payload = read_worked_example()
    w = np.array(w, dtype=np.int8)
    planes = oracle.pack(w)
    assert planes.tobytes() == payload
    assert oracle.byte_len(rows, cols) == len(payload) == 32
    oracle.validate(np.frombuffer(payload, np.uint8), rows, cols)
    assert np.array_equal(oracle.unpack(np.frombuffer(payload, np.uint8), rows, cols), w)


def test_worked_example_products():
    rows, cols, scale, w, payload = read_worked_example()
    planes = np.frombuffer(payload, np.uint8)
    for x in ([5, 7, 11], [-128, 127, -1], [0, 0, 0], [1, 1, 1]):
        acc, y32, y64 = oracle.gemv(planes, rows, cols, np.array(x, np.int8), 1.0, scale)
        # W = [[+1, -1, 0], [0, +1, +1]]: row 0 = x0 - x1, row 1 = x1 + x2.
        assert acc.tolist() == [x[0] - x[1], x[1] + x[2]]
        assert y64.tolist() == [0.5 * (x[0] - x[1]), 0.5 * (x[1] + x[2])]


# ----------------------------------------------------------------------------- packing

SHAPES_R = (1, 2, 3, 16, 17)
SHAPES_C = (1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 2560, 6912)


@pytest.mark.parametrize("cols", SHAPES_C)
@pytest.mark.parametrize("rows", SHAPES_R)
def test_pack_roundtrip_and_layout(rows, cols):
    for kind in ("zero", "random"):
        w = np.zeros((rows, cols), np.int8) if kind == "zero" else synth.trits(7 + rows * 100000 + cols, rows, cols)
        planes = oracle.pack(w)
        assert planes.size == rows * ((cols + 63) // 64) * 16
        assert np.array_equal(planes, np_pack(w)), "bit/plane/row order differs from numpy.packbits"
        oracle.validate(planes, rows, cols)
        assert np.array_equal(oracle.unpack(planes, rows, cols), w), "round trip lost or moved a value"
        # no column dropped at a ragged tail: every nonzero is present in the planes
        pl = planes.reshape(rows, -1, 2, 8)
        assert int(np.unpackbits(pl).sum()) == int(np.count_nonzero(w))


def test_tail_mask_widths():
    for c in range(0, 200):
        t = oracle.tail_mask(c)
        r = c % 64
        assert t == ((1 << 64) - 1 if r == 0 else (1 << r) - 1)
        assert bin(t).count("1") == (64 if r == 0 else r)
    for r in (1, 31, 32, 33, 63):  # the remainders a 32-bit shift gets wrong
        assert oracle.tail_mask(64 + r) == (1 << r) - 1


@pytest.mark.parametrize("cols", (1, 31, 32, 33, 63, 64, 65, 100, 127, 128))
def test_padding_bit_rejected_exactly_past_cols(cols):
    rows = 3
    w = synth.trits(99 + cols, rows, cols)
    base = oracle.pack(w)
    bpr = (cols + 63) // 64
    r_valid = cols % 64 or 64
    for plane in (0, 1):
        for k in range(64):
            p = base.copy().reshape(rows, bpr, 2, 8)
            # set bit k of one plane in row 1's last beat and clear it in the other plane,
            # so the only possible violation is a padding bit
            word = int.from_bytes(p[1, bpr - 1, plane].tobytes(), "little")
            other = int.from_bytes(p[1, bpr - 1, 1 - plane].tobytes(), "little")
            word |= 1 << k
            other &= ~(1 << k)
            p[1, bpr - 1, plane] = np.frombuffer(word.to_bytes(8, "little"), np.uint8)
            p[1, bpr - 1, 1 - plane] = np.frombuffer(other.to_bytes(8, "little"), np.uint8)
            flat = p.reshape(-1)
            if k < r_valid:
                oracle.validate(flat, rows, cols)
            else:
                with pytest.raises(oracle.OracleError) as ei:
                    oracle.validate(flat, rows, cols)
                assert ei.value.code == oracle.E_P2
                assert ei.value.row == 1 and ei.value.beat == bpr - 1
                assert ei.value.col == 64 * (bpr - 1) + k


def test_both_bits_rejected_with_position():
    rows, cols = 5, 200
    w = synth.trits(3, rows, cols)
    planes = oracle.pack(w).reshape(rows, 4, 2, 8)
    # set bit 37 of beat 2 of row 3 in both planes, and a later violation in row 4
    for r, b, k in ((4, 0, 1), (3, 2, 37)):
        for plane in (0, 1):
            word = int.from_bytes(planes[r, b, plane].tobytes(), "little") | (1 << k)
            planes[r, b, plane] = np.frombuffer(word.to_bytes(8, "little"), np.uint8)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.validate(planes.reshape(-1), rows, cols)
    assert (ei.value.code, ei.value.row, ei.value.beat, ei.value.col) == (oracle.E_P1, 3, 2, 2 * 64 + 37)
    with pytest.raises(oracle.OracleError):
        oracle.gemv(planes.reshape(-1), rows, cols, np.zeros(cols, np.int8))


def test_p1_reported_before_p2_in_same_beat():
    rows, cols = 1, 10
    planes = np.zeros(16, np.uint8)
    planes[0] = 0b1  # pos bit 0
    planes[8] = 0b1  # neg bit 0 -> P1
    planes[1] = 0b100  # pos bit 10 -> padding (P2)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.validate(planes, rows, cols)
    assert ei.value.code == oracle.E_P1 and ei.value.col == 0


def test_length_and_value_errors():
    with pytest.raises(oracle.OracleError) as ei:
        oracle.validate(np.zeros(31, np.uint8), 2, 3)
    assert ei.value.code == oracle.E_SIZE
    with pytest.raises(oracle.OracleError) as ei:
        oracle.validate(np.zeros(48, np.uint8), 2, 3)
    assert ei.value.code == oracle.E_SIZE
    w = np.zeros((3, 70), np.int8)
    w[2, 66] = 2
    with pytest.raises(oracle.OracleError) as ei:
        oracle.pack(w)
    assert (ei.value.code, ei.value.row, ei.value.beat, ei.value.col) == (oracle.E_INVAL, 2, 1, 66)


# ----------------------------------------------------------------------------- brute force

EXTREME_X = (-128, -1, 0, 1, 127)


@pytest.mark.parametrize("cols", range(1, 9))
def test_exhaustive_rows_against_dense_product(cols):
    """Every ternary row of length cols (3^cols of them, rows are independent) against x vectors."""
    w = all_rows(cols)
    planes = oracle.pack(w)
    if cols <= 4:
        xs = list(itertools.product(EXTREME_X, repeat=cols))
    else:
        rng = np.random.default_rng(cols)
        xs = [tuple(v) for v in rng.integers(-128, 128, size=(60, cols))]
        xs += [tuple([e] * cols) for e in EXTREME_X]
    for x in xs:
        x = np.array(x, np.int8)
        acc, _, _ = oracle.gemv(planes, w.shape[0], cols, x)
        assert np.array_equal(acc, dense_acc(w, x))
        assert np.array_equal(oracle.gemv_bitserial(planes, w.shape[0], cols, x), acc)


def test_random_shapes_against_dense_product():
    rng = np.random.default_rng(1234)
    shapes = [(int(r), int(c)) for r, c in zip(rng.integers(1, 18, 40), rng.integers(1, 201, 40))]
    shapes += [(64, 2560), (33, 6912), (7, 8193)]
    for i, (r, c) in enumerate(shapes):
        z = (0.0, 0.2966, 0.4219, 0.5148, 1.0)[i % 5]
        w = synth.trits(500 + i, r, c, z)
        x = rng.integers(-128, 128, size=c).astype(np.int8)
        planes = oracle.pack(w)
        acc, _, _ = oracle.gemv(planes, r, c, x)
        assert np.array_equal(acc, dense_acc(w, x))
        assert np.array_equal(oracle.gemv_bitserial(planes, r, c, x), acc)


# ----------------------------------------------------------------------------- invariants

def test_invariants():
    rows, cols = 9, 777
    x = synth.activation(42, cols)[0]
    sx = int(x.astype(np.int64).sum())
    zero = oracle.pack(np.zeros((rows, cols), np.int8))
    plus = oracle.pack(np.ones((rows, cols), np.int8))
    minus = oracle.pack(-np.ones((rows, cols), np.int8))
    assert np.all(oracle.gemv(zero, rows, cols, x)[0] == 0)
    assert np.all(oracle.gemv(plus, rows, cols, x)[0] == sx)
    assert np.all(oracle.gemv(minus, rows, cols, x)[0] == -sx)

    w = synth.trits(43, rows, cols)
    planes = oracle.pack(w)
    acc = oracle.gemv(planes, rows, cols, x)[0]
    # swapping the planes negates every row
    assert np.array_equal(oracle.gemv(swap_planes(planes), rows, cols, x)[0], -acc)
    # additivity over disjoint supports
    mask = synth.uniform(44, rows * cols).reshape(rows, cols) < 0.5
    w1 = np.where(mask, w, 0).astype(np.int8)
    w2 = np.where(mask, 0, w).astype(np.int8)
    a1 = oracle.gemv(oracle.pack(w1), rows, cols, x)[0].astype(np.int64)
    a2 = oracle.gemv(oracle.pack(w2), rows, cols, x)[0].astype(np.int64)
    assert np.array_equal(a1 + a2, acc)
    # a joint permutation of columns leaves every row unchanged
    perm = np.argsort(synth.uniform(45, cols))
    assert np.array_equal(oracle.gemv(oracle.pack(w[:, perm].copy()), rows, cols, x[perm].copy())[0], acc)
    # x entries past cols are never read
    xl = np.concatenate([x, np.full(100, 127, np.int8)])
    assert np.array_equal(oracle.gemv(planes, rows, cols, xl)[0], acc)


def test_extremes_minus128():
    """6912 weights of -1 against x = -128 (the widening case the paper's golden set keeps)."""
    cols = 6912
    x = np.full(cols, -128, np.int8)
    w = np.stack([-np.ones(cols, np.int8), np.ones(cols, np.int8), np.zeros(cols, np.int8)])
    acc = oracle.gemv(oracle.pack(w), 3, cols, x)[0]
    assert acc.tolist() == [884736, -884736, 0]
    assert oracle.gemv_bitserial(oracle.pack(w), 3, cols, x).tolist() == [884736, -884736, 0]
    one = oracle.pack(np.array([[-1], [1]], np.int8))
    assert oracle.gemv(one, 2, 1, np.array([-128], np.int8))[0].tolist() == [128, -128]


# ----------------------------------------------------------------------------- dequantisation

def test_dequant_against_exact_rationals():
    rows, cols = 64, 2560
    case = synth.ternary_case(5, 0, 1, rows, cols)
    planes = oracle.pack(case.w)
    acc, y32, y64 = oracle.gemv(planes, rows, cols, case.x, case.x_scale, case.w_scale)
    for a, f32, f64 in zip(acc.tolist(), y32.tolist(), y64.tolist()):
        exact = Fraction(a) * Fraction(case.x_scale) * Fraction(case.w_scale)
        assert f64 == float(exact)  # one rounding of the exact product
        if a == 0:
            assert f32 == 0.0
        else:  # two binary32 roundings: relative error below 2 * 2^-24 (+ second order)
            assert abs(Fraction(f32) - exact) <= Fraction(1, 2 ** 23) * abs(exact) * Fraction(1001, 1000)
    # unit scales give the integer back exactly
    acc1, y1, _ = oracle.gemv(planes, rows, cols, case.x, 1.0, 1.0)
    assert np.array_equal(y1, acc1.astype(np.float32))


# ----------------------------------------------------------------------------- small batch

def test_small_batch_is_per_token_gemv():
    rows, cols = 40, 300
    w = synth.trits(77, rows, cols)
    planes = oracle.pack(w)
    X, sc = synth.small_batch_x(78, 5, cols)
    ldx = cols + 17
    Xl = np.full((5, ldx), -7, np.int8)
    Xl[:, :cols] = X
    acc, y32, y64 = oracle.gemm_small_batch(planes, rows, cols, Xl, sc, 1.25)
    for t in range(5):
        assert np.array_equal(acc[t], dense_acc(w, X[t]))
        a1, f1, d1 = oracle.gemv(planes, rows, cols, X[t], sc[t], 1.25)
        assert np.array_equal(a1, acc[t]) and np.array_equal(f1, y32[t]) and np.array_equal(d1, y64[t])


# ----------------------------------------------------------------------------- dense head

def bf16_to_f64(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_dense_head_one_hot_columns():
    w, _ = synth.head_case(11, rows=300, cols=256)
    for h in (0, 1, 100, 255):
        x = np.zeros(256, np.uint16)
        x[h] = 0x3F80  # 1.0 in bfloat16
        y, s = oracle.dense_head(w, x)
        assert np.array_equal(y, bf16_to_f64(w[:, h]))
        assert np.array_equal(s, np.abs(bf16_to_f64(w[:, h])))


def test_dense_head_against_library_product():
    w, x = synth.head_case(12, rows=1000, cols=2560)
    y, s = oracle.dense_head(w, x)
    wf, xf = bf16_to_f64(w), bf16_to_f64(x)
    ref = wf @ xf
    assert np.all(np.abs(y - ref) <= 1e-12 * np.abs(wf * xf).sum(axis=1) + 1e-300)
    assert np.allclose(s, np.abs(wf * xf).sum(axis=1), rtol=1e-12, atol=0)


# ----------------------------------------------------------------------------- byte accounting

def test_decode_step_byte_accounting():
    """BitNet b1.58 2B4T: 2,084,044,800 trits in 210 tensors (format page section 5; BITCOS
    essay, worked example) and about 521 MB of ternary planes (format page section 2.4)."""
    shapes = synth.decode_step_shapes()
    assert len(shapes) == 210
    assert sum(r * c for _, _, _, r, c in shapes) == 2_084_044_800
    planes = sum(oracle.byte_len(r, c) for _, _, _, r, c in shapes)
    assert planes == 521_011_200 and round(planes / 1e6) == 521
    assert synth.VOCAB * synth.HIDDEN == 328_335_360


def test_dequant_applies_scales_in_turn():
    """The fp32 value is the integer times x_scale, rounded, then times w_scale, rounded (the
    paper's "Why exactness, concretely": the reference multiplies by each scale in turn).
    Each intermediate product is exact in float64 (24-bit by 24-bit significands), so one
    float32 rounding of it is the correctly rounded binary32 result."""
    rows, cols = 256, 2560
    case = synth.ternary_case(6, 0, 3, rows, cols)
    acc, y32, _ = oracle.gemv(oracle.pack(case.w), rows, cols, case.x, case.x_scale, case.w_scale)
    t = (acc.astype(np.float64) * np.float64(np.float32(case.x_scale))).astype(np.float32)
    y = (t.astype(np.float64) * np.float64(np.float32(case.w_scale))).astype(np.float32)
    assert np.array_equal(y32, y)


# ----------------------------------------------------------------------------- activation quantisation
# [TP] "Numerics": Folded mode takes absmax codes from h * g and moves 1/rms into the per-token scale.


def _residual(seed, n, spread=3.0):
    h = synth.normal_f32(seed, n) * np.float32(spread)
    g = (np.float32(0.5) + synth.uniform(seed + 1, n).astype(np.float32))
    return h.astype(np.float32), g.astype(np.float32)


@pytest.mark.parametrize("n", (1, 7, 64, 2560, 6912, 8193))
def test_folded_codes_equal_reference_codes_up_to_ties(n):
    """In exact arithmetic both modes give the same codes (absmax codes are invariant under the
    uniform positive scale 1/rms) and the same scale; in float32 a code may move by one at a tie."""
    total = mismatched = 0
    for seed in range(20):
        h, g = _residual(9000 + 17 * seed + n, n, spread=10.0 ** ((seed % 7) - 3))
        qr, sr = oracle.quantize(h, g, 1e-5, folded=False)
        qf, sf = oracle.quantize(h, g, 1e-5, folded=True)
        d = qr.astype(np.int32) - qf.astype(np.int32)
        assert np.all(np.abs(d) <= 1)
        total += n
        mismatched += int(np.count_nonzero(d))
        assert abs(sr - sf) <= 4e-7 * abs(sf)
    assert mismatched <= max(1, total // 500)


@pytest.mark.parametrize("k", (-12, -3, 1, 5, 20))
def test_quantize_power_of_two_scaling(k):
    """Scaling h by 2^k (eps = 0) changes nothing; scaling g by 2^k scales the Folded scale by 2^k.
    Power-of-two factors commute with every rounding involved, so the equalities are exact."""
    h, g = _residual(77, 2560)
    f = np.float32(2.0 ** k)
    for folded in (False, True):
        q0, s0 = oracle.quantize(h, g, 0.0, folded)
        q1, s1 = oracle.quantize(h * f, g, 0.0, folded)
        assert np.array_equal(q0, q1) and s0 == s1
    q0, s0 = oracle.quantize(h, g, 0.0, True)
    q2, s2 = oracle.quantize(h, g * f, 0.0, True)
    assert np.array_equal(q0, q2) and s2 == np.float32(s0 * f)


def test_quantize_closed_forms():
    n = 2560
    # one non-zero entry: code +-127 there, 0 elsewhere; Folded scale (|c|/127)/(|c|/sqrt(n)) = sqrt(n)/127
    for c in (3.5, -0.25, 1e-3):
        h = np.zeros(n, np.float32)
        h[123] = c
        g = np.ones(n, np.float32)
        q, s = oracle.quantize(h, g, 0.0, True)
        assert q[123] == (127 if c > 0 else -127) and np.count_nonzero(q) == 1
        assert s == np.float32(np.sqrt(n) / 127.0)
    # constant input: every code 127 * sign(c); Folded scale 1/127
    for c in (2.0, -5.0):
        q, s = oracle.quantize(np.full(n, c, np.float32), np.ones(n, np.float32), 0.0, True)
        assert np.all(q == (127 if c > 0 else -127)) and s == np.float32(1.0 / 127.0)
    # a negative gain flips every code; zeros give zero codes and scale
    h, g = _residual(5, n)
    qa, sa = oracle.quantize(h, g, 1e-5, True)
    qb, sb = oracle.quantize(h, -g, 1e-5, True)
    assert np.array_equal(qa, -qb) and sa == sb
    q, s = oracle.quantize(np.zeros(n, np.float32), g, 1e-5, True)
    assert not q.any() and s == 0.0


def test_quantize_eps_inside_the_root_closed_forms():
    """The norm's epsilon sits under the root: rms = sqrt(mean(h^2) + eps). Inputs are chosen so the
    mean square plus eps is an exact square of a dyadic number, which makes the expected scale exact;
    an eps added outside the root (or dropped) gives a different float32 scale in every case.
    Constant h = c, g = 1: every code 127 sign(c), Folded scale (|c| / 127) / sqrt(c^2 + eps).
    One-hot h = c e_k over n: code +-127 at k only, scale (|c| / 127) / sqrt(c^2 / n + eps).
    The Reference mode materialises h / rms and gives the same scale here (rms is exact)."""
    from fractions import Fraction
    cases = [  # (n, one-hot?, c, eps, exact rms)
        (64, False, 0.375, 7 / 64, Fraction(1, 2)),   # 9/64 + 7/64 = 1/4
        (2560, False, -0.75, 0.4375, Fraction(1)),    # 9/16 + 7/16 = 1
        (4, True, 1.0, 0.75, Fraction(1)),            # 1/4 + 3/4 = 1
        (16, True, -2.0, 0.0, Fraction(1, 2)),        # 4/16 + 0 = 1/4
        (256, True, 4.0, 3 / 16, Fraction(1, 2)),     # 16/256 + 3/16 = 1/4
    ]
    for n, onehot, c, eps, rms in cases:
        h = np.zeros(n, np.float32) if onehot else np.full(n, c, np.float32)
        if onehot:
            h[n // 3] = c
        g = np.ones(n, np.float32)
        want = np.float32(float(Fraction(abs(c)) / 127 / rms))
        for folded in (True, False):
            q, s = oracle.quantize(h, g, eps, folded)
            assert s == want, (n, c, eps, folded, s, want)
            if onehot:
                assert q[n // 3] == (127 if c > 0 else -127) and np.count_nonzero(q) == 1
            else:
                assert np.all(q == (127 if c > 0 else -127))
        if eps > 0:  # the closed form separates eps under the root from eps added to the root
            mean_sq = float(Fraction(c) ** 2 / (n if onehot else 1))
            outside = np.float32((abs(c) / 127.0) / (mean_sq ** 0.5 + eps))
            assert outside != want


def test_quantize_non_finite_rule():
    """Reading adopted on both sides: a code whose float32 value is NaN is 0 (a NaN input, or an
    infinite one once the absmax is infinite); NaN never raises the absmax; finite codes are
    unaffected by a NaN elsewhere."""
    n = 64
    h = np.linspace(-1.0, 1.0, n, dtype=np.float32)
    g = np.ones(n, np.float32)
    q0, s0 = oracle.quantize(h, g, 0.0, True)
    hn = h.copy()
    hn[5] = np.nan
    q1, s1 = oracle.quantize(hn, g, 0.0, True)
    assert q1[5] == 0
    keep = np.arange(n) != 5
    assert np.array_equal(q1[keep], q0[keep])  # max |u| is unchanged: the NaN never wins a comparison
    assert np.isnan(s1)                          # the sum of squares carries the NaN into the scale
    hi = h.copy()
    hi[7] = np.inf
    q2, s2 = oracle.quantize(hi, g, 0.0, True)
    assert q2[7] == 0 and not q2[keep & (np.arange(n) != 7)].any()  # finite / inf = 0, inf / inf = NaN -> 0
    gn = g.copy()
    gn[9] = np.nan  # NaN gain, finite h: only that code is affected
    q3, _ = oracle.quantize(h, gn, 0.0, True)
    keep9 = np.arange(n) != 9
    assert q3[9] == 0 and np.array_equal(q3[keep9], q0[keep9])


def test_quantize_codes_against_exact_rationals():
    """Each Folded code is the float32 rounding of 127 u / m; checked against the exact rational
    value: the code is within 1/2 + (float32 error) of it, and equals it at exactly representable
    ratios."""
    from fractions import Fraction
    h, g = _residual(31, 300)
    q, s = oracle.quantize(h, g, 1e-5, True)
    u = [Fraction(float(np.float32(a) * np.float32(b))) for a, b in zip(h, g)]
    m = max(abs(x) for x in u)
    for code, x in zip(q.tolist(), u):
        exact = 127 * x / m
        assert abs(Fraction(code) - exact) <= Fraction(1, 2) + Fraction(1, 1 << 16)


# ----------------------------------------------------------------------------- IntMlp epilogue
# [TP] "Numerics", IntMlp: with gate g = a_g S_g and up u = a_u S_u (uniform positive scales), the
# squared-ReLU stage relu(g)^2 u equals t K for the integer t = relu(a_g)^2 a_u and K = S_g^2 S_u.


def _pair(seed, rows, cols, p_zero=synth.P_ZERO_2B4T):
    wg = synth.trits(seed, rows, cols, p_zero)
    wu = synth.trits(seed + 1, rows, cols, p_zero)
    x, xs = synth.activation(seed + 2, cols)
    return wg, wu, x, xs, synth.weight_scale(seed + 3), synth.weight_scale(seed + 4)


@pytest.mark.parametrize("rows,cols", ((1, 1), (5, 63), (9, 64), (17, 200), (33, 2560), (3, 6912)))
def test_intmlp_equals_squared_relu_of_dequantised_projections(rows, cols):
    """relu(g)^2 * u evaluated in exact rationals from the dequantised projections (dense numpy
    product, relu taken of the real value g) equals t * S_g^2 * S_u exactly; K is the float64
    rounding of S_g^2 * S_u (two roundings: within 2^-52 relative)."""
    wg, wu, x, xs, sg32, su32 = _pair(700 + rows + cols, rows, cols)
    t, k, ag, au = oracle.intmlp(np_pack(wg), np_pack(wu), rows, cols, x, xs, sg32, su32)
    dg, du = dense_acc(wg, x), dense_acc(wu, x)
    assert np.array_equal(ag, dg) and np.array_equal(au, du)
    Sg = Fraction(float(np.float32(xs))) * Fraction(float(np.float32(sg32)))
    Su = Fraction(float(np.float32(xs))) * Fraction(float(np.float32(su32)))
    Kx = Sg * Sg * Su
    for r in range(rows):
        g = int(dg[r]) * Sg
        u = int(du[r]) * Su
        assert max(g, Fraction(0)) ** 2 * u == int(t[r]) * Kx
    assert abs(Fraction(k) - Kx) <= Kx * Fraction(1, 1 << 52)


def test_intmlp_tiny_exhaustive():
    """Every pair of ternary rows over 3 columns, x over {-128, -1, 0, 1, 127}^3, against Python's
    unbounded integers applied to the dense sums."""
    rows = np.array(list(itertools.product((-1, 0, 1), repeat=3)), dtype=np.int8)  # 27 rows
    for xv in itertools.product((-128, -1, 0, 1, 127), repeat=3):
        x = np.array(xv, dtype=np.int8)
        for shift in (0, 5, 11):
            wg = rows
            wu = np.roll(rows, shift, axis=0)
            t, k, _, _ = oracle.intmlp(np_pack(wg), np_pack(wu), 27, 3, x, 1.0, 1.0, 1.0)
            for r in range(27):
                a = sum(int(wg[r, c]) * int(x[c]) for c in range(3))
                b = sum(int(wu[r, c]) * int(x[c]) for c in range(3))
                assert int(t[r]) == (a if a > 0 else 0) * (a if a > 0 else 0) * b
            assert k == 1.0


def test_intmlp_special_cases():
    rows, cols = 40, 2560
    wg, wu, x, xs, sg, su = _pair(91, rows, cols)
    pg, pu = np_pack(wg), np_pack(wu)
    t, k, ag, au = oracle.intmlp(pg, pu, rows, cols, x, xs, sg, su)
    assert np.all(t[ag <= 0] == 0)                       # relu kills non-positive gate rows
    assert np.all(np.sign(t[ag > 0]) == np.sign(au[ag > 0]))
    t2, k2, _, _ = oracle.intmlp(pg, swap_planes(pu), rows, cols, x, xs, sg, su)
    assert np.array_equal(t2, -t) and k2 == k           # negated up weights negate t
    t3, _, a3, _ = oracle.intmlp(pg, pg, rows, cols, x, xs, sg, sg)
    assert np.array_equal(t3, np.where(a3 > 0, a3.astype(np.int64) ** 3, 0))  # gate == up: relu(a)^3
    t4, k4, _, _ = oracle.intmlp(pg, pu, rows, cols, x, xs, np.float32(2 * sg), su)
    assert np.array_equal(t4, t) and k4 == 4 * k        # a power-of-two weight scale only moves K


@pytest.mark.parametrize("cols", (2560, 16383))
def test_intmlp_bound_extremes(cols):
    """x = -128 everywhere, gate all -1 and up all +1: a_g = 128 cols, a_u = -128 cols, the largest
    |t| any pair of this width can give. At 2560 columns |t| < 2^55 (the pages' bound); up to
    16383 columns it still fits int64 exactly."""
    x = np.full(cols, -128, dtype=np.int8)
    wg = np.full((2, cols), -1, dtype=np.int8)
    wu = np.full((2, cols), 1, dtype=np.int8)
    t, _, ag, au = oracle.intmlp(np_pack(wg), np_pack(wu), 2, cols, x, 1.0, 1.0, 1.0)
    want = -((128 * cols) ** 3)
    assert int(ag[0]) == 128 * cols and int(au[0]) == -128 * cols
    assert [int(v) for v in t] == [want, want]
    if cols == 2560:
        assert abs(want) < 2 ** 55


def test_intmlp_range_error_past_int64():
    """At 16384 columns the extreme pair reaches 2^63, which int64 cannot hold: the oracle refuses."""
    cols = 16384
    x = np.full(cols, -128, dtype=np.int8)
    wg = np.full((1, cols), -1, dtype=np.int8)
    wu = np.full((1, cols), -1, dtype=np.int8)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.intmlp(np_pack(wg), np_pack(wu), 1, cols, x, 1.0, 1.0, 1.0)
    assert ei.value.code == oracle.E_RANGE


def test_byte_len_refuses_shapes_whose_count_does_not_fit():
    """(2^60 + 1) beats of 16 bytes is 16 modulo 2^64: a wrapped count would match a 16-byte buffer."""
    rows, cols = 17 * 241 * 61681, 4562284561 * 64
    assert rows * (cols // 64) == 2**60 + 1
    assert oracle.byte_len(rows, cols) == -1 and oracle.byte_len(-1, 64) == -1
    assert oracle.byte_len(2**31 - 1, 64) == (2**31 - 1) * 16
    with pytest.raises(oracle.OracleError) as e:
        oracle.validate(np.zeros(16, np.uint8), rows, cols)
    assert e.value.code == oracle.E_SIZE
