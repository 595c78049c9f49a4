"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
  * hand-worked blocks (tests/golden/q4_0_blocks.txt), derived by hand from
    the format rule, with their bytes, scales and dequantised values;
  * an exact-rational re-derivation of the quantiser on small random and
    edge-case blocks (IEEE rounding done explicitly on Fractions, no NumPy
    float arithmetic), which checks the oracle's fp32/fp16 semantics;
  * invariants the rule implies: code of the largest element, the round-trip
    bound |x - (q-8) d| <= |d|/2 (plus the fp32 rounding slack derived below);
  * closed forms of the matmul: one-hot and all-ones activations, exact
    rational dot products on tiny shapes;
  * planted mistakes: each plausible slip in the quantiser or the matmul
    must make at least one pin fail.
"""

import math
from fractions import Fraction as Fr

import numpy as np
import pytest

import oracle
import synth
from _golden import load

BLOCKS, GEMVS = load()


# ---------------------------------------------------------------- golden blocks

@pytest.mark.parametrize("blk", BLOCKS, ids=[b.name for b in BLOCKS])
def test_golden_block_bytes(blk):
    packed = oracle.quantize(blk.x[None, :])
    assert packed.shape == (1, 18)
    assert packed.tobytes().hex() == blk.hex
    d, q = oracle.unpack(packed, 1, 32)
    assert int(d.view(np.uint16)[0, 0]) == blk.dbits
    assert q.min() >= 0 and q.max() <= 15


@pytest.mark.parametrize("blk", [b for b in BLOCKS if b.deq is not None],
                         ids=[b.name for b in BLOCKS if b.deq is not None])
def test_golden_block_dequant(blk):
    deq = oracle.dequantize(oracle.quantize(blk.x[None, :]), 1, 32)[0]
    assert np.array_equal(deq, blk.deq)
    assert np.array_equal(np.signbit(deq), np.signbit(blk.deq))


@pytest.mark.parametrize("blk", BLOCKS, ids=[b.name for b in BLOCKS])
def test_golden_block_fp16_input(blk):
    """fp16 weights widen exactly, so fp16-representable blocks give the same bytes."""
    xh = blk.x.astype(np.float16)
    if not np.array_equal(xh.astype(np.float32), blk.x):
        pytest.skip("block is not exactly representable in fp16")
    assert oracle.quantize(xh[None, :]).tobytes().hex() == blk.hex


@pytest.mark.parametrize("case", GEMVS, ids=[g.block for g in GEMVS])
def test_golden_gemv(case):
    blk = next(b for b in BLOCKS if b.name == case.block)
    packed = oracle.quantize(blk.x[None, :])
    y, S = oracle.matmul_ref(np.ones((1, 32), np.float32), packed, 1, 32)
    assert y[0, 0] == case.y and S[0, 0] == case.S


# ------------------------------------------------ exact-rational re-derivation

def _rne(fr: Fr, p: int, emin: int, emax: int):
    """Round a rational to a binary format (p significand bits) to nearest even.

    Returns (negative?, value) with value a Fraction, or float('inf').
    """
    neg = fr < 0
    a = -fr if neg else fr
    if a == 0:
        return neg, Fr(0)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fr(2) ** e > a:
        e -= 1
    while Fr(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fr(2) ** (e - (p - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fr(2) ** (emax + 1):
        return neg, float("inf")
    return neg, r


def _fp16_bits(neg: bool, val: Fr) -> int:
    """IEEE binary16 bits of an exactly representable finite value."""
    if val == 0:
        return 0x8000 if neg else 0
    e = val.numerator.bit_length() - val.denominator.bit_length()
    while Fr(2) ** e > val:
        e -= 1
    while Fr(2) ** (e + 1) <= val:
        e += 1
    if e < -14:  # subnormal
        mant = val / Fr(2) ** -24
        assert mant.denominator == 1
        bits = int(mant)
    else:
        mant = (val / Fr(2) ** e - 1) * 1024
        assert mant.denominator == 1
        bits = ((e + 15) << 10) | int(mant)
    return bits | (0x8000 if neg else 0)


def exact_quantize_block(xs: np.ndarray) -> bytes:
    """The format rule evaluated on exact rationals with explicit IEEE rounding."""
    vals = [Fr(float(v)) for v in xs]
    signs = [bool(np.signbit(v)) for v in xs]
    mags = [abs(v) for v in vals]
    j = mags.index(max(mags))                  # first index of the largest magnitude
    m, m_neg = vals[j], signs[j]
    # fp32 quotient m / -8, then fp16; a zero quotient carries the opposite sign of m
    t_neg, t = _rne(m / -8, 24, -126, 127)
    if m == 0:
        t_neg = not m_neg
    d_neg, d = _rne(-t if t_neg else t, 11, -14, 15)
    if t == 0 or d == 0:
        d_neg = t_neg                          # rounding to zero keeps the sign
    assert d != float("inf")
    D = -d if d_neg else d
    qs = []
    for v in vals:
        if D == 0:
            qs.append(8)
            continue
        u_neg, u = _rne(v / D, 24, -126, 127)
        u = -u if u_neg else u
        v_neg, s = _rne(u + Fr(17, 2), 24, -126, 127)
        s = -s if v_neg else s
        q = int(s) if s >= 0 else -int(-s)     # trunc
        qs.append(min(15, max(0, q)))
    out = _fp16_bits(d_neg, d).to_bytes(2, "little")
    out += bytes(qs[i] | (qs[i + 16] << 4) for i in range(16))
    return out


@pytest.mark.parametrize("blk", BLOCKS, ids=[b.name for b in BLOCKS])
def test_exact_rederivation_matches_golden(blk):
    """The golden bytes themselves follow from the rule in exact arithmetic."""
    assert exact_quantize_block(blk.x).hex() == blk.hex


def test_block_h_reciprocal_would_differ():
    """Block H separates true division from multiply-by-reciprocal."""
    blk = next(b for b in BLOCKS if b.name == "H")
    D = np.array([blk.dbits], np.uint16).view(np.float16)[0].astype(np.float32)
    x1 = blk.x[1]
    assert int(np.trunc(x1 / D + np.float32(8.5))) == 2
    assert int(np.trunc(x1 * (np.float32(1) / D) + np.float32(8.5))) == 3


@pytest.mark.parametrize("kind", ["normal", "outlier", "student_t", "edge"])
def test_oracle_matches_exact_rederivation(kind):
    n, k = 6, 32 * 12
    w = synth.edge_case_weights(5, n, k) if kind == "edge" else synth.random_weights(7, n, k, kind)
    packed = oracle.quantize(w)
    wb = w.reshape(-1, 32)
    pb = packed.reshape(-1, 18)
    for i in range(wb.shape[0]):
        assert pb[i].tobytes() == exact_quantize_block(wb[i]), f"block {i}"


def test_fp16_weights_match_exact_rederivation():
    w = synth.random_weights(11, 4, 256, "student_t").astype(np.float16)
    packed = oracle.quantize(w).reshape(-1, 18)
    wb = w.astype(np.float32).reshape(-1, 32)
    for i in range(wb.shape[0]):
        assert packed[i].tobytes() == exact_quantize_block(wb[i])


# ------------------------------------------------------------------ invariants

def _blocks(w):
    n, k = w.shape
    packed = oracle.quantize(w)
    d, q = oracle.unpack(packed, n, k)
    return w.reshape(-1, 32).astype(np.float64), d.reshape(-1).astype(np.float64), \
        q.reshape(-1, 32).astype(np.int64)


@pytest.mark.parametrize("kind", ["normal", "outlier", "student_t", "edge"])
def test_largest_element_gets_code_zero(kind):
    w = synth.edge_case_weights(1, 64, 512) if kind == "edge" else synth.random_weights(3, 64, 512, kind)
    x, D, q = _blocks(w)
    j = np.argmax(np.abs(x), axis=1)
    normal = np.abs(D) >= 2.0 ** -14
    assert normal.sum() > 0
    assert np.all(q[normal, j[normal]] == 0)
    # and it decodes to -8 d, i.e. m up to the fp16 rounding of d
    m = x[np.arange(len(j)), j]
    assert np.all(np.abs(-8 * D[normal] - m[normal]) <= 8 * np.abs(D[normal]) * 2.0 ** -11)


@pytest.mark.parametrize("kind", ["normal", "outlier", "student_t", "edge"])
def test_round_trip_bound(kind):
    """|x - (q-8) d| <= |d| / 2 for unclamped elements.

    The codes come from fp32 arithmetic: u = fl(x/d) is off by at most
    2^-24 |x/d| <= 2^-24 * 8.004 and fl(u + 8.5) by at most 2^-20, so the exact
    bound is |d| * (1/2 + 1.5e-6); blocks with a subnormal d (relative scale
    error up to 1/2) are outside the bound and only checked for code range.
    """
    w = synth.edge_case_weights(2, 64, 512) if kind == "edge" else synth.random_weights(4, 256, 512, kind)
    x, D, q = _blocks(w)
    normal = np.abs(D) >= 2.0 ** -14
    r = np.divide(x, D[:, None], out=np.zeros_like(x), where=D[:, None] != 0)
    clamped = r >= 7.5 - 1e-5
    ok = normal[:, None] & ~clamped
    err = np.abs(x - (q - 8) * D[:, None])
    bound = np.broadcast_to(np.abs(D)[:, None] * (0.5 + 1.5e-6), err.shape)
    assert ok.sum() > 0
    assert np.all(err[ok] <= bound[ok])
    assert np.all((q >= 0) & (q <= 15))
    # clamped elements sit on the side opposite to m and decode to 7 d
    assert np.all(q[normal[:, None] & (r >= 7.5 + 1e-5)] == 15)


def test_zero_scale_blocks_are_all_eight():
    w = np.zeros((2, 64), np.float32)
    w[1, :32] = -0.0
    w[1, 32:] = 1e-9
    d, q = oracle.unpack(oracle.quantize(w), 2, 64)
    assert np.all(q == 8)
    assert list(d.view(np.uint16).reshape(-1)) == [0x8000, 0x8000, 0x0000, 0x8000]


# ------------------------------------------------------------ matmul closed forms

def test_one_hot_activations_give_weight_columns():
    n = k = 64
    w = synth.random_weights(9, n, k, "student_t")
    packed = oracle.quantize(w)
    deq = oracle.dequantize(packed, n, k)
    for kk in [0, 1, 15, 16, 17, 31, 32, 47, 63]:
        x = np.zeros((1, k), np.float32)
        x[0, kk] = 1.0
        y, S = oracle.matmul_ref(x, packed, n, k)
        assert np.array_equal(y[0], deq[:, kk].astype(np.float64))
        assert np.array_equal(S[0], np.abs(deq[:, kk]).astype(np.float64))


def test_one_hot_selects_the_right_nibble():
    """Element i of a block lives in the low nibble of byte i, element i+16 in its high nibble."""
    blk = next(b for b in BLOCKS if b.name == "A")
    packed = oracle.quantize(blk.x[None, :])
    codes = bytes.fromhex(blk.hex)[2:]
    for i in range(32):
        x = np.zeros((1, 32), np.float32)
        x[0, i] = 1.0
        y, _ = oracle.matmul_ref(x, packed, 1, 32)
        q = codes[i] & 0xF if i < 16 else codes[i - 16] >> 4
        assert y[0, 0] == 2.0 * (q - 8)


def test_all_ones_gives_row_sums():
    n, k = 17, 96
    w = synth.random_weights(10, n, k)
    packed = oracle.quantize(w)
    y, _ = oracle.matmul_ref(np.ones((1, k), np.float16), packed, n, k)
    deq = oracle.dequantize(packed, n, k).astype(np.float64)
    assert np.allclose(y[0], deq.sum(axis=1), rtol=0, atol=1e-15)


@pytest.mark.parametrize("xdt", ["f16", "f32"])
def test_exact_rational_dot_products(xdt):
    m, n, k = 3, 5, 64
    w = synth.random_weights(12, n, k, "outlier")
    x = synth.random_activations(13, m, k, xdt)
    packed = oracle.quantize(w)
    y, S = oracle.matmul_ref(x, packed, n, k)
    # decode bytes directly: byte i -> elements i (low) and i+16 (high)
    raw = packed.reshape(n, k // 32, 18)
    for mi in range(m):
        for ni in range(n):
            acc = Fr(0)
            sacc = Fr(0)
            for b in range(k // 32):
                d = Fr(float(raw[ni, b, :2].view("<f2")[0]))
                for i in range(16):
                    byte = int(raw[ni, b, 2 + i])
                    for e, q in ((i, byte & 0xF), (i + 16, byte >> 4)):
                        term = Fr(float(x[mi, b * 32 + e])) * (q - 8) * d
                        acc += term
                        sacc += abs(term)
            assert abs(Fr(float(y[mi, ni])) - acc) <= Fr(1, 10 ** 12) * max(sacc, Fr(1))
            assert abs(Fr(float(S[mi, ni])) - sacc) <= Fr(1, 10 ** 12) * max(sacc, Fr(1))


def test_cols_subset_equals_full_columns():
    """matmul_ref(..., cols=c) returns the full product's columns c, in the
    order given (unsorted and repeated indices included), for y and S."""
    m, n, k = 4, 37, 96
    w = synth.random_weights(14, n, k, "student_t")
    x = synth.random_activations(15, m, k, "f16")
    packed = oracle.quantize(w)
    y, S = oracle.matmul_ref(x, packed, n, k)
    for cols in ([0], [n - 1, 0, 5], [3, 3, 36, 17], list(range(n))):
        yc, Sc = oracle.matmul_ref(x, packed, n, k, cols=cols)
        assert yc.shape == (m, len(cols))
        assert np.array_equal(yc, y[:, cols]) and np.array_equal(Sc, S[:, cols])


def test_cancellation_case_closed_form():
    """Blocks with one weight +-1.0 (code 0, d = -+0.125) and 31 zeros (code 8):
    y is the sum of the activations at the nonzero weights, signed, exactly
    (every value is dyadic), and S the sum of their magnitudes."""
    n, k = 8, 128
    w = np.zeros((n, k), np.float32)
    for r in range(n):
        w[r, (r % 4)::32] = 1.0 if (r // 4) % 2 == 0 else -1.0
    x = np.full((2, k), 1024.0, np.float32)
    x[:, 0::32] = np.float32(2.0 ** -10)
    x[1, 1::32] = np.float32(-3 * 2.0 ** -10)
    packed = oracle.quantize(w)
    d, q = oracle.unpack(packed, n, k)
    assert set(np.unique(q)) == {0, 8}
    assert set(np.abs(d.astype(np.float32)).ravel()) == {0.125}
    y, S = oracle.matmul_ref(x.astype(np.float16), packed, n, k)
    for r in range(n):
        sgn = 1.0 if (r // 4) % 2 == 0 else -1.0
        for i in range(2):
            col = x[i, (r % 4)::32].astype(np.float64)
            assert y[i, r] == sgn * col.sum()
            assert S[i, r] == np.abs(col).sum()


def test_packed_size_matches_quantized_bytes():
    """n rows of k / 32 blocks of 18 bytes: the byte count quantize produces."""
    for n, k in ((1, 32), (3, 64), (17, 96), (5, 512)):
        w = synth.random_weights(16, n, k)
        assert oracle.packed_size(n, k) == oracle.quantize(w).nbytes == n * (k // 32) * 18
    with pytest.raises(ValueError):
        oracle.packed_size(4, 48)


# ---------------------------------------------------------------- bf16 inputs

def _bf16_by_fields(bits: int) -> float:
    """The value a bfloat16 pattern denotes, decoded field by field (sign, 8-bit
    biased exponent, 7-bit fraction; exponent 0 is subnormal, 255 inf/nan)."""
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return sign * float("inf") if f == 0 else float("nan")
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


@pytest.mark.parametrize("bits,value", [
    (0x3F80, 1.0), (0xC000, -2.0), (0x4049, 3.140625), (0x3E80, 0.25), (0x4480, 1024.0),
    (0x477F, 65280.0), (0x0001, 2.0 ** -133), (0x0080, 2.0 ** -126), (0x7F7F, 255 * 2.0 ** 120),
    (0x0000, 0.0), (0xBF81, -1.0078125)])
def test_bf16_widening_known_values(bits, value):
    v = oracle.widen_bf16(np.array([bits], np.uint16))[0]
    assert v.dtype == np.float32 and float(v) == value


def test_bf16_widening_every_pattern():
    """All 65536 patterns against a field-by-field decoding; -0 keeps its sign."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns
        got = oracle.widen_bf16(bits).astype(np.float64)
    want = np.array([_bf16_by_fields(int(b)) for b in bits])
    finite = np.isfinite(want)
    assert np.array_equal(got[finite], want[finite])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.array_equal(np.isinf(got), np.isinf(want))
    assert np.signbit(oracle.widen_bf16(np.array([0x8000], np.uint16))[0])


def test_exact_rational_dot_products_bf16():
    """bf16 activations: the oracle's sums against exact rational sums of the
    field-decoded activation values and the byte-decoded weights."""
    m, n, k = 2, 4, 64
    w = synth.random_weights(14, n, k, "student_t")
    xb = synth.random_activations(15, m, k, "bf16")
    packed = oracle.quantize(w)
    y, S = oracle.matmul_ref(oracle.widen_bf16(xb), packed, n, k)
    raw = packed.reshape(n, k // 32, 18)
    for mi in range(m):
        for ni in range(n):
            acc = Fr(0)
            for b in range(k // 32):
                d = Fr(float(raw[ni, b, :2].view("<f2")[0]))
                for i in range(16):
                    byte = int(raw[ni, b, 2 + i])
                    for e, q in ((i, byte & 0xF), (i + 16, byte >> 4)):
                        acc += Fr(_bf16_by_fields(int(xb[mi, b * 32 + e]))) * (q - 8) * d
            assert abs(Fr(float(y[mi, ni])) - acc) <= Fr(1, 10 ** 12) * max(abs(acc), Fr(1))


def test_check_bound():
    y = np.array([[1.0, -2.0]])
    S = np.array([[10.0, 1000.0]])
    tol = oracle.tolerance(S)
    assert oracle.check(y + 0.99 * tol, y, S)[0]
    ok, worst, idx = oracle.check(y + np.array([[0.0, 1.01]]) * tol, y, S)
    assert not ok and worst > 1.0 and idx == (0, 1)
    assert not oracle.check(np.array([[np.nan, -2.0]]), y, S)[0]


# ---------------------------------------------------------------- planted slips

def _mutant_quantize(w, slip):
    """The quantiser with one deliberate mistake (slip=None reproduces the oracle)."""
    x = w.astype(np.float32)
    n, k = x.shape
    xb = x.reshape(n, k // 32, 32)
    if slip == "last_index_tie":
        j = 31 - np.argmax(np.abs(xb)[..., ::-1], axis=-1)
    elif slip == "signed_max":
        j = np.argmax(xb, axis=-1)
    else:
        j = np.argmax(np.abs(xb), axis=-1)
    m = np.take_along_axis(xb, j[..., None], axis=-1)[..., 0]
    t = m / np.float32(8.0 if slip == "positive_scale" else -8.0)
    d = t.astype(np.float16)
    D = t if slip == "fp32_scale" else d.astype(np.float32)
    zero = D == 0
    Ds = np.where(zero, np.float32(1), D)[..., None]
    if slip == "reciprocal":
        u = xb * (np.float32(1) / Ds)
    else:
        u = xb / Ds
    if slip == "round_half_even":
        q = np.rint(u + np.float32(8.0))
    else:
        q = np.trunc(u + np.float32(8.5))
    if slip == "wrap_not_clamp":
        q = np.maximum(q, 0).astype(np.int64) & 0xF
    else:
        q = np.minimum(15, np.maximum(0, q)).astype(np.int64)
    q[zero] = 0 if slip == "zero_scale_code0" else 8
    q = q.astype(np.uint8)
    if slip == "nibble_swap":
        codes = (q[..., :16] << 4) | q[..., 16:]
    elif slip == "adjacent_pairs":
        codes = q[..., 0::2] | (q[..., 1::2] << 4)
    else:
        codes = q[..., :16] | (q[..., 16:] << 4)
    dt = ">f2" if slip == "big_endian_scale" else "<f2"
    db = d.astype(dt).view(np.uint8).reshape(n, k // 32, 2)
    return np.concatenate([db, codes.astype(np.uint8)], -1).reshape(n, -1)


SLIPS = ["last_index_tie", "signed_max", "positive_scale", "fp32_scale", "reciprocal",
         "round_half_even", "wrap_not_clamp", "zero_scale_code0", "nibble_swap",
         "adjacent_pairs", "big_endian_scale"]


def test_mutant_harness_is_faithful():
    for b in BLOCKS:
        assert _mutant_quantize(b.x[None, :], None).tobytes().hex() == b.hex
    w = synth.edge_case_weights(3, 8, 384)
    assert np.array_equal(_mutant_quantize(w, None), oracle.quantize(w))


@pytest.mark.parametrize("slip", SLIPS)
def test_golden_blocks_catch_slip(slip):
    fails = [b.name for b in BLOCKS if _mutant_quantize(b.x[None, :], slip).tobytes().hex() != b.hex]
    assert fails, f"no golden block detects slip {slip}"


@pytest.mark.parametrize("slip", ["offset7", "transpose", "drop_last_block", "signed_S"])
def test_matmul_pins_catch_slip(slip):
    """Slips in the matmul reference are caught by the closed forms above."""
    n = k = 64
    w = synth.random_weights(9, n, k, "student_t")
    packed = oracle.quantize(w)
    deq = oracle.dequantize(packed, n, k).astype(np.float64)
    if slip == "offset7":
        d, q = oracle.unpack(packed, n, k)
        deq = ((q.astype(np.float64) - 7).reshape(n, -1, 32) * d.astype(np.float64)[..., None]).reshape(n, k)
    x = np.zeros((1, k))
    x[0, 40] = 1.0
    if slip == "transpose":
        y = x @ deq
    elif slip == "drop_last_block":
        y = x[:, :32] @ deq[:, :32].T
    else:
        y = x @ deq.T
    S = x @ np.abs(deq).T if slip != "signed_S" else x @ deq.T
    good = oracle.dequantize(packed, n, k)[:, 40].astype(np.float64)
    assert not (np.array_equal(y[0], good) and np.array_equal(S[0], np.abs(good)))
