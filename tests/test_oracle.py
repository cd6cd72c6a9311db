"""Pins for the CPU oracle: each test ties the oracle to something other than
itself -- a textbook identity, a library routine, a closed form, the numbers
printed on the SignRot explainer page, or brute force on tiny inputs.

Pages cited: the SignRot abstract (arXiv 2611.16502) and the explainer page
"SignRot for 4-bit LLM quantization -- Sign-adjusted Hadamard rotation"
(paragraphs on the quantizer, on rotation, on the failure mode, on the sign
adjustment, on symmetric vs asymmetric quantizers, and the worked example).
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg

import oracle as O
import signrot_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Hadamard construction
# --------------------------------------------------------------------------


@pytest.mark.parametrize("k", range(1, 10))
def test_sylvester_is_scipy_hadamard(k):
    assert np.array_equal(O.sylvester(k).astype(np.int64), scipy.linalg.hadamard(1 << k))


def test_paley28_is_skew_hadamard():
    h = O.paley28().astype(np.int64)
    assert h.shape == (28, 28)
    assert set(np.unique(h)) == {-1, 1}
    assert np.array_equal(h @ h.T, 28 * np.eye(28, dtype=np.int64))
    # skew type: H + H^T = 2I, so H is not symmetric
    assert np.array_equal(h + h.T, 2 * np.eye(28, dtype=np.int64))
    assert np.all(h[0] == 1)


def test_paley28_fingerprints():
    """The order-28 matrix the library and the oracle both build from Paley's
    construction I over GF(27) = GF(3)[t]/(t^3 + 2t + 1): rows 1 and 2 as sign
    strings, row 0 all +1, and the index-weighted sum of all entries.  A
    relabelling of the field elements, another modulus or a transposed S would
    keep H H^T = 28 I and H + H^T = 2 I but change these."""
    h = O.paley28().astype(np.int64)

    def signs(row):
        return "".join("+" if v > 0 else "-" for v in row)

    assert signs(h[0]) == "+" * 28
    assert signs(h[1]) == "-+-++++----+---+--+++-+-++-+"
    assert signs(h[2]) == "-++-+++-----++--+---++++-++-"
    i, j = np.indices((28, 28))
    assert int((h * (28 * i + j)).sum()) == 756


def test_gf27_field_axioms():
    """The multiplication used for the quadratic character is a field: every
    nonzero element has an inverse and exactly 13 nonzero squares exist."""
    els = O.gf27_elements()
    one = (1, 0, 0)
    nz = [e for e in els if e != (0, 0, 0)]
    for a in nz:
        assert sum(O.signrot_oracle._gf27_mul(a, b) == one for b in nz) == 1
    assert len({O.signrot_oracle._gf27_mul(a, a) for a in nz}) == 13
    # associativity/commutativity on a sample
    rng = np.random.default_rng(0)
    mul = O.signrot_oracle._gf27_mul
    for _ in range(200):
        a, b, c = (els[i] for i in rng.integers(0, 27, 3))
        assert mul(a, b) == mul(b, a)
        assert mul(mul(a, b), c) == mul(a, mul(b, c))


# Outer orders of the general rule (Paley I where m - 1 is a prime power = 3
# mod 4, else Paley II), including the ones common model widths need:
# 12 (24576), 20 (5120), 108 (13824, 27648), 140 (8960), 148 (18944) and 344
# (11008 = 43 * 2^8, where 172 has no Paley construction).
PALEY_M = [12, 20, 36, 44, 52, 60, 68, 76, 84, 100, 108, 124, 132, 140, 148, 164, 180, 344]


@pytest.mark.parametrize("m", PALEY_M)
def test_paley_orders_are_hadamard(m):
    h = O.paley(m).astype(np.int64)
    assert h.shape == (m, m) and set(np.unique(h)) == {-1, 1}
    assert np.array_equal(h @ h.T, m * np.eye(m, dtype=np.int64))
    kind, q = O.paley_kind(m)
    if kind == "I":  # skew type: H + H^T = 2I, first row all +1
        assert q == m - 1
        assert np.array_equal(h + h.T, 2 * np.eye(m, dtype=np.int64))
        assert np.all(h[0] == 1)
    else:  # from a symmetric conference matrix: H is symmetric
        assert q == m // 2 - 1
        assert np.array_equal(h, h.T)


def test_general_paley_reproduces_paley28():
    """The general construction with the lexicographic-first modulus gives the
    hand-written GF(27) matrix (modulus t^3 + 2t + 1) entry for entry."""
    assert O.gf_modulus(3, 3) == [1, 2, 0, 1]
    assert np.array_equal(O.paley(28), O.paley28())


@pytest.mark.parametrize("q", [9, 25, 27, 49, 121, 125, 243, 343])
def test_prime_power_field_axioms(q):
    """GF(q) from the first irreducible modulus is a field: every nonzero
    element has exactly one inverse, (q - 1)/2 nonzero squares, x^(q-1) = 1,
    and the quadratic character is multiplicative (sampled)."""
    f = O.GF(q)
    one = 1
    nz = range(1, q)
    inv = {a: [b for b in nz if f.mul(a, b) == one] for a in nz}
    assert all(len(v) == 1 for v in inv.values())
    chi = f.chi()
    assert int((chi == 1).sum()) == (q - 1) // 2 and chi[0] == 0
    rng = np.random.default_rng(q)
    for a, b in rng.integers(1, q, size=(60, 2)):
        x = 1
        for _ in range(q - 1):
            x = f.mul(x, int(a))
        assert x == 1
        assert chi[f.mul(int(a), int(b))] == chi[a] * chi[b]


def test_outer_factor_rule():
    """n = o 2^v: m = o 2^j for the smallest j >= 2 with a Paley matrix of
    order m <= 512; n = 2^v is pure Sylvester."""
    want = {11008: (344, 5), 13824: (108, 7), 14336: (28, 9), 28672: (28, 10), 3584: (28, 7),
            24576: (12, 11), 18944: (148, 7), 5120: (20, 8), 8960: (140, 6), 27648: (108, 8),
            4096: (1, 12), 2: (1, 1), 12: (12, 0), 344: (344, 0), 28: (28, 0)}
    for n, (m, k) in want.items():
        assert O.factor(n) == (m, k)
        assert m * (1 << k) == n
    # minimality, by brute force over the powers of two
    for n, (m, k) in want.items():
        o = n
        while o % 2 == 0:
            o //= 2
        if o > 1:
            assert all(O.paley_kind(o << j) is None for j in range(2, (m // o).bit_length() - 1))
    for n in (3, 6, 47 * 512, 23 * 4, 43 * 4):  # no construction within the bound
        with pytest.raises(ValueError):
            O.factor(n)


SMALL_N = [2, 4, 8, 16, 32, 64, 128, 28, 56, 112, 224, 448, 12, 24, 40, 36, 72, 344]


@pytest.mark.parametrize("n", SMALL_N)
def test_dense_hadamard_orthogonal(n):
    h = O.hadamard(n).astype(np.int64)
    assert np.array_equal(h @ h.T, n * np.eye(n, dtype=np.int64))


@pytest.mark.parametrize("n", [4096, 8192, 14336, 28672, 11008, 13824, 18944, 24576])
def test_large_hadamard_sampled_rows_orthogonal(n):
    rng = np.random.default_rng(n)
    rows = rng.choice(n, size=12, replace=False)
    r = np.stack([O.hadamard_row(n, int(c)).astype(np.int64) for c in rows])
    assert np.array_equal(r @ r.T, n * np.eye(len(rows), dtype=np.int64))
    # the column-block builder agrees with the row builder (H[i, j] both ways)
    cols = O.hadamard_cols(n, 0, 256)
    for i, c in enumerate(rows):
        assert np.array_equal(cols[c], r[i, :256].astype(np.float64))


@pytest.mark.parametrize("n", [2, 4, 8, 16, 32, 64])
def test_textbook_fwht_equals_dense_product(n):
    x = np.random.default_rng(n).standard_normal((5, n))
    y = O.rotate(x) * math.sqrt(n)
    assert np.allclose(O.fwht_textbook(x), y, rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [28, 56, 112, 24, 40, 216, 344])
def test_kronecker_two_stage_equals_dense(n):
    """x.H for H = H_m (x) H_{2^k} equals: mix the m blocks of 2^k by H_m
    (block a feeds block a' with weight H_m[a, a']), then a textbook FWHT
    inside every block."""
    m, k = O.factor(n)
    x = np.random.default_rng(n).standard_normal((3, n))
    hm = O.outer_matrix(m).astype(np.float64)
    blocks = x.reshape(3, m, 1 << k)
    mixed = np.einsum("tab,ac->tcb", blocks, hm)
    two_stage = O.fwht_textbook(mixed).reshape(3, n) if k else mixed.reshape(3, n)
    assert np.allclose(two_stage, O.rotate(x) * math.sqrt(n), rtol=0, atol=1e-9)


def test_brute_force_n2_n4():
    x = np.array([[3.0, 5.0, -2.0, 7.0]])
    y4 = O.rotate(x) * 2.0
    # by hand: rows of H4 in natural order are ++++, +-+-, ++--, +--+ (symmetric)
    assert np.allclose(y4, [[13.0, -11.0, 3.0, 7.0]])
    y2 = O.rotate(np.array([[1.0, 2.0]]))
    assert np.allclose(y2, [[3 / math.sqrt(2), -1 / math.sqrt(2)]])


def test_row_vector_orientation_is_observable_for_paley():
    """y = x.H uses row c of H for a one-hot input at c; H.x would use column
    c.  For the skew Paley factor these differ, so the convention is pinned."""
    n = 28
    x = np.zeros((1, n))
    x[0, 5] = 1.0
    y = O.rotate(x)[0] * math.sqrt(n)
    h = O.hadamard(n).astype(np.float64)
    assert np.array_equal(y, h[5])
    assert not np.array_equal(y, h[:, 5])


# --------------------------------------------------------------------------
# The pages' closed form and worked example
# --------------------------------------------------------------------------


def test_closed_form_shift_printed_value():
    """Failure-mode paragraph: a lone outlier M contributes +-M/sqrt(n) to every
    output; the page prints 1510/sqrt(11008) as about 14.39."""
    g = _golden("explainer_worked_token.json")
    shift = g["outlier_M"] / math.sqrt(g["n"])
    assert round(shift, 2) == g["shift_M_over_sqrt_n"]


@pytest.mark.parametrize("n,c", [(4096, 1234), (14336, 2090), (28, 3), (8192, 0)])
def test_closed_form_lone_outlier(n, c):
    """x = M e_c -> |y_j| = M/sqrt(n) for every j, with signs = row c of H.
    At n = 4096 and the page's M = 1510 this is exactly 1510/64 = 23.59375."""
    x = np.zeros((1, n))
    x[0, c] = 1510.0
    y = O.rotate(x)[0]
    assert np.allclose(np.abs(y), 1510.0 / math.sqrt(n), rtol=1e-15, atol=0)
    assert np.array_equal(np.sign(y), O.hadamard_row(n, c).astype(np.float64))
    if n == 4096:
        assert np.all(np.abs(y) == 23.59375)
    # the same through bf16: 1510 rounds to 1512 (bf16 spacing is 8 there)
    M = 1512.0
    bits = np.zeros((1, n), dtype=np.uint16)
    bits[0, c] = W.f32_to_bf16_bits(np.array([1510.0], np.float32))[0]
    assert O.bf16_bits_to_f64(bits)[0, c] == M
    # after the SignRot flip the row is the constant sigma*M/sqrt(n) ...
    cal = O.calibrate(bits)
    assert cal["c"] == c and cal["sigma"] == 1
    yd = O.rotate(O.bf16_bits_to_f64(bits), cal["d"])[0]
    assert np.allclose(yd, M / math.sqrt(n), rtol=1e-15, atol=0)
    # ... a degenerate range: s = 1, z = -min, every code 0, and the
    # dequantized row is that constant.
    q, s, z = O.quant_asym(yd[None, :])
    assert s[0] == 1.0 and np.all(q == 0)
    assert np.allclose(O.dequant(q, s, z)[0], yd)


def _page_row(signs):
    """A row whose magnitudes span exactly the page's [13.13, 15.63]."""
    mags = np.array([13.13, 15.63, 13.13, 15.63, 14.0, 14.5, 13.5, 15.0])
    return (mags * np.asarray(signs, np.float64))[None, :]


def test_worked_example_printed_steps():
    """'Worked example': symmetric step 15.63/7 ~ 2.23 (max error ~1.12, only the
    levels at +-13.40 and +-15.63 used, 11 of 15 empty); asymmetric without the
    flip 31.26/15 ~ 2.08; flip + asymmetric 2.50/15 ~ 0.167 (max error ~0.083);
    roughly 13x finer."""
    g = _golden("explainer_worked_token.json")
    plain = _page_row([1, 1, -1, -1, -1, 1, -1, 1])  # both crowds present
    flipped = np.abs(plain)  # the sign adjustment puts every value on one side

    qs, ss = O.quant_sym(plain)
    assert round(ss[0], 2) == g["sym_step"]
    assert round(ss[0] / 2, 2) == g["sym_max_error"]
    used = np.unique(np.abs(qs))
    assert set(used.tolist()) == {6, 7}
    assert sorted(np.round(used * ss[0], 2).tolist()) == g["sym_occupied_level_values"]
    all_levels = set(range(-7, 8))
    assert len(all_levels) == g["sym_levels_total"]
    assert len(all_levels - set(np.unique(qs).tolist())) == g["sym_levels_empty"]
    assert np.max(np.abs(plain - O.dequant_sym(qs, ss))) <= ss[0] / 2 + 1e-12

    qa, sa, za = O.quant_asym(plain)
    assert round(sa[0], 2) == g["asym_noflip_step"]

    qf, sf, zf = O.quant_asym(flipped)
    assert round(sf[0] * 15, 2) == g["signrot_asym_range_width"]
    assert round(sf[0], 3) == g["signrot_asym_step"]
    assert round(sf[0] / 2, 3) == g["signrot_asym_max_error"]
    assert np.max(np.abs(flipped - O.dequant(qf, sf, zf))) <= sf[0] / 2 + 1e-12
    assert round(ss[0] / sf[0]) == g["step_ratio_about"]
    # the flip alone does nothing for the symmetric quantizer
    qs2, ss2 = O.quant_sym(flipped)
    assert ss2[0] == ss[0]


def test_worked_example_replica_at_14336():
    """A synthetic token shaped like the page's: one outlier whose share
    M/sqrt(n) ~ 14.4 dominates Gaussian background; after plain rotation the
    magnitudes form two crowds near +-14.4, after SignRot one crowd."""
    n = 14336
    rng = np.random.default_rng(47)
    x = rng.standard_normal(n) * 0.32
    c = 777
    x[c] = 1720.0
    bits = W.f32_to_bf16_bits(x.astype(np.float32))[None, :]
    xb = O.bf16_bits_to_f64(bits)
    cal = O.calibrate(bits)
    assert cal["c"] == c
    y_plain = O.rotate(xb)
    y_sr = O.rotate(xb, cal["d"])
    lo, hi = np.abs(y_plain).min(), np.abs(y_plain).max()
    assert 12.5 < lo < 13.6 and 15.1 < hi < 16.2  # page: 13.13 .. 15.63
    assert np.all(y_sr > 0)
    _, ss = O.quant_sym(y_plain)
    _, sa, _ = O.quant_asym(y_plain)
    _, sf, _ = O.quant_asym(y_sr)
    assert abs(ss[0] - 2.23) < 0.1
    assert abs(sa[0] - 2.08) < 0.1
    assert 0.12 < sf[0] < 0.22
    assert 9 < ss[0] / sf[0] < 19


# --------------------------------------------------------------------------
# SignRot invariants
# --------------------------------------------------------------------------


@pytest.mark.parametrize("n,c,sigma", [(4096, 1234, 1), (14336, 9999, -1), (28672, 28671, 1), (56, 13, -1)])
def test_flip_makes_outlier_row_constant(n, c, sigma):
    """Sign-adjustment paragraph: after the flip the outlier row of H is all
    one sign, so every output receives the outlier with one sign; D is its own
    inverse."""
    M = sigma * 1024.0
    bits = np.zeros((1, n), dtype=np.uint16)
    bits[0, c] = W.f32_to_bf16_bits(np.array([M], np.float32))[0]
    cal = O.calibrate(bits)
    assert (cal["c"], cal["sigma"]) == (c, sigma)
    d = cal["d"].astype(np.int64)
    row = O.hadamard_row(n, c).astype(np.int64)
    assert np.all(row * d == sigma)  # x_c * H[c, j] * d_j = |x_c| for all j
    assert np.all(d * d == 1)


def test_symmetric_quantizer_ignores_the_flip():
    """Symmetric-vs-asymmetric paragraph: flipping signs keeps every absolute
    value, so the symmetric grid (sized by max |y|) is unchanged and the codes
    flip with the values; the error is identical."""
    bits, _ = W.batch("n4096_t64")
    cal = O.calibrate(bits)
    x = O.bf16_bits_to_f64(bits)
    y = O.rotate(x)
    yd = O.rotate(x, cal["d"])
    assert np.allclose(yd, y * cal["d"][None, :], rtol=0, atol=0)
    q, s = O.quant_sym(y)
    qd, sd = O.quant_sym(yd)
    assert np.array_equal(s, sd)
    assert np.array_equal(qd, (q.astype(np.int64) * cal["d"][None, :]).astype(np.int8))
    assert np.array_equal(O.mse(y, O.dequant_sym(q, s)), O.mse(yd, O.dequant_sym(qd, sd)))


def test_rotation_is_orthogonal_mse_domain():
    x = np.random.default_rng(5).standard_normal((4, 56))
    y = O.rotate(x)
    assert np.allclose((y * y).sum(1), (x * x).sum(1))


# --------------------------------------------------------------------------
# Quantizer, packing, dequantizer
# --------------------------------------------------------------------------


def test_quantizer_nearest_level_brute_force():
    """Quantizer paragraph: 16 levels spread evenly from the token's smallest to
    its largest value, each value snapped to the nearest level."""
    rng = np.random.default_rng(11)
    for trial in range(200):
        n = int(rng.integers(2, 40))
        y = rng.standard_normal((1, n)) * rng.uniform(0.01, 100) + rng.uniform(-50, 50)
        q, s, z = O.quant_asym(y)
        mn, mx = y.min(), y.max()
        levels = mn + np.arange(16) * (mx - mn) / 15
        d = np.abs(y[0][:, None] - levels[None, :])
        best = d.min(axis=1)
        chosen = d[np.arange(n), q[0]]
        assert np.all(chosen <= best + 1e-12)
        assert q[0][np.argmin(y[0])] == 0 and q[0][np.argmax(y[0])] == 15
        assert np.all(q <= 15)
        assert np.allclose(O.dequant(q, s, z)[0], levels[q[0]], rtol=1e-12, atol=1e-12)
        assert np.max(np.abs(y - O.dequant(q, s, z))) <= s[0] / 2 * (1 + 1e-12)


def test_zero_point_is_unrounded_and_may_leave_code_range():
    y = np.array([[100.0, 101.0, 102.5]])
    q, s, z = O.quant_asym(y)
    assert s[0] == pytest.approx(2.5 / 15)
    assert z[0] == pytest.approx(-100.0 / (2.5 / 15))
    assert z[0] < -500  # far outside 0..15: the zero-point is a float


def test_round_half_even_on_exact_ties():
    # range 0..15 with s = 1: values 0.5, 1.5, 2.5 round to 0, 2, 2
    y = np.array([[0.0, 0.5, 1.5, 2.5, 15.0]])
    q, s, _ = O.quant_asym(y)
    assert s[0] == 1.0
    assert q[0].tolist() == [0, 0, 2, 2, 15]


def test_code_position_hand_values():
    """Quantizer paragraph: the position of a value among the 16 levels is
    (y - mn) / s with s = (mx - mn) / 15.  Rows whose positions are exact
    small numbers in either precision."""
    y = np.array([[2.0, 4.0, 32.0, 17.0, 3.0], [-1.0, -1.0, -1.0, -1.0, -1.0]])
    for prec in ("f64", "f32"):
        p = O.code_position(y, prec)
        assert p[0].tolist() == [0.0, 1.0, 15.0, 7.5, 0.5]
        assert p[1].tolist() == [0.0] * 5  # mx == mn: s = 1, every value at level 0


def test_code_position_against_exact_rationals():
    """The float64 position is the exact rational (y - mn) / ((mx - mn) / 15)
    to a few ulps; the binary32 one stays within binary32's error bound
    2^-24 (4 r + 15), r = max|y| / s, and on the planted row it crosses the
    half-integer that the exact position stays below, which is why the two
    precisions pick different codes there."""
    from fractions import Fraction

    rng = np.random.default_rng(17)
    rows = [rng.standard_normal(9) * rng.uniform(0.1, 10) + rng.uniform(-5, 5) for _ in range(40)]
    planted = [-0.5411198139190674, 1.566705346107483, 2.2082173824310303]  # binary32 values
    y = np.zeros((41, 9))
    for i, r in enumerate(rows):
        y[i] = r
    y[40] = planted + [planted[0]] * 6
    y32 = y.astype(np.float32).astype(np.float64)
    p64 = O.code_position(y32, "f64")
    p32 = O.code_position(y32, "f32")
    for i in range(y32.shape[0]):
        mn, mx = Fraction(y32[i].min()), Fraction(y32[i].max())
        s = (mx - mn) / 15
        r = float(max(abs(mn), abs(mx)) / s)
        for j in range(y32.shape[1]):
            exact = (Fraction(y32[i, j]) - mn) / s
            assert abs(p64[i, j] - float(exact)) <= 4 * 2.0 ** -52 * max(1.0, float(exact))
            assert abs(p32[i, j] - float(exact)) <= 2.0 ** -24 * (4 * r + 15)
    exact = (Fraction(planted[1]) - Fraction(planted[0])) / ((Fraction(planted[2]) - Fraction(planted[0])) / 15)
    assert exact < Fraction(23, 2) and p32[40, 1] > 11.5
    q64, _, _ = O.quant_asym(y32[40:], "f64")
    q32, _, _ = O.quant_asym(y32[40:], "f32")
    assert (q64[0, 1], q32[0, 1]) == (11, 12)


def test_mse_hand_values():
    """The error measure is the mean over a token's channels of the squared
    difference, one value per token."""
    assert O.mse(np.array([[1.0, 2.0, 3.0, 4.0]]), np.array([[1.0, 2.0, 3.0, 5.0]])).tolist() == [0.25]
    got = O.mse(np.array([[0.0, 0.0], [3.0, 4.0]]), np.array([[1.0, 1.0], [0.0, 0.0]]))
    assert got.tolist() == [1.0, 12.5]
    # a quantized row: levels 0, 1, ..., 15 (s = 1); 0.25 goes to level 0
    y = np.array([[0.0, 0.25, 15.0]])
    q, s, z = O.quant_asym(y)
    assert q.tolist() == [[0, 0, 15]]
    assert O.mse(y, O.dequant(q, s, z)).tolist() == [0.0625 / 3]


def test_pack_unpack_roundtrip_and_nibble_order():
    q = np.array([[1, 2, 15, 0, 7, 8]], dtype=np.uint8)
    p = O.pack_int4(q)
    assert p.tolist() == [[0x21, 0x0F, 0x87]]
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    assert np.array_equal(O.unpack_int4(O.pack_int4(q)), q)


def test_f32_and_f64_quantizers_agree_away_from_boundaries():
    bits, _ = W.batch("n4096_t64")
    y = O.rotate(O.bf16_bits_to_f64(bits), O.calibrate(bits)["d"])
    q64, s64, z64 = O.quant_asym(y, "f64")
    q32, s32, z32 = O.quant_asym(y, "f32")
    pos = O.code_position(y)
    near = np.abs(pos - np.floor(pos) - 0.5) < 1e-4
    assert np.array_equal(q64[~near], q32[~near])
    assert np.allclose(s32, s64, rtol=1e-6)


# --------------------------------------------------------------------------
# Calibration
# --------------------------------------------------------------------------


def _bits(vals):
    return W.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_calibration_tie_breaks_and_sign():
    # equal |x| in channels 3 and 1 -> channel 1; within channel 1, token 0
    x = np.zeros((3, 8), np.float32)
    x[2, 3] = -8.0
    x[1, 1] = 8.0
    x[2, 1] = -8.0
    r = O.calibrate(_bits(x))
    assert (r["c"], r["t"], r["m_c"], r["sigma"]) == (1, 1, 8.0, 1)
    x[1, 1] = 0.5
    r = O.calibrate(_bits(x))
    assert (r["c"], r["t"], r["m_c"], r["sigma"]) == (1, 2, -8.0, -1)
    # brute force over all (t, j) on random small batches with repeated values
    rng = np.random.default_rng(9)
    for _ in range(100):
        xx = rng.integers(-4, 5, size=(4, 8)).astype(np.float32)
        r = O.calibrate(_bits(xx))
        best = max(itertools.product(range(4), range(8)),
                   key=lambda tj: (abs(xx[tj]), -tj[1], -tj[0]))
        assert (r["t"], r["c"]) == best


def test_calibration_zero_batch_and_negative_zero():
    z = np.zeros((2, 8), np.uint16)
    r = O.calibrate(z)
    assert (r["c"], r["t"], r["sigma"]) == (0, 0, 1)
    z[0, 0] = 0x8000  # -0.0
    assert O.calibrate(z)["sigma"] == 1
    assert np.array_equal(r["d"], O.hadamard_row(8, 0))


@pytest.mark.parametrize("name", ["n4096_t64", "n8192_t2048", "n14336_t4096"])
def test_calibration_recovers_planted_channel(name):
    cal_bits, meta = W.calibration_batch(name)
    r = O.calibrate(cal_bits)
    assert r["c"] == meta["channel"]
    x = O.bf16_bits_to_f64(cal_bits)
    assert r["m_c"] == x[r["t"], r["c"]]
    assert r["sigma"] == (1 if r["m_c"] >= 0 else -1)


# --------------------------------------------------------------------------
# Statistical consequences the pages state
# --------------------------------------------------------------------------


def _codes_used_interval(q_row):
    u = np.unique(q_row)
    return u.max() - u.min() + 1 == len(u)


def test_signrot_collapses_bimodal_tokens():
    """Failure-mode and sign-adjustment paragraphs: a dominating outlier splits a
    plainly rotated token into two crowds with an empty middle; after the flip
    the token is one crowd (one sign, contiguous codes)."""
    bits, meta = W.batch("n14336_t4096", tokens=64)
    cal = O.calibrate(W.calibration_batch("n14336_t4096")[0])
    rows = meta["outlier_tokens"][meta["outlier_tokens"] < 64]
    assert len(rows) >= 5
    x = O.bf16_bits_to_f64(bits[rows])
    y_plain = O.rotate(x)
    y_sr = O.rotate(x, cal["d"])
    q_plain, _, _ = O.quant_asym(y_plain)
    q_sr, _, _ = O.quant_asym(y_sr)
    for i in range(len(rows)):
        assert np.all(np.sign(y_sr[i]) == np.sign(y_sr[i][0]))
        assert _codes_used_interval(q_sr[i])
        assert not _codes_used_interval(q_plain[i])


def test_mse_ordering_on_outlier_and_control_tokens():
    """SignRot+asym beats plain+asym and plain+sym on outlier tokens; on tokens
    without an outlier it is no worse in a statistically meaningful way."""
    bits, meta = W.batch("n14336_t4096", tokens=128)
    cal = O.calibrate(W.calibration_batch("n14336_t4096")[0])
    x = O.bf16_bits_to_f64(bits)
    y_plain = O.rotate(x)
    y_sr = O.rotate(x, cal["d"])

    def asym(y):
        q, s, z = O.quant_asym(y)
        return O.mse(y, O.dequant(q, s, z))

    def sym(y):
        q, s = O.quant_sym(y)
        return O.mse(y, O.dequant_sym(q, s))

    out = np.zeros(len(x), bool)
    out[meta["outlier_tokens"][meta["outlier_tokens"] < len(x)]] = True
    m_sr, m_pa, m_ps = asym(y_sr), asym(y_plain), sym(y_plain)
    assert np.all(m_sr[out] < m_pa[out]) and np.all(m_sr[out] < m_ps[out])
    assert m_sr[~out].mean() < 1.1 * m_pa[~out].mean()


def _mse_grid():
    import json
    import os

    with open(os.path.join(os.path.dirname(__file__), "golden", "mse_grid.json")) as f:
        return json.load(f)


def test_mse_grid_directions():
    """Stored MSE grid (written by tests/golden/make_mse_grid.py from the oracle):
    the flip leaves the symmetric quantizer unchanged on every workload; on
    outlier tokens SignRot + asymmetric INT4 cuts the error of both plain
    quantizers by more than 10x; without an outlier it matches plain + asym."""
    g = _mse_grid()["workloads"]
    assert set(g) == {"n4096_t64", "n8192_t2048", "n14336_t4096", "n28672_t8192", "n14336_control"}
    for name, w in g.items():
        for part in ("outlier", "no_outlier"):
            if part not in w:
                continue
            c = w[part]
            assert c["signrot_sym"] == c["plain_sym"], (name, part)
            if part == "outlier":
                assert c["tokens"] > 0
                assert c["signrot_asym"] * 10 < c["plain_asym"] < c["plain_sym"], (name, c)
            else:
                assert abs(c["signrot_asym"] - c["plain_asym"]) < 0.05 * c["plain_asym"], (name, c)


def test_mse_grid_is_the_oracles():
    """The stored n = 4096 cells are what the oracle computes now."""
    g = _mse_grid()["workloads"]["n4096_t64"]
    bits, meta = W.batch("n4096_t64")
    d = O.calibrate(W.calibration_batch("n4096_t64")[0])["d"]
    x = O.bf16_bits_to_f64(bits)
    y_sr = O.rotate(x, d)
    q, s, z = O.quant_asym(y_sr)
    m = O.mse(y_sr, O.dequant(q, s, z))
    has = np.zeros(len(x), bool)
    has[meta["outlier_tokens"]] = True
    assert g["outlier"]["tokens"] == int(has.sum())
    assert abs(m[has].mean() - g["outlier"]["signrot_asym"]) <= 1e-12 * g["outlier"]["signrot_asym"]
    assert abs(m[~has].mean() - g["no_outlier"]["signrot_asym"]) <= 1e-12 * g["no_outlier"]["signrot_asym"]


@pytest.mark.parametrize("n", [28, 56, 64, 112, 256])
def test_fold_preserves_the_down_projection(n):
    """x . W^T = x' . W'^T exactly (float64 round-off) for the rotated and
    flipped activations x' and the folded weights W', with the calibrated
    sign vector: the fold undoes the activation transform inside the product."""
    g = np.random.default_rng([31, n])
    x_bits = W.f32_to_bf16_bits(g.standard_normal((5, n)).astype(np.float32))
    x_bits[:, n // 3] = W.f32_to_bf16_bits(np.full(5, 900.0, np.float32))
    w_bits = W.f32_to_bf16_bits((g.standard_normal((7, n)) / np.sqrt(n)).astype(np.float32))
    d = O.calibrate(x_bits)["d"]
    x = O.bf16_bits_to_f64(x_bits)
    wt = O.bf16_bits_to_f64(w_bits)
    ref = x @ wt.T
    got = O.rotate(x, d) @ O.fold_weights(w_bits, d).T
    assert np.allclose(got, ref, rtol=0, atol=1e-12 * np.abs(x).max() * np.abs(wt).max() * n)


@pytest.mark.parametrize("n", [28, 64, 14336])
def test_fold_of_unit_rows_is_the_flipped_hadamard_row(n):
    """Folding the unit row e_j gives d (.) H[j, :] / sqrt(n): row j of H, built
    entry by entry from the Kronecker definition."""
    j = (5 * n) // 7
    w = np.zeros((1, n), np.uint16)
    w[0, j] = 0x3F80  # bf16 1.0
    d = np.where(np.arange(n) % 3 == 0, -1, 1).astype(np.int8)
    got = O.fold_weights(w, d)[0]
    want = d.astype(np.float64) * O.hadamard_row(n, j).astype(np.float64) / math.sqrt(n)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# The consumer product (explainer, paragraph on symmetric versus asymmetric
# quantizers: the zero-point's share is the zero-point times a precomputed sum
# of the weights)
# ---------------------------------------------------------------------------


def _nibble(codes, t, j):
    b = int(codes[t, j // 2])
    return (b >> 4) if (j & 1) else (b & 15)


def test_int4_linear_brute_force_on_a_tiny_case():
    """Dequantize-then-multiply equals the sum, written out term by term from
    the nibbles, of scale * (q - zero) * w."""
    g = np.random.default_rng(71)
    t, n, rows = 3, 10, 4
    codes = g.integers(0, 256, size=(t, n // 2), dtype=np.uint8)
    scale = np.array([0.5, 0.03125, 2.0])
    zero = np.array([-3.25, 7.0, 80.5])
    w_bits = W.f32_to_bf16_bits(g.standard_normal((rows, n)).astype(np.float32))
    wv = O.bf16_bits_to_f64(w_bits)
    got = O.int4_linear(codes, scale, zero, w_bits)
    for ti in range(t):
        for k in range(rows):
            want = 0.0
            for j in range(n):
                want += scale[ti] * (_nibble(codes, ti, j) - zero[ti]) * wv[k, j]
            assert abs(got[ti, k] - want) <= 1e-12 * (1 + abs(want))


def test_int4_linear_zero_point_form_is_exact_on_integers():
    """With integer weights, a power-of-two scale and an integer zero-point
    every quantity is an integer times the scale, so the integer-GEMM form
    scale * (q . W^T - zero * rowsum(W)) -- evaluated here in int64 -- equals
    the dequantize-then-multiply definition exactly."""
    g = np.random.default_rng(72)
    t, n, rows = 6, 96, 5
    codes = g.integers(0, 256, size=(t, n // 2), dtype=np.uint8)
    wi = g.integers(-8, 9, size=(rows, n))
    w_bits = W.f32_to_bf16_bits(wi.astype(np.float32))
    scale = np.ldexp(1.0, g.integers(-6, 3, size=t)).astype(np.float64)
    zero = g.integers(-90, 20, size=t).astype(np.float64)
    q = np.empty((t, n), np.int64)
    for ti in range(t):
        for j in range(n):
            q[ti, j] = _nibble(codes, ti, j)
    rowsum = wi.sum(axis=1)
    want = scale[:, None] * (q @ wi.T - zero.astype(np.int64)[:, None] * rowsum[None, :])
    assert np.array_equal(O.int4_linear(codes, scale, zero, w_bits), want)
    assert np.array_equal(O.weight_rowsum(w_bits), rowsum.astype(np.float64))


@pytest.mark.parametrize("n", [28, 512, 14336])
def test_rowsum_of_the_folded_weight_is_one_weight_column(n):
    """With d = sigma * (row c of H), W' . 1 = W . H . d / sqrt(n) =
    sigma * sqrt(n) * W[:, c], because the rows of H are orthogonal with norm
    sqrt(n): the whole sum of a folded weight row is the outlier channel's
    weight."""
    g = np.random.default_rng([73, n])
    c = (3 * n) // 5
    w_bits = W.f32_to_bf16_bits((g.standard_normal((6, n)) / np.sqrt(n)).astype(np.float32))
    for sigma in (1, -1):
        d = (sigma * O.hadamard_row(n, c)).astype(np.int8)
        folded = O.fold_weights(w_bits, d)
        want = sigma * math.sqrt(n) * O.bf16_bits_to_f64(w_bits)[:, c]
        assert np.allclose(folded.sum(axis=1), want, rtol=0, atol=1e-12 * math.sqrt(n))


@pytest.mark.parametrize("n", [28, 1024])
def test_quantized_product_on_the_folded_weight_approximates_the_projection(n):
    """The whole chain -- calibrate, rotate + flip + INT4 on the activations,
    fold + bf16 rounding on the weights, dequantized product -- stays within
    its rigorous error bound of x . W^T:
    |out - x W^T| <= (s/2) sum_j |W'_bf16| + sum_j |y_j| |W'_bf16 - W'|,
    since x W^T = y W'^T exactly and every level is within s/2 of its value."""
    g = np.random.default_rng([74, n])
    x_bits = W.f32_to_bf16_bits(g.standard_normal((9, n)).astype(np.float32))
    x_bits[:, n // 4] = W.f32_to_bf16_bits(np.full(9, 600.0, np.float32))
    w_bits = W.f32_to_bf16_bits((g.standard_normal((11, n)) / np.sqrt(n)).astype(np.float32))
    d = O.calibrate(x_bits)["d"]
    codes, s, z, y = O.rotate_quant_int4(x_bits, d, precision="f64")
    wf = O.fold_weights(w_bits, d)
    wf_bits = W.f32_to_bf16_bits(wf.astype(np.float32))
    wfb = O.bf16_bits_to_f64(wf_bits)
    got = O.int4_linear(codes, s, z, wf_bits)
    ref = O.bf16_bits_to_f64(x_bits) @ O.bf16_bits_to_f64(w_bits).T
    bound = (s[:, None] / 2) * np.abs(wfb).sum(axis=1)[None, :] + np.abs(y) @ np.abs(wfb - wf).T
    assert np.all(np.abs(got - ref) <= bound * (1 + 1e-9) + 1e-12)
    # and the bound is not vacuous: the product keeps most of the signal
    assert np.linalg.norm(got - ref) < 0.2 * np.linalg.norm(ref)


# ---------------------------------------------------------------------------
# Integer zero-point variant (the GyRot abstract on the pages: a rounded
# zero-point that makes dequantization integer arithmetic)
# ---------------------------------------------------------------------------


def test_zint_codes_are_the_nearest_level_of_the_integer_window():
    """Brute force: with the window of levels s*(k - z), k = 0..15, each code
    is the index of the nearest level (ties to the even k), and z is the
    integer nearest to -mn/s."""
    g = np.random.default_rng(81)
    y = np.concatenate([g.normal(0, 1, (6, 20)), 14 + g.random((3, 20)) * 2.5, -30 + g.random((2, 20))])
    q, s, z = O.quant_asym_zint(y, "f64")
    for t in range(y.shape[0]):
        mn = y[t].min()
        assert z[t] == float(round(-mn / s[t]))
        for j in range(y.shape[1]):
            dist = [abs(y[t, j] - s[t] * (k - z[t])) for k in range(16)]
            best = min(range(16), key=lambda k: (dist[k], k % 2))
            assert q[t, j] == best


def test_zint_error_bound_and_integer_dequant():
    """Every value is within s/2 of its level (the rounded zero-point moves the
    window by at most half a step), and q - z is an integer."""
    g = np.random.default_rng(82)
    y = np.concatenate([g.normal(0, 3, (20, 256)), 12 + g.random((20, 256)) * 4])
    q, s, z = O.quant_asym_zint(y, "f64")
    yhat = s[:, None] * (q.astype(np.float64) - z[:, None])
    assert np.all(np.abs(yhat - y) <= s[:, None] / 2 * (1 + 1e-12))
    assert np.all(z == np.rint(z))


def test_zint_equals_the_float_zero_point_quantizer_when_the_zero_is_integral():
    """When -mn/s is already an integer the two quantizers coincide."""
    s = 0.25
    y = np.array([[-2.0, -1.9, 0.1, 0.37, 1.0, 1.75]])
    y[0, -1] = y[0, 0] + 15 * s  # range exactly 15 steps, -mn/s = 8
    qz, sz, zz = O.quant_asym_zint(y, "f64")
    qf, sf, zf = O.quant_asym(y, "f64")
    assert sz[0] == sf[0] == s and zz[0] == zf[0] == 8.0
    assert np.array_equal(qz, qf)


def test_zint_degenerate_row():
    y = np.full((1, 8), 2.3)
    q, s, z = O.quant_asym_zint(y, "f64")
    assert s[0] == 1.0 and z[0] == -2.0 and np.all(q == 0)


# --------------------------------------------------------------------------
# SwiGLU producer of the down-projection input (explainer, paragraph on the
# down-projection: the gated nonlinearity is why the rotation runs online)
# --------------------------------------------------------------------------


def _bf16_value(bits):
    return float(O.bf16_bits_to_f64(np.array([bits], np.uint16))[0])


def test_f64_to_bf16_is_the_nearest_bf16_brute_force():
    """Against the definition: among the bf16 values next to x, the nearest,
    and on an exact tie the one with an even last significand bit."""
    rng = np.random.default_rng(31)
    xs = np.concatenate([rng.standard_normal(300) * 10.0 ** rng.integers(-8, 9, 300), [1.0, -3.5, 0.0]])
    got = O.f64_to_bf16_bits(xs)
    for x, b in zip(xs, got):
        t = int(np.float32(x).view(np.uint32)) >> 16
        cands = []
        for cb in range(t - 2, t + 3):
            cb &= 0xFFFF
            v = _bf16_value(cb)
            if np.isfinite(v) and (v == 0 or np.sign(v) == np.sign(x) or x == 0):
                cands.append((abs(v - x), cb & 1, v, cb))
        cands.sort()
        best = cands[0][0]
        ties = [c for c in cands if c[0] == best]
        want = min(ties, key=lambda c: c[1])[2]
        assert _bf16_value(int(b)) == want, (x, hex(int(b)))


def test_f64_to_bf16_ties_go_to_even():
    """Exact midpoints between neighbouring bf16 values round to the even one."""
    for lo_bits in (0x3F80, 0x3F81, 0x4120, 0xC2F3, 0x0101):
        lo, hi = _bf16_value(lo_bits), _bf16_value(lo_bits + 1)
        mid = (lo + hi) / 2.0
        b = int(O.f64_to_bf16_bits(np.array([mid]))[0])
        assert b in (lo_bits, lo_bits + 1) and (b & 1) == 0, hex(b)
        assert O.bf16_midpoint_distance(np.array([mid]))[0] == 0.0


def test_bf16_midpoint_distance_brute_force():
    rng = np.random.default_rng(37)
    xs = rng.standard_normal(200) * 10.0 ** rng.integers(-5, 6, 200)
    d = O.bf16_midpoint_distance(xs)
    for x, dx in zip(xs, d):
        t = int(np.float32(x).view(np.uint32)) >> 16
        vals = [_bf16_value((t + k) & 0xFFFF) for k in range(-2, 3)]
        mids = [(vals[i] + vals[i + 1]) / 2 for i in range(4)]
        want = min(abs(x - m) for m in mids) / abs(x)
        assert abs(dx - want) <= 1e-12 * max(want, 1e-30) + 1e-18, (x, dx, want)


def test_silu_closed_forms():
    """SiLU(0) = 0; SiLU(z) - SiLU(-z) = z s(z) + z s(-z) = z, because
    s(-z) = 1 - s(z) for the logistic s; SiLU(1) = 1 / (1 + 1/e) =
    0.7310585786300049."""
    assert O.silu(np.array([0.0]))[0] == 0.0
    z = np.linspace(-30, 30, 241)
    assert np.allclose(O.silu(z) - O.silu(-z), z, rtol=1e-15, atol=1e-13)
    assert abs(O.silu(np.array([1.0]))[0] - 0.7310585786300049) < 1e-16
    assert abs(O.silu(np.array([-1.0]))[0] + 0.2689414213699951) < 1e-16
    big = O.silu(np.array([50.0, -50.0]))
    assert big[0] == 50.0 and -1e-19 < big[1] < 0


def test_swiglu_bf16_elementwise():
    """x = bf16(SiLU(gate) * up) element by element, on a tiny hand case and on
    the seeded producer inputs (the outlier channel carries the massive value)."""
    g = W.f32_to_bf16_bits(np.array([[0.0, 1.0, -1.0, 8.0]], np.float32))
    u = W.f32_to_bf16_bits(np.array([[5.0, 2.0, 2.0, 250.0]], np.float32))
    x = O.bf16_bits_to_f64(O.swiglu_bf16(g, u))[0]
    assert x[0] == 0.0
    assert x[1] == _bf16_value(int(O.f64_to_bf16_bits(np.array([2 * 0.7310585786300049]))[0]))
    assert x[2] == _bf16_value(int(O.f64_to_bf16_bits(np.array([-2 * 0.2689414213699951]))[0]))
    assert abs(x[3] - 8.0 / (1 + math.exp(-8.0)) * 250.0) <= 2.0 ** -8 * x[3]
    gate, up, meta = W.swiglu_batch("n14336_t8192", tokens=32)
    xb = O.bf16_bits_to_f64(O.swiglu_bf16(gate, up))
    out = meta["outlier_tokens"]
    assert len(out) > 0
    assert np.all(np.abs(xb[out, meta["channel"]]) >= 700)
    assert np.abs(np.delete(xb, meta["channel"], axis=1)).max() < 100
