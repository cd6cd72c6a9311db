"""Plain CPU oracle for SignRot's online activation path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it.  It shares no code with the HIP library and imports
nothing from it.

Everything here is written from the definitions, in float64 numpy, slowly and
in the order the method states its steps:

  y = (x . H) / sqrt(n)      rotation by an orthonormal Hadamard matrix
  y <- y (.) d               SignRot's element-wise sign flip
  per token: min, max -> 16 evenly spaced levels -> nearest level -> int4

Sources (pages, cited by title and section):
  [abs]  "SignRot: LLM Quantization with Massive Outlier-Aware Sign-Adjusted
         Rotation" (arXiv 2611.16502), abstract.
  [expl] "SignRot for 4-bit LLM quantization -- Sign-adjusted Hadamard
         rotation" (explainer page): its paragraphs on the 4-bit quantizer,
         on rotation, on the failure mode (the LLaMA2-7B layer-2 token), on
         the down-projection, on the sign adjustment, on symmetric versus
         asymmetric quantizers, and its "Worked example".

Readings where the pages are silent are labelled READING and are collected in
the design notes; the outer Hadamard factors (Paley's constructions I and II
over GF(q), order 28 by construction I over GF(27)) are not on the pages at
all -- the only thing they fix is that the transform is a Hadamard matrix
with entries +-1/sqrt(n).

Parity status: every public function below is pinned by the oracle self-tests
(closed forms, the pages' printed numbers, textbook identities, brute force).
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# bf16 <-> float64 (exact widening; bf16 is the top half of an IEEE binary32)
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen raw bf16 bit patterns (uint16) to float64.  Exact."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 (ties to even mantissa), in
    one rounding step from float64 (no detour through binary32), and return
    the uint16 bit patterns.  For zero and for finite values inside bf16's
    normal range (|x| in [2^-126, 2^128)); anything else is rejected."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(~np.isfinite(x)) or np.any((a != 0) & ((a < 2.0 ** -126) | (a >= 2.0 ** 128))):
        raise ValueError("value outside bf16's normal range")
    f, e = np.frexp(x)  # x = f * 2^e, 0.5 <= |f| < 1: bf16 keeps 8 significant bits
    q = np.rint(f * 256.0)  # round half to even on the 8-bit significand
    r = np.ldexp(q, e - 8)  # exactly representable in bf16 (or 2^128 after a carry: rejected above)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# The producer of the down-projection input  (explainer, paragraph on the
# down-projection: the gated nonlinearity sits between the up/gate
# projections and the down-projection, which is why the rotation there has
# to run online).  READING: the gated unit is SwiGLU, x = SiLU(gate) * up
# with SiLU(z) = z / (1 + e^-z), evaluated in float64 and stored as bf16
# (nearest, ties to even) -- what a bf16 model hands to the down-projection.
# ---------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)), float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_bf16(gate_bits: np.ndarray, up_bits: np.ndarray) -> np.ndarray:
    """x = bf16(SiLU(gate) * up) from bf16 gate and up (bit patterns [T, n]),
    the product taken in float64 and rounded once to bf16.  uint16 bits."""
    return f64_to_bf16_bits(silu(bf16_bits_to_f64(gate_bits)) * bf16_bits_to_f64(up_bits))


def bf16_midpoint_distance(x: np.ndarray) -> np.ndarray:
    """Distance of each float64 value from the nearest point halfway between
    two neighbouring bf16 values, relative to |x| (inf for x == 0): the
    margin by which a rounding to bf16 is decided."""
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    g = np.where(x == 0, 256.0, np.abs(f) * 256.0)  # significand in [128, 256)
    d = np.abs(g - np.floor(g) - 0.5) / g
    return np.where(x == 0, np.inf, d)


# ---------------------------------------------------------------------------
# Hadamard matrices
# ---------------------------------------------------------------------------


def sylvester(k: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order 2^k in natural order (READING):
    H[i, j] = (-1)^popcount(i & j).  int8 entries +-1."""
    idx = np.arange(1 << k, dtype=np.int64)
    par = (np.bitwise_count(idx[:, None] & idx[None, :]) & 1).astype(np.int64)
    return (1 - 2 * par).astype(np.int8)


def _gf27_mul(a, b):
    """Multiply two elements of GF(27) = GF(3)[t] / (t^3 + 2t + 1).
    Elements are coefficient triples (c0, c1, c2) of c0 + c1 t + c2 t^2.
    The modulus gives t^3 = t + 2 (mod 3)."""
    prod = [0] * 5
    for i in range(3):
        for j in range(3):
            prod[i + j] += a[i] * b[j]
    # reduce degrees 4 and 3:  t^d = t^(d-3) * (t + 2)
    for d in (4, 3):
        c = prod[d]
        prod[d] = 0
        prod[d - 2] += c
        prod[d - 3] += 2 * c
    return tuple(v % 3 for v in prod[:3])


def gf27_elements():
    """The 27 field elements in index order e = c0 + 3 c1 + 9 c2."""
    return [(e % 3, (e // 3) % 3, (e // 9) % 3) for e in range(27)]


def paley28() -> np.ndarray:
    """Order-28 Hadamard matrix by Paley's construction I over GF(27) (READING:
    the pages do not name the order-28 factor).

    chi is the quadratic character of GF(27) (chi(0)=0, +1 on the 13 nonzero
    squares, -1 otherwise); Q[i][j] = chi(e_i - e_j) is the Jacobsthal matrix;
    S is Q bordered by a row of +1 and a column of -1 with a 0 corner; and
    H28 = I + S.  Because q = 27 = 3 (mod 4), Q and S are antisymmetric, so
    H28 + H28^T = 2 I: the matrix is NOT symmetric, which makes the choice
    between x.H and H.x observable."""
    els = gf27_elements()
    zero = (0, 0, 0)
    squares = {_gf27_mul(x, x) for x in els if x != zero}

    def chi(a):
        if a == zero:
            return 0
        return 1 if a in squares else -1

    q = np.array(
        [[chi(tuple((ei[t] - ej[t]) % 3 for t in range(3))) for ej in els] for ei in els],
        dtype=np.int64,
    )
    s = np.zeros((28, 28), dtype=np.int64)
    s[0, 1:] = 1
    s[1:, 0] = -1
    s[1:, 1:] = q
    return (np.eye(28, dtype=np.int64) + s).astype(np.int8)


# --- general outer factors (READING: the pages fix no Hadamard order) -------
#
# n = o * 2^v with o odd.  o = 1: the Sylvester matrix of order n.  Otherwise
# H_n = H_m (x) H_{2^k} with m = o * 2^j for the smallest j >= 2 such that a
# Paley matrix of order m exists and m <= MAX_OUTER (k = v - j), Paley I
# preferred over Paley II.  Order 28 (o = 7) is the paley28() matrix above.
# GF(p^e) uses the first monic irreducible polynomial of degree e over GF(p)
# in lexicographic order of its coefficients (a_{e-1}, ..., a_0), and the
# element with base-p digits (c_0, c_1, ...) has index c_0 + c_1 p + ...;
# for GF(27) that is t^3 + 2t + 1, the paley28() modulus.

MAX_OUTER = 512


def _is_prime(p: int) -> bool:
    return p >= 2 and all(p % d for d in range(2, int(math.isqrt(p)) + 1))


def prime_power(q: int):
    """(p, e) with q = p^e, p prime, or None."""
    for p in range(2, q + 1):
        if q % p == 0:
            if not _is_prime(p):
                return None
            e = 0
            while q % p == 0:
                q //= p
                e += 1
            return (p, e) if q == 1 else None
    return None


def _poly_divides(f, g, p):
    """True when monic g divides f over GF(p) (coefficient lists, low first)."""
    r = list(f)
    dg = len(g) - 1
    for d in range(len(r) - 1, dg - 1, -1):
        c = r[d] % p
        if c:
            for t in range(dg + 1):
                r[d - dg + t] = (r[d - dg + t] - c * g[t]) % p
    return all(v % p == 0 for v in r[:dg])


def gf_modulus(p: int, e: int):
    """The first monic irreducible polynomial of degree e over GF(p), as the
    coefficient list [a_0, ..., a_{e-1}, 1] (lexicographic in a_{e-1} .. a_0)."""
    import itertools

    def monic(deg):
        for cs in itertools.product(range(p), repeat=deg):
            yield list(reversed(cs)) + [1]

    for cs in itertools.product(range(p), repeat=e):
        f = list(reversed(cs)) + [1]
        if all(not _poly_divides(f, g, p) for d in range(1, e // 2 + 1) for g in monic(d)):
            return f
    raise ValueError("no irreducible polynomial")


class GF:
    """GF(q), q = p^e: elements are indices 0..q-1 (base-p digits are the
    polynomial coefficients); arithmetic from the definitions."""

    def __init__(self, q: int):
        pe = prime_power(q)
        if pe is None:
            raise ValueError(f"{q} is not a prime power")
        self.q, (self.p, self.e) = q, pe
        self.mod = gf_modulus(self.p, self.e) if self.e > 1 else [0, 1]
        idx = np.arange(q)
        self.digits = np.stack([(idx // self.p**t) % self.p for t in range(self.e)], axis=1)

    def index(self, digits) -> int:
        return int(sum(int(c) * self.p**t for t, c in enumerate(digits)))

    def sub_table(self) -> np.ndarray:
        """sub[i, j] = index of e_i - e_j."""
        d = (self.digits[:, None, :] - self.digits[None, :, :]) % self.p
        w = self.p ** np.arange(self.e)
        return (d * w).sum(axis=2)

    def mul(self, i: int, j: int) -> int:
        a, b = self.digits[i], self.digits[j]
        prod = [0] * (2 * self.e - 1)
        for s_ in range(self.e):
            for t in range(self.e):
                prod[s_ + t] += int(a[s_]) * int(b[t])
        for d in range(len(prod) - 1, self.e - 1, -1):  # t^d = t^(d-e) * (-(a_0 + ... ))
            c = prod[d] % self.p
            prod[d] = 0
            for t in range(self.e):
                prod[d - self.e + t] -= c * self.mod[t]
        return self.index([v % self.p for v in prod[: self.e]])

    def chi(self) -> np.ndarray:
        """Quadratic character by index: 0 at 0, +1 on nonzero squares, else -1."""
        sq = {self.mul(x, x) for x in range(1, self.q)}
        c = np.array([1 if x in sq else -1 for x in range(self.q)], dtype=np.int64)
        c[0] = 0
        return c


def paley_kind(m: int):
    """('I', q) when q = m - 1 is a prime power = 3 (mod 4); else ('II', q) when
    q = m/2 - 1 is a prime power = 1 (mod 4); else None."""
    if m % 4:
        return None
    if m - 1 >= 3 and (m - 1) % 4 == 3 and prime_power(m - 1):
        return ("I", m - 1)
    q = m // 2 - 1
    if q >= 5 and q % 4 == 1 and prime_power(q):
        return ("II", q)
    return None


def _jacobsthal(q: int) -> np.ndarray:
    f = GF(q)
    return f.chi()[f.sub_table()]  # Q[i, j] = chi(e_i - e_j)


def paley(m: int) -> np.ndarray:
    """Hadamard matrix of order m by Paley's constructions (int8 +-1).
    I  (q = m - 1 = 3 mod 4): S = [[0, 1^T], [-1, Q]], H = I + S.
    II (q = m/2 - 1 = 1 mod 4): C = [[0, 1^T], [1, Q]] (symmetric), and
       H = C (x) [[1, 1], [1, -1]] + I (x) [[1, -1], [-1, -1]]."""
    kind = paley_kind(m)
    if kind is None:
        raise ValueError(f"no Paley construction of order {m}")
    t, q = kind
    qm = _jacobsthal(q)
    if t == "I":
        s_ = np.zeros((m, m), dtype=np.int64)
        s_[0, 1:] = 1
        s_[1:, 0] = -1
        s_[1:, 1:] = qm
        return (np.eye(m, dtype=np.int64) + s_).astype(np.int8)
    c = np.zeros((q + 1, q + 1), dtype=np.int64)
    c[0, 1:] = 1
    c[1:, 0] = 1
    c[1:, 1:] = qm
    a = np.array([[1, 1], [1, -1]], dtype=np.int64)
    b = np.array([[1, -1], [-1, -1]], dtype=np.int64)
    return (np.kron(c, a) + np.kron(np.eye(q + 1, dtype=np.int64), b)).astype(np.int8)


_OUTER_CACHE: dict = {}


def outer_matrix(m: int) -> np.ndarray:
    """H_m for the outer factor (paley28() for m = 28)."""
    if m not in _OUTER_CACHE:
        _OUTER_CACHE[m] = paley28() if m == 28 else paley(m)
    return _OUTER_CACHE[m]


def factor(n: int):
    """Split n = m * 2^k: m = 1 for n = 2^k (k >= 1), else the outer order of
    the rule above.  Returns (m, k) or raises."""
    if n < 2:
        raise ValueError(f"unsupported n={n}")
    o, v = n, 0
    while o % 2 == 0:
        o //= 2
        v += 1
    if o == 1:
        return 1, v
    for j in range(2, v + 1):
        m = o << j
        if m > MAX_OUTER:
            break
        if paley_kind(m) is not None:
            return m, v - j
    raise ValueError(f"unsupported n={n}: no Paley outer factor o*2^j <= {MAX_OUTER}")


def hadamard(n: int) -> np.ndarray:
    """Dense H_n (int8 +-1).  For n = m*2^k (m > 1) it is the Kronecker product
    H_m (x) H_{2^k} (READING), so that with i = a*2^k + b and j = a'*2^k + b',
    H[i, j] = H_m[a, a'] * Syl[b, b'].  Use only for small n."""
    m, k = factor(n)
    s = sylvester(k)
    if m == 1:
        return s
    return np.kron(outer_matrix(m).astype(np.int64), s.astype(np.int64)).astype(np.int8)


def hadamard_cols(n: int, j0: int, j1: int) -> np.ndarray:
    """Columns j0..j1-1 of H_n as float64 [n, j1-j0], built entry by entry from
    the Kronecker definition (no n x n matrix is ever formed)."""
    m, k = factor(n)
    i = np.arange(n, dtype=np.int64)
    j = np.arange(j0, j1, dtype=np.int64)
    bmask = (1 << k) - 1
    par = (np.bitwise_count((i[:, None] & bmask) & (j[None, :] & bmask)) & 1).astype(np.int64)
    blk = (1 - 2 * par).astype(np.float64)
    if m > 1:
        hm = outer_matrix(m).astype(np.float64)
        blk *= hm[(i >> k)[:, None], (j >> k)[None, :]]
    return blk


def hadamard_row(n: int, c: int) -> np.ndarray:
    """Row c of H_n as int8 (entry by entry from the Kronecker definition)."""
    m, k = factor(n)
    j = np.arange(n, dtype=np.int64)
    bmask = (1 << k) - 1
    par = (np.bitwise_count((c & bmask) & (j & bmask)) & 1).astype(np.int64)
    row = 1 - 2 * par
    if m > 1:
        row = row * outer_matrix(m).astype(np.int64)[c >> k, j >> k]
    return row.astype(np.int8)


# ---------------------------------------------------------------------------
# Calibration  ([abs]; [expl] paragraph on the sign adjustment)
# ---------------------------------------------------------------------------


def calibrate(x_bits: np.ndarray) -> dict:
    """Find the massive-outlier channel and build the sign vector d.

    The channel is the one holding the largest absolute activation over the
    whole calibration batch ([expl], sign-adjustment paragraph).  READING for
    ties: the smallest channel index wins, then the smallest token index.
    M_c is the signed value at that (token, channel).  d_j multiplies column j
    of H by sign(M_c) * sign(H[c, j]), so that every output receives the
    outlier with one common sign; sign(+-0) is taken as +1.

    x_bits: uint16 bf16 bit patterns, shape [T, n], T >= 1.
    Returns dict(c, t, m_c, sigma, d) with d an int8 [n] vector of +-1.
    """
    x = bf16_bits_to_f64(x_bits)
    if x.ndim != 2 or x.shape[0] < 1:
        raise ValueError("calibration batch must be [T>=1, n]")
    a = np.abs(x)
    top = a.max()
    col_max = a.max(axis=0)
    c = int(np.flatnonzero(col_max == top)[0])
    t = int(np.flatnonzero(a[:, c] == top)[0])
    m_c = float(x[t, c])
    sigma = -1 if m_c < 0 else 1
    n = x.shape[1]
    d = (sigma * hadamard_row(n, c).astype(np.int64)).astype(np.int8)
    return {"c": c, "t": t, "m_c": m_c, "sigma": sigma, "d": d}


# ---------------------------------------------------------------------------
# Rotation  ([expl] rotation paragraph: entries +-1/sqrt(n); sign-adjustment
# paragraph: the flip applies to the columns of H, i.e. to output channels)
# ---------------------------------------------------------------------------


def rotate(x: np.ndarray, d: np.ndarray | None = None, block: int = 1024) -> np.ndarray:
    """Y = (X . H) / sqrt(n), then Y <- Y (.) d (when d is given).

    X is float64 [T, n] (row vectors, READING: y_j = sum_i x_i H[i, j]).  The
    product is evaluated one block of output columns at a time; this is the
    plain matrix product, split only to bound memory."""
    x = np.asarray(x, dtype=np.float64)
    t, n = x.shape
    y = np.empty((t, n), dtype=np.float64)
    for j0 in range(0, n, block):
        j1 = min(n, j0 + block)
        y[:, j0:j1] = x @ hadamard_cols(n, j0, j1)
    y /= math.sqrt(n)
    if d is not None:
        y *= np.asarray(d, dtype=np.float64)[None, :]
    return y


def fold_weights(w_bits: np.ndarray, d: np.ndarray) -> np.ndarray:
    """Offline weight fold (explainer, paragraph on the sign adjustment: the
    matching flip goes into the weights offline).  For out = x . W^T with W
    [rows, n] bf16 bits, W' = W . H . D / sqrt(n): each row w becomes
    (w . H / sqrt(n)) (.) d, so that x . W^T = x' . W'^T with
    x' = (x . H / sqrt(n)) (.) d, because H D / sqrt(n) is orthogonal.
    float64 [rows, n]."""
    return rotate(bf16_bits_to_f64(w_bits), d)


def fwht_textbook(x: np.ndarray) -> np.ndarray:
    """Unnormalised Walsh-Hadamard transform of each row by the iterative
    radix-2 butterfly recursion (natural order).  Used only to cross-check the
    dense product for small n = 2^k."""
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        for s in range(0, n, 2 * h):
            u = y[..., s : s + h].copy()
            v = y[..., s + h : s + 2 * h].copy()
            y[..., s : s + h] = u + v
            y[..., s + h : s + 2 * h] = u - v
        h *= 2
    return y


# ---------------------------------------------------------------------------
# Per-token asymmetric INT4  ([expl] quantizer paragraph: 16 levels spread
# evenly from the token's smallest to its largest value, every value snapped
# to the nearest level; symmetric-vs-asymmetric paragraph: the zero-point)
# ---------------------------------------------------------------------------


def quant_asym(y: np.ndarray, precision: str = "f64"):
    """Per-token asymmetric INT4.

    mn, mx = min and max of the token's values (READING: the range is not
    widened to include 0 -- the worked example's 13.13..15.63 range needs
    that).  s = (mx - mn)/15; a token with mx == mn gets s = 1 (READING).
    z = -mn / s in code units, not rounded and not clamped (READING).
    q = clip(round_half_even((y - mn) / s), 0, 15) (READING: ties to even).

    precision="f32" takes every step in IEEE binary32 (the precision the GPU
    decides codes in); "f64" in binary64.

    Returns (codes uint8 [T, n] with values 0..15, scale [T], zero [T]) as
    float64 arrays for scale and zero.
    """
    dt = {"f64": np.float64, "f32": np.float32}[precision]
    yy = np.asarray(y).astype(dt)
    mn = yy.min(axis=1)
    mx = yy.max(axis=1)
    s = (mx - mn) / dt(15)
    s = np.where(s == 0, dt(1), s).astype(dt)
    z = (-mn / s).astype(dt)
    q = np.rint((yy - mn[:, None]) / s[:, None])
    q = np.clip(q, 0, 15).astype(np.uint8)
    return q, s.astype(np.float64), z.astype(np.float64)


def quant_asym_zint(y: np.ndarray, precision: str = "f64"):
    """Per-token asymmetric INT4 with an integer zero-point (the GyRot
    abstract, a related paper on the pages: the zero-point is rounded so that
    dequantization is integer arithmetic times the scale; READING of the
    formula, which the abstract does not print): s as in quant_asym,
    z = round_half_even(-mn / s), q = clip(round_half_even(y / s) + z, 0, 15).
    Returns (codes uint8 [T, n], scale [T], zero [T]) with integral zero."""
    dt = {"f64": np.float64, "f32": np.float32}[precision]
    yy = np.asarray(y).astype(dt)
    mn = yy.min(axis=1)
    mx = yy.max(axis=1)
    s = (mx - mn) / dt(15)
    s = np.where(s == 0, dt(1), s).astype(dt)
    z = np.rint(-mn / s).astype(dt)
    q = np.clip(np.rint(yy / s[:, None]) + z[:, None], 0, 15).astype(np.uint8)
    return q, s.astype(np.float64), z.astype(np.float64)


def code_position(y: np.ndarray, precision: str = "f64") -> np.ndarray:
    """(y - mn)/s per element, before rounding (used to find elements that sit
    next to a rounding boundary)."""
    dt = {"f64": np.float64, "f32": np.float32}[precision]
    yy = np.asarray(y).astype(dt)
    mn = yy.min(axis=1)
    mx = yy.max(axis=1)
    s = (mx - mn) / dt(15)
    s = np.where(s == 0, dt(1), s).astype(dt)
    return ((yy - mn[:, None]) / s[:, None]).astype(np.float64)


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Two codes per byte: channel 2m in the low nibble, channel 2m+1 in the
    high nibble (READING).  [T, n] -> [T, n/2] uint8."""
    q = np.asarray(q, dtype=np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    p = np.asarray(p, dtype=np.uint8)
    t, h = p.shape
    q = np.empty((t, 2 * h), dtype=np.uint8)
    q[:, 0::2] = p & 0x0F
    q[:, 1::2] = p >> 4
    return q


def dequant(q: np.ndarray, scale: np.ndarray, zero: np.ndarray) -> np.ndarray:
    """Level value of each code: s * (q - z), i.e. mn + q*s."""
    q = np.asarray(q, dtype=np.float64)
    return np.asarray(scale, np.float64)[:, None] * (q - np.asarray(zero, np.float64)[:, None])


# ---------------------------------------------------------------------------
# Symmetric INT4 baseline  ([expl] worked example: levels -7..+7 steps of
# max|y|/7) -- only for the quantization-error comparison
# ---------------------------------------------------------------------------


def quant_sym(y: np.ndarray):
    """Per-token symmetric INT4: s = max|y| / 7 (0 -> 1),
    q = clip(round_half_even(y / s), -8, 7).  Returns (q int8, s float64)."""
    y = np.asarray(y, dtype=np.float64)
    s = np.abs(y).max(axis=1) / 7.0
    s = np.where(s == 0, 1.0, s)
    q = np.clip(np.rint(y / s[:, None]), -8, 7).astype(np.int8)
    return q, s


def dequant_sym(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    return np.asarray(s, np.float64)[:, None] * np.asarray(q, np.float64)


def mse(y: np.ndarray, y_hat: np.ndarray) -> np.ndarray:
    """Mean squared quantization error per token, in the rotated domain (equal
    to the error in the original domain: H/sqrt(n) and D are orthogonal)."""
    diff = np.asarray(y, np.float64) - np.asarray(y_hat, np.float64)
    return (diff * diff).mean(axis=1)


# ---------------------------------------------------------------------------
# The consumer product  ([expl] symmetric-vs-asymmetric paragraph: with an
# asymmetric quantizer the matrix multiply also needs the zero-point times a
# precomputed sum of the weights)
# ---------------------------------------------------------------------------


def weight_rowsum(w_bits: np.ndarray) -> np.ndarray:
    """Sum of each row of a bf16 weight [rows, n] (one row per output
    feature), float64."""
    return bf16_bits_to_f64(w_bits).sum(axis=1)


def int4_linear(codes: np.ndarray, scale: np.ndarray, zero: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """The down-projection on the quantized activations: dequantize every code
    to its level, yhat = scale * (q - zero), then multiply by the folded
    weight, out = yhat . W'^T.  codes packed [T, n/2], W' bf16 bits
    [rows, n] -> float64 [T, rows]."""
    yhat = dequant(unpack_int4(codes), scale, zero)
    return yhat @ bf16_bits_to_f64(w_bits).T


# ---------------------------------------------------------------------------
# The whole online path, end to end
# ---------------------------------------------------------------------------


def rotate_quant_int4(x_bits: np.ndarray, d: np.ndarray, precision: str = "f32"):
    """bf16 bits [T, n] -> (packed codes [T, n/2], scale [T], zero [T], Y [T, n]).
    Y is the float64 rotated-and-flipped activation."""
    y = rotate(bf16_bits_to_f64(x_bits), d)
    q, s, z = quant_asym(y, precision)
    return pack_int4(q), s, z, y
