"""Parity of the HIP path with the oracle at widths n = m * 2^k whose outer
factor H_m is a Paley matrix of an order other than 28 (Paley I for
m - 1 = 11, 19, 43, 107, 139, 343, ...; Paley II for m / 2 - 1 = 5, 9, 13,
49, 73, ...).  Widths with 32 <= n / m <= 256 in the outer-order MFMA
kernel's table (16 <= n / m <= 256) run it; the others run the generic
kernel.  The oracle builds H_m by its own finite-field
arithmetic (numpy), the library by its own (C++).  The last test takes one
width for each remaining shape of the MFMA kernel's table, and the widths
that reach it with Sylvester bits moved into the outer factor.

Tolerances are the ones in parity.py (rotated values within 1e-5 of the
token's max |y|, scale and zero-point within 1e-6, codes bit-exact except at
a rounding boundary).
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import rotation_activation_quantization_amd as R  # noqa: E402
import signrot_workloads as W  # noqa: E402
from parity import compare, expected  # noqa: E402
from test_gpu_zint import compare_zint  # noqa: E402

pytestmark = pytest.mark.gpu

# (n, (m, k)): small orders that still span several outer blocks, and the
# MLP widths of common models (11008, 13824, 18944) plus two-factor widths
WIDTHS = [12, 20, 24, 40, 72, 344, 1000, 2560, 4864, 5120, 5632, 8960, 11008, 13824, 17408, 18944, 24576, 27648]
CHEAP = [n for n in WIDTHS if n <= 8960]
# widths read with Sylvester bits moved into the outer factor (2^k >= 256,
# or a Sylvester width without its own kernel): n -> (outer order, 2^k) the
# MFMA kernel sees
FOLDED = {64: (4, 16), 128: (4, 32), 256: (8, 32), 512: (4, 128), 1024: (8, 128), 2048: (16, 128), 6144: (48, 128),
          10240: (40, 256), 12288: (48, 256), 20480: (160, 128), 24576: (192, 128), 32768: (128, 256),
          # 2^k = 256 read with 128 columns (not where that reading has 3 K chunks: 9216, 11264)
          3072: (24, 128), 5120: (40, 128), 13312: (104, 128), 17408: (136, 128), 21504: (168, 128)}
# the kernel each width runs: (K chunks, column tiles) of the MFMA kernel's table
OUTER_MFMA = {2560: (1, 8), 4864: (3, 4), 5632: (2, 8), 8960: (5, 4), 11008: (11, 2),
              13824: (4, 8), 18944: (5, 8), 27648: (4, 16)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(bits, ld=None):
    t, n = bits.shape
    ld = (n + 7) // 8 * 8 if ld is None else ld
    buf = np.zeros((max(t, 1), ld), np.uint16)
    buf[:t, :n] = bits
    return torch.from_numpy(buf.view(np.int16)).cuda().view(torch.bfloat16)[:t, :n]


def to_np(outs):
    return [o.cpu().numpy() if o is not None else None for o in outs]


def test_widths_use_the_intended_outer_orders_and_kernels():
    for n in WIDTHS:
        m, k = O.factor(n)
        assert m not in (1, 28) and R.outer_order(n) == m, n
        if n in OUTER_MFMA:
            assert OUTER_MFMA[n] == ((m + 31) // 32, (1 << k) // 16), n
            assert R.kernel_name(n) == "rq_outer_mfma", n
        elif n in FOLDED:
            assert R.kernel_name(n) == "rq_outer_mfma", n
            f = R.outer_fold(n)
            assert (m << f, 1 << (k - f)) == FOLDED[n], n
        else:
            assert R.kernel_name(n) == "rq_generic", n


@pytest.mark.parametrize("n", WIDTHS)
def test_calibrate_bit_exact(n):
    bits = W.random_rows(40, n, seed=n + 1, scale=0.9)
    c = (n * 5) // 7
    bits[::3, c] = W.f32_to_bf16_bits(np.array([-1400.0], np.float32))[0]
    say(f"[gpu] paley calibrate n={n} m={R.outer_order(n)}")
    d, c_g, t, mc = R.calibrate(dev(bits))
    ref = O.calibrate(bits)
    assert (c_g, t, mc) == (ref["c"], ref["t"], np.float32(ref["m_c"]))
    assert c_g == c
    assert np.array_equal(d.cpu().numpy(), ref["d"])


@pytest.mark.parametrize("n", WIDTHS)
def test_rotate_quant_matches_oracle(n):
    """37 tokens with a planted outlier in a third of them; d from the
    oracle's calibration (the SignRot form), and for the cheaper widths also a
    random sign vector and d = 1 (plain Hadamard)."""
    t = 37
    bits = W.random_rows(t, n, seed=n, scale=1.0)
    c = (n * 7 // 11) % n
    bits[::3, c] = W.f32_to_bf16_bits(np.array([900.0], np.float32))[0]
    ds = [("signrot-d", O.calibrate(bits)["d"])]
    if n in CHEAP:
        g = np.random.default_rng([7, n])
        ds.append(("random-d", np.where(g.random(n) < 0.5, -1, 1).astype(np.int8)))
        ds.append(("plain-hadamard", np.ones(n, np.int8)))
    x = dev(bits)
    for label, d in ds:
        say(f"[gpu] paley rotate n={n} m={R.outer_order(n)} {label}")
        codes, scale, zero, y = to_np(R.rotate_quant_int4(x, torch.from_numpy(d).cuda(), y_out=True))
        st = compare(expected(bits, d), codes, scale, zero, y, label=f"n={n} {label}")
        say(f"[gpu] paley rotate n={n} {label}: {st}")


@pytest.mark.parametrize("n", [12, 40, 344, 1000, 2560, 4864, 5120, 5632, 8960, 11008, 13824, 17408, 18944, 27648])
def test_outlier_form_matches_vector_form(n):
    """(c, sigma) against the explicit vector sigma * H[c, .] for channels in
    the first, a middle and the last outer block, bit for bit; the first pair
    also against the oracle."""
    m, k = O.factor(n)
    B = 1 << k
    picks = [(0, 1), ((m // 2) * B + B // 3, -1), (n - 1, -1), ((m - 2) * B, 1)]
    for i, (c, sigma) in enumerate(picks):
        bits = W.random_rows(19, n, seed=c + 3, scale=0.8)
        bits[:, c] = W.f32_to_bf16_bits(np.array([1100.0 * sigma], np.float32))[0]
        d = (sigma * O.hadamard_row(n, c)).astype(np.int8)
        say(f"[gpu] paley outlier form n={n} c={c} sigma={sigma}")
        x = dev(bits)
        a = to_np(R.rotate_quant_int4_outlier(x, c, sigma, y_out=True))
        b = to_np(R.rotate_quant_int4(x, torch.from_numpy(d).cuda(), y_out=True))
        for u, v, name in zip(a, b, ("codes", "scale", "zero", "y")):
            assert np.array_equal(u, v), (name, c)
        if i == 0:
            compare(expected(bits, d), a[0], a[1], a[2], a[3], label=f"outlier n={n} c={c}")


@pytest.mark.parametrize("n", [24, 344, 2560, 4864, 5120, 5632, 8960, 11008, 13824, 17408, 18944, 27648])
def test_zint_matches_oracle(n):
    g = np.random.default_rng([84, n])
    c, sigma = int(g.integers(n)), -1
    bits = W.random_rows(33, n, seed=c, scale=0.7, outlier=1300.0 * sigma)
    bits[::4, c] = W.f32_to_bf16_bits(np.array([0.3], np.float32))[0]
    d = (sigma * O.hadamard_row(n, c)).astype(np.int8)
    say(f"[gpu] paley zint n={n} c={c}")
    codes, scale, zero = to_np(R.rotate_quant_int4_zint(dev(bits), c, sigma))
    y = O.rotate(O.bf16_bits_to_f64(bits), d)
    compare_zint(y, codes, scale, zero, f"paley zint n={n}")


@pytest.mark.parametrize("n", [40, 1000, 2048, 5120, 11008, 13824, 24576])
def test_fold_weights_matches_oracle(n):
    g = np.random.default_rng([42, n])
    rows = 33
    w_bits = W.f32_to_bf16_bits((g.standard_normal((rows, n)) / np.sqrt(n)).astype(np.float32))
    d = O.calibrate(W.random_rows(16, n, seed=5, scale=0.7, outlier=1300.0))["d"]
    say(f"[gpu] paley fold n={n}")
    wf = R.fold_weights(dev(w_bits), torch.from_numpy(d).cuda()).cpu().numpy()
    ref = O.fold_weights(w_bits, d)
    err = np.abs(wf - ref).max(axis=1) / np.abs(ref).max(axis=1)
    assert err.max() <= 1e-5


@pytest.mark.parametrize("n", [12, 344, 5120, 11008, 13824, 27648])
def test_degenerate_rows(n):
    c = n // 3
    rows = np.zeros((5, n), np.uint16)
    rows[1, :] = W.f32_to_bf16_bits(np.full(n, 2.5, np.float32))
    rows[2, c] = W.f32_to_bf16_bits(np.array([1512.0], np.float32))[0]
    rows[3, ::2] = 0x8000
    rows[4] = W.random_rows(1, n, seed=3, scale=1e-3)[0]
    d = O.calibrate(rows[2:3])["d"]
    codes, scale, zero, y = to_np(R.rotate_quant_int4(dev(rows), torch.from_numpy(d).cuda(), y_out=True))
    st = compare(expected(rows, d), codes, scale, zero, y, label=f"paley degenerate n={n}")
    assert scale[0] == 1.0 and np.all(codes[0] == 0)
    assert scale[2] == 1.0 and np.all(codes[2] == 0)  # lone outlier after the flip
    assert st["code_mismatches"] == 0


@pytest.mark.parametrize("n,t", [(11008, 1), (11008, 5), (11008, 255), (11008, 257), (11008, 769), (11008, 2053),
                                 (13824, 511), (13824, 513), (27648, 255), (27648, 257), (5120, 1025)])
def test_strided_rows_and_ragged_token_counts(n, t):
    """Row stride n + 64 and token counts around the launch grid (one or
    several rows per work-group, fewer rows than work-groups); a seeded
    sample of rows (first and last included) against the oracle, and on every
    row the extremes map to codes 0 and 15."""
    bits = W.random_rows(t, n, seed=t, scale=0.7, outlier=1200.0)
    d = O.calibrate(bits)["d"]
    say(f"[gpu] paley ragged n={n} T={t}")
    codes, scale, zero, y = to_np(R.rotate_quant_int4(dev(bits, ld=n + 64), torch.from_numpy(d).cuda(),
                                                      y_out=True))
    g = np.random.default_rng([12, n, t])
    rows = np.unique(np.concatenate([[0, t - 1], g.choice(t, min(t, 16), replace=False)]))
    compare(expected(bits[rows], d), codes[rows], scale[rows], zero[rows], y[rows], label=f"ragged T={t}")
    q = O.unpack_int4(codes)
    assert np.all(q.min(axis=1) == 0) and np.all(q.max(axis=1) == 15)


def test_full_size_workload_sampled():
    """The n = 11008 workload at 8192 tokens, d from its calibration batch,
    in the outlier form the benchmark times: every token on the GPU, a seeded
    sample of 32 rows (first and last included) against the oracle, the
    vector form bit-equal on every row."""
    name = "n11008_t8192"
    bits, meta = W.batch(name)
    cal = O.calibrate(W.calibration_batch(name)[0])
    assert cal["c"] == meta["channel"]
    say(f"[gpu] paley full size {name}")
    x = dev(bits)
    a = R.rotate_quant_int4_outlier(x, cal["c"], cal["sigma"])
    b = R.rotate_quant_int4(x, torch.from_numpy(cal["d"]).cuda())
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)
    codes, scale, zero = to_np(a)
    t = bits.shape[0]
    g = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[0, t - 1], g.choice(t, 30, replace=False)]))
    compare(expected(bits[rows], cal["d"]), codes[rows], scale[rows], zero[rows], None, label=name)
    q = O.unpack_int4(codes)
    assert np.all(q.min(axis=1) == 0) and np.all(q.max(axis=1) == 15)


# one width per shape of the MFMA kernel's table not covered above:
# (K chunks, column tiles) -> n
MORE_SHAPES = {(1, 2): 384, (1, 4): 768, (2, 2): 1152, (2, 4): 2304, (2, 16): 9216, (3, 2): 2176,
               (3, 8): 8704, (4, 2): 3200, (4, 4): 6400, (5, 2): 4224, (6, 2): 5248, (6, 4): 10496, (6, 8): 20992,
               (7, 2): 6272, (7, 4): 12544, (8, 2): 7296, (8, 4): 14592, (9, 2): 8832, (10, 2): 9600, (12, 2): 11648,
               # one column tile (2^k = 16): 5504 = 344 * 16 is half of 11008
               (1, 1): 192, (2, 1): 704, (4, 1): 1728, (5, 1): 2368, (11, 1): 5504, (12, 1): 5824}


@pytest.mark.parametrize("n", sorted(MORE_SHAPES.values()) + sorted(FOLDED))
def test_every_mfma_shape_matches_oracle(n):
    """For each remaining shape: the calibrated sign vector and a random one
    through the d-vector entry point against the oracle, the outlier form
    bit-equal to the vector form, and the integer zero-point form against the
    oracle."""
    m, k = O.factor(n)
    assert n in FOLDED or MORE_SHAPES[((m + 31) // 32, (1 << k) // 16)] == n
    assert R.kernel_name(n) == "rq_outer_mfma"
    t = 19
    bits = W.random_rows(t, n, seed=n + 7, scale=0.8)
    c = (n * 5) // 13
    bits[::2, c] = W.f32_to_bf16_bits(np.array([-1000.0], np.float32))[0]
    cal = O.calibrate(bits)
    assert cal["c"] == c
    g = np.random.default_rng([17, n])
    rnd = np.where(g.random(n) < 0.5, -1, 1).astype(np.int8)
    x = dev(bits)
    for label, d in (("signrot-d", cal["d"]), ("random-d", rnd)):
        say(f"[gpu] shape n={n} m={m} {label}")
        codes, scale, zero, y = to_np(R.rotate_quant_int4(x, torch.from_numpy(d).cuda(), y_out=True))
        compare(expected(bits, d), codes, scale, zero, y, label=f"n={n} {label}")
    a = to_np(R.rotate_quant_int4_outlier(x, cal["c"], cal["sigma"], y_out=True))
    b = to_np(R.rotate_quant_int4(x, torch.from_numpy(cal["d"]).cuda(), y_out=True))
    for u, v, name in zip(a, b, ("codes", "scale", "zero", "y")):
        assert np.array_equal(u, v), name
    codes, scale, zero = to_np(R.rotate_quant_int4_zint(x, cal["c"], cal["sigma"]))
    compare_zint(O.rotate(O.bf16_bits_to_f64(bits), cal["d"]), codes, scale, zero, f"zint n={n}")



@pytest.mark.parametrize("n", [11008, 24576])
def test_graph_replays_match_eager_calls(n):
    """The outer-order kernel captured in a HIP graph (after an eager call on
    the device, which builds its sign tables): three replays, with other
    eager work and synchronisations between them, each bit-equal to the
    eager call on the same input."""
    t = 8
    bits = W.random_rows(t, n, seed=n + 11, scale=0.7, outlier=1300.0)
    cal = O.calibrate(bits)
    x = dev(bits)
    ref = [v.clone() for v in R.rotate_quant_int4_outlier(x, cal["c"], cal["sigma"])]
    codes = torch.empty_like(ref[0])
    scale = torch.empty_like(ref[1])
    zero = torch.empty_like(ref[2])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(3):
                R.rotate_quant_int4_outlier(x, cal["c"], cal["sigma"], out=(codes, scale, zero))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        codes.zero_()
        scale.zero_()
        zero.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(codes, ref[0]) and torch.equal(scale, ref[1]) and torch.equal(zero, ref[2]), rep
        other = R.rotate_quant_int4_outlier(x, cal["c"], cal["sigma"])  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other[0], ref[0])
    del g
