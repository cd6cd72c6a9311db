"""The calibrated-form entry point signrot_rotate_quant_int4_outlier (d given
as the outlier channel c and sigma) against the oracle, and bit for bit against
signrot_rotate_quant_int4 called with the same d as a vector."""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import rotation_activation_quantization_amd as R  # noqa: E402
import signrot_workloads as W  # noqa: E402
from parity import compare, expected  # noqa: E402

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(bits):
    """bf16 rows on the GPU with the row stride padded to a multiple of 8."""
    t, n = bits.shape
    ld = (n + 7) // 8 * 8
    buf = np.zeros((max(t, 1), ld), np.uint16)
    buf[:t, :n] = bits
    return torch.from_numpy(buf.view(np.int16)).cuda().view(torch.bfloat16)[:t, :n]


@pytest.mark.parametrize("n,t", [(4096, 70), (8192, 33), (14336, 45), (28672, 20), (28, 9), (1792, 17), (64, 5),
                                 (16384, 3)])
def test_outlier_form_matches_vector_form_and_oracle(n, t):
    g = np.random.default_rng([61, n])
    for c, sigma in ((0, 1), (n - 1, -1), (int(g.integers(n)), -1), (int(g.integers(n)), 1)):
        bits = W.random_rows(t, n, seed=int(c), scale=0.8, outlier=900.0 * sigma)  # outlier on channel c
        d = (sigma * O.hadamard_row(n, c)).astype(np.int8)
        say(f"[gpu] outlier form n={n} T={t} c={c} sigma={sigma} kernel={R.kernel_name(n)}")
        x = dev(bits)
        a = R.rotate_quant_int4_outlier(x, c, sigma, y_out=True)
        b = R.rotate_quant_int4(x, torch.from_numpy(d).cuda(), y_out=True)
        torch.cuda.synchronize()
        a = [v.cpu().numpy() for v in a]
        b = [v.cpu().numpy() for v in b]
        for u, v, name in zip(a, b, ("codes", "scale", "zero", "y")):
            assert np.array_equal(u, v), name
        compare(expected(bits, d), a[0], a[1], a[2], a[3], label=f"outlier n={n} c={c}")


def test_outlier_form_on_the_workload_with_calibrated_c_and_sigma():
    """(c, sigma) straight from signrot_calibrate on the n = 14336 workload."""
    cal, _ = W.calibration_batch("n14336_t8192")
    bits, _ = W.batch("n14336_t8192", tokens=512)
    d, c, _, m = R.calibrate(dev(cal))
    sigma = -1 if m < 0 else 1
    codes, scale, zero = R.rotate_quant_int4_outlier(dev(bits), c, sigma)
    ref = R.rotate_quant_int4(dev(bits), d)
    torch.cuda.synchronize()
    assert torch.equal(codes, ref[0]) and torch.equal(scale, ref[1]) and torch.equal(zero, ref[2])


@pytest.mark.parametrize("n,t", [(14336, 1), (14336, 45), (14336, 3000), (7168, 37), (7168, 2100), (3584, 9),
                                 (3584, 1500), (28672, 1), (28672, 1100)])
def test_outlier_form_without_y_output(n, t):
    """The calibrated-form entry without y output for n = 28 * 2^k.  The
    outlier channel is placed once in each of the seven groups of four a-rows
    (each staged and zeroed by its own wave), with both signs, at row counts
    below the grid and at several rows per work-group (so that x_c of the next
    row is taken while the current one is processed).  At n = 28672 the
    channel alternates between the two 512-channel halves of its a-row, which
    that kernel stages in different phases of a row and whose half bit picks
    the sign of the second output half.  Codes, scale and zero equal the
    vector-form call bit for bit, and sampled rows meet the oracle's
    tolerances."""
    g = np.random.default_rng([63, n, t])
    blk = n // 28  # a-row length
    rows = np.unique(np.concatenate([[0, t - 1], g.choice(t, min(t, 10), replace=False)]))
    for wv in range(7):
        if n == 28672:
            c = int((4 * wv + g.integers(4)) * blk + 512 * (wv % 2) + g.integers(512))
        else:
            c = int((4 * wv + g.integers(4)) * blk + g.integers(blk))
        sigma = 1 if wv % 2 == 0 else -1
        bits = W.random_rows(t, n, seed=c, scale=0.8, outlier=700.0 * sigma)
        bits[1::3, c] = W.f32_to_bf16_bits(np.array([0.25], np.float32))[0]  # rows without the outlier
        d = (sigma * O.hadamard_row(n, c)).astype(np.int8)
        say(f"[gpu] outlier form, no y: n={n} T={t} c={c} (wave {wv}) sigma={sigma}")
        x = dev(bits)
        a = R.rotate_quant_int4_outlier(x, c, sigma)
        b = R.rotate_quant_int4(x, torch.from_numpy(d).cuda())
        torch.cuda.synchronize()
        a = [v.cpu().numpy() for v in a]
        b = [v.cpu().numpy() for v in b]
        for u, v, name in zip(a, b, ("codes", "scale", "zero")):
            assert np.array_equal(u, v), name
        compare(expected(bits[rows], d), a[0][rows], a[1][rows], a[2][rows], label=f"outlier no-y n={n} c={c}")
