"""Parity of the consumer product signrot_int4_linear (and the row sums it
uses) with the oracle.

Inputs are seeded codes, scales, zero-points and bf16 weights that both
sides receive as they are; nothing the GPU computes is fed to the oracle.  The
products q * w are exact in binary32 on both kernels, so the only differences
are binary32 rounding of the sums, bounded per output by

    tol = |s| (2 sqrt(n) u A + 2 u |z| |rowsum|) + 4 u |ref|,
    A = sum_j q_j |w_kj|,  u = 2^-24,

a probabilistic bound for the sum of n rounded terms (a term dropped or
counted twice moves an output by about A / n * 7, far above 2 sqrt(n) u A at
every n used here), the rounding of rowsum and of the two epilogue
operations.  Integer weights with a power-of-two scale and an integer
zero-point make every step exact, and those cases are compared bit for bit.
"""

import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import rotation_activation_quantization_amd as R  # noqa: E402
import signrot_workloads as W  # noqa: E402

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev_bf16(bits: np.ndarray, ld: int | None = None):
    rows, n = bits.shape
    ld = n if ld is None else ld
    buf = np.zeros((max(rows, 1), ld), np.uint16)
    buf[:rows, :n] = bits
    return torch.from_numpy(buf.view(np.int16)).cuda().view(torch.bfloat16)[:rows, :n]


def dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def inputs(t, n, rows, seed, integer=False):
    """Codes uniform over 0..15; per-token scale and zero-point in the ranges
    the quantizer produces (outlier tokens: zero near -80, small steps);
    weights like a folded down-projection, N(0, 1/n) in bf16, or integers
    -8..8 with power-of-two scales and integer zero-points."""
    g = np.random.default_rng([91, t, n, rows, seed])
    codes = g.integers(0, 256, size=(t, n // 2), dtype=np.uint8)
    if integer:
        w = g.integers(-8, 9, size=(rows, n)).astype(np.float32)
        scale = np.ldexp(1.0, g.integers(-6, 3, size=t)).astype(np.float32)
        zero = g.integers(-90, 20, size=t).astype(np.float32)
    else:
        w = (g.standard_normal((rows, n)) / np.sqrt(n)).astype(np.float32)
        scale = (g.uniform(0.05, 3.0, size=t)).astype(np.float32)
        zero = g.uniform(-2.0, 17.0, size=t).astype(np.float32)
        out = g.random(t) < 0.2
        scale[out] = g.uniform(0.1, 0.3, size=out.sum())
        zero[out] = g.uniform(-95.0, -60.0, size=out.sum())
    return codes, scale, zero, W.f32_to_bf16_bits(w)


def tolerance(codes, scale, zero, w_bits, ref, rows_idx=None):
    q = O.unpack_int4(codes).astype(np.float64)
    wv = O.bf16_bits_to_f64(w_bits if rows_idx is None else w_bits[rows_idx])
    n = q.shape[1]
    a = q @ np.abs(wv).T
    rs = np.abs(wv.sum(axis=1))
    s = np.abs(scale.astype(np.float64))[:, None]
    z = np.abs(zero.astype(np.float64))[:, None]
    return s * (2 * math.sqrt(n) * U32 * a + 2 * U32 * z * rs[None, :]) + 4 * U32 * np.abs(ref) + 1e-30


def run_linear(codes, scale, zero, w_bits, ldw=None):
    w = dev_bf16(w_bits, ldw)
    c = dev(codes)
    rs = R.weight_rowsum(w)
    name = R.int4_linear_kernel_name(c, w)
    out = R.int4_linear(c, dev(scale), dev(zero), w, rs)
    torch.cuda.synchronize()
    return out.cpu().numpy(), rs.cpu().numpy(), name


@pytest.mark.parametrize("n,rows", [(64, 7), (1000, 33), (4096, 4096), (14336, 300), (28672, 64)])
def test_weight_rowsum_is_the_correctly_rounded_sum(n, rows):
    g = np.random.default_rng([92, n])
    w_bits = W.f32_to_bf16_bits((g.standard_normal((rows, n)) * 3).astype(np.float32))
    say(f"[gpu] rowsum n={n} rows={rows}")
    rs = R.weight_rowsum(dev_bf16(w_bits, ld=n + 8)).cpu().numpy()
    want = O.weight_rowsum(w_bits).astype(np.float32)  # binary64 sum (exact here) rounded once
    assert np.array_equal(rs, want)


@pytest.mark.parametrize(
    "t,n,rows,ldw,kernel",
    [
        (300, 1024, 600, None, "int4_linear_mfma"),     # 3 x 3 tiles, ragged in both
        (129, 14336, 257, None, "int4_linear_mfma"),    # one past a tile in both
        (1, 4096, 1, None, "int4_linear_mfma"),
        (64, 64, 256, 72, "int4_linear_mfma"),          # one k step, padded rows
        (5, 28, 7, None, "int4_linear_simple"),
        (33, 1000, 17, None, "int4_linear_simple"),     # n % 64 != 0
        (40, 4096, 24, 4100, "int4_linear_simple"),     # rows not 16-byte aligned
    ],
)
def test_int4_linear_matches_oracle(t, n, rows, ldw, kernel):
    codes, scale, zero, w_bits = inputs(t, n, rows, seed=1)
    say(f"[gpu] int4_linear T={t} n={n} rows={rows} ldw={ldw}")
    out, rs, name = run_linear(codes, scale, zero, w_bits, ldw)
    assert name == kernel
    ref = O.int4_linear(codes, scale, zero, w_bits)
    tol = tolerance(codes, scale, zero, w_bits, ref)
    err = np.abs(out - ref)
    say(f"[gpu] int4_linear {name}: max err/tol {(err / tol).max():.3f}")
    assert np.all(err <= tol)


@pytest.mark.parametrize("t,n,rows,ldw", [(300, 14336, 600, None), (77, 2048, 130, None), (9, 1000, 5, None),
                                          (20, 512, 40, 520)])
def test_int4_linear_bit_exact_on_integer_operands(t, n, rows, ldw):
    codes, scale, zero, w_bits = inputs(t, n, rows, seed=2, integer=True)
    say(f"[gpu] int4_linear exact T={t} n={n} rows={rows}")
    out, rs, name = run_linear(codes, scale, zero, w_bits, ldw)
    ref = O.int4_linear(codes, scale, zero, w_bits)
    assert np.array_equal(out.astype(np.float64), ref), name


def test_int4_linear_full_size_sampled():
    """The benchmark's shape: 8192 tokens x n = 14336 into 4096 output rows, in
    the launch configuration the benchmark times.  Every output is computed on
    the GPU; the oracle checks 24 whole token rows and 40 whole weight rows
    (every tile row and column is hit)."""
    t, n, rows = 8192, 14336, 4096
    codes, scale, zero, w_bits = inputs(t, n, rows, seed=3)
    say(f"[gpu] int4_linear full size T={t} n={n} rows={rows}")
    out, rs, name = run_linear(codes, scale, zero, w_bits)
    assert name == "int4_linear_mfma"
    g = np.random.default_rng(93)
    ts = np.unique(np.concatenate([[0, t - 1], g.choice(t, 22, replace=False)]))
    ks = np.unique(np.concatenate([[0, rows - 1], g.choice(rows, 38, replace=False)]))
    ref_t = O.int4_linear(codes[ts], scale[ts], zero[ts], w_bits)
    tol_t = tolerance(codes[ts], scale[ts], zero[ts], w_bits, ref_t)
    assert np.all(np.abs(out[ts] - ref_t) <= tol_t)
    ref_k = O.int4_linear(codes, scale, zero, w_bits[ks])
    tol_k = tolerance(codes, scale, zero, w_bits, ref_k, rows_idx=ks)
    assert np.all(np.abs(out[:, ks] - ref_k) <= tol_k)
    assert np.isfinite(out).all()


def test_int4_linear_zero_sizes():
    c = torch.empty((0, 32), dtype=torch.uint8, device="cuda")
    w = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    out = R.int4_linear(c, e, e, w, R.weight_rowsum(w))
    assert out.shape == (0, 8)


def test_quantized_chain_on_the_gpu_approximates_the_projection():
    """calibrate -> rotate_quant_int4 -> fold_weights -> bf16 -> weight_rowsum
    -> int4_linear, all on the GPU, against x . W^T in float64 within the
    rigorous bound (s/2) sum_j |W'_bf16| + sum_j |y_j| |W'_bf16 - W'| (every
    level is within s/2 of its value; x W^T = y W'^T exactly).  s, y and W'
    are the oracle's; W'_bf16 is the rounded weight the product consumed."""
    n, rows = 14336, 96
    bits, meta = W.batch("n14336_t4096", tokens=48)
    cal = W.calibration_batch("n14336_t4096")[0]
    g = np.random.default_rng(94)
    w_bits = W.f32_to_bf16_bits((g.standard_normal((rows, n)) / np.sqrt(n)).astype(np.float32))
    say("[gpu] quantized chain n=14336")
    d, _, _, _ = R.calibrate(dev_bf16(cal))
    codes, scale, zero = R.rotate_quant_int4(dev_bf16(bits), d)
    wf = R.fold_weights(dev_bf16(w_bits), d)
    wfb = wf.to(torch.bfloat16)
    out = R.int4_linear(codes, scale, zero, wfb, R.weight_rowsum(wfb))
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    d_o = O.calibrate(cal)["d"]
    assert np.array_equal(d.cpu().numpy(), d_o)
    _, s_o, _, y_o = O.rotate_quant_int4(bits, d_o, precision="f64")
    wf_o = O.fold_weights(w_bits, d_o)
    wfb64 = wfb.float().cpu().numpy().astype(np.float64)
    ref = O.bf16_bits_to_f64(bits) @ O.bf16_bits_to_f64(w_bits).T
    yv = np.abs(y_o)
    bound = (s_o[:, None] / 2) * np.abs(wfb64).sum(axis=1)[None, :] + yv @ np.abs(wfb64 - wf_o).T
    # binary32 rounding of the GPU's rotation, levels and sums: 1e-5 of each term's scale
    bound = bound * (1 + 1e-4) + 1e-5 * (yv @ np.abs(wfb64).T) + 1e-6 * np.abs(ref)
    assert np.all(np.abs(out - ref) <= bound)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    say(f"[gpu] quantized chain: relative error {rel:.3e}")
    assert rel < 0.1
