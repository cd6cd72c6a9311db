"""The online path with the SwiGLU producer fused in, against the oracle.

signrot_swiglu_rotate_quant_int4 computes x = bf16(SiLU(gate) * up) in
binary32 inside the rotate kernel.  The oracle takes the product in float64
and rounds it once (oracle.swiglu_bf16), then runs the unfused path on that x.
The two roundings to bf16 agree wherever the float64 value is not within the
binary32 error (about 2e-6 relative) of a point halfway between two bf16
numbers; the inputs are therefore conditioned first, with the oracle: every
element whose float64 product lies within 2^-14 (relative) of such a point
has its gate, then its up, moved to the next bf16 number, alternately, until
none does (about 2.5 % of the elements move; moving up alone does not
converge where SiLU(gate) is close to a power of two, since the product then
keeps its position between two bf16 numbers).  Then x, and so every output, must match exactly what
the oracle gives, within the usual tolerances, and bit for bit what the
unfused entry point gives on the oracle's x.
"""

import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle as O  # noqa: E402
import rotation_activation_quantization_amd as R  # noqa: E402
import signrot_workloads as W  # noqa: E402
from parity import compare, expected  # noqa: E402

pytestmark = pytest.mark.gpu

MARGIN = 2.0 ** -14


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def condition(gate, up):
    """Move gate and up away from bf16 rounding midpoints of SiLU(gate) * up
    (decided by the oracle); returns new (gate, up)."""
    gate, up = gate.copy(), up.copy()
    for k in range(16):
        x = O.silu(O.bf16_bits_to_f64(gate)) * O.bf16_bits_to_f64(up)
        near = O.bf16_midpoint_distance(x) < MARGIN
        if not near.any():
            return gate, up
        which = gate if k % 2 == 0 else up
        which[near] = (which[near].astype(np.uint32) + 1).astype(np.uint16)
    raise AssertionError("conditioning did not converge")


def dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def check(gate, up, label, cal_x=None):
    gate, up = condition(gate, up)
    x = O.swiglu_bf16(gate, up)
    cal = O.calibrate(x if cal_x is None else cal_x)
    n = x.shape[1]
    say(f"[gpu] swiglu {label}: T={x.shape[0]} n={n} kernel={R.kernel_name(n)} c={cal['c']}")
    codes, scale, zero, y = R.swiglu_rotate_quant_int4(dev(gate), dev(up), cal["c"], cal["sigma"], y_out=True)
    c2, s2, z2 = R.rotate_quant_int4_outlier(dev(x), cal["c"], cal["sigma"])
    torch.cuda.synchronize()
    # the fused producer reproduces the oracle's x exactly, so the outputs
    # equal those of the unfused entry point on that x, bit for bit
    assert torch.equal(codes, c2) and torch.equal(scale, s2) and torch.equal(zero, z2), label
    st = compare(expected(x, cal["d"]), codes.cpu().numpy(), scale.cpu().numpy(), zero.cpu().numpy(),
                 y.cpu().numpy(), label=label)
    say(f"[gpu] swiglu {label}: {st}")


@pytest.mark.parametrize("n", [14336, 28672, 4096, 8192, 3584, 7168, 16384])
def test_swiglu_fused_matches_oracle(n):
    gate, up = W.swiglu_rows(37, n, seed=n)
    check(gate, up, f"n={n}")


@pytest.mark.parametrize("n", [28672, 14336])
def test_swiglu_fused_several_rows_per_work_group(n):
    """600 tokens: more rows than resident work-groups, so that work-groups
    take a second row while the first is processed."""
    gate, up = W.swiglu_rows(600, n, seed=n + 7)
    check(gate, up, f"n={n} T=600")


@pytest.mark.timeout(600)
def test_swiglu_fused_full_batch_n14336():
    """Every row of an 8192-token batch at n = 14336, calibrated on its own
    256-token calibration batch."""
    gate, up, meta = W.swiglu_batch("n14336_t8192")
    cg, cu, _ = W.swiglu_batch("n14336_t8192", tokens=256, stream=11)
    cal_x = O.swiglu_bf16(*condition(cg, cu))
    check(gate, up, "n14336_t8192", cal_x=cal_x)


def test_swiglu_strided_rows_and_decode_sizes():
    """Row stride ld = n + 64 and 1 / 4 / 16-token batches."""
    n = 14336
    for t in (1, 4, 16):
        gate, up = condition(*W.swiglu_rows(t, n, seed=t + 100))
        ld = n + 64
        gb = np.zeros((t, ld), np.uint16)
        ub = np.zeros((t, ld), np.uint16)
        gb[:, :n] = gate
        ub[:, :n] = up
        x = O.swiglu_bf16(gate, up)
        cal = O.calibrate(x)
        codes, scale, zero = R.swiglu_rotate_quant_int4(dev(gb)[:, :n], dev(ub)[:, :n], cal["c"], cal["sigma"])
        torch.cuda.synchronize()
        st = compare(expected(x, cal["d"]), codes.cpu().numpy(), scale.cpu().numpy(), zero.cpu().numpy(),
                     label=f"swiglu strided T={t}")
        say(f"[gpu] swiglu strided T={t}: {st}")
