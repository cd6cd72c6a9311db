"""Large batches and concurrent calls through the C ABI.

A 65536-token batch at n = 14336 (1.9 GB of bf16 input) is checked on
sampled rows against the oracle; a few of the rows are planted with the
largest-magnitude outliers so the index arithmetic past 2^31 bytes is used.
Calls from several host threads, each on its own stream, must give the same
bits as one call on the default stream.
"""

import sys
import threading

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


def test_65536_tokens_at_14336_sampled():
    n, t = 14336, 65536
    base, _ = W.batch("n14336_t8192")  # 8192 rows of the workload law
    say(f"[gpu] large batch n={n} T={t}")
    x = torch.from_numpy(base.view(np.int16)).cuda().view(torch.bfloat16).repeat(t // base.shape[0], 1)
    g = np.random.default_rng(17)
    rows = np.unique(np.concatenate([[0, t - 1, t // 2], g.choice(t, 29, replace=False)]))
    cal, _ = W.calibration_batch("n14336_t8192")
    ref = O.calibrate(cal)
    codes, scale, zero = R.rotate_quant_int4_outlier(x, ref["c"], ref["sigma"])
    torch.cuda.synchronize()
    bits = base[rows % base.shape[0]]
    codes_s = codes[torch.from_numpy(rows).cuda()].cpu().numpy()
    st = compare(expected(bits, ref["d"]), codes_s, scale.cpu().numpy()[rows], zero.cpu().numpy()[rows],
                 label="large batch")
    say(f"[gpu] large batch: {st}")
    # every repeat of a row gives the same bits
    c = codes.view(t // base.shape[0], base.shape[0], -1)
    assert torch.equal(c[0], c[-1]) and torch.equal(c[0], c[3])


def test_concurrent_calls_on_separate_streams():
    n = 14336
    bits, _ = W.batch("n14336_t8192", tokens=1024)
    cal, _ = W.calibration_batch("n14336_t8192")
    ref = O.calibrate(cal)
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    want = R.rotate_quant_int4_outlier(x, ref["c"], ref["sigma"])
    d = torch.from_numpy(ref["d"]).cuda()
    torch.cuda.synchronize()
    results, errors = {}, []

    def work(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                outs = []
                for _ in range(20):
                    if i % 2:
                        outs.append(R.rotate_quant_int4(x, d))
                    else:
                        outs.append(R.rotate_quant_int4_outlier(x, ref["c"], ref["sigma"]))
            s.synchronize()
            results[i] = outs
        except Exception as e:  # noqa: BLE001
            errors.append(e)

    th = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for h in th:
        h.start()
    for h in th:
        h.join()
    assert not errors, errors
    for outs in results.values():
        for o in outs:
            assert all(torch.equal(a, b) for a, b in zip(o, want))


@pytest.mark.parametrize("n,t", [(14336, 37), (28672, 5), (8, 3), (4104, 9)])
def test_stream_ceiling_moves_every_byte(n, t):
    """The traffic-ceiling kernel (a measurement aid) reads every input chunk
    and writes every output word: out word j of a row is the XOR of the four
    words of 16-byte input chunk j; s0/s1 hold the row's first two words."""
    say(f"[gpu] stream ceiling n={n} T={t}")
    ld = n + 8
    bits = W.random_rows(t, ld, seed=n, scale=3.0)
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)[:, :n]
    out, s0, s1 = R.signrot_stream_ceiling(x)
    torch.cuda.synchronize()
    words = bits[:, :n].copy().view(np.uint32).reshape(t, n // 8, 4)
    want = words[:, :, 0] ^ words[:, :, 1] ^ words[:, :, 2] ^ words[:, :, 3]
    assert np.array_equal(out.cpu().numpy().view(np.uint32).reshape(t, n // 8), want)
    assert np.array_equal(s0.cpu().numpy().view(np.uint32), words[:, 0, 0])
    assert np.array_equal(s1.cpu().numpy().view(np.uint32), words[:, 0, 1])
