"""Write tests/golden/mse_grid.json: the quantization-MSE comparison of plain
Hadamard rotation versus SignRot, each with a symmetric and an asymmetric
per-token INT4 quantizer, on every synthetic workload.

Calls only the oracle and the seeded input generators.  The pages state the
direction of the effect (explainer "SignRot for 4-bit LLM quantization",
paragraphs on symmetric versus asymmetric quantizers and the worked example):
the flip changes nothing for a symmetric quantizer and shrinks the asymmetric
step size on tokens that carry the massive outlier.

Usage: python tests/golden/make_mse_grid.py   (about a minute on 8 cores)
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import signrot_workloads as W  # noqa: E402

# tokens per workload: enough outlier tokens for a stable mean, bounded CPU time
SAMPLE = {"n4096_t64": 64, "n8192_t2048": 512, "n14336_t4096": 512, "n28672_t8192": 192}
CONTROL_TOKENS = 256


def cells(y_plain: np.ndarray, y_sr: np.ndarray) -> dict:
    def asym(y):
        q, s, z = O.quant_asym(y)
        return O.mse(y, O.dequant(q, s, z))

    def sym(y):
        q, s = O.quant_sym(y)
        return O.mse(y, O.dequant_sym(q, s))

    return {"plain_sym": sym(y_plain), "plain_asym": asym(y_plain),
            "signrot_sym": sym(y_sr), "signrot_asym": asym(y_sr)}


def summarise(per_token: dict, mask: np.ndarray) -> dict:
    out = {"tokens": int(mask.sum())}
    for k, v in per_token.items():
        out[k] = float(v[mask].mean()) if mask.any() else None
    return out


def main() -> None:
    grid = {"_about": "mean per-token quantization MSE (rotated domain = input domain), "
                      "oracle float64; rows split by whether the token carries the planted outlier",
            "workloads": {}}
    for name, t in SAMPLE.items():
        bits, meta = W.batch(name, tokens=t)
        d = O.calibrate(W.calibration_batch(name)[0])["d"]
        x = O.bf16_bits_to_f64(bits)
        pt = cells(O.rotate(x), O.rotate(x, d))
        has = np.zeros(t, bool)
        has[meta["outlier_tokens"][meta["outlier_tokens"] < t]] = True
        grid["workloads"][name] = {"n": int(bits.shape[1]), "sample_tokens": t,
                                   "outlier": summarise(pt, has), "no_outlier": summarise(pt, ~has)}
        print(name, json.dumps(grid["workloads"][name]), flush=True)
    bits, _ = W.control_batch("n14336_decode", tokens=CONTROL_TOKENS)
    d = O.calibrate(W.calibration_batch("n14336_decode")[0])["d"]
    x = O.bf16_bits_to_f64(bits)
    pt = cells(O.rotate(x), O.rotate(x, d))
    grid["workloads"]["n14336_control"] = {"n": int(bits.shape[1]), "sample_tokens": CONTROL_TOKENS,
                                         "no_outlier": summarise(pt, np.ones(CONTROL_TOKENS, bool))}
    with open(os.path.join(HERE, "mse_grid.json"), "w") as f:
        json.dump(grid, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
