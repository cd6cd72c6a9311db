"""Seeded synthetic activations for the SignRot online path.

This module only draws random inputs; it holds none of the method's
arithmetic (no rotation, no quantization).  Both the CPU oracle's tests and
the GPU path read the very same bf16 bit patterns produced here.

Each workload stands in for the input of an LLM down-projection (the width n
of the MLP hidden layer): Gaussian or Student-t background activations, one
"massive outlier" channel that carries a huge value in a fraction of tokens,
and, for the widest case, a few mildly amplified channels.  Values are drawn
in float32 and rounded to bf16 (round to nearest, ties to even).

Random streams: numpy.random.default_rng([2611, seed, stream]) with
stream 0 = the batch, 1 = the calibration batch, 2 = channel choices,
3 = the no-outlier control batch, 100 + r = decode repetition r.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 2611
_CHUNK = 256  # rows drawn per call: fixes the draw order, bounds memory


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int  # the workload's own seed stream
    n: int
    tokens: int
    law: str  # "normal" or "t"
    width: float  # std for "normal", multiplier for "t"
    df: float = 0.0
    p_outlier: float = 0.0
    m_lo: float = 0.0
    m_hi: float = 0.0
    p_positive: float = 1.0
    fixed_channel: int | None = None  # None -> seeded
    mild_channels: int = 0
    mild_factor: float = 1.0
    calib_tokens: int = 256
    calib_same: bool = False
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # n = 2^12, N(0,1), channel 1234 = +M in 25% of tokens, calibrate on the batch
    "n4096_t64": Workload("n4096_t64", 1, 4096, 64, "normal", 1.0, p_outlier=0.25, m_lo=500, m_hi=2000,
                     fixed_channel=1234, calib_tokens=64, calib_same=True),
    # n = 2^13, Student-t(4)*0.5, seeded channel = +-M (90% +) in 30% of tokens
    "n8192_t2048": Workload("n8192_t2048", 2, 8192, 2048, "t", 0.5, df=4, p_outlier=0.30, m_lo=500, m_hi=2000,
                     p_positive=0.9, calib_tokens=256),
    # n = 28 * 2^9 (LLaMA3-8B down_proj input), N(0, 0.7), +M in 20% of tokens
    "n14336_t4096": Workload("n14336_t4096", 3, 14336, 4096, "normal", 0.7, p_outlier=0.20, m_lo=800, m_hi=2500,
                     calib_tokens=256),
    # the throughput workload: the same law at 8192 tokens
    "n14336_t8192": Workload("n14336_t8192", 3, 14336, 8192, "normal", 0.7, p_outlier=0.20, m_lo=800, m_hi=2500,
                       calib_tokens=256),
    # n = 28 * 2^10 (LLaMA3-70B), Student-t(3)*0.4, +M in 15%, 8 mild channels x20
    "n28672_t8192": Workload("n28672_t8192", 4, 28672, 8192, "t", 0.4, df=3, p_outlier=0.15, m_lo=1000, m_hi=3000,
                     mild_channels=8, mild_factor=20.0, calib_tokens=512),
    # n = 43 * 2^8 (LLaMA-2-7B down_proj input; outer Paley factor of order 344),
    # N(0, 0.7), +M in 20% of tokens
    "n11008_t8192": Workload("n11008_t8192", 6, 11008, 8192, "normal", 0.7, p_outlier=0.20, m_lo=800, m_hi=2500,
                       calib_tokens=256),
    # decode-shaped batches with the n = 14336 law (1, 4 or 16 tokens per call)
    "n14336_decode": Workload("n14336_decode", 5, 14336, 16, "normal", 0.7, p_outlier=0.20, m_lo=800, m_hi=2500,
                     calib_tokens=256, extra={"batches": (1, 4, 16), "repeats": 10000}),
}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([SEED_ROOT, seed, stream])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bf16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def channels(w: Workload):
    """(outlier channel c, array of mild channels) drawn from stream 2."""
    g = rng(w.seed, 2)
    c = int(g.integers(0, w.n)) if w.fixed_channel is None else int(w.fixed_channel)
    mild = np.zeros(0, dtype=np.int64)
    if w.mild_channels:
        pool = np.setdiff1d(np.arange(w.n), [c])
        mild = np.sort(g.choice(pool, size=w.mild_channels, replace=False))
    return c, mild


def _draw(w: Workload, tokens: int, g: np.random.Generator, with_outlier: bool = True):
    c, mild = channels(w)
    has = g.random(tokens) < (w.p_outlier if with_outlier else 0.0)
    mag = g.uniform(w.m_lo, w.m_hi, size=tokens) if w.m_hi > 0 else np.zeros(tokens)
    pos = g.random(tokens) < w.p_positive
    out = np.empty((tokens, w.n), dtype=np.uint16)
    for r0 in range(0, tokens, _CHUNK):
        r1 = min(tokens, r0 + _CHUNK)
        if w.law == "normal":
            v = g.standard_normal((r1 - r0, w.n), dtype=np.float32) * np.float32(w.width)
        else:
            v = g.standard_t(w.df, size=(r1 - r0, w.n)).astype(np.float32) * np.float32(w.width)
        if mild.size:
            v[:, mild] *= np.float32(w.mild_factor)
        sel = has[r0:r1]
        if sel.any():
            val = np.where(pos[r0:r1], mag[r0:r1], -mag[r0:r1]).astype(np.float32)
            v[sel, c] = val[sel]
        out[r0:r1] = f32_to_bf16_bits(v)
    meta = {"channel": c, "mild": mild, "outlier_tokens": np.flatnonzero(has),
            "outlier_value": np.where(pos, mag, -mag)}
    return out, meta


def batch(name: str, tokens: int | None = None):
    """The workload's token batch: (bf16 bits uint16 [T, n], metadata)."""
    w = WORKLOADS[name]
    t = w.tokens if tokens is None else int(tokens)
    return _draw(w, t, rng(w.seed, 0))


def calibration_batch(name: str):
    """The calibration batch (the 64-token n = 4096 workload calibrates on its own batch)."""
    w = WORKLOADS[name]
    if w.calib_same:
        return batch(name)
    return _draw(w, w.calib_tokens, rng(w.seed, 1))


def control_batch(name: str = "n14336_decode", tokens: int = 4096):
    """No-outlier control batch with the workload's background law."""
    w = WORKLOADS[name]
    return _draw(w, tokens, rng(w.seed, 3), with_outlier=False)


def decode_batch(name: str, tokens: int, repetition: int):
    """One decode-shaped batch of `tokens` rows for repetition r."""
    w = WORKLOADS[name]
    return _draw(w, tokens, rng(w.seed, 100 + repetition))


def random_rows(tokens: int, n: int, seed: int, scale: float = 1.0, outlier: float = 0.0):
    """Small generic bf16 rows for edge-case tests: N(0, scale), and channel
    (seed % n) set to +outlier when outlier != 0."""
    g = np.random.default_rng([SEED_ROOT, 99, seed])
    v = g.standard_normal((tokens, n), dtype=np.float32) * np.float32(scale)
    if outlier and n:
        v[:, seed % n] = np.float32(outlier)
    return f32_to_bf16_bits(v)


def swiglu_batch(name: str, tokens: int | None = None, stream: int = 10):
    """gate and up inputs of a SwiGLU producer (bf16 bits [T, n] each) for the
    workload's width: gate ~ N(0, 1.5), up ~ N(0, 0.6); in the workload's
    outlier tokens the outlier channel gets gate ~ U[6, 9] and up = M / gate
    with M ~ U[m_lo, m_hi], so that SiLU(gate) * up carries the massive value
    there.  Stream 10 + k of the workload's seed (k = 0 the batch, 1 the
    calibration batch)."""
    w = WORKLOADS[name]
    t = w.tokens if tokens is None else int(tokens)
    g = rng(w.seed, stream)
    c, _ = channels(w)
    has = g.random(t) < w.p_outlier
    mag = g.uniform(w.m_lo, w.m_hi, size=t)
    gc = g.uniform(6.0, 9.0, size=t)
    gate = np.empty((t, w.n), dtype=np.uint16)
    up = np.empty((t, w.n), dtype=np.uint16)
    for r0 in range(0, t, _CHUNK):
        r1 = min(t, r0 + _CHUNK)
        gv = g.standard_normal((r1 - r0, w.n), dtype=np.float32) * np.float32(1.5)
        uv = g.standard_normal((r1 - r0, w.n), dtype=np.float32) * np.float32(0.6)
        sel = has[r0:r1]
        if sel.any():
            gv[sel, c] = gc[r0:r1][sel].astype(np.float32)
            uv[sel, c] = (mag[r0:r1][sel] / gc[r0:r1][sel]).astype(np.float32)
        gate[r0:r1] = f32_to_bf16_bits(gv)
        up[r0:r1] = f32_to_bf16_bits(uv)
    return gate, up, {"channel": c, "outlier_tokens": np.flatnonzero(has)}


def swiglu_rows(tokens: int, n: int, seed: int, outlier: float = 1500.0):
    """Small generic gate / up rows (bf16 bits [T, n] each) for edge-case tests:
    gate ~ N(0, 1.5), up ~ N(0, 0.6); channel (seed % n) gets gate = 8 and
    up = outlier / 8 in every third token."""
    g = np.random.default_rng([SEED_ROOT, 98, seed])
    gv = g.standard_normal((tokens, n), dtype=np.float32) * np.float32(1.5)
    uv = g.standard_normal((tokens, n), dtype=np.float32) * np.float32(0.6)
    if outlier and n:
        gv[::3, seed % n] = np.float32(8.0)
        uv[::3, seed % n] = np.float32(outlier / 8.0)
    return f32_to_bf16_bits(gv), f32_to_bf16_bits(uv)
