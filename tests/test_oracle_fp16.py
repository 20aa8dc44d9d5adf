"""Pins for the oracle's hand-written IEEE binary16 conversions.

The oracle rounds fp32 -> fp16 to nearest even in its own code (no compiler
half type is used).  Pinned exhaustively against library routines: every one of
the 2^32 fp32 bit patterns against torch's CPU conversion (F16C, IEEE round to
nearest even), a sample of them against numpy's, and all 2^16 fp16 patterns
back to fp32 against numpy.
"""
import numpy as np
import pytest
import torch

import oracle


def _nan16(a):
    return ((a & 0x7C00) == 0x7C00) & ((a & 0x03FF) != 0)


def test_f16_to_f32_all_patterns():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(v)) for v in h], np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f32_to_f16_all_patterns_vs_torch():
    n = 1 << 25
    base = torch.arange(n, dtype=torch.int32)
    for c in range((1 << 32) // n):
        first = c * n
        signed = first if first < (1 << 31) else first - (1 << 32)
        ref = (base + signed).view(torch.float32).to(torch.float16).view(torch.int16)
        got = torch.from_numpy(oracle.f32_to_f16_range(first, n).view(np.int16))
        bad = ref != got
        if bad.any():
            r = ref[bad].numpy().view(np.uint16)
            o = got[bad].numpy().view(np.uint16)
            assert (_nan16(r) & _nan16(o)).all(), f"chunk {c}: fp32 -> fp16 mismatch"


def test_f32_to_f16_sample_vs_numpy():
    g = np.random.default_rng(7)
    sub = g.integers(0, 1 << 32, size=20000, dtype=np.uint64).astype(np.uint32)
    with np.errstate(over="ignore"):
        ref = sub.view(np.float32).astype(np.float16).view(np.uint16)
    got = np.array([oracle.f32_to_f16(float(v)) for v in sub.view(np.float32)], np.uint16)
    assert np.all((got == ref) | (_nan16(got) & _nan16(ref)))
    # a dense stride through every fp16 rounding region, in one consecutive run
    d0, d1 = 0x33000000, 0x47800000
    run = oracle.f32_to_f16_range(d0, d1 - d0)[::61]
    dense = np.arange(d0, d1, 61, dtype=np.uint32)
    with np.errstate(over="ignore"):
        ref_d = dense.view(np.float32).astype(np.float16).view(np.uint16)
    assert np.array_equal(run, ref_d)


@pytest.mark.parametrize("val,bits", [
    (1.0, 0x3C00), (65504.0, 0x7BFF), (65520.0, 0x7C00), (65519.99, 0x7BFF),
    (2.0 ** -24, 0x0001), (2.0 ** -25, 0x0000), (3 * 2.0 ** -26, 0x0001),
    (2.0 ** -14, 0x0400), (-2.0, 0xC000), (1.0 + 2.0 ** -11, 0x3C00),
    (1.0 + 3 * 2.0 ** -11, 0x3C02),
])
def test_f32_to_f16_known_values(val, bits):
    # IEEE 754 binary16: max finite 65504, min subnormal 2^-24, min normal 2^-14;
    # halfway cases round to the even neighbour.
    assert oracle.f32_to_f16(val) == bits
