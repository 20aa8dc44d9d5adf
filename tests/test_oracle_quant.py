"""Pins for the oracle's activation quantizers (Q8_1, Q8_0 and Q8_K).

Reading adopted (the pages name the Q8 activation quantizers but not their
arithmetic): Q8_1 stores d = fp16(amax/127) and quantizes against the stored d,
rounding x/d half away from zero and clamping to [-127, 127]; s = fp16(d * sum q).
Q8_0 (vllm.cpp PR #523, What changed: the Q8_0 activation quantizer) is the same
arithmetic in the 34-byte block without s.  Q8_K keeps d = amax/127 in fp32 and
stores 16-element group sums.
Pins: the round-off invariant |x - q d| <= d/2 (plus the fp32 quotient's own
error), the argmax element maps to +-127, odd symmetry, power-of-two scaling,
zero blocks, group sums, and the stored scale fields against numpy's fp16.
"""
import numpy as np
import pytest

import oracle
from block_quantized_matvec_amd import synth
from tests import brute

ACT = ("Q8_1", "Q8_0", "Q8_K")


def _fields(afmt, q):
    code, scale, _ = brute.unpack(afmt, q)
    be = synth.BLOCK[afmt][0]
    return code, scale[:, 0], be


@pytest.mark.parametrize("afmt", ACT)
@pytest.mark.parametrize("scale", [1.0, 1e-3, 37.5])
def test_roundoff_invariant(afmt, scale):
    x = synth.activations(8, 2048, synth.rng(10)) * np.float32(scale)
    q = oracle.quantize(afmt, x)
    code, d, be = _fields(afmt, q)
    xb = x.reshape(-1, be).astype(np.float64)
    err = np.abs(xb - code * d[:, None])
    clamped = np.abs(code) == 127
    # |x/d| rounds to within 1/2; the fp32 quotient adds at most 127.5 * 2^-24
    assert np.all(err[~clamped] <= (d[:, None] * (0.5 + 2.0 ** -17)).repeat(be, 1)[~clamped])
    # clamped elements: for Q8_1 the stored fp16 d can sit up to 2^-11 below amax/127
    assert np.all(err[clamped] <= (d[:, None] * 0.57).repeat(be, 1)[clamped])


@pytest.mark.parametrize("afmt", ACT)
def test_argmax_maps_to_127_and_odd_symmetry(afmt):
    x = synth.activations(4, 1024, synth.rng(11))
    q = oracle.quantize(afmt, x)
    qn = oracle.quantize(afmt, -x)
    code, _, be = _fields(afmt, q)
    coden, _, _ = _fields(afmt, qn)
    xb = x.reshape(-1, be)
    am = np.argmax(np.abs(xb), axis=1)
    top = code[np.arange(code.shape[0]), am]
    assert np.all(np.abs(top) >= 126)            # fp16 rounding of d may give 126
    if afmt == "Q8_K":
        assert np.all(np.abs(top) == 127)        # fp32 d: exactly 127
    assert np.array_equal(coden, -code)


@pytest.mark.parametrize("afmt", ACT)
def test_power_of_two_scaling(afmt):
    x = synth.activations(2, 512, synth.rng(12))
    q0 = oracle.quantize(afmt, x)
    q1 = oracle.quantize(afmt, x * np.float32(8.0))
    c0, d0, _ = _fields(afmt, q0)
    c1, d1, _ = _fields(afmt, q1)
    assert np.array_equal(c0, c1) and np.array_equal(d1, 8.0 * d0)


@pytest.mark.parametrize("afmt", ACT)
def test_zero_block(afmt):
    be, bb = synth.BLOCK[afmt]
    q = oracle.quantize(afmt, np.zeros((1, be), np.float32))
    assert not q.any()


def test_q8_1_stored_fields():
    x = synth.activations(16, 1024, synth.rng(13))
    q = oracle.quantize("Q8_1", x).reshape(-1, 36)
    xb = x.reshape(-1, 32)
    amax = np.abs(xb).max(1).astype(np.float32)
    d_ref = (amax / np.float32(127.0)).astype(np.float16)
    assert np.array_equal(q[:, 0:2].copy().view(np.float16).ravel(), d_ref)
    code = q[:, 4:].view(np.int8).astype(np.int64)
    s_ref = (d_ref.astype(np.float32) * code.sum(1).astype(np.float32)).astype(np.float16)
    assert np.array_equal(q[:, 2:4].copy().view(np.float16).ravel(), s_ref)
    # the codes are round-half-away of the fp32 quotient against the stored d
    quot = xb / d_ref.astype(np.float32)[:, None]
    # round half away from zero, decided on the float32 quotient
    exact = np.where(np.abs(quot - np.trunc(quot)) == 0.5, np.trunc(quot) + np.sign(quot),
                     np.rint(quot))
    assert np.array_equal(code, np.clip(exact, -127, 127).astype(np.int64))


def test_q8_k_stored_fields():
    x = synth.activations(8, 1024, synth.rng(14))
    q = oracle.quantize("Q8_K", x).reshape(-1, 292)
    xb = x.reshape(-1, 256)
    d_ref = np.abs(xb).max(1).astype(np.float32) / np.float32(127.0)
    assert np.array_equal(q[:, 0:4].copy().view(np.float32).ravel(), d_ref)
    code = q[:, 4:260].view(np.int8).astype(np.int64)
    bs = q[:, 260:292].copy().view(np.int16).astype(np.int64)
    assert np.array_equal(bs, code.reshape(-1, 16, 16).sum(-1))


def test_half_way_rounds_away_from_zero():
    # a block whose amax is 127 gives d = 1 exactly, so x/d are the x themselves
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 127.0
    x[0, 1:6] = [0.5, -0.5, 2.5, -2.5, 126.5]
    q = oracle.quantize("Q8_1", x)
    code = q[0, 4:].view(np.int8)
    assert list(code[:6]) == [127, 1, -1, 3, -3, 127]


def test_q8_0_stored_fields():
    x = synth.activations(16, 1024, synth.rng(15))
    q = oracle.quantize("Q8_0", x).reshape(-1, 34)
    xb = x.reshape(-1, 32)
    amax = np.abs(xb).max(1).astype(np.float32)
    d_ref = (amax / np.float32(127.0)).astype(np.float16)
    assert np.array_equal(q[:, 0:2].copy().view(np.float16).ravel(), d_ref)
    code = q[:, 2:].view(np.int8).astype(np.int64)
    quot = xb / d_ref.astype(np.float32)[:, None]
    exact = np.where(np.abs(quot - np.trunc(quot)) == 0.5, np.trunc(quot) + np.sign(quot),
                     np.rint(quot))
    assert np.array_equal(code, np.clip(exact, -127, 127).astype(np.int64))


def test_q8_0_dots_against_numpy():
    """Q8_0 activations in the matvec and the integer partials: numpy int64 and fp64
    from an independent unpack of both sides."""
    g = synth.rng(16)
    n, k, t = 7, 512, 2
    W = synth.weights("Q4_K", n, k, g)
    xq = oracle.quantize("Q8_0", synth.activations(t, k, g))
    wc, ws, wm = brute.unpack("Q4_K", W.reshape(-1, 144))
    wv = (wc * ws - wm).reshape(n, k)
    ac, asc, _ = brute.unpack("Q8_0", xq.reshape(-1, 34))
    av = (ac * asc).reshape(t, k)
    y = oracle.matvec("Q4_K", W, n, k, "Q8_0", xq, t)
    ref = av @ wv.T
    assert np.max(np.abs(y - ref)) <= 1e-6 * np.max(np.abs(ref))
    p = oracle.block_dots("Q4_K", W, n, k, "Q8_0", xq, t)
    ip = (wc.reshape(n, 1, k // 32, 32) * ac.reshape(1, t, k // 32, 32)).sum(-1).transpose(1, 0, 2)
    assert np.array_equal(p, ip.astype(np.int64))
