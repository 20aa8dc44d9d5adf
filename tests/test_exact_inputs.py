"""CPU checks of the dyadic inputs the exact GPU comparisons use
(tests/test_parity_exact.py): their decoded weights are multiples of the stated
quantum within the stated range, and on them the oracle's fp64 keep-quant result
is exactly its fp32 output (so an exact GPU result has one right answer)."""
import numpy as np
import pytest

import oracle
from block_quantized_matvec_amd import synth
from tests import test_parity_exact as ex

QUANTUM = {f: 2.0 ** -9 for f in ex.MMVQ_FORMATS}
QUANTUM["MXFP4"] = 2.0 ** -2


@pytest.mark.parametrize("w", ex.MMVQ_FORMATS)
def test_dyadic_weights_decode(w):
    g = synth.rng(950, ex.MMVQ_FORMATS.index(w))
    n, k = 12, 1024
    W = ex.dyadic_weights(w, n, k, g)
    v = oracle.dequant(w, W, n, k).astype(np.float64) / QUANTUM[w]
    assert np.array_equal(v, np.rint(v)), "weights are not multiples of the quantum"
    assert np.max(np.abs(v)) <= ex.ATOM[w], (w, np.max(np.abs(v)))
    assert np.count_nonzero(v) > v.size // 4


@pytest.mark.parametrize("w", ex.MMVQ_FORMATS)
@pytest.mark.parametrize("a", ["Q8_1", "Q8_K"])
def test_dyadic_matvec_is_exact(w, a):
    g = synth.rng(951, ex.MMVQ_FORMATS.index(w), a == "Q8_K")
    n, k, t = 9, 4608 if a == "Q8_1" else 4096, 3
    W = ex.dyadic_weights(w, n, k, g)
    xq, q = ex.dyadic_act(a, t, k, g, qmax=4)
    ex.assert_exact_bound(w, a, q)
    y = oracle.matvec(w, W, n, k, a, xq, t)
    kq = oracle.matvec_keepquant(w, W, n, k, a, xq, t)
    assert np.array_equal(y.astype(np.float64), kq)


@pytest.mark.parametrize("a,blk", [("Q8_1", 32), ("Q8_K", 256)])
def test_dyadic_x_quantizes_to_its_codes(a, blk):
    g = synth.rng(952, blk)
    x, q = ex.dyadic_x(3, 1024, blk, g, qmax=3)
    xq = oracle.quantize(a, x)
    bb = synth.BLOCK[a][1]
    blocks = xq.reshape(3, -1, bb)
    off = 4
    codes = blocks[:, :, off:off + blk].view(np.int8).reshape(3, 1024)
    assert np.array_equal(codes.astype(np.int32), q)
    if a == "Q8_1":
        d = blocks[:, :, 0:2].copy().view(np.float16).astype(np.float64)
    else:
        d = blocks[:, :, 0:4].copy().view(np.float32).astype(np.float64)
    assert np.all(np.log2(d) == np.rint(np.log2(d)))


def test_dyadic_weights_combine():
    w = ex.dyadic_w(50, 8, synth.rng(953))
    assert np.all(w >= 1 / 16) and np.all(np.sum(w, axis=1) == 1.0)
    assert np.array_equal(w * 16, np.rint(w * 16))


def test_skewed_ids():
    ids = ex.skewed_ids(256, 64, 8, synth.rng(954))
    assert all(len(set(r)) == 8 for r in ids)
    c = np.bincount(ids.reshape(-1), minlength=64)
    assert c[0] == 256 and tuple(c[1:6]) == (48, 49, 47, 96, 97)
