"""GPU parity: activation quantizers and dequantization, bit-exact vs the oracle."""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_matvec_amd import ft, synth
from tests.gpu_util import dev, host, log, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("act", ["Q8_1", "Q8_K", "Q8_0"])
@pytest.mark.parametrize("rows,k", [(1, 256), (3, 2048), (17, 4096), (5, 14336), (512, 4096)])
def test_quantize_bit_exact(act, rows, k):
    log(f"quantize {act} rows={rows} k={k}")
    x = synth.activations(rows, k, synth.rng(100, rows, k))
    got = host(ft.quantize_act(act, dev(x)))
    ref = oracle.quantize(act, x)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("act", ["Q8_1", "Q8_K", "Q8_0"])
@pytest.mark.parametrize("pad", [1, 3, 4])
def test_quantize_strided_rows(act, pad):
    """rows k + pad floats apart (ldx = k + pad): a row stride that is not a
    multiple of 4 floats takes the scalar-load path of the quantizers"""
    rows, k = 6, 2048
    log(f"quantize {act} strided pad={pad}")
    x = synth.activations(rows, k, synth.rng(102, pad))
    big = np.zeros((rows, k + pad), dtype=np.float32)
    big[:, :k] = x
    xd = dev(big)[:, :k]
    got = host(ft.quantize_act(act, xd))
    assert np.array_equal(got, oracle.quantize(act, x))


@pytest.mark.parametrize("act", ["Q8_1", "Q8_K"])
def test_quantize_edge_values(act):
    be = synth.BLOCK[act][0]
    g = synth.rng(101)
    blocks = [
        np.zeros(be),                                   # all zero
        np.full(be, 1e-30),                             # d underflows (fp16 for Q8_1)
        g.standard_normal(be) * 1e-6,                   # fp16 subnormal scales
        g.standard_normal(be) * 3e4,                    # large
        np.concatenate([[127.0], np.arange(be - 1) % 7 - 3.5]),   # exact .5 quotients
        np.concatenate([[-1.0], np.full(be - 1, 1.0 / 254)]),     # ties at +-0.5
        g.standard_normal(be).astype(np.float32),
    ]
    x = np.stack(blocks).astype(np.float32)
    got = host(ft.quantize_act(act, dev(x)))
    assert np.array_equal(got, oracle.quantize(act, x))


@pytest.mark.parametrize("act", ["Q8_1", "Q8_K", "Q8_0"])
def test_quantize_near_half_integers(act):
    """Quotients v / d within a few ulps of a half-integer, on both sides, for scales
    that are not powers of two: the quantizers take the code from a reciprocal
    product and fall back to the division near half-integers, so these are the
    elements where the two could part; every code must equal the oracle's."""
    be = synth.BLOCK[act][0]
    g = synth.rng(103)
    blocks = []
    for amax in (100.0, 3.3, 0.0123, 7770.0, 1.0 / 3.0):
        d32 = np.float32(amax) / np.float32(127.0)
        d = np.float32(np.float16(d32)) if act in ("Q8_1", "Q8_0") else d32
        for _ in range(6):
            k = g.integers(-127, 127, be)
            v = (k.astype(np.float32) + np.float32(0.5)) * d
            for i, steps in enumerate(g.integers(-4, 5, be)):
                for _ in range(abs(int(steps))):
                    v[i] = np.nextafter(v[i], np.float32(np.inf if steps > 0 else -np.inf), dtype=np.float32)
            v = np.clip(v, -np.float32(amax), np.float32(amax)).astype(np.float32)
            v[0] = np.float32(amax)
            blocks.append(v)
    x = np.stack(blocks).astype(np.float32)
    got = host(ft.quantize_act(act, dev(x)))
    assert np.array_equal(got, oracle.quantize(act, x))


@pytest.mark.parametrize("fmt", synth.WEIGHT_FORMATS)
@pytest.mark.parametrize("rows,k", [(1, 256), (7, 512), (33, 1536)])
def test_dequant_bit_exact(fmt, rows, k):
    log(f"dequant {fmt} rows={rows} k={k}")
    W = synth.weights(fmt, rows, k, synth.rng(102, rows, k))
    got = host(ft.dequant(fmt, dev(W), rows, k))
    ref = oracle.dequant(fmt, W, rows, k)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_dequant_q4_0_full_size():
    n = k = 2048
    W = synth.weights("Q4_0", n, k, synth.rng(103))
    got = host(ft.dequant("Q4_0", dev(W), n, k))
    assert np.array_equal(got.view(np.uint32), oracle.dequant("Q4_0", W, n, k).view(np.uint32))


def test_dequant_mxfp4_exponent_edges():
    # every E2M1 code at scales that produce fp32 subnormals and large values
    codes = np.arange(16, dtype=np.uint8)
    qs = codes | (codes[::-1] << 4)
    W = np.stack([np.concatenate([[e], qs]).astype(np.uint8) for e in (0, 1, 2, 64, 118, 127, 200, 253)])
    got = host(ft.dequant("MXFP4", dev(W.reshape(-1)), 8, 32))
    assert np.array_equal(got.view(np.uint32), oracle.dequant("MXFP4", W, 8, 32).view(np.uint32))
