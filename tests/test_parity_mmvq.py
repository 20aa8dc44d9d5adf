"""GPU parity: integer block partials (bit-exact) and the quantized matvec
(fp32, normwise 1e-5 / NMSE 1e-9) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_matvec_amd import ft, synth
from tests.gpu_util import abs_terms, check_fp32, check_fp32_small, dev, host, log, need_gpu

pytestmark = pytest.mark.gpu

PAIRS = [(w, a) for w in synth.WEIGHT_FORMATS for a in synth.ACT_FORMATS]
MMVQ_Q8_1 = [(w, "Q8_1") for w in synth.WEIGHT_FORMATS]
# the non-grouped op's other activations: Q8_0 for every format, Q8_K for the
# grouped-GEMM formats
MMVQ = (MMVQ_Q8_1 + [(w, "Q8_0") for w in synth.WEIGHT_FORMATS] +
        [(w, "Q8_K") for w in ("Q4_K", "Q5_K", "Q6_K", "MXFP4")])


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("w,a", PAIRS)
def test_block_dots_bit_exact(w, a):
    n, k, t = 37, 1536, 3
    log(f"block_dots {w}x{a}")
    g = synth.rng(200, synth.WEIGHT_FORMATS.index(w))
    W = synth.weights(w, n, k, g)
    xq = oracle.quantize(a, synth.activations(t, k, g))
    got = host(ft.debug_block_dots(w, dev(W), n, k, a, dev(xq), t))
    ref = oracle.block_dots(w, W, n, k, a, xq, t)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("w,a", PAIRS)
def test_block_dots_extreme_codes(w, a):
    # all-ones weight bytes (every code at its maximum) against activation codes
    # alternating -128 / +127
    n, k, t = 3, 512, 1
    be, bb = synth.BLOCK[w]
    W = np.full((n, k // be * bb), 0xFF, np.uint8)
    abe, abb = synth.BLOCK[a]
    xq = np.zeros((t, k // abe, abb), np.uint8)
    c0 = 2 if a == "Q8_0" else 4          # Q8_0 has no sum field: codes from byte 2
    xq[:, :, 0:c0] = 0x3C
    xq[:, :, c0:c0 + abe] = np.where(np.arange(abe) % 2 == 0, 0x80, 0x7F).astype(np.uint8)
    got = host(ft.debug_block_dots(w, dev(W), n, k, a, dev(xq.reshape(t, -1)), t))
    assert np.array_equal(got, oracle.block_dots(w, W, n, k, a, xq, t))


@pytest.mark.parametrize("w,a", MMVQ)
@pytest.mark.parametrize("n,k", [(1, 256), (45, 512), (301, 2048), (130, 4352)])
@pytest.mark.parametrize("t", [1, 2, 3, 4, 5, 8, 9])
def test_mmvq_small(w, a, n, k, t):
    log(f"mmvq {w} n={n} k={k} t={t}")
    g = synth.rng(201, n, k, t)
    W = synth.weights(w, n, k, g)
    xq = oracle.quantize(a, synth.activations(t, k, g))
    y = host(ft.mul_mat_vec_q(w, dev(W), n, k, a, dev(xq), t))
    ref = oracle.matvec(w, W, n, k, a, xq, t)
    if y.size < 16:   # a handful of outputs: the per-output bound on the term sums
        check_fp32_small(y, ref, abs_terms(w, W, n, k, a, xq, t), f"{w} n={n} k={k} t={t}")
    else:
        check_fp32(y, ref, f"{w} n={n} k={k} t={t}")


@pytest.mark.parametrize("w", ["Q4_0", "Q8_0"])
@pytest.mark.parametrize("n,k", [(77, 800), (300, 1056)])
@pytest.mark.parametrize("t", [2, 4, 8])
def test_mmvq_k_not_whole_chunks(w, n, k, t):
    """K that is not a multiple of 256: several tokens take the dot4 kernels."""
    log(f"mmvq {w} n={n} k={k} t={t}")
    g = synth.rng(203, n, k, t)
    W = synth.weights(w, n, k, g)
    xq = oracle.quantize("Q8_1", synth.activations(t, k, g))
    y = host(ft.mul_mat_vec_q(w, dev(W), n, k, "Q8_1", dev(xq), t))
    check_fp32(y, oracle.matvec(w, W, n, k, "Q8_1", xq, t), f"{w} n={n} k={k} t={t}")


@pytest.mark.parametrize("w,n,k,t", [
    ("Q8_0", 96, 16640, 1), ("Q8_0", 96, 16640, 2), ("Q4_0", 130, 16640, 1),   # > 512 units per row
    ("Q4_0", 200, 4128, 5), ("Q8_0", 70, 4128, 6),                              # 4 segments x 8 token slots
    ("Q4_K", 40, 32768, 2),                                                     # the largest K: 8 segments
])
def test_mmvq_long_rows(w, n, k, t):
    """Rows or token counts beyond what the per-wave ring holds in registers take the
    workgroup-tile kernel (Q4_K rows stop at 512 units at the largest K, 32768, and
    still take the per-wave ring)."""
    log(f"mmvq long rows {w} n={n} k={k} t={t}")
    g = synth.rng(205, n, k, t)
    W = synth.weights(w, n, k, g)
    xq = oracle.quantize("Q8_1", synth.activations(t, k, g))
    y = host(ft.mul_mat_vec_q(w, dev(W), n, k, "Q8_1", dev(xq), t))
    check_fp32(y, oracle.matvec(w, W, n, k, "Q8_1", xq, t), f"{w} n={n} k={k} t={t}")


@pytest.mark.parametrize("w,a", MMVQ_Q8_1)
@pytest.mark.parametrize("t", [1, 2, 8])
def test_mmvq_extreme_codes(w, a, t):
    """Every weight byte 0xFF (codes at their extremes, largest scales) against
    activation codes alternating -128 / +127: the integer block sums are at their
    largest magnitudes."""
    n, k = 50, 1024
    be, bb = synth.BLOCK[w]
    W = np.full((n, k // be * bb), 0xFF, np.uint8)
    blocks = W.reshape(n, k // be, bb)
    # finite scales where the format keeps them (GGUF layouts): d at 0 (Q4_0, Q8_0),
    # d and dmin at 0 (Q4_K, Q5_K), d at 208 after the int8 sub-block scales (Q6_K),
    # the E8M0 exponent in byte 0 (MXFP4, 127: unit scale), d and dmin at 80 after
    # the scale bytes and codes (Q2_K), d at 108 (Q3_K), d (and m) at 0 (Q5_0, Q4_1,
    # Q5_1)
    if w in ("Q4_0", "Q8_0"):
        blocks[:, :, 0:2] = np.frombuffer(np.float16(0.0625).tobytes(), np.uint8)
    elif w in ("Q4_K", "Q5_K"):
        blocks[:, :, 0:4] = np.frombuffer(np.array([0.0625, 0.03125], np.float16).tobytes(), np.uint8)
    elif w == "Q6_K":
        blocks[:, :, 208:210] = np.frombuffer(np.float16(0.0625).tobytes(), np.uint8)
    elif w == "Q2_K":
        blocks[:, :, 80:84] = np.frombuffer(np.array([0.0625, 0.03125], np.float16).tobytes(), np.uint8)
    elif w == "Q3_K":
        blocks[:, :, 108:110] = np.frombuffer(np.float16(0.0625).tobytes(), np.uint8)
    elif w == "Q5_0":
        blocks[:, :, 0:2] = np.frombuffer(np.float16(0.0625).tobytes(), np.uint8)
    elif w in ("Q4_1", "Q5_1"):
        blocks[:, :, 0:4] = np.frombuffer(np.array([0.0625, -0.5], np.float16).tobytes(), np.uint8)
    else:
        blocks[:, :, 0] = 127
    abe, abb = synth.BLOCK[a]
    xq = np.zeros((t, k // abe, abb), np.uint8)
    xq[:, :, 0:4] = np.frombuffer(np.array([0.5, 0.0], np.float16).tobytes(), np.uint8)
    xq[:, :, 4:4 + abe] = np.where(np.arange(abe) % 2 == 0, 0x80, 0x7F).astype(np.uint8)
    xq[:, 1::3, 4:4 + abe] = 0x81
    xq = xq.reshape(t, -1)
    y = host(ft.mul_mat_vec_q(w, dev(W), n, k, a, dev(xq), t))
    check_fp32(y, oracle.matvec(w, W, n, k, a, xq, t), f"{w} extreme t={t}")


@pytest.mark.parametrize("w,a", MMVQ)
def test_mmvq_ldy_and_row_tail(w, a):
    n, k, t = 1000, 1024, 3
    g = synth.rng(202)
    W = synth.weights(w, n, k, g)
    xq = oracle.quantize(a, synth.activations(t, k, g))
    out = torch.full((t, n + 24), 7.0, device="cuda")
    dW, dxq = dev(W), dev(xq)          # keep the device copies alive across the call
    st = ft.lib().ft_mul_mat_vec_q(ft.TYPES[w], ft._ptr(dW), n, k, ft.TYPES[a], ft._ptr(dxq), t,
                                   ft._ptr(out), n + 24, ft._stream())
    assert st == 0
    o = host(out)
    check_fp32(o[:, :n], oracle.matvec(w, W, n, k, a, xq, t))
    assert np.all(o[:, n:] == 7.0)


def test_q4_0_matvec_full_size():
    n = k = 2048
    g = synth.rng(203)
    W = synth.weights("Q4_0", n, k, g)
    x = synth.activations(1, k, g)
    xq_gpu = ft.quantize_act("Q8_1", dev(x))
    xq = oracle.quantize("Q8_1", x)
    assert np.array_equal(host(xq_gpu), xq)
    y = host(ft.mul_mat_vec_q("Q4_0", dev(W), n, k, "Q8_1", xq_gpu, 1))
    check_fp32(y, oracle.matvec("Q4_0", W, n, k, "Q8_1", xq, 1))


@pytest.mark.parametrize("w", ["Q8_0", "Q4_K"])
@pytest.mark.parametrize("n,k", [(14336, 4096), (4096, 14336)])
@pytest.mark.parametrize("t", [1, 2, 4, 8])
def test_dense_decode_full_size_sampled(w, n, k, t):
    """Full dense-decode shapes in the bench's launch configuration; the oracle
    computes a sample of rows: the first 64 and last 40 rows, the rows on both sides
    of every multiple of 16 .. 1024 that the kernels' row shares fall on (a sample
    of them), and scattered rows."""
    log(f"dense decode {w} {n}x{k} t={t}")
    g = synth.rng(204, n, k, t)
    W = synth.weights(w, n, k, g)
    x = synth.activations(t, k, g)
    xq_gpu = ft.quantize_act("Q8_1", dev(x))
    xq = oracle.quantize("Q8_1", x)
    assert np.array_equal(host(xq_gpu), xq)
    y = host(ft.mul_mat_vec_q(w, dev(W), n, k, "Q8_1", xq_gpu, t))
    edges = np.concatenate([np.arange(s, n, s * 7) for s in (16, 64, 256, 1024)])
    edges = np.concatenate([edges - 1, edges])
    rows = np.unique(np.concatenate([np.arange(64), np.arange(n - 40, n), edges[(edges >= 0) & (edges < n)],
                                     g.choice(n, 200, replace=False)]))
    ref = oracle.matvec(w, np.ascontiguousarray(W[rows]), len(rows), k, "Q8_1", xq, t)
    check_fp32(y[:, rows], ref, f"{w} {n}x{k} t={t}")
