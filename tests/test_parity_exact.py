"""GPU parity with exactly representable outputs: the matrix-core paths against
the oracle with np.array_equal.

The int8-MFMA matvec, the grouped GEMM (int8 MFMA, FP4 MFMA for MXFP4) and the
FP4-MFMA MoE kernels form the per-block integer dots inside the matrix cores,
where no debug tap can read them.  Here every input is dyadic: weight and
activation scales are powers of two and the codes are small, so that every
partial sum any kernel can form (integer dots, scaled block terms, their fp32
sums in any order) is an exact multiple of one quantum below 2^24 quanta.  Then
the fp32 output is the exact value, the oracle's fp64 result rounds to that same
value, and the comparison is bit for bit: an off-by-one in any sub-block's
integer partial, a wrong scale or a dropped term changes the output.

Each test first asserts the exactness precondition on its own inputs (a bound
on the sum of the absolute atoms, per output) instead of relying on it.
"""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_matvec_amd import ft, synth
from tests.gpu_util import check_fp32, dev, host, log, need_gpu

pytestmark = pytest.mark.gpu

MMVQ_FORMATS = ("Q4_0", "Q8_0", "Q4_K", "Q5_K", "Q6_K", "MXFP4", "Q2_K", "Q3_K", "Q4_1", "Q5_0", "Q5_1")

# Largest magnitude of the atoms one activation code can meet in any split a
# kernel may use (scale x code parts, offsets and min terms taken separately,
# Q4_K's high nibble as 16n - 128), in units of the smallest weight scale 2^-9
# (scales here are 2^-9 or 2^-8, factor 2 included).
ATOM = {"Q4_0": 2 * (15 + 8), "Q8_0": 2 * 2 * 15, "Q4_K": 2 * (3 * 15 + 3 * 16 + 3),
        "Q5_K": 2 * (3 * 31 + 3 * 16 + 3), "Q6_K": 2 * 3 * (63 + 32), "MXFP4": 2 * 12,
        "Q2_K": 2 * (3 * 3 + 3 + 8), "Q3_K": 2 * 3 * (7 + 4), "Q4_1": 2 * (15 + 2),
        "Q5_0": 2 * (31 + 16), "Q5_1": 2 * (31 + 2)}
LIMIT = 2 ** 23   # half the fp32 significand range: a 2x margin on the bound


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _p2(g, n, lo=8, hi=9):
    """n fp16 powers of two 2^-lo .. 2^-hi as [n, 2] bytes."""
    return (2.0 ** -g.integers(lo, hi + 1, n)).astype(np.float16).view(np.uint8).reshape(n, 2)


def dyadic_weights(fmt, rows, k, g):
    """Random blocks of `fmt` whose scales are 2^-8 or 2^-9 and whose scale fields
    and codes are small (see ATOM); codes that carry no scale stay uniform."""
    W = synth.weights(fmt, rows, k, g)
    bb = synth.BLOCK[fmt][1]
    b = W.reshape(-1, bb)
    nb = b.shape[0]
    small = lambda *s: g.integers(0, 4, s).astype(np.uint8)
    if fmt in ("Q4_0", "Q5_0"):
        b[:, 0:2] = _p2(g, nb)
    elif fmt == "Q8_0":
        b[:, 0:2] = _p2(g, nb)
        b[:, 2:34] = g.integers(-15, 16, (nb, 32)).astype(np.int8).view(np.uint8)
    elif fmt in ("Q4_1", "Q5_1"):
        b[:, 0:2] = _p2(g, nb)
        m = _p2(g, nb)
        m[:, 1] |= (g.integers(0, 2, nb) << 7).astype(np.uint8)   # random sign of m
        b[:, 2:4] = m
    elif fmt in ("Q4_K", "Q5_K"):
        b[:, 0:2] = _p2(g, nb)
        b[:, 2:4] = _p2(g, nb)
        sc, m = small(nb, 8), small(nb, 8)
        b[:, 4:8] = sc[:, :4]
        b[:, 8:12] = m[:, :4]
        b[:, 12:16] = sc[:, 4:] | (m[:, 4:] << 4)
    elif fmt == "Q6_K":
        b[:, 192:208] = g.integers(-3, 4, (nb, 16)).astype(np.int8).view(np.uint8)
        b[:, 208:210] = _p2(g, nb)
    elif fmt == "MXFP4":
        b[:, 0] = g.integers(126, 128, nb).astype(np.uint8)
    elif fmt == "Q2_K":
        b[:, 0:16] = small(nb, 16) | (small(nb, 16) << 4)
        b[:, 80:82] = _p2(g, nb)
        b[:, 82:84] = _p2(g, nb)
    elif fmt == "Q3_K":
        lo = small(nb, 16)
        b[:, 96:104] = lo[:, :8] | (lo[:, 8:] << 4)
        b[:, 104:108] = 0xAA       # top two bits 2 for every scale: sc - 32 = lo
        b[:, 108:110] = _p2(g, nb)
    else:
        raise ValueError(fmt)
    return W


def dyadic_act(afmt, t, k, g, qmax):
    """Activation blocks [t][k/blk] with codes uniform in [-qmax, qmax] and one
    power-of-two scale 2^-s per token (s in 3..8); Q8_1's s field and Q8_K's group
    sums are filled consistently."""
    be, bb = synth.BLOCK[afmt]
    nb = k // be
    out = np.zeros((t, nb, bb), np.uint8)
    q = g.integers(-qmax, qmax + 1, (t, nb, be)).astype(np.int8)
    for i in range(t):
        d = 2.0 ** -int(g.integers(3, 9))
        if afmt == "Q8_1":
            out[i, :, 0:2] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
            s = (d * q[i].astype(np.float64).sum(axis=1)).astype(np.float16)
            out[i, :, 2:4] = s.view(np.uint8).reshape(nb, 2)
            out[i, :, 4:36] = q[i].view(np.uint8)
        elif afmt == "Q8_0":
            out[i, :, 0:2] = np.frombuffer(np.float16(d).tobytes(), np.uint8)
            out[i, :, 2:34] = q[i].view(np.uint8)
        else:
            out[i, :, 0:4] = np.frombuffer(np.float32(d).tobytes(), np.uint8)
            out[i, :, 4:260] = q[i].view(np.uint8)
            bs = q[i].astype(np.int16).reshape(nb, 16, 16).sum(axis=2).astype(np.int16)
            out[i, :, 260:292] = bs.view(np.uint8).reshape(nb, 32)
    return out.reshape(t, nb * bb), q.reshape(t, k)


def dyadic_x(t, k, blk, g, qmax):
    """fp32 activations the quantizer maps to power-of-two scales exactly: x = q * 2^-s
    with |q| <= qmax and one element of +-127 * 2^-s in every `blk`-element block, so
    that amax / 127 = 2^-s and every x / d is an integer.  Returns x and its codes."""
    q = g.integers(-qmax, qmax + 1, (t, k)).astype(np.int32)
    nb = k // blk
    pos = g.integers(0, blk, (t, nb)) + blk * np.arange(nb)
    sgn = np.where(g.integers(0, 2, (t, nb)) == 0, -127, 127)
    np.put_along_axis(q, pos, sgn, axis=1)
    s = g.integers(3, 9, (t, 1))
    return (q * 2.0 ** -s).astype(np.float32), q


def atom_sum(wfmt, afmt, q):
    """Per row of activation codes: the sum over elements of what one code adds to
    the atoms.  FP4-MFMA paths (MXFP4 x Q8_K) take the code as 16*hi + lo with
    both halves' products formed separately."""
    q = q.astype(np.int64)
    if wfmt == "MXFP4" and afmt == "Q8_K":
        return (16 * np.abs(q >> 4) + (q & 15)).sum(axis=-1)
    return np.abs(q).sum(axis=-1)


def assert_exact_bound(wfmt, afmt, q):
    worst = int(atom_sum(wfmt, afmt, q).max()) * ATOM[wfmt]
    assert worst < LIMIT, f"inputs too large for an exact comparison ({worst} quanta)"


def dyadic_w(t, topk, g):
    """[t][topk] combine weights: multiples of 1/16 summing to 1, each >= 1/16."""
    w = np.empty((t, topk), np.float32)
    for i in range(t):
        cuts = np.sort(g.choice(np.arange(1, 16), topk - 1, replace=False))
        w[i] = np.diff(np.concatenate([[0], cuts, [16]])) / 16.0
    return w


# ---------------------------------------------------------------------------
# matvec: every format on dot4 (1-4 tokens) and on the int8 MFMA (long rows from
# 2-3 tokens, every row length from 5 tokens)
# ---------------------------------------------------------------------------
def _long_k(w):
    return 8704 if w in ("Q4_K", "Q5_K") else 4608   # rows of more than 128 units


@pytest.mark.parametrize("w", MMVQ_FORMATS)
@pytest.mark.parametrize("rows", ["short", "long"])
@pytest.mark.parametrize("t", [1, 2, 3, 4, 5, 8])
def test_mmvq_exact(w, rows, t):
    n, k = (100, 1024) if rows == "short" else (70, _long_k(w))
    log(f"mmvq exact {w} n={n} k={k} t={t}")
    g = synth.rng(900, MMVQ_FORMATS.index(w), k, t)
    W = dyadic_weights(w, n, k, g)
    xq, q = dyadic_act("Q8_1", t, k, g, qmax=4)
    assert_exact_bound(w, "Q8_1", q)
    y = host(ft.mul_mat_vec_q(w, dev(W), n, k, "Q8_1", dev(xq), t))
    ref = oracle.matvec(w, W, n, k, "Q8_1", xq, t)
    bad = np.argwhere(y != ref)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[0]}: {y[tuple(bad[0])]!r} vs {ref[tuple(bad[0])]!r}"


@pytest.mark.parametrize("w,a", [(w, "Q8_0") for w in ("Q4_0", "Q8_0", "Q4_K", "Q6_K", "MXFP4", "Q3_K")] +
                         [(w, "Q8_K") for w in ("Q4_K", "Q5_K", "Q6_K", "MXFP4")])
@pytest.mark.parametrize("t", [1, 2, 5, 8])
def test_mmvq_exact_other_activations(w, a, t):
    """Q8_0 activations (through their Q8_1 layout, dot4 and MFMA) and Q8_K
    activations (dot4 at every t), long rows."""
    n, k = 70, _long_k(w)
    log(f"mmvq exact {w} x {a} n={n} k={k} t={t}")
    g = synth.rng(904, MMVQ_FORMATS.index(w), a == "Q8_K", t)
    W = dyadic_weights(w, n, k, g)
    xq, q = dyadic_act(a, t, k, g, qmax=4)
    assert_exact_bound(w, a, q)
    y = host(ft.mul_mat_vec_q(w, dev(W), n, k, a, dev(xq), t))
    ref = oracle.matvec(w, W, n, k, a, xq, t)
    bad = np.argwhere(y != ref)
    assert bad.size == 0, f"{len(bad)} outputs differ, first {bad[0]}: {y[tuple(bad[0])]!r} vs {ref[tuple(bad[0])]!r}"


# ---------------------------------------------------------------------------
# grouped GEMM: every format, both activation layouts, skewed routing that sends
# experts through one, two and up to six passes over their weights
# ---------------------------------------------------------------------------
def skewed_ids(t, E, topk, g):
    """[t][topk] distinct ids per token.  With t = 256, E = 64, top-8 (mean 32 pairs
    per expert, 48 pairs per pass): expert 0 in every token (256 pairs, 6 passes),
    experts 1/2/3 with exactly 48/49/47 pairs, 4/5 with 96/97; the other slots are
    uniform over the remaining experts."""
    hot = 6
    ids = np.empty((t, topk), np.int32)
    for i in range(t):
        ids[i] = g.choice(np.arange(hot, E), topk, replace=False)
    ids[:, 0] = 0
    ids[0:48, 1] = 1
    ids[48:97, 1] = 2
    ids[97:144, 1] = 3
    ids[0:96, 2] = 4
    ids[96:193, 2] = 5
    return ids


@pytest.mark.parametrize("w", ["Q4_K", "Q5_K", "Q6_K", "MXFP4"])
@pytest.mark.parametrize("x_per_pair", [False, True])
def test_grouped_exact_skewed(w, x_per_pair):
    t, E, topk, n, k = 256, 64, 8, 144, 2048
    log(f"grouped exact skewed {w} per_pair={x_per_pair}")
    g = synth.rng(901, ["Q4_K", "Q5_K", "Q6_K", "MXFP4"].index(w), x_per_pair)
    Wb = dyadic_weights(w, E * n, k, g).reshape(E, n, -1)
    ids = skewed_ids(t, E, topk, g)
    counts = np.bincount(ids.reshape(-1), minlength=E)
    assert counts[0] == 256 and tuple(counts[1:6]) == (48, 49, 47, 96, 97)
    rows = t * topk if x_per_pair else t
    xq, q = dyadic_act("Q8_K", rows, k, g, qmax=4 if w != "MXFP4" else 2)
    assert_exact_bound(w, "Q8_K", q)
    y = host(ft.grouped_gemm_q(w, dev(Wb), E, n, k, "Q8_K", dev(xq), x_per_pair, dev(ids)))
    ref = oracle.grouped(w, Wb, E, n, k, "Q8_K", xq, x_per_pair, ids)
    bad = np.argwhere(y != ref)
    assert bad.size == 0, f"{len(bad)} outputs differ, first pair/row {bad[0]}"


# ---------------------------------------------------------------------------
# routed MoE: gate/up (g and u exact) and down from given quantized h (exact),
# the weighted combine within the fp32 tolerance, on the direct route (Q4_K dot4,
# MXFP4 FP4 MFMA) and the sorted tiles (MXFP4 FP4 MFMA, K-quants int8 MFMA)
# ---------------------------------------------------------------------------
MOE = {
    "q4k": dict(w="Q4_K", a="Q8_1", hidden=2048, inter=768, E=16, topk=8, xq=3),
    "mxfp4": dict(w="MXFP4", a="Q8_K", hidden=4096, inter=2048, E=12, topk=8, xq=2),
    "q4k8k": dict(w="Q4_K", a="Q8_K", hidden=2048, inter=768, E=10, topk=8, xq=3),
    "q5k": dict(w="Q5_K", a="Q8_K", hidden=2048, inter=1536, E=10, topk=8, xq=3),
    "q6k": dict(w="Q6_K", a="Q8_K", hidden=2048, inter=1536, E=10, topk=8, xq=2),
}
_mbanks = {}


def _mbank(name):
    if name not in _mbanks:
        c = MOE[name]
        g = synth.rng(902, list(MOE).index(name))
        wg = dyadic_weights(c["w"], c["E"] * c["inter"], c["hidden"], g).reshape(c["E"], c["inter"], -1)
        wu = dyadic_weights(c["w"], c["E"] * c["inter"], c["hidden"], g).reshape(c["E"], c["inter"], -1)
        wd = dyadic_weights(c["w"], c["E"] * c["hidden"], c["inter"], g).reshape(c["E"], c["hidden"], -1)
        _mbanks[name] = (wg, wu, wd, dev(wg), dev(wu), dev(wd))
    return _mbanks[name]


@pytest.mark.parametrize("name,t,route", [("q4k", 1, 1), ("q4k", 3, 1), ("q4k", 4, 1),
                                          ("mxfp4", 1, 1), ("mxfp4", 4, 1), ("mxfp4", 8, 1),
                                          ("mxfp4", 5, 2), ("mxfp4", 24, 2),
                                          ("q4k8k", 3, 2), ("q5k", 9, 0), ("q6k", 24, 2)])
def test_moe_exact(name, t, route):
    c = MOE[name]
    wg, wu, wd, dwg, dwu, dwd = _mbank(name)
    H, I, E, K, A = c["hidden"], c["inter"], c["E"], c["topk"], c["a"]
    log(f"moe exact {name} t={t} route={route}")
    g = synth.rng(903, list(MOE).index(name), t, route)
    x, qx = dyadic_x(t, H, synth.BLOCK[A][0], g, c["xq"])
    assert_exact_bound(c["w"], A, qx)
    ids = synth.expert_ids(t, E, K, g)
    ew = dyadic_w(t, K, g)
    hq, qh = dyadic_act(A, t * K, I, g, qmax=2 if c["w"] in ("MXFP4", "Q6_K") else 4)
    assert_exact_bound(c["w"], A, qh)
    np_ = t * K
    taps = {"g": torch.empty(np_, I, device="cuda"), "u": torch.empty(np_, I, device="cuda"),
            "hq": torch.empty(np_, ft.row_bytes(A, I), dtype=torch.uint8, device="cuda"),
            "down": torch.empty(np_, H, device="cuda")}
    y = host(ft.moe_q_vec(c["w"], dwg, dwu, dwd, E, H, I, A, dev(x), dev(ids), dev(ew), route=route, taps=taps,
                          in_hq=dev(hq)))
    xq = oracle.quantize(A, x)
    rg, ru, _ = oracle.moe_gate_up(c["w"], wg, wu, E, H, I, A, xq, ids)
    assert np.array_equal(host(taps["g"]), rg), "gate projections differ"
    assert np.array_equal(host(taps["u"]), ru), "up projections differ"
    rd = oracle.moe_down(c["w"], wd, E, H, I, A, hq, ids)
    assert np.array_equal(host(taps["down"]), rd), "down projections differ"
    # the weighted combine is an fp32 sum of products (no integer stage): normwise
    check_fp32(y, oracle.moe_combine(rd, ew), "weighted combine")
