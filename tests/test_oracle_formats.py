"""Pins for the oracle's block layouts and dequantization.

Layouts are the public GGUF block formats (the pages name the formats only).
Pins: (1) agreement, element for element, with an independent numpy unpack on
random blocks and on every single-bit flip of a base block; (2) closed forms
built by hand from the format description; (3) the OCP MX E2M1 value table.
Parity with real GGUF files is unpinned: no GGUF file is available here.
"""
import numpy as np
import pytest

import oracle
from block_quantized_matvec_amd import synth
from tests import brute

WF = synth.WEIGHT_FORMATS


def _f16bytes(v):
    return np.array([v], np.float16).view(np.uint8)


@pytest.mark.parametrize("fmt", WF)
def test_dequant_random_blocks_match_brute(fmt):
    g = synth.rng(1, WF.index(fmt))
    rows, k = 5, 512
    W = synth.weights(fmt, rows, k, g)
    got = oracle.dequant(fmt, W, rows, k)
    ref = brute.dequant(fmt, W, rows, k)
    # fp32 rounding of the exact value: equal to the fp64 value rounded once
    assert np.array_equal(got, ref.astype(np.float32))


@pytest.mark.parametrize("fmt", WF)
def test_every_bit_flip_matches_brute(fmt):
    be, bb = synth.BLOCK[fmt]
    base = synth.weights(fmt, 1, be, synth.rng(2, WF.index(fmt)))[0].copy()
    # keep the fp16 / E8M0 scale fields fixed at sane values; flip every other bit
    scale_bytes = {"Q4_0": {0, 1}, "Q8_0": {0, 1}, "Q4_K": {0, 1, 2, 3}, "Q5_K": {0, 1, 2, 3},
                   "Q6_K": {208, 209}, "MXFP4": {0}, "Q2_K": {80, 81, 82, 83},
                   "Q3_K": {108, 109}, "Q4_1": {0, 1, 2, 3}, "Q5_0": {0, 1},
                   "Q5_1": {0, 1, 2, 3}}[fmt]
    for byte in range(bb):
        if byte in scale_bytes:
            continue
        for bit in range(8):
            blk = base.copy()
            blk[byte] ^= np.uint8(1 << bit)
            got = np.array([oracle.elem(fmt, blk, e) for e in range(be)])
            ref = brute.dequant(fmt, blk, 1, be)[0]
            assert np.array_equal(got, ref), (fmt, byte, bit)


def test_q4_0_closed_form():
    # d = 0.5; qs bytes 0xF0: low nibbles (elements 0..15) are 0 -> (0-8)*d,
    # high nibbles (elements 16..31) are 15 -> (15-8)*d
    blk = np.concatenate([_f16bytes(0.5), np.full(16, 0xF0, np.uint8)])
    w = oracle.dequant("Q4_0", blk, 1, 32)[0]
    assert np.all(w[:16] == -4.0) and np.all(w[16:] == 3.5)


def test_q8_0_closed_form():
    q = (np.arange(32) - 16).astype(np.int8)
    blk = np.concatenate([_f16bytes(0.25), q.view(np.uint8)])
    assert np.array_equal(oracle.dequant("Q8_0", blk, 1, 32)[0], 0.25 * q.astype(np.float32))


def _pack_kquant_scales(sc, m):
    """Pack eight 6-bit (scale, min) pairs the way the K-quant header stores them."""
    b = np.zeros(12, np.uint8)
    for j in range(4):
        b[j] = (sc[j] & 63) | ((sc[j + 4] >> 4) << 6)
        b[j + 4] = (m[j] & 63) | ((m[j + 4] >> 4) << 6)
        b[j + 8] = (sc[j + 4] & 15) | ((m[j + 4] & 15) << 4)
    return b


@pytest.mark.parametrize("fmt", ["Q4_K", "Q5_K"])
def test_kquant_scales_and_subblocks(fmt):
    sc = np.array([1, 9, 17, 33, 40, 48, 57, 63])
    m = np.array([63, 50, 41, 30, 22, 13, 5, 0])
    d, dmin = 2.0 ** -6, 2.0 ** -9
    hdr = np.concatenate([_f16bytes(d), _f16bytes(dmin), _pack_kquant_scales(sc, m)])
    nib = np.full(128, 0x31, np.uint8)          # low nibble 1, high nibble 3
    if fmt == "Q4_K":
        blk = np.concatenate([hdr, nib])
        n_lo, n_hi = 1, 3
    else:
        qh = np.full(32, 0b10101010, np.uint8)  # fifth bit set for every odd sub-block
        blk = np.concatenate([hdr, qh, nib])
        n_lo, n_hi = 1, 3 + 16
    w = oracle.dequant(fmt, blk, 1, 256)[0]
    for j in range(8):
        n = n_lo if j % 2 == 0 else n_hi       # even sub-blocks take low nibbles
        expect = np.float32(d * sc[j] * n - dmin * m[j])
        assert np.all(w[32 * j:32 * j + 32] == expect), j


def test_q5_k_fifth_bit_position():
    hdr = np.concatenate([_f16bytes(1.0), _f16bytes(0.0),
                          _pack_kquant_scales(np.ones(8, int), np.zeros(8, int))])
    for b in range(8):
        for l in (0, 17, 31):
            qh = np.zeros(32, np.uint8)
            qh[l] = 1 << b
            blk = np.concatenate([hdr, qh, np.zeros(128, np.uint8)])
            w = oracle.dequant("Q5_K", blk, 1, 256)[0]
            nz = np.nonzero(w)[0]
            # bit b of qh[l] is the fifth bit of element l of sub-block b
            assert list(nz) == [32 * b + l] and w[32 * b + l] == 16.0


def test_q6_k_closed_form():
    sc = (np.arange(16) * 7 - 50).astype(np.int8)
    d = 2.0 ** -7
    ql = np.zeros(128, np.uint8)
    qh = np.zeros(64, np.uint8)
    blk = np.concatenate([ql, qh, sc.view(np.uint8), _f16bytes(d)])
    w = oracle.dequant("Q6_K", blk, 1, 256)[0]
    # every 6-bit code 0 -> (0 - 32); scale per 16 elements
    assert np.array_equal(w, np.repeat(d * sc.astype(np.float64) * -32.0, 16).astype(np.float32))
    # all ones in every code field -> q6 = 63 -> +31
    blk = np.concatenate([np.full(128, 0xFF, np.uint8), np.full(64, 0xFF, np.uint8),
                          sc.view(np.uint8), _f16bytes(d)])
    w = oracle.dequant("Q6_K", blk, 1, 256)[0]
    assert np.array_equal(w, np.repeat(d * sc.astype(np.float64) * 31.0, 16).astype(np.float32))


def test_q4_1_closed_form():
    # d = 0.25, m = -1.5; nibble bytes 0x5A: low nibbles (elements 0..15) 10,
    # high nibbles (16..31) 5
    blk = np.concatenate([_f16bytes(0.25), _f16bytes(-1.5), np.full(16, 0x5A, np.uint8)])
    w = oracle.dequant("Q4_1", blk, 1, 32)[0]
    assert np.all(w[:16] == 0.25 * 10 - 1.5) and np.all(w[16:] == 0.25 * 5 - 1.5)


@pytest.mark.parametrize("fmt", ["Q5_0", "Q5_1"])
@pytest.mark.parametrize("e", [0, 7, 8, 15, 16, 23, 31])
def test_q5_fifth_bit_position(fmt, e):
    # all nibbles 3; only bit e of the little-endian 32-bit qh set: element e gets 16 + 3
    qh = np.zeros(4, np.uint8)
    qh[e // 8] = 1 << (e % 8)
    hdr = [_f16bytes(0.5)] + ([_f16bytes(2.0)] if fmt == "Q5_1" else [])
    blk = np.concatenate(hdr + [qh, np.full(16, 0x33, np.uint8)])
    w = oracle.dequant(fmt, blk, 1, 32)[0]
    off = -16 if fmt == "Q5_0" else 0
    add = 2.0 if fmt == "Q5_1" else 0.0
    expect = np.full(32, 0.5 * (3 + off) + add)
    expect[e] = 0.5 * (19 + off) + add
    assert np.array_equal(w, expect.astype(np.float32))


# Q2_K / Q3_K: the 2-bit field r of code byte 32g + l holds element 128g + 32r + l;
# 16-element sub-blocks, so element e uses scale e // 16.
def _elem_r(e):
    return (e // 32) % 4


def test_q2_k_closed_form():
    d, dmin = 2.0 ** -4, 2.0 ** -6
    scales = np.array([j | ((15 - j) << 4) for j in range(16)], np.uint8)  # sc_j = j, m_j = 15 - j
    codes = np.full(64, 0b11100100, np.uint8)                               # field r holds r
    blk = np.concatenate([scales, codes, _f16bytes(d), _f16bytes(dmin)])
    w = oracle.dequant("Q2_K", blk, 1, 256)[0]
    e = np.arange(256)
    expect = d * (e // 16) * _elem_r(e) - dmin * (15 - e // 16)
    assert np.array_equal(w, expect.astype(np.float32))


@pytest.mark.parametrize("g,r,l", [(0, 0, 0), (1, 1, 5), (0, 3, 31), (1, 2, 16)])
def test_q2_k_code_position(g, r, l):
    codes = np.zeros(64, np.uint8)
    codes[32 * g + l] = 2 << (2 * r)
    blk = np.concatenate([np.full(16, 1, np.uint8), codes, _f16bytes(1.0), _f16bytes(0.0)])
    w = oracle.dequant("Q2_K", blk, 1, 256)[0]
    assert list(np.nonzero(w)[0]) == [128 * g + 32 * r + l] and w[128 * g + 32 * r + l] == 2.0


def _pack_q3k_scales(u):
    """Sixteen 6-bit stored scales (value + 32) -> the 12 packed bytes: low four bits
    in the low nibbles of bytes 0-7 (scales 0-7) and their high nibbles (8-15), the top
    two bits of scale j in bits 2(j // 4) of byte 8 + j % 4."""
    b = np.zeros(12, np.uint8)
    for j in range(16):
        b[j % 8] |= (u[j] & 15) << (4 * (j // 8))
        b[8 + j % 4] |= (u[j] >> 4) << (2 * (j // 4))
    return b


@pytest.mark.parametrize("third", [0x00, 0xFF])
def test_q3_k_closed_form(third):
    u = np.array([(5 * j + 3) % 64 for j in range(16)])
    d = 2.0 ** -5
    blk = np.concatenate([np.full(32, third, np.uint8), np.full(64, 0b11100100, np.uint8),
                          _pack_q3k_scales(u), _f16bytes(d)])
    w = oracle.dequant("Q3_K", blk, 1, 256)[0]
    e = np.arange(256)
    q = _elem_r(e) - (0 if third else 4)      # third bit clear subtracts 4
    expect = d * (u[e // 16] - 32) * q
    assert np.array_equal(w, expect.astype(np.float32))


@pytest.mark.parametrize("g,r,l", [(0, 0, 0), (1, 2, 7), (0, 3, 31), (1, 3, 20)])
def test_q3_k_third_bit_position(g, r, l):
    hm = np.zeros(32, np.uint8)
    hm[l] = 1 << (4 * g + r)
    blk = np.concatenate([hm, np.zeros(64, np.uint8), _pack_q3k_scales(np.full(16, 33)),
                          _f16bytes(1.0)])
    w = oracle.dequant("Q3_K", blk, 1, 256)[0]
    # every code is 0 - 4 except the one whose third bit is set
    e = 128 * g + 32 * r + l
    assert w[e] == 0.0 and np.all(np.delete(w, e) == -4.0)


@pytest.mark.parametrize("e8", [0, 1, 2, 118, 126, 127, 128, 254])
def test_mxfp4_matches_ocp_table(e8):
    codes = np.arange(16, dtype=np.uint8)
    qs = (codes | (codes[::-1] << 4)).astype(np.uint8)   # element j: code j; element 16+j: code 15-j
    blk = np.concatenate([np.array([e8], np.uint8), qs])
    w = np.array([oracle.elem("MXFP4", blk, e) for e in range(32)])
    table = brute.E2M1_VALUES
    expect = np.concatenate([table[codes], table[codes[::-1]]]) * 2.0 ** (e8 - 127)
    assert np.array_equal(w, expect)
    # fp32 dequant is the value rounded once: exact, subnormals included, and
    # overflowing to infinity only at the top exponent (6 * 2^127)
    with np.errstate(over="ignore"):
        assert np.array_equal(oracle.dequant("MXFP4", blk, 1, 32)[0], expect.astype(np.float32))


def test_activation_layouts():
    x = synth.activations(3, 512, synth.rng(3))
    for afmt in synth.ACT_FORMATS:
        q = oracle.quantize(afmt, x)
        got = oracle.dequant(afmt, q, 3, 512)
        assert np.array_equal(got, brute.dequant(afmt, q, 3, 512).astype(np.float32))


def test_sizes():
    for f, (be, bb) in synth.BLOCK.items():
        assert oracle.block_elems(f) == be and oracle.block_bytes(f) == bb
