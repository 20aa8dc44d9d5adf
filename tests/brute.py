"""Independent numpy brute-force unpack of the block formats (test helper).

Written separately from the C oracle, in vectorised numpy, so that the two
agreeing pins both to the stated GGUF block layouts.  Each unpacker returns
per-element integer codes and per-element fp64 scale and offset such that the
dequantized weight is  w = scale * code - offset.

Published constants used here (cited, not derived):
  * OCP Microscaling Formats (MX) v1.0, FP4 E2M1 element values:
    0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes 0..7, negated for codes 8..15;
    E8M0 scale 2^(e - 127).
"""
from __future__ import annotations

import numpy as np

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])

BLOCK = {"Q4_0": (32, 18), "Q8_0": (32, 34), "Q4_K": (256, 144), "Q5_K": (256, 176),
         "Q6_K": (256, 210), "MXFP4": (32, 17), "Q8_1": (32, 36), "Q8_K": (256, 292),
         "Q2_K": (256, 84), "Q3_K": (256, 110), "Q4_1": (32, 20), "Q5_0": (32, 22), "Q5_1": (32, 24)}


def _blocks(fmt, data):
    be, bb = BLOCK[fmt]
    return np.asarray(data, np.uint8).reshape(-1, bb)


def _f16(b2):
    return np.ascontiguousarray(b2).view(np.float16).reshape(-1).astype(np.float64)


def _nibbles_q4_0_order(qs):
    """16 packed bytes -> 32 values: low nibbles are elements 0..15, high nibbles 16..31."""
    return np.concatenate([qs & 15, qs >> 4], axis=1).astype(np.int64)


def _kquant_scales(s):
    """12 packed bytes per block -> (sc[8], m[8])."""
    s = s.astype(np.int64)
    sc = np.empty((s.shape[0], 8), np.int64)
    m = np.empty_like(sc)
    sc[:, :4] = s[:, 0:4] & 63
    m[:, :4] = s[:, 4:8] & 63
    sc[:, 4:] = (s[:, 8:12] & 15) | ((s[:, 0:4] >> 6) << 4)
    m[:, 4:] = (s[:, 8:12] >> 4) | ((s[:, 4:8] >> 6) << 4)
    return sc, m


def _kquant_nibbles(qs):
    """128 bytes -> 256 values ordered (chunk c, half h, lane l): h=0 low nibble."""
    q = qs.reshape(-1, 4, 1, 32).astype(np.int64)
    return np.concatenate([q & 15, q >> 4], axis=2).reshape(-1, 256)


def unpack(fmt, data):
    """-> (code int64 [nb, be], scale f64 [nb, be], offset f64 [nb, be])"""
    b = _blocks(fmt, data)
    nb = b.shape[0]
    if fmt == "Q4_0":
        code = _nibbles_q4_0_order(b[:, 2:18]) - 8
        scale = np.repeat(_f16(b[:, 0:2])[:, None], 32, 1)
        off = np.zeros_like(scale)
    elif fmt == "Q8_0":
        code = b[:, 2:34].view(np.int8).astype(np.int64)
        scale = np.repeat(_f16(b[:, 0:2])[:, None], 32, 1)
        off = np.zeros_like(scale)
    elif fmt in ("Q4_K", "Q5_K"):
        d, dmin = _f16(b[:, 0:2]), _f16(b[:, 2:4])
        sc, m = _kquant_scales(b[:, 4:16])
        if fmt == "Q4_K":
            code = _kquant_nibbles(b[:, 16:144])
        else:
            code = _kquant_nibbles(b[:, 48:176])
            qh = b[:, 16:48].astype(np.int64)                       # [nb, 32]
            bit = np.arange(8)[None, :, None]                        # sub-block 2c+h
            hb = (qh[:, None, :] >> bit) & 1                         # [nb, 8, 32]
            code = code + 16 * hb.reshape(nb, 256)
        scale = np.repeat(d[:, None] * sc, 32, 1)
        off = np.repeat(dmin[:, None] * m, 32, 1)
    elif fmt == "Q6_K":
        ql = b[:, 0:128].astype(np.int64).reshape(nb, 2, 2, 32)      # [g][half][l]
        qh = b[:, 128:192].astype(np.int64).reshape(nb, 2, 32)       # [g][l]
        lo = np.stack([ql[:, :, 0] & 15, ql[:, :, 1] & 15, ql[:, :, 0] >> 4, ql[:, :, 1] >> 4], 2)
        hi = np.stack([(qh >> (2 * r)) & 3 for r in range(4)], 2)    # [g][r][l]
        code = ((lo | (hi << 4)) - 32).reshape(nb, 256)
        sc = b[:, 192:208].view(np.int8).astype(np.float64)          # [nb, 16]
        scale = np.repeat(_f16(b[:, 208:210])[:, None] * sc, 16, 1)
        off = np.zeros_like(scale)
    elif fmt in ("Q4_1", "Q5_0", "Q5_1"):
        qo = {"Q4_1": 4, "Q5_0": 6, "Q5_1": 8}[fmt]                   # first nibble byte
        code = _nibbles_q4_0_order(b[:, qo:qo + 16])
        if fmt != "Q4_1":
            qh = np.unpackbits(b[:, qo - 4:qo], axis=1, bitorder="little").astype(np.int64)  # bit e of qh
            code = code + 16 * qh
        if fmt == "Q5_0":
            code = code - 16
        scale = np.repeat(_f16(b[:, 0:2])[:, None], 32, 1)
        off = np.zeros_like(scale) if fmt == "Q5_0" else -np.repeat(_f16(b[:, 2:4])[:, None], 32, 1)
    elif fmt in ("Q2_K", "Q3_K"):
        # 64 code bytes as [g][l]; the element order is (g, r, l) with the 2-bit
        # field r of each byte
        qb = b[:, 16:80] if fmt == "Q2_K" else b[:, 32:96]
        qb = qb.astype(np.int64).reshape(nb, 2, 1, 32)
        code = ((qb >> (2 * np.arange(4)[None, None, :, None])) & 3).reshape(nb, 256)
        if fmt == "Q2_K":
            s = b[:, 0:16].astype(np.int64)
            scale = np.repeat(_f16(b[:, 80:82])[:, None] * (s & 15), 16, 1)
            off = np.repeat(_f16(b[:, 82:84])[:, None] * (s >> 4), 16, 1)
        else:
            hm = b[:, 0:32].astype(np.int64)                               # [nb, l]
            third = (hm[:, None, :] >> np.arange(8)[None, :, None]) & 1    # [nb, 4g + r, l]
            code = code + 4 * third.reshape(nb, 256) - 4
            s = b[:, 96:108].astype(np.int64)
            low = np.concatenate([s[:, 0:8] & 15, s[:, 0:8] >> 4], 1)      # scales 0..15
            top = np.concatenate([(s[:, 8:12] >> (2 * q)) & 3 for q in range(4)], 1)
            sc = (low | (top << 4)) - 32
            scale = np.repeat(_f16(b[:, 108:110])[:, None] * sc, 16, 1)
            off = np.zeros_like(scale)
    elif fmt == "MXFP4":
        c = _nibbles_q4_0_order(b[:, 1:17])
        code = (2 * E2M1_VALUES[c]).astype(np.int64)                 # doubled: integers
        scale = np.repeat(np.ldexp(1.0, b[:, 0].astype(np.int64) - 128)[:, None], 32, 1)
        off = np.zeros_like(scale)
    elif fmt == "Q8_1":
        code = b[:, 4:36].view(np.int8).astype(np.int64)
        scale = np.repeat(_f16(b[:, 0:2])[:, None], 32, 1)
        off = np.zeros_like(scale)
    elif fmt == "Q8_K":
        code = b[:, 4:260].view(np.int8).astype(np.int64)
        scale = np.repeat(np.ascontiguousarray(b[:, 0:4]).view(np.float32).reshape(-1)
                          .astype(np.float64)[:, None], 256, 1)
        off = np.zeros_like(scale)
    else:
        raise ValueError(fmt)
    return code, scale, off


def dequant(fmt, data, rows, k):
    code, scale, off = unpack(fmt, data)
    return (scale * code - off).reshape(rows, k)


def codes(fmt, data, rows, k):
    return unpack(fmt, data)[0].reshape(rows, k)


def block_dots(wfmt, W, n, k, afmt, xq, t, sub):
    cw = codes(wfmt, W, n, k)                         # [n, k]
    ca = codes(afmt, xq, t, k)                        # [t, k]
    prod = ca[:, None, :] * cw[None, :, :]            # [t, n, k]
    return prod.reshape(t, n, k // sub, sub).sum(-1)  # int64


def matvec(wfmt, W, n, k, afmt, xq, t):
    return dequant(afmt, xq, t, k) @ dequant(wfmt, W, n, k).T   # fp64 [t, n]
