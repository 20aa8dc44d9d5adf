"""CPU oracle for block-quantized matvec and routed MoE -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline`` leg
may import this package.  It wraps ``liboracle.so`` (plain C, built from
``oracle.c`` in this directory) with numpy in/out; it shares no code with the GPU
library.  See ``oracle.h`` for what every function computes and which passage of
the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_DIR, "liboracle.so")
SRC_PATH = os.path.join(_DIR, "oracle.c")

# this library's own format codes (oracle.h)
FMT = {"Q4_0": 0, "Q8_0": 1, "Q4_K": 2, "Q5_K": 3, "Q6_K": 4, "MXFP4": 5, "Q8_1": 6, "Q8_K": 7,
       "Q2_K": 8, "Q3_K": 9, "Q4_1": 10, "Q5_0": 11, "Q5_1": 12}
WEIGHT_FORMATS = ("Q4_0", "Q8_0", "Q4_K", "Q5_K", "Q6_K", "MXFP4", "Q2_K", "Q3_K", "Q4_1", "Q5_0", "Q5_1")
ACT_FORMATS = ("Q8_1", "Q8_K", "Q8_0")

# -O3 with the x86-64-v3 level (AVX2) rather than -march=native: the library is
# built in one place and may run on another host's CPU.  No contraction and no
# fast-math, so vectorisation cannot change a result.
_BUILD_CMD = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
              "-Wall", "-shared", "-fPIC", SRC_PATH, "-o", LIB_PATH, "-lm"]


def build() -> str:
    """Compile liboracle.so from oracle.c (always recompiles)."""
    tmp = LIB_PATH + ".tmp"
    cmd = list(_BUILD_CMD)
    cmd[cmd.index(LIB_PATH)] = tmp
    subprocess.run(cmd, check=True, cwd=_DIR)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        sig = {
            "or_block_elems": (I, [I]), "or_block_bytes": (I, [I]), "or_sub_elems": (I, [I]),
            "or_threads": (I, []), "or_set_threads": (None, [I]),
            "or_f16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
            "or_f32_to_f16": (ctypes.c_uint16, [ctypes.c_float]),
            "or_f32_to_f16_range": (None, [ctypes.c_uint32, ctypes.c_uint32, P]),
            "or_elem": (ctypes.c_double, [I, P, I]),
            "or_dequant_f32": (None, [I, P, I64, I64, P]),
            "or_quantize": (None, [I, P, I64, I64, I64, P]),
            "or_block_dots": (I, [I, P, I64, I64, I, P, I64, P]),
            "or_matvec": (I, [I, P, I64, I64, I, P, I64, P, I64]),
            "or_matvec_keepquant": (I, [I, P, I64, I64, I, P, I64, P]),
            "or_route": (I, [P, I64, I64, I, P, P]),
            "or_sort_pairs": (I, [P, I64, I, I64, P, P, P]),
            "or_moe_gate_up": (I, [I, P, P, I64, I64, I64, I, P, I64, P, I, P, P, P]),
            "or_moe_down": (I, [I, P, I64, I64, I64, I, P, I64, P, I, P]),
            "or_moe_combine": (None, [P, P, I64, I, I64, P]),
            "or_grouped": (I, [I, P, I64, I64, I64, I, P, I, P, I64, I, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u8(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a).view(np.uint8).reshape(-1))


def block_elems(fmt: str) -> int:
    return lib().or_block_elems(FMT[fmt])


def block_bytes(fmt: str) -> int:
    return lib().or_block_bytes(FMT[fmt])


def sub_elems(fmt: str) -> int:
    return lib().or_sub_elems(FMT[fmt])


def threads() -> int:
    return lib().or_threads()


def set_threads(n: int) -> None:
    lib().or_set_threads(n)


def row_bytes(fmt: str, k: int) -> int:
    return k // block_elems(fmt) * block_bytes(fmt)


def f16_to_f32(h: int) -> float:
    return lib().or_f16_to_f32(h)


def f32_to_f16(f: float) -> int:
    return lib().or_f32_to_f16(f)


def f32_to_f16_range(first: int, count: int) -> np.ndarray:
    out = np.empty(count, np.uint16)
    lib().or_f32_to_f16_range(first, count, _p(out))
    return out


def elem(fmt: str, block, e: int) -> float:
    b = _u8(block)
    return lib().or_elem(FMT[fmt], _p(b), e)


def dequant(fmt: str, blocks, rows: int, k: int) -> np.ndarray:
    b = _u8(blocks)
    assert b.size == rows * row_bytes(fmt, k)
    out = np.empty((rows, k), np.float32)
    lib().or_dequant_f32(FMT[fmt], _p(b), rows, k, _p(out))
    return out


def quantize(afmt: str, x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    x2 = x.reshape(-1, x.shape[-1])
    rows, k = x2.shape
    assert k % block_elems(afmt) == 0
    out = np.empty(rows * row_bytes(afmt, k), np.uint8)
    lib().or_quantize(FMT[afmt], _p(x2), rows, k, k, _p(out))
    return out.reshape(rows, row_bytes(afmt, k))


def block_dots(wfmt, W, n, k, afmt, xq, t) -> np.ndarray:
    w, a = _u8(W), _u8(xq)
    out = np.empty((t, n, k // sub_elems(wfmt)), np.int32)
    rc = lib().or_block_dots(FMT[wfmt], _p(w), n, k, FMT[afmt], _p(a), t, _p(out))
    assert rc == 0, "unsupported pair"
    return out


def matvec(wfmt, W, n, k, afmt, xq, t) -> np.ndarray:
    w, a = _u8(W), _u8(xq)
    y = np.empty((t, n), np.float32)
    rc = lib().or_matvec(FMT[wfmt], _p(w), n, k, FMT[afmt], _p(a), t, _p(y), n)
    assert rc == 0, "unsupported pair or shape"
    return y


def matvec_keepquant(wfmt, W, n, k, afmt, xq, t) -> np.ndarray:
    w, a = _u8(W), _u8(xq)
    y = np.empty((t, n), np.float64)
    rc = lib().or_matvec_keepquant(FMT[wfmt], _p(w), n, k, FMT[afmt], _p(a), t, _p(y))
    assert rc == 0, "unsupported pair or shape"
    return y


def route(logits: np.ndarray, topk: int):
    l = np.ascontiguousarray(logits, np.float32)
    t, e = l.shape
    ids = np.empty((t, topk), np.int32)
    w = np.empty((t, topk), np.float32)
    assert lib().or_route(_p(l), t, e, topk, _p(ids), _p(w)) == 0
    return ids, w


def sort_pairs(ids: np.ndarray, n_expert: int):
    ids = np.ascontiguousarray(ids, np.int32)
    t, topk = ids.shape
    counts = np.empty(n_expert, np.int32)
    offsets = np.empty(n_expert + 1, np.int32)
    pairs = np.empty(t * topk, np.int32)
    rc = lib().or_sort_pairs(_p(ids), t, topk, n_expert, _p(counts), _p(offsets), _p(pairs))
    assert rc == 0, "expert id out of range"
    return counts, offsets, pairs


def moe_gate_up(wfmt, w_gate, w_up, n_expert, hidden, inter, afmt, xq, ids):
    ids = np.ascontiguousarray(ids, np.int32)
    t, topk = ids.shape
    g = np.empty((t * topk, inter), np.float32)
    u = np.empty_like(g)
    h = np.empty_like(g)
    wg, wu, a = _u8(w_gate), _u8(w_up), _u8(xq)
    rc = lib().or_moe_gate_up(FMT[wfmt], _p(wg), _p(wu), n_expert, hidden, inter,
                              FMT[afmt], _p(a), t, _p(ids), topk, _p(g), _p(u), _p(h))
    assert rc == 0
    return g, u, h


def moe_down(wfmt, w_down, n_expert, hidden, inter, afmt, hq, ids):
    ids = np.ascontiguousarray(ids, np.int32)
    t, topk = ids.shape
    d = np.empty((t * topk, hidden), np.float32)
    wd, a = _u8(w_down), _u8(hq)
    rc = lib().or_moe_down(FMT[wfmt], _p(wd), n_expert, hidden, inter, FMT[afmt],
                           _p(a), t, _p(ids), topk, _p(d))
    assert rc == 0
    return d


def moe_combine(d: np.ndarray, w: np.ndarray) -> np.ndarray:
    w = np.ascontiguousarray(w, np.float32)
    d = np.ascontiguousarray(d, np.float32)
    t, topk = w.shape
    hidden = d.shape[1]
    y = np.empty((t, hidden), np.float32)
    lib().or_moe_combine(_p(d), _p(w), t, topk, hidden, _p(y))
    return y


def moe_forward(wfmt, w_gate, w_up, w_down, n_expert, hidden, inter, afmt, x, ids, w):
    """End to end: quantize x, gate/up + SwiGLU, quantize h, down, weighted combine.
    Returns a dict with every stage."""
    xq = quantize(afmt, x)
    g, u, h = moe_gate_up(wfmt, w_gate, w_up, n_expert, hidden, inter, afmt, xq, ids)
    hq = quantize(afmt, h)
    d = moe_down(wfmt, w_down, n_expert, hidden, inter, afmt, hq, ids)
    y = moe_combine(d, w)
    return {"xq": xq, "g": g, "u": u, "h": h, "hq": hq, "d": d, "y": y}


def grouped(wfmt, W, n_expert, n, k, afmt, xq, x_per_pair, ids) -> np.ndarray:
    ids = np.ascontiguousarray(ids, np.int32)
    t, topk = ids.shape
    y = np.empty((t * topk, n), np.float32)
    w, a = _u8(W), _u8(xq)
    rc = lib().or_grouped(FMT[wfmt], _p(w), n_expert, n, k, FMT[afmt], _p(a),
                          1 if x_per_pair else 0, _p(ids), t, topk, _p(y))
    assert rc == 0
    return y
