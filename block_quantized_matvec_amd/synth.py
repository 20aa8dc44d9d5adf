"""Seeded synthetic inputs for the block-quantized matvec / routed-MoE path.

This module draws random bytes and numbers only; it holds none of the method's
arithmetic (no dequantization, no quantization, no dot products).  Both the GPU
tests/bench and the CPU oracle are fed from it, so the same bytes reach both.

Recipe (plainest reading of the workloads the pages describe; the pages give no
value distributions, so these are stated choices):
  * fp16 scales d (and dmin) are fp16(U[1e-3, 1e-2]).
  * nibble / code bytes, packed 6-bit scale bytes and high-bit bytes are uniform
    random bytes, which makes every packed field uniform over its range.
  * Q8_0 codes are clip(rint(N(0, 40)), -127, 127).
  * Q6_K int8 scales are uniform over [-128, 127].
  * MXFP4 E8M0 exponents are uniform over 118..126.
  * Q4_1 / Q5_1 d and m, Q5_0 d, Q2_K d and dmin and Q3_K d are fp16 scales as above; their scale, code and
    third-bit bytes are uniform random bytes.
  * activations and router logits are fp32 N(0, 1).
Weight block layouts (byte offsets of the scale fields) follow the public GGUF
block formats.
"""
from __future__ import annotations

import numpy as np

BLOCK = {  # name: (elements, bytes)
    "Q4_0": (32, 18), "Q8_0": (32, 34), "Q4_K": (256, 144), "Q5_K": (256, 176),
    "Q6_K": (256, 210), "MXFP4": (32, 17), "Q8_1": (32, 36), "Q8_K": (256, 292),
    "Q2_K": (256, 84), "Q3_K": (256, 110), "Q4_1": (32, 20), "Q5_0": (32, 22), "Q5_1": (32, 24),
}
WEIGHT_FORMATS = ("Q4_0", "Q8_0", "Q4_K", "Q5_K", "Q6_K", "MXFP4", "Q2_K", "Q3_K", "Q4_1", "Q5_0", "Q5_1")
ACT_FORMATS = ("Q8_1", "Q8_K", "Q8_0")   # Q8_0: also a weight format, same layout


def rng(*seed) -> np.random.Generator:
    return np.random.default_rng(list(seed))


def row_bytes(fmt: str, k: int) -> int:
    be, bb = BLOCK[fmt]
    assert k % be == 0, f"{fmt}: k={k} not a multiple of {be}"
    return k // be * bb


def _fp16_scales(g: np.random.Generator, n: int) -> np.ndarray:
    return g.uniform(1e-3, 1e-2, n).astype(np.float16).view(np.uint8).reshape(n, 2)


def weights(fmt: str, rows: int, k: int, g: np.random.Generator) -> np.ndarray:
    """rows x k weights as raw blocks: uint8 array [rows, row_bytes(fmt, k)]."""
    be, bb = BLOCK[fmt]
    nb = rows * (k // be)
    b = g.integers(0, 256, size=(nb, bb), dtype=np.uint8)
    if fmt in ("Q4_0", "Q5_0"):
        b[:, 0:2] = _fp16_scales(g, nb)
    elif fmt in ("Q4_1", "Q5_1"):
        b[:, 0:2] = _fp16_scales(g, nb)      # d
        b[:, 2:4] = _fp16_scales(g, nb)      # m
    elif fmt == "Q8_0":
        b[:, 0:2] = _fp16_scales(g, nb)
        q = np.clip(np.rint(g.normal(0.0, 40.0, size=(nb, 32))), -127, 127).astype(np.int8)
        b[:, 2:34] = q.view(np.uint8)
    elif fmt in ("Q4_K", "Q5_K"):
        b[:, 0:2] = _fp16_scales(g, nb)      # d
        b[:, 2:4] = _fp16_scales(g, nb)      # dmin
    elif fmt == "Q6_K":
        b[:, 208:210] = _fp16_scales(g, nb)  # d (scales[16] at 192 stay uniform int8)
    elif fmt == "MXFP4":
        b[:, 0] = g.integers(118, 127, size=nb, dtype=np.uint8)
    elif fmt == "Q2_K":
        b[:, 80:82] = _fp16_scales(g, nb)    # d
        b[:, 82:84] = _fp16_scales(g, nb)    # dmin
    elif fmt == "Q3_K":
        b[:, 108:110] = _fp16_scales(g, nb)  # d
    else:
        raise ValueError(f"not a weight format: {fmt}")
    return b.reshape(rows, row_bytes(fmt, k))


def expert_bank(fmt: str, n_expert: int, rows: int, k: int, g: np.random.Generator) -> np.ndarray:
    """[E][rows][k/blk] blocks as uint8 [E, rows, row_bytes]."""
    return weights(fmt, n_expert * rows, k, g).reshape(n_expert, rows, row_bytes(fmt, k))


def activations(t: int, k: int, g: np.random.Generator) -> np.ndarray:
    return g.standard_normal(size=(t, k), dtype=np.float32)


def logits(t: int, n_expert: int, g: np.random.Generator) -> np.ndarray:
    return g.standard_normal(size=(t, n_expert), dtype=np.float32)


# Workload shapes (the sizes the pages' workloads are run at).
Q4_0_MATVEC = dict(fmt="Q4_0", act="Q8_1", n=2048, k=2048, t=1)
DENSE_DECODE = dict(formats=("Q8_0", "Q4_K"), act="Q8_1",
                    shapes=((14336, 4096), (4096, 14336)), tokens=(1, 2, 4, 8))
# every weight format against Q8_1 at the first dense-decode shape
DECODE_FORMATS = dict(formats=WEIGHT_FORMATS, act="Q8_1", shapes=((14336, 4096),), tokens=(1, 2, 4, 8))
MOE_Q4K = dict(fmt="Q4_K", act="Q8_1", hidden=2048, inter=768, n_expert=128, topk=8,
               tokens=(1, 2, 3, 4))
GROUPED_KQ = dict(formats=("Q5_K", "Q6_K"), act="Q8_K", tokens=512, hidden=4096,
                  inter=1536, n_expert=128, topk=8)
# the grouped-GEMM workload's shapes as a whole routed layer on the sorted tiles
MOE_KQ_LAYER = dict(fmt="Q5_K", act="Q8_K", hidden=4096, inter=1536, n_expert=128, topk=8, tokens=(512,))
MOE_MXFP4 = dict(fmt="MXFP4", act="Q8_K", hidden=4096, inter=2048, n_expert=256, topk=8,
                 tokens=(1, 2, 3, 4, 5, 32, 128, 512))


def expert_ids(t: int, n_expert: int, topk: int, g: np.random.Generator) -> np.ndarray:
    """[t][topk] int32: for each token, topk distinct experts drawn uniformly
    (the distribution top-k of iid router logits gives)."""
    out = np.empty((t, topk), np.int32)
    for i in range(t):
        out[i] = g.choice(n_expert, size=topk, replace=False)
    return out


def expert_weights(t: int, topk: int, g: np.random.Generator) -> np.ndarray:
    """[t][topk] float32 positive combine weights (a Dirichlet(1) draw per token)."""
    return g.dirichlet(np.ones(topk), size=t).astype(np.float32)
