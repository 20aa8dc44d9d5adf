"""Python binding of libft.so (argument marshalling only).

Every step of the path runs in the gfx950 kernels behind the C ABI declared in
include/ft.h; this module turns torch tensors (device memory, current stream)
into pointers and sizes and raises on a non-OK status.  There is no CPU
fallback: if libft.so is missing or cannot load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so libft.so binds to the same HIP runtime as torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libft.so")

TYPES = {"Q4_0": 0, "Q8_0": 1, "Q4_K": 2, "Q5_K": 3, "Q6_K": 4, "MXFP4": 5, "Q8_1": 6, "Q8_K": 7,
         "Q2_K": 8, "Q3_K": 9, "Q4_1": 10, "Q5_0": 11, "Q5_1": 12}
OPS = {"quantize": 0, "dequant": 1, "mmvq": 2, "moe_vec": 3, "grouped": 4, "block_dots": 5}
STATUS = {0: "FT_OK", 1: "FT_ERR_INVALID_ARG", 2: "FT_ERR_UNSUPPORTED", 3: "FT_ERR_SHAPE",
          4: "FT_ERR_ALIGNMENT", 5: "FT_ERR_NO_SCRATCH", 6: "FT_ERR_HIP"}


class FtError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({lib().ft_status_str(status).decode()})")


class _MoeOpts(ctypes.Structure):
    _fields_ = [("route", ctypes.c_int), ("direct_max_t", ctypes.c_int),
                ("tap_g", ctypes.c_void_p), ("tap_u", ctypes.c_void_p), ("tap_h", ctypes.c_void_p),
                ("tap_hq", ctypes.c_void_p), ("tap_down", ctypes.c_void_p), ("in_hq", ctypes.c_void_p),
                ("logits", ctypes.c_void_p), ("ids_out", ctypes.c_void_p), ("w_out", ctypes.c_void_p)]


EXPORTS = {
    "ft_block_elems": (ctypes.c_int, [ctypes.c_int]),
    "ft_block_bytes": (ctypes.c_size_t, [ctypes.c_int]),
    "ft_supported": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "ft_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "ft_version": (ctypes.c_char_p, []),
    "ft_quantize_act": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]),
    "ft_dequant": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_void_p, ctypes.c_void_p]),
    "ft_mul_mat_vec_q": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                        ctypes.c_int64, ctypes.c_void_p]),
    "ft_moe_route": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "ft_moe_sort": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "ft_moe_q_vec": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(_MoeOpts), ctypes.c_void_p]),
    "ft_moe_q_vec_noalloc": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(_MoeOpts),
                                            ctypes.c_void_p]),
    "ft_grouped_gemm_q": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p]),
    "ft_debug_block_dots": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                           ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "ft_debug_ceiling": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_void_p, ctypes.c_void_p]),
    "ft_scratch_reserve": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t]),
    "ft_moe_scratch_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_int64, ctypes.c_int]),
    "ft_grouped_scratch_bytes": (ctypes.c_size_t, [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                    ctypes.c_int, ctypes.c_int]),
    "ft_shutdown": (None, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load libft.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m block_quantized_matvec_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        raise FtError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def block_elems(ty: str) -> int:
    return lib().ft_block_elems(TYPES[ty])


def block_bytes(ty: str) -> int:
    return lib().ft_block_bytes(TYPES[ty])


def row_bytes(ty: str, k: int) -> int:
    return k // block_elems(ty) * block_bytes(ty)


def supported(op: str, w: str, act: str) -> bool:
    return bool(lib().ft_supported(OPS[op], TYPES[w], TYPES[act]))


def version() -> str:
    return lib().ft_version().decode()


def quantize_act(act: str, x: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """x: (rows, k) fp32 on the device; rows may be strided (row stride -> ldx)."""
    if not x.is_cuda:
        raise ValueError("x must be a device tensor")
    rows, k = x.shape
    if x.stride(1) != 1 or (rows > 1 and x.stride(0) < k):
        raise ValueError("x must have unit element stride and rows at least k apart")
    ldx = x.stride(0) if rows > 1 else k
    if out is None:
        out = torch.empty((rows, row_bytes(act, k)), dtype=torch.uint8, device=x.device)
    _check(lib().ft_quantize_act(TYPES[act], _ptr(x), rows, k, ldx, _ptr(out), _stream(stream)), "ft_quantize_act")
    return out


def dequant(w: str, blocks: torch.Tensor, rows: int, k: int, out: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    _dev(blocks, "blocks")
    if out is None:
        out = torch.empty((rows, k), dtype=torch.float32, device=blocks.device)
    _check(lib().ft_dequant(TYPES[w], _ptr(blocks), rows, k, _ptr(out), _stream(stream)), "ft_dequant")
    return out


def mul_mat_vec_q(w: str, W: torch.Tensor, n: int, k: int, act: str, xq: torch.Tensor, t: int,
                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    _dev(W, "W")
    _dev(xq, "xq")
    if out is None:
        out = torch.empty((t, n), dtype=torch.float32, device=W.device)
    _check(lib().ft_mul_mat_vec_q(TYPES[w], _ptr(W), n, k, TYPES[act], _ptr(xq), t, _ptr(out), out.shape[-1],
                                  _stream(stream)), "ft_mul_mat_vec_q")
    return out


def moe_route(logits: torch.Tensor, topk: int, ids: torch.Tensor | None = None, w: torch.Tensor | None = None,
              stream=None):
    _dev(logits, "logits")
    t, e = logits.shape
    if ids is None:
        ids = torch.empty((t, topk), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((t, topk), dtype=torch.float32, device=logits.device)
    _check(lib().ft_moe_route(_ptr(logits), t, e, topk, _ptr(ids), _ptr(w), _stream(stream)), "ft_moe_route")
    return ids, w


def moe_sort(ids: torch.Tensor, n_expert: int, stream=None):
    _dev(ids, "ids")
    t, topk = ids.shape
    counts = torch.empty(n_expert, dtype=torch.int32, device=ids.device)
    offsets = torch.empty(n_expert + 1, dtype=torch.int32, device=ids.device)
    pairs = torch.empty(t * topk, dtype=torch.int32, device=ids.device)
    _check(lib().ft_moe_sort(_ptr(ids), t, topk, n_expert, _ptr(counts), _ptr(offsets), _ptr(pairs),
                             _stream(stream)), "ft_moe_sort")
    return counts, offsets, pairs


def _moe(entry: str, w: str, w_gate, w_up, w_down, n_expert: int, hidden: int, inter: int, act: str,
         x: torch.Tensor, ids, expert_w, out, route: int, taps, in_hq, direct_max_t: int, stream,
         logits=None, topk=None, ids_out=None, w_out=None) -> torch.Tensor:
    for nm, tt in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down), ("x", x), ("ids", ids),
                   ("expert_w", expert_w), ("logits", logits), ("ids_out", ids_out), ("w_out", w_out)):
        if tt is not None:
            _dev(tt, nm)
    t = x.shape[0]
    if topk is None:
        topk = ids.shape[1]
    if out is None:
        out = torch.empty((t, hidden), dtype=torch.float32, device=x.device)
    taps = taps or {}
    opts = _MoeOpts(route, direct_max_t, *(_ptr(taps.get(k)) for k in ("g", "u", "h", "hq", "down")), _ptr(in_hq),
                    _ptr(logits), _ptr(ids_out), _ptr(w_out))
    _check(getattr(lib(), entry)(TYPES[w], _ptr(w_gate), _ptr(w_up), _ptr(w_down), n_expert, hidden, inter,
                                 TYPES[act], _ptr(x), t, _ptr(ids), _ptr(expert_w), topk, _ptr(out),
                                 ctypes.byref(opts), _stream(stream)), entry)
    return out


def moe_q_vec(w: str, w_gate, w_up, w_down, n_expert: int, hidden: int, inter: int, act: str,
              x: torch.Tensor, ids, expert_w, out: torch.Tensor | None = None,
              route: int = 0, taps: dict | None = None, in_hq: torch.Tensor | None = None,
              direct_max_t: int = 0, stream=None, logits=None, topk=None, ids_out=None,
              w_out=None) -> torch.Tensor:
    """taps: optional dict of preallocated device tensors g, u, h, hq, down.  With
    logits ([t][n_expert]) the layer routes itself (ids / expert_w may be None;
    topk is then required) and ids_out / w_out receive the routing."""
    return _moe("ft_moe_q_vec", w, w_gate, w_up, w_down, n_expert, hidden, inter, act, x, ids, expert_w, out,
                route, taps, in_hq, direct_max_t, stream, logits, topk, ids_out, w_out)


def moe_q_vec_noalloc(w: str, w_gate, w_up, w_down, n_expert: int, hidden: int, inter: int, act: str,
                      x: torch.Tensor, ids: torch.Tensor, expert_w: torch.Tensor, out: torch.Tensor | None = None,
                      route: int = 0, taps: dict | None = None, in_hq: torch.Tensor | None = None,
                      direct_max_t: int = 0, stream=None) -> torch.Tensor:
    """As moe_q_vec, with the library's fixed per-GPU scratch instead of the stream's pool."""
    return _moe("ft_moe_q_vec_noalloc", w, w_gate, w_up, w_down, n_expert, hidden, inter, act, x, ids, expert_w,
                out, route, taps, in_hq, direct_max_t, stream)


def grouped_gemm_q(w: str, W: torch.Tensor, n_expert: int, n: int, k: int, act: str, xq: torch.Tensor,
                   x_per_pair: bool, ids: torch.Tensor, out: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    _dev(W, "W")
    _dev(xq, "xq")
    _dev(ids, "ids")
    t, topk = ids.shape
    if out is None:
        out = torch.empty((t * topk, n), dtype=torch.float32, device=W.device)
    _check(lib().ft_grouped_gemm_q(TYPES[w], _ptr(W), n_expert, n, k, TYPES[act], _ptr(xq),
                                   1 if x_per_pair else 0, _ptr(ids), t, topk, _ptr(out), _stream(stream)),
           "ft_grouped_gemm_q")
    return out


def debug_block_dots(w: str, W: torch.Tensor, n: int, k: int, act: str, xq: torch.Tensor, t: int,
                     stream=None) -> torch.Tensor:
    _dev(W, "W")
    _dev(xq, "xq")
    sub = 16 if w in ("Q6_K", "Q2_K", "Q3_K") else 32
    out = torch.empty((t, n, k // sub), dtype=torch.int32, device=W.device)
    _check(lib().ft_debug_block_dots(TYPES[w], _ptr(W), n, k, TYPES[act], _ptr(xq), t, _ptr(out),
                                     _stream(stream)), "ft_debug_block_dots")
    return out


def debug_ceiling(which: str, buf: torch.Tensor | None = None, iters: int = 0, out: torch.Tensor | None = None,
                  stream=None) -> None:
    """Enqueue one measurement microkernel: "stream_read" over buf, "mfma_i8"
    (K = 32), "mfma_i8_k64" or "dot4" for iters rounds.  out: a device int32 scalar
    (allocated if None)."""
    code = {"stream_read": 0, "mfma_i8": 1, "dot4": 2, "mfma_i8_k64": 3}[which]
    dev = buf.device if buf is not None else torch.device("cuda")
    if out is None:
        out = torch.zeros(1, dtype=torch.int32, device=dev)
    nbytes = 0
    if buf is not None:
        _dev(buf, "buf")
        nbytes = buf.numel() * buf.element_size()
    _check(lib().ft_debug_ceiling(code, _ptr(buf) if buf is not None else None, nbytes, iters, _ptr(out),
                                  _stream(stream)), "ft_debug_ceiling")


def scratch_reserve(nbytes: int, stream=None) -> None:
    _check(lib().ft_scratch_reserve(_stream(stream), nbytes), "ft_scratch_reserve")


def moe_scratch_bytes(w: str, act: str, n_expert: int, hidden: int, inter: int, t: int, topk: int) -> int:
    return lib().ft_moe_scratch_bytes(TYPES[w], TYPES[act], n_expert, hidden, inter, t, topk)
