"""ctypes binding of the CPU oracle (oracle/libmoe_oracle.so).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg import this module.  It never touches the HIP library.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import numpy as np

from . import build as _build

_lib = None


class OraDims(C.Structure):
    _fields_ = [("d", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("ffn", C.c_int32), ("shared_ffn", C.c_int32), ("norm_topk_prob", C.c_int32),
                ("weight_format", C.c_int32)]


FMT = {"q8_0": 0, "q4_k": 1, "q3_k": 2}


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = C.CDLL(_build.LIB)
        vp, i32, i64, dbl = C.c_void_p, C.c_int32, C.c_int64, C.c_double
        sig = {
            "ora_half_to_float": (None, [vp, vp, i64]),
            "ora_float_to_half": (None, [vp, vp, i64]),
            "ora_router_logits": (None, [vp, i32, i32, vp, vp, i32, vp]),
            "ora_topk": (None, [vp, i32, i32, i32, vp]),
            "ora_route_weights": (None, [vp, vp, i32, i32, i32, i32, vp]),
            "ora_shared_gate": (None, [vp, i32, i32, vp, vp]),
            "ora_csr": (None, [vp, i32, i32, i32, i32, vp, vp, vp]),
            "ora_quantize_q8": (None, [vp, i64, vp, vp]),
            "ora_q8_dot": (dbl, [vp, vp, vp, i32]),
            "ora_q8_block_sums": (None, [vp, i32, vp, i32, i64, i32, vp]),
            "ora_q4k_dequant": (None, [vp, i32, vp]),
            "ora_q4k_dot": (dbl, [vp, vp, vp, i32]),
            "ora_q3k_dequant": (None, [vp, i32, vp]),
            "ora_q3k_dot": (dbl, [vp, vp, vp, i32]),
            "ora_expert_ffn_fmt": (None, [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "ora_expert_ffn": (None, [i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "ora_moe_tokens": (i32, [C.POINTER(OraDims), vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, i32, vp, vp, vp, vp, vp]),
            "ora_moe_grouped": (i32, [C.POINTER(OraDims), vp, i32, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp]),
            "ora_combine_f32": (None, [vp, vp, vp, i32, i32, i32, i32, vp]),
            "ora_rmsnorm": (None, [vp, i32, i32, dbl, vp]),
            "ora_num_threads": (i32, []),
            "ora_set_num_threads": (None, [i32]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def dims_of(shape, fmt: str = "q8_0") -> OraDims:
    return OraDims(shape.d, shape.n_experts, shape.top_k, shape.ffn, shape.shared_ffn,
                   1 if shape.norm_topk_prob else 0, FMT[fmt])


def half_to_float(h: np.ndarray) -> np.ndarray:
    h = _c(h, np.uint16)
    f = np.empty(h.shape, np.float32)
    lib().ora_half_to_float(_p(h), _p(f), h.size)
    return f


def float_to_half(f: np.ndarray) -> np.ndarray:
    f = _c(f, np.float32)
    h = np.empty(f.shape, np.uint16)
    lib().ora_float_to_half(_p(f), _p(h), f.size)
    return h


def router_logits(x, w, bias=None) -> np.ndarray:
    x = _c(x, np.float32)
    w = _c(w, np.float32)
    n, d = x.shape
    E = w.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((n, E), np.float32)
    lib().ora_router_logits(_p(x), n, d, _p(w), _p(b), E, _p(out))
    return out


def topk(logits, k) -> np.ndarray:
    l = _c(logits, np.float32)
    n, E = l.shape
    ids = np.empty((n, k), np.int32)
    lib().ora_topk(_p(l), n, E, k, _p(ids))
    return ids


def route_weights(logits, ids, norm: bool) -> np.ndarray:
    l = _c(logits, np.float32)
    ids = _c(ids, np.int32)
    n, E = l.shape
    k = ids.shape[1]
    w = np.empty((n, k), np.float64)
    lib().ora_route_weights(_p(l), _p(ids), n, E, k, 1 if norm else 0, _p(w))
    return w


def shared_gate(x, g) -> np.ndarray:
    x = _c(x, np.float32)
    g = _c(g, np.float32)
    n, d = x.shape
    gs = np.empty(n, np.float64)
    lib().ora_shared_gate(_p(x), n, d, _p(g), _p(gs))
    return gs


def csr(ids, n_experts: int, has_shared: bool = False):
    ids = _c(ids, np.int32)
    n, k = ids.shape
    hs = 1 if has_shared else 0
    start = np.empty(n_experts + 1 + hs, np.int32)
    ti = np.empty(n * (k + hs), np.int32)
    tk = np.empty(n * (k + hs), np.int32)
    lib().ora_csr(_p(ids), n, n_experts, k, hs, _p(start), _p(ti), _p(tk))
    return start, ti, tk


def quantize_q8(v):
    v = _c(v, np.float32)
    assert v.size % 32 == 0
    q = np.empty(v.shape, np.int8)
    s = np.empty(v.shape[:-1] + (v.shape[-1] // 32,), np.uint16)
    lib().ora_quantize_q8(_p(v), v.size, _p(q), _p(s))
    return q, s


def q8_dot(qa, sa16, w_row) -> float:
    qa = _c(qa, np.int8)
    sa16 = _c(sa16, np.uint16)
    w_row = _c(w_row, np.uint8)
    return lib().ora_q8_dot(_p(qa), _p(sa16), _p(w_row), qa.size // 32)


def q8_block_sums(qa, w_rows, kblock: int) -> np.ndarray:
    """Exact int32 sums of block `kblock`: qa int8 [m][32] codes against the
    Q8_0 weight rows w_rows (uint8 [n][row_bytes]) -> int32 [m][n]."""
    qa = _c(qa, np.int8).reshape(-1, 32)
    w_rows = _c(w_rows, np.uint8)
    m, n = qa.shape[0], w_rows.shape[0]
    assert 0 <= kblock and (kblock + 1) * 34 <= w_rows.shape[1]
    out = np.empty((m, n), np.int32)
    lib().ora_q8_block_sums(_p(qa), m, _p(w_rows), n, w_rows.shape[1], int(kblock), _p(out))
    return out


def q4k_dequant(w_rows, in_dim: int) -> np.ndarray:
    """Q4_K rows (uint8 [rows][in_dim/256*144]) -> fp64 [rows][in_dim]."""
    w_rows = _c(np.atleast_2d(w_rows), np.uint8)
    out = np.empty((w_rows.shape[0], in_dim), np.float64)
    for r in range(w_rows.shape[0]):
        lib().ora_q4k_dequant(_p(w_rows[r]), in_dim, out[r].ctypes.data_as(C.c_void_p))
    return out


def q4k_dot(qa, sa16, w_row) -> float:
    qa = _c(qa, np.int8)
    sa16 = _c(sa16, np.uint16)
    w_row = _c(w_row, np.uint8)
    return lib().ora_q4k_dot(_p(qa), _p(sa16), _p(w_row), qa.size)


def q3k_dequant(w_rows, in_dim: int) -> np.ndarray:
    """Q3_K rows (uint8 [rows][in_dim/256*110]) -> fp64 [rows][in_dim]."""
    w_rows = _c(np.atleast_2d(w_rows), np.uint8)
    out = np.empty((w_rows.shape[0], in_dim), np.float64)
    for r in range(w_rows.shape[0]):
        lib().ora_q3k_dequant(_p(w_rows[r]), in_dim, out[r].ctypes.data_as(C.c_void_p))
    return out


def q3k_dot(qa, sa16, w_row) -> float:
    qa = _c(qa, np.int8)
    sa16 = _c(sa16, np.uint16)
    w_row = _c(w_row, np.uint8)
    return lib().ora_q3k_dot(_p(qa), _p(sa16), _p(w_row), qa.size)


def expert_ffn(d, ffn, xq, xs, gate, up, down, fmt: str = "q8_0"):
    xq = _c(xq, np.int8)
    xs = _c(xs, np.uint16)
    gate = _c(gate, np.uint8)
    up = _c(up, np.uint8)
    down = _c(down, np.uint8)
    y = np.empty(d, np.float64)
    hq = np.empty(ffn, np.int8)
    hs = np.empty(ffn // 32, np.uint16)
    h = np.empty(ffn, np.float64)
    lib().ora_expert_ffn_fmt(FMT[fmt], d, ffn, _p(xq), _p(xs), _p(gate), _p(up), _p(down), _p(y), _p(hq),
                             _p(hs), _p(h))
    return y, hq, hs, h


def _weights_args(lw):
    return [_c(lw.router_w, np.float32),
            None if lw.router_bias is None else _c(lw.router_bias, np.float32),
            _c(lw.gate_q8, np.uint8), _c(lw.up_q8, np.uint8), _c(lw.down_q8, np.uint8),
            None if lw.sh_gate_q8 is None else _c(lw.sh_gate_q8, np.uint8),
            None if lw.sh_up_q8 is None else _c(lw.sh_up_q8, np.uint8),
            None if lw.sh_down_q8 is None else _c(lw.sh_down_q8, np.uint8),
            None if lw.sh_gate_vec is None else _c(lw.sh_gate_vec, np.float32)]


def moe_tokens(lw, x, tokens: Optional[Sequence[int]] = None, want_partial: bool = False):
    """Per-token loop over `tokens` (all when None).  Returns a dict with out
    [n][d] fp64 and ids/w/gs (+ partial [n][k+s][d])."""
    s = lw.shape
    x = _c(x, np.float32)
    n_tokens = x.shape[0]
    tl = np.arange(n_tokens, dtype=np.int32) if tokens is None else _c(tokens, np.int32)
    n = tl.size
    kk = s.top_k + (1 if s.shared_ffn else 0)
    out = np.empty((n, s.d), np.float64)
    part = np.empty((n, kk, s.d), np.float64) if want_partial else None
    ids = np.empty((n, s.top_k), np.int32)
    w = np.empty((n, s.top_k), np.float64)
    gs = np.empty(n, np.float64)
    dm = dims_of(s, lw.fmt)
    args = _weights_args(lw)
    rc = lib().ora_moe_tokens(C.byref(dm), _p(x), n_tokens, *[_p(a) for a in args], _p(tl), n,
                              _p(out), _p(part), _p(ids), _p(w), _p(gs))
    if rc != 0:
        raise ValueError("ora_moe_tokens rejected its arguments")
    res = {"out": out, "ids": ids, "w": w, "gs": gs, "tokens": tl}
    if want_partial:
        res["partial"] = part
    return res


def moe_grouped(lw, x) -> np.ndarray:
    s = lw.shape
    x = _c(x, np.float32)
    out = np.empty((x.shape[0], s.d), np.float64)
    dm = dims_of(s, lw.fmt)
    args = _weights_args(lw)
    rc = lib().ora_moe_grouped(C.byref(dm), _p(x), x.shape[0], *[_p(a) for a in args], _p(out))
    if rc != 0:
        raise ValueError("ora_moe_grouped rejected its arguments")
    return out


def combine_f32(partial, w, gs=None) -> np.ndarray:
    partial = _c(partial, np.float32)
    w = _c(w, np.float32)
    n, kk, d = partial.shape
    k = w.shape[1]
    g = None if gs is None else _c(gs, np.float32)
    out = np.empty((n, d), np.float32)
    lib().ora_combine_f32(_p(partial), _p(w), _p(g), n, k, kk, d, _p(out))
    return out


def rmsnorm(x, eps: float = 1e-5) -> np.ndarray:
    x = _c(x, np.float32)
    n, d = x.shape
    out = np.empty((n, d), np.float64)
    lib().ora_rmsnorm(_p(x), n, d, eps, _p(out))
    return out


def routing(lw, x):
    """Router, top-k, weights, shared gate, quantised activations and CSR for
    all tokens, each from its own oracle step."""
    s = lw.shape
    logits = router_logits(x, lw.router_w, lw.router_bias)
    ids = topk(logits, s.top_k)
    w = route_weights(logits, ids, s.norm_topk_prob)
    gs = shared_gate(x, lw.sh_gate_vec) if s.shared_ffn else None
    xq, xs = quantize_q8(x)
    start, ti, tk = csr(ids, s.n_experts, bool(s.shared_ffn))
    return {"logits": logits, "ids": ids, "w": w, "gs": gs, "xq": xq, "xs": xs,
            "exp_start": start, "tok_i": ti, "tok_k": tk}


def num_threads() -> int:
    return int(lib().ora_num_threads())


def set_num_threads(n: int) -> None:
    lib().ora_set_num_threads(int(n))
