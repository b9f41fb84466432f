"""ctypes binding of libmoe_ffn.so -- argument marshalling only.

Every function here has the name of the C entry point it calls
(include/moe_ffn.h) and forwards device pointers, sizes and the stream; all of
the computation runs in the library's HIP kernels.  Torch tensors are accepted
as the carriers of device memory (``tensor.data_ptr()``), and the current torch
stream is used when no stream is given.  There is no fallback: if the library
is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_ffn.so")

MOE_FFN_OK = 0
MOE_FFN_INVALID_ARG = -1
MOE_FFN_UNSUPPORTED = -2
MOE_FFN_WORKSPACE_TOO_SMALL = -3
MOE_FFN_OUT_OF_MEMORY = -4
MOE_FFN_HIP_ERROR = -5
MOE_FFN_SCRATCH_TOO_SMALL = -6

EXPORTED = ("moe_ffn_weights_create", "moe_ffn_weights_create_fmt", "moe_ffn_weights_destroy", "moe_ffn_weights_dims",
            "moe_ffn_workspace_size", "moe_ffn_workspace_size_for_dims", "moe_ffn_prefill", "moe_ffn_prefill_static", "moe_ffn_prefill_chunked", "moe_ffn_prefill_residual", "moe_ffn_prefill_profiled",
            "moe_ffn_decode",
            "moe_ffn_decode_profiled", "moe_ffn_combine",
            "moe_ffn_quantize", "moe_ffn_residual_rmsnorm", "moe_ffn_dbg_block_sums", "moe_ffn_status_str")


class MoeFfnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_str(status)} ({status})")


class moe_ffn_dims(C.Structure):
    _fields_ = [("d_model", C.c_int32), ("n_experts", C.c_int32), ("top_k", C.c_int32),
                ("d_ffn", C.c_int32), ("d_shared_ffn", C.c_int32), ("norm_topk_prob", C.c_int32)]


class moe_ffn_routing(C.Structure):
    _fields_ = [("topk_ids", C.c_void_p), ("topk_w", C.c_void_p), ("shared_gate", C.c_void_p),
                ("exp_start", C.c_void_p), ("exp_tok_i", C.c_void_p), ("exp_tok_k", C.c_void_p),
                ("xq", C.c_void_p), ("xs", C.c_void_p), ("partial", C.c_void_p)]


_lib = None


def lib():
    """Load libmoe_ffn.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m mixture_experts_ffn_gemm_amd.build`"
                               " (or __graft_entry__.build()) first")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        sig = {
            "moe_ffn_weights_create": [C.POINTER(moe_ffn_dims), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       C.POINTER(vp)],
            "moe_ffn_weights_create_fmt": [C.POINTER(moe_ffn_dims), i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           C.POINTER(vp)],
            "moe_ffn_weights_destroy": [vp],
            "moe_ffn_weights_dims": [vp, C.POINTER(moe_ffn_dims)],
            "moe_ffn_workspace_size": [vp, i32, C.POINTER(sz)],
            "moe_ffn_workspace_size_for_dims": [C.POINTER(moe_ffn_dims), i32, C.POINTER(sz)],
            "moe_ffn_prefill": [vp, vp, i32, vp, vp, sz, C.POINTER(moe_ffn_routing), vp],
            "moe_ffn_prefill_static": [vp, vp, i32, vp, C.POINTER(moe_ffn_routing), vp],
            "moe_ffn_prefill_chunked": [vp, vp, i32, i32, i32, vp, vp, sz, vp],
            "moe_ffn_prefill_residual": [vp, vp, i32, vp, vp, C.c_float, vp, sz, C.POINTER(moe_ffn_routing), vp],
            "moe_ffn_decode": [vp, vp, i32, vp, vp, sz, C.POINTER(moe_ffn_routing), vp],
            "moe_ffn_prefill_profiled": [vp, vp, i32, vp, vp, sz, C.POINTER(moe_ffn_routing), vp,
                                         C.POINTER(vp)],
            "moe_ffn_decode_profiled": [vp, vp, i32, vp, vp, sz, C.POINTER(moe_ffn_routing), vp,
                                        C.POINTER(vp)],
            "moe_ffn_combine": [vp, vp, vp, i32, i32, i32, vp, vp],
            "moe_ffn_quantize": [vp, i64, vp, vp, vp],
            "moe_ffn_residual_rmsnorm": [vp, vp, vp, i32, i32, C.c_float, vp],
            "moe_ffn_dbg_block_sums": [vp, vp, sz, i32, i32, i32, i32, i32, vp, vp, vp, vp],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = C.c_int
        L.moe_ffn_status_str.argtypes = [C.c_int]
        L.moe_ffn_status_str.restype = C.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_ffn_status_str(int(status)).decode()


def _ptr(t) -> Optional[int]:
    """Device address of a tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(fn: str, rc: int) -> None:
    if rc != MOE_FFN_OK:
        raise MoeFfnError(fn, rc)


def make_dims(d_model, n_experts, top_k, d_ffn, d_shared_ffn=0, norm_topk_prob=False) -> moe_ffn_dims:
    return moe_ffn_dims(int(d_model), int(n_experts), int(top_k), int(d_ffn), int(d_shared_ffn),
                        1 if norm_topk_prob else 0)


def moe_ffn_weights_create(dims: moe_ffn_dims, router_w, router_bias, gate_q8, up_q8, down_q8,
                           sh_gate_q8=None, sh_up_q8=None, sh_down_q8=None, sh_gate_vec=None,
                           stream=None) -> int:
    h = C.c_void_p()
    rc = lib().moe_ffn_weights_create(C.byref(dims), _ptr(router_w), _ptr(router_bias), _ptr(gate_q8),
                                      _ptr(up_q8), _ptr(down_q8), _ptr(sh_gate_q8), _ptr(sh_up_q8),
                                      _ptr(sh_down_q8), _ptr(sh_gate_vec), _stream(stream), C.byref(h))
    _check("moe_ffn_weights_create", rc)
    return h.value


FMT_Q8_0 = 0
FMT_Q4_K = 1
FMT_Q3_K = 2
FORMATS = {"q8_0": FMT_Q8_0, "q4_k": FMT_Q4_K, "q3_k": FMT_Q3_K}


def moe_ffn_weights_create_fmt(dims: moe_ffn_dims, fmt: int, router_w, router_bias, gate, up, down,
                               sh_gate=None, sh_up=None, sh_down=None, sh_gate_vec=None, stream=None) -> int:
    """moe_ffn_weights_create with the expert rows in format fmt (FMT_Q8_0, FMT_Q4_K or FMT_Q3_K)."""
    h = C.c_void_p()
    rc = lib().moe_ffn_weights_create_fmt(C.byref(dims), int(fmt), _ptr(router_w), _ptr(router_bias), _ptr(gate),
                                          _ptr(up), _ptr(down), _ptr(sh_gate), _ptr(sh_up), _ptr(sh_down),
                                          _ptr(sh_gate_vec), _stream(stream), C.byref(h))
    _check("moe_ffn_weights_create_fmt", rc)
    return h.value


def moe_ffn_weights_destroy(handle: int) -> None:
    _check("moe_ffn_weights_destroy", lib().moe_ffn_weights_destroy(handle))


def moe_ffn_weights_dims(handle: int) -> moe_ffn_dims:
    dm = moe_ffn_dims()
    _check("moe_ffn_weights_dims", lib().moe_ffn_weights_dims(handle, C.byref(dm)))
    return dm


def moe_ffn_workspace_size(handle: int, max_tokens: int) -> int:
    n = C.c_size_t()
    _check("moe_ffn_workspace_size", lib().moe_ffn_workspace_size(handle, int(max_tokens), C.byref(n)))
    return n.value


def moe_ffn_workspace_size_for_dims(dims: moe_ffn_dims, max_tokens: int) -> int:
    n = C.c_size_t()
    _check("moe_ffn_workspace_size_for_dims",
           lib().moe_ffn_workspace_size_for_dims(C.byref(dims), int(max_tokens), C.byref(n)))
    return n.value


def make_routing(**bufs) -> moe_ffn_routing:
    r = moe_ffn_routing()
    for k, v in bufs.items():
        setattr(r, k, _ptr(v))
    return r


def moe_ffn_prefill(handle: int, x, n_tokens: int, out, ws, ws_bytes: int,
                    routing: Optional[moe_ffn_routing] = None, stream=None) -> None:
    rc = lib().moe_ffn_prefill(handle, _ptr(x), int(n_tokens), _ptr(out), _ptr(ws), int(ws_bytes),
                               C.byref(routing) if routing is not None else None, _stream(stream))
    _check("moe_ffn_prefill", rc)


CHUNK_SERPENTINE = 1


def moe_ffn_prefill_chunked(handle: int, x, n_tokens: int, chunk_tokens: int, flags: int, out, ws, ws_bytes: int,
                            stream=None) -> None:
    """The layer over consecutive chunks of chunk_tokens tokens on one workspace."""
    rc = lib().moe_ffn_prefill_chunked(handle, _ptr(x), int(n_tokens), int(chunk_tokens), int(flags), _ptr(out),
                                       _ptr(ws), int(ws_bytes), _stream(stream))
    _check("moe_ffn_prefill_chunked", rc)


STATIC_SCRATCH_BYTES = 160 << 20


def moe_ffn_prefill_static(handle: int, x, n_tokens: int, out,
                           routing: Optional[moe_ffn_routing] = None, stream=None) -> None:
    """moe_ffn_prefill with the library's static per-device workspace (no allocation)."""
    rc = lib().moe_ffn_prefill_static(handle, _ptr(x), int(n_tokens), _ptr(out),
                                      C.byref(routing) if routing is not None else None, _stream(stream))
    _check("moe_ffn_prefill_static", rc)


def moe_ffn_prefill_residual(handle: int, x, n_tokens: int, h, xn, eps: float, ws, ws_bytes: int,
                             routing: Optional[moe_ffn_routing] = None, stream=None) -> None:
    """The layer inside a residual stack: h += layer(x), xn = RMSNorm(h) (xn may be x)."""
    rc = lib().moe_ffn_prefill_residual(handle, _ptr(x), int(n_tokens), _ptr(h), _ptr(xn), float(eps),
                                        _ptr(ws), int(ws_bytes),
                                        C.byref(routing) if routing is not None else None, _stream(stream))
    _check("moe_ffn_prefill_residual", rc)


N_STAGE_EVENTS = 7
STAGES = ("router_logits", "route", "bucket_quantise", "gateup_swiglu", "down", "combine")


def moe_ffn_prefill_profiled(handle: int, x, n_tokens: int, out, ws, ws_bytes: int, stage_events,
                             routing: Optional[moe_ffn_routing] = None, stream=None) -> None:
    """stage_events: N_STAGE_EVENTS hipEvent_t handles (ints)."""
    ev = (C.c_void_p * N_STAGE_EVENTS)(*stage_events)
    rc = lib().moe_ffn_prefill_profiled(handle, _ptr(x), int(n_tokens), _ptr(out), _ptr(ws), int(ws_bytes),
                                        C.byref(routing) if routing is not None else None,
                                        _stream(stream), ev)
    _check("moe_ffn_prefill_profiled", rc)


def moe_ffn_decode(handle: int, x, n_tokens: int, out, ws, ws_bytes: int,
                   routing: Optional[moe_ffn_routing] = None, stream=None) -> None:
    rc = lib().moe_ffn_decode(handle, _ptr(x), int(n_tokens), _ptr(out), _ptr(ws), int(ws_bytes),
                              C.byref(routing) if routing is not None else None, _stream(stream))
    _check("moe_ffn_decode", rc)


N_DECODE_STAGE_EVENTS = 5
DECODE_STAGES = ("router_quantise", "route_gateup_swiglu", "down", "combine")


def moe_ffn_decode_profiled(handle: int, x, n_tokens: int, out, ws, ws_bytes: int, stage_events,
                            routing: Optional[moe_ffn_routing] = None, stream=None) -> None:
    """stage_events: N_DECODE_STAGE_EVENTS hipEvent_t handles (ints)."""
    ev = (C.c_void_p * N_DECODE_STAGE_EVENTS)(*stage_events)
    rc = lib().moe_ffn_decode_profiled(handle, _ptr(x), int(n_tokens), _ptr(out), _ptr(ws), int(ws_bytes),
                                       C.byref(routing) if routing is not None else None,
                                       _stream(stream), ev)
    _check("moe_ffn_decode_profiled", rc)


def moe_ffn_combine(partial, topk_w, shared_gate, n: int, k: int, d: int, out, stream=None) -> None:
    rc = lib().moe_ffn_combine(_ptr(partial), _ptr(topk_w), _ptr(shared_gate), int(n), int(k), int(d),
                               _ptr(out), _stream(stream))
    _check("moe_ffn_combine", rc)


def moe_ffn_quantize(v, n_values: int, q, scales, stream=None) -> None:
    rc = lib().moe_ffn_quantize(_ptr(v), int(n_values), _ptr(q), _ptr(scales), _stream(stream))
    _check("moe_ffn_quantize", rc)


def moe_ffn_residual_rmsnorm(h, y, xn, n: int, d: int, eps: float, stream=None) -> None:
    rc = lib().moe_ffn_residual_rmsnorm(_ptr(h), _ptr(y), _ptr(xn), int(n), int(d), float(eps),
                                        _stream(stream))
    _check("moe_ffn_residual_rmsnorm", rc)


def moe_ffn_dbg_block_sums(handle: int, ws, ws_bytes: int, n_tokens: int, gemm: int, tile: int, strip: int,
                           kblock: int, sums, a_codes, info, stream=None) -> None:
    """The exact int32 block sums of one k-block of one (tile, strip) of the
    gate/up (gemm=0) or down (gemm=1) GEMM of the last prefill on ws."""
    rc = lib().moe_ffn_dbg_block_sums(handle, _ptr(ws), int(ws_bytes), int(n_tokens), int(gemm), int(tile),
                                      int(strip), int(kblock), _ptr(sums), _ptr(a_codes), _ptr(info),
                                      _stream(stream))
    _check("moe_ffn_dbg_block_sums", rc)


def moe_ffn_status_str(status: int) -> str:
    return status_str(status)
