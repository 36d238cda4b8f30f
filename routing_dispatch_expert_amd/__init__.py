"""Python binding of the gfx950 MoE layer library (librde_moe.so).

Argument marshalling only: every function here has the name of a C entry
point of include/moe.h, turns torch tensors into device pointers and the
current torch stream into a hipStream_t, calls the library and raises
MoeError on a non-zero status.  All computation runs in the library's HIP
kernels; there is no fallback path: when the library is missing, every call
raises.  PyTorch provides device memory and streams only.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librde_moe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_E4M3 = 0, 1, 2
MOE_SWIGLU, MOE_RELU2 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID = 0, 1

# every symbol the header declares
EXPORTS = ("moe_workspace_bytes", "moe_workspace_init", "moe_route", "moe_dispatch",
           "moe_expert_ffn", "moe_shared_ffn", "moe_combine", "moe_forward", "moe_forward_static",
           "moe_error", "moe_status_string")
MOE_STATIC_SCRATCH_BYTES = 32 << 20


class moe_problem(C.Structure):
    _fields_ = [(n, C.c_int32) for n in ("T", "H", "E", "k", "I", "C", "n_shared", "I_shared",
                                         "act_dtype", "w_dtype", "act", "renormalize",
                                         "score_func")] + [("route_scale", C.c_float)]


MOE_N_STAGES = 8
STAGES = ("begin", "route", "count", "scatter", "gemm1", "gemm2", "shared", "combine")


class moe_meta(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("ids", "w", "counts", "offsets", "row_src", "route_dst",
                                          "stage_events")]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({_status_string(status)})")


_lib = None


def lib() -> C.CDLL:
    """The loaded library; raises when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python routing_dispatch_expert_amd/build.py` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        P, S, i32 = C.c_void_p, C.c_size_t, C.c_int32
        pp = C.POINTER(moe_problem)
        sig = {
            "moe_workspace_bytes": [pp, C.POINTER(C.c_size_t)],
            "moe_workspace_init": [P, S, P],
            "moe_route": [pp, P, P, P, P, P, S, P],
            "moe_dispatch": [pp, P, P, P, P, P, P, P, P, S, P],
            "moe_expert_ffn": [pp, P, P, P, P, P, P, P, P, S, P],
            "moe_shared_ffn": [pp, P, P, P, P, P, S, P],
            "moe_combine": [pp, P, P, P, P, P, P, S, P],
            "moe_forward": [pp, P, P, P, P, P, P, P, P, P, P, P, P, C.POINTER(moe_meta), P, S, P],
            "moe_forward_static": [pp, P, P, P, P, P, P, P, P, P, P, P, P, C.POINTER(moe_meta), P],
            "moe_error": [P, S, P, C.POINTER(i32)],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = i32
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = C.c_char_p
        _lib = L
    return _lib


def _status_string(s: int) -> str:
    try:
        return lib().moe_status_string(s).decode()
    except Exception:  # library missing
        return "?"


def make_problem(T, H, E, k, I, C_cap, n_shared=0, I_shared=0, act_dtype=MOE_BF16,
                 w_dtype=MOE_BF16, act=MOE_SWIGLU, renormalize=0, score_func=MOE_SOFTMAX,
                 route_scale=1.0) -> moe_problem:
    return moe_problem(T, H, E, k, I, C_cap, n_shared, I_shared, act_dtype, w_dtype, act,
                       renormalize, score_func, route_scale)


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, st: int):
    if st != MOE_OK:
        raise MoeError(fn, st)


# ---- entry points -------------------------------------------------------------

def moe_workspace_bytes(p: moe_problem) -> int:
    n = C.c_size_t(0)
    _check("moe_workspace_bytes", lib().moe_workspace_bytes(C.byref(p), C.byref(n)))
    return n.value


def moe_workspace_init(ws, stream=None):
    _check("moe_workspace_init", lib().moe_workspace_init(_p(ws), ws.numel(), _stream(stream)))


def moe_route(p, logits, score_bias, ids, w, ws, stream=None):
    _check("moe_route", lib().moe_route(C.byref(p), _p(logits), _p(score_bias), _p(ids), _p(w),
                                        _p(ws), ws.numel(), _stream(stream)))


def moe_dispatch(p, x, ids, counts, offsets, row_src, route_dst, x_disp, ws, stream=None):
    _check("moe_dispatch", lib().moe_dispatch(C.byref(p), _p(x), _p(ids), _p(counts),
                                              _p(offsets), _p(row_src), _p(route_dst),
                                              _p(x_disp), _p(ws), ws.numel(), _stream(stream)))


def moe_expert_ffn(p, x_disp, offsets, w13, w2, s13, s2, y_disp, ws, stream=None):
    _check("moe_expert_ffn", lib().moe_expert_ffn(C.byref(p), _p(x_disp), _p(offsets), _p(w13),
                                                  _p(w2), _p(s13), _p(s2), _p(y_disp), _p(ws),
                                                  ws.numel(), _stream(stream)))


def moe_shared_ffn(p, x, w13_sh, w2_sh, y_shared, ws, stream=None):
    _check("moe_shared_ffn", lib().moe_shared_ffn(C.byref(p), _p(x), _p(w13_sh), _p(w2_sh),
                                                  _p(y_shared), _p(ws), ws.numel(),
                                                  _stream(stream)))


def moe_combine(p, y_disp, route_dst, w, y_shared, out, ws, stream=None):
    _check("moe_combine", lib().moe_combine(C.byref(p), _p(y_disp), _p(route_dst), _p(w),
                                            _p(y_shared), _p(out), _p(ws), ws.numel(),
                                            _stream(stream)))


def _meta(meta):
    """moe_meta from a dict (see moe_forward); the event array is returned
    too, to be kept alive across the call."""
    if not meta:
        return None, None
    vals = [_p(meta.get(n)) for n, _ in moe_meta._fields_[:6]]
    evs = meta.get("stage_events")
    keep = None
    if evs is not None:
        assert len(evs) == MOE_N_STAGES
        keep = (C.c_void_p * MOE_N_STAGES)(*[None if e is None else e.cuda_event for e in evs])
    return moe_meta(*vals, C.cast(keep, C.c_void_p) if keep is not None else None), keep


def moe_forward(p, x, logits, score_bias, ids_in, w_in, w13, w2, s13, s2, w13_sh, w2_sh, out,
                meta, ws, stream=None):
    """`meta` is None or a dict with any of ids, w, counts, offsets, row_src,
    route_dst (device tensors receiving the metadata) and stage_events (a
    list of MOE_N_STAGES torch.cuda.Event or None)."""
    m, keep = _meta(meta)
    _check("moe_forward", lib().moe_forward(
        C.byref(p), _p(x), _p(logits), _p(score_bias), _p(ids_in), _p(w_in), _p(w13), _p(w2),
        _p(s13), _p(s2),
        _p(w13_sh), _p(w2_sh), _p(out), C.byref(m) if m is not None else None, _p(ws),
        ws.numel(), _stream(stream)))
    del keep


def moe_forward_static(p, x, logits, score_bias, ids_in, w_in, w13, w2, s13, s2, w13_sh, w2_sh,
                       out, meta, stream=None):
    """moe_forward without a workspace argument: the library's own
    per-device array of MOE_STATIC_SCRATCH_BYTES serves as workspace."""
    m, keep = _meta(meta)
    _check("moe_forward_static", lib().moe_forward_static(
        C.byref(p), _p(x), _p(logits), _p(score_bias), _p(ids_in), _p(w_in), _p(w13), _p(w2),
        _p(s13), _p(s2), _p(w13_sh), _p(w2_sh), _p(out), C.byref(m) if m is not None else None,
        _stream(stream)))
    del keep


def moe_error(ws, stream=None) -> int:
    n = C.c_int32(0)
    _check("moe_error", lib().moe_error(_p(ws), ws.numel(), _stream(stream), C.byref(n)))
    return n.value


def moe_status_string(s: int) -> str:
    return lib().moe_status_string(s).decode()
