"""ctypes access to the CPU oracle in oracle/moe_oracle.c.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module; the GPU library never does.

Arrays are numpy; bf16 tensors travel as their raw uint16 bits, e4m3 weights
as uint8 codes.  `from_torch` turns a CPU torch tensor into such an array.

Parity status of each oracle function (what pins it, see tests/test_oracle.py):
  route           pinned: +-16 closed form, brute-force top-k, long-double softmax
  dispatch        pinned: bincount / cumsum / stable argsort, inverse identity
  gather_rows     pinned: inverse identity
  expert_rows     pinned: float64 numpy matmul on widened inputs, closed forms
  combine         pinned: identity-expert closed form
  e4m3 decode     pinned: torch float8_e4m3fn over all 256 codes
  round_bf16      pinned: torch float32 -> bfloat16 rounding on exact inputs
"""
from __future__ import annotations

import ctypes as C
import os
import time
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16, E4M3 = 0, 1, 2
SWIGLU, RELU2 = 0, 1

_p = C.c_void_p
_i = C.c_int
_i64 = C.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b  # compile on first use
            _b.build()
        L = C.CDLL(_LIB_PATH)
        L.oracle_bf16_to_double.restype = C.c_double
        L.oracle_bf16_to_double.argtypes = [C.c_uint16]
        L.oracle_e4m3_to_double.restype = C.c_double
        L.oracle_e4m3_to_double.argtypes = [C.c_uint8]
        L.oracle_round_bf16.restype = C.c_double
        L.oracle_round_bf16.argtypes = [C.c_double]
        L.oracle_route.restype = _i
        L.oracle_route.argtypes = [_i, _i, _i, _i, _p, _p, _p]
        L.oracle_route_sigmoid.restype = _i
        L.oracle_route_sigmoid.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p]
        L.oracle_route_scored.restype = _i
        L.oracle_route_scored.argtypes = [_i, _i, _i, _i, _i, C.c_double, _p, _p, _p, _p]
        L.oracle_dispatch.restype = _i64
        L.oracle_dispatch.argtypes = [_i, _i, _i, _i, _p, _p, _p, _p, _i64, _p, _p]
        L.oracle_gather_rows.restype = None
        L.oracle_gather_rows.argtypes = [_i64, _i, _i64, _p, _p, _p]
        L.oracle_expert_rows.restype = _i
        L.oracle_expert_rows.argtypes = [_i, _i, _i, _i, _i, _p, _i, _p, _p, _p, _p, _i, _p]
        L.oracle_combine.restype = None
        L.oracle_combine.argtypes = [_i, _i, _i, _p, _p, _p, _p, _p]
        L.oracle_forward.restype = _i64
        L.oracle_forward.argtypes = [_i] * 13 + [C.c_double] + [_p] * 11 + [_p] * 7
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def from_torch(t):
    """CPU torch tensor -> numpy array in the oracle's storage convention."""
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()


def fmt_of(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3
    raise TypeError(a.dtype)


# ---- element conversions -------------------------------------------------

def bf16_to_double(bits: int) -> float:
    return lib().oracle_bf16_to_double(bits)


def e4m3_to_double(code: int) -> float:
    return lib().oracle_e4m3_to_double(code)


def round_bf16(v: float) -> float:
    return lib().oracle_round_bf16(v)


# ---- steps ---------------------------------------------------------------

SOFTMAX = 0
SIGMOID = 1


def route(logits: np.ndarray, k: int, renormalize: int = 0, score_func: int = SOFTMAX,
          bias: Optional[np.ndarray] = None, route_scale: float = 1.0):
    """ids [T,k] int32 and w [T,k] float64 of softmax (default) or sigmoid
    routing; `bias` is the float32 selection-only correction of sigmoid
    routing, `route_scale` multiplies every weight."""
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        assert bias.shape == (E,)
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    rc = lib().oracle_route_scored(T, E, k, score_func, renormalize, route_scale,
                                   _ptr(logits), _ptr(bias), _ptr(ids), _ptr(w))
    assert rc == 0
    return ids, w


def dispatch(ids: np.ndarray, E: int, C_cap: int):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    T, k = ids.shape
    r_max = min(T * k, E * C_cap)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    row_src = np.zeros(max(r_max, 1), np.int32)
    route_dst = np.zeros((T, k), np.int32)
    bad = np.zeros(max(T, 1), np.uint8)
    n_bad = lib().oracle_dispatch(T, E, k, C_cap, _ptr(ids), _ptr(counts), _ptr(offsets),
                                  _ptr(row_src), r_max, _ptr(route_dst), _ptr(bad))
    assert n_bad >= 0
    return dict(counts=counts, offsets=offsets, row_src=row_src[:r_max],
                route_dst=route_dst, token_bad=bad[:T], n_bad=int(n_bad))


def gather_rows(x: np.ndarray, row_src: np.ndarray, R: int, k: int) -> np.ndarray:
    x = np.ascontiguousarray(x)
    row_src = np.ascontiguousarray(row_src, dtype=np.int32)
    out = np.zeros((max(R, 1),) + x.shape[1:], x.dtype)
    lib().oracle_gather_rows(R, k, x.shape[1] * x.itemsize, _ptr(x), _ptr(row_src), _ptr(out))
    return out[:R]


def expert_rows(x_rows: np.ndarray, w13: np.ndarray, w2: np.ndarray, act: int,
                s13: Optional[np.ndarray] = None, s2: Optional[np.ndarray] = None,
                round_h: Optional[bool] = None) -> np.ndarray:
    """y [n,H] (float64) of one expert applied to n rows."""
    x_rows = np.ascontiguousarray(x_rows)
    w13 = np.ascontiguousarray(w13)
    w2 = np.ascontiguousarray(w2)
    n, H = x_rows.shape
    I = w2.shape[1]
    if round_h is None:
        round_h = fmt_of(x_rows) == BF16
    y = np.zeros((max(n, 1), H), np.float64)
    s13c = None if s13 is None else np.ascontiguousarray(s13, dtype=np.float32)
    s2c = None if s2 is None else np.ascontiguousarray(s2, dtype=np.float32)
    rc = lib().oracle_expert_rows(n, H, I, act, fmt_of(x_rows), _ptr(x_rows), fmt_of(w13),
                                  _ptr(w13), _ptr(w2), _ptr(s13c), _ptr(s2c), int(round_h),
                                  _ptr(y))
    assert rc == 0
    return y[:n]


def combine(route_dst: np.ndarray, w: np.ndarray, y: np.ndarray,
            y_shared: Optional[np.ndarray] = None) -> np.ndarray:
    route_dst = np.ascontiguousarray(route_dst, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float64)
    y = np.ascontiguousarray(y, dtype=np.float64)
    T, k = route_dst.shape
    H = y.shape[1] if y.ndim == 2 and y.shape[0] else (y_shared.shape[1] if y_shared is not None else 0)
    if y.size == 0:
        y = np.zeros((1, max(H, 1)), np.float64)
    ysh = None if y_shared is None else np.ascontiguousarray(y_shared, dtype=np.float64)
    out = np.zeros((T, H), np.float64)
    lib().oracle_combine(T, k, H, _ptr(route_dst), _ptr(w), _ptr(y), _ptr(ysh), _ptr(out))
    return out


def forward(cs, x, logits, w13, w2, s13=None, s2=None, w13_sh=None, w2_sh=None,
            ids_in=None, w_in=None, score_bias=None):
    """The whole layer for case `cs` (a synth.Case); arrays in oracle storage
    convention.  Returns a dict with ids, w, counts, offsets, row_src,
    route_dst, out (float64), n_bad and the wall time in seconds."""
    T, H, E, k, I, Cc = cs.T, cs.H, cs.E, cs.k, cs.I, cs.C
    r_max = min(T * k, E * Cc)
    ids = np.zeros((T, k), np.int32)
    w = np.zeros((T, k), np.float64)
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    row_src = np.zeros(max(r_max, 1), np.int32)
    route_dst = np.zeros((T, k), np.int32)
    out = np.zeros((T, H), np.float64)
    arrs = [np.ascontiguousarray(a) if a is not None else None
            for a in (x, logits, ids_in, w_in, w13, w2, s13, s2, w13_sh, w2_sh, score_bias)]
    x, logits, ids_in, w_in, w13, w2, s13, s2, w13_sh, w2_sh, score_bias = arrs
    if score_bias is not None:
        score_bias = score_bias.astype(np.float32)
    if ids_in is not None:
        ids_in = ids_in.astype(np.int32)
        w_in = w_in.astype(np.float64)
    if logits is not None:
        logits = logits.astype(np.float32)
    t0 = time.perf_counter()
    n_bad = lib().oracle_forward(
        T, H, E, k, I, Cc, cs.act, fmt_of(x), fmt_of(w13), cs.n_shared, cs.I_shared,
        cs.renormalize, cs.score_func, cs.route_scale, _ptr(x), _ptr(logits),
        _ptr(score_bias), _ptr(ids_in), _ptr(w_in), _ptr(w13),
        _ptr(w2), _ptr(s13), _ptr(s2), _ptr(w13_sh), _ptr(w2_sh),
        _ptr(ids), _ptr(w), _ptr(counts), _ptr(offsets), _ptr(row_src), _ptr(route_dst),
        _ptr(out))
    dt = time.perf_counter() - t0
    assert n_bad >= 0, f"oracle_forward failed: {n_bad}"
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, row_src=row_src[:r_max],
                route_dst=route_dst, out=out, n_bad=int(n_bad), seconds=dt)


def inputs_numpy(inp):
    """synth.Inputs (CPU tensors) -> dict of oracle-convention numpy arrays."""
    conv = lambda t: None if t is None else from_torch(t)
    return dict(x=conv(inp.x), logits=conv(inp.logits), w13=conv(inp.w13), w2=conv(inp.w2),
                s13=conv(inp.s13), s2=conv(inp.s2), w13_sh=conv(inp.w13_sh),
                w2_sh=conv(inp.w2_sh), score_bias=conv(inp.score_bias))
