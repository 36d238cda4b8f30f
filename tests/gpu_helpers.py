"""Helpers of the GPU parity tests: run the library's entry points on a
synthetic case and compare with the oracle.

Inputs come from synth (the same bytes go to both sides); expected values
come from the oracle only.  Tolerances are the layer's contract:
  bf16 tensors: max|d| <= 1e-2 * max|ref| + 1e-3
  fp32 tensors: max|d| <= 1e-5 * max|ref|
  ids, counts, offsets, row_src, route_dst, x_disp: bit-exact

A bf16 comparison is only accepted where it can fail: with outputs far below
the 1e-3 floor an all-zero result would pass, so `assert_bf16_close` refuses
any reference whose floor exceeds 2.5 % of max|ref| (then a result off by 5 %
of max|ref| always fails).  Parity cases therefore run on `synth.unit_scale`
inputs, whose outputs are O(1).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import routing_dispatch_expert_amd as rde
import synth

DEV = "cuda:0"
BF16_REL, BF16_FLOOR = 1e-2, 1e-3
# largest accepted floor / max|ref|: a 5 % error then exceeds 1 % + 2.5 %
MAX_FLOOR_FRACTION = 0.025
ORACLE_THREADS = 12


def parity_case(name: str, **over) -> synth.Case:
    """A named workload (optionally reduced) at the unit value scale."""
    return synth.unit_scale(synth.case(name, **over))


class VacuousComparison(AssertionError):
    """The reference is so small that the tolerance floor alone covers it."""


def bf16_tolerance(ref: np.ndarray) -> float:
    """max|d| allowed for a bf16 tensor: 1e-2 * max|ref| + 1e-3, refused
    (VacuousComparison) where the 1e-3 floor exceeds 2.5 % of max|ref|."""
    ref = np.asarray(ref, np.float64)
    fin = np.isfinite(ref)
    m = float(np.abs(ref[fin]).max()) if fin.any() else 0.0
    if BF16_FLOOR > MAX_FLOOR_FRACTION * m:
        raise VacuousComparison(f"max|ref| = {m:.3e}: the floor {BF16_FLOOR:g} alone would "
                                f"accept an all-zero result")
    return BF16_REL * m + BF16_FLOOR


def problem(cs: synth.Case) -> rde.moe_problem:
    return rde.make_problem(cs.T, cs.H, cs.E, cs.k, cs.I, cs.C, cs.n_shared, cs.I_shared,
                            act_dtype=cs.act_fmt, w_dtype=cs.w_fmt, act=cs.act,
                            renormalize=cs.renormalize, score_func=cs.score_func,
                            route_scale=cs.route_scale)


def workspace(p) -> torch.Tensor:
    n = rde.moe_workspace_bytes(p)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=DEV)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    rde.moe_workspace_init(ws)
    return ws


def act_dtype(cs):
    return torch.float32 if cs.act_fmt == synth.FMT_F32 else torch.bfloat16


def r_max(cs):
    return min(cs.T * cs.k, cs.E * cs.C)


def assert_bf16_close(got: torch.Tensor, ref: np.ndarray, what=""):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g) == np.isfinite(ref)), f"{what}: finiteness differs"
    fin = np.isfinite(ref)
    if not fin.any():
        return
    tol = bf16_tolerance(ref)
    d = np.abs(g[fin] - ref[fin]).max()
    assert d <= tol, f"{what}: max|d| = {d:.3e} > {tol:.3e}"


def assert_f32_close(got: torch.Tensor, ref: np.ndarray, what="", rel=1e-5):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isnan(g) == np.isnan(ref)), f"{what}: NaN pattern differs"
    fin = ~np.isnan(ref)
    if not fin.any():
        return
    d = np.abs(g[fin] - ref[fin]).max()
    tol = rel * np.abs(ref[fin]).max()
    assert d <= tol, f"{what}: max|d| = {d:.3e} > {tol:.3e}"


def assert_close(cs, got, ref, what=""):
    if cs.act_fmt == synth.FMT_F32:
        assert_f32_close(got, ref, what)
    else:
        assert_bf16_close(got, ref, what)


def np_i32(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy().astype(np.int32)


def host_expert(inp_dev: synth.Inputs, e: int):
    """Host (oracle-convention) copies of one expert's weights."""
    cv = oracle.from_torch
    s13 = None if inp_dev.s13 is None else cv(inp_dev.s13[e])
    s2 = None if inp_dev.s2 is None else cv(inp_dev.s2[e])
    return cv(inp_dev.w13[e]), cv(inp_dev.w2[e]), s13, s2


def parallel_map(fn, items):
    """fn over items on a few host threads (the oracle's C calls release the
    GIL; each call is itself single-threaded)."""
    with ThreadPoolExecutor(ORACLE_THREADS) as ex:
        return list(ex.map(fn, items))


def oracle_token_rows(cs, inp_dev, x_host, ids, w, route_dst, tokens, y_shared_host=None):
    """Oracle outputs of the given tokens (float64 [len, H]) from the oracle's
    own routing (ids, w) and dispatch (route_dst), computing only the experts
    those tokens use: every expert's rows in one oracle call, experts on
    several host threads."""
    tokens = list(tokens)
    uses = {}
    for i, t in enumerate(tokens):
        for j in range(cs.k):
            if route_dst[t, j] >= 0:
                uses.setdefault(int(ids[t, j]), []).append((i, j))
    y = np.zeros((len(tokens), cs.k, cs.H))

    def run(e):
        a, b, sa, sb = host_expert(inp_dev, e)
        rows = [tokens[i] for i, _ in uses[e]]
        return e, oracle.expert_rows(x_host[rows], a, b, cs.act, sa, sb)

    for e, ye in parallel_map(run, sorted(uses)):
        for n, (i, j) in enumerate(uses[e]):
            y[i, j] = ye[n]
    out = np.zeros((len(tokens), cs.H))
    for i, t in enumerate(tokens):
        rd = route_dst[t:t + 1]
        # combine with the routed rows renumbered 0..k-1 for this token
        local = np.where(rd >= 0, np.arange(cs.k)[None, :], rd).astype(np.int32)
        ysh = None if y_shared_host is None else y_shared_host[i:i + 1]
        out[i] = oracle.combine(local, w[t:t + 1], y[i], ysh)[0]
    return out


def oracle_shared(cs, inp_host, tokens):
    """Oracle shared-expert sum for the given tokens (float64)."""
    if not cs.n_shared:
        return None
    x = inp_host["x"][tokens]
    tot = np.zeros((len(tokens), cs.H))
    for s in range(cs.n_shared):
        tot += oracle.expert_rows(x, inp_host["w13_sh"][s], inp_host["w2_sh"][s], oracle.SWIGLU)
    return tot
