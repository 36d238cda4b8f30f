"""Helpers of the GPU parity tests: run the library's entry points on a
synthetic case and compare with the oracle.

Inputs come from synth (the same bytes go to both sides); expected values
come from the oracle only.  Tolerances are the layer's contract:
  bf16 tensors: max|d| <= 1e-2 * max|ref| + 1e-3
  fp32 tensors: max|d| <= 1e-5 * max|ref|
  ids, counts, offsets, row_src, route_dst, x_disp: bit-exact
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import routing_dispatch_expert_amd as rde
import synth

DEV = "cuda:0"


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
    d = np.abs(g[fin] - ref[fin]).max()
    tol = 1e-2 * np.abs(ref[fin]).max() + 1e-3
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


def oracle_token_rows(cs, inp_dev, x_host, ids, w, route_dst, tokens, y_shared_host=None):
    """Oracle outputs of the given tokens (float64 [len, H]) from the oracle's
    own routing (ids, w) and dispatch (route_dst), computing only the experts
    those tokens use."""
    cache = {}
    ys = []
    for t in tokens:
        acc_rows = np.zeros((1, cs.H))
        y_rows = []
        for j in range(cs.k):
            if route_dst[t, j] < 0:
                y_rows.append(np.zeros((1, cs.H)))
                continue
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = host_expert(inp_dev, e)
            a, b, sa, sb = cache[e]
            y_rows.append(oracle.expert_rows(x_host[t:t + 1], a, b, cs.act, sa, sb))
        ysh = None if y_shared_host is None else y_shared_host[t:t + 1]
        rd = route_dst[t:t + 1]
        yy = np.concatenate(y_rows, 0)
        # combine with the routed rows renumbered 0..k-1 for this token
        local = np.where(rd >= 0, np.arange(cs.k)[None, :], rd).astype(np.int32)
        acc_rows = oracle.combine(local, w[t:t + 1], yy, ysh)
        ys.append(acc_rows[0])
    return np.stack(ys) if ys else np.zeros((0, cs.H))


def oracle_shared(cs, inp_host, tokens):
    """Oracle shared-expert sum for the given tokens (float64)."""
    if not cs.n_shared:
        return None
    x = inp_host["x"][tokens]
    tot = np.zeros((len(tokens), cs.H))
    for s in range(cs.n_shared):
        tot += oracle.expert_rows(x, inp_host["w13_sh"][s], inp_host["w2_sh"][s], oracle.SWIGLU)
    return tot
