"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Batches with at most 12 routes per expert on average run the slot-indexed
expert GEMMs; the others run the tiled grouped GEMM; both are covered.

Each test prints the case it runs before touching the GPU.  Small cases are
compared element by element against the full oracle; they span several
m-tiles (256 rows for bf16, 64 for float32) with a ragged last tile, several
k-tiles and n-tiles.  The
full-size workloads (the pages' shapes) are compared bit-exactly on all
routing / dispatch metadata and on sampled token rows for the FFN outputs.

Outputs are compared at the unit value scale (synth.unit_scale: x ~ N(0,1),
weights N(0, 1/K)), where every output tensor is O(1) and the bf16 contract
max|d| <= 1e-2 max|ref| + 1e-3 is decided by the kernel's error, not by the
floor; the comparison helper refuses references small enough for an all-zero
result to pass.  Routing and dispatch do not depend on the value scale.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import routing_dispatch_expert_amd as rde
import synth
from gpu_helpers import (DEV, act_dtype, assert_bf16_close, assert_close, assert_f32_close,
                         host_expert, np_i32, oracle_shared, oracle_token_rows, parallel_map,
                         parity_case, problem, r_max, workspace)

pytestmark = pytest.mark.gpu

# Small cases: the whole oracle finishes in seconds.
SMALL = {
    "tiny_fp32": ("tiny_fp32", {}),
    "multi_tile_swiglu": ("prefill_T256", dict(T=600, H=256, E=4, k=2, I=256, C=600)),
    "ragged_skew_capacity": ("skewed_bf16", dict(T=777, H=256, E=16, k=4, I=128, C=100)),
    # experts of 280, 171, 92, 68 (heavy tiles), 52 (three-stage ring with a
    # 64-row A part) and at most 32 rows (three-stage ring): every bf16 layout,
    # their transitions, and the mixed tile order of light and heavy experts
    "skewed_all_layouts": ("skewed_bf16", dict(T=400, H=512, E=16, k=2, I=256, C=400)),
    "relu2_small": ("relu2_distinct_R8", dict(H=256, I=256)),
    "decode_shared_small": ("decode_T8", dict(T=37, H=256, I=128, I_shared=256, C=37)),
    "fp8_small": ("skewed_fp8", dict(T=300, H=256, E=8, I=256, C=96)),
    # e4m3 down projection with K = 128 (two k-tiles): the weight scales
    # staged in LDS at a tile's start are published by its second k-tile
    "fp8_k128": ("skewed_fp8", dict(T=300, H=256, E=8, I=128, C=96)),
    # e4m3 weights with K >= 640 in both projections (64-wide k-tiles: the
    # combine epilogue's routes staged in LDS) over two m-tiles per expert,
    # the second ragged, and a ragged last n-tile
    "fp8_k640_two_mtiles": ("skewed_fp8", dict(T=600, H=768, E=4, k=2, I=640, C=600)),
    "k1_e1": ("prefill_T256", dict(T=130, H=128, E=1, k=1, I=128, C=130)),
    # routes of one count block placed by that block, with capacity drops
    "one_block_capacity": ("prefill_T256", dict(T=200, H=256, E=8, k=4, I=128, C=50)),
    "fp32_relu2_renorm": ("tiny_fp32", dict(act=synth.ACT_RELU2, renormalize=1, T=100, C=40)),
    # hidden / intermediate not multiples of the 256-column tile
    "ragged_n_relu2": ("relu2_distinct_R8", dict(H=384, I=384)),
    "ragged_n_swiglu": ("prefill_T256", dict(T=300, H=384, E=4, k=2, I=384, C=300)),
    # down projection with K >= 320 (the combine epilogue's routes staged in LDS)
    # over two m-tiles per expert, the second ragged
    "multi_tile_k384": ("prefill_T256", dict(T=600, H=256, E=4, k=2, I=384, C=600)),
    # decode-shaped (few rows per expert): slot-indexed expert GEMMs
    "decode_fp8": ("skewed_fp8", dict(T=16, H=256, E=32, k=4, I=256, C=16)),
    "decode_rows_over_32": ("skewed_bf16", dict(T=180, H=256, E=32, k=2, I=128, C=180)),
    # decode-shaped with more than 1024 kept rows (1280): routes read from
    # global memory instead of the kernel's LDS copy
    "decode_rows_over_1024": ("prefill_T256", dict(T=160, H=256, E=128, k=8, I=128, C=160)),
    "decode_shared_T64": ("decode_T32", dict(T=64, H=256, I=128, I_shared=256, C=64)),
    # routing and dispatch inside the gate/up decode launch, with capacity drops
    "decode_fused_capacity": ("decode_T8", dict(T=8, H=256, E=16, k=8, I=128, I_shared=128, C=2)),
    # the largest expert count (1024): the expert GEMMs' LDS tile tables full
    "e1024_prefill": ("prefill_T256", dict(T=2048, H=128, E=1024, k=8, I=128, C=2048)),
    "e1024_decode": ("decode_T8", dict(T=64, H=128, E=1024, k=8, I=128, I_shared=128, C=64)),
    # sigmoid routing with a selection-only bias, normalised and scaled weights
    "sigmoid_relu2_small": ("sigmoid_relu2_R16", dict(H=256, I=256)),
    "sigmoid_prefill_small": ("sigmoid_T2048", dict(T=300, H=256, E=16, k=4, I=256, C=300)),
    # sigmoid routing inside the gate/up decode launch (8 tokens, 240 experts)
    "sigmoid_decode_fused": ("sigmoid_relu2_R16", dict(T=8, H=256, I=256, C=8)),
    # more than 8 (and 16) slots per token with capacity drops: the combine
    # loads a token's rows 8 slots at a time, and dropped slots fall in every
    # batch; tiled path, slot-indexed decode path, float32 combine
    "k20_capacity_prefill": ("prefill_T256", dict(T=300, H=256, E=32, k=20, I=128, C=60)),
    "k20_capacity_decode": ("decode_T8", dict(T=24, H=256, E=64, k=20, I=128, I_shared=128, C=3)),
    "k12_capacity_fp32": ("tiny_fp32", dict(k=12, C=20)),
}
# Full-size workloads.
FULL = ["tiny_fp32", "prefill_T256", "prefill_T2048", "prefill_T8192", "decode_T1", "decode_T8",
        "decode_T32", "relu2_distinct_R1", "relu2_shared_R1", "relu2_distinct_R8",
        "relu2_shared_R8", "relu2_distinct_R16", "relu2_shared_R16", "skewed_bf16", "skewed_fp8",
        "sigmoid_relu2_R16", "sigmoid_T2048"]


def _case(key):
    if key in SMALL:
        name, over = SMALL[key]
        return parity_case(name, **over)
    return parity_case(key)


def _say(*a):
    print("[gpu-case]", *a, flush=True)


# ---- routing -----------------------------------------------------------------

def _route_gpu(cs, logits_dev, bias_dev=None):
    p = problem(cs)
    ws = workspace(p)
    ids = torch.empty((cs.T, cs.k), dtype=torch.int32, device=DEV)
    w = torch.empty((cs.T, cs.k), dtype=torch.float32, device=DEV)
    rde.moe_route(p, logits_dev, bias_dev, ids, w, ws)
    torch.cuda.synchronize()
    return ids, w


def _oracle_route(cs, logits, bias):
    return oracle.route(logits, cs.k, cs.renormalize, cs.score_func,
                        None if bias is None else oracle.from_torch(bias), cs.route_scale)


def _check_route(cs, logits, bias=None):
    ids, w = _route_gpu(cs, logits.to(DEV), None if bias is None else bias.to(DEV))
    oi, ow = _oracle_route(cs, logits.numpy(), bias)
    np.testing.assert_array_equal(np_i32(ids), oi)
    assert_f32_close(w, ow, "w")
    return ids, w, oi, ow


@pytest.mark.parametrize("key", list(SMALL) + FULL)
def test_route(key):
    cs = _case(key)
    _say("route", key, cs.T, cs.E, cs.k)
    _check_route(cs, synth.make_logits(cs), synth.make_score_bias(cs))


def test_route_pm16_bit_exact():
    for key in ("relu2_distinct_R16", "relu2_shared_R16"):
        cs = synth.case(key)
        _say("route pm16", key)
        ids, w, oi, _ = _check_route(cs, synth.make_logits(cs))
        # +16 / -16: every selected weight is exactly fl32(1/9)
        assert torch.all(w.cpu() == torch.tensor(1.0, dtype=torch.float32) / 9)


@pytest.mark.parametrize("E,k", [(7, 3), (9, 9), (32, 32), (64, 6), (130, 32), (200, 9), (1024, 32)])
def test_route_ties_and_special_values(E, k):
    _say("route ties", E, k)
    g = torch.Generator().manual_seed(E)
    pool = torch.tensor([-1.0, -0.0, 0.0, 1.0, 2.5, float("-inf"), float("nan")])
    T = 300
    lg = pool[torch.randint(0, len(pool), (T, E), generator=g)]
    lg[0] = float("-inf")             # all -inf: NaN weights, lowest indices
    lg[1] = torch.arange(E, dtype=torch.float32)
    cs = synth.Case("ties", T=T, H=128, E=E, k=k, I=128, C=T)
    ids, w = _route_gpu(cs, lg.to(DEV))
    oi, ow = oracle.route(lg.numpy(), k)
    np.testing.assert_array_equal(np_i32(ids), oi)
    assert_f32_close(w, ow, "w")


@pytest.mark.parametrize("E,k", [(7, 3), (9, 9), (32, 32), (64, 6), (130, 32), (240, 9), (1024, 32)])
def test_route_sigmoid_ties_and_special_values(E, k):
    # large logits saturate the float32 score to 1.0 (ties decided by index),
    # grid biases make score + bias exact ties too; NaN and +-inf included
    _say("route sigmoid ties", E, k)
    g = torch.Generator().manual_seed(100 + E)
    pool = torch.tensor([-1.0, 0.0, 1.0, 2.5, 20.0, 35.0, -40.0, float("inf"), float("-inf"),
                         float("nan")])
    T = 300
    lg = pool[torch.randint(0, len(pool), (T, E), generator=g)]
    lg[1] = torch.arange(E, dtype=torch.float32) / 8
    bias = torch.randint(-8, 9, (E,), generator=g).to(torch.float32) / 32
    for renorm, scale, b in ((0, 1.0, None), (1, 2.5, bias), (0, 0.75, bias)):
        cs = synth.Case("sig_ties", T=T, H=128, E=E, k=k, I=128, C=T,
                        score_func=synth.SCORE_SIGMOID, renormalize=renorm, route_scale=scale)
        ids, w = _route_gpu(cs, lg.to(DEV), None if b is None else b.to(DEV))
        oi, ow = _oracle_route(cs, lg.numpy(), b)
        np.testing.assert_array_equal(np_i32(ids), oi)
        assert_f32_close(w, ow, "w")


@pytest.mark.parametrize("T,E,k", [(5, 9, 9), (40, 240, 9), (64, 64, 6), (33, 512, 32)])
def test_forward_small_batch_routing_ties(T, E, k):
    # the single-workgroup dispatch of small batches routes several tokens per
    # wavefront; its routes are compared through the forward's metadata
    _say("small-batch routing ties", T, E, k)
    g = torch.Generator().manual_seed(7 * E + T)
    pool = torch.tensor([-1.0, -0.0, 0.0, 1.0, 2.5, float("-inf"), float("nan")])
    lg = pool[torch.randint(0, len(pool), (T, E), generator=g)]
    cs = synth.Case("small_ties", T=T, H=128, E=E, k=k, I=128, C=T)
    inp = dataclasses.replace(synth.make_inputs(cs, DEV), logits=lg.to(DEV))
    _, meta, _ = _forward_gpu(cs, inp)
    oi, ow = oracle.route(lg.numpy(), k)
    np.testing.assert_array_equal(np_i32(meta["ids"]), oi)
    assert_f32_close(meta["w"], ow, "w")


# ---- dispatch ----------------------------------------------------------------

def _dispatch_gpu(cs, x_dev, ids_dev):
    p = problem(cs)
    ws = workspace(p)
    R = r_max(cs)
    counts = torch.empty(cs.E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(cs.E + 1, dtype=torch.int32, device=DEV)
    row_src = torch.full((max(R, 1),), 12345, dtype=torch.int32, device=DEV)
    route_dst = torch.empty((cs.T, cs.k), dtype=torch.int32, device=DEV)
    x_disp = torch.zeros((max(R, 1), cs.H), dtype=act_dtype(cs), device=DEV)
    rde.moe_dispatch(p, x_dev, ids_dev, counts, offsets, row_src, route_dst, x_disp, ws)
    n_bad = rde.moe_error(ws)
    return dict(counts=counts, offsets=offsets, row_src=row_src[:R], route_dst=route_dst,
                x_disp=x_disp, n_bad=n_bad)


def _check_dispatch(cs, x, ids_np):
    g = _dispatch_gpu(cs, x.to(DEV), torch.from_numpy(ids_np).to(DEV))
    d = oracle.dispatch(ids_np, cs.E, cs.C)
    for key in ("counts", "offsets", "row_src", "route_dst"):
        np.testing.assert_array_equal(np_i32(g[key]), d[key], err_msg=key)
    assert g["n_bad"] == d["n_bad"]
    R = int(d["offsets"][-1])
    xo = oracle.gather_rows(oracle.from_torch(x), d["row_src"], R, cs.k)
    xg = oracle.from_torch(g["x_disp"][:R].cpu())
    assert np.array_equal(xg.view(np.uint8), xo.view(np.uint8)), "x_disp differs"
    return d


@pytest.mark.parametrize("key", list(SMALL) + FULL)
def test_dispatch(key):
    cs = _case(key)
    _say("dispatch", key, cs.T, cs.E, cs.k, cs.C)
    ids, _ = oracle.route(synth.make_logits(cs).numpy(), cs.k)
    d = _check_dispatch(cs, synth.make_x(cs), ids)
    assert d["counts"].sum() == cs.T * cs.k


@pytest.mark.parametrize("kind", ["dummy", "negative", "wide", "duplicate"])
def test_dispatch_malformed_routes(kind):
    _say("dispatch malformed", kind)
    cs = synth.Case("bad", T=40, H=256, E=16, k=4, I=128, C=40)
    ids = synth.bad_routes(cs.T, cs.k, cs.E, kind).numpy()
    d = _check_dispatch(cs, synth.make_x(cs), ids)
    assert d["n_bad"] == 1


@pytest.mark.parametrize("k", [3, 9, 32])
def test_dispatch_dense_malformed_routes(k):
    # ids drawn with replacement from a small range plus out-of-range values:
    # many duplicates inside tokens, including tokens whose slots straddle a
    # 64-route step (k not dividing 64) and a 2048-route block
    _say("dispatch dense malformed", k)
    T, E = 700, 40
    g = torch.Generator().manual_seed(k)
    ids = torch.randint(-2, E + 2, (T, k), generator=g).to(torch.int32)
    ids[::5] = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(0, T, 5)]).to(torch.int32)
    cs = synth.Case("dense_bad", T=T, H=128, E=E, k=k, I=128, C=T)
    d = _check_dispatch(cs, synth.make_x(cs), ids.numpy())
    assert 0 < d["n_bad"] < T * k


def test_dispatch_ragged_blocks_and_max_k():
    # route counts around the 2048-route block boundary, k = 32, E = 1024; up
    # to 4096 routes one workgroup places them all (4096 exactly: 4 per lane),
    # above that the count kernel hands its totals to its last block
    for T, E, k, C in ((2049 // 8 + 1, 128, 8, 7), (64, 1024, 32, 3), (4097, 33, 1, 4097),
                       (512, 100, 8, 30), (8300, 64, 8, 2000)):
        _say("dispatch ragged", T, E, k, C)
        cs = synth.Case("rag", T=T, H=128, E=E, k=k, I=128, C=C, seed=T)
        ids, _ = oracle.route(synth.make_logits(cs).numpy(), k)
        _check_dispatch(cs, synth.make_x(cs), ids)


# ---- expert FFN ----------------------------------------------------------------

def _expert_ffn_gpu(cs, inp_dev, x_disp_dev, offsets_dev):
    p = problem(cs)
    ws = workspace(p)
    R = r_max(cs)
    y = torch.full((max(R, 1), cs.H), float("nan"), dtype=act_dtype(cs), device=DEV)
    rde.moe_expert_ffn(p, x_disp_dev, offsets_dev, inp_dev.w13, inp_dev.w2, inp_dev.s13,
                       inp_dev.s2, y, ws)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("key", list(SMALL) + ["prefill_T2048", "decode_T32", "relu2_shared_R16",
                                               "skewed_bf16", "skewed_fp8"])
def test_expert_ffn(key):
    """y_disp of every non-empty expert: all rows on the small cases; the
    first, middle and last row of each expert at full size (on the skewed
    workloads that includes the light experts whose m-tiles hold a few rows)."""
    cs = _case(key)
    _say("expert_ffn", key)
    inp_dev = synth.make_inputs(cs, DEV)
    ids, _ = oracle.route(oracle.from_torch(inp_dev.logits), cs.k)
    d = oracle.dispatch(ids, cs.E, cs.C)
    R = int(d["offsets"][-1])
    xh = oracle.from_torch(inp_dev.x)
    xd = oracle.gather_rows(xh, d["row_src"], R, cs.k)
    xd_dev = torch.from_numpy(xd.view(np.int16) if xd.dtype == np.uint16 else xd).to(DEV)
    if xd.dtype == np.uint16:
        xd_dev = xd_dev.view(torch.bfloat16)
    y = _expert_ffn_gpu(cs, inp_dev, xd_dev, torch.from_numpy(d["offsets"]).to(DEV))
    small = key in SMALL
    experts = [e for e in range(cs.E) if d["offsets"][e + 1] > d["offsets"][e]]

    def rows_of(e):
        a, b = int(d["offsets"][e]), int(d["offsets"][e + 1])
        return list(range(a, b)) if small else sorted({a, b - 1, (a + b) // 2})

    def run(e):
        w13, w2, s13, s2 = host_expert(inp_dev, e)
        return oracle.expert_rows(xd[rows_of(e)], w13, w2, cs.act, s13, s2)

    refs = parallel_map(run, experts)
    for e, ref in zip(experts, refs):
        assert_close(cs, y[rows_of(e)], ref, f"y_disp expert {e}")


def test_shared_ffn():
    for key in ("decode_T1", "decode_T32", "decode_shared_small"):
        cs = _case(key)
        _say("shared_ffn", key)
        inp_dev = synth.make_inputs(cs, DEV)
        p = problem(cs)
        ws = workspace(p)
        ysh = torch.empty((cs.T, cs.H), dtype=torch.float32, device=DEV)
        rde.moe_shared_ffn(p, inp_dev.x, inp_dev.w13_sh, inp_dev.w2_sh, ysh, ws)
        torch.cuda.synchronize()
        host = oracle.inputs_numpy(inp_dev.to("cpu"))
        tokens = list(range(cs.T))
        assert_bf16_close(ysh, oracle_shared(cs, host, tokens), "y_shared")


# ---- combine -------------------------------------------------------------------

@pytest.mark.parametrize("key", ["tiny_fp32", "ragged_skew_capacity", "decode_shared_small",
                                 "prefill_T2048"])
def test_combine(key):
    cs = _case(key)
    _say("combine", key)
    ids, w = oracle.route(synth.make_logits(cs).numpy(), cs.k)
    d = oracle.dispatch(ids, cs.E, cs.C)
    R = max(int(d["offsets"][-1]), 1)
    g = torch.Generator().manual_seed(3)
    y32 = torch.randn((R, cs.H), generator=g)
    y = y32.to(act_dtype(cs))
    ysh = torch.randn((cs.T, cs.H), generator=g) if cs.n_shared else None
    p = problem(cs)
    ws = workspace(p)
    out = torch.empty((cs.T, cs.H), dtype=act_dtype(cs), device=DEV)
    w32 = torch.from_numpy(w.astype(np.float32))
    rde.moe_combine(p, y.to(DEV), torch.from_numpy(d["route_dst"]).to(DEV), w32.to(DEV),
                    None if ysh is None else ysh.to(DEV), out, ws)
    torch.cuda.synchronize()
    ref = oracle.combine(d["route_dst"], w32.double().numpy(), y.double().numpy(),
                         None if ysh is None else ysh.double().numpy())
    assert_close(cs, out, ref, "out")


# ---- whole layer -----------------------------------------------------------------

def _forward_gpu(cs, inp_dev, ids_in=None, w_in=None, with_meta=True):
    p = problem(cs)
    ws = workspace(p)
    R = r_max(cs)
    out = torch.empty((cs.T, cs.H), dtype=act_dtype(cs), device=DEV)
    meta = None
    if with_meta:
        meta = dict(ids=torch.empty((cs.T, cs.k), dtype=torch.int32, device=DEV),
                    w=torch.empty((cs.T, cs.k), dtype=torch.float32, device=DEV),
                    counts=torch.empty(cs.E, dtype=torch.int32, device=DEV),
                    offsets=torch.empty(cs.E + 1, dtype=torch.int32, device=DEV),
                    row_src=torch.empty(max(R, 1), dtype=torch.int32, device=DEV),
                    route_dst=torch.empty((cs.T, cs.k), dtype=torch.int32, device=DEV))
    rde.moe_forward(p, inp_dev.x, inp_dev.logits, inp_dev.score_bias, ids_in, w_in,
                    inp_dev.w13, inp_dev.w2,
                    inp_dev.s13, inp_dev.s2, inp_dev.w13_sh, inp_dev.w2_sh, out, meta, ws)
    n_bad = rde.moe_error(ws)
    return out, meta, n_bad


def _check_meta(cs, meta, r):
    np.testing.assert_array_equal(np_i32(meta["ids"]), r["ids"])
    assert_f32_close(meta["w"], r["w"], "w")
    for key in ("counts", "offsets", "route_dst"):
        np.testing.assert_array_equal(np_i32(meta[key]), r[key], err_msg=key)
    np.testing.assert_array_equal(np_i32(meta["row_src"])[:len(r["row_src"])], r["row_src"])


@pytest.mark.parametrize("key", list(SMALL))
def test_forward_small(key):
    cs = _case(key)
    _say("forward small", key)
    inp_dev = synth.make_inputs(cs, DEV)
    out, meta, n_bad = _forward_gpu(cs, inp_dev)
    r = oracle.forward(cs, **oracle.inputs_numpy(inp_dev.to("cpu")))
    _check_meta(cs, meta, r)
    assert n_bad == 0
    assert_close(cs, out, r["out"], "out")


# Other input seeds for cases that between them take every bf16 tile layout,
# the e4m3 weights, the routing inside the decode gate/up launch (softmax and
# sigmoid), capacity drops with k = 20, and more kept rows than the decode
# kernel stages in LDS: the data-dependent paths (row spreads over m-tiles,
# layout changes between tiles, ranks and drops) see other expert loads.
SEEDED = ["skewed_all_layouts", "multi_tile_swiglu", "fp8_small", "decode_fused_capacity",
          "sigmoid_decode_fused", "k20_capacity_decode", "decode_rows_over_1024"]


@pytest.mark.parametrize("seed", [1, 2, 3])
@pytest.mark.parametrize("key", SEEDED)
def test_forward_small_other_seeds(key, seed):
    cs = dataclasses.replace(_case(key), seed=seed)
    _say("forward small", key, "seed", seed)
    inp_dev = synth.make_inputs(cs, DEV)
    out, meta, n_bad = _forward_gpu(cs, inp_dev)
    r = oracle.forward(cs, **oracle.inputs_numpy(inp_dev.to("cpu")))
    _check_meta(cs, meta, r)
    assert n_bad == 0
    assert_close(cs, out, r["out"], "out")


@pytest.mark.parametrize("T", [1, 300])   # slot-indexed decode kernels; tiled expert GEMMs
def test_forward_e4m3_widening_exact(T):
    """Every finite e4m3 code through the expert GEMMs, bit-exact.  ReLU-square
    experts with x = e_0 and a gate row 0 of 1.0 give h = e_0, so output
    column o of the down projection is the e4m3 weight w2[o, 0] times a
    per-row scale of 1.  With logits +16 / -16 and top-1 the routing weight
    is exactly 1 (softmax of two logits 32 apart rounds to 1 in float32), so
    every output value is the widened code itself; e4m3 values are bf16
    values, so nothing may round.  Expected values: torch's float8_e4m3fn
    decoding on the CPU (-0.0 as +0.0, see below)."""
    H, I, E = 256, 128, 2
    cs = synth.Case("e4m3_codes", T=T, H=H, E=E, k=1, I=I, C=T, act=synth.ACT_RELU2,
                    w_fmt=synth.FMT_E4M3)
    _say("e4m3 widening", T)
    codes = torch.arange(256, dtype=torch.int32)
    codes[(codes & 0x7F) == 0x7F] = 0                      # the two NaN codes
    codes = codes.to(torch.uint8)
    x = torch.zeros((T, H), dtype=torch.bfloat16)
    x[:, 0] = 1.0
    lg = torch.full((T, E), -16.0)
    lg[:, 0] = 16.0
    w13 = torch.zeros((E, I, H), dtype=torch.uint8)
    w13[:, 0, 0] = 0x38                                      # e4m3 1.0
    w2 = torch.zeros((E, H, I), dtype=torch.uint8)
    w2[:, :, 0] = codes
    inp = synth.Inputs(cs, x.to(DEV), lg.to(DEV), w13.to(DEV), w2.to(DEV),
                       torch.ones((E, I), device=DEV), torch.ones((E, H), device=DEV))
    out, meta, n_bad = _forward_gpu(cs, inp)
    assert n_bad == 0
    np.testing.assert_array_equal(np_i32(meta["ids"]), np.zeros((T, 1), np.int32))
    assert torch.equal(meta["w"].cpu(), torch.ones((T, 1)))
    want = codes.view(torch.float8_e4m3fn).float()
    # the code 0x80 (-0.0) reaches the output through a sum of products that
    # starts from +0, and +0 + (-0) = +0
    want = torch.where(want == 0, torch.zeros_like(want), want).to(torch.bfloat16)
    got = out.cpu()
    bad = (got.view(torch.int16) != want.view(torch.int16).expand(T, H)).nonzero()
    assert bad.numel() == 0, f"{bad.shape[0]} values differ, first (token, code) {bad[0].tolist()}"


def _light_tokens(cs, ids, d, max_rows=32):
    """Tokens with a kept route to an expert holding 1..max_rows rows."""
    counts = np.diff(d["offsets"])
    light = (counts > 0) & (counts <= max_rows)
    kept_light = (d["route_dst"] >= 0) & light[np.clip(ids, 0, cs.E - 1)]
    return np.nonzero(kept_light.any(axis=1))[0].tolist()


@pytest.mark.parametrize("key", FULL)
def test_forward_full_size(key):
    cs = _case(key)
    _say("forward full", key)
    inp_dev = synth.make_inputs(cs, DEV)
    out, meta, _ = _forward_gpu(cs, inp_dev)
    logits = oracle.from_torch(inp_dev.logits)
    ids, w = _oracle_route(cs, logits, inp_dev.score_bias)
    d = oracle.dispatch(ids, cs.E, cs.C)
    r = dict(ids=ids, w=w, **d)
    _check_meta(cs, meta, r)
    rng = np.random.default_rng(0)
    skewed = key.startswith("skewed")
    n_sample = 56 if skewed else 12
    tokens = set(rng.choice(cs.T, size=min(n_sample, cs.T), replace=False).tolist()) | {0, cs.T - 1}
    if skewed:
        # the last token that lost a route to capacity, and 8 tokens routed
        # to experts holding at most 32 rows (m-tiles the light experts barely fill)
        dropped = np.nonzero((d["route_dst"] < 0).any(axis=1))[0]
        assert len(dropped)
        tokens.add(int(dropped[-1]))
        light = _light_tokens(cs, ids, d)
        assert len(light) >= 8
        tokens |= set(rng.choice(light, size=8, replace=False).tolist())
        assert len(tokens) >= 64
    tokens = sorted(tokens)
    xh = oracle.from_torch(inp_dev.x)
    host_sh = None
    if cs.n_shared:
        host_sh = oracle_shared(cs, dict(x=xh, w13_sh=oracle.from_torch(inp_dev.w13_sh),
                                         w2_sh=oracle.from_torch(inp_dev.w2_sh)), tokens)
    ref = oracle_token_rows(cs, inp_dev, xh, ids, w, d["route_dst"], tokens, None)
    if host_sh is not None:
        ref = ref + host_sh
    assert_close(cs, out[tokens], ref, f"out rows of {len(tokens)} tokens")


def test_forward_preselected_is_bitwise_internal():
    # the same routes given as preselected ids / weights give bitwise the
    # same layer output (PR 33963: all outputs bitwise equal across the two
    # routing modes on identical routes)
    for key in ("relu2_distinct_R16", "multi_tile_swiglu", "tiny_fp32", "sigmoid_relu2_small"):
        cs = _case(key)
        _say("preselected bitwise", key)
        inp_dev = synth.make_inputs(cs, DEV)
        out1, meta, _ = _forward_gpu(cs, inp_dev)
        out2, _, _ = _forward_gpu(cs, inp_dev, meta["ids"].clone(), meta["w"].clone())
        assert torch.equal(out1.view(torch.int16) if out1.dtype == torch.bfloat16 else out1.view(torch.int32),
                           out2.view(torch.int16) if out2.dtype == torch.bfloat16 else out2.view(torch.int32))


def test_forward_deterministic_and_batch_invariant():
    cs = _case("multi_tile_swiglu")
    _say("determinism / batch invariance")
    inp_dev = synth.make_inputs(cs, DEV)
    a, _, _ = _forward_gpu(cs, inp_dev, with_meta=False)
    b, _, _ = _forward_gpu(cs, inp_dev, with_meta=False)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # capacity >= T*k: a sub-batch gives bitwise the same rows
    sub = list(range(100, 160))
    cs2 = synth.replace(cs, T=len(sub), C=len(sub) * cs.k)
    inp2 = synth.Inputs(cs2, inp_dev.x[sub].contiguous(), inp_dev.logits[sub].contiguous(),
                        inp_dev.w13, inp_dev.w2)
    c, _, _ = _forward_gpu(cs2, inp2, with_meta=False)
    assert torch.equal(c.view(torch.int16), a[sub].view(torch.int16))


@pytest.mark.parametrize("kind", ["dummy", "negative", "wide", "duplicate"])
def test_forward_malformed_routes_poison_only_their_token(kind):
    cs = parity_case("prefill_T256", T=24, H=256, E=16, k=4, I=128, C=24)
    _say("forward malformed", kind)
    inp_dev = synth.make_inputs(cs, DEV)
    ids = synth.bad_routes(cs.T, cs.k, cs.E, kind)
    w = torch.full((cs.T, cs.k), 0.25)
    out, meta, n_bad = _forward_gpu(cs, inp_dev, ids.to(DEV), w.to(DEV))
    assert n_bad == 1
    r = oracle.forward(cs, **oracle.inputs_numpy(inp_dev.to("cpu")), ids_in=ids.numpy(),
                       w_in=w.double().numpy())
    np.testing.assert_array_equal(np_i32(meta["route_dst"]), r["route_dst"])
    o = out.float().cpu()
    assert torch.isnan(o[1]).all() and torch.isfinite(o[[0] + list(range(2, cs.T))]).all()
    assert_close(cs, out, r["out"], "out")


# Shapes of the graph and preselected tests: rows per expert decide the path
# (tiled grouped GEMM above 12 routes per expert on average, slot-indexed
# expert GEMMs at or below it).
GRAPH_SHAPES = {
    "prefill": ("prefill_T256", dict(T=300, H=256, E=16, k=4, I=128, C=300)),
    "decode": ("decode_T8", dict(H=256, I=128, I_shared=256)),
}


def _capture_forward(cs, inp_dev, ids_in, w_in, out, meta, p, ws):
    """moe_forward captured into a graph on a side stream."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rde.moe_forward(p, inp_dev.x, None if ids_in is not None else inp_dev.logits,
                        None if ids_in is not None else inp_dev.score_bias, ids_in, w_in,
                        inp_dev.w13, inp_dev.w2, inp_dev.s13, inp_dev.s2, inp_dev.w13_sh,
                        inp_dev.w2_sh, out, meta, ws)
    torch.cuda.current_stream().wait_stream(s)
    return g


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("shape", list(GRAPH_SHAPES))
@pytest.mark.parametrize("kind", ["dummy", "negative", "wide", "duplicate"])
def test_forward_malformed_routes_graph_replay(kind, shape):
    # the graph execution of the count-first record's invalid-route runs:
    # every replay poisons only the planted token and counts one bad route
    name, over = GRAPH_SHAPES[shape]
    cs = synth.case(name, **over)
    _say("graph malformed", kind, shape)
    inp_dev = synth.make_inputs(cs, DEV)
    ids = synth.bad_routes(cs.T, cs.k, cs.E, kind).to(DEV)
    w = torch.full((cs.T, cs.k), 1.0 / cs.k, device=DEV)
    ref, meta_e, n_bad = _forward_gpu(cs, inp_dev, ids, w)
    assert n_bad == 1
    p = problem(cs)
    ws = workspace(p)
    out = torch.empty_like(ref)
    route_dst = torch.empty((cs.T, cs.k), dtype=torch.int32, device=DEV)
    g = _capture_forward(cs, inp_dev, ids, w, out, dict(route_dst=route_dst), p, ws)
    for rep in range(3):
        out.fill_(0)
        route_dst.fill_(7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"replay {rep}"
        assert torch.equal(route_dst, meta_e["route_dst"])
        assert rde.moe_error(ws) == 1
        o = out.float().cpu()
        assert torch.isnan(o[1]).all() and torch.isfinite(o[[0] + list(range(2, cs.T))]).all()


@pytest.mark.parametrize("shape", list(GRAPH_SHAPES) + ["sigmoid"])
def test_forward_graph_replay_matches_eager(shape):
    # internal routing inside the graph; replays interleaved with eager work
    name, over = GRAPH_SHAPES.get(shape, ("sigmoid_T2048", dict(T=300, H=256, E=16, k=4, I=128,
                                                                C=300)))
    cs = synth.case(name, **over)
    _say("graph replay", shape)
    inp_dev = synth.make_inputs(cs, DEV)
    ref, meta_e, _ = _forward_gpu(cs, inp_dev)
    p = problem(cs)
    ws = workspace(p)
    out = torch.empty_like(ref)
    meta = {k: torch.empty_like(v) for k, v in meta_e.items()}
    g = _capture_forward(cs, inp_dev, None, None, out, meta, p, ws)
    for rep in range(3):
        out.fill_(0)
        for v in meta.values():
            v.fill_(-5)
        junk, _, _ = _forward_gpu(cs, inp_dev, with_meta=False)   # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"replay {rep}"
        for key, v in meta.items():
            assert torch.equal(_bits(v), _bits(meta_e[key])), (rep, key)
    assert rde.moe_error(ws) == 0


@pytest.mark.parametrize("shape", list(GRAPH_SHAPES))
def test_forward_preselected_k32(shape):
    # preselected float32 weights with k = 32 (the largest k), taken unchanged
    name, over = GRAPH_SHAPES[shape]
    over = dict(over, E=64, k=32, C=over.get("C", 8) * 32)
    if shape == "decode":
        over["T"] = 4
        over["C"] = 4
    cs = parity_case(name, **over)
    _say("preselected k32", shape, cs.T)
    inp_dev = synth.make_inputs(cs, DEV)
    ids = synth.bad_routes(cs.T, cs.k, cs.E, "none", seed=32)
    g = torch.Generator().manual_seed(33)
    w = torch.rand((cs.T, cs.k), generator=g) * 0.1
    out, meta, n_bad = _forward_gpu(cs, inp_dev, ids.to(DEV), w.to(DEV))
    assert n_bad == 0
    assert torch.equal(meta["ids"].cpu(), ids) and torch.equal(meta["w"].cpu(), w)
    r = oracle.forward(cs, **oracle.inputs_numpy(inp_dev.to("cpu")), ids_in=ids.numpy(),
                       w_in=w.double().numpy())
    _check_meta(cs, meta, r)
    assert_close(cs, out, r["out"], "out")
    # without metadata outputs the routes are read in place: same bits
    out2, _, _ = _forward_gpu(cs, inp_dev, ids.to(DEV), w.to(DEV), with_meta=False)
    assert torch.equal(_bits(out2), _bits(out))


@pytest.mark.parametrize("T,k", [(64, 9), (40, 32), (7, 3)])
def test_forward_small_batch_dense_malformed(T, k):
    # batches of at most 64 tokens are routed and dispatched by one workgroup:
    # many duplicate / out-of-range ids, tokens straddling 64-route steps
    cs = parity_case("prefill_T256", T=T, H=256, E=40, k=k, I=128, C=T)
    _say("forward small dense malformed", T, k)
    inp_dev = synth.make_inputs(cs, DEV)
    g = torch.Generator().manual_seed(T * k)
    ids = torch.randint(-1, cs.E + 1, (T, k), generator=g).to(torch.int32)
    ids[::4] = torch.stack([torch.randperm(cs.E, generator=g)[:k] for _ in range(0, T, 4)]).to(torch.int32)
    w = torch.rand((T, k), generator=g)
    out, meta, n_bad = _forward_gpu(cs, inp_dev, ids.to(DEV), w.to(DEV))
    r = oracle.forward(cs, **oracle.inputs_numpy(inp_dev.to("cpu")), ids_in=ids.numpy(),
                       w_in=w.double().numpy())
    assert n_bad == r["n_bad"] > 0
    _check_meta(cs, meta, r)
    assert_close(cs, out, r["out"], "out")


def test_forward_empty_batch():
    cs = synth.case("prefill_T256", T=0, H=256, E=16, I=128)
    _say("forward empty")
    p = problem(cs)
    ws = workspace(p)
    counts = torch.full((cs.E,), 7, dtype=torch.int32, device=DEV)
    offsets = torch.full((cs.E + 1,), 7, dtype=torch.int32, device=DEV)
    z = torch.empty((0, cs.H), dtype=torch.bfloat16, device=DEV)
    zl = torch.empty((0, cs.E), dtype=torch.float32, device=DEV)
    w13 = torch.zeros((cs.E, 2 * cs.I, cs.H), dtype=torch.bfloat16, device=DEV)
    w2 = torch.zeros((cs.E, cs.H, cs.I), dtype=torch.bfloat16, device=DEV)
    rde.moe_forward(p, z, zl, None, None, None, w13, w2, None, None, None, None, z,
                    dict(counts=counts, offsets=offsets), ws)
    torch.cuda.synchronize()
    assert counts.sum().item() == 0 and offsets.sum().item() == 0


def test_forward_matches_separate_entry_points():
    for key in ("decode_shared_small", "ragged_skew_capacity", "tiny_fp32",
                "sigmoid_prefill_small"):
        cs = _case(key)
        _say("forward vs separate", key)
        inp_dev = synth.make_inputs(cs, DEV)
        out_f, meta, _ = _forward_gpu(cs, inp_dev)
        p = problem(cs)
        ws = workspace(p)
        R = r_max(cs)
        ids = torch.empty((cs.T, cs.k), dtype=torch.int32, device=DEV)
        w = torch.empty((cs.T, cs.k), dtype=torch.float32, device=DEV)
        rde.moe_route(p, inp_dev.logits, inp_dev.score_bias, ids, w, ws)
        counts = torch.empty(cs.E, dtype=torch.int32, device=DEV)
        offsets = torch.empty(cs.E + 1, dtype=torch.int32, device=DEV)
        row_src = torch.empty(max(R, 1), dtype=torch.int32, device=DEV)
        route_dst = torch.empty((cs.T, cs.k), dtype=torch.int32, device=DEV)
        x_disp = torch.empty((max(R, 1), cs.H), dtype=act_dtype(cs), device=DEV)
        rde.moe_dispatch(p, inp_dev.x, ids, counts, offsets, row_src, route_dst, x_disp, ws)
        y = torch.empty((max(R, 1), cs.H), dtype=act_dtype(cs), device=DEV)
        rde.moe_expert_ffn(p, x_disp, offsets, inp_dev.w13, inp_dev.w2, inp_dev.s13, inp_dev.s2,
                           y, ws)
        ysh = None
        if cs.n_shared:
            ysh = torch.empty((cs.T, cs.H), dtype=torch.float32, device=DEV)
            rde.moe_shared_ffn(p, inp_dev.x, inp_dev.w13_sh, inp_dev.w2_sh, ysh, ws)
        out_s = torch.empty_like(out_f)
        rde.moe_combine(p, y, route_dst, w, ysh, out_s, ws)
        torch.cuda.synchronize()
        assert torch.equal(ids, meta["ids"]) and torch.equal(w, meta["w"])
        assert torch.equal(route_dst, meta["route_dst"]) and torch.equal(offsets, meta["offsets"])
        ref = out_s.double().cpu().numpy()
        assert_close(cs, out_f, ref, "fused vs separate")


# Large terms cancelling across K tiles (PR 33963, "Motivation and Context":
# the cancellation regression; the commit keeping unit contributions outside
# large-magnitude tensor-core partials).  Paths: the tiled grouped GEMM (one
# expert holds 300 rows, so rows 1, 8, 17 and 129 of its m-tile all carry the
# fixture), the slot-indexed decode GEMMs after the single-workgroup dispatch
# (40 tokens) and with the routing inside the gate/up launch (8 tokens).
CANCEL_PATHS = {"tiled": (300, 2), "slot_indexed": (40, 16), "slot_indexed_fused": (8, 16)}


@pytest.mark.parametrize("path", list(CANCEL_PATHS))
@pytest.mark.parametrize("act", ["relu2", "swiglu"])
def test_forward_cancellation(act, path):
    T, E = CANCEL_PATHS[path]
    a = synth.ACT_RELU2 if act == "relu2" else synth.ACT_SWIGLU
    _say("cancellation", act, path, T, E)
    inp = synth.cancellation_inputs(T, 256, E, 2, 256, a, device=DEV)
    cs = inp.case
    out, meta, n_bad = _forward_gpu(cs, inp)
    assert n_bad == 0
    r = oracle.forward(cs, **oracle.inputs_numpy(inp.to("cpu")))
    _check_meta(cs, meta, r)
    assert_bf16_close(out, r["out"], "out")
    if a == synth.ACT_RELU2:
        # integer products, partial sums below 2^24: the exact result in any
        # summation order, rounded once to bf16
        want = torch.from_numpy(r["out"]).float().to(torch.bfloat16)
        bad = (out.cpu().view(torch.int16) != want.view(torch.int16)).nonzero()
        assert bad.numel() == 0, f"{bad.shape[0]} values differ, first {bad[0].tolist()}"
