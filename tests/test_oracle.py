"""Pins of the CPU oracle against values fixed by the pages and by mathematics.

Nothing here compares the oracle with itself: every check uses a closed form,
a brute-force enumeration, an invariant, or a library routine (numpy, scipy,
torch CPU) that computes a special case of the same definition.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---- storage formats -----------------------------------------------------

def test_e4m3_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        got = oracle.e4m3_to_double(c)
        if math.isnan(ref[c]):
            assert math.isnan(got), c
        else:
            assert got == ref[c], (c, got, ref[c])
    # the format's landmarks: largest finite 448, smallest subnormal 2^-9
    assert oracle.e4m3_to_double(0x7E) == 448.0
    assert oracle.e4m3_to_double(0x01) == 2.0 ** -9
    assert math.isnan(oracle.e4m3_to_double(0x7F)) and math.isnan(oracle.e4m3_to_double(0xFF))


def test_e4m3_widening_to_bf16_is_exact():
    # every finite e4m3 value has <= 4 significant bits and exponent in
    # [-9, 8], so it is a bf16 value: rounding it to bf16 is the identity
    for c in range(256):
        v = oracle.e4m3_to_double(c)
        if not math.isnan(v):
            assert oracle.round_bf16(v) == v


def test_round_bf16_matches_torch_on_float32_inputs():
    g = torch.Generator().manual_seed(5)
    v = torch.randn(20000, generator=g) * torch.exp(torch.randn(20000, generator=g) * 8)
    # plant exact ties (lower 16 bits 0x8000) and their neighbours
    bits = torch.randint(0, 2 ** 15, (3000,), generator=g, dtype=torch.int32) << 16
    ties = (bits | 0x8000 | 0x3F000000).view(torch.float32)
    v = torch.cat([v, ties, -ties, torch.tensor([0.0, -0.0, 1e-40, -3e-39, 3.3e38])])
    ref = v.to(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.round_bf16(float(a)) for a in v.to(torch.float64).numpy()])
    np.testing.assert_array_equal(got, ref)


def test_bf16_widening():
    for bits, val in ((0x3F80, 1.0), (0xBF80, -1.0), (0x4049, 3.140625), (0x0001, 2.0 ** -133)):
        assert oracle.bf16_to_double(bits) == val


# ---- routing ---------------------------------------------------------------

def test_pm16_closed_form_from_the_pages():
    fx = json.load(open(os.path.join(GOLDEN, "pm16_routing.json")))
    E, k = fx["E"], fx["k"]
    for kk in (1, 2, 6, 8, k):
        for first in (0, 17, E - kk):
            lg = np.full((1, E), fx["other_logit"], np.float32)
            lg[0, first:first + kk] = fx["selected_logit"]
            ids, w = oracle.route(lg, kk)
            # all selected logits tie: slots hold the set in ascending order
            assert list(ids[0]) == list(range(first, first + kk))
            exact = 1.0 / (kk + (E - kk) * math.exp(-32.0))
            # a sequential double sum of E terms is within E * 2^-53 relative
            np.testing.assert_allclose(w[0], exact, rtol=2 * E * 2.0 ** -53)
            # in float32 the weight is exactly 1/k (9 -> 1/9, as printed)
            assert np.all(w[0].astype(np.float32) == np.float32(1.0) / np.float32(kk))
            _, wr = oracle.route(lg, kk, renormalize=1)
            assert np.all(wr[0] == 1.0 / kk)
    assert fx["selected_weight_num"] / fx["selected_weight_den"] == pytest.approx(1 / 9)


def _order_key(v, i):
    # NaN after every number, then larger first, equal values by index
    return (1, 0.0, i) if math.isnan(v) else (0, -v, i)


def test_topk_bruteforce_small_with_ties():
    pool = np.array([-1.0, -0.0, 0.0, 1.0, -np.inf, np.nan, 2.5], np.float32)
    rng = np.random.default_rng(3)
    for E in range(1, 8):
        for k in range(1, min(E, 4) + 1):
            for _ in range(40):
                lg = rng.choice(pool, size=(1, E)).astype(np.float32)
                ids, _ = oracle.route(lg, k)
                vals = [float(v) for v in lg[0]]
                # enumerate all k-subsets: exactly one is closed upward
                winners = []
                for S in itertools.combinations(range(E), k):
                    worst = max(_order_key(vals[i], i) for i in S)
                    if all(_order_key(vals[o], o) > worst for o in range(E) if o not in S):
                        winners.append(S)
                assert len(winners) == 1
                want = sorted(winners[0], key=lambda i: _order_key(vals[i], i))
                assert list(ids[0]) == want, (lg, ids, want)


def test_softmax_against_longdouble_and_scipy():
    rng = np.random.default_rng(11)
    lg = (rng.standard_normal((50, 64)) * 3).astype(np.float32)
    ids, w = oracle.route(lg, 6)
    p_sc = scipy.special.softmax(lg.astype(np.float64), axis=1)
    ld = lg.astype(np.longdouble)
    e = np.exp(ld - ld.max(axis=1, keepdims=True))
    p_ld = e / e.sum(axis=1, keepdims=True)
    assert abs(float(p_ld.sum(axis=1).max()) - 1.0) < 1e-15
    for t in range(50):
        np.testing.assert_allclose(w[t], p_ld[t, ids[t]].astype(np.float64), rtol=1e-13)
        np.testing.assert_allclose(w[t], p_sc[t, ids[t]], rtol=1e-12)
        # ids are the top-6 by numpy's stable argsort of the negated logits
        assert list(ids[t]) == list(np.argsort(-lg[t], kind="stable")[:6])
    _, wr = oracle.route(lg, 6, renormalize=1)
    for t in range(50):
        np.testing.assert_allclose(wr[t], scipy.special.softmax(lg[t, ids[t]].astype(np.float64)),
                                   rtol=1e-12)


# ---- sigmoid routing with a selection-only correction bias -----------------

def test_sigmoid_bias_selects_but_does_not_weight():
    # equal logits give every expert the score sigma(0) = 1/2 exactly, so the
    # selection is decided by the bias alone (grid values: 1/2 + b is exact in
    # float32, ties included) while the weights stay those of equal scores
    rng = np.random.default_rng(21)
    for E, k in ((8, 3), (16, 5), (64, 6), (240, 9)):
        lg = np.zeros((6, E), np.float32)
        b = (rng.integers(-64, 65, size=E) / 256.0).astype(np.float32)
        want = list(np.argsort(-b, kind="stable")[:k])
        ids, w = oracle.route(lg, k, 0, oracle.SIGMOID, b)
        assert all(list(r) == want for r in ids)
        assert np.all(w == 0.5)
        _, wn = oracle.route(lg, k, 1, oracle.SIGMOID, b, 2.5)
        np.testing.assert_allclose(wn, 2.5 / k, rtol=4e-16)


def test_sigmoid_pm16_with_small_bias_orders_within_the_selected_set():
    # +16 on the selected set, -16 elsewhere: a bias of magnitude < 1/2 cannot
    # change the set (sigma(16) - sigma(-16) > 0.99) but orders it; the
    # normalised weights are 1/k whatever the order
    rng = np.random.default_rng(22)
    E, k = 240, 9
    lg = np.full((4, E), -16.0, np.float32)
    for t in range(4):
        lg[t, 9 * t:9 * t + 9] = 16.0
    b = (rng.standard_normal(E) * 0.1).astype(np.float32)
    ids, w = oracle.route(lg, k, 1, oracle.SIGMOID, b)
    for t in range(4):
        sel = np.arange(9 * t, 9 * t + 9)
        key = np.float32(scipy.special.expit(16.0)) + b[sel]
        assert list(ids[t]) == list(sel[np.argsort(-key, kind="stable")])
    np.testing.assert_allclose(w, 1.0 / k, rtol=4e-16)


def test_sigmoid_scores_against_expit_with_float32_ties():
    # logits up to +-30: sigma rounds to 1.0f (or to denormal-free tiny values)
    # for many experts, so the float32 keys tie and the lower index must win;
    # the weights are the unrounded scores
    rng = np.random.default_rng(23)
    lg = (rng.standard_normal((40, 128)) * 12).astype(np.float32)
    ids, w = oracle.route(lg, 8, 0, oracle.SIGMOID)
    s = scipy.special.expit(lg.astype(np.float64))
    key = s.astype(np.float32)
    n_tied = 0
    for t in range(40):
        want = np.argsort(-key[t], kind="stable")[:8]
        assert list(ids[t]) == list(want)
        np.testing.assert_allclose(w[t], s[t, want], rtol=1e-15)
        n_tied += int((key[t, want] == np.float32(1.0)).sum() > 1)
    assert n_tied > 10   # the case really exercises ties
    # a different order from the raw-logit top-k somewhere (ties resolved by index)
    assert any(list(ids[t]) != list(np.argsort(-lg[t], kind="stable")[:8]) for t in range(40))


def test_sigmoid_topk_bruteforce_with_nan_inf_and_bias():
    pool = np.array([-1.0, 0.0, 1.0, -np.inf, np.inf, np.nan, 2.5, 40.0], np.float32)
    bpool = np.array([0.0, 0.25, -0.25, 0.5], np.float32)
    rng = np.random.default_rng(24)
    for E in range(1, 8):
        for k in range(1, min(E, 4) + 1):
            for _ in range(30):
                lg = rng.choice(pool, size=(1, E)).astype(np.float32)
                b = rng.choice(bpool, size=E).astype(np.float32)
                ids, w = oracle.route(lg, k, 0, oracle.SIGMOID, b)
                with np.errstate(over="ignore"):
                    sc = scipy.special.expit(lg[0].astype(np.float64))
                key = [float(np.float32(np.float32(v) + bb)) for v, bb in zip(sc, b)]
                winners = []
                for S in itertools.combinations(range(E), k):
                    worst = max(_order_key(key[i], i) for i in S)
                    if all(_order_key(key[o], o) > worst for o in range(E) if o not in S):
                        winners.append(S)
                assert len(winners) == 1
                want = sorted(winners[0], key=lambda i: _order_key(key[i], i))
                assert list(ids[0]) == want, (lg, b, ids, want)
                np.testing.assert_allclose(w[0], sc[want], rtol=1e-15)


def test_route_scale_and_renormalised_sum():
    rng = np.random.default_rng(25)
    lg = rng.standard_normal((30, 64)).astype(np.float32)
    b = (rng.standard_normal(64) * 0.1).astype(np.float32)
    for sf, bias in ((oracle.SOFTMAX, None), (oracle.SIGMOID, b)):
        i1, w1 = oracle.route(lg, 6, 1, sf, bias)
        i2, w2 = oracle.route(lg, 6, 1, sf, bias, 2.5)
        np.testing.assert_array_equal(i1, i2)
        np.testing.assert_allclose(w2, 2.5 * w1, rtol=2e-16)
        np.testing.assert_allclose(w2.sum(axis=1), 2.5, rtol=1e-14)
        i4, w4 = oracle.route(lg, 6, 0, sf, bias, 4.0)
        np.testing.assert_array_equal(w4, 4.0 * oracle.route(lg, 6, 0, sf, bias)[1])


def test_all_minus_inf_row_poisons_weights():
    lg = np.full((2, 8), -np.inf, np.float32)
    lg[1] = np.arange(8, dtype=np.float32)
    ids, w = oracle.route(lg, 3)
    assert np.all(np.isnan(w[0]))
    assert list(ids[0]) == [0, 1, 2]
    assert list(ids[1]) == [7, 6, 5] and np.all(np.isfinite(w[1]))


# ---- count-first dispatch --------------------------------------------------

def _dispatch_by_sort(ids, E, C):
    """Library special case: histogram = bincount, scan = cumsum, stable ranks
    from numpy's stable argsort of the flattened expert ids."""
    flat = ids.reshape(-1)
    counts = np.bincount(flat, minlength=E)
    kept = np.minimum(counts, C)
    offsets = np.concatenate([[0], np.cumsum(kept)])
    order = np.argsort(flat, kind="stable")
    start = np.concatenate([[0], np.cumsum(counts)])
    rank = np.empty_like(flat)
    rank[order] = np.arange(flat.size) - start[flat[order]]
    dst = np.where(rank < C, offsets[flat] + rank, -1)
    return counts, offsets, dst.reshape(ids.shape)


@pytest.mark.parametrize("T,E,k,C,kind", [
    (64, 16, 2, 64, "normal"), (300, 32, 4, 16, "zipf"), (257, 128, 8, 2048, "normal"),
    (1, 64, 6, 1, "normal"), (0, 8, 2, 4, "normal"), (50, 8, 8, 3, "normal")])
def test_dispatch_against_sort_and_inverse(T, E, k, C, kind):
    cs = synth.Case("t", T=T, H=16, E=E, k=k, I=16, C=C, logits_kind=kind, seed=T)
    lg = synth.make_logits(cs).numpy()
    ids, _ = oracle.route(lg, k) if T else (np.zeros((0, k), np.int32), None)
    d = oracle.dispatch(ids, E, C)
    counts, offsets, dst = _dispatch_by_sort(ids.astype(np.int64), E, C)
    np.testing.assert_array_equal(d["counts"], counts)
    np.testing.assert_array_equal(d["offsets"], offsets)
    np.testing.assert_array_equal(d["route_dst"], dst)
    # invariants: sum of raw counts is T*k, offsets non-decreasing,
    # R = sum min(counts, C) <= r_max
    assert d["counts"].sum() == T * k
    assert np.all(np.diff(d["offsets"]) >= 0)
    R = int(d["offsets"][-1])
    assert R == np.minimum(d["counts"], C).sum() <= min(T * k, E * C)
    # inverse: row_src and route_dst are mutually inverse on kept routes
    rs, rd = d["row_src"], d["route_dst"].reshape(-1)
    assert np.all(rs[R:] == -1)
    for r in range(R):
        assert rd[rs[r]] == r
    for q in range(T * k):
        if rd[q] >= 0:
            assert rs[rd[q]] == q
    # dispatch followed by its inverse: gathered rows are the token rows
    x = np.arange(max(T, 1) * 4, dtype=np.float32).reshape(max(T, 1), 4)[:T]
    xd = oracle.gather_rows(x, rs, R, k)
    for q in range(T * k):
        if rd[q] >= 0:
            np.testing.assert_array_equal(xd[rd[q]], x[q // k])


def test_capacity_drops_latest_routes_skewed():
    cs = synth.Case("t", T=512, H=16, E=32, k=4, I=16, C=16, logits_kind="zipf")
    ids, _ = oracle.route(synth.make_logits(cs).numpy(), 4)
    d = oracle.dispatch(ids, 32, 16)
    flat = ids.reshape(-1)
    rd = d["route_dst"].reshape(-1)
    assert (d["counts"] > 16).any() and (d["counts"] < 16).any()
    for e in range(32):
        qs = np.nonzero(flat == e)[0]
        assert np.all(rd[qs[:16]] >= 0) and np.all(rd[qs[16:]] == -1)


@pytest.mark.parametrize("kind", ["dummy", "negative", "wide", "duplicate"])
def test_malformed_routes_are_isolated(kind):
    T, k, E = 6, 4, 16
    ids = synth.bad_routes(T, k, E, kind).numpy()
    d = oracle.dispatch(ids, E, 64)
    assert d["n_bad"] == 1
    assert list(d["token_bad"]) == [0, 1, 0, 0, 0, 0]
    valid = np.ones_like(ids, bool)
    valid[1] = [(0 <= e < E) and e not in ids[1, :j] for j, e in enumerate(ids[1])]
    assert d["counts"].sum() == valid.sum() == T * k - 1
    assert np.all(d["route_dst"][~valid] == -2)
    # the combine poisons exactly the token holding the malformed route
    y = np.ones((max(int(d["offsets"][-1]), 1), 3))
    out = oracle.combine(d["route_dst"], np.full((T, k), 0.5), y)
    assert np.all(np.isnan(out[1])) and np.all(np.isfinite(np.delete(out, 1, 0)))


# ---- expert FFN --------------------------------------------------------------

def _widen(a):
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


@pytest.mark.parametrize("act", [oracle.SWIGLU, oracle.RELU2])
@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_expert_rows_against_numpy_matmul(act, fmt):
    n, H, I = 5, 48, 40
    g = torch.Generator().manual_seed(7 + act)
    x = torch.randn(n, H, generator=g)
    w13 = torch.randn(2 * I if act == oracle.SWIGLU else I, H, generator=g) * 0.2
    w2 = torch.randn(H, I, generator=g) * 0.2
    if fmt == "bf16":
        x, w13, w2 = (t.to(torch.bfloat16) for t in (x, w13, w2))
    xn, an, bn = (oracle.from_torch(t) for t in (x, w13, w2))
    y = oracle.expert_rows(xn, an, bn, act, round_h=False)
    X, A, B = _widen(xn), _widen(an), _widen(bn)
    G = X @ A[:I].T
    if act == oracle.SWIGLU:
        U = X @ A[I:].T
        h = G * scipy.special.expit(G) * U
    else:
        h = np.maximum(G, 0) ** 2
    np.testing.assert_allclose(y, h @ B.T, rtol=1e-11, atol=1e-13)
    # with the bf16 store boundary, h is rounded before the second projection
    yr = oracle.expert_rows(xn, an, bn, act, round_h=True)
    hr = np.vectorize(oracle.round_bf16)(h)
    np.testing.assert_allclose(yr, hr @ B.T, rtol=1e-9, atol=1e-12)


def test_silu_identity_and_relu2_exact_grid():
    # silu(a) - silu(-a) = a, with u = 1: two rows x and -x through an
    # expert whose up projection reproduces 1 and whose down projection is
    # the identity on the first I coordinates.
    # The input carries a constant-1 column so that u = 1.
    H = I = 8
    xv = np.linspace(-3, 3, H).astype(np.float32)
    x = np.stack([xv, -xv])
    H2 = H + 1
    xa = np.concatenate([x, np.ones((2, 1), np.float32)], axis=1)
    w13a = np.zeros((2 * I, H2), np.float32)
    w13a[:I, :H] = np.eye(I, H)
    w13a[I:, H] = 1.0
    w2a = np.zeros((H2, I), np.float32)
    w2a[:I, :I] = np.eye(I)
    y = oracle.expert_rows(xa, w13a, w2a, oracle.SWIGLU, round_h=False)
    np.testing.assert_allclose(y[0, :I] - y[1, :I], xv.astype(np.float64), rtol=1e-14, atol=1e-15)
    assert y[0, 4] == pytest.approx(float(xv[4]) / (1 + math.exp(-float(xv[4]))), rel=1e-15)
    # ReLU-square on integer grids: every h is an exact bf16 value, so the
    # rounded path equals exact integer arithmetic
    rng = np.random.default_rng(2)
    xb = rng.integers(-2, 3, (4, 16)).astype(np.float32)
    a = rng.integers(-1, 2, (8, 16)).astype(np.float32)
    b = rng.integers(-1, 2, (16, 8)).astype(np.float32)
    bf = lambda m: oracle.from_torch(torch.from_numpy(m).to(torch.bfloat16))
    yb = oracle.expert_rows(bf(xb), bf(a), bf(b), oracle.RELU2, round_h=True)
    want = (np.maximum(xb.astype(np.int64) @ a.T.astype(np.int64), 0) ** 2) @ b.T.astype(np.int64)
    np.testing.assert_array_equal(yb, want.astype(np.float64))


def test_e4m3_weights_apply_row_scales():
    n, H, I = 3, 32, 24
    g = torch.Generator().manual_seed(1)
    x = torch.randn(n, H, generator=g).to(torch.bfloat16)
    a32 = torch.randn(2 * I, H, generator=g) * 0.02
    b32 = torch.randn(H, I, generator=g) * 0.02
    q13, s13 = synth._quant_e4m3_rows(a32)
    q2, s2 = synth._quant_e4m3_rows(b32)
    y = oracle.expert_rows(oracle.from_torch(x), q13.numpy(), q2.numpy(), oracle.SWIGLU,
                           s13.numpy(), s2.numpy(), round_h=False)
    A = q13.view(torch.float8_e4m3fn).double().numpy() * s13.double().numpy()[:, None]
    B = q2.view(torch.float8_e4m3fn).double().numpy() * s2.double().numpy()[:, None]
    X = x.double().numpy()
    G, U = X @ A[:I].T, X @ A[I:].T
    np.testing.assert_allclose(y, (G * scipy.special.expit(G) * U) @ B.T, rtol=1e-10, atol=1e-15)


# ---- combine and the whole layer ---------------------------------------------

def test_identity_expert_reproduces_input():
    # y := x_disp (the FFN skipped): combine gives sum_j w_j x_t; with +-16
    # logits every w_j = 1/(k + (E-k) e^-32), so out = x * k * w_j.
    E = 64
    for k in (1, 2, 4, 6, 8):
        T, H = 12, 10
        lg = np.full((T, E), -16.0, np.float32)
        for t in range(T):
            lg[t, (np.arange(k) * 7 + t) % E] = 16.0
        ids, w = oracle.route(lg, k)
        d = oracle.dispatch(ids, E, T)
        x = np.random.default_rng(k).standard_normal((T, H)).astype(np.float32)
        R = int(d["offsets"][-1])
        xd = oracle.gather_rows(x, d["row_src"], R, k).astype(np.float64)
        out = oracle.combine(d["route_dst"], w, xd)
        scale = k / (k + (E - k) * math.exp(-32.0))
        # the weights carry the E-term softmax sum error (E * 2^-53), then k adds
        np.testing.assert_allclose(out, x.astype(np.float64) * scale, rtol=2 * (E + k) * 2.0 ** -53, atol=0)
        assert np.all(out.astype(np.float32) == x)


def test_shared_only_and_dropped_routes():
    T, k, H = 3, 2, 4
    rd = np.array([[0, -1], [1, 2], [-1, -1]], np.int32)
    w = np.full((T, k), 0.5)
    y = np.arange(12, dtype=np.float64).reshape(3, 4)
    ysh = np.ones((T, H)) * 10
    out = oracle.combine(rd, w, y, ysh)
    np.testing.assert_array_equal(out[0], 0.5 * y[0] + 10)
    np.testing.assert_array_equal(out[1], 0.5 * y[1] + 0.5 * y[2] + 10)
    np.testing.assert_array_equal(out[2], ysh[2])
    out0 = oracle.combine(rd, np.zeros((T, k)), y, ysh)
    np.testing.assert_array_equal(out0, ysh)


def _numpy_layer(cs, inp):
    """The layer from library routines: stable argsort top-k, scipy softmax,
    bincount/cumsum/argsort dispatch, float64 matmuls, expit."""
    lg = inp["logits"].astype(np.float64)
    T, E, k, I = cs.T, cs.E, cs.k, cs.I
    if cs.score_func == synth.SCORE_SIGMOID:
        s = scipy.special.expit(lg)
        key = s.astype(np.float32)
        if inp.get("score_bias") is not None:
            key = key + inp["score_bias"].astype(np.float32)   # float32 addition
        ids = np.argsort(-key, axis=1, kind="stable")[:, :k]
        w = np.take_along_axis(s, ids, axis=1)
    else:
        ids = np.argsort(-inp["logits"], axis=1, kind="stable")[:, :k]
        p = scipy.special.softmax(lg, axis=1)
        w = np.take_along_axis(p, ids, axis=1)
        if cs.renormalize:
            w = np.take_along_axis(np.exp(lg - lg.max(axis=1, keepdims=True)), ids, axis=1)
    if cs.renormalize:
        w = w / w.sum(axis=1, keepdims=True)
    w = w * cs.route_scale
    _, offsets, dst = _dispatch_by_sort(ids.astype(np.int64), E, cs.C)
    X = _widen(inp["x"])
    rnd = np.vectorize(oracle.round_bf16) if inp["x"].dtype == np.uint16 else (lambda a: a)
    out = np.zeros((T, cs.H))
    for t in range(T):
        for j in range(k):
            if dst[t, j] < 0:
                continue
            e = ids[t, j]
            A, B = _widen(inp["w13"][e]), _widen(inp["w2"][e])
            G = X[t] @ A[:I].T
            h = G * scipy.special.expit(G) * (X[t] @ A[I:].T) if cs.act == 0 else np.maximum(G, 0) ** 2
            out[t] += w[t, j] * (rnd(h) @ B.T)
    for s in range(cs.n_shared):
        A, B = _widen(inp["w13_sh"][s]), _widen(inp["w2_sh"][s])
        Is = cs.I_shared
        G = X @ A[:Is].T
        out += rnd(G * scipy.special.expit(G) * (X @ A[Is:].T)) @ B.T
    return ids, w, offsets, dst, out


@pytest.mark.parametrize("name,over", [
    ("tiny_fp32", {}),
    ("prefill_T256", dict(T=24, H=64, E=8, I=32, C=20)),
    ("decode_T8", dict(H=64, I=48, I_shared=40)),
    ("relu2_distinct_R8", dict(H=64, I=32)),
    ("skewed_bf16", dict(T=64, H=64, E=16, I=32, C=12)),
    ("sigmoid_relu2_R16", dict(H=64, I=32)),
    ("sigmoid_T2048", dict(T=24, H=64, E=8, I=32, C=20)),
])
def test_forward_against_library_layer(name, over):
    cs = synth.case(name, **over)
    inp = oracle.inputs_numpy(synth.make_inputs(cs))
    r = oracle.forward(cs, **inp)
    ids, w, offsets, dst, out = _numpy_layer(cs, inp)
    np.testing.assert_array_equal(r["ids"], ids)
    np.testing.assert_allclose(r["w"], w, rtol=1e-12)
    np.testing.assert_array_equal(r["offsets"], offsets)
    np.testing.assert_array_equal(r["route_dst"], dst)
    np.testing.assert_allclose(r["out"], out, rtol=1e-9, atol=1e-12 * np.abs(out).max())


def test_forward_deterministic_and_batch_invariant():
    cs = synth.case("prefill_T256", T=16, H=64, E=8, I=32, C=16)
    inp = oracle.inputs_numpy(synth.make_inputs(cs))
    a = oracle.forward(cs, **inp)
    b = oracle.forward(cs, **inp)
    np.testing.assert_array_equal(a["out"], b["out"])
    # capacity >= T: a token's output does not depend on the other tokens
    for t in (0, 5, 15):
        one = synth.replace(cs, T=1, C=1)
        sub = dict(inp, x=inp["x"][t:t + 1].copy(), logits=inp["logits"][t:t + 1].copy())
        s = oracle.forward(one, **sub)
        np.testing.assert_array_equal(s["out"][0], a["out"][t])


def test_forward_preselected_routes_poison_only_bad_tokens():
    cs = synth.case("prefill_T256", T=6, H=32, E=16, k=4, I=16, C=64)
    inp = oracle.inputs_numpy(synth.make_inputs(cs))
    ids = synth.bad_routes(6, 4, 16, "duplicate").numpy()
    w = np.full((6, 4), 0.25)
    r = oracle.forward(cs, **inp, ids_in=ids, w_in=w)
    assert r["n_bad"] == 1
    assert np.all(np.isnan(r["out"][1])) and np.all(np.isfinite(np.delete(r["out"], 1, 0)))
    good = ids.copy()
    good[1] = [0, 1, 2, 3]
    r2 = oracle.forward(cs, **inp, ids_in=good, w_in=w)
    # other tokens match a run where token 1 is well-formed (no capacity
    # effect: C = 64 >= T*k)
    for t in (0, 2, 3, 4, 5):
        np.testing.assert_allclose(r["out"][t], r2["out"][t], rtol=0, atol=0)
