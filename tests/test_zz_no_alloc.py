"""moe_forward_static (no workspace argument, no allocation) against
moe_forward with a caller workspace, through the C ABI.

Three calls in a row share the library's per-device array: a tiled prefill
batch whose routes span two count blocks (the count kernel's arrival
ticket), then a smaller decode batch with shared experts (single-workgroup
dispatch, slot-indexed GEMMs), then the first batch again.  Each call's
metadata must equal moe_forward's bit for bit and its output must agree to
the layer's bf16 contract (the same kernels run, so bit-equal is expected
and checked too).  A problem whose workspace exceeds the array is refused
before anything is enqueued."""
import numpy as np
import pytest
import torch

import routing_dispatch_expert_amd as rde
import synth
from gpu_helpers import DEV, assert_bf16_close, np_i32, parity_case, problem, r_max, workspace

pytestmark = pytest.mark.gpu

CASES = [
    ("prefill_two_count_blocks", parity_case("prefill_T256", T=300, H=256, E=16, k=8, I=128,
                                             C=300)),
    ("decode_shared_smaller", parity_case("decode_T8", T=40, H=256, I=128, I_shared=128, C=40)),
]


def _meta(cs):
    R = max(r_max(cs), 1)
    return dict(ids=torch.full((cs.T, cs.k), -7, dtype=torch.int32, device=DEV),
                w=torch.full((cs.T, cs.k), -7.0, dtype=torch.float32, device=DEV),
                counts=torch.full((cs.E,), -7, dtype=torch.int32, device=DEV),
                offsets=torch.full((cs.E + 1,), -7, dtype=torch.int32, device=DEV),
                row_src=torch.full((R,), -7, dtype=torch.int32, device=DEV),
                route_dst=torch.full((cs.T, cs.k), -7, dtype=torch.int32, device=DEV))


def _run(cs, inp, static):
    p = problem(cs)
    out = torch.full((cs.T, cs.H), float("nan"), dtype=torch.bfloat16, device=DEV)
    meta = _meta(cs)
    args = (p, inp.x, inp.logits, inp.score_bias, None, None, inp.w13, inp.w2, inp.s13, inp.s2,
            inp.w13_sh, inp.w2_sh, out, meta)
    if static:
        rde.moe_forward_static(*args)
    else:
        ws = workspace(p)
        rde.moe_forward(*args, ws)
        assert rde.moe_error(ws) == 0
    torch.cuda.synchronize()
    return out, meta


def test_static_matches_workspace_entry_point():
    for name, cs in CASES + CASES[:1]:
        print("[gpu-case] forward_static", name, cs.T, cs.E, cs.k, flush=True)
        assert rde.moe_workspace_bytes(problem(cs)) <= rde.MOE_STATIC_SCRATCH_BYTES
        inp = synth.make_inputs(cs, DEV)
        ref, meta_ref = _run(cs, inp, static=False)
        got, meta = _run(cs, inp, static=True)
        for key in meta:
            assert torch.equal(meta[key], meta_ref[key]), (name, key)
        assert_bf16_close(got, ref.double().cpu().numpy(), f"{name} out")
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), name


def test_static_refuses_problems_beyond_its_array():
    cs = synth.case("prefill_T2048")
    p = problem(cs)
    assert rde.moe_workspace_bytes(p) > rde.MOE_STATIC_SCRATCH_BYTES
    st = rde.lib().moe_forward_static(rde.C.byref(p), None, None, None, None, None, None, None,
                                      None, None, None, None, None, None, None)
    assert st == rde.MOE_ERR_WORKSPACE
