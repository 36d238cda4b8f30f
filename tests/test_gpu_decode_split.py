"""The slot-indexed decode GEMMs with each split of a unit over a
workgroup's wavefronts (1, 2 or 4), forced through MOE_DECODE_SPLIT (read by
the library on every call) on shapes with many rounds of units: every form
must meet the oracle's bf16 contract with bit-exact metadata.  The 2-way
split pads the second pair's last position past the end of the units, so the
shapes are chosen with unit counts that are not a multiple of the pairs."""
import contextlib
import os

import numpy as np
import pytest
import torch

import oracle
import routing_dispatch_expert_amd as rde
import synth
from gpu_helpers import DEV, act_dtype, assert_bf16_close, np_i32, parity_case, problem, r_max, workspace

pytestmark = pytest.mark.gpu

# decode with shared experts (several rounds of units per launch), 8 distinct
# ReLU-square rows (72 touched experts), one ReLU-square row (one round), and
# e4m3 weights on a reduced decode shape
SHAPES = {
    "decode_T8": {},
    "relu2_distinct_R8": {},
    "relu2_shared_R1": {},
    "decode_fp8": dict(base="skewed_fp8", T=16, H=256, E=32, k=4, I=256, C=16),
}


@contextlib.contextmanager
def split(v):
    old = os.environ.get("MOE_DECODE_SPLIT")
    os.environ["MOE_DECODE_SPLIT"] = str(v)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("MOE_DECODE_SPLIT", None)
        else:
            os.environ["MOE_DECODE_SPLIT"] = old


def _case(name):
    over = dict(SHAPES[name])
    base = over.pop("base", name)
    return parity_case(base, **over)


@pytest.mark.parametrize("name", list(SHAPES))
def test_decode_splits_match_oracle(name):
    cs = _case(name)
    assert cs.T * cs.k <= 12 * cs.E, "a decode-shaped batch"
    inp = synth.make_inputs(cs, DEV)
    p = problem(cs)
    ws = workspace(p)
    r = oracle.forward(cs, **oracle.inputs_numpy(inp.to("cpu")))
    outs = {}
    for v in (1, 2, 4):
        print(f"[gpu-case] decode split {name} ways={v}", flush=True)
        out = torch.empty((cs.T, cs.H), dtype=act_dtype(cs), device=DEV)
        meta = dict(route_dst=torch.empty((cs.T, cs.k), dtype=torch.int32, device=DEV),
                    offsets=torch.empty(cs.E + 1, dtype=torch.int32, device=DEV),
                    row_src=torch.empty(max(r_max(cs), 1), dtype=torch.int32, device=DEV))
        with split(v):
            rde.moe_forward(p, inp.x, inp.logits, inp.score_bias, None, None, inp.w13, inp.w2,
                            inp.s13, inp.s2, inp.w13_sh, inp.w2_sh, out, meta, ws)
            assert rde.moe_error(ws) == 0
        for key in ("route_dst", "offsets"):
            np.testing.assert_array_equal(np_i32(meta[key]), r[key], err_msg=f"{key} ways={v}")
        np.testing.assert_array_equal(np_i32(meta["row_src"])[:len(r["row_src"])], r["row_src"])
        assert_bf16_close(out, r["out"], f"{name} ways={v}")
        outs[v] = out.float().cpu().numpy()
    # the forms differ only in how each unit's K is summed
    ref = np.abs(r["out"]).max()
    for v in (2, 4):
        assert np.abs(outs[v] - outs[1]).max() <= 2e-2 * ref
