"""Run in a child process by test_gpu_count_handoff.py with MOE_COUNT_DELAY
set in its environment (the library reads it once): block 0 of the count
kernel holds back its arrival ticket, so it is the last block to arrive and
the one that reads every other block's write-through totals and scans them.
moe_dispatch (with the row copy) on more than 4096 routes (below that one
workgroup places every route) and moe_forward on batches whose per-block
totals also number more than 2048 (below that the metadata scatter scans
them itself and the count blocks hand nothing over) must still match the
oracle bit for bit on their metadata.  Prints "ok" on success."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [os.path.dirname(HERE), HERE]

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
import routing_dispatch_expert_amd as rde  # noqa: E402
import synth  # noqa: E402
from gpu_helpers import DEV, np_i32, parity_case, problem, r_max, workspace  # noqa: E402


def dispatch_case():
    # 2100 tokens x top-8 = 16800 routes: 9 count blocks x 256 experts, with the hand-off
    cs = parity_case("prefill_T2048", T=2100, H=256, E=256, k=8, I=128, C=300)
    print("[case] dispatch", cs.T, cs.E, cs.k, flush=True)
    x = synth.make_x(cs)
    ids, _ = oracle.route(synth.make_logits(cs).numpy(), cs.k)
    d = oracle.dispatch(ids, cs.E, cs.C)
    R = int(d["offsets"][-1])
    xo = oracle.gather_rows(oracle.from_torch(x), d["row_src"], R, cs.k)
    p = problem(cs)
    ws = workspace(p)
    Rm = r_max(cs)
    for rep in range(3):
        g = dict(counts=torch.empty(cs.E, dtype=torch.int32, device=DEV),
                 offsets=torch.empty(cs.E + 1, dtype=torch.int32, device=DEV),
                 row_src=torch.full((Rm,), 12345, dtype=torch.int32, device=DEV),
                 route_dst=torch.empty((cs.T, cs.k), dtype=torch.int32, device=DEV))
        x_disp = torch.zeros((Rm, cs.H), dtype=torch.bfloat16, device=DEV)
        rde.moe_dispatch(p, x.to(DEV), torch.from_numpy(ids).to(DEV), g["counts"], g["offsets"],
                         g["row_src"], g["route_dst"], x_disp, ws)
        assert rde.moe_error(ws) == 0
        for key in ("counts", "offsets", "row_src", "route_dst"):
            np.testing.assert_array_equal(np_i32(g[key]), d[key], err_msg=f"{key} rep {rep}")
        assert np.array_equal(oracle.from_torch(x_disp[:R].cpu()), xo), "x_disp"


def forward_case():
    # 4800 routes: 3 count blocks x 1024 experts
    cs = parity_case("prefill_T256", T=600, H=256, E=1024, k=8, I=128, C=200)
    print("[case] forward", cs.T, cs.E, cs.k, flush=True)
    inp = synth.make_inputs(cs, DEV)
    p = problem(cs)
    ws = workspace(p)
    meta = dict(route_dst=torch.empty((cs.T, cs.k), dtype=torch.int32, device=DEV),
                offsets=torch.empty(cs.E + 1, dtype=torch.int32, device=DEV),
                row_src=torch.empty(r_max(cs), dtype=torch.int32, device=DEV))
    out = torch.empty((cs.T, cs.H), dtype=torch.bfloat16, device=DEV)
    rde.moe_forward(p, inp.x, inp.logits, None, None, None, inp.w13, inp.w2, None, None, None, None,
                    out, meta, ws)
    assert rde.moe_error(ws) == 0
    r = oracle.forward(cs, **oracle.inputs_numpy(inp.to("cpu")))
    for key in ("route_dst", "offsets", "row_src"):
        np.testing.assert_array_equal(np_i32(meta[key]), r[key], err_msg=key)
    d = np.abs(out.float().cpu().numpy() - r["out"]).max()
    assert d <= 1e-2 * np.abs(r["out"]).max() + 1e-3, d


if __name__ == "__main__":
    assert int(os.environ.get("MOE_COUNT_DELAY", "0")) > 0
    dispatch_case()
    forward_case()
    torch.cuda.synchronize()
    print("ok", flush=True)
