"""Seeded synthetic inputs for one MoE layer forward.

This module only draws numbers and lays them out; it holds none of the
layer's arithmetic (no routing, dispatch, FFN or combine).  Both the HIP
path and the CPU oracle are fed from the very same bytes it produces: a test
generates a case once, hands host copies to the oracle and device copies to
the library.

Workloads (shapes, value distributions and routing structure) follow the
problem statements of the pages:
  * "Extend MoEPacked for Bolt ReLU-square routing and BF16 IQ2 precision"
    (onnxruntime PR 33963, "Measured CUDA kernel latency"): hidden 1024, 240
    experts, top-9, ReLU-square experts, selected logits +16 and the others
    -16, rows in {1, 8, 16}, routes shared or distinct across rows.
  * the afdEP count-first validation record ("setup"): bf16, hidden 2048,
    top-8 of 128 experts, capacity 2048, the benchmark bucket is the token
    count.
  * the DeepSeek fleet megakernel report on MI300X (per-op table, tile sweep):
    hidden 2048, 64 routed experts top-6 plus 2 shared experts, expert
    intermediate 1408, batch-1 decode.

Every tensor has its own generator seeded from (seed, tensor id, expert), so
any single expert's weights can be regenerated on its own.  Values are drawn
in float32 with torch's generator on the requested device and rounded to
bf16 (round-to-nearest-even) where the case is bf16.  fp8 weights are
quantised per output row at generation time: scale = max|w| / 448 and the
code is the OCP e4m3fn value nearest to w / scale.

Two value scales.  The workloads' own scale draws x and every weight from
N(0, 0.02^2) (the benchmark inputs).  `unit_scale` gives the same shapes and
routes with x ~ N(0, 1) and each weight matrix drawn N(0, 1/K) for its input
width K (H for w13, I for w2), so every layer output is O(1): a comparison
against the oracle with an absolute floor of 1e-3 then measures the kernel,
not the floor.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import torch

# activation kinds and storage formats, mirrored by the C-ABI enums
ACT_SWIGLU = 0
ACT_RELU2 = 1
FMT_F32 = 0
FMT_BF16 = 1
FMT_E4M3 = 2
SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1

_TENSOR_IDS = {"x": 1, "logits": 2, "w13": 3, "w2": 4, "w13_sh": 5, "w2_sh": 6,
               "score_bias": 7}


@dataclass(frozen=True)
class Case:
    """One synthetic workload.  Shapes follow the row-major layouts:
    x [T,H], logits [T,E] f32, w13 [E,2I,H] (SwiGLU: gate rows then up rows)
    or [E,I,H] (ReLU-square), w2 [E,H,I], shared w13_sh [S,2Is,H],
    w2_sh [S,H,Is]."""
    name: str
    T: int
    H: int
    E: int
    k: int
    I: int
    C: int
    act: int = ACT_SWIGLU
    act_fmt: int = FMT_BF16
    w_fmt: int = FMT_BF16
    n_shared: int = 0
    I_shared: int = 0
    renormalize: int = 0
    score_func: int = SCORE_SOFTMAX    # sigmoid: selection on sigmoid + bias
    route_scale: float = 1.0           # multiplies every routing weight
    bias_std: float = 0.0              # sigmoid correction bias N(0, bias_std^2); 0 = none
    logits_kind: str = "normal"        # normal | pm16_shared | pm16_distinct | zipf
    zipf_s: float = 1.1
    w_std: float = 0.02
    x_std: float = 0.02
    fan_in: bool = False               # weights N(0, 1/K) for input width K (w_std unused)
    seed: int = 0

    @property
    def w13_rows(self) -> int:
        return 2 * self.I if self.act == ACT_SWIGLU else self.I

    @property
    def r_max(self) -> int:
        return min(self.T * self.k, self.E * self.C)


def _cases() -> Dict[str, Case]:
    c: Dict[str, Case] = {}
    # Tiny fp32 layer: everything float32.
    c["tiny_fp32"] = Case("tiny_fp32", T=64, H=256, E=16, k=2, I=512, C=64,
                          act_fmt=FMT_F32, w_fmt=FMT_F32)
    # Prefill dispatch shape, bucket swept over the token count.
    for T in (256, 2048, 8192):
        c[f"prefill_T{T}"] = Case(f"prefill_T{T}", T=T, H=2048, E=128, k=8,
                                  I=1024, C=2048)
    # Decode shape with two always-on shared experts; capacity = T (no drops).
    for T in (1, 8, 32):
        c[f"decode_T{T}"] = Case(f"decode_T{T}", T=T, H=2048, E=64, k=6,
                                 I=1408, C=T, n_shared=2, I_shared=1408)
    # Wide-expert ReLU-square shape, +-16 logits.
    for rows in (1, 8, 16):
        for kind in ("distinct", "shared"):
            c[f"relu2_{kind}_R{rows}"] = Case(
                f"relu2_{kind}_R{rows}", T=rows, H=1024, E=240, k=9, I=1536,
                C=rows, act=ACT_RELU2, logits_kind=f"pm16_{kind}")
    # Large skewed prefill, Zipf(1.1) per-expert popularity, capacity 512.
    c["skewed_bf16"] = Case("skewed_bf16", T=8192, H=7168, E=256, k=8, I=2048,
                            C=512, logits_kind="zipf")
    c["skewed_fp8"] = replace(c["skewed_bf16"], name="skewed_fp8",
                              w_fmt=FMT_E4M3)
    # Sigmoid routing with a float32 selection-only correction bias and
    # normalised, scaled weights, on the ReLU-square expert shape (16 rows)
    # and on the 2048-token prefill shape.
    c["sigmoid_relu2_R16"] = Case("sigmoid_relu2_R16", T=16, H=1024, E=240, k=9, I=1536,
                                  C=16, act=ACT_RELU2, score_func=SCORE_SIGMOID,
                                  renormalize=1, route_scale=2.5, bias_std=0.1)
    c["sigmoid_T2048"] = replace(c["prefill_T2048"], name="sigmoid_T2048",
                                 score_func=SCORE_SIGMOID, renormalize=1,
                                 route_scale=2.5, bias_std=0.1)
    return c


CASES: Dict[str, Case] = _cases()


def case(name: str, **over) -> Case:
    """Look up a named workload, optionally overriding fields (for reduced
    sizes in tests: same structure, fewer tokens or experts)."""
    base = CASES[name]
    return replace(base, **over) if over else base


def unit_scale(cs: Case) -> Case:
    """The same workload with O(1) outputs: x ~ N(0, 1), w13 ~ N(0, 1/H),
    w2 ~ N(0, 1/I) (shared experts: 1/H and 1/I_shared); e4m3 weights are
    quantised from those."""
    return replace(cs, x_std=1.0, fan_in=True)


def _gen(seed: int, tensor: str, expert: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    # a fixed mixing of the three indices into one 63-bit seed
    s = (seed * 1_000_003 + _TENSOR_IDS[tensor]) * 1_000_033 + (expert + 1)
    g.manual_seed(s & ((1 << 63) - 1))
    return g


def _normal(shape, std, seed, tensor, expert, device) -> torch.Tensor:
    g = _gen(seed, tensor, expert, device)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _store(t32: torch.Tensor, fmt: int) -> torch.Tensor:
    if fmt == FMT_F32:
        return t32
    if fmt == FMT_BF16:
        return t32.to(torch.bfloat16)
    raise ValueError(fmt)


def _quant_e4m3_rows(t32: torch.Tensor):
    """Per-output-row fp8 e4m3fn codes (uint8) and float32 scales."""
    amax = t32.abs().amax(dim=-1, keepdim=True).clamp_min(1e-30)
    scale = (amax / 448.0).to(torch.float32)
    q = (t32 / scale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.squeeze(-1).contiguous()


def make_logits(cs: Case, device="cpu") -> torch.Tensor:
    T, E = cs.T, cs.E
    if cs.logits_kind == "normal":
        return _normal((T, E), 1.0, cs.seed, "logits", -1, device)
    if cs.logits_kind == "zipf":
        base = _normal((T, E), 1.0, cs.seed, "logits", -1, device)
        # log of a Zipf(s) popularity by expert index
        bias = -cs.zipf_s * torch.log(torch.arange(1, E + 1, device=device,
                                                   dtype=torch.float64))
        return (base.double() + bias).to(torch.float32)
    if cs.logits_kind in ("pm16_shared", "pm16_distinct"):
        lg = torch.full((T, E), -16.0, dtype=torch.float32, device=device)
        for t in range(T):
            first = 0 if cs.logits_kind == "pm16_shared" else t * cs.k
            if first + cs.k > E:
                raise ValueError("distinct routes need T*k <= E")
            lg[t, first:first + cs.k] = 16.0
        return lg
    raise ValueError(cs.logits_kind)


def make_score_bias(cs: Case, device="cpu") -> Optional[torch.Tensor]:
    """float32 [E] correction bias of sigmoid routing, or None."""
    if cs.score_func != SCORE_SIGMOID or cs.bias_std == 0.0:
        return None
    return _normal((cs.E,), cs.bias_std, cs.seed, "score_bias", -1, device)


def make_x(cs: Case, device="cpu") -> torch.Tensor:
    return _store(_normal((cs.T, cs.H), cs.x_std, cs.seed, "x", -1, device),
                  cs.act_fmt)


def make_expert_weights(cs: Case, e: int, device="cpu", shared: bool = False):
    """Weights of one expert: (w13 [rows,H], w2 [H,I], s13 or None, s2 or None)."""
    I = cs.I_shared if shared else cs.I
    rows = 2 * I if (shared or cs.act == ACT_SWIGLU) else I
    t13, t2 = ("w13_sh", "w2_sh") if shared else ("w13", "w2")
    std13 = 1.0 / math.sqrt(cs.H) if cs.fan_in else cs.w_std
    std2 = 1.0 / math.sqrt(I) if cs.fan_in else cs.w_std
    a = _normal((rows, cs.H), std13, cs.seed, t13, e, device)
    b = _normal((cs.H, I), std2, cs.seed, t2, e, device)
    if cs.w_fmt == FMT_E4M3 and not shared:
        q13, s13 = _quant_e4m3_rows(a)
        q2, s2 = _quant_e4m3_rows(b)
        return q13, q2, s13, s2
    fmt = FMT_BF16 if (shared and cs.w_fmt == FMT_E4M3) else cs.w_fmt
    return _store(a, fmt), _store(b, fmt), None, None


@dataclass
class Inputs:
    case: Case
    x: torch.Tensor
    logits: torch.Tensor
    w13: torch.Tensor
    w2: torch.Tensor
    s13: Optional[torch.Tensor] = None
    s2: Optional[torch.Tensor] = None
    w13_sh: Optional[torch.Tensor] = None
    w2_sh: Optional[torch.Tensor] = None
    score_bias: Optional[torch.Tensor] = None

    def to(self, device) -> "Inputs":
        mv = lambda t: None if t is None else t.to(device)
        return Inputs(self.case, mv(self.x), mv(self.logits), mv(self.w13),
                      mv(self.w2), mv(self.s13), mv(self.s2), mv(self.w13_sh),
                      mv(self.w2_sh), mv(self.score_bias))


def make_inputs(cs: Case, device="cpu", experts: Optional[List[int]] = None) -> Inputs:
    """All tensors of a case on `device`.  `experts` restricts generation to a
    subset of expert ids (the others stay zero): used for full-size cases
    where only the touched experts are needed on the host."""
    x = make_x(cs, device)
    logits = make_logits(cs, device)
    rows, I, H, E = cs.w13_rows, cs.I, cs.H, cs.E
    if cs.w_fmt == FMT_E4M3:
        w13 = torch.zeros((E, rows, H), dtype=torch.uint8, device=device)
        w2 = torch.zeros((E, H, I), dtype=torch.uint8, device=device)
        s13 = torch.zeros((E, rows), dtype=torch.float32, device=device)
        s2 = torch.zeros((E, H), dtype=torch.float32, device=device)
    else:
        dt = torch.float32 if cs.w_fmt == FMT_F32 else torch.bfloat16
        w13 = torch.zeros((E, rows, H), dtype=dt, device=device)
        w2 = torch.zeros((E, H, I), dtype=dt, device=device)
        s13 = s2 = None
    for e in (range(E) if experts is None else experts):
        a, b, sa, sb = make_expert_weights(cs, e, device)
        w13[e].copy_(a)
        w2[e].copy_(b)
        if sa is not None:
            s13[e].copy_(sa)
            s2[e].copy_(sb)
    w13_sh = w2_sh = None
    if cs.n_shared:
        sh = [make_expert_weights(cs, s, device, shared=True) for s in range(cs.n_shared)]
        w13_sh = torch.stack([a for a, _, _, _ in sh]).contiguous()
        w2_sh = torch.stack([b for _, b, _, _ in sh]).contiguous()
    return Inputs(cs, x, logits, w13, w2, s13, s2, w13_sh, w2_sh, make_score_bias(cs, device))


def bad_routes(T: int, k: int, E: int, kind: str, seed: int = 0) -> torch.Tensor:
    """Preselected int32 ids [T,k] (distinct experts per token) with one
    malformed route of the count-first validation record's classes planted in
    token 1: "dummy" = the index E of a dummy expert just past the real ones,
    "negative" = -1, "wide" = the largest int32, "duplicate" = slot 1 repeats
    slot 0; "none" plants nothing."""
    g = torch.Generator().manual_seed(seed)
    ids = torch.stack([torch.randperm(E, generator=g)[:k] for _ in range(T)]).to(torch.int32)
    if kind == "dummy":
        ids[1, k // 2] = E
    elif kind == "negative":
        ids[1, 0] = -1
    elif kind == "wide":
        ids[1, k - 1] = 2 ** 31 - 1
    elif kind == "duplicate":
        if k < 2:
            raise ValueError("duplicate needs k >= 2")
        ids[1, 1] = ids[1, 0]
    elif kind != "none":
        raise ValueError(kind)
    return ids


def cancellation_inputs(T: int, H: int, E: int, k: int, I: int, act: int, device="cpu",
                        seed: int = 0) -> Inputs:
    """Large terms that cancel across K tiles, with unit terms kept apart.

    The cancellation regression of "Extend MoEPacked for Bolt ReLU-square
    routing and BF16 IQ2 precision" (PR 33963, "Motivation and Context" and
    the commit that keeps unit contributions outside large-magnitude
    tensor-core partials) separates results that differ only in how large
    partial sums absorb unit terms.  Here every product is an integer (or, in
    the second SwiGLU projection, a bf16 value of modest size) and every
    partial sum stays below 2^24, so the exact result does not depend on the
    order in which K is summed, inside an MFMA or across K tiles:

      x[t, p+] = x[t, p-] = 2^10 and w13[e, i, p+] = 2^10, w13[e, i, p-] = -2^10
        on every row i: the two 2^20 products cancel; p+ lies in the first
        64-wide K block, p- in the last;
      x[t, pb] = 8 and w13[e, i, pb] = 8 (ReLU-square, or the gate and up
        rows of SwiGLU) only on two rows b1 < b2 of each expert, which then
        carry 64 + (unit terms), i.e. h ~ 64^2 (ReLU-square) or ~ 12^2-sized
        values for SwiGLU (there pb gets 3.5 and 3.5, see below);
      w2[e, o, b1] = +L2, w2[e, o, b2] = -L2 with h[b1] = h[b2] (identical
        rows), so the down projection's large terms cancel too; b1 lies in
        the first K block of I, b2 in the last;
      unit terms: x in {0, 1} and weights in {-1, 0, 1}, sparse, only in
        16-wide K chunks that hold none of the large positions.

    Logits are +16 on k experts per token ((t + j) mod E) and -16 elsewhere,
    so with k in {1, 2, 4, 8} every weight is exactly 1/k.  ReLU-square
    results are exact integers (or halves, quarters ...) on both sides; SwiGLU
    results differ only by the rounding of silu.  bf16 storage throughout."""
    if H % 64 or I % 64 or H < 128 or I < 128:
        raise ValueError("H and I must be multiples of 64, at least 128")
    g = torch.Generator().manual_seed(seed * 7919 + 101)
    p_plus, p_minus, p_big = 3, H - 5, H // 2 + 1
    b1, b2 = 2, I - 3
    big_cols = {p_plus // 16, p_minus // 16, p_big // 16}
    unit_k = torch.tensor([c // 16 not in big_cols for c in range(H)])
    unit_i = torch.tensor([c // 16 not in {b1 // 16, b2 // 16} for c in range(I)])

    x = (torch.rand((T, H), generator=g) < 0.125).float() * unit_k
    x[:, p_plus] = 1024.0
    x[:, p_minus] = 1024.0
    x[:, p_big] = 8.0 if act == ACT_RELU2 else 3.5

    def sparse_pm1(shape, density):
        r = torch.rand(shape, generator=g)
        s = torch.where(torch.rand(shape, generator=g) < 0.5, -1.0, 1.0)
        return (r < density).float() * s

    rows = 2 * I if act == ACT_SWIGLU else I
    w13 = sparse_pm1((E, rows, H), 1.0 / 16) * unit_k
    w13[:, :, p_plus] = 1024.0
    w13[:, :, p_minus] = -1024.0
    big_rows = [b1, b2] + ([I + b1, I + b2] if act == ACT_SWIGLU else [])
    # identical rows b1 / b2 (and their up rows): equal h, exact cancellation
    w13[:, b2] = w13[:, b1]
    if act == ACT_SWIGLU:
        w13[:, I + b2] = w13[:, I + b1]
    for r in big_rows:
        w13[:, r, p_big] = 8.0 if act == ACT_RELU2 else 3.5
    w2 = sparse_pm1((E, H, I), 1.0 / 8) * unit_i
    L2 = 1024.0 if act == ACT_RELU2 else 32.0
    w2[:, :, b1] = L2
    w2[:, :, b2] = -L2

    lg = torch.full((T, E), -16.0)
    for t in range(T):
        for j in range(k):
            lg[t, (t + j) % E] = 16.0
    cs = Case("cancellation", T=T, H=H, E=E, k=k, I=I, C=T, act=act)
    bf = lambda t: t.to(torch.bfloat16).to(device)
    return Inputs(cs, bf(x), lg.to(device), bf(w13), bf(w2))
