"""The bf16 output comparison of the parity tests can fail.

The layer's contract for bf16 outputs is max|d| <= 1e-2 * max|ref| + 1e-3.
These CPU checks show that, as the parity tests apply it, an all-zero
result and a result 5 % off are rejected, a result within rounding is
accepted, and a reference small enough for the 1e-3 floor to cover an
all-zero result is refused outright.  They also check that the unit-scale
parity inputs give O(1) oracle outputs on a reduced prefill and a reduced
decode shape, while the workloads' own N(0, 0.02^2) scale would not."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import VacuousComparison, assert_bf16_close, bf16_tolerance


def _ref(scale=1.0, seed=0):
    g = np.random.default_rng(seed)
    return g.standard_normal((64, 256)) * scale


def test_zero_output_fails():
    ref = _ref()
    with pytest.raises(AssertionError, match="max\\|d\\|"):
        assert_bf16_close(torch.zeros(ref.shape, dtype=torch.bfloat16), ref, "zeros")


@pytest.mark.parametrize("scale", [0.04, 0.1, 1.0, 30.0])
def test_five_percent_error_fails(scale):
    ref = _ref(scale)
    got = torch.from_numpy(ref * 1.05).to(torch.bfloat16)
    with pytest.raises(AssertionError, match="max\\|d\\|"):
        assert_bf16_close(got, ref, "5 % off")


@pytest.mark.parametrize("scale", [0.04, 1.0, 30.0])
def test_rounded_output_passes(scale):
    ref = _ref(scale)
    assert_bf16_close(torch.from_numpy(ref).to(torch.bfloat16), ref, "bf16 of ref")


@pytest.mark.parametrize("scale", [1e-4, 1e-3, 0.005])
def test_vacuous_reference_is_refused(scale):
    ref = _ref(scale)
    # the 1e-3 floor is above 2.5 % of max|ref| here
    assert 1e-3 > 0.025 * np.abs(ref).max()
    with pytest.raises(VacuousComparison):
        bf16_tolerance(ref)
    with pytest.raises(VacuousComparison):
        assert_bf16_close(torch.zeros(ref.shape, dtype=torch.bfloat16), ref, "tiny")


def test_nonfinite_pattern_must_match():
    ref = _ref()
    ref[3, 5] = np.nan
    got = torch.from_numpy(np.nan_to_num(ref)).to(torch.bfloat16)
    with pytest.raises(AssertionError, match="finiteness"):
        assert_bf16_close(got, ref, "nan")


@pytest.mark.parametrize("name,over", [
    ("prefill_T256", dict(T=96, H=256, E=8, k=2, I=128, C=96)),
    ("decode_T8", dict(T=8, H=256, I=128, I_shared=128, C=8)),
    ("relu2_distinct_R8", dict(H=256, I=256)),
])
def test_unit_scale_outputs_are_order_one(name, over):
    base = synth.case(name, **over)
    unit = synth.unit_scale(base)
    big = oracle.forward(unit, **oracle.inputs_numpy(synth.make_inputs(unit)))["out"]
    small = oracle.forward(base, **oracle.inputs_numpy(synth.make_inputs(base)))["out"]
    bf16_tolerance(big)                       # accepted
    assert np.abs(big).max() > 0.1
    with pytest.raises(VacuousComparison):    # the benchmark scale would be vacuous
        bf16_tolerance(small)
