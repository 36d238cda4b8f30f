"""Host-side checks of bench.py: the whole-layer work accounting against the
algorithmic bytes and flops of the workload table (count-first MoE layer:
weights of the touched and shared experts, logits, route metadata, x once,
row copy and h written and read, out written), and the one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


# (workload, kept rows R, touched experts, GB, GFLOP) of the seed-0 workloads
TABLE = [
    ("prefill_T256", 2048, 128, 1.638, 25.8),
    ("prefill_T2048", 16384, 128, 1.830, 206.2),
    ("prefill_T8192", 65536, 128, 2.488, 824.9),
    ("decode_T1", 6, 6, 0.139, 0.1),
    ("relu2_shared_R1", 9, 9, 0.057, 0.1),
    ("relu2_distinct_R16", 144, 144, 0.908, 0.9),
]


@pytest.mark.parametrize("name,R,touched,gb,gflop", TABLE)
def test_layer_work_matches_table(name, R, touched, gb, gflop):
    byts, flops = bench.layer_work(synth.case(name), R, touched)
    assert round(byts / 1e9, 3) == pytest.approx(gb, abs=1e-3)
    assert round(flops / 1e9, 1) == pytest.approx(gflop, abs=0.1)


def test_layer_roofline_bound_and_fraction():
    res = {"cs": synth.case("prefill_T8192"), "R": 65536, "touched": 128,
           "wall": 2 * 1.0e-3, "steps": 2}
    lr = bench.layer_roofline(res, ceiling_gbps=4000.0)
    assert lr["bound"] == "mfma"                      # 824.9 GFLOP > 2.488 GB at the ridge
    assert lr["t_roofline_us"] == pytest.approx(329.96, abs=0.01)
    assert lr["frac"] == pytest.approx(0.32996, abs=1e-4)
    # at 4 TB/s the byte term (622 us) exceeds the flop term
    assert lr["frac_measured"] == pytest.approx(2.488270848e9 / 4e12 / 1e-3, abs=1e-3)


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr


def test_dispatch_bytes_count_the_row_copy():
    # moe_dispatch with x_disp: ids read, counts / offsets / route_dst /
    # row_src written, every token row read once, one copy per kept route
    cs = synth.case("prefill_T2048")
    route, disp = bench.dispatch_bytes(cs, R=16384)
    Q = 2048 * 8
    assert route == 2048 * 128 * 4 + Q * 8
    assert disp == Q * 4 + 128 * 4 + 129 * 4 + Q * 4 + 16384 * 4 + 2048 * 2048 * 2 + 16384 * 2048 * 2
    assert round(disp / 1e6, 1) == 75.7


def test_forward_scatter_bytes_are_metadata_only_for_bf16():
    # bf16 layers place routes only (the expert GEMM reads x in place);
    # float32 layers copy the rows
    bf = bench.stage_bytes_flops(synth.case("prefill_T2048"), 16384, 128, 2, 2)
    Q = 2048 * 8
    assert bf["scatter"][0] == Q * 16 + Q * 4
    f32 = synth.case("tiny_fp32")
    bf32 = bench.stage_bytes_flops(f32, 128, 16, 4, 4)
    assert bf32["scatter"][0] == 64 * 256 * 4 + 128 * 256 * 4 + 128 * 16 + 128 * 4


def test_layer_roofline_divides_by_the_plain_step_count():
    # a sweep workload times more plain steps than event-timed ones: the
    # plain wall time is divided by its own step count
    cs = synth.case("prefill_T8192")
    a = bench.layer_roofline({"cs": cs, "R": 65536, "touched": 128, "wall": 2e-3, "steps": 2})
    b = bench.layer_roofline({"cs": cs, "R": 65536, "touched": 128, "wall": 8e-3, "steps": 2,
                              "n_plain": 8})
    assert a["frac"] == pytest.approx(b["frac"])


def test_decode_launch_bytes_include_the_shared_experts():
    # decode T=1: the gate/up launch streams the 6 routed experts' gate/up
    # weights and the 2 shared experts' (and routes the token itself); the
    # down-projection launch both down projections.  The counter summary of
    # these launches reads 92.6 MB and 46.5 MB.
    cs = synth.case("decode_T1")
    assert bench.decode_mode(cs) and bench.fused_mode(cs)
    bf = bench.stage_bytes_flops(cs, 6, 6, 2, 2)
    w13 = 2 * 1408 * 2048 * 2
    w2 = 1408 * 2048 * 2
    assert bf["gemm1"][0] > 8 * w13 and bf["gemm1"][0] < 8 * w13 + 2e5
    assert bf["gemm2"][0] > 8 * w2 and bf["gemm2"][0] < 8 * w2 + 2e5
    assert bf["shared"] == (0, 0) and bf["route"] == (0, 0)
    assert round(bf["gemm1"][0] / 1e6, 1) == pytest.approx(92.3, abs=0.5)
    # prefill: the shared experts (none here) and the routing keep their stages
    p = bench.stage_bytes_flops(synth.case("prefill_T2048"), 16384, 128, 2, 2)
    assert p["route"][0] == 2048 * 128 * 4 + 2048 * 8 * 8


def test_float32_layer_uses_the_fp32_peak():
    cs = synth.case("tiny_fp32")
    assert bench.flops_peak_tflops(cs) == bench.F32_PEAK_TFLOPS
    lr = bench.layer_roofline({"cs": cs, "R": 128, "touched": 16, "wall": 1e-5, "steps": 1})
    assert lr["bound"] == "hbm"


def test_cpu_sample_is_bounded():
    for name in ("skewed_bf16", "prefill_T2048", "decode_T1", "tiny_fp32"):
        cs = synth.case(name)
        n = bench.cpu_sample_tokens(cs)
        assert 1 <= n <= cs.T
        n_w = 2 * cs.I
        work = n * cs.k * 2 * cs.H * (n_w + cs.I) / bench.ORACLE_FLOPS
        assert work < 2 * bench.CPU_SAMPLE_S
