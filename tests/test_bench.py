"""Host-side checks of bench.py: the algorithmic work it prices each step at
(closed forms of the layer's parameter counts) and its one-GPU contract.
Nothing here touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import moe_inputs as mi  # noqa: E402

H, E, K, I, Is = 2048, 256, 8, 512, 512
EXPERT_BYTES = 2 * 3 * H * I          # gate, up and down of one expert, bf16: 6,291,456 B


def test_step_bytes_one_token_decode():
    # 8 touched experts + shared expert + router + shared gate + x and out.
    nbytes, flops = bench.step_work(mi.FULL, 1, 8)
    assert nbytes == 8 * EXPERT_BYTES + EXPERT_BYTES + 2 * E * H + 2 * H + 2 * 2 * H == 57_683_968
    # Per token: K experts (3 H I multiply-adds each), the shared expert, the router and the gate.
    assert flops == 2 * (K * 3 * H * I + 3 * H * Is + E * H + H) == 57_675_776


def test_step_bytes_prefill_all_experts():
    nbytes, flops = bench.step_work(mi.FULL, 4096, 256)
    assert nbytes == 256 * EXPERT_BYTES + EXPERT_BYTES + 2 * E * H + 2 * H + 4096 * 2 * 2 * H == 1_651_511_296
    assert flops == 4096 * 57_675_776 == 236_239_978_496


def test_phase_work_adds_up_to_the_step():
    T, U = 64, 222.625
    parts = [bench.phase_work(mi.FULL, T, U, p) for p in ("router", "dispatch", "gate_up", "down", "combine")]
    _, step_flops = bench.step_work(mi.FULL, T, U)
    assert sum(f for _, f in parts) == step_flops
    # gate_up streams each touched expert's gate and up rows once, down its down rows once.
    gu_bytes, _ = bench.phase_work(mi.FULL, T, U, "gate_up")
    dn_bytes, _ = bench.phase_work(mi.FULL, T, U, "down")
    assert gu_bytes == 2 * (U * 2 * I * H + 2 * Is * H + T * H)
    assert dn_bytes == 2 * (U * H * I + H * Is)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stdout


def test_attainable_fraction_is_the_larger_roofline_time():
    # One-token decode: memory time (57.7 MB at 8 TB/s = 7.2 us) dominates the
    # compute time (57.7 MFLOP at 2.5 PFLOP/s = 0.023 us); a 21.19 us step is
    # then 7.21 / 21.19 = 34 % of the attainable roofline, the HBM fraction.
    nbytes, flops = bench.step_work(mi.FULL, 1, 8)
    sec = 21.19e-6
    frac = bench.attainable_frac(nbytes, flops, sec)
    assert abs(frac - nbytes / 8e12 / sec) < 1e-12
    assert abs(frac - 0.3403) < 1e-3
    # A compute-bound step (above the ridge) takes the MFMA time instead.
    frac_c = bench.attainable_frac(1e6, 2.5e15, 2.0)
    assert abs(frac_c - 0.5) < 1e-12


def test_load_stats_of_a_zipf_law():
    import numpy as np
    loads = np.round(1e4 * np.arange(1, 257, dtype=np.float64) ** -1.1)
    s = bench.load_stats(np.random.default_rng(0).permutation(loads))
    assert abs(s["loglog_slope"] + 1.1) < 0.02
    assert s["max"] == 10000 and s["sorted_loads"][0] == 10000
    assert abs(s["max_over_mean"] - 10000 / loads.mean()) < 1e-2
