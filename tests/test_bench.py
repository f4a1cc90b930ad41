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
