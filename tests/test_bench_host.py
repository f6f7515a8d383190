"""Host-side checks of bench.py (CPU): the one-GPU contract and the
algorithmic work it divides by, against the byte and flop counts the
DeepSeek-V3-shaped workload implies (T=8192, H=7168, top-8, I=2048)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_algorithmic_work_of_the_dsv3_step():
    sys.path.insert(0, ROOT)
    from bench import stage_work
    from synth import get_config
    cfg = get_config("dsv3")
    w = stage_work(cfg, active_experts=256)
    # every token row read once and written to 8 receive rows (1.059 GB);
    # 8 rows read back per token and one row written (1.058 GB)
    assert abs(w["dispatch"]["bytes"] - 1.0585e9) < 1e6
    assert abs(w["combine"]["bytes"] - 1.0578e9) < 1e6
    # SwiGLU: 2 * 2I * H flop per row for gate/up, 2 * I * H for down,
    # 65536 rows: 5.77 TFLOP in all
    total = w["expert_gate_up"]["flops"] + w["expert_down"]["flops"]
    assert abs(total - 5.772e12) < 1e9
    # weights of 256 experts: 3 * I * H bf16 each (22.5 GB)
    wb = 4 * 256 * 2048 * 7168 + 2 * 256 * 7168 * 2048
    assert w["expert_gate_up"]["bytes"] + w["expert_down"]["bytes"] > wb
    assert abs(wb - 22.55e9) < 0.01e9
