"""bench.py's host-side contract, checked without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_flops_per_slot_match_the_method_totals():
    sys.path.insert(0, ROOT)
    import bench
    import synth
    for name in ("qwen3_30b_a3b", "gptoss120b", "gptoss20b"):
        c = synth.get_config(name)
        f = bench.gemm_flops_per_slot(c)
        d, F, r = c.d, c.F, c.r
        fwd = f["proj_gu"] + f["gateup"] + f["proj_d"] + f["down"]
        bwd = f["proj_dout"] + f["down_bwd"] + f["proj_dgu"] + f["gateup_bwd"] + f["lora_grad"]
        assert fwd == 6 * d * F + 6 * r * (d + F)            # forward per routed slot
        assert bwd == 6 * d * F + 12 * r * (d + F)           # backward, base frozen
