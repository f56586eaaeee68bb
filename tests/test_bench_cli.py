"""bench.py's command-line contract that needs no GPU: more than one GPU, and
the tiered mode with a prefill rule it does not take, are refused with a JSON
line and exit status 2."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    rec = json.loads(r.stdout.strip().splitlines()[-1])
    assert rec["n_gpus"] == 2 and "one GPU" in rec["error"]


def test_step_bytes_of_the_128k_workload():
    sys.path.insert(0, ROOT)
    import bench
    from lsh_eviction_amd import configs, datagen
    n, s = datagen.lengths(configs.LONG128K)
    # 8 KV heads x 32768 slots x (4 code bytes + 2 x 128 x 2 K/V bytes), plus the new token's
    # K, V, code and position per head, plus q read and out written (fp32)
    assert bench.step_bytes(configs.LONG128K, s) == 8 * 32768 * 516 + 8 * (512 + 4 + 4) + 32 * 128 * 4 * 2


def test_tier_mode_refuses_other_prefill_rules():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--tier", "--prefill", "chunk"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--tier" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
