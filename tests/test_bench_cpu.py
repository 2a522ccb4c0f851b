"""The benchmark's contract on the host: the algorithmic byte and flop counts its
roofline figures divide by, and the refusal of more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_prefill_algorithmic_bytes():
    # Q, K, V read and Y written in bf16: 4 x 128 x 2 = 1,024 B per head-token (+4 B of alpha
    # gated); the fp32 state (128 x 128 + 128 floats = 66,048 B) read and written per head
    assert bench.STATE_BYTES == 66048
    assert bench.prefill_bytes(4, 16, 4096, False) == 64 * 4096 * 1024 + 2 * 64 * 66048 == 276889600
    assert bench.prefill_bytes(2, 16, 16384, True) == 32 * 16384 * 1028 + 2 * 32 * 66048


def test_prefill_useful_flops():
    # per head-token (C + 1)(d + dv) for the causal score and read-out products and 4 d dv for the
    # read of the carried state and the state write: 82,176 at C = 64, 98,560 at C = 128
    per = lambda C: (C + 1) * 256 + 4 * 128 * 128
    assert per(64) == 82176 and per(128) == 98560
    assert bench.prefill_useful_flops(4, 16, 4096, 64) == 64 * 4096 * per(64)
    assert bench.prefill_useful_flops(1, 32, 131072, 128) == 32 * 131072 * per(128)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_mix_ceiling():
    # reads at the read rate and writes at the write rate, one after the other
    ceil = {"read_GBps": 6000.0, "write_GBps": 7000.0}
    r, w = 3e9, 1e9
    t = r / 6000.0 + w / 7000.0
    assert abs(bench.mix_ceiling(ceil, r, w) - (r + w) / t) < 1e-9
    assert abs(bench.mix_ceiling(ceil, r, 0.0) - 6000.0) < 1e-9
    assert abs(bench.mix_ceiling(ceil, 0.0, w) - 7000.0) < 1e-9
