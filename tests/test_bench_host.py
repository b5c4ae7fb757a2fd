"""bench.py host logic on the CPU: the one-GPU guard and the algorithmic byte
counts that the roofline figure divides by the measured FC1 duration."""
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_fc1_algorithmic_bytes_at_the_ep4_shape():
    """E=96 active experts of FC1 [6144, 7168] (SwiGLU, I=3072), T=1024 tokens,
    R=6144 routed rows. Packed E2M1 + one E4M3 scale per 16 elements is 9/16 byte
    per element, plus one FP32 scale per expert, token and row."""
    import bench
    w = SimpleNamespace(N1=6144, H=7168, I=3072, K=6)
    counts = np.full(96, 64)
    ab = bench.algorithmic_bytes(w, counts, T=1024, R=6144)
    weights = 96 * (6144 * 7168 * 9 // 16 + 4)      # 2,378,170,752
    x_read = 1024 * (7168 * 9 // 16 + 4)             # 4,132,864
    hq_write = 6144 * (3072 * 9 // 16 + 4)           # 10,641,408
    assert ab["fc1"] == weights + x_read + hq_write == 2392945024
    # experts without routed rows stream no weights
    counts[::2] = 0
    assert bench.algorithmic_bytes(w, counts, T=1024, R=6144)["fc1"] == \
        48 * (6144 * 7168 * 9 // 16 + 4) + x_read + hq_write
