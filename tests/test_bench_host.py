"""Host-side checks of bench.py (no GPU): the one-GPU contract and the source hash that ties a
traffic summary to the kernels it was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_source_hash_covers_the_kernels_and_their_headers():
    import bench

    csrc = os.path.join(ROOT, "mxfp4_routed_expert_k3x_amd", "csrc")
    for f in bench.LATENT_SOURCES:
        assert os.path.exists(os.path.join(csrc, f)), f
    # every header the hashed kernels include is hashed with them
    hashed = set(bench.KERNEL_SOURCES)
    for f in bench.KERNEL_SOURCES:
        for line in open(os.path.join(csrc, f)):
            if line.startswith('#include "') and "/" not in line:
                assert line.split('"')[1] in hashed, (f, line)
    assert bench.sources_hash("decode_t1_e896_router") != bench.sources_hash("latent_t1_e896")
