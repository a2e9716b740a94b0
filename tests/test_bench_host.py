"""Host-side checks of bench.py (no GPU): the one-GPU contract and the byte
accounting the decode figures are computed from."""
import os
import subprocess
import sys

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    for args in (["--gpus", "2"], ["--gpus", "8"]):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args,
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2
        assert "one GPU" in r.stderr and r.stdout == ""


def test_step_bytes_are_storage_plus_activations():
    sys.path.insert(0, ROOT)
    import bench
    from synth import gen
    for L in gen.LLAMA8B:
        for M in (1, 8):
            assert bench.decode_bytes(L, M) == O.storage_bytes(L.N, L.K) + 2 * M * (L.K + L.N)
