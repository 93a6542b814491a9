"""The library binds to the HIP runtime torch uses (CPU-only check: which
copies of libamdhip64 the dynamic linker maps)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_loading_the_library_first_still_maps_one_hip_runtime():
    """A fresh process that loads the binding before touching torch itself:
    load() imports torch first, so exactly one HIP runtime is mapped."""
    code = ("import stochastic_sparse_attention_amd._lib as L; L.load(); "
            "rt = L.hip_runtimes_mapped(); print(len(rt)); assert len(rt) == 1, rt")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == "1"
