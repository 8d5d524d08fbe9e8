"""The library binds to the HIP runtime torch already loaded (CPU only).

libattn_sinks.so links libamdhip64; the binding imports torch first, so the
dynamic loader resolves that dependency to the runtime torch mapped, and
the process holds exactly one HIP runtime (two would each keep their own
device state, streams and allocations).  Checked in a fresh process through
/proc/self/maps.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = r"""
import sys
sys.path.insert(0, sys.argv[1])
import gqa_paged_attention_amd as ga
ga.library()
paths = set()
for line in open("/proc/self/maps"):
    parts = line.split()
    if len(parts) >= 6 and "libamdhip64" in parts[5]:
        paths.add(parts[5])
print("\n".join(sorted(paths)))
"""


def test_one_hip_runtime_mapped():
    res = subprocess.run([sys.executable, "-c", SCRIPT, ROOT], capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, res.stderr
    paths = [p for p in res.stdout.split("\n") if p]
    assert len(paths) == 1, f"HIP runtimes mapped: {paths}"
    assert "torch" in paths[0] or "rocm" in paths[0], paths
