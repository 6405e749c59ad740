"""The benchmark's command-line contract on the host (no GPU): it measures one
GPU and refuses more with a message and a non-zero status."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _local_includes(csrc, name, seen):
    import re
    if name in seen:
        return
    seen.add(name)
    with open(os.path.join(csrc, name)) as fh:
        for line in fh:
            m = re.match(r'\s*#include "([^"/]+)"', line)
            if m and os.path.exists(os.path.join(csrc, m.group(1))):
                _local_includes(csrc, m.group(1), seen)


def test_counter_summaries_are_keyed_to_the_kernels_own_sources():
    """Each measured kernel's counter summary is trusted only while its source
    files hash to the recorded value; those files must be the kernel's own file
    and exactly the local headers it includes (transitively), so that a change
    elsewhere neither voids nor a change here escapes the check."""
    sys.path.insert(0, ROOT)
    import bench
    csrc = bench.CSRC
    for kernel, files in bench.KERNEL_SOURCES.items():
        seen = set()
        _local_includes(csrc, files[0], seen)
        assert set(files) == seen, (kernel, sorted(files), sorted(seen))
