"""bench.py on the CPU: the one-GPU contract and the stored traffic counters.

A bench line reports `roofline.traffic` only from a committed counter summary
(`profiles/traffic_<line>.txt`) taken on the current kernel sources; these
tests check that every committed summary parses and is keyed to the sources
of the line it belongs to, so a kernel edited after its profile shows here
rather than as a silent null on the GPU."""
import glob
import os
import subprocess
import sys

import bench

HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(HERE, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=HERE, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _source_set(name):
    if "_bwd" in name:
        return bench.BACKWARD_SOURCES
    if name.startswith(("mamba2_", "mlstm_", "linattn_")):
        return bench.SSD_SOURCES
    return bench.FORWARD_SOURCES


def test_stored_traffic_files_match_their_kernel_sources():
    files = sorted(glob.glob(os.path.join(HERE, "profiles", "traffic_*.txt")))
    assert files, "no stored traffic summaries"
    for path in files:
        name = os.path.basename(path)[len("traffic_"):-len(".txt")]
        sources = _source_set(name)
        got = bench.stored_traffic(name, sources)
        assert got is not None and got > 0, f"{name}: stale or unreadable (sources hash {bench.kernel_source_hash(sources)})"


def test_headline_line_has_stored_traffic():
    import workloads
    assert bench.stored_traffic(workloads.WORKLOADS[2].name) is not None
