"""Host-side pieces of bench.py: reading HBM traffic figures back from the
rocprofv3 counter summaries (no GPU needed)."""
import hashlib
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402


def _summary(root, src_text, lines):
    os.makedirs(os.path.join(root, "profiles"), exist_ok=True)
    with open(os.path.join(root, "k.hip"), "w") as f:
        f.write(src_text)
    h = hashlib.sha256(src_text.encode()).hexdigest()[:16]
    with open(os.path.join(root, "profiles", "k.txt"), "w") as f:
        f.write("\n".join(lines + ["kernel_sources_sha256_16: %s  (k.hip)" % h]) + "\n")


def test_traffic_figures_with_and_without_notes(tmp_path, monkeypatch):
    root = str(tmp_path)
    _summary(root, "kernel v1", ["traffic_bytes_per_launch: 546374602",
                                 "traffic_bytes_per_launch_T4: 612501158  (read 612107942, "
                                 "write 393216; 7 dispatches)"])
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.profiled_traffic("k.txt") == 546374602
    assert bench.profiled_traffic("k.txt", "traffic_bytes_per_launch_T4") == 612501158
    assert bench.profiled_traffic("k.txt", "traffic_bytes_per_launch_T16") is None
    assert bench.profiled_traffic("missing.txt") is None


def test_traffic_is_dropped_once_the_kernel_source_changes(tmp_path, monkeypatch):
    root = str(tmp_path)
    _summary(root, "kernel v1", ["traffic_bytes_per_launch: 1000"])
    monkeypatch.setattr(bench, "ROOT", root)
    assert bench.profiled_traffic("k.txt") == 1000
    with open(os.path.join(root, "k.hip"), "w") as f:
        f.write("kernel v2")
    assert bench.profiled_traffic("k.txt") is None
