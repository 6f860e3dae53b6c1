"""bench.py's host-side contract, checked without a GPU: it measures one GPU
only and refuses other counts before touching a device, and its traffic
lookup follows the committed counter summary only while the attention source
is the one that was measured."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""           # no JSON line


def test_traffic_lookup_follows_source_hash(tmp_path, monkeypatch):
    src = tmp_path / "sparse_attn.hip"
    src.write_bytes(b"// kernel source\n")
    import hashlib
    h = hashlib.sha256(src.read_bytes()).hexdigest()[:16]
    prof = tmp_path / "traffic.txt"
    prof.write_text("void mha_attn_kernel<128, 1, 2, false>   42   32880.3   272.0   67.611\n"
                    "void combine_kernel<128, 128, 4, 8>      42     154.6    34.0    0.351\n"
                    "void index_scores_kernel<4, 4, 1, false>  6    4195.9   128.0    8.723\n"
                    f"sparse_attn.hip sha256[:16] at measurement time: {h}\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    monkeypatch.setattr(bench, "ATTN_SOURCE", str(src))
    assert abs(bench.measured_traffic() - (67.611 + 0.351) * 1e6) < 1.0   # gather + combine only
    src.write_bytes(b"// kernel source, edited\n")
    assert bench.measured_traffic() is None                                # stale counters are not reported
