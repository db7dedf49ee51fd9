"""The bench's host-side contract, without a GPU: more than one GPU is
refused with a message, and the committed HBM traffic summary is read back
only for the key-pass sources it was taken from."""
import os
import subprocess
import sys

import bench

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "2"})):
        res = subprocess.run([sys.executable, os.path.join(REPO, "bench.py"), *args],
                             env=dict(os.environ, **env), capture_output=True,
                             text=True, timeout=60)
        assert res.returncode == 2
        assert "one GPU" in res.stderr and res.stdout == ""


def test_traffic_summary_follows_the_sources(tmp_path, monkeypatch):
    h = bench.kernel_source_hash()
    assert len(h) == 64 and h == bench.kernel_source_hash()
    f = tmp_path / "traffic.txt"
    f.write_text("# comment: ignored\nkernel: k_entmax_scores_mfma\n"
                 "source_sha256: %s\nfetch_bytes_per_launch: 1000\n"
                 "write_bytes_per_launch: 24\n" % h)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("k_entmax_scores_mfma") == 1024
    assert bench.measured_traffic("k_score") is None
    f.write_text(f.read_text().replace(h, "0" * 64))
    assert bench.measured_traffic("k_entmax_scores_mfma") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.measured_traffic("k_entmax_scores_mfma") is None
