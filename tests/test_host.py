"""Host-side logic of the benchmark script (no GPU)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    rec = {"kernel_source_hash": bench.kernel_source_hash(),
           "kernels": {"decode_gateup": {"hbm_bytes_per_launch": 123}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("decode_gateup") == 123
    assert bench.measured_traffic("decode_router") is None
    rec["kernel_source_hash"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic("decode_gateup") is None


def test_kernel_source_hash_is_stable():
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash()) == 16


def test_bucket_binding_refuses_short_buffers():
    """The binding checks each output buffer against T*k and E before the
    library sees it (a short perm or pos would take writes past its end)."""
    import pytest
    import torch
    from quantized_moe_amd import lib
    idx = torch.zeros((4, 2), dtype=torch.int32)
    good = dict(counts=torch.empty(8, dtype=torch.int32), offsets=torch.empty(9, dtype=torch.int32),
                perm=torch.empty(8, dtype=torch.int32), pos=torch.empty(8, dtype=torch.int32))
    for name, n in (("counts", 7), ("offsets", 8), ("perm", 7), ("pos", 4)):
        bad = dict(good, **{name: torch.empty(n, dtype=torch.int32)})
        with pytest.raises(ValueError, match=name):
            lib.bucket(idx, 8, bad["counts"], bad["offsets"], bad["perm"], bad["pos"])
