"""Host-side logic of bench.py (no GPU): the one-GPU contract and the guard
on the committed HBM traffic record (it is reported only while the kernel
source it was measured on is unchanged)."""
import hashlib
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _fake_root(tmp_path):
    rec = json.load(open(os.path.join(ROOT, "profiles", "attn_splitk_decode_118750_traffic.json")))
    os.makedirs(tmp_path / "profiles")
    src_dst = tmp_path / rec["source"]
    os.makedirs(src_dst.parent)
    shutil.copy(os.path.join(ROOT, rec["source"]), src_dst)
    shutil.copy(os.path.join(ROOT, "profiles", "attn_splitk_decode_118750_traffic.json"),
                tmp_path / "profiles" / "attn_splitk_decode_118750_traffic.json")
    return rec, src_dst


def test_traffic_record_follows_the_kernel_source(tmp_path, monkeypatch):
    import bench
    rec, src = _fake_root(tmp_path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    # the record names the source it was measured on by its SHA-256
    digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    expect = rec["bytes_per_launch"] if digest == rec["source_sha256"] else None
    assert bench.measured_traffic() == expect
    # any edit to the source voids it
    with open(src, "ab") as f:
        f.write(b"\n// edited\n")
    assert bench.measured_traffic() is None
    # and a missing record reports nothing rather than failing
    os.remove(tmp_path / "profiles" / "attn_splitk_decode_118750_traffic.json")
    assert bench.measured_traffic() is None



def test_spread_is_nearest_rank_percentiles_in_us():
    import bench
    ts = [0.001 * i for i in range(1, 101)]  # 1 .. 100 us, in ms
    sp = bench.spread_us(list(reversed(ts)))
    assert sp == {"launches": 100, "median_us": 51.0, "p10_us": 11.0, "p90_us": 90.0}
    one = bench.spread_us([0.02])
    assert one["median_us"] == one["p10_us"] == one["p90_us"] == 20.0
