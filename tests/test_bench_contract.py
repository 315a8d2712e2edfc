"""bench.py's command-line contract, on the CPU: more than one GPU is refused
with a message and a non-zero status before any device work starts."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_help_lists_the_contract_flags():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def test_traffic_record_is_used_only_for_the_profiled_sources(tmp_path, monkeypatch):
    """roofline.traffic comes from the committed counter summary's record only
    while the attention sources hash to the value it names; a stale or
    unreadable record gives null with the reason."""
    sys.path.insert(0, ROOT)
    import bench
    prof = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    good = {"sources_sha256": bench.attend_sources_sha256(), "attend_call_bytes": 123456789,
            "fetch_factor": 2.0, "taken": "test"}
    prof.write_text("# summary\n\nbench-record: " + json.dumps(good) + "\n")
    value, rec = bench.profiled_attend_traffic()
    assert value == 123456789.0 and rec["taken"] == "test"
    prof.write_text("bench-record: " + json.dumps(dict(good, sources_sha256="0" * 64)) + "\n")
    value, why = bench.profiled_attend_traffic()
    assert value is None and "changed" in why
    prof.write_text("bench-record: {not json\n")
    value, why = bench.profiled_attend_traffic()
    assert value is None and "unreadable" in why
    prof.write_text("no record here\n")
    assert bench.profiled_attend_traffic()[0] is None
