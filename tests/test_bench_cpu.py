"""Host-side checks of bench.py that need no GPU: the one-GPU refusal, the
HBM-traffic arithmetic behind `roofline.traffic`, and the slot-order switch."""

import json
import os
import subprocess
import sys
import types

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout.strip() == ""


def _counter_json(tmp_path, fetch_kib, write_kib, copy_fetch, copy_write, sha):
    c = {"workload": "w", "unit": "KiB per dispatch", "commands": "",
         "copy": {"kernel": "copy", "bytes": bench.COPY_BYTES, "fetch_kib": copy_fetch, "write_kib": copy_write},
         "kernels": {"k_group_dh": {"dispatch": "d", "fetch_kib": fetch_kib, "write_kib": write_kib,
                                    "source_sha256": sha}}}
    p = tmp_path / "hbm_counters_w_step.json"
    p.write_text(json.dumps(c))
    return str(p)


def test_measured_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    # the copy of 1 GiB reads as half its bytes on FETCH_SIZE and exactly on WRITE_SIZE
    path = _counter_json(tmp_path, 1000.0, 300.0, bench.COPY_BYTES / 1024 / 2, bench.COPY_BYTES / 1024,
                         bench.source_sha256("k_group_dh"))
    monkeypatch.setattr(bench, "counter_file", lambda workload: path)
    assert bench.measured_traffic("w", "k_group_dh") == int(round(1024 * (1000.0 * 2 + 300.0 * 1)))


def test_measured_traffic_is_null_for_other_sources(tmp_path, monkeypatch):
    path = _counter_json(tmp_path, 1000.0, 300.0, 1.0, 1.0, "0" * 64)
    monkeypatch.setattr(bench, "counter_file", lambda workload: path)
    assert bench.measured_traffic("w", "k_group_dh") is None
    monkeypatch.setattr(bench, "counter_file", lambda workload: str(tmp_path / "absent.json"))
    assert bench.measured_traffic("w", "k_group_dh") is None


def test_sorted_slots_switch_leaves_the_index_sets_alone():
    called = []
    hs = types.SimpleNamespace(order_slots=lambda *a, **k: called.append(a))
    name = bench.prepare_slots(hs, None, None, 32, types.SimpleNamespace(sorted_slots=True))
    assert called == [] and "sorted" in name
