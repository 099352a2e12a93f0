"""Host-side checks of the bench's measurement code (no GPU): the
algorithmic bytes behind `roofline.achieved`, the copy-calibrated HBM
traffic of the profile summaries, the one-GPU refusal, and the host-only
prefix-cache mode."""
import csv
import json
import os
import subprocess
import sys
import types

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402

# KV bytes one decode launch must read: each KV head's cached K and V once
# per sequence, real tokens only, FP8 scales and INT4 (scale, zero) included,
# a shared prefix once.  Per token: bf16 2 * 8 heads * 128 * 2 B; FP8
# 2 * 8 * (128 + 4); INT4 2 * 8 * (64 + 16).
EXPECTED = {"c1": (512, 223_232), "c2": (4096, 633_569_280), "c3": (2112, 326_684_160),
            "c4": (4096, 2_327_375_872), "c5": (1280, 335_544_320)}


@pytest.mark.parametrize("name", sorted(EXPECTED))
def test_algorithmic_bytes(name):
    wl = workloads.get(name)
    plan = workloads.plan(wl)
    per_tok, total = EXPECTED[name]
    assert bench.kv_bytes_per_token(wl) == per_tok
    assert bench.unique_tokens(plan.lengths, wl) * per_tok == total


def _write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def test_profile_summary_traffic(tmp_path, monkeypatch):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what they
    read for the copy kernel of known size; traffic is in bytes."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    kname = "void pkv::streamk_decode_kernel<1, 1, 128, 16, true>(pkv::DecodeParams)"
    d = {k: str(tmp_path / k) for k in ("stats", "fetch", "write", "cfetch", "cwrite")}
    _write_csv(os.path.join(d["stats"], "run_kernel_stats.csv"),
               [{"Name": kname, "Calls": 52, "TotalDurationNs": 5.2e6, "AverageNs": 1.0e5,
                 "Percentage": 50.0, "MinNs": 9e4, "MaxNs": 1.1e5, "StdDev": 1.0}])
    row = lambda n, v, k: {"Counter_Name": n, "Counter_Value": v, "Kernel_Name": k}  # noqa: E731
    _write_csv(os.path.join(d["fetch"], "run_counter_collection.csv"),
               [row("FETCH_SIZE", 300_000.0, kname), row("FETCH_SIZE", 320_000.0, kname)])
    _write_csv(os.path.join(d["write"], "run_counter_collection.csv"),
               [row("WRITE_SIZE", 100.0, kname)])
    copy = "pkv::bench_copy_kernel(...)"
    _write_csv(os.path.join(d["cfetch"], "run_counter_collection.csv"),
               [row("FETCH_SIZE", bench.COPY_BYTES / 1024 / 2, copy)])
    _write_csv(os.path.join(d["cwrite"], "run_counter_collection.csv"),
               [row("WRITE_SIZE", bench.COPY_BYTES / 1024, copy)])
    args = types.SimpleNamespace(summarize_profiles=[d[k] for k in ("stats", "fetch", "write",
                                                                    "cfetch", "cwrite")],
                                 partition=None, kernel=None, command="a;;b")
    wl = workloads.get("c2")
    bench.summarize_profiles(args, wl)
    prof = bench.read_profile(bench.profile_path(wl, "streamk_decode_kernel"))
    assert float(prof["fetch_scale"]) == 2.0 and float(prof["write_scale"]) == 1.0
    want = (310_000.0 * 2.0 + 100.0 * 1.0) * 1024
    assert float(prof["traffic_bytes_per_launch"]) == pytest.approx(want, abs=1)
    assert bench.traffic_from_profile(wl, "streamk_decode_kernel") == pytest.approx(want, abs=1)
    # the ratio divides by the bytes of the counter runs' own launches
    alg = float(prof["algorithmic_bytes_per_launch"].split()[0])
    lengths = workloads.plan(wl).lengths + bench.COUNTER_STEPS
    assert alg == bench.unique_tokens(lengths, wl) * bench.kv_bytes_per_token(wl)
    assert bench.traffic_ratio_from_profile(wl, "streamk_decode_kernel") == \
        pytest.approx(want / alg, rel=1e-3)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_prefix_cache_mode_runs_on_the_host():
    pytest.importorskip("paged_kv_cache_250_amd")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--prefix-cache",
                        "--steps", "2"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["unit"] == "us" and line["value"] > 0
    assert 0.5 < line["compute_saved_frac"] < 1.0
    assert line["blocks_per_request_peak"] < line["blocks_per_request_unshared"]
