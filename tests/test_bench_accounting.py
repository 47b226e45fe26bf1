"""The benchmark's work accounting (CPU): the closed form for the visible
(query, key) pairs that the FLOP counts rest on, against a direct count of
the mask, and the traffic lookup's refusal of unknown parts."""

import numpy as np
import pytest

import bench


@pytest.mark.parametrize("S", [1, 2, 63, 64, 65, 128, 129, 300, 1000])
@pytest.mark.parametrize("W", [0, 1, 2, 64, 127, 128, 129, 5000])
def test_pairs_per_head_matches_a_direct_count(S, W):
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    visible = (j <= i) & ((W == 0) | (i - j < W))
    assert bench.pairs_per_head(S, W) == int(visible.sum())


def test_workload_pair_counts():
    # the B = 4, S = 4096, 64-head step: full-causal and sliding-128 layers
    assert 4 * 64 * bench.pairs_per_head(4096, 0) == 2_148_007_936
    assert bench.pairs_per_head(4096, 128) == 128 * 129 // 2 + (4096 - 128) * 128


def test_traffic_lookup_refuses_unknown_parts():
    assert bench.measured_traffic("no_such_part_full") is None


def _counter_csv(path, counter, rows):
    path.mkdir(parents=True)
    lines = ["Kernel_Name,Counter_Name,Counter_Value"]
    lines += [f'"void ns::{k}(Params)",{counter},{v}' for k, v in rows]
    (path / "run_counter_collection.csv").write_text("\n".join(lines) + "\n")


def test_traffic_digest_keeps_unmeasured_parts_only_on_unchanged_sources(tmp_path, monkeypatch):
    import json
    (tmp_path / "profiles").mkdir()
    digests = {"fwd": "F", "varlen_fwd": "F", "bwd": "B2", "varlen_bwd": "B2", "decode": "D2"}
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda part: digests[part])
    old = {"source_sha256": {"fwd": "F", "varlen_fwd": "F", "bwd": "B1", "varlen_bwd": "B1", "decode": "D1"},
           "bytes_per_launch": {"fwd_full": 11, "fwd_w128": 12, "bwd_full": 99, "decode_full": 7},
           "per_kernel_bytes": {"fwd_full:fwd_kernel": [10, 1], "decode_full:decode_split_kernel": [6, 1]}}
    (tmp_path / "profiles" / "traffic.json").write_text(json.dumps(old))
    runs = tmp_path / "runs"
    kib = bench.COPY_BYTES // 1024
    _counter_csv(runs / "copy_FETCH_SIZE", "FETCH_SIZE", [("copy_kernel", kib // 2)])  # reads x2
    _counter_csv(runs / "copy_WRITE_SIZE", "WRITE_SIZE", [("copy_kernel", kib)])
    for w in bench.WINDOWS:
        _counter_csv(runs / f"bwd_{w}_FETCH_SIZE", "FETCH_SIZE",
                     [("bwd_dq_kernel", 100), ("bwd_dq_kernel", 300), ("bwd_dkdv_kernel", 50)])
        _counter_csv(runs / f"bwd_{w}_WRITE_SIZE", "WRITE_SIZE", [("bwd_dq_kernel", 10), ("bwd_dkdv_kernel", 20)])
    bench.digest_traffic(str(runs))
    new = json.loads((tmp_path / "profiles" / "traffic.json").read_text())
    # re-measured: reads averaged per kernel and doubled, writes as read
    assert new["bytes_per_launch"]["bwd_full"] == (200 * 2 + 50 * 2 + 10 + 20) * 1024
    assert new["per_kernel_bytes"]["bwd_full:bwd_dq_kernel"] == [400 * 1024, 10 * 1024]
    assert new["source_sha256"]["bwd"] == "B2"
    # not re-measured, same sources: kept; changed sources: dropped
    assert new["bytes_per_launch"]["fwd_full"] == 11 and new["bytes_per_launch"]["fwd_w128"] == 12
    assert new["per_kernel_bytes"]["fwd_full:fwd_kernel"] == [10, 1]
    assert new["source_sha256"]["fwd"] == "F"
    assert "decode_full" not in new["bytes_per_launch"] and "decode" not in new["source_sha256"]
    assert not any(k.startswith("decode") for k in new["per_kernel_bytes"])
    assert "varlen_bwd" not in new["source_sha256"]


def test_dpm_level_parsing():
    assert bench.parse_dpm_level("0: 500Mhz\n1: 1400Mhz\n2: 2100Mhz *\n") == 2100.0
    assert bench.parse_dpm_level("S: 1733Mhz *\n") == 1733.0
    assert bench.parse_dpm_level("0: 500Mhz\n1: 2100Mhz\n") is None


def test_traffic_digest_refuses_a_part_measured_in_part(tmp_path, monkeypatch):
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda part: "X")
    runs = tmp_path / "runs"
    kib = bench.COPY_BYTES // 1024
    _counter_csv(runs / "copy_FETCH_SIZE", "FETCH_SIZE", [("copy_kernel", kib // 2)])
    _counter_csv(runs / "copy_WRITE_SIZE", "WRITE_SIZE", [("copy_kernel", kib)])
    _counter_csv(runs / "bwd_0_FETCH_SIZE", "FETCH_SIZE", [("bwd_dq_kernel", 1)])
    with pytest.raises(SystemExit, match="bwd_128_FETCH_SIZE"):
        bench.digest_traffic(str(runs))
    assert not (tmp_path / "profiles" / "traffic.json").exists()


def test_source_digest_covers_per_source_build_flags(monkeypatch):
    base = bench.source_digest("fwd")
    flags = dict(bench.build_source_flags())
    assert bench.source_digest("bwd") != base
    flags["fwd.hip"] = ["-mllvm", "-some-other-flag"]
    monkeypatch.setattr(bench, "build_source_flags", lambda: flags)
    assert bench.source_digest("fwd") != base
    assert bench.source_digest("varlen_fwd") == bench.source_digest("fwd")
