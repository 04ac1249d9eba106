"""The bench reads per-launch figures of the dominant kernel (HBM bytes from
rocprofv3 byte counters, counted vector instructions) from the committed
summaries under profiles/.  Every record must be reachable by its stage,
whatever the kernel is named in the pattern family the workload uses
(pretok_kernel or pretok_case_kernel), and a record whose kernel sources have
changed since the counters were taken must read as absent."""
import glob
import json
import os

import bench

PROFILES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")


def records():
    for path in sorted(glob.glob(os.path.join(PROFILES, "traffic_*.json"))):
        w = os.path.basename(path)[len("traffic_"):-len(".json")]
        with open(path) as fh:
            yield w, json.load(fh)


def test_every_record_is_reached_by_its_stage():
    seen = 0
    for w, rec in records():
        assert w in bench.WORKLOADS, w
        for name, k in rec["kernels"].items():
            assert k["stage"] in bench.STAGE_KERNELS, (w, name)
            got = bench.profiled(w, k["stage"], "bytes_per_launch")
            if k["source_sha256"] == bench.source_digest(k["stage"]):
                assert got == k["bytes_per_launch"], (w, name)
                seen += 1
            else:
                assert got is None, (w, name)
    assert seen > 0


def test_a_changed_source_digest_reads_as_absent(tmp_path, monkeypatch):
    w, rec = next(records())
    stage = next(iter(rec["kernels"].values()))["stage"]
    for k in rec["kernels"].values():
        k["source_sha256"] = "0" * 64
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / f"traffic_{w}.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled(w, stage, "bytes_per_launch") is None
