"""bench.py's use of the committed counter records (host logic only, no GPU): a traffic
record counts only for the path variant and the kernel sources it was taken on."""
import json

import bench
import synth


def _record(tmp_path, w, variant, files):
    rec = {"stage": "markov_sample", "workload": w.name, "bytes_per_call": 12345, "variant": variant,
           "source_files": files}
    (tmp_path / f"markov_sample_{w.name}_traffic.json").write_text(json.dumps(rec))


def test_traffic_record_needs_the_same_variant_and_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    w = synth.get("admission")
    src = "draft_sampling_lossless_amd/csrc/markov.hip"
    h = bench.src_hash(f"{bench.ROOT}/{src}")
    _record(tmp_path, w, "deferred/rejection/path", {src: h})
    assert bench.measured_traffic("markov_sample", w, "deferred/rejection/path") == 12345
    # another path variant launches other kernels: its counters are not these
    assert bench.measured_traffic("markov_sample", w, "stored/rejection/path") is None
    assert bench.measured_traffic("markov_sample", w, "deferred/coupled/path") is None
    # a source changed since the counters were taken
    _record(tmp_path, w, "deferred/rejection/path", {src: "0" * 16})
    assert bench.measured_traffic("markov_sample", w, "deferred/rejection/path") is None
    # no record at all
    assert bench.measured_traffic("verify", w, "deferred/rejection/path") is None


def test_committed_records_name_their_variant():
    import glob
    import os
    for f in glob.glob(os.path.join(bench.PROFILES, "*_traffic.json")):
        d = json.load(open(f))
        assert d.get("variant") in {"deferred/rejection/path", "stored/rejection/path", "deferred/rejection/full",
                                    "stored/rejection/full", "stored/coupled/path", "stored/coupled/full"}, f
        assert d.get("source_files"), f
