"""Host-side checks of the profiling helpers: the committed traffic summary parses, and a
summary whose kernel-source digest does not match is ignored by bench.py."""
import json
import os

import bench
from chunk_gated_delta_amd.build import source_digest
from chunk_gated_delta_amd.prof_summary import TRAFFIC_TAG, read_traffic


def test_committed_traffic_summary_parses():
    rec = read_traffic(bench.TRAFFIC_SUMMARY)
    assert rec is not None
    assert set(rec["bytes_per_launch"]) >= {"fwd_prep_kernel", "fwd_state_kernel", "bwd_state_kernel",
                                             "bwd_chunk_kernel"}
    for v in rec["bytes_per_launch"].values():
        assert v["read"] > 0 and v["write"] > 0


def test_stale_digest_gives_no_traffic(tmp_path, monkeypatch):
    rec = {"source_digest": "0" * 16, "fetch_scale": 2.0, "write_scale": 1.0,
           "bytes_per_launch": {"bwd_chunk_kernel": {"read": 10, "write": 5}}}
    path = tmp_path / "t.md"
    path.write_text("# x\n" + TRAFFIC_TAG + json.dumps(rec) + " -->\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(path))
    assert bench.measured_traffic("bwd_chunk_grads") is None
    rec["source_digest"] = source_digest()
    path.write_text("# x\n" + TRAFFIC_TAG + json.dumps(rec) + " -->\n")
    assert bench.measured_traffic("bwd_chunk_grads") == 15
    assert bench.measured_traffic("no_such_stage") is None


def test_source_digest_is_stable():
    assert source_digest() == source_digest()
    assert len(source_digest()) == 16
