"""Host-side pieces of bench.py that need no GPU: the validity rule of the
counter-measured traffic record, the oracle baseline's worker pool and the
shape of its result."""

import bench
import workloads


def test_traffic_record_only_for_its_sources_and_split_count():
    rec = bench.TRAFFIC["c2"]
    splits = rec["splits"]
    if rec["kernels_sha256"] == bench.kernel_sha():
        assert bench.traffic_for("c2", splits) == rec["bytes_per_launch"]
    else:
        assert bench.traffic_for("c2", splits) is None
    assert bench.traffic_for("c2", splits + 8) is None
    assert bench.traffic_for("no such workload", splits) is None


def test_traffic_record_matches_its_committed_summary():
    """The counter summary the record names exists and states the same
    source hash and the same bytes per launch."""
    import os
    rec = bench.TRAFFIC["c2"]
    path = os.path.join(bench.ROOT, rec["source"])
    text = open(path).read()
    assert rec["kernels_sha256"] in text
    assert f"{rec['bytes_per_launch'] / 1e6:.2f} MB" in text


def test_host_workers_within_the_host_share():
    n = bench.host_workers()
    assert 1 <= n <= 16


def test_cpu_baseline_on_a_small_sample():
    data = workloads.make("c1", n=96, m=80)
    res = bench.cpu_baseline(data, budget=96 * 80 * 16 * 4.0)
    assert res["kind"] == "oracle" and res["unit"] == "n*m*iters/s"
    assert res["cores"] == bench.host_workers()
    assert res["value"] > 0
    assert "worker processes" in res["sample"]
    assert not bench._CPU_JOB  # the fork-shared inputs are released
