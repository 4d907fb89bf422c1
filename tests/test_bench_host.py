"""Host-side checks of the benchmark's bookkeeping (no GPU): the recorded attention traffic is
reported only for the launch it was measured on and only while the kernel sources are the ones
it was measured with."""
import bench


def test_recorded_traffic_matches_current_sources():
    for cfg in ("c5", "c2"):
        v = bench.recorded_traffic(cfg)
        assert v is not None and v > 0, cfg


def test_recorded_traffic_only_for_one_sample():
    assert bench.recorded_traffic("c2", batch=2) is None
    assert bench.recorded_traffic("c5", batch=2) is None


def test_recorded_traffic_absent_config_is_null():
    assert bench.recorded_traffic("c3") is None
    assert bench.recorded_traffic("c1") is None


def test_recorded_traffic_null_after_a_source_change(monkeypatch):
    monkeypatch.setattr(bench, "attention_source_hash", lambda: "0" * 64)
    assert bench.recorded_traffic("c5") is None
    assert bench.recorded_traffic("c2") is None


def test_host_cpu_model_is_named():
    m = bench.host_cpu_model()
    assert isinstance(m, str) and m
