"""Host-side pieces of bench.py that need no GPU: the algorithmic work per
token-head, and the traffic lookup that is keyed to the kernel sources."""
import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_host", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_prefill_flops_per_token_head(bench):
    # 6 d^2 + (C - 1) d + 4 (C + 1) d + C^2 / 3 at d = 128
    assert bench.prefill_flops_per_token_head(64) == pytest.approx(98304 + 8064 + 33280 + 4096 / 3)
    assert bench.prefill_flops_per_token_head(32) == pytest.approx(98304 + 3968 + 16896 + 1024 / 3)
    assert bench.prefill_flops_per_token_head(16) == pytest.approx(98304 + 1920 + 8704 + 256 / 3)


def test_traffic_lookup_follows_the_sources(bench):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        t = json.load(f)
    for name, files in bench.KERNEL_SOURCES.items():
        entry = t.get(name)
        assert entry is not None, name
        got = bench.measured_traffic(name)
        if entry["source_sha"] == bench.source_sha(*files):
            assert got == entry["bytes_per_launch"]
        else:
            assert got is None            # counters taken on other sources are not reported


def test_traffic_entries_are_calibrated(bench):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        t = json.load(f)
    for name in bench.KERNEL_SOURCES:
        e = t[name]
        # bytes = KiB per dispatch / the copy calibration factor (stored rounded to 5 digits)
        assert e["read_bytes"] == pytest.approx(e["fetch_kib_per_dispatch"] * 1024
                                                / t["copy_factor_fetch"], rel=1e-4)
        assert e["write_bytes"] == pytest.approx(e["write_kib_per_dispatch"] * 1024
                                                 / t["copy_factor_write"], rel=1e-4)
        assert abs(e["bytes_per_launch"] - e["read_bytes"] - e["write_bytes"]) <= 1
