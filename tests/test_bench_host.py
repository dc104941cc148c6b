"""Host-side pieces of bench.py (no GPU): step-time percentiles, and the
committed rocprofv3 records (HBM traffic, shader clock) that the bench line
reports only while the GEMM kernel sources are the ones they were measured
on."""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_percentiles(bench):
    p = bench.pctl([1.0, 2.0, 3.0, 4.0, 5.0])
    assert p == {"median": 3.0, "p10": 1.4, "p90": 4.6}


def test_records_follow_the_kernel_sources(bench, monkeypatch):
    traffic = bench.measured_traffic("gemm_rowscale_swiglu")
    clock = bench.measured_clock_ghz("gemm_rowscale_swiglu")
    # records taken on the current sources are reported (null otherwise,
    # until the counters are taken again)
    assert traffic is None or (isinstance(traffic, int) and traffic > 0)
    assert clock is None or 1.0 < clock < 2.5
    # any change to the sources voids them
    monkeypatch.setattr(bench, "kernel_sources_sha256", lambda: "0" * 64)
    assert bench.measured_traffic("gemm_rowscale_swiglu") is None
    assert bench.measured_clock_ghz("gemm_rowscale_swiglu") is None
    assert bench.measured_traffic("no_such_kernel") is None


def test_split_reduction_parts(bench):
    """Parts double while tiles x parts stays below the compute-unit count and
    the reduction still divides into 64-element stages per part."""
    assert bench.splitk_parts(2048, 2048, 8192, 256) == 4      # dWo: 64 tiles
    assert bench.splitk_parts(2048, 8192, 8192, 256) == 1      # dWd: 256 tiles
    assert bench.splitk_parts(16384, 2048, 8192, 256) == 1     # dW': 512 tiles
    assert bench.splitk_parts(256, 256, 8192, 256) == 16       # one tile: capped at 16
    assert bench.splitk_parts(2048, 2048, 192, 256) == 1       # 192 is not a multiple of 128
    assert bench.splitk_parts(2048, 2048, 256, 256) == 4       # 4 parts of one stage each
    assert bench.splitk_parts(2048, 2048, 384, 256) == 2       # 2 parts of 192 (not 4 of 96)
    for M, N, K in ((2048, 2048, 8192), (300, 272, 4096), (1, 16, 65536)):
        p = bench.splitk_parts(M, N, K, 256)
        assert K % (64 * p) == 0 and 1 <= p <= 16
