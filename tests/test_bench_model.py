"""The benchmark's byte accounting against the figures the pages print.

tests/golden/p4_perf_table.tsv holds the inverse RoPE + FP8 quant page's
performance table.  Its effective bandwidths are the page's 1.5 KiB per
(token, head) convention over its kernel times; bench.py reports that
convention beside its own algorithmic bytes, which add the scales, positions
and cos/sin rows.
"""
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p4_perf_table.tsv")


def rows():
    with open(GOLDEN) as f:
        lines = [l.rstrip("\n") for l in f if l.strip() and not l.startswith("#")]
    head = lines[0].split("\t")
    return [dict(zip(head, l.split("\t"))) for l in lines[1:]]


def test_fixture_has_the_three_gpus():
    assert [r["gpu"] for r in rows()] == ["B200", "H200", "H100"]


@pytest.mark.parametrize("r", rows(), ids=lambda r: r["gpu"])
def test_pages_bandwidths_follow_from_1536_bytes_per_head(r):
    N, H = 16384, 32
    assert N * H == 524288  # the intro's program count
    pages_bytes = N * H * 1536
    # the page prints times to 1 us, bandwidths to 0.1 TB/s, speedups to 0.01:
    # each printed figure must lie in the interval its rounded inputs allow
    before, after = float(r["before_us"]), float(r["after_us"])
    tb_lo = pages_bytes / ((after + 0.5) * 1e-6) / 1e12
    tb_hi = pages_bytes / ((after - 0.5) * 1e-6) / 1e12
    assert tb_lo - 0.05 <= float(r["tbps"]) <= tb_hi + 0.05
    sp_lo, sp_hi = (before - 0.5) / (after + 0.5), (before + 0.5) / (after - 0.5)
    assert sp_lo - 0.005 <= float(r["speedup"]) <= sp_hi + 0.005


def test_bench_algorithmic_bytes_extend_the_pages_convention():
    N, H = 16384, 32
    pages_bytes = N * H * 1536
    assert pages_bytes == 805306368
    # + 16 B of fp32 scales per head, 8 B position and a 256 B cos/sin row per token
    assert bench.irq_bytes(N, H) == pages_bytes + N * H * 16 + N * (8 + 256) == 818020352
    assert bench.irq_bytes(N, H, "ue8m0") == pages_bytes + N * H * 4 + N * 264


def test_rotation_keeps_every_config_off_the_cache():
    # at least two buffer sets, and together at least 1 GiB: 4x the 256 MB MALL
    assert bench.rotation_sets(bench.irq_bytes(16384, 32)) == 2
    assert bench.rotation_sets(bench.irq_bytes(4096, 48)) == 4
    for b in (1, 4096, 14942208, 103841792, 306216960, 818020352, 1612776448):
        s = bench.rotation_sets(b)
        assert s >= 2 and s * b >= bench.ROTATE_BYTES
        assert s == 2 or (s - 1) * b < bench.ROTATE_BYTES  # no more sets than needed


def test_metric_names_the_headline_workload():
    import json
    import re
    src = open(bench.__file__).read()
    metric = json.loads(re.search(r'"metric": ("[^"]*")', src).group(1))
    assert metric == ("achieved HBM GB/s (% of peak) + tokens/s, "
                      "inv_rope_fp8_quant 16k tok×32 heads")


def test_more_than_one_gpu_is_refused_with_a_message():
    import subprocess
    import sys
    res = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
