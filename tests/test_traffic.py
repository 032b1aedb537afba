"""Byte accounting of the benchmark, pinned to figures the pages print
(tests/golden/page_bandwidth.json) and to the per-tensor sum."""
import json
import os

import pytest

from layer_mhc_seam_amd.traffic import page_bytes, seam_bytes, total_bytes

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_bandwidth.json")))


@pytest.mark.parametrize("row", GOLD["bytes"])
def test_page_byte_figures(row):
    b = page_bytes(row["T"], GOLD["H"], row["form"], row["out_dtype"])
    assert abs(b / 1e9 - row["GB"]) < 0.0005


@pytest.mark.parametrize("row", GOLD["rates"])
def test_page_rate_figures(row):
    tbps = page_bytes(row["T"], GOLD["H"]) / (row["us"] * 1e-6) / 1e12
    assert abs(tbps - row["TBps"]) < 0.005


def test_copy_floor():
    f = GOLD["copy_floor"]
    us = page_bytes(f["T"], GOLD["H"]) / (f["TBps"] * 1e12) * 1e6
    assert abs(us - f["us"]) < 1


def test_workload_totals():
    H = 5120
    assert total_bytes(8, 512) == 281_184
    assert total_bytes(4, H) == 2_386_784
    assert total_bytes(384, H, "post", "mxfp8") == 43_399_264
    assert total_bytes(4160, H, "no_post", "bf16") == 215_434_336
    assert total_bytes(16384, H, "post", "fp8_grid") == 1_850_615_904
    r, w = seam_bytes(16384, H, "post", "fp8_grid")
    assert r == 8 * 16384 * H + 2 * 16384 * H + 96 * 16384 + 386 * H + 96
    assert total_bytes(16, 512, identity_pre=True) == total_bytes(16, 512) - 16 * 16


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU; --gpus N > 1 exits with status 2 and a
    message, before it touches a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus 2 is not supported" in r.stderr
    assert r.stdout == ""
