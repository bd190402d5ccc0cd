"""The benchmark's byte accounting, pinned by the page's own printed numbers.

The torchao dim1-cast page prints (time_us, mem_bw_gbps) for three runs of a
16384^2 bf16 column-wise MX cast (tests/golden/dim1_cast_timings.txt).  Those
pairs are reproduced to the printed digits by bytes = 2MK (bf16 read) + MK
(one E4M3 byte per element) + MK/32 (one E8M0 scale per block) and
GB = 1e9 bytes; dropping the scale bytes would not reproduce them.
"""
import os

import pytest

import bench

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dim1_cast_timings.txt")


def rows():
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            label, M, K, us, gbs = [f.strip() for f in line.split("|")]
            yield label, int(M), int(K), float(us), float(gbs)


@pytest.mark.parametrize("label,M,K,us,gbs", list(rows()))
def test_page_numbers_reproduce(label, M, K, us, gbs):
    b = bench.mx_bytes(M, K, directions=1)
    assert b == 813_694_976
    assert abs(b / (us * 1e3) - gbs) < 1e-6 * gbs
    no_scales = 3 * M * K
    assert abs(no_scales / (us * 1e3) - gbs) > 1e-3 * gbs


def test_metric_and_other_byte_counts():
    assert bench.mx_bytes(16384, 16384, 2) == 1_090_519_040
    assert bench.nvfp4_bytes(16384, 16384, 2) == 838_860_800
    assert bench.mx_bytes(8192, 8192, 2, extra_inputs=1) == 406_847_488


def test_multi_gpu_request_exits(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
