"""Host-side logic of bench.py (no GPU): the one-GPU guard, the FLOP
convention, per-launch statistics and the source-hash check that decides
whether the committed HBM-traffic figure may be reported."""
import json

import pytest

import bench


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_flop_convention():
    # 4*D per (query, key) pair, causal counts half of B*H*N^2
    assert bench.fwd_flops(4, 32, 4096, 128, True) == pytest.approx(5.497558138880e11)
    assert bench.fwd_flops(1, 1, 128, 64, False) == 4 * 128 * 128 * 64


def test_launch_stats():
    st = bench.launch_stats("w", 1e12, [2.0, 1.0, 4.0])
    assert st["ms_median"] == 2.0 and st["ms_min"] == 1.0
    assert st["ms_mean"] == pytest.approx(7.0 / 3, abs=1e-4)
    assert st["tflops"] == pytest.approx(500.0)  # 1e12 flops in 2 ms
    assert st["frac"] == pytest.approx(500.0 / bench.PEAK_BF16_TFLOPS, abs=1e-4)
    json.dumps(st)


def test_traffic_only_for_matching_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic() is None  # no file
    f.write_text("source_hash: %s\ntraffic_bytes_per_launch: 123456789\n"
                 % bench.kernel_source_hash())
    assert bench.measured_traffic() == 123456789.0
    f.write_text("source_hash: 0000000000000000\ntraffic_bytes_per_launch: 1\n")
    assert bench.measured_traffic() is None  # taken on other sources
