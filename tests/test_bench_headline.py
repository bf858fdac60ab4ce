"""The headline line bench.py prints last: at most 2 KB, with the keys the
benchmark contract names, built from stub measurements (no GPU)."""
import json
import types

import pytest

import bench


def stub():
    m = {"N": 8, "M": 67_108_864, "es": 4, "ms_per_step": 0.66412,
         "per_launch_ms": [0.6641, 0.6649, 0.6632], "rank_stride_bytes": (256 << 20) + (256 << 10)}
    args = types.SimpleNamespace(steps=20, warmup=5, dtype="f32", algo="ring", fuse_depth=0)
    roof = {"bound": "hbm", "kernel": "k_ring_fused", "achieved": 6466.7, "peak": 8000.0, "unit": "GB/s",
            "frac": 0.8083, "traffic": 4295314125, "traffic_over_algorithmic": 1.0001,
            "avg_launch_ms": 0.66412, "min_launch_ms": 0.6559}
    twin = {"ms_per_step": 0.33771, "GBps": 6358.9, "pct_of_peak": 79.49, "parity": True, "oracle_s": 1.523}
    ab = {"n": 8, "alpha_us": 2.017, "beta_ps_per_byte": 3.035, "link_GBps": 329.5, "n_star_bytes": 664643,
          "sizes": "4KiB..64MiB per rank", "max_rel_residual": 0.11}
    cpu = {"value": 4.789, "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": "the whole workload (ring AllReduce SUM, N=8, M=67108864 f32), step-explicit NumPy "
                     "simulator, single-threaded; 12 runs in 10.8 s, median 0.897 s",
           "host": "AMD EPYC 9575F 64-Core Processor, 256 logical CPUs, 16 in affinity"}
    return m, args, roof, twin, ab, cpu


def test_headline_size_and_keys():
    m, args, roof, twin, ab, cpu = stub()
    h = bench.make_headline(m, args, roof, twin, ab, cpu, True)
    line = bench.headline_line(h)
    assert len(line.encode()) <= 2048
    d = json.loads(line)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "pct_of_peak", "busbw_GBps", "parity",
              "roofline", "cpu_baseline"):
        assert k in d, k
    for k in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert k in d["roofline"], k
    for k in ("value", "unit", "cores", "kind", "sample"):
        assert k in d["cpu_baseline"], k
    assert d["config"]["workload"] == "ring_allreduce_sum_n8_m67108864_f32"
    assert d["config"]["rank_stride_bytes"] == (256 << 20) + (256 << 10)
    assert d["n_gpus"] == 1 and d["unit"] == "GB/s" and d["parity"] is True
    # value = algorithmic bytes / time per step; busbw = (M s / T) 2 (N-1) / N
    assert d["value"] == pytest.approx(2 * 8 * 67_108_864 * 4 / 0.66412e-3 / 1e9, rel=1e-5)
    assert d["busbw_GBps"] == pytest.approx(67_108_864 * 4 / 0.66412e-3 * 2 * 7 / 8 / 1e9, rel=1e-5)
    assert d["pct_of_peak"] == pytest.approx(100 * d["value"] / 8000.0, abs=0.01)


def test_headline_without_optional_parts():
    m, args, roof, _, _, _ = stub()
    d = json.loads(bench.headline_line(bench.make_headline(m, args, roof, None, None, None, None)))
    assert d["parity"] is None and d["cpu_baseline"] is None


def test_headline_too_long_is_refused():
    m, args, roof, twin, ab, cpu = stub()
    cpu = dict(cpu, sample="x" * 3000)
    with pytest.raises(ValueError):
        bench.headline_line(bench.make_headline(m, args, roof, twin, ab, cpu, True))


def test_gpus_above_one_exits_with_a_message(capsys, monkeypatch):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "8"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err
