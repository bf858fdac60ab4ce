"""profsum's readers on synthetic rocprofv3 CSV files (no GPU): the grid
filter that keeps one launch size of a kernel, and the wave-counter ratios."""
import csv
import os

import pytest

from ring_allreduce_reduction_02_amd import profsum

TRACE_FIELDS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Grid_Size_X"]


def _write(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        w.writerows(rows)


def test_grid_filter_keeps_one_launch_size(tmp_path):
    k = "void cc::k_ring_fused<2, 0, 8>(cc::FusedArgs)"
    rows = [{"Kernel_Name": k, "Start_Timestamp": 1000 * i, "End_Timestamp": 1000 * i + d, "Grid_Size_X": g}
            for i, (g, d) in enumerate([(8388608, 330_000), (8388608, 340_000), (176128, 11_000),
                                        (1363712, 55_000), (8388608, 335_000)])]
    rows.append({"Kernel_Name": "void cc::k_ring_fused<1, 0, 8>(cc::FusedArgs)", "Start_Timestamp": 0,
                 "End_Timestamp": 660_000, "Grid_Size_X": 8388608})
    _write(str(tmp_path / "t" / "k_kernel_trace.csv"), TRACE_FIELDS, rows)
    st = profsum.kernel_stats_of_grid(str(tmp_path / "t"), "k_ring_fused<2, 0, 8>", 8388608)
    assert st["Calls"] == 3 and st["other_calls"] == 2
    assert st["AverageNs"] == pytest.approx(335_000)
    assert st["MinNs"] == 330_000 and st["MaxNs"] == 340_000
    with pytest.raises(KeyError):
        profsum.kernel_stats_of_grid(str(tmp_path / "t"), "k_ring_fused<2, 0, 8>", 4096)


def test_limiter_ratios_count_every_xcd(tmp_path):
    k = "void cc::k_quant_ef_fused<2>(cc::QArgs)"
    vals = {"SQ_WAVES": 1000.0, "SQ_WAVE_CYCLES": 2.0e6, "SQ_ACTIVE_INST_VALU": 4.0e5, "SQ_WAIT_INST_ANY": 1.0e5,
            "SQ_INSTS_VALU": 9.0e5, "SQ_INSTS_VMEM_RD": 2.0e4, "SQ_INSTS_VALU_TRANS_F32": 0.0,
            "GRBM_GUI_ACTIVE": 8 * 1.0e6}
    rows = [{"Kernel_Name": k, "Counter_Name": n, "Counter_Value": v} for n, v in vals.items()]
    _write(str(tmp_path / "l" / "k_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    d = profsum.limiter_counters(str(tmp_path / "l"), "k_quant_ef_fused<2>")["derived"]
    assert d["valu_cycles_over_wave_cycles"] == pytest.approx(0.2)
    assert d["wait_any_over_wave_cycles"] == pytest.approx(0.05)
    # 4e5 wave-quad-cycles of VALU over 1024 SIMDs during 1e6 cycles of one XCD
    assert d["valu_busy_of_simds"] == pytest.approx(4.0e5 * 4 / 1024 / 1.0e6)
    assert d["valu_insts_per_wave"] == pytest.approx(900.0)
