"""Host logic of the rocprofv3 summaries: byte scaling against the calibration copy and the MFMA
utilisation figures, on hand-made counter files whose answers are worked out below."""
import csv

import pytest

from grouped_gemm_fp32_amd import profiling as P

COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
        "End_Timestamp"]
GATHER = "void moe::(anonymous namespace)::gather_rows_kernel(int const*, int)"
TALL0 = ("void moe::(anonymous namespace)::ggemm_tall8_kernel<0, false>"
         "(moe::(anonymous namespace)::GemmArgs)")
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::AddFunctor<int> >(int)"
FILL = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<int> >(int)"


def _write(d, rows):
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, COLS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(COLS, r)))
    return str(d)


def test_traffic_scales_by_the_calibration_copy(tmp_path):
    # 4 MiB copy: FETCH_SIZE reads half of it (2048 KiB), WRITE_SIZE all of it (4096 KiB)
    fetch = _write(tmp_path / "f", [
        (1, FILL, "FETCH_SIZE", 3.0, 0, 10),            # the fills before it read almost nothing
        (2, COPY, "FETCH_SIZE", 2048.0, 20, 30),
        (3, GATHER, "FETCH_SIZE", 100.0, 40, 50),
        (4, GATHER, "FETCH_SIZE", 300.0, 60, 70),
    ])
    write = _write(tmp_path / "w", [
        (1, FILL, "WRITE_SIZE", 8192.0, 0, 10),
        (2, COPY, "WRITE_SIZE", 4096.0, 20, 30),
        (3, GATHER, "WRITE_SIZE", 500.0, 40, 50),
        (4, GATHER, "WRITE_SIZE", 500.0, 60, 70),
    ])
    t = P.traffic(fetch, write, calib_mib=4)
    assert t["fetch_calibration"]["dispatch"] == 2
    assert t["fetch_calibration"]["scale"] == pytest.approx(2.0)
    assert t["write_calibration"]["scale"] == pytest.approx(1.0)
    g = t["kernels"]["gather_rows_kernel"]
    assert g["fetch_bytes"] == pytest.approx(200.0 * 1024 * 2)    # mean of 100 and 300 KiB, x2
    assert g["write_bytes"] == pytest.approx(500.0 * 1024)
    assert g["bytes_per_launch"] == pytest.approx(200.0 * 1024 * 2 + 500.0 * 1024)


def test_traffic_rejects_runs_that_do_not_line_up(tmp_path):
    fetch = _write(tmp_path / "f", [(2, COPY, "FETCH_SIZE", 2048.0, 0, 1)])
    write = _write(tmp_path / "w", [(2, GATHER, "WRITE_SIZE", 4096.0, 0, 1)])
    with pytest.raises(ValueError):
        P.traffic(fetch, write, calib_mib=4)
    nocal = _write(tmp_path / "n", [(1, GATHER, "FETCH_SIZE", 2048.0, 0, 1)])
    with pytest.raises(ValueError):
        P.traffic(nocal, write, calib_mib=4)


def test_mfma_utilisation(tmp_path):
    # 1000 matrix instructions of 32 busy cycles each; 2000 cycles per XCD in 1000 ns: 2 GHz,
    # and 32000 busy cycles out of 1024 SIMDs x 2000 cycles
    rows = []
    for disp, ns in ((5, 1000), (9, 2000)):
        rows += [(disp, TALL0, "SQ_INSTS_MFMA", 1000.0, 100, 100 + ns),
                 (disp, TALL0, "SQ_VALU_MFMA_BUSY_CYCLES", 32000.0, 100, 100 + ns),
                 (disp, TALL0, "GRBM_GUI_ACTIVE", 8 * 2000.0, 100, 100 + ns)]
    rows.append((6, GATHER, "GRBM_GUI_ACTIVE", 80.0, 0, 5))   # no matrix instructions: skipped
    u = P.mfma_util(_write(tmp_path / "m", rows))
    assert set(u) == {"ggemm_tall8_kernel<0,false>"}
    e = u["ggemm_tall8_kernel<0,false>"]
    assert e["dispatches"] == 2
    assert e["cycles_per_inst"] == pytest.approx(32.0)
    assert e["busy_frac"] == pytest.approx(32000 / (1024 * 2000))
    assert e["clock_ghz"] == pytest.approx((2.0 + 1.0) / 2)          # 2 GHz, then 1 GHz
    assert e["us"] == pytest.approx(1.5)
    table = P.mfma_table(str(tmp_path / "m"))
    assert "fwd_gateup" in table and "1.6%" in table


def test_unit_utilisation(tmp_path):
    # 1000 cycles per XCD: 256 CUs give 256000 CU cycles; LDS serves indexed accesses in 64000 of
    # them (25%), 2560 stalled by bank conflicts (1%); the TA is busy 128000 (50%); waves wait on
    # LDS 300 of their 3000 cycles (10%)
    lds = _write(tmp_path / "l", [
        (3, TALL0, "SQ_LDS_IDX_ACTIVE", 64000.0, 0, 500),
        (3, TALL0, "SQ_LDS_BANK_CONFLICT", 2560.0, 0, 500),
        (3, TALL0, "GRBM_GUI_ACTIVE", 8 * 1000.0, 0, 500),
        (4, GATHER, "SQ_LDS_IDX_ACTIVE", 0.0, 600, 700),       # not in the TA run: left out
        (4, GATHER, "SQ_LDS_BANK_CONFLICT", 0.0, 600, 700),
        (4, GATHER, "GRBM_GUI_ACTIVE", 800.0, 600, 700)])
    ta = _write(tmp_path / "t", [
        (3, TALL0, "TA_TA_BUSY", 128000.0, 0, 500),
        (3, TALL0, "SQ_WAIT_INST_LDS", 300.0, 0, 500),
        (3, TALL0, "SQ_WAVE_CYCLES", 3000.0, 0, 500),
        (3, TALL0, "GRBM_GUI_ACTIVE", 8 * 1000.0, 0, 500)])
    u = P.unit_util(lds, ta)
    assert set(u) == {"ggemm_tall8_kernel<0,false>"}
    e = u["ggemm_tall8_kernel<0,false>"]
    assert e["lds_active"] == pytest.approx(0.25)
    assert e["lds_bank_conflict"] == pytest.approx(0.01)
    assert e["ta_busy"] == pytest.approx(0.5)
    assert e["lds_wait"] == pytest.approx(0.1)
    assert e["us"] == pytest.approx(0.5)
    table = P.units_table(lds, ta)
    assert "fwd_gateup" in table and "| 25.0% | 1.0% | 50.0% | 10.0% |" in table
