"""Host-side summaries of rocprofv3 CSV output (CPU only, synthetic CSV files)."""
import csv
import os

import pytest

from paged_kv_attention_prefill_amd import profiling as PR

COLS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


@pytest.fixture
def pmc_dir(tmp_path):
    rows = []
    # two dispatches of the attention kernel (100 us and 200 us), one of a copy kernel
    for disp, t0, t1, mfma, gui in ((1, 1_000, 101_000, 40.0, 8 * 200_000), (2, 500_000, 700_000, 50.0, 8 * 400_000)):
        for name, val in (("MfmaUtil", mfma), ("VALUBusy", 30.0), ("GRBM_GUI_ACTIVE", gui), ("SQ_INSTS_MFMA", 10.0)):
            rows.append([disp, "void pa::flash_attn_kernel<2, 128, true>(...)", name, val, t0, t1])
    rows.append([3, "__amd_rocclr_copyBuffer", "MfmaUtil", 0.0, 0, 10])
    _write(tmp_path / "pmc_counter_collection.csv", COLS, rows)
    _write(tmp_path / "pmc_agent_info.csv", ["Agent_Type", "Num_Xcc"], [["CPU", 1], ["GPU", 8]])
    return str(tmp_path)


def test_utilisation_averages_dispatches_and_divides_the_gui_count_by_the_xcds(pmc_dir):
    u = PR.utilisation(pmc_dir, "flash_attn_kernel")
    assert u["dispatches"] == 2
    assert u["avg_us"] == pytest.approx(150.0)
    assert u["MfmaUtil"] == pytest.approx(45.0)
    assert u["VALUBusy"] == pytest.approx(30.0)
    # 200 000 GUI-active cycles per XCD in 100 us, 400 000 in 200 us: 2 GHz
    assert u["clock_ghz"] == pytest.approx(2.0)
    assert u["SQ_INSTS_MFMA"] == pytest.approx(10.0)
    assert "LDSBankConflict" not in u


def test_utilisation_of_a_kernel_that_is_not_there(pmc_dir):
    with pytest.raises(SystemExit):
        PR.utilisation(pmc_dir, "mla_rows8_kernel")


def test_kernel_stats_from_a_trace(tmp_path):
    _write(tmp_path / "kt_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [["k_a", 0, 3_000], ["k_a", 10_000, 15_000], ["k_b", 0, 1_000]])
    stats = PR.kernel_stats(str(tmp_path))
    assert [s["kernel"] for s in stats] == ["k_a", "k_b"]  # by total time
    assert stats[0]["calls"] == 2 and stats[0]["avg_us"] == pytest.approx(4.0)
    assert stats[0]["min_us"] == pytest.approx(3.0) and stats[0]["max_us"] == pytest.approx(5.0)
    assert os.path.basename(PR.TRAFFIC_JSON) == "traffic.json"


def test_kernel_sources_follow_each_family_and_its_includes():
    from paged_kv_attention_prefill_amd import profiling as P
    gqa = P.kernel_sources("gqa_decode_split_kernel")
    assert {"gqa_decode.hip", "balance.h", "mfma_common.h", "device_common.h", "params.h",
            "api.cpp"} <= set(gqa)
    assert "mla_decode.hip" not in gqa and "flash_attn.hip" not in gqa
    flash = P.kernel_sources("flash_attn_kernel")
    assert "flash_attn.hip" in flash and "balance.h" not in flash
    assert "mla_decode.hip" in P.kernel_sources("mla_rows8_kernel")
    # unknown names hash every source
    assert set(P.kernel_sources("")) >= set(gqa) | set(flash)
    assert P.kernel_source_hash("gqa_decode_split_kernel") != P.kernel_source_hash("flash_attn_kernel")
