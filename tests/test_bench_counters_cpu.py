"""CPU checks of bench.py's counter-CSV handling (--counters): dispatches are
grouped and ordered by id, counters summed over their rows, kernels keyed by
name, and the timed launches picked after the warm-up and settling ones."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

HEADER = ("Correlation_Id,Dispatch_Id,Agent_Id,Queue_Id,Process_Id,Thread_Id,Grid_Size,"
          "Kernel_Id,Kernel_Name,Workgroup_Size,LDS_Block_Size,Scratch_Size,VGPR_Count,"
          "Accum_VGPR_Count,SGPR_Count,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp")


def _row(did, name, ctr, val, t0, t1):
    return f"{did},{did},1,1,1,1,256,7,\"{name}\",512,0,0,224,0,96,{ctr},{val},{t0},{t1}"


def test_read_counter_csv_and_timed_window(tmp_path):
    fwd = "void mha::mha_fwd_kernel<mha::BF16, 128, true>(mha::Params)"
    copy = "__amd_rocclr_copyBuffer"
    rows = [HEADER]
    # dispatch ids out of order in the file; two rows of one counter per dispatch
    # (per-XCD instances) must be summed
    plan = [(3, fwd, 30.0), (1, copy, 10.0), (2, fwd, 20.0), (5, fwd, 50.0), (4, fwd, 40.0),
            (6, fwd, 60.0), (7, fwd, 70.0)]
    for did, name, val in plan:
        rows.append(_row(did, name, "FETCH_SIZE", val / 2, 100 * did, 100 * did + 90))
        rows.append(_row(did, name, "FETCH_SIZE", val / 2, 100 * did, 100 * did + 90))
    path = tmp_path / "p_counter_collection.csv"
    path.write_text("\n".join(rows) + "\n")
    ds = bench.read_counter_csv(str(path))
    assert [d["FETCH_SIZE"] for d in ds] == [10.0, 20.0, 30.0, 40.0, 50.0, 60.0, 70.0]
    assert ds[0]["key"] == "__amd_rocclr_copyBuffer"
    assert all(d["key"] == "mha_fwd_kernel" for d in ds[1:])
    assert ds[2]["end"] - ds[2]["start"] == 90
    # forward launches: 20 (warm-up), 30 and 40 (settling), then the timed ones
    timed = bench._timed(ds, "mha_fwd_kernel", {"settle_launches": 2}, 3)
    assert [d["FETCH_SIZE"] for d in timed] == [50.0, 60.0, 70.0]


def test_kernel_key():
    assert bench._kernel_key("void mha::mha_bwd_dkdv_kernel<mha::F16, 64, false>(mha::BwdParams)") \
        == "mha_bwd_dkdv_kernel"
    assert bench._kernel_key("void mha::mha_split_partial_kernel<mha::BF16, 128, 1, false>(x)") \
        == "mha_split_partial_kernel"
    assert bench._kernel_key("some_other_kernel") is None
