"""The bench's reduction of rocprofv3 counter CSVs (no GPU): per-dispatch
sums over a counter's instance rows, other counters ignored."""
import bench


def test_pmc_per_dispatch_sums_instances(tmp_path):
    path = tmp_path / "pmc_counter_collection.csv"
    rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value",
            "1,void dkv::(anonymous namespace)::attn_split_kernel(dkv::StepArgs),FETCH_SIZE,10.5",
            "1,void dkv::(anonymous namespace)::attn_split_kernel(dkv::StepArgs),FETCH_SIZE,4.5",
            "1,void dkv::(anonymous namespace)::attn_split_kernel(dkv::StepArgs),WRITE_SIZE,99",
            "2,__amd_rocclr_copyBuffer,FETCH_SIZE,7"]
    path.write_text("\n".join(rows) + "\n")
    got = bench.pmc_per_dispatch(str(path), "FETCH_SIZE")
    assert got == {1: ("void dkv::(anonymous namespace)::attn_split_kernel(dkv::StepArgs)", 15.0),
                   2: ("__amd_rocclr_copyBuffer", 7.0)}
    assert bench.pmc_per_dispatch(str(path), "WRITE_SIZE")[1][1] == 99.0


def test_committed_traffic_records_match_the_kernel_sources():
    """Every committed split-kernel counter record was taken on the code the
    split kernel is compiled from now (the bench reports a record's traffic
    only while its hash matches), and its reduction is self-consistent:
    traffic = scaled FETCH_SIZE + scaled WRITE_SIZE, and the ratio to the
    algorithmic bytes is the one stored."""
    import glob
    import json
    import os
    records = sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "attn_split_*_traffic.json")))
    assert records
    sha = bench.split_kernel_sha256()
    for path in records:
        with open(path) as f:
            rec = json.load(f)
        name = os.path.basename(path)
        assert rec["split_kernel_sources_sha256"] == sha, name
        cal = rec["calibration"]
        traffic = (rec["fetch_size_kib_per_dispatch"] * cal["fetch_scale"]
                   + rec["write_size_kib_per_dispatch"] * cal["write_scale"]) * 1024
        assert abs(traffic - rec["traffic_bytes_per_launch"]) <= 1e-6 * traffic + 2048, name
        ratio = rec["traffic_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
        assert abs(ratio - rec["traffic_over_algorithmic"]) < 1e-9, name
        assert rec["traffic_over_algorithmic"] >= 1.0, name
