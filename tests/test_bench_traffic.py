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
