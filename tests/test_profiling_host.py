"""Host-side checks of the rocprofv3 summariser (no GPU, no profiler)."""
import csv
import os

from exact_means_clustering_flashassign_amd import profiling as P


def _write_counters(path, rows):
    cols = ["Correlation_Id", "Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (k, c, v) in enumerate(rows):
            w.writerow({"Correlation_Id": i, "Dispatch_Id": i, "Kernel_Name": k, "Counter_Name": c,
                        "Counter_Value": v})


def test_phase_classification():
    assert P.phase_of("void fk::(anonymous namespace)::assign_smalld_kernel<1, 8>(int)") == "assign"
    assert P.phase_of("void fk::(anonymous namespace)::segreduce_kernel<1>(void const*)") == "update"
    assert P.phase_of("fk::(anonymous namespace)::norms_kernel<1>(float const*)") == "norms"
    assert P.phase_of("void fk::(anonymous namespace)::norms_vec_kernel<1, 32>(float const*)") == "norms"
    assert P.phase_of("void fk::(anonymous namespace)::widen_kernel<1>(unsigned short const*)") == "setup"
    assert P.phase_of("void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>") == "copy"
    assert P.phase_of("void at::native::distribution_elementwise_grid_stride_kernel<float>") == "other"


def test_counter_means_and_copy_calibration(tmp_path):
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(x)>(int)"
    asg = "void fk::(anonymous namespace)::assign_smalld_kernel<1, 8, 2, 64, true, true>(int)"
    f = tmp_path / "fetch.csv"
    _write_counters(f, [(copy, "FETCH_SIZE", 512.0), (copy, "FETCH_SIZE", 512.0),
                        (asg, "FETCH_SIZE", 100.0), (asg, "FETCH_SIZE", 300.0),
                        (asg, "GRBM_GUI_ACTIVE", 7.0)])
    fetch = P.read_counter(str(f), "FETCH_SIZE")
    assert fetch[asg] == 200.0 and fetch[copy] == 512.0
    write = {copy: 1024.0, asg: 10.0}
    per, ff, fw = P.traffic_summary(fetch, write, 1024 * 1024)
    # the copy moved 1 MiB each way: the fetch counter reads half, the write counter all of it
    assert ff == 2.0 and fw == 1.0
    assert per[asg]["read_bytes"] == 200.0 * 1024 * 2.0
    assert per[asg]["write_bytes"] == 10.0 * 1024
    assert per[asg]["phase"] == "assign"


def test_source_digest_tracks_kernel_sources():
    a, u = P.source_digest("assign"), P.source_digest("update")
    assert len(a) == 16 and len(u) == 16 and a != u
    assert os.path.exists(os.path.join(P.CSRC, "assign.hip"))
