"""Host logic of the measurement helpers: kernel-name mapping and stale-counter detection."""
import json
import os

from state_space_sequence_mamba_amd import profiling as PR


def test_kernel_key_mapping():
    assert PR.kernel_key("void ssd::chunk_scan_rows_kernel<float, 64, 64, 2>(...)") == "chunk_scan"
    assert PR.kernel_key("void ssd::chunk_state_kernel<__bf16, 64, 128>(...)") == "chunk_state"
    assert PR.kernel_key("void ssd::conv1d_silu_kernel<__bf16, 4>(...)") == "conv1d_silu"
    assert PR.kernel_key("void ssd::conv1d_silu_step_kernel<float, 4>(...)") == "conv1d_silu_step"
    assert PR.kernel_key("void ssd::ssd_step_kernel<float, 64, 64>(...)") == "ssd_step"
    assert PR.kernel_key("__amd_rocclr_copyBuffer") == "copy"
    assert PR.kernel_key("some_other_kernel") is None


def test_load_traffic_rejects_other_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(PR, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    good = PR.source_digest("chunk_scan")
    t = {"kernels": {"chunk_scan": {"bytes": 123.0, "source_digest": good},
                     "chunk_state": {"bytes": 7.0, "source_digest": "0" * 64}}}
    with open(tmp_path / "profiles" / "traffic_w.json", "w") as fh:
        json.dump(t, fh)
    assert PR.load_traffic("w", "chunk_scan") == 123.0
    assert PR.load_traffic("w", "chunk_state") is None         # taken on other sources
    assert PR.load_traffic("w", "ssd_step") is None            # not measured
    assert PR.load_traffic("missing", "chunk_scan") is None
    # digests differ between kernels, so one kernel's change leaves the others' counters valid
    assert PR.source_digest("chunk_scan") != PR.source_digest("chunk_state")


def test_mfma_summary_counts_512_flops_per_mop(tmp_path):
    """The MFMA counter summary: counted flops = 512 x MOPS per dispatch (summed over counter
    instances, averaged over dispatches), divided by the algorithmic flops and by the duration
    taken from a kernel-trace summary."""
    import argparse
    import csv

    d = tmp_path / "pmc"
    d.mkdir()
    name = "void ssd::chunk_scan_rows_kernel<float, 64, 64, 1, true>(float const*)"
    with open(d / "x_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp, mops in ((1, 1000.0), (2, 3000.0)):            # two dispatches: mean 2000 MOPS
            for c in PR.MFMA_COUNTERS:
                v = {"SQ_INSTS_VALU_MFMA_MOPS_F32": mops / 2, "SQ_INSTS_VALU_MFMA_MOPS_BF16": 0.0,
                     "SQ_WAVE_CYCLES": 100.0, "SQ_WAIT_INST_ANY": 25.0}.get(c, 1.0)
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": c, "Counter_Value": v})
    log = tmp_path / "b.log"
    log.write_text(json.dumps({"metric": "m", "dtype": "f32",
                               "kernels": {"chunk_scan": {"us": 99.0, "alg_flops": 512000}}}) + "\n")
    trace = tmp_path / "t.md"
    trace.write_text("| kernel | calls | rocprofv3 average (us) | share | ev |\n|---|---|---|---|---|\n"
                     "| `_ZN3ssd22chunk_scan_rows_kernelIfLi64ELi64ELi1ELb1EEEvPKT_` | 7 | 2.00 | 50 % | 2.1 |\n")
    out = tmp_path / "m.md"
    PR.mfma(argparse.Namespace(pmc=str(d), log=str(log), trace_md=str(trace), workload="w", command="c",
                               out=str(out)))
    row = [ln for ln in out.read_text().splitlines() if ln.startswith("| chunk_scan")][0]
    cells = [c.strip() for c in row.split("|")[1:-1]]
    assert cells[1] == "2"                                  # dispatches
    assert cells[2] == "0.001"                              # 512 * 2000 flops = 1.024e6 flops
    assert cells[4] == "2.00"                               # against 512000 algorithmic flops
    assert cells[5] == "2.00"                               # duration from the trace, not the log
    assert cells[6] == "0.5"                                # 1.024e6 flops / 2 us = 0.512 TFLOP/s
    assert cells[8] == "25 %"                               # wait share
