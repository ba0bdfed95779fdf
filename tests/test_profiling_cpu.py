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
