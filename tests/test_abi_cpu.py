"""CPU-side checks of the C ABI: the library loads, exports every declared symbol, and its
host-only logic (workspace sizing, status strings, argument validation that returns before
any HIP call) behaves as include/ssd.h states.  No kernel is launched here."""
import ctypes
import glob
import os
import re
import subprocess

import pytest

from state_space_sequence_mamba_amd import ssd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions(peak=False):
    """Functions declared by include/*.h: those of ssd_peak.h (the measurement-only
    libssd_peak.so) with peak=True, the others (libssd.so) without."""
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        if (os.path.basename(h) == "ssd_peak.h") != peak:
            continue
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(ssd_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ssd.LIB_PATH):
        pytest.fail("libssd.so is not built (run __graft_entry__.build())")
    return ssd.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"ssd_fwd", "ssd_fwd_ex", "ssd_step", "ssd_step_ex", "ssd_fwd_workspace_size", "ssd_status_string",
            "ssd_bwd_ex", "ssd_conv1d_silu_ex", "ssd_fwd_state_path"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(names) <= exported


def test_peak_probe_library_exports_its_declared_symbols():
    from state_space_sequence_mamba_amd import build as B
    if not os.path.exists(B.LIB_PEAK):
        pytest.fail("libssd_peak.so is not built (run __graft_entry__.build())")
    names = _declared_functions(peak=True)
    assert names == ["ssd_peak_mfma_flops", "ssd_peak_mfma_launch"]
    peak = ctypes.CDLL(B.LIB_PEAK)
    peak.ssd_peak_mfma_flops.restype = ctypes.c_double
    peak.ssd_peak_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int]
    assert peak.ssd_peak_mfma_flops(0, 2, 3) == 2048.0 * 4 * 3 * 4 * 2
    assert peak.ssd_peak_mfma_flops(1, 1, 1) == 16384.0 * 16
    # invalid arguments return 1 before any HIP call
    peak.ssd_peak_mfma_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                          ctypes.c_void_p]
    assert peak.ssd_peak_mfma_launch(0, 0, 1, None, None) == 1
    assert peak.ssd_peak_mfma_launch(5, 1, 1, ctypes.c_void_p(16), None) == 1


def test_library_is_built_for_gfx950():
    out = subprocess.run(["strings", ssd.LIB_PATH], capture_output=True, text=True).stdout
    assert "gfx950" in out


def test_status_strings(lib):
    for code in range(6):
        s = ssd.ssd_status_string(code)
        assert s and s != "unknown status"
    assert ssd.ssd_status_string(99) == "unknown status"


def _dims(**kw):
    d = dict(batch=1, seqlen=256, nheads=4, headdim=16, dstate=16, ngroups=1, dtype=0)
    d.update(kw)
    return ssd.ssd_dims_t(**d)


def test_workspace_size_layout(lib):
    # 1 x 256 tokens, H=4, Q=64 -> nc=4; dt' and cumsum: 4*4*64 floats = 4096 B each (256-aligned);
    # states: 4 chunks * 4 heads * 16 * 16 floats = 16384 B; fp32 adds C B^T once per group:
    # 4 chunks * 1 group * 1 block pair (Q/64 = 1) * 16 KB = 65536 B
    assert ssd.ssd_fwd_workspace_size(_dims(), 64) == 2 * 4096 + 16384 + 65536
    # ragged: L=300, Q=128 -> nc=3; 2*4*3*128*4 = 12288 B each; states 2*3*4*64*128*4 = 786432 B;
    # bf16 adds the entering states rounded to bf16 (786432 / 2 B) and the segmented path's
    # exponents, 2 x (B, H, nc) floats, each region 256-aligned: 2 * 256 B
    d = _dims(batch=2, seqlen=300, headdim=64, dstate=128, dtype=1)
    assert ssd.ssd_fwd_workspace_size(d, 128) == 2 * 12288 + 786432 + 393216 + 2 * 256
    # 1 x 5 tokens, H=3, Q=64: 3*64*4 = 768 B (already 256-aligned); states 3*16*16*4 = 3072; C B^T 16 KB
    assert ssd.ssd_fwd_workspace_size(_dims(seqlen=5, nheads=3), 64) == 2 * 768 + 3072 + 16384
    # alignment padding: H=1, L=1, Q=64 -> 256 B regions
    assert ssd.ssd_fwd_workspace_size(_dims(seqlen=1, nheads=1, headdim=16, dstate=16), 64) == \
        2 * 256 + 1024 + 16384
    # Q=256 -> 4 row blocks, 10 (rb, J <= rb) block pairs of 16 KB per chunk and group;
    # L=300 -> 2 chunks (cumsums 4*2*256*4 B, states 2*4*16*16*4 B), G=2: 2 * 2 * 10 * 16384 B
    d = _dims(seqlen=300, ngroups=2)
    assert ssd.ssd_fwd_workspace_size(d, 256) == 2 * 8192 + 2 * 4 * 16 * 16 * 4 + 2 * 2 * 10 * 16384


@pytest.mark.parametrize("kw,q", [
    (dict(headdim=48), 64), (dict(dstate=128, dtype=0), 64), (dict(dstate=16, dtype=1), 64),
    (dict(dtype=5), 64), ({}, 32), ({}, 512), (dict(nheads=6, ngroups=4), 64), (dict(seqlen=-1), 64),
    (dict(nheads=0), 64), (dict(dt_min=-0.1, dt_max=1.0), 64), (dict(dt_min=0.5, dt_max=0.1), 64),
    (dict(dt_min=0.1, dt_max=0.0), 64), (dict(dt_min=0.0, dt_max=float("nan")), 64),
])
def test_workspace_size_rejects(lib, kw, q):
    assert ssd.ssd_fwd_workspace_size(_dims(**kw), q) == 0


def _fwd_status(lib, dims, chunk=64, ptr=0x100000, **over):
    p = dict(x=ptr, dt=ptr, dt_bias=ptr, A=ptr, B=ptr, C=ptr, D=None, z=None, init=None, y=ptr, fin=None,
             ws=ptr, ws_bytes=1 << 30)
    p.update(over)
    vp = ctypes.c_void_p
    return lib.ssd_fwd(None if dims is None else ctypes.byref(dims), vp(p["x"]), vp(p["dt"]), vp(p["dt_bias"]),
                       vp(p["A"]), vp(p["B"]), vp(p["C"]), vp(p["D"]), vp(p["z"]), chunk, vp(p["init"]), vp(p["y"]),
                       vp(p["fin"]), vp(p["ws"]), p["ws_bytes"], None)


def test_fwd_host_validation_returns_before_any_launch(lib):
    assert _fwd_status(lib, None) == ssd.SSD_ERR_INVALID_ARG
    assert _fwd_status(lib, _dims(), chunk=100) == ssd.SSD_ERR_UNSUPPORTED
    assert _fwd_status(lib, _dims(headdim=24)) == ssd.SSD_ERR_UNSUPPORTED
    assert _fwd_status(lib, _dims(nheads=5, ngroups=2)) == ssd.SSD_ERR_INVALID_ARG
    assert _fwd_status(lib, _dims(batch=0)) == ssd.SSD_OK               # no-op, nothing touched
    assert _fwd_status(lib, _dims(), x=None) == ssd.SSD_ERR_INVALID_ARG
    assert _fwd_status(lib, _dims(), y=None) == ssd.SSD_ERR_INVALID_ARG
    assert _fwd_status(lib, _dims(), x=0x100004) == ssd.SSD_ERR_INVALID_ARG   # not 16-byte aligned
    assert _fwd_status(lib, _dims(dtype=1, dstate=32), dt=0x100001) == ssd.SSD_ERR_INVALID_ARG
    assert _fwd_status(lib, _dims(), ws=None) == ssd.SSD_ERR_WORKSPACE
    assert _fwd_status(lib, _dims(), ws_bytes=100) == ssd.SSD_ERR_WORKSPACE
    assert _fwd_status(lib, _dims(dtype=1, dstate=32), z=0x100001) == ssd.SSD_ERR_INVALID_ARG
    assert _fwd_status(lib, _dims(dt_min=0.2, dt_max=0.1)) == ssd.SSD_ERR_INVALID_ARG
    assert _fwd_status(lib, _dims(dt_min=-1.0, dt_max=0.1)) == ssd.SSD_ERR_INVALID_ARG


def test_step_host_validation(lib):
    vp = ctypes.c_void_p
    p = vp(0x100000)
    d = _dims()
    assert lib.ssd_step(None, p, p, p, p, p, p, p, None, None, p, None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_step(ctypes.byref(_dims(dstate=24)), p, p, p, p, p, p, p, None, None, p,
                        None) == ssd.SSD_ERR_UNSUPPORTED
    assert lib.ssd_step(ctypes.byref(d), None, p, p, p, p, p, p, None, None, p, None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_step(ctypes.byref(d), vp(0x100008), p, p, p, p, p, p, None, None, p,
                        None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_step(ctypes.byref(d), p, p, p, p, p, p, p, None, vp(0x100002), p,
                        None) == ssd.SSD_ERR_INVALID_ARG                   # z misaligned for fp32
    assert lib.ssd_step(ctypes.byref(_dims(dt_min=0.3, dt_max=0.2)), p, p, p, p, p, p, p, None, None, p,
                        None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_step(ctypes.byref(_dims(batch=0)), p, p, p, p, p, p, p, None, None, p, None) == ssd.SSD_OK


def test_bwd_workspace_size_and_validation(lib):
    # 1 x 256 tokens, H=4, P=N=16, Q=64: cum regions 4096 B, states 16384 B, per-head dB/dC
    # 256*4*16*4 = 65536 B, per-chunk partials 64 -> 256 B, dD partials 4*4*16*4 = 1024 B, and
    # (fp32) the C B^T blocks of the recomputed forward (4 chunks * 16 KB), which bwd_dc reads,
    # and their transposed copy for bwd_dxdb
    base = 2 * 4096 + 2 * 16384 + 2 * 65536 + 4 * 4096 + 2 * 256 + 1024 + 2 * 65536
    assert ssd.ssd_bwd_workspace_size(_dims(), 64, 0) == base
    # the gate adds the pre-gate output and the gated gradient (2 * 256 * 4 * 16 * 4 B)
    assert ssd.ssd_bwd_workspace_size(_dims(), 64, 1) == base + 2 * 65536
    assert ssd.ssd_bwd_workspace_size(_dims(headdim=24), 64, 0) == 0
    vp = ctypes.c_void_p
    p = vp(0x100000)
    d = _dims()

    def call(dims=d, chunk=64, z=None, dz=None, ws=p, ws_bytes=1 << 30, **over):
        a = dict(x=p, dt=p, dt_bias=p, A=p, B=p, C=p, D=None, init=None, dout=p, dfinal=None, dx=p, ddt=p,
                 ddt_bias=p, dA=p, dB=p, dC=p, dD=None, dinit=None)
        a.update(over)
        return lib.ssd_bwd(None if dims is None else ctypes.byref(dims), a["x"], a["dt"], a["dt_bias"], a["A"],
                           a["B"], a["C"], a["D"], z, chunk, a["init"], a["dout"], a["dfinal"], a["dx"], a["ddt"],
                           a["ddt_bias"], a["dA"], a["dB"], a["dC"], a["dD"], dz, a["dinit"], ws, ws_bytes, None)

    assert call(dims=None) == ssd.SSD_ERR_INVALID_ARG
    assert call(chunk=32) == ssd.SSD_ERR_UNSUPPORTED
    assert call(z=p) == ssd.SSD_ERR_INVALID_ARG                  # gate without dz
    assert call(dz=p) == ssd.SSD_ERR_INVALID_ARG                 # dz without gate
    assert call(dout=None) == ssd.SSD_ERR_INVALID_ARG
    assert call(dA=None) == ssd.SSD_ERR_INVALID_ARG
    assert call(dout=vp(0x100004)) == ssd.SSD_ERR_INVALID_ARG    # not 16-byte aligned
    assert call(ws=None) == ssd.SSD_ERR_WORKSPACE
    assert call(ws_bytes=100) == ssd.SSD_ERR_WORKSPACE
    # no tokens: the per-head gradients are still written (zeros), so they must be device memory
    assert call(dims=_dims(batch=0)) == ssd.SSD_ERR_DEVICE_PTR


def test_conv_host_validation(lib):
    vp = ctypes.c_void_p
    p = vp(0x100000)
    d = _dims()
    # fwd: (dims, K, xbc, weight, bias, state_in, state_out, x, B, C, stream)
    assert lib.ssd_conv1d_silu(None, 4, p, p, None, None, None, p, p, p, None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_conv1d_silu(ctypes.byref(d), 5, p, p, None, None, None, p, p, p, None) == ssd.SSD_ERR_UNSUPPORTED
    assert lib.ssd_conv1d_silu(ctypes.byref(d), 0, p, p, None, None, None, p, p, p, None) == ssd.SSD_ERR_UNSUPPORTED
    assert lib.ssd_conv1d_silu(ctypes.byref(d), 4, None, p, None, None, None, p, p, p, None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_conv1d_silu(ctypes.byref(d), 4, p, None, None, None, None, p, p, p, None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_conv1d_silu(ctypes.byref(d), 4, p, p, None, None, None, vp(0x100008), p, p,
                               None) == ssd.SSD_ERR_INVALID_ARG                # output not 16-byte aligned
    # states that overlap without being the same buffer
    assert lib.ssd_conv1d_silu(ctypes.byref(d), 4, p, p, None, vp(0x200000), vp(0x200010), p, p, p,
                               None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_conv1d_silu(ctypes.byref(_dims(batch=0)), 4, p, p, None, None, None, p, p, p, None) == ssd.SSD_OK
    assert lib.ssd_conv1d_silu(ctypes.byref(_dims(headdim=24)), 4, p, p, None, None, None, p, p, p,
                               None) == ssd.SSD_ERR_UNSUPPORTED
    # seqlen 0 without a state to write: nothing to do
    assert lib.ssd_conv1d_silu(ctypes.byref(_dims(seqlen=0)), 4, None, None, None, None, None, None, None, None,
                               None) == ssd.SSD_OK
    # step: (dims, K, state, xbc, weight, bias, x, B, C, stream); the state is required for K > 1
    assert lib.ssd_conv1d_silu_step(ctypes.byref(d), 4, None, p, p, None, p, p, p, None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_conv1d_silu_step(ctypes.byref(d), 4, vp(0x100004), p, p, None, p, p, p,
                                    None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_conv1d_silu_step(ctypes.byref(_dims(batch=0)), 4, p, p, p, None, p, p, p, None) == ssd.SSD_OK


def test_binding_raises_without_library(monkeypatch, tmp_path):
    """The product path has no fallback: a missing library is an error, not a CPU detour."""
    monkeypatch.setattr(ssd, "_lib", None)
    monkeypatch.setattr(ssd, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not found"):
        ssd.load_library()


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "state_space_sequence_mamba_amd")
    for f in glob.glob(os.path.join(pkg, "**", "*"), recursive=True):
        if f.endswith((".py", ".hip", ".h", ".cpp")):
            text = open(f).read()
            assert not re.search(r"\boracle\b", text.replace("the oracle", "")) or f.endswith("inputs.py"), f


def test_fwd_state_path_choice_is_host_logic():
    """The chunk-state path ssd_fwd takes (pure host logic, no GPU needed): one pass for bf16
    P64 N128 from batch x heads >= 256 (segments instead at chunk 256 for 16 or more chunks when a
    group has at least four slices of heads), segments below that at chunk 256 (three or more
    chunks), two launches otherwise; per-call options force a path where an instantiation exists;
    invalid or empty sizes give 0."""
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    cases = [((8, 4096, 32, 64, 128, 1, bf), 256, 3), ((8, 4096, 32, 64, 128, 1, bf), 128, 2),
             ((16, 2048, 32, 64, 128, 1, bf), 256, 2), ((4, 4096, 64, 64, 128, 8, bf), 256, 2),
             ((8, 4096, 32, 64, 128, 1, bf), 64, 1), ((4, 4096, 32, 64, 128, 1, bf), 256, 3),
             ((2, 16384, 80, 64, 128, 8, bf), 256, 3), ((2, 512, 8, 64, 128, 1, bf), 256, 1),
             ((4, 4096, 32, 64, 128, 1, bf), 128, 1), ((8, 4096, 32, 64, 64, 1, bf), 256, 1),
             ((16, 1024, 24, 64, 64, 1, f32), 256, 1), ((8, 0, 32, 64, 128, 1, bf), 256, 0),
             ((8, 4096, 32, 64, 128, 1, bf), 100, 0)]
    for args, q, want in cases:
        assert ssd.fwd_state_path(ssd.make_dims(*args), q) == want, (args, q)
    p = lambda *a: ssd.make_dims(*a)  # noqa: E731
    assert ssd.fwd_state_path(p(4, 1024, 24, 64, 64, 1, f32), 256, {"state_path": 2}) == 2
    assert ssd.fwd_state_path(p(4, 1024, 24, 64, 64, 1, f32), 256, {"state_path": 2, "state_slice": 32}) == 2
    # no such instantiation: two launches
    assert ssd.fwd_state_path(p(4, 1024, 24, 64, 64, 1, f32), 256, {"state_path": 2, "state_slice": 16}) == 1
    assert ssd.fwd_state_path(p(8, 4096, 32, 64, 128, 1, bf), 256, {"state_path": 1}) == 1
    # segments of 8 chunks for the B2 L16384 H80 G8 shape (at least 256 workgroups), forced sizes
    assert ssd.fwd_state_segment_chunks(p(2, 16384, 80, 64, 128, 8, bf), 256) == 8
    assert ssd.fwd_state_segment_chunks(p(2, 16384, 80, 64, 128, 8, bf), 256, {"state_chunks": 4}) == 4
    assert ssd.fwd_state_segment_chunks(p(8, 4096, 32, 64, 128, 1, bf), 256) == 4
    assert ssd.fwd_state_segment_chunks(p(16, 2048, 32, 64, 128, 1, bf), 256) == 0
    assert ssd.fwd_state_path(p(16, 2048, 32, 64, 128, 1, bf), 256, {"state_path": 3, "state_heads": 4}) == 3
    assert ssd.fwd_state_path(p(8, 4096, 32, 64, 128, 1, bf), 256, {"state_path": 2}) == 2
    # options are per call: nothing of the calls above is kept
    assert ssd.fwd_state_path(p(16, 2048, 32, 64, 128, 1, bf), 256) == 2
    assert ssd.fwd_state_path(p(4, 1024, 24, 64, 64, 1, f32), 256, ssd.launch_opts()) == 1


def test_noalloc_refuses_oversize_before_any_device_call(lib):
    """ssd_fwd_noalloc checks the sizes against its fixed scratch first: an oversize problem is
    refused (no launch, no device query), and invalid sizes keep their usual codes."""
    import torch
    big = ssd.make_dims(8, 4096, 32, 64, 128, 1, torch.bfloat16)
    assert ssd.ssd_fwd_workspace_size(big, 256) > ssd.NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(0x100000)
    args = [p, p, p, p, p, p, None, None, 256, None, p, None, None]
    assert lib.ssd_fwd_noalloc(ctypes.byref(big), *args) == ssd.SSD_ERR_SCRATCH_LIMIT
    bad = ssd.make_dims(8, 4096, 33, 64, 128, 2, torch.bfloat16)       # heads not a multiple of groups
    assert lib.ssd_fwd_noalloc(ctypes.byref(bad), *args) == ssd.SSD_ERR_INVALID_ARG
    args[8] = 100                                                       # chunk size
    assert lib.ssd_fwd_noalloc(ctypes.byref(big), *args) == ssd.SSD_ERR_UNSUPPORTED
    assert "scratch" in ssd.ssd_status_string(ssd.SSD_ERR_SCRATCH_LIMIT)


def test_gated_rmsnorm_host_validation(lib):
    vp, f = ctypes.c_void_p, ctypes.c_float
    p = vp(0x100000)
    d = _dims()                                   # H = 4
    # (dims, y, z, weight, eps, norm_heads, out, stream)
    assert lib.ssd_gated_rmsnorm(None, p, None, p, f(1e-5), 4, p, None) == ssd.SSD_ERR_INVALID_ARG
    for nh in (0, 3, 5, -1):                      # must divide H
        assert lib.ssd_gated_rmsnorm(ctypes.byref(d), p, None, p, f(1e-5), nh, p, None) == ssd.SSD_ERR_INVALID_ARG
    for eps in (-1.0, float("nan"), float("inf")):
        assert lib.ssd_gated_rmsnorm(ctypes.byref(d), p, None, p, f(eps), 4, p, None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), None, None, p, f(1e-5), 4, p, None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), p, None, None, f(1e-5), 2, p, None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), vp(0x100008), None, p, f(1e-5), 2, vp(0x900000),
                                 None) == ssd.SSD_ERR_INVALID_ARG        # y not 16-byte aligned
    # out overlapping y without being y, or overlapping z
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), p, None, vp(0x800000), f(1e-5), 1, vp(0x100010),
                                 None) == ssd.SSD_ERR_INVALID_ARG
    assert lib.ssd_gated_rmsnorm(ctypes.byref(d), p, vp(0x200000), vp(0x800000), f(1e-5), 1, vp(0x200000),
                                 None) == ssd.SSD_ERR_INVALID_ARG
    # no tokens: nothing to do, the pointers may be NULL
    assert lib.ssd_gated_rmsnorm(ctypes.byref(_dims(batch=0)), None, None, None, f(0.0), 4, None,
                                 None) == ssd.SSD_OK
    assert lib.ssd_gated_rmsnorm(ctypes.byref(_dims(seqlen=0)), None, None, None, f(0.0), 2, None,
                                 None) == ssd.SSD_OK
