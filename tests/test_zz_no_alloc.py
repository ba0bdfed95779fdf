"""GPU test of ssd_fwd_noalloc, the forward that takes its workspace from the library's fixed
scratch instead of the caller: through the C ABI, its outputs must equal ssd_fwd's (same kernels,
same launch choice: bit for bit) on consecutive calls, the second smaller than the first, and
match the float64 oracle; sizes beyond the scratch are refused before anything is written.
"""
import sys

import numpy as np
import pytest
import torch

from helpers import TOL, rel_err, to64
from oracle import ssd_recurrence
from state_space_sequence_mamba_amd import inputs as I
from state_space_sequence_mamba_amd import ssd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _dev(inp):
    return {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}


def _both(inp, Q, z=None, init=None):
    """(ssd_fwd outputs, ssd_fwd_noalloc outputs) for the same arguments."""
    d = _dev(inp)
    args = (d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"])
    y_ref, f_ref = ssd.ssd_fwd(*args, chunk_size=Q, z=z, initial_state=init)
    y = torch.full_like(d["x"], float("nan"))
    fin = torch.full_like(f_ref, float("nan"))
    ssd.ssd_fwd_noalloc(*args, chunk_size=Q, y=y, final_state=fin, z=z, initial_state=init)
    torch.cuda.synchronize()
    return (y_ref, f_ref), (y, fin)


@pytest.mark.parametrize("first,second", [
    # (dtype, B, L, H, P, N, G, Q): the second call smaller than the first
    (("bf16", 2, 700, 8, 64, 128, 2, 256), ("bf16", 1, 130, 4, 64, 64, 1, 64)),
    (("f32", 2, 1000, 12, 64, 64, 1, 256), ("f32", 1, 77, 4, 32, 32, 2, 128)),
])
def test_noalloc_matches_ssd_fwd_on_consecutive_calls(first, second):
    for k, (dtype, Bt, L, H, P, N, G, Q) in enumerate((first, second)):
        _say(f"ssd_fwd_noalloc call {k + 1}: {dtype} B{Bt} L{L} H{H} P{P} N{N} G{G} Q{Q}")
        dims = ssd.make_dims(Bt, L, H, P, N, G, {"f32": torch.float32, "bf16": torch.bfloat16}[dtype])
        assert 0 < ssd.ssd_fwd_workspace_size(dims, Q) <= ssd.NOALLOC_SCRATCH_BYTES
        inp = I.make_fwd_inputs(Bt, L, H, P, N, G, dtype, seed=300 + k + L, d_init="normal")
        z = I.make_gate((Bt, L, H, P), dtype, seed=310 + k).to(DEV) if k == 0 else None
        init = torch.randn(Bt, H, P, N, generator=torch.Generator().manual_seed(320 + k)).to(DEV) if k == 0 else None
        (y_ref, f_ref), (y, fin) = _both(inp, Q, z=z, init=init)
        assert torch.equal(y, y_ref), "y differs from ssd_fwd"
        assert torch.equal(fin, f_ref), "final_state differs from ssd_fwd"
        yr, fr = ssd_recurrence(to64(inp["x"]), to64(inp["dt"]), to64(inp["dt_bias"]), to64(inp["A"]),
                                to64(inp["B"]), to64(inp["C"]), to64(inp["D"]),
                                initial_state=None if init is None else to64(init),
                                z=None if z is None else to64(z))
        assert rel_err(to64(y), yr) <= TOL[dtype]
        assert rel_err(to64(fin), fr) <= TOL[dtype]


def test_noalloc_refuses_sizes_beyond_its_scratch():
    _say("ssd_fwd_noalloc over the scratch limit")
    Bt, L, H, P, N, G = 8, 4096, 32, 64, 128, 1
    dims = ssd.make_dims(Bt, L, H, P, N, G, torch.bfloat16)
    assert ssd.ssd_fwd_workspace_size(dims, 256) > ssd.NOALLOC_SCRATCH_BYTES
    x = torch.zeros(Bt, L, H, P, dtype=torch.bfloat16, device=DEV)
    dt = torch.zeros(Bt, L, H, dtype=torch.bfloat16, device=DEV)
    Bm = torch.zeros(Bt, L, G, N, dtype=torch.bfloat16, device=DEV)
    y = torch.full_like(x, float("nan"))
    fin = torch.full((Bt, H, P, N), float("nan"), device=DEV)
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_fwd_noalloc(x, dt, torch.zeros(H, device=DEV), -torch.ones(H, device=DEV), Bm, Bm.clone(),
                            chunk_size=256, y=y, final_state=fin)
    assert e.value.status == ssd.SSD_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.isnan(y).all() and torch.isnan(fin).all()
