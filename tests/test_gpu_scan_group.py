"""GPU parity of the group form of chunk_scan (one workgroup per chunk, group and slice of the
group's heads, C B^T formed once per slice; bf16, chunk 256, headdim 64, dstate 128), through the
C ABI.

It performs the row-block form's MFMA sequence and decay factors, so its outputs agree with that
form's to rounding (a few elements move by a rounding step); both are compared with the float64
oracle (rel_err <= 2e-2, bf16 inputs).
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


def _agree(a, b, what):
    """a and b differ on a few elements only, each by less than one bf16 step at the tensor's
    scale (an intermediate bf16 product that rounds the other way moves a small output by more
    than its own step, but not beyond the scale of the terms it sums)."""
    da, db = a.float(), b.float()
    diff = (da - db).abs()
    scale = float(db.abs().max())
    assert float(diff.max()) <= scale * 2.0**-8, f"{what}: difference {float(diff.max()):.3e} (scale {scale:.3e})"
    assert float((diff > 0).float().mean()) < 1e-2, f"{what}: too many elements differ"


def _run(d, opts, z=None, init=None):
    y, fin = ssd.ssd_fwd(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d.get("D"), chunk_size=256,
                         z=z, initial_state=init, opts=opts)
    torch.cuda.synchronize()
    return y, fin


CASES = [
    # (B, L, H, G, heads per workgroup): ragged and single-chunk lengths, several groups and
    # slice sizes, a chunk shorter than one 16-row strip
    (1, 1, 4, 1, 4), (2, 7, 4, 2, 1), (1, 255, 6, 2, 3), (2, 256, 8, 1, 4), (1, 257, 8, 4, 2),
    (2, 700, 8, 2, 2), (1, 1101, 12, 3, 4), (3, 513, 10, 1, 5), (1, 2048, 16, 2, 8),
]


@pytest.mark.parametrize("Bt,L,H,G,hs", CASES)
def test_group_form_equals_row_blocks_and_oracle(Bt, L, H, G, hs):
    _say(f"scan group B{Bt} L{L} H{H} G{G} hs{hs}")
    inp = I.make_fwd_inputs(Bt, L, H, 64, 128, G, "bf16", seed=400 + L + H, d_init="normal")
    d = {k: v.to(DEV) for k, v in inp.items()}
    y1, f1 = _run(d, {"scan_variant": 1, "state_path": 1})
    y3, f3 = _run(d, {"scan_variant": 3, "heads_per_block": hs, "state_path": 1})
    _agree(y3, y1, "y")
    assert torch.equal(f3, f1)           # the states come from the same chunk-state kernels
    yr, fr = ssd_recurrence(*(to64(inp[k]) for k in ("x", "dt", "dt_bias", "A", "B", "C", "D")))
    assert rel_err(to64(y3), yr) <= TOL["bf16"]
    assert rel_err(to64(f3), fr) <= TOL["bf16"]


@pytest.mark.parametrize("gate,init,noD", [(True, False, False), (False, True, False), (True, True, True)])
def test_group_form_gate_initial_state_no_D(gate, init, noD):
    _say(f"scan group gate={gate} init={init} noD={noD}")
    Bt, L, H, G = 2, 600, 8, 2
    inp = I.make_fwd_inputs(Bt, L, H, 64, 128, G, "bf16", seed=420, d_init="normal")
    if noD:
        inp["D"] = None
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    z = I.make_gate((Bt, L, H, 64), "bf16", seed=421) if gate else None
    h0 = torch.randn(Bt, H, 64, 128, generator=torch.Generator().manual_seed(422)) if init else None
    zd = None if z is None else z.to(DEV)
    hd = None if h0 is None else h0.to(DEV)
    for path in (1, 2):
        y1, f1 = _run(d, {"scan_variant": 1, "state_path": path}, z=zd, init=hd)
        y3, f3 = _run(d, {"scan_variant": 3, "heads_per_block": 2, "state_path": path}, z=zd, init=hd)
        _agree(y3, y1, f"y path {path}")
        assert torch.equal(f3, f1), path
    yr, fr = ssd_recurrence(*(None if inp[k] is None else to64(inp[k]) for k in ("x", "dt", "dt_bias", "A", "B", "C",
                                                                                 "D")),
                            initial_state=None if h0 is None else to64(h0), z=None if z is None else to64(z))
    assert rel_err(to64(y3), yr) <= TOL["bf16"]
    assert rel_err(to64(f3), fr) <= TOL["bf16"]


def test_group_form_other_shapes_fall_back():
    """Sizes without a group instantiation (fp32, chunk 128, dstate 64) take the row blocks:
    asking for the group form changes nothing."""
    _say("scan group fallback")
    for dtype, N, Q in (("f32", 64, 256), ("bf16", 128, 128), ("bf16", 64, 256)):
        inp = I.make_fwd_inputs(1, 300, 4, 64, N, 1, dtype, seed=430, d_init="normal")
        d = {k: v.to(DEV) for k, v in inp.items()}
        a = ssd.ssd_fwd(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"], chunk_size=Q)
        b = ssd.ssd_fwd(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], d["D"], chunk_size=Q,
                        opts={"scan_variant": 3})
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), (dtype, N, Q)
