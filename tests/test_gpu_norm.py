"""GPU parity of the gated RMSNorm (ssd_gated_rmsnorm through the C ABI) against the float64
oracle (oracle/gated_norm.py): fp32 and bf16, with and without the gate, norm groups of one head,
of several heads and of all heads (group lengths that are and are not multiples of the 512
channels a wavefront sweeps at once), decode-shaped input, in place, no tokens, determinism, and
the B2 L16384 H80 P64 bf16 scan output on sampled tokens.  Bars: rel_err <= 1e-4 (fp32),
2e-2 (bf16)."""
import sys

import numpy as np
import pytest
import torch

from helpers import TOL, p999_rel_err, rel_err, to64
from oracle.gated_norm import gated_rmsnorm as ref_norm
from state_space_sequence_mamba_amd import inputs as I
from state_space_sequence_mamba_amd import ssd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


CASES = [
    # (B, L, H, P, norm_heads)
    (2, 37, 4, 64, 4), (2, 37, 4, 64, 1), (2, 37, 4, 64, 2), (1, 5, 6, 32, 6), (1, 5, 6, 32, 3),
    (3, 1, 3, 16, 3), (1, 130, 10, 64, 10), (2, 3, 16, 64, 16),
    (1, 3, 96, 64, 96), (1, 2, 81, 64, 81),            # groups beyond the 5120 channels kept in registers
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate", [True, False])
@pytest.mark.parametrize("Bt,L,H,P,nh", CASES)
def test_gated_rmsnorm_matches_oracle(dtype, gate, Bt, L, H, P, nh):
    _say(f"norm {dtype} gate={gate} B{Bt} L{L} H{H} P{P} nh{nh}")
    inp = I.make_norm_inputs(Bt, L, H, P, dtype, seed=600 + L + H + nh)
    d = {k: v.to(DEV) for k, v in inp.items()}
    eps = 1e-5 if dtype == "bf16" else 1e-3
    out = ssd.gated_rmsnorm(d["y"], d["weight"], z=d["z"] if gate else None, eps=eps, norm_heads=nh)
    torch.cuda.synchronize()
    ref = ref_norm(inp["y"], inp["z"] if gate else None, inp["weight"], eps=eps, norm_heads=nh)
    assert out.dtype == d["y"].dtype and out.shape == d["y"].shape
    assert rel_err(to64(out), ref) <= TOL[dtype]
    print(f"[gpu-case] rel_err {rel_err(to64(out), ref):.2e} p99.9 {p999_rel_err(to64(out), ref):.2e}", flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_in_place_decode_shape_and_determinism(dtype):
    _say(f"norm in place / decode {dtype}")
    inp = I.make_norm_inputs(4, 1, 8, 64, dtype, seed=610)
    y3 = inp["y"][:, 0].contiguous()                     # (B, H, P): one decode token per sequence
    z3 = inp["z"][:, 0].contiguous()
    ref = ref_norm(y3.unsqueeze(1), z3.unsqueeze(1), inp["weight"], eps=1e-5, norm_heads=4)[:, 0]
    yd, zd, wd = y3.to(DEV), z3.to(DEV), inp["weight"].to(DEV)
    a = ssd.gated_rmsnorm(yd, wd, z=zd, norm_heads=4)
    b = ssd.gated_rmsnorm(yd, wd, z=zd, norm_heads=4)
    yi = yd.clone()
    c = ssd.gated_rmsnorm(yi, wd, z=zd, norm_heads=4, out=yi)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(a, c) and c.data_ptr() == yi.data_ptr()
    assert rel_err(to64(a), ref) <= TOL[dtype]


def test_no_tokens():
    _say("norm no tokens")
    w = torch.ones(4 * 64, device=DEV)
    for shape in ((0, 3, 4, 64), (2, 0, 4, 64)):
        y = torch.empty(shape, dtype=torch.bfloat16, device=DEV)
        out = ssd.gated_rmsnorm(y, w, z=torch.empty_like(y))
        assert out.shape == y.shape


def test_full_size_bf16_sampled_tokens():
    """The B2 L16384 H80 P64 bf16 scan output normalised over all 80 heads (5120 channels) with the
    gate; sampled tokens of every batch row, first and last included, against the oracle."""
    _say("norm full size B2 L16384 H80 P64 bf16")
    Bt, L, H, P = 2, 16384, 80, 64
    inp = I.make_norm_inputs(Bt, L, H, P, "bf16", seed=620)
    d = {k: v.to(DEV) for k, v in inp.items()}
    out = to64(ssd.gated_rmsnorm(d["y"], d["weight"], z=d["z"], eps=1e-5))
    toks = np.unique(np.concatenate([[0, 1, L - 1], np.random.default_rng(621).integers(0, L, 29)]))
    for b in range(Bt):
        ref = ref_norm(inp["y"][b:b + 1, toks], inp["z"][b:b + 1, toks], inp["weight"], eps=1e-5)
        assert rel_err(out[b:b + 1, toks], ref) <= TOL["bf16"], b
