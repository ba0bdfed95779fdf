"""GPU parity of the one-pass chunk-state path (chunk_state_seq: one workgroup per (b, h,
headdim slice) walks the chunks in order with the carried state in its MFMA accumulators, in
place of chunk_state + state_passing), through the C ABI, against the float64 oracle.

The path is forced with the launch options (state_path = 2, state_slice = rows) on small shapes that
still span several chunks, 64-token tiles and a ragged last chunk; the built-in choice takes it
for bf16 P64 N128 once batch x heads >= 256, which test_built_in_choice_takes_one_pass_for_large_bf16_batches
covers without the knob.
Bar as in the other parity tests: rel_err <= 1e-4 (fp32 inputs), <= 2e-2 (bf16 inputs).
"""
import sys

import numpy as np
import pytest
import torch

from helpers import TOL, rel_err, to64
from oracle import ssd_recurrence, ssd_stages
from state_space_sequence_mamba_amd import inputs as I
from state_space_sequence_mamba_amd import ssd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


_OPTS = None      # launch options _run passes (set by _one_pass / _two_launch)


class _forced:
    """Pass the given launch options to every _run call of a block."""

    def __init__(self, **opts):
        self.opts = opts

    def __enter__(self):
        global _OPTS
        _OPTS = self.opts

    def __exit__(self, *exc):
        global _OPTS
        _OPTS = None


def _one_pass(ps):
    return _forced(state_path=2, state_slice=ps)


def _two_launch():
    return _forced(state_path=1)


def _run(inp, Q, init=None, z=None, dt_limit=None, workspace=None):
    dev = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    y, fin = ssd.ssd_fwd(dev["x"], dev["dt"], dev["dt_bias"], dev["A"], dev["B"], dev["C"], dev.get("D"),
                         chunk_size=Q, initial_state=None if init is None else init.to(DEV),
                         z=None if z is None else z.to(DEV), dt_limit=dt_limit, workspace=workspace, opts=_OPTS)
    torch.cuda.synchronize()
    return y, fin


def _oracle(inp, init=None, z=None, dt_limit=None):
    return ssd_recurrence(to64(inp["x"]), to64(inp["dt"]), to64(inp["dt_bias"]), to64(inp["A"]),
                          to64(inp["B"]), to64(inp["C"]), None if inp.get("D") is None else to64(inp["D"]),
                          initial_state=None if init is None else to64(init),
                          z=None if z is None else to64(z), dt_limit=dt_limit)


def _dims(inp):
    Bt, L, H, P = inp["x"].shape
    G, N = inp["B"].shape[2], inp["B"].shape[3]
    return ssd.make_dims(Bt, L, H, P, N, G, inp["x"].dtype)


CASES = []
for dtype, P, N, ps in (("f32", 64, 64, 64), ("f32", 64, 64, 32), ("bf16", 64, 128, 64)):
    for L, Q, G in ((1, 256, 1), (63, 128, 1), (200, 256, 2), (256, 256, 1), (700, 256, 1), (700, 128, 4),
                    (1024, 256, 2)):
        CASES.append((dtype, P, N, ps, L, Q, G))


@pytest.mark.parametrize("dtype,P,N,ps,L,Q,G", CASES)
def test_one_pass_matches_oracle(dtype, P, N, ps, L, Q, G):
    _say(f"one-pass dtype={dtype} P={P} N={N} ps={ps} L={L} Q={Q} G={G}")
    H = 4
    inp = I.make_fwd_inputs(2, L, H, P, N, G, dtype, seed=500 + L + Q + G, d_init="normal")
    with _one_pass(ps):
        assert ssd.fwd_state_path(_dims(inp), Q, _OPTS) == 2
        y, fin = _run(inp, Q)
    yr, fr = _oracle(inp)
    assert np.all(np.isfinite(to64(y))) and np.all(np.isfinite(to64(fin)))
    ey, ef = rel_err(to64(y), yr), rel_err(to64(fin), fr)
    assert ey <= TOL[dtype], f"y rel_err {ey:.3e}"
    assert ef <= TOL[dtype], f"final_state rel_err {ef:.3e}"


@pytest.mark.parametrize("dtype,P,N,ps", [("f32", 64, 64, 64), ("bf16", 64, 128, 64)])
def test_one_pass_initial_state_gate_and_clamp(dtype, P, N, ps):
    """The initial state seeds the carried accumulators; the gate and the dt' clamp as in the
    two-launch path."""
    _say(f"one-pass init/gate/clamp dtype={dtype}")
    inp = I.make_fwd_inputs(2, 600, 4, P, N, 2, dtype, seed=77, d_init="normal")
    g = torch.Generator().manual_seed(78)
    init = torch.randn(2, 4, P, N, generator=g)
    z = I.make_gate(tuple(inp["x"].shape), dtype, seed=79)
    lim = (0.01, 0.05)
    with _one_pass(ps):
        y, fin = _run(inp, 256, init=init, z=z, dt_limit=lim)
    yr, fr = _oracle(inp, init=init, z=z, dt_limit=lim)
    assert rel_err(to64(y), yr) <= TOL[dtype]
    assert rel_err(to64(fin), fr) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_pass_agrees_with_two_launch_path(dtype):
    """Same sums in another order: the two paths agree far inside the parity bar, and each is
    deterministic from run to run."""
    _say(f"one-pass vs two launches {dtype}")
    P, N = (64, 64) if dtype == "f32" else (64, 128)
    inp = I.make_fwd_inputs(2, 900, 8, P, N, 2, dtype, seed=81, d_init="normal")
    with _two_launch():
        y1, f1 = _run(inp, 256)
    with _one_pass(64):
        y2, f2 = _run(inp, 256)
        y3, f3 = _run(inp, 256)
    assert torch.equal(y2, y3) and torch.equal(f2, f3)
    # fp32: summation order only; bf16: the entering states are rounded to bf16 on both paths,
    # so an order difference can move one rounding step
    tol_y = 1e-5 if dtype == "f32" else 1e-2
    assert rel_err(to64(y2), to64(y1)) <= tol_y
    assert rel_err(to64(f2), to64(f1)) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_pass_stage_intermediates(dtype):
    """Workspace after a one-pass call: dt' and the segment cumsum, and the states entering each
    chunk (fp32 in region [2]; bf16 rounded to bf16 in region [4])."""
    _say(f"one-pass stages {dtype}")
    Bt, L, H, G, Q = 2, 600, 4, 2, 256
    P, N = (64, 64) if dtype == "f32" else (64, 128)
    inp = I.make_fwd_inputs(Bt, L, H, P, N, G, dtype, seed=83)
    dims = _dims(inp)
    ws = torch.zeros(ssd.ssd_fwd_workspace_size(dims, Q), dtype=torch.uint8, device=DEV)
    with _one_pass(64):
        _run(inp, Q, workspace=ws)
    nc = (L + Q - 1) // Q
    cum = Bt * H * nc * Q * 4
    cum_al = (cum + 255) // 256 * 256
    f = ws.view(torch.float32)
    dtp = f[: cum // 4].view(Bt, H, nc, Q)
    dacs = f[cum_al // 4: cum_al // 4 + cum // 4].view(Bt, H, nc, Q)
    n_st = Bt * nc * H * P * N
    r_dtp, r_dacs = ssd_stages.chunk_cumsum(to64(inp["dt"]), to64(inp["dt_bias"]), to64(inp["A"]), Q)
    S = ssd_stages.chunk_state(to64(inp["x"]), to64(inp["B"]), r_dtp, r_dacs)
    r_prev, _ = ssd_stages.state_passing(S, r_dacs)
    assert rel_err(to64(dtp), r_dtp) <= 1e-6
    assert rel_err(to64(dacs), r_dacs) <= 1e-5
    if dtype == "f32":
        states = f[2 * cum_al // 4: 2 * cum_al // 4 + n_st].view(Bt, nc, H, P, N)
        assert rel_err(to64(states), r_prev) <= TOL[dtype]
    else:
        off = 2 * cum_al + (n_st * 4 + 255) // 256 * 256          # region [4] (no C B^T region: 2 heads per group)
        prev16 = ws[off: off + n_st * 2].view(torch.bfloat16).view(Bt, nc, H, P, N)
        assert rel_err(to64(prev16), r_prev) <= TOL[dtype]


def test_built_in_choice_takes_one_pass_for_large_bf16_batches():
    """bf16 P64 N128 with batch x heads >= 256 runs the one-pass path without any knob."""
    _say("built-in one-pass choice bf16 B8 H32")
    inp = I.make_fwd_inputs(8, 300, 32, 64, 128, 1, "bf16", seed=85, d_init="normal")
    assert ssd.fwd_state_path(_dims(inp), 256) == 2
    y, fin = _run(inp, 256)
    yr, fr = _oracle(inp)
    assert rel_err(to64(y), yr) <= TOL["bf16"]
    assert rel_err(to64(fin), fr) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_one_pass_graph_capture_replays_match_eager(dtype):
    """The one-pass forward captured into a HIP graph: every replay, with unrelated eager work
    and synchronisation in between, reproduces the eager outputs bit for bit."""
    _say(f"one-pass graph capture {dtype}")
    P, N = (64, 64) if dtype == "f32" else (64, 128)
    inp = {k: v.to(DEV) for k, v in I.make_fwd_inputs(2, 500, 4, P, N, 1, dtype, seed=87).items()}
    dims = ssd.make_dims(2, 500, 4, P, N, 1, inp["x"].dtype)
    ws = torch.empty(ssd.ssd_fwd_workspace_size(dims, 256), dtype=torch.uint8, device=DEV)
    y = torch.empty_like(inp["x"])
    st = torch.empty(2, 4, P, N, device=DEV)

    def run():
        ssd.ssd_fwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"], chunk_size=256,
                    y=y, final_state=st, workspace=ws)

    with _one_pass(64):
        run()
        torch.cuda.synchronize()
        ref = (y.clone(), st.clone())
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.graph(graph, stream=cap):
            run()
        torch.cuda.synchronize()
    other = {k: v.to(DEV) for k, v in I.make_fwd_inputs(2, 300, 4, P, N, 1, dtype, seed=88).items()}
    for rep in range(3):
        y.fill_(float("nan"))
        st.fill_(float("nan"))
        ssd.ssd_fwd(other["x"], other["dt"], other["dt_bias"], other["A"], other["B"], other["C"], other["D"],
                    chunk_size=64)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]) and torch.equal(st, ref[1]), rep
