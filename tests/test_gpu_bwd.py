"""GPU parity of the SSD backward (ssd_bwd) against the float64 backward oracle.

Every gradient (dx, ddt, ddt_bias, dA, dB, dC, dD, dz, dinitial_state) is compared element by
element: rel_err = max|gpu - oracle| / max|oracle| per tensor, <= 1e-4 for fp32 inputs and
<= 2e-2 for bf16 inputs (fp32 accumulation).  The upstream gradients are seeded N(0, 1).
"""
import sys

import numpy as np
import pytest
import torch

from helpers import TOL, rel_err, to64
from oracle.ssd_backward import ssd_recurrence_bwd
from state_space_sequence_mamba_amd import inputs as I
from state_space_sequence_mamba_amd import ssd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
LIMIT = (0.004, 0.04)
GRADS = ["dx", "ddt", "ddt_bias", "dA", "dB", "dC", "dD", "dz", "dinitial_state"]


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _upstream(Bt, L, H, P, N, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    dout = torch.randn(Bt, L, H, P, generator=g).to({"f32": torch.float32, "bf16": torch.bfloat16}[dtype])
    dfin = torch.randn(Bt, H, P, N, generator=g)
    return dout, dfin


def _run(inp, Q, dout, dfin=None, init=None, z=None, dt_limit=None, opts=None):
    d = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    out = ssd.ssd_bwd(d["x"], d["dt"], d["dt_bias"], d["A"], d["B"], d["C"], dout.to(DEV), D=d.get("D"),
                      chunk_size=Q, initial_state=None if init is None else init.to(DEV),
                      dfinal_state=None if dfin is None else dfin.to(DEV),
                      z=None if z is None else z.to(DEV), dt_limit=dt_limit, opts=opts)
    torch.cuda.synchronize()
    return {k: (None if v is None else to64(v)) for k, v in out.items()}


def _oracle(inp, dout, dfin=None, init=None, z=None, dt_limit=None):
    return ssd_recurrence_bwd(to64(inp["x"]), to64(inp["dt"]), to64(inp["dt_bias"]), to64(inp["A"]),
                              to64(inp["B"]), to64(inp["C"]), to64(dout),
                              None if inp.get("D") is None else to64(inp["D"]),
                              initial_state=None if init is None else to64(init),
                              z=None if z is None else to64(z), dt_limit=dt_limit,
                              dfinal=None if dfin is None else to64(dfin))


def _compare(got, ref, tol, skip=()):
    for k in GRADS:
        if k in skip or ref.get(k) is None:
            continue
        assert got[k] is not None, k
        assert np.all(np.isfinite(got[k])), f"{k} not finite"
        e = rel_err(got[k], ref[k])
        assert e <= tol, f"{k} rel_err {e:.3e} > {tol}"


CASES = []
for dtype, shapes in (("f32", [(16, 16, 1), (32, 32, 2), (64, 64, 1), (16, 64, 4), (64, 16, 2)]),
                      ("bf16", [(64, 128, 1), (32, 64, 2), (16, 32, 4)])):
    for i, (P, N, G) in enumerate(shapes):
        for L in (1, 63, 130, 300):
            CASES.append((dtype, P, N, G, L, (64, 128, 256)[(i + L) % 3]))


@pytest.mark.parametrize("dtype,P,N,G,L,Q", CASES)
def test_bwd_matches_oracle(dtype, P, N, G, L, Q):
    _say(f"bwd dtype={dtype} P={P} N={N} G={G} L={L} Q={Q}")
    H = 4
    inp = I.make_fwd_inputs(2, L, H, P, N, G, dtype, seed=200 + L + P + N, d_init="normal")
    dout, dfin = _upstream(2, L, H, P, N, dtype, seed=201 + L)
    got = _run(inp, Q, dout, dfin)
    _compare(got, _oracle(inp, dout, dfin), TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("gate,clamp,init", [(True, False, False), (False, True, True), (True, True, True)])
def test_bwd_gate_clamp_initial_state(dtype, gate, clamp, init):
    _say(f"bwd {dtype} gate={gate} clamp={clamp} init={init}")
    Bt, L, H, P, G = 2, 333, 6, 32, 3
    N = 32 if dtype == "f32" else 64
    inp = I.make_fwd_inputs(Bt, L, H, P, N, G, dtype, seed=210, d_init="normal")
    dout, dfin = _upstream(Bt, L, H, P, N, dtype, seed=211)
    z = I.make_gate((Bt, L, H, P), dtype, seed=212) if gate else None
    h0 = torch.randn(Bt, H, P, N, generator=torch.Generator().manual_seed(213)) if init else None
    lim = LIMIT if clamp else None
    got = _run(inp, 128, dout, dfin, init=h0, z=z, dt_limit=lim)
    _compare(got, _oracle(inp, dout, dfin, init=h0, z=z, dt_limit=lim), TOL[dtype])


@pytest.mark.parametrize("L,Q,init", [(300, 128, False), (517, 256, True)])
def test_bwd_bf16_head_slices_on_chip(L, Q, init):
    """bf16 with slices of four heads per bwd_dxdb / bwd_dc workgroup (dB and dC summed over the
    slice in registers before they leave the chip) and with one head per workgroup: both against
    the oracle, and dB, dC of the two agree to the rounding of their bf16 outputs."""
    Bt, H, P, N, G = 2, 8, 64, 128, 2
    _say(f"bwd bf16 head slices L={L} Q={Q} init={init}")
    inp = I.make_fwd_inputs(Bt, L, H, P, N, G, "bf16", seed=260 + L, d_init="normal")
    dout, dfin = _upstream(Bt, L, H, P, N, "bf16", seed=261 + L)
    h0 = torch.randn(Bt, H, P, N, generator=torch.Generator().manual_seed(262)) if init else None
    dims = ssd.make_dims(Bt, L, H, P, N, G, torch.bfloat16)
    assert ssd.bwd_heads(dims, Q, {"bwd_heads": 4}) == 4 and ssd.bwd_heads(dims, Q, {"bwd_heads": 1}) == 1
    ref = _oracle(inp, dout, dfin, init=h0)
    four = _run(inp, Q, dout, dfin, init=h0, opts={"bwd_heads": 4})
    one = _run(inp, Q, dout, dfin, init=h0, opts={"bwd_heads": 1})
    _compare(four, ref, TOL["bf16"])
    _compare(one, ref, TOL["bf16"])
    for k in ("dB", "dC"):
        assert rel_err(four[k], one[k]) <= 1e-2, k


def test_bwd_gate_with_shared_cb_blocks():
    """bf16 with 20 heads per group and a gate: the backward's forward recompute forms C B^T
    once per group for the pre-gate output."""
    _say("bwd bf16 gate H=20 G=1")
    Bt, L, H, P, N, G = 1, 200, 20, 32, 64, 1
    inp = I.make_fwd_inputs(Bt, L, H, P, N, G, "bf16", seed=220, d_init="normal")
    dout, dfin = _upstream(Bt, L, H, P, N, "bf16", seed=221)
    z = I.make_gate((Bt, L, H, P), "bf16", seed=222)
    got = _run(inp, 64, dout, dfin, z=z)
    _compare(got, _oracle(inp, dout, dfin, z=z), TOL["bf16"])


def test_bwd_no_D_no_upstream_state():
    _say("bwd D=None dfinal=None")
    inp = I.make_fwd_inputs(2, 200, 4, 32, 32, 1, "f32", seed=220)
    inp["D"] = None
    dout, _ = _upstream(2, 200, 4, 32, 32, "f32", seed=221)
    got = _run(inp, 64, dout)
    ref = _oracle(inp, dout)
    _compare(got, ref, TOL["f32"], skip=("dD",))
    # dD is still the gradient with respect to a (zero) skip weight: sum over tokens of dy * x
    dD = (to64(dout) * to64(inp["x"])).sum(axis=(0, 1))
    assert rel_err(got["dD"], dD) <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_chunk_size_invariance_and_determinism(dtype):
    _say(f"bwd chunk invariance {dtype}")
    N = 64 if dtype == "f32" else 128
    inp = I.make_fwd_inputs(2, 700, 6, 64, N, 3, dtype, seed=230)
    dout, dfin = _upstream(2, 700, 6, 64, N, dtype, seed=231)
    ref = _oracle(inp, dout, dfin)
    for Q in (64, 128, 256):
        got = _run(inp, Q, dout, dfin)
        _compare(got, ref, TOL[dtype])
        if Q == 256:
            again = _run(inp, Q, dout, dfin)
            for k in GRADS:
                if got[k] is not None:
                    assert np.array_equal(got[k], again[k]), k


def test_bwd_seqlen_zero():
    _say("bwd seqlen 0")
    x = torch.empty(2, 0, 4, 16, device=DEV)
    dt = torch.empty(2, 0, 4, device=DEV)
    Bm = torch.empty(2, 0, 1, 16, device=DEV)
    dfin = torch.randn(2, 4, 16, 16, device=DEV)
    out = ssd.ssd_bwd(x, dt, torch.zeros(4, device=DEV), -torch.ones(4, device=DEV), Bm, Bm.clone(),
                      torch.empty_like(x), D=torch.ones(4, 16, device=DEV), chunk_size=64, dfinal_state=dfin)
    torch.cuda.synchronize()
    assert torch.equal(out["dinitial_state"], dfin)
    assert torch.count_nonzero(out["dA"]) == 0 and torch.count_nonzero(out["ddt_bias"]) == 0
    assert torch.count_nonzero(out["dD"]) == 0


def test_bwd_full_size_f32_workload():
    """The fp32 B4 L1024 H24 P64 N64 G1 Q256 forward's backward, every gradient in full."""
    w = I.WORKLOAD_LIST[1]
    _say(f"bwd {w.name}")
    inp = I.make_workload_inputs(w)
    dout, dfin = _upstream(w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, "f32", seed=240)
    got = _run(inp, w.chunk, dout, dfin)
    _compare(got, _oracle(inp, dout, dfin), TOL["f32"])


def test_bwd_full_length_bf16_one_row():
    """One batch row, 8 heads, at the B8 L4096 H32 P64 N128 bf16 workload's sequence length and
    head sizes (the float64 oracle keeps every state: 4097 x 8 x 64 x 128 values), every
    gradient in full."""
    w = I.WORKLOAD_LIST[2]
    _say(f"bwd {w.name} (batch row 0, heads 0-7)")
    inp = I.make_workload_inputs(w)
    H = 8
    inp = {k: (v[:1, :, :H].contiguous() if k in ("x", "dt") else
               v[:1].contiguous() if k in ("B", "C") else v[:H].contiguous()) for k, v in inp.items()}
    dout, dfin = _upstream(1, w.seqlen, H, w.headdim, w.dstate, "bf16", seed=241)
    got = _run(inp, w.chunk, dout, dfin)
    _compare(got, _oracle(inp, dout, dfin), TOL["bf16"])


def test_bwd_batch_zero_writes_zero_head_gradients():
    """No sequences: ddt_bias, dA and dD are still outputs of the call and come back zero."""
    _say("bwd batch 0")
    H, P, N = 4, 16, 16
    x = torch.empty(0, 10, H, P, device=DEV)
    dt = torch.empty(0, 10, H, device=DEV)
    Bm = torch.empty(0, 10, 1, N, device=DEV)
    out = {"dx": torch.empty_like(x), "ddt": torch.empty_like(dt), "dB": torch.empty_like(Bm),
           "dC": torch.empty_like(Bm), "ddt_bias": torch.full((H,), float("nan"), device=DEV),
           "dA": torch.full((H,), float("nan"), device=DEV), "dD": torch.full((H, P), float("nan"), device=DEV),
           "dz": None, "dinitial_state": torch.empty(0, H, P, N, device=DEV)}
    ssd.ssd_bwd(x, dt, torch.zeros(H, device=DEV), -torch.ones(H, device=DEV), Bm, Bm.clone(), torch.empty_like(x),
                D=torch.ones(H, P, device=DEV), chunk_size=64, out=out)
    torch.cuda.synchronize()
    for k in ("ddt_bias", "dA", "dD"):
        assert torch.count_nonzero(out[k]) == 0 and not torch.isnan(out[k]).any(), k


def test_bwd_bf16_workload_launch_sparse_upstream():
    """The backward at the bf16 B8 L4096 H32 P64 N128 workload's own sizes and launch shape, with
    the upstream gradients nonzero only on batch rows R and heads S.  The gradients are linear in
    the upstream ones, so every output equals the oracle's on the (R, S) slice (dB, dC summed over
    the heads of S, dA, d dt_bias, dD over the rows of R), and is exactly zero outside it."""
    w = I.WORKLOAD_LIST[2]
    R, S = [0, 7], [0, 31]
    _say(f"bwd {w.name} (upstream gradients on rows {R}, heads {S})")
    inp = I.make_workload_inputs(w)
    Bt, L, H, P, N = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate
    d_s, f_s = _upstream(len(R), L, len(S), P, N, "bf16", seed=242)
    dout = torch.zeros(Bt, L, H, P, dtype=torch.bfloat16)
    dfin = torch.zeros(Bt, H, P, N)
    for i, b in enumerate(R):
        for j, h in enumerate(S):
            dout[b, :, h] = d_s[i, :, j]
            dfin[b, h] = f_s[i, j]
    got = _run(inp, w.chunk, dout, dfin)
    sub = {k: (v[R][:, :, S].contiguous() if k in ("x", "dt") else v[R].contiguous() if k in ("B", "C")
               else v[S].contiguous()) for k, v in inp.items()}
    ref = _oracle(sub, d_s, f_s)
    tol = TOL["bf16"]
    rows, heads = np.array(R), np.array(S)
    for k in ("dx", "ddt"):
        e = rel_err(got[k][rows][:, :, heads], ref[k])
        assert e <= tol, f"{k} rel_err {e:.3e}"
        mask = np.ones(got[k].shape[:3], dtype=bool)
        mask[np.ix_(rows, np.arange(L), heads)] = False
        assert np.count_nonzero(got[k][mask]) == 0, f"{k} nonzero outside the upstream slice"
    for k in ("dB", "dC"):
        e = rel_err(got[k][rows], ref[k])
        assert e <= tol, f"{k} rel_err {e:.3e}"
        others = np.setdiff1d(np.arange(Bt), rows)
        assert np.count_nonzero(got[k][others]) == 0, f"{k} nonzero outside rows {R}"
    for k in ("dA", "ddt_bias", "dD"):
        e = rel_err(got[k][heads], ref[k])
        assert e <= tol, f"{k} rel_err {e:.3e}"
        assert np.count_nonzero(got[k][np.setdiff1d(np.arange(H), heads)]) == 0, k
    e = rel_err(got["dinitial_state"][rows][:, heads], ref["dinitial_state"])
    assert e <= tol, f"dinitial_state rel_err {e:.3e}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_graph_replay_and_timed_entry_match_eager(dtype):
    """ssd_bwd captured into a HIP graph gives the eager result on every replay; the timed entry
    point gives the same result and refuses a capturing stream."""
    from state_space_sequence_mamba_amd.timing import HipEvents
    _say(f"bwd graph + timed {dtype}")
    N = 64 if dtype == "f32" else 128
    inp = {k: v.to(DEV) for k, v in I.make_fwd_inputs(2, 500, 8, 64, N, 2, dtype, seed=250).items()}
    dout, dfin = (t.to(DEV) for t in _upstream(2, 500, 8, 64, N, dtype, seed=251))
    args = (inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], dout)
    ref = ssd.ssd_bwd(*args, D=inp["D"], chunk_size=128, dfinal_state=dfin)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in ref.items() if v is not None}
    out = ssd.ssd_bwd(*args, D=inp["D"], chunk_size=128, dfinal_state=dfin)
    dims = ssd.make_dims(2, 500, 8, 64, N, 2, inp["x"].dtype)
    ws = torch.empty(ssd.ssd_bwd_workspace_size(dims, 128), dtype=torch.uint8, device=DEV)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        ssd.ssd_bwd(*args, D=inp["D"], chunk_size=128, dfinal_state=dfin, workspace=ws, out=out)
    for rep in range(3):
        for v in out.values():
            if v is not None:
                v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in ref.items():
            assert torch.equal(out[k], v), (rep, k)
    hev = HipEvents()
    evs = [hev.create() for _ in range(20)]
    timed = ssd.ssd_bwd(*args, D=inp["D"], chunk_size=128, dfinal_state=dfin, stage_events=evs)
    torch.cuda.synchronize()
    for k, v in ref.items():
        assert torch.equal(timed[k], v), k
    assert all(hev.elapsed_ms(evs[2 * k], evs[2 * k + 1]) >= 0.0 for k in range(10))
    assert all(hev.elapsed_ms(evs[2 * k], evs[2 * k + 1]) > 0.0 for k in (0, 1, 4, 5, 6, 7, 8, 9))
    g2 = torch.cuda.CUDAGraph()
    with pytest.raises(ssd.SsdError) as ei:
        with torch.cuda.graph(g2, stream=cap):
            ssd.ssd_bwd(*args, D=inp["D"], chunk_size=128, dfinal_state=dfin, workspace=ws, out=out,
                        stage_events=evs)
    assert ei.value.status == ssd.SSD_ERR_UNSUPPORTED
    hev.close()
