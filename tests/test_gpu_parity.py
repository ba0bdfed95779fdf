"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Bar: rel_err = max|gpu - oracle| / max|oracle| per output tensor (y, final_state)
<= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs (fp32 accumulation).
Small shapes are compared element by element in full; the full-size workloads are
compared on sampled (batch, head) slices that the oracle evaluates on their own.
"""
import sys

import numpy as np
import pytest
import torch

from helpers import TOL, oracle_slices, oracle_step_slices, p999_rel_err, rel_err, to64
from oracle import ssd_recurrence, ssd_step_ref
from oracle import ssd_stages
from state_space_sequence_mamba_amd import inputs as I
from state_space_sequence_mamba_amd import ssd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"\n[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def _fwd_gpu(inp, chunk, initial_state=None, opts=None):
    dev = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    init = None if initial_state is None else initial_state.to(DEV)
    y, fin = ssd.ssd_fwd(dev["x"], dev["dt"], dev["dt_bias"], dev["A"], dev["B"], dev["C"], dev.get("D"),
                         chunk_size=chunk, initial_state=init, opts=opts)
    torch.cuda.synchronize()
    return y, fin


def _check_full(inp, chunk, tol, initial_state=None):
    y, fin = _fwd_gpu(inp, chunk, initial_state)
    yr, fr = ssd_recurrence(to64(inp["x"]), to64(inp["dt"]), to64(inp["dt_bias"]), to64(inp["A"]),
                            to64(inp["B"]), to64(inp["C"]), None if inp.get("D") is None else to64(inp["D"]),
                            initial_state=None if initial_state is None else to64(initial_state))
    ey, ef = rel_err(to64(y), yr), rel_err(to64(fin), fr)
    assert np.all(np.isfinite(to64(y))) and np.all(np.isfinite(to64(fin)))
    assert ey <= tol, f"y rel_err {ey:.3e} > {tol}"
    assert ef <= tol, f"final_state rel_err {ef:.3e} > {tol}"
    return ey, ef


# ------------------------------------------------------------------ the five workloads

def test_workload_fwd_f32_small():
    w = I.WORKLOAD_LIST[0]
    _say(w.name)
    inp = I.make_workload_inputs(w)
    _check_full(inp, w.chunk, TOL[w.dtype])


def test_workload_fwd_f32_b4_l1024():
    w = I.WORKLOAD_LIST[1]
    _say(w.name)
    inp = I.make_workload_inputs(w)
    _check_full(inp, w.chunk, TOL[w.dtype])


def _sampled_pairs(Bt, H, G):
    """At least one head of every group in every batch row (heads varied across rows), plus the
    first and last (b, h)."""
    hpg = H // G
    pairs = {(b, g * hpg + (3 * b + 7 * g + 1) % hpg) for b in range(Bt) for g in range(G)}
    pairs |= {(0, 0), (Bt - 1, H - 1)}
    return sorted(pairs)


def _check_sampled(inp, y, fin, pairs, tol, what):
    yc, fc = to64(y), to64(fin)
    assert np.all(np.isfinite(yc)) and np.all(np.isfinite(fc))
    ref = oracle_slices(inp, pairs)
    worst = 0.0
    for (b, h), (yr, fr) in ref.items():
        ey, ef = rel_err(yc[b, :, h], yr), rel_err(fc[b, h], fr)
        worst = max(worst, ey, ef)
        assert ey <= tol, f"{what} (b={b}, h={h}) y rel_err {ey:.3e}"
        assert ef <= tol, f"{what} (b={b}, h={h}) final rel_err {ef:.3e}"
    b0, h0 = pairs[0]
    print(f"[parity] {what}: {len(pairs)} slices, worst rel_err {worst:.3e}, "
          f"p99.9 rel (b={b0}, h={h0}) {p999_rel_err(yc[b0, :, h0], ref[(b0, h0)][0]):.3e}", flush=True)


@pytest.mark.parametrize("widx", [2, 4])
def test_workload_fwd_bf16_full_size_sampled(widx):
    """The bf16 B8 L4096 H32 and B2 L16384 H80 G8 workloads at full size: one head of every
    group in every batch row against the oracle."""
    w = I.WORKLOAD_LIST[widx]
    _say(w.name)
    inp = I.make_workload_inputs(w)
    y, fin = _fwd_gpu(inp, w.chunk)
    pairs = _sampled_pairs(w.batch, w.nheads, w.ngroups)
    assert len(pairs) >= w.batch * w.ngroups
    _check_sampled(inp, y, fin, pairs, TOL[w.dtype], w.name)


# weak decay: the carried state survives many chunks, so an error in how it is passed from
# far back is not damped below the bar (with A = 0 the scan reduces to a cumulative sum)
LONG_CHAIN = [
    # (batch, seqlen, heads, groups, A, options): the B2 L16384 H80 G8 launch (64 chunks in
    # segments of 8), the same with a ragged last chunk, and the B8 L4096 H32 launch (16 chunks
    # in segments of 4, and forced onto the one-pass path)
    (2, 16384, 80, 8, 0.0, None), (2, 16384, 80, 8, -1e-3, None), (2, 16307, 80, 8, -1e-3, None),
    (8, 4096, 32, 1, 0.0, None), (8, 4096, 32, 1, -1e-3, None),
    (8, 4096, 32, 1, 0.0, {"state_path": 2}), (8, 4096, 32, 1, -1e-3, {"state_path": 2}),
]


@pytest.mark.parametrize("Bt,L,H,G,Aval,opts", LONG_CHAIN)
def test_bf16_weak_decay_long_chain(Bt, L, H, G, Aval, opts):
    _say(f"weak decay bf16 B{Bt} L{L} H{H} G{G} A={Aval} opts={opts}")
    inp = I.make_fwd_inputs(Bt, L, H, 64, 128, G, "bf16", seed=70 + Bt + G, d_init="normal")
    inp["A"] = torch.full_like(inp["A"], Aval)
    dims = ssd.make_dims(Bt, L, H, 64, 128, G, torch.bfloat16)
    path = ssd.fwd_state_path(dims, 256, opts)
    assert path == (2 if opts else 3)                # one pass, or segments of chunks
    y, fin = _fwd_gpu(inp, 256, opts=opts)
    hpg = H // G
    pairs = sorted({(b, g * hpg + (5 * b + 3 * g) % hpg) for b in range(Bt) for g in range(G)
                    if (b + g) % 2 == 0 or Bt * G <= 8} | {(Bt - 1, H - 1)})
    _check_sampled(inp, y, fin, pairs, TOL["bf16"], f"weak decay A={Aval} L={L} path {path}")


def test_workload_step_bf16_1000_steps_sampled():
    w = I.WORKLOAD_LIST[3]
    _say(w.name)
    inp = I.make_step_inputs(w.batch, w.nheads, w.headdim, w.dstate, w.ngroups, w.steps, w.dtype, w.seed,
                             w.d_init, device=DEV)
    record = {0, 1, 9, 99, 499, 999}
    state = inp["state0"].clone()
    ys = {}
    for t in range(w.steps):
        y = ssd.ssd_step(state, inp["x"][t], inp["dt"][t], inp["dt_bias"], inp["A"], inp["B"][t], inp["C"][t],
                         inp["D"])
        if t in record:
            ys[t] = to64(y)
    torch.cuda.synchronize()
    stc = to64(state)
    # 16 (b, h) pairs, one in every 16-row slice of the batch (so every quarter four times)
    pairs = [(16 * k + (5 * k) % 16, (37 * k + 11) % w.nheads) for k in range(16)] + [(0, 0),
                                                                                      (w.batch - 1, w.nheads - 1)]
    ref = oracle_step_slices(inp, pairs, w.steps, record)
    for (b, h), (yr, sr) in ref.items():
        for t in record:
            e = rel_err(ys[t][b, h], yr[t])
            assert e <= TOL[w.dtype], f"(b={b}, h={h}, step {t + 1}) y rel_err {e:.3e}"
        e = rel_err(stc[b, h], sr)
        assert e <= TOL[w.dtype], f"(b={b}, h={h}) state rel_err {e:.3e}"


# ------------------------------------------------------------------ shape sweep

SWEEP = []
for dtype, shapes in (("f32", [(16, 16), (32, 32), (64, 64), (16, 64), (64, 16)]),
                      ("bf16", [(64, 128), (32, 64), (16, 32), (64, 32)])):
    for i, (P, N) in enumerate(shapes):
        for L in (1, 7, 63, 64, 65, 200, 513):
            SWEEP.append((dtype, P, N, L, (64, 128, 256)[(i + L) % 3], (1, 2, 4)[(i + L) % 3]))


@pytest.mark.parametrize("dtype,P,N,L,Q,G", SWEEP)
def test_shape_sweep(dtype, P, N, L, Q, G):
    _say(f"sweep dtype={dtype} P={P} N={N} L={L} Q={Q} G={G}")
    H = 4
    inp = I.make_fwd_inputs(2, L, H, P, N, G, dtype, seed=100 + L + P + N, d_init="normal")
    _check_full(inp, Q, TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_size_invariance(dtype):
    _say(f"chunk invariance {dtype}")
    inp = I.make_fwd_inputs(2, 700, 6, 64, 64, 3, dtype, seed=7)
    outs = []
    for Q in (64, 128, 256):
        outs.append(_check_full(inp, Q, TOL[dtype]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_run_to_run_bitwise_determinism(dtype):
    _say(f"determinism {dtype}")
    inp = I.make_fwd_inputs(2, 1000, 8, 64, 64, 2, dtype, seed=8)
    y1, f1 = _fwd_gpu(inp, 256)
    y2, f2 = _fwd_gpu(inp, 256)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


@pytest.mark.parametrize("L,Q,G", [(700, 256, 1), (300, 128, 1), (130, 64, 2), (64, 256, 1)])
def test_bf16_shared_cb_blocks_match_in_kernel_cb(L, Q, G):
    """bf16 with at least 20 heads per group: the row blocks read C B^T formed once per group by
    chunk_state; the whole-chunk decomposition forms it itself from the bf16 rows.  Same MFMA
    sequence, so the results agree bit for bit (ragged last chunks, every chunk size, with a
    gate), and both match the oracle."""
    _say(f"bf16 shared C B^T L={L} Q={Q} G={G}")
    H = 20 * G
    inp = I.make_fwd_inputs(2, L, H, 64, 128, G, "bf16", seed=31 + L, d_init="normal")
    z = I.make_gate(tuple(inp["x"].shape), "bf16", seed=32)
    dev = {k: (None if v is None else v.to(DEV)) for k, v in inp.items()}
    for gate in (None, z.to(DEV)):
        outs = []
        for variant in (1, 2):
            y, f = ssd.ssd_fwd(dev["x"], dev["dt"], dev["dt_bias"], dev["A"], dev["B"], dev["C"], dev["D"],
                               chunk_size=Q, z=gate, opts={"scan_variant": variant})
            torch.cuda.synchronize()
            outs.append((y, f))
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1]), gate is None
    _check_full(inp, Q, TOL["bf16"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_launch_shapes_do_not_change_results(dtype):
    """Both chunk_scan decompositions, every head-block size and every row-block dispatch
    grouping give bit-identical results."""
    _say(f"launch shape invariance {dtype}")
    inp = I.make_fwd_inputs(2, 700, 12, 64, 64, 1, dtype, seed=9)
    ref = None
    for variant in (1, 2):
        for hb in (1, 2):
            for group in ((1, 16, 1000) if variant == 1 else (0,)):
                # row-block dispatch groups change the order of work only
                y, f = _fwd_gpu(inp, 256, opts={"scan_variant": variant, "heads_per_block": hb,
                                                "rows_group": group})
                if ref is None:
                    ref = (y, f)
                else:
                    assert torch.equal(y, ref[0]) and torch.equal(f, ref[1]), (variant, hb, group)
    _check_full(inp, 256, TOL[dtype])


# ------------------------------------------------------------------ state in / out

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_initial_state(dtype):
    _say(f"initial_state {dtype}")
    inp = I.make_fwd_inputs(2, 300, 4, 64, 64 if dtype == "f32" else 128, 2, dtype, seed=10)
    init = torch.randn(2, 4, 64, inp["B"].shape[3], generator=torch.Generator().manual_seed(3))
    _check_full(inp, 128, TOL[dtype], initial_state=init)


def test_split_sequence_resume_and_decode_continuity():
    """fwd(x[:L1]) -> final_state -> fwd(x[L1:], init) -> final_state -> ssd_step == oracle on all tokens."""
    _say("resume + decode continuity")
    L, L1 = 400, 150
    inp = I.make_fwd_inputs(2, L + 3, 4, 32, 32, 1, "f32", seed=11)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    sl = lambda k, a, b: dev[k][:, a:b].contiguous()  # noqa: E731
    y1, f1 = ssd.ssd_fwd(sl("x", 0, L1), sl("dt", 0, L1), dev["dt_bias"], dev["A"], sl("B", 0, L1),
                         sl("C", 0, L1), dev["D"], chunk_size=64)
    y2, f2 = ssd.ssd_fwd(sl("x", L1, L), sl("dt", L1, L), dev["dt_bias"], dev["A"], sl("B", L1, L),
                         sl("C", L1, L), dev["D"], chunk_size=128, initial_state=f1)
    state = f2.clone()
    ys = []
    for t in range(L, L + 3):
        ys.append(ssd.ssd_step(state, dev["x"][:, t].contiguous(), dev["dt"][:, t].contiguous(), dev["dt_bias"],
                               dev["A"], dev["B"][:, t].contiguous(), dev["C"][:, t].contiguous(), dev["D"]))
    torch.cuda.synchronize()
    got = np.concatenate([to64(y1), to64(y2), np.stack([to64(v) for v in ys], axis=1)], axis=1)
    yr, fr = ssd_recurrence(*(to64(inp[k]) for k in ("x", "dt", "dt_bias", "A", "B", "C", "D")))
    assert rel_err(got, yr) <= TOL["f32"]
    assert rel_err(to64(state), fr) <= TOL["f32"]


def test_seqlen_zero_writes_initial_state():
    _say("seqlen 0")
    x = torch.empty(2, 0, 4, 16, device=DEV)
    dt = torch.empty(2, 0, 4, device=DEV)
    Bm = torch.empty(2, 0, 1, 16, device=DEV)
    init = torch.randn(2, 4, 16, 16, device=DEV)
    y, f = ssd.ssd_fwd(x, dt, torch.zeros(4, device=DEV), -torch.ones(4, device=DEV), Bm, Bm.clone(),
                       chunk_size=64, initial_state=init)
    y0, f0 = ssd.ssd_fwd(x, dt, torch.zeros(4, device=DEV), -torch.ones(4, device=DEV), Bm, Bm.clone(),
                         chunk_size=64)
    torch.cuda.synchronize()
    assert y.numel() == 0 and torch.equal(f, init) and torch.count_nonzero(f0) == 0


def test_batch_zero_is_noop():
    _say("batch 0")
    x = torch.empty(0, 10, 4, 16, device=DEV)
    y, f = ssd.ssd_fwd(x, torch.empty(0, 10, 4, device=DEV), torch.zeros(4, device=DEV),
                       -torch.ones(4, device=DEV), torch.empty(0, 10, 1, 16, device=DEV),
                       torch.empty(0, 10, 1, 16, device=DEV), chunk_size=64)
    assert y.numel() == 0 and f.numel() == 0


def test_special_values_A_zero_and_large_dt():
    _say("A = 0, large dt")
    inp = I.make_fwd_inputs(1, 200, 4, 32, 32, 1, "f32", seed=12)
    inp["A"] = torch.zeros(4)
    inp["dt"][:, 50:60] = 40.0          # softplus in its linear branch
    _check_full(inp, 64, TOL["f32"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_strong_decay_stays_finite(dtype):
    """A = -16 and dt' = 3 over 80 tokens: decays across one 16-token tile reach e^-768, far
    past fp32 range; every factor the kernels form must stay finite (outputs match the oracle)."""
    _say(f"strong decay {dtype}")
    N = 64 if dtype == "f32" else 128
    inp = I.make_fwd_inputs(2, 300, 4, 64, N, 1, dtype, seed=15)
    inp["A"] = torch.full((4,), -16.0)
    inp["dt"][:, 100:180] = 3.0
    for Q in (64, 256):
        _check_full(inp, Q, TOL[dtype])


def test_no_D_term():
    _say("D = NULL")
    inp = I.make_fwd_inputs(1, 130, 4, 32, 32, 1, "f32", seed=13)
    inp["D"] = None
    _check_full(inp, 64, TOL["f32"])


# ------------------------------------------------------------------ stages

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_stage_intermediates_match_staged_oracle(dtype):
    """Read the workspace after a call: dt', segment cumsum and the states entering each chunk."""
    _say(f"stages {dtype}")
    Bt, L, H, P, N, G, Q = 2, 200, 4, 32, 32 if dtype == "f32" else 64, 2, 64
    inp = I.make_fwd_inputs(Bt, L, H, P, N, G, dtype, seed=14)
    dev = {k: v.to(DEV) for k, v in inp.items()}
    dims = ssd.make_dims(Bt, L, H, P, N, G, dev["x"].dtype)
    ws = torch.zeros(ssd.ssd_fwd_workspace_size(dims, Q), dtype=torch.uint8, device=DEV)
    ssd.ssd_fwd(dev["x"], dev["dt"], dev["dt_bias"], dev["A"], dev["B"], dev["C"], dev["D"], chunk_size=Q,
                workspace=ws)
    torch.cuda.synchronize()
    nc = (L + Q - 1) // Q
    cum = Bt * H * nc * Q * 4
    cum_al = (cum + 255) // 256 * 256
    f = ws.view(torch.float32) if ws.numel() % 4 == 0 else None
    dtp = f[: cum // 4].view(Bt, H, nc, Q)
    dacs = f[cum_al // 4: cum_al // 4 + cum // 4].view(Bt, H, nc, Q)
    n_st = Bt * nc * H * P * N
    states = f[2 * cum_al // 4: 2 * cum_al // 4 + n_st].view(Bt, nc, H, P, N)
    r_dtp, r_dacs = ssd_stages.chunk_cumsum(to64(inp["dt"]), to64(inp["dt_bias"]), to64(inp["A"]), Q)
    S = ssd_stages.chunk_state(to64(inp["x"]), to64(inp["B"]), r_dtp, r_dacs)
    r_prev, _ = ssd_stages.state_passing(S, r_dacs)
    assert rel_err(to64(dtp), r_dtp) <= 1e-6
    assert rel_err(to64(dacs), r_dacs) <= 1e-5
    if dtype == "f32":
        # region [2]: the per-chunk states, overwritten in place by the states entering each chunk
        assert rel_err(to64(states), r_prev) <= TOL[dtype]
    else:
        # region [2] keeps each chunk's own contribution; region [4] (the last one) holds the
        # entering states rounded to bf16
        assert rel_err(to64(states), S) <= TOL[dtype]
        st_al = (n_st * 4 + 255) // 256 * 256
        off = 2 * cum_al + st_al
        prev16 = ws[off: off + n_st * 2].view(torch.bfloat16).view(Bt, nc, H, P, N)
        assert rel_err(to64(prev16), r_prev) <= TOL[dtype]


# ------------------------------------------------------------------ ABI error paths

def test_error_paths_leave_outputs_untouched():
    _say("error paths")
    inp = {k: v.to(DEV) for k, v in I.make_fwd_inputs(1, 64, 4, 16, 16, 1, "f32", seed=1).items()}
    y = torch.full_like(inp["x"], 7.0)
    f = torch.full((1, 4, 16, 16), 7.0, device=DEV)
    host_x = inp["x"].cpu()
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_fwd(host_x, inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"], chunk_size=64,
                    y=y, final_state=f)
    assert e.value.status == ssd.SSD_ERR_DEVICE_PTR
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_fwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"], chunk_size=32,
                    y=y, final_state=f)
    assert e.value.status == ssd.SSD_ERR_UNSUPPORTED
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_fwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"], chunk_size=64,
                    y=y, final_state=f, workspace=small)
    assert e.value.status == ssd.SSD_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(y == 7.0) and torch.all(f == 7.0)


def test_step_small_shapes_against_oracle():
    _say("step small shapes")
    for dtype, P, N, G in (("f32", 16, 16, 1), ("f32", 64, 64, 2), ("bf16", 64, 128, 4), ("bf16", 32, 32, 1)):
        inp = I.make_step_inputs(3, 4, P, N, G, 5, dtype, seed=P + N, device=DEV)
        st = inp["state0"].clone()
        ref_st = to64(inp["state0"])
        for t in range(5):
            y = ssd.ssd_step(st, inp["x"][t], inp["dt"][t], inp["dt_bias"], inp["A"], inp["B"][t], inp["C"][t],
                             inp["D"])
            yr, ref_st = ssd_step_ref(ref_st, to64(inp["x"][t]), to64(inp["dt"][t]), to64(inp["dt_bias"]),
                                      to64(inp["A"]), to64(inp["B"][t]), to64(inp["C"][t]), to64(inp["D"]))
            assert rel_err(to64(y), yr) <= TOL[dtype]
        torch.cuda.synchronize()
        assert rel_err(to64(st), ref_st) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_graph_capture_replays_match_eager(dtype):
    """ssd_fwd + ssd_step captured into a HIP graph: every replay, with unrelated eager work
    and synchronisation in between, reproduces the eager outputs bit for bit."""
    _say(f"graph capture {dtype}")
    N = 64 if dtype == "f32" else 128
    inp = {k: v.to(DEV) for k, v in I.make_fwd_inputs(2, 500, 8, 64, N, 2, dtype, seed=21).items()}
    dec = {k: v[0].contiguous() for k, v in I.make_step_inputs(2, 8, 64, N, 2, 1, dtype, seed=22,
                                                               device=DEV).items() if k in ("x", "dt", "B", "C")}
    dims = ssd.make_dims(2, 500, 8, 64, N, 2, inp["x"].dtype)
    ws = torch.empty(ssd.ssd_fwd_workspace_size(dims, 128), dtype=torch.uint8, device=DEV)
    y = torch.empty_like(inp["x"])
    st = torch.empty(2, 8, 64, N, device=DEV)
    y1 = torch.empty_like(dec["x"])

    def run(events=None):
        ssd.ssd_fwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"], chunk_size=128,
                    y=y, final_state=st, workspace=ws, stage_events=events)
        ssd.ssd_step(st, dec["x"], dec["dt"], inp["dt_bias"], inp["A"], dec["B"], dec["C"], inp["D"], y=y1)

    run()
    torch.cuda.synchronize()
    ref = (y.clone(), st.clone(), y1.clone())
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=cap):
        run()
    torch.cuda.synchronize()
    other = {k: v.to(DEV) for k, v in I.make_fwd_inputs(2, 300, 8, 64, N, 2, dtype, seed=23).items()}
    for rep in range(3):
        y.fill_(float("nan"))
        st.fill_(float("nan"))
        y1.fill_(float("nan"))
        ssd.ssd_fwd(other["x"], other["dt"], other["dt_bias"], other["A"], other["B"], other["C"], other["D"],
                    chunk_size=64)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref[0]) and torch.equal(st, ref[1]) and torch.equal(y1, ref[2]), rep


def test_stage_events_time_each_kernel_and_refuse_capture():
    """ssd_fwd_ex records a start and a stop event with each kernel's dispatch; on a
    capturing stream it refuses (nothing launched) instead of breaking the capture."""
    _say("stage events")
    from state_space_sequence_mamba_amd.timing import HipEvents
    hev = HipEvents()
    evs = [hev.create() for _ in range(6)]
    inp = {k: v.to(DEV) for k, v in I.make_fwd_inputs(2, 1000, 8, 64, 64, 1, "f32", seed=24).items()}
    y, _ = ssd.ssd_fwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"],
                       chunk_size=256, stage_events=evs)
    torch.cuda.synchronize()
    # each kernel's own start / stop pair, and the kernels in launch order
    assert all(hev.elapsed_ms(evs[2 * k], evs[2 * k + 1]) > 0 for k in range(3))
    assert all(hev.elapsed_ms(evs[2 * k + 1], evs[2 * k + 2]) >= 0 for k in range(2))
    y_ref, _ = ssd.ssd_fwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"],
                           chunk_size=256)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with pytest.raises(ssd.SsdError) as e:
        with torch.cuda.graph(graph, stream=cap):
            ssd.ssd_fwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"],
                        chunk_size=256, stage_events=evs)
    assert e.value.status == ssd.SSD_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    hev.close()
