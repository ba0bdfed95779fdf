"""Pins of the float64 oracle to facts that do not come from the oracle itself.

Each test pins part of the oracle against the mathematics: hand-worked closed
forms, a brute-force quadratic form, library routines in special cases
(np.cumsum when A = 0, scipy.signal.lfilter for a scalar channel), and
structural invariants (linearity, causality, NaN isolation, group broadcast,
resumption from a carried state, decode loop == forward).  A plausible slip
in the oracle (a dropped D term, a wrong sign of A, a missing dt bias, B and
C swapped, y read from the old state, a wrong head->group map, a dropped
ragged tail) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal

from oracle import ssd_quadratic, ssd_recurrence, ssd_step_ref, softplus
from oracle import ssd_stages
from state_space_sequence_mamba_amd.inputs import make_fwd_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _golden(name):
    with open(GOLDEN) as f:
        ex = json.load(f)[name]
    arr = {k: np.array(v, dtype=np.float64) for k, v in ex.items() if k != "dims"}
    return arr


def _np_inputs(**kw):
    t = make_fwd_inputs(**kw)
    return {k: v.double().numpy() for k, v in t.items()}


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# --------------------------------------------------------------------------- softplus

def test_softplus_values():
    # log(1 + e^v) from math.log1p / math.exp, a library routine independent of logaddexp
    for v in [-30.0, -5.0, -1.0, 0.0, 0.5, 3.0, 20.0]:
        assert softplus(np.float64(v)) == pytest.approx(math.log1p(math.exp(v)), rel=1e-15)
    assert softplus(np.float64(0.0)) == pytest.approx(math.log(2.0), rel=1e-16)
    assert softplus(np.float64(800.0)) == pytest.approx(800.0, rel=1e-15)  # no overflow


# --------------------------------------------------------------------------- hand examples

def test_hand_example_one_head_two_steps():
    e = _golden("one_head_two_steps")
    ln2 = math.log(2.0)
    # dt' = softplus(0 + 0) = ln 2;  a = exp(-ln 2) = 1/2
    h0 = ln2                       # 0 * 1/2 + ln2 * 1 * 1
    y0 = h0 * 1.0 + 1.0 * 1.0      # C h0 + D x0
    h1 = 0.5 * h0 + ln2 * 2.0      # = 2.5 ln 2
    y1 = h1 * 1.0 + 1.0 * 2.0
    y, fin = ssd_recurrence(e["x"], e["dt"], e["dt_bias"], e["A"], e["B"], e["C"], e["D"])
    assert y[0, :, 0, 0] == pytest.approx([y0, y1], rel=1e-15)
    assert fin[0, 0, 0, 0] == pytest.approx(h1, rel=1e-15)
    assert h1 == pytest.approx(2.5 * ln2, rel=1e-15)
    yq = ssd_quadratic(e["x"], e["dt"], e["dt_bias"], e["A"], e["B"], e["C"], e["D"])
    assert yq[0, :, 0, 0] == pytest.approx([y0, y1], rel=1e-15)
    # two decode steps from a zero state give the same numbers
    st = np.zeros((1, 1, 1, 1))
    ys = []
    for t in range(2):
        yt, st = ssd_step_ref(st, e["x"][:, t], e["dt"][:, t], e["dt_bias"], e["A"],
                              e["B"][:, t], e["C"][:, t], e["D"])
        ys.append(yt[0, 0, 0])
    assert ys == pytest.approx([y0, y1], rel=1e-15)
    assert st[0, 0, 0, 0] == pytest.approx(h1, rel=1e-15)


def test_hand_example_two_channels_two_states():
    """Nonzero bias, B != C, two channels with different D: catches swaps and dropped terms."""
    e = _golden("two_channels_two_states")
    ln2 = math.log(2.0)
    d1 = math.log1p(math.exp(2.0))       # softplus(1 + 1)
    a1 = math.exp(-d1)                   # = 1 / (1 + e^2)
    # h0 = ln2 * x0 (outer) B0 = ln2 * [[1, 0], [-1, 0]]
    h0 = np.array([[ln2, 0.0], [-ln2, 0.0]])
    y0 = np.array([ln2 + 0.5 * 1.0, -ln2 + 2.0 * -1.0])
    # h1 = a1 h0 + d1 * x1 (outer) B1 = [[a1 ln2, 2 d1], [-a1 ln2, 0.5 d1]]
    h1 = np.array([[a1 * ln2, 2.0 * d1], [-a1 * ln2, 0.5 * d1]])
    y1 = np.array([3 * a1 * ln2 + 4 * 2 * d1 + 0.5 * 2.0, -3 * a1 * ln2 + 4 * 0.5 * d1 + 2.0 * 0.5])
    assert np.allclose(h0 @ np.array([1.0, 2.0]) + e["D"][0] * e["x"][0, 0, 0], y0, rtol=1e-15)
    y, fin = ssd_recurrence(e["x"], e["dt"], e["dt_bias"], e["A"], e["B"], e["C"], e["D"])
    np.testing.assert_allclose(y[0, 0, 0], y0, rtol=1e-14)
    np.testing.assert_allclose(y[0, 1, 0], y1, rtol=1e-14)
    np.testing.assert_allclose(fin[0, 0], h1, rtol=1e-14)
    yq = ssd_quadratic(e["x"], e["dt"], e["dt_bias"], e["A"], e["B"], e["C"], e["D"])
    np.testing.assert_allclose(yq[0, :, 0], np.stack([y0, y1]), rtol=1e-14)
    for Q in (1, 2, 4):
        ys, fs, _ = ssd_stages.ssd_chunked(e["x"], e["dt"], e["dt_bias"], e["A"], e["B"], e["C"],
                                           e["D"], chunk_size=Q)
        np.testing.assert_allclose(ys[0, :, 0], np.stack([y0, y1]), rtol=1e-14)
        np.testing.assert_allclose(fs[0, 0], h1, rtol=1e-14)


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("shape", [
    dict(batch=1, seqlen=1, nheads=1, headdim=1, dstate=1, ngroups=1),
    dict(batch=2, seqlen=9, nheads=2, headdim=3, dstate=4, ngroups=1),
    dict(batch=1, seqlen=17, nheads=4, headdim=2, dstate=3, ngroups=2),
    dict(batch=1, seqlen=33, nheads=3, headdim=2, dstate=5, ngroups=3),
])
def test_quadratic_form_equals_recurrence(shape):
    inp = _np_inputs(seed=11, **shape)
    y, _ = ssd_recurrence(**inp)
    yq = ssd_quadratic(**inp)
    assert _rel(y, yq) < 1e-12


def test_N1_quadratic_is_semiseparable_form():
    """For N = 1 the quadratic form is diag(p) M diag(q) X with p = C, q = dt' B and
    M[t, s] = prod_{k=s+1..t} a_k (the 1-semiseparable causal mask): built here from
    a cumulative product, not from sums of exponents."""
    inp = _np_inputs(seed=5, batch=1, seqlen=12, nheads=1, headdim=3, dstate=1, ngroups=1)
    d = np.log1p(np.exp(inp["dt"][0, :, 0] + inp["dt_bias"][0]))
    a = np.exp(d * inp["A"][0])
    L = d.shape[0]
    M = np.zeros((L, L))
    for s in range(L):
        M[s, s] = 1.0
        for t in range(s + 1, L):
            M[t, s] = M[t - 1, s] * a[t]
    p = inp["C"][0, :, 0, 0]
    q = d * inp["B"][0, :, 0, 0]
    Y = np.diag(p) @ M @ np.diag(q) @ inp["x"][0, :, 0, :] + inp["D"][0] * inp["x"][0, :, 0, :]
    y, _ = ssd_recurrence(**inp)
    assert _rel(y[0, :, 0, :], Y) < 1e-12


# --------------------------------------------------------------------------- special cases

def test_A_zero_is_cumulative_sum():
    inp = _np_inputs(seed=3, batch=1, seqlen=40, nheads=2, headdim=3, dstate=4, ngroups=1)
    inp["A"] = np.zeros_like(inp["A"])
    y, fin = ssd_recurrence(**inp)
    for h in range(2):
        d = np.log1p(np.exp(inp["dt"][0, :, h] + inp["dt_bias"][h]))
        outer = d[:, None, None] * inp["x"][0, :, h, :, None] * inp["B"][0, :, 0, None, :]
        Hc = np.cumsum(outer, axis=0)                                   # (L, P, N)
        yy = np.einsum("tpn,tn->tp", Hc, inp["C"][0, :, 0, :]) + inp["D"][h] * inp["x"][0, :, h, :]
        assert _rel(y[0, :, h, :], yy) < 1e-12
        assert _rel(fin[0, h], Hc[-1]) < 1e-12


def test_scalar_channel_is_first_order_iir_filter():
    L = 64
    rng = np.random.default_rng(7)
    xs = rng.standard_normal(L)
    dt_raw = 0.3
    for A in (-0.5, -3.0, -12.0):
        d = math.log1p(math.exp(dt_raw))
        a = math.exp(d * A)
        ref = scipy.signal.lfilter([d], [1.0, -a], xs)
        y, _ = ssd_recurrence(xs.reshape(1, L, 1, 1), np.full((1, L, 1), dt_raw), np.zeros(1),
                              np.array([A]), np.ones((1, L, 1, 1)), np.ones((1, L, 1, 1)), None)
        assert _rel(y[0, :, 0, 0], ref) < 1e-12


def test_memoryless_limit():
    inp = _np_inputs(seed=9, batch=1, seqlen=20, nheads=2, headdim=3, dstate=4, ngroups=1)
    inp["A"] = np.full(2, -1e4)
    inp["dt"] = np.abs(inp["dt"]) + 2.0          # dt' > 2, so exp(dt' A) == 0 exactly
    y, _ = ssd_recurrence(**inp)
    for h in range(2):
        d = np.log1p(np.exp(inp["dt"][0, :, h] + inp["dt_bias"][h]))
        cb = np.sum(inp["C"][0, :, 0, :] * inp["B"][0, :, 0, :], axis=-1)
        yy = (d * cb)[:, None] * inp["x"][0, :, h, :] + inp["D"][h] * inp["x"][0, :, h, :]
        assert _rel(y[0, :, h, :], yy) < 1e-13


def test_constant_step_zero_input_decays_initial_state():
    H, P, N, L = 2, 3, 4, 6
    rng = np.random.default_rng(2)
    init = rng.standard_normal((1, H, P, N))
    C = rng.standard_normal((1, L, 1, N))
    A = np.array([-0.7, -2.0])
    y, fin = ssd_recurrence(np.zeros((1, L, H, P)), np.zeros((1, L, H)), np.zeros(H), A,
                            np.zeros((1, L, 1, N)), C, None, initial_state=init)
    ln2 = math.log(2.0)
    for h in range(H):
        a = math.exp(ln2 * A[h])
        for t in range(L):
            np.testing.assert_allclose(y[0, t, h], a ** (t + 1) * init[0, h] @ C[0, t, 0], rtol=1e-13)
        np.testing.assert_allclose(fin[0, h], a ** L * init[0, h], rtol=1e-13)


# --------------------------------------------------------------------------- invariants

def test_linearity_in_x():
    inp = _np_inputs(seed=4, batch=2, seqlen=30, nheads=2, headdim=3, dstate=5, ngroups=1)
    x2 = np.random.default_rng(1).standard_normal(inp["x"].shape)
    y1, f1 = ssd_recurrence(**inp)
    y2, f2 = ssd_recurrence(**{**inp, "x": x2})
    y3, f3 = ssd_recurrence(**{**inp, "x": 2.5 * inp["x"] - 0.75 * x2})
    assert _rel(y3, 2.5 * y1 - 0.75 * y2) < 1e-12
    assert _rel(f3, 2.5 * f1 - 0.75 * f2) < 1e-12


def test_causality_impulse_and_perturbation():
    # the pages' own causal test shape: a unit impulse at t = 5 leaves t < 5 exactly zero
    inp = _np_inputs(seed=6, batch=1, seqlen=10, nheads=2, headdim=4, dstate=3, ngroups=1)
    imp = np.zeros_like(inp["x"])
    imp[:, 5] = 1.0
    y, _ = ssd_recurrence(**{**inp, "x": imp})
    assert np.all(y[:, :5] == 0.0)
    assert np.all(np.abs(y[:, 5]) > 0.0)
    # perturbing x at t0 leaves every earlier output bit-identical
    y0, _ = ssd_recurrence(**inp)
    xp = inp["x"].copy()
    xp[:, 7] += 3.0
    y1, _ = ssd_recurrence(**{**inp, "x": xp})
    assert np.array_equal(y0[:, :7], y1[:, :7])
    assert not np.array_equal(y0[:, 7], y1[:, 7])


def test_nan_isolation():
    inp = _np_inputs(seed=8, batch=2, seqlen=12, nheads=3, headdim=4, dstate=3, ngroups=1)
    x = inp["x"].copy()
    x[1, 4, 2, 3] = np.nan
    y, fin = ssd_recurrence(**{**inp, "x": x})
    bad = np.isnan(y)
    expect = np.zeros_like(bad)
    expect[1, 4:, 2, 3] = True
    assert np.array_equal(bad, expect)
    fbad = np.isnan(fin)
    fexp = np.zeros_like(fbad)
    fexp[1, 2, 3, :] = True
    assert np.array_equal(fbad, fexp)


def test_group_broadcast_equals_repeated_groups():
    inp = _np_inputs(seed=12, batch=1, seqlen=15, nheads=6, headdim=2, dstate=3, ngroups=2)
    y, fin = ssd_recurrence(**inp)
    rep = {**inp,
           "B": np.repeat(inp["B"], 3, axis=2),      # heads 0-2 -> group 0, heads 3-5 -> group 1
           "C": np.repeat(inp["C"], 3, axis=2)}
    y2, fin2 = ssd_recurrence(**rep)
    assert np.array_equal(y, y2) and np.array_equal(fin, fin2)


def test_batch_and_head_independence():
    inp = _np_inputs(seed=13, batch=3, seqlen=11, nheads=4, headdim=2, dstate=3, ngroups=2)
    y, fin = ssd_recurrence(**inp)
    b, h = 2, 3
    g = h // 2
    ys, fs = ssd_recurrence(inp["x"][b:b + 1, :, h:h + 1], inp["dt"][b:b + 1, :, h:h + 1],
                            inp["dt_bias"][h:h + 1], inp["A"][h:h + 1],
                            inp["B"][b:b + 1, :, g:g + 1], inp["C"][b:b + 1, :, g:g + 1],
                            inp["D"][h:h + 1])
    assert np.array_equal(ys[0, :, 0], y[b, :, h]) and np.array_equal(fs[0, 0], fin[b, h])


def test_split_sequence_resume():
    inp = _np_inputs(seed=14, batch=2, seqlen=25, nheads=2, headdim=3, dstate=4, ngroups=1)
    y, fin = ssd_recurrence(**inp)
    L1 = 9
    first = {k: (v[:, :L1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    rest = {k: (v[:, L1:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    ya, fa = ssd_recurrence(**first)
    yb, fb = ssd_recurrence(**rest, initial_state=fa)
    assert _rel(np.concatenate([ya, yb], axis=1), y) < 1e-13
    assert _rel(fb, fin) < 1e-13


def test_decode_loop_equals_forward():
    inp = _np_inputs(seed=15, batch=2, seqlen=14, nheads=4, headdim=3, dstate=2, ngroups=2)
    y, fin = ssd_recurrence(**inp)
    st = np.zeros_like(fin)
    for t in range(14):
        yt, st = ssd_step_ref(st, inp["x"][:, t], inp["dt"][:, t], inp["dt_bias"], inp["A"],
                              inp["B"][:, t], inp["C"][:, t], inp["D"])
        assert _rel(yt, y[:, t]) < 1e-13
    assert _rel(st, fin) < 1e-13


# --------------------------------------------------------------------------- staged form

@pytest.mark.parametrize("Q", [1, 2, 3, 4, 16, 64])
@pytest.mark.parametrize("L", [1, 7, 40, 65])
def test_staged_chunks_equal_recurrence(Q, L):
    inp = _np_inputs(seed=16 + L, batch=2, seqlen=L, nheads=4, headdim=3, dstate=5, ngroups=2)
    init = np.random.default_rng(L).standard_normal((2, 4, 3, 5))
    y, fin = ssd_recurrence(**inp, initial_state=init)
    ys, fs, mid = ssd_stages.ssd_chunked(**inp, chunk_size=Q, initial_state=init)
    assert _rel(ys, y) < 1e-12
    assert _rel(fs, fin) < 1e-12
    nc = (L + Q - 1) // Q
    assert mid["dtp"].shape == (2, 4, nc, Q)
    if L % Q:   # padding of the last chunk: no step, flat cumsum
        pad = L % Q
        assert np.all(mid["dtp"][:, :, -1, pad:] == 0.0)
        assert np.all(mid["dAcs"][:, :, -1, pad:] == mid["dAcs"][:, :, -1, pad - 1:pad])


def test_staged_chunk_size_invariance_at_workload_scale():
    """Chunk size must not change the result (the tail is kept, never dropped)."""
    inp = _np_inputs(seed=1, batch=1, seqlen=300, nheads=2, headdim=4, dstate=8, ngroups=1)
    y, fin = ssd_recurrence(**inp)
    for Q in (64, 128, 256):
        ys, fs, _ = ssd_stages.ssd_chunked(**inp, chunk_size=Q)
        assert _rel(ys, y) < 1e-12 and _rel(fs, fin) < 1e-12


# --------------------------------------------------------------------------- gate and dt clamp

def test_silu_against_library_sigmoid():
    import scipy.special
    from oracle import silu
    v = np.linspace(-40.0, 40.0, 161)
    np.testing.assert_allclose(silu(v), v * scipy.special.expit(v), rtol=1e-14, atol=1e-300)
    assert silu(np.float64(0.0)) == 0.0


def test_gate_multiplies_the_full_output():
    """y_gated = (scan + D x) * silu(z): z = 0 silences every output, and the gated output is the
    ungated one times v * sigmoid(v) (library sigmoid), in all four oracle forms."""
    import scipy.special
    inp = _np_inputs(seed=31, batch=2, seqlen=21, nheads=4, headdim=3, dstate=2, ngroups=2)
    z = np.random.default_rng(5).standard_normal(inp["x"].shape) * 3.0
    y0, f0 = ssd_recurrence(**inp)
    yz, fz = ssd_recurrence(**inp, z=z)
    np.testing.assert_allclose(yz, y0 * z * scipy.special.expit(z), rtol=1e-13, atol=1e-15)
    assert np.array_equal(f0, fz)                          # the gate never touches the state
    yq = ssd_quadratic(**inp, z=z)
    assert _rel(yq, yz) < 1e-12
    ys, fs, _ = ssd_stages.ssd_chunked(**inp, z=z, chunk_size=8)
    assert _rel(ys, yz) < 1e-12 and _rel(fs, fz) < 1e-12
    y_off, _ = ssd_recurrence(**inp, z=np.zeros_like(z))
    assert np.all(y_off == 0.0)
    st = np.zeros_like(f0)
    for t in range(21):
        yt, st = ssd_step_ref(st, inp["x"][:, t], inp["dt"][:, t], inp["dt_bias"], inp["A"], inp["B"][:, t],
                              inp["C"][:, t], inp["D"], z=z[:, t])
        assert _rel(yt, yz[:, t]) < 1e-13


def test_dt_clamp_saturated_is_constant_step_filter():
    """With every softplus(dt + bias) above dt_max the step is dt_max everywhere: the scalar
    channel becomes the IIR filter with d = dt_max (library lfilter); below dt_min, d = dt_min."""
    L = 50
    xs = np.random.default_rng(8).standard_normal(L)
    A = -3.0
    for dt_raw, (lo, hi), d in ((5.0, (1e-3, 0.1), 0.1), (-30.0, (0.02, 0.1), 0.02)):
        a = math.exp(d * A)
        ref = scipy.signal.lfilter([d], [1.0, -a], xs)
        y, _ = ssd_recurrence(xs.reshape(1, L, 1, 1), np.full((1, L, 1), dt_raw), np.zeros(1), np.array([A]),
                              np.ones((1, L, 1, 1)), np.ones((1, L, 1, 1)), None, dt_limit=(lo, hi))
        assert _rel(y[0, :, 0, 0], ref) < 1e-12


def test_dt_clamp_inactive_and_staged():
    inp = _np_inputs(seed=32, batch=1, seqlen=40, nheads=3, headdim=2, dstate=3, ngroups=1)
    y0, f0 = ssd_recurrence(**inp)
    yw, fw = ssd_recurrence(**inp, dt_limit=(0.0, 1e9))         # wide limits change nothing
    assert np.array_equal(y0, yw) and np.array_equal(f0, fw)
    yc, fc = ssd_recurrence(**inp, dt_limit=(1e-2, 5e-2))
    assert _rel(yc, y0) > 1e-3                                   # a binding clamp does change results
    ys, fs, mid = ssd_stages.ssd_chunked(**inp, chunk_size=16, dt_limit=(1e-2, 5e-2))
    assert _rel(ys, yc) < 1e-12 and _rel(fs, fc) < 1e-12
    valid = mid["dtp"][:, :, :, :][mid["dtp"] > 0]
    assert valid.min() >= 1e-2 and valid.max() <= 5e-2
    yq = ssd_quadratic(**inp, dt_limit=(1e-2, 5e-2))
    assert _rel(yq, yc) < 1e-12
