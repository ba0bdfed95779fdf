"""Pins of the backward oracle (oracle/ssd_backward.py).

Every gradient is checked element by element against central finite differences of the
forward oracle (ssd_recurrence, itself pinned in test_oracle_pins.py) for the scalar loss
    loss = sum(w_y * y) + sum(w_f * final_state)
with fixed random weights, on tiny shapes that still have several heads per group, a nonzero
initial state, the D skip, the gate and the clamp.  A second check uses torch's float64
autograd through an independently written quadratic (materialised-matrix) form.
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import ssd_recurrence
from oracle.ssd_backward import ssd_recurrence_bwd


def _inputs(seed, Bt=2, L=5, H=4, P=3, N=2, G=2, with_D=True, with_init=True, with_z=False):
    r = np.random.default_rng(seed)
    inp = dict(
        x=r.standard_normal((Bt, L, H, P)), dt=r.standard_normal((Bt, L, H)) * 0.7,
        dt_bias=r.uniform(-2.0, 0.5, H), A=-r.uniform(0.3, 2.0, H),
        B=r.standard_normal((Bt, L, G, N)), C=r.standard_normal((Bt, L, G, N)),
        D=r.standard_normal((H, P)) if with_D else None,
        initial_state=r.standard_normal((Bt, H, P, N)) if with_init else None,
        z=r.standard_normal((Bt, L, H, P)) if with_z else None,
    )
    wy = r.standard_normal((Bt, L, H, P))
    wf = r.standard_normal((Bt, H, P, N))
    return inp, wy, wf


def _loss(inp, wy, wf, dt_limit):
    y, f = ssd_recurrence(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], inp["D"],
                          initial_state=inp["initial_state"], z=inp["z"], dt_limit=dt_limit)
    return float((wy * y).sum() + (wf * f).sum())


def _fd_check(inp, wy, wf, dt_limit=None, eps=1e-6, tol=2e-7):
    got = ssd_recurrence_bwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], wy, inp["D"],
                             initial_state=inp["initial_state"], z=inp["z"], dt_limit=dt_limit, dfinal=wf)
    names = {"x": "dx", "dt": "ddt", "dt_bias": "ddt_bias", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
             "initial_state": "dinitial_state", "z": "dz"}
    for k, gk in names.items():
        if inp[k] is None:
            assert got[gk] is None or k == "initial_state"
            continue
        fd = np.zeros_like(inp[k])
        for idx in itertools.product(*map(range, inp[k].shape)):
            keep = inp[k][idx]
            inp[k][idx] = keep + eps
            up = _loss(inp, wy, wf, dt_limit)
            inp[k][idx] = keep - eps
            dn = _loss(inp, wy, wf, dt_limit)
            inp[k][idx] = keep
            fd[idx] = (up - dn) / (2 * eps)
        scale = max(1.0, np.abs(fd).max())
        err = np.abs(got[gk] - fd).max() / scale
        assert err < tol, f"{gk}: max error {err:.2e} against finite differences"


def test_gradients_plain():
    inp, wy, wf = _inputs(0, with_D=False, with_init=False)
    _fd_check(inp, wy, wf)


def test_gradients_with_D_and_initial_state():
    inp, wy, wf = _inputs(1)
    _fd_check(inp, wy, wf)


def test_gradients_with_gate():
    inp, wy, wf = _inputs(2, with_z=True)
    _fd_check(inp, wy, wf)


def test_gradients_with_clamp_both_ends_binding():
    inp, wy, wf = _inputs(3, with_z=True, L=6)
    d = np.logaddexp(0.0, inp["dt"] + inp["dt_bias"][None, None, :])
    lo, hi = np.quantile(d, 0.25), np.quantile(d, 0.75)
    # keep every step at least 10 eps away from a clamp edge so the differences do not straddle it
    assert np.abs(d - lo).min() > 1e-5 and np.abs(d - hi).min() > 1e-5
    _fd_check(inp, wy, wf, dt_limit=(lo, hi))
    # clamped positions pass no gradient to dt
    got = ssd_recurrence_bwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], wy, inp["D"],
                             initial_state=inp["initial_state"], z=inp["z"], dt_limit=(lo, hi), dfinal=wf)
    out = (d < lo) | (d > hi)
    assert out.any() and np.all(got["ddt"][out] == 0.0)


def test_gradients_one_group_many_heads_longer():
    inp, wy, wf = _inputs(4, Bt=1, L=9, H=3, P=2, N=3, G=1)
    _fd_check(inp, wy, wf)


def _torch_quadratic_loss(t, wy, wf, G):
    """Independent float64 torch forward: the materialised causal matrix per (b, h) plus the
    final state as the decayed sum of outer products."""
    x, dt, bias, A, B, C, D, h0 = (t[k] for k in ("x", "dt", "dt_bias", "A", "B", "C", "D", "initial_state"))
    Bt, L, H, P = x.shape
    d = torch.nn.functional.softplus(dt + bias)                  # (Bt, L, H)
    lam = torch.cumsum(d * A, dim=1)                              # log of the running decay
    heads = torch.arange(H) // (H // G)
    Bh, Ch = B[:, :, heads], C[:, :, heads]                      # (Bt, L, H, N)
    loss = 0.0
    tt = torch.arange(L)
    mask = (tt[:, None] >= tt[None, :]).double()
    for b in range(Bt):
        for h in range(H):
            dec = torch.exp(lam[b, :, h][:, None] - lam[b, :, h][None, :]) * mask
            M = (Ch[b, :, h] @ Bh[b, :, h].T) * dec * d[b, :, h][None, :]
            y = M @ x[b, :, h] + D[h][None, :] * x[b, :, h]
            y = y + torch.exp(lam[b, :, h])[:, None] * (Ch[b, :, h] @ h0[b, h].T)
            fin = torch.exp(lam[b, -1, h]) * h0[b, h] + \
                ((torch.exp(lam[b, -1, h] - lam[b, :, h]) * d[b, :, h])[:, None] * x[b, :, h]).T @ Bh[b, :, h]
            loss = loss + (wy[b, :, h] * y).sum() + (wf[b, h] * fin).sum()
    return loss


def test_gradients_match_torch_autograd_of_quadratic_form():
    inp, wy, wf = _inputs(5, Bt=2, L=7, H=4, P=3, N=5, G=2)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp.items() if v is not None}
    loss = _torch_quadratic_loss(t, torch.tensor(wy), torch.tensor(wf), G=2)
    loss.backward()
    got = ssd_recurrence_bwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], wy, inp["D"],
                             initial_state=inp["initial_state"], dfinal=wf)
    for k, gk in (("x", "dx"), ("dt", "ddt"), ("dt_bias", "ddt_bias"), ("A", "dA"), ("B", "dB"), ("C", "dC"),
                  ("D", "dD"), ("initial_state", "dinitial_state")):
        ref = t[k].grad.numpy()
        assert np.allclose(got[gk], ref, rtol=1e-10, atol=1e-10), gk


@pytest.mark.parametrize("seed", [6, 7])
def test_zero_upstream_gives_zero_gradients(seed):
    inp, wy, wf = _inputs(seed, with_z=True)
    got = ssd_recurrence_bwd(inp["x"], inp["dt"], inp["dt_bias"], inp["A"], inp["B"], inp["C"], np.zeros_like(wy),
                             inp["D"], initial_state=inp["initial_state"], z=inp["z"], dfinal=None)
    for k, v in got.items():
        assert v is None or np.count_nonzero(v) == 0, k
