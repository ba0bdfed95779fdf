"""Pins of the conv1d oracle (oracle/conv1d.py) to facts outside itself.

Library routines computing the same depthwise causal convolution (numpy's full
convolution, torch's grouped conv1d in float64), a hand example with a closed form,
the causality test of "Agent 228: MAMBA-2 Implementation Gaps" (unit tests: an
impulse at t = 5 leaves every earlier output at zero), and the carried-state
invariants that decoding relies on.
"""
import math

import numpy as np
import pytest
import torch

from oracle import conv1d as CV
from oracle import silu


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_example_closed_form():
    # one channel, w = [1, 2, 3, 4] (w[K-1] multiplies the current input), unit impulse at t = 0:
    # u[t] = w[K-1-t] + bias  -> 4, 3, 2, 1 then bias alone
    v = np.array([1.0, 0, 0, 0, 0, 0]).reshape(1, 6, 1)
    w = np.array([[1.0, 2.0, 3.0, 4.0]])
    u, st = CV.causal_conv1d(v, w, np.array([0.5]))
    assert np.allclose(u[0, :, 0], [4.5, 3.5, 2.5, 1.5, 0.5, 0.5], rtol=0, atol=1e-15)
    out, _ = CV.causal_conv1d_silu(v, w, np.array([0.5]))
    assert math.isclose(out[0, 0, 0], 4.5 / (1.0 + math.exp(-4.5)), rel_tol=1e-15)
    assert np.array_equal(st[0, :, 0], [0.0, 0.0, 0.0])     # last three inputs


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_against_numpy_full_convolution(K):
    Bt, L, Dc = 2, 37, 5
    v, w, b = _rand((Bt, L, Dc), 1), _rand((Dc, K), 2), _rand(Dc, 3)
    u, _ = CV.causal_conv1d(v, w, b)
    for bi in range(Bt):
        for c in range(Dc):
            # np.convolve flips its second operand, so the taps go in reversed
            ref = np.convolve(v[bi, :, c], w[c, ::-1])[:L] + b[c]
            assert np.allclose(u[bi, :, c], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("K", [2, 4])
def test_against_torch_grouped_conv1d(K):
    """The pages' layer: Conv1d(groups=channels, kernel K, padding K-1), first L outputs, then SiLU."""
    Bt, L, Dc = 3, 50, 8
    v, w, b = _rand((Bt, L, Dc), 4), _rand((Dc, K), 5), _rand(Dc, 6)
    out, _ = CV.causal_conv1d_silu(v, w, b)
    tv = torch.from_numpy(v).transpose(1, 2)                              # (Bt, Dc, L)
    ref = torch.nn.functional.conv1d(tv, torch.from_numpy(w)[:, None, :], torch.from_numpy(b),
                                     padding=K - 1, groups=Dc)[:, :, :L]
    ref = torch.nn.functional.silu(ref).transpose(1, 2).numpy()
    assert np.allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_causality_impulse_at_t5():
    """An input at t = 5 (zero bias) leaves outputs t < 5 at exactly zero and reaches t = 5..8."""
    Bt, L, Dc, K = 1, 10, 64, 4
    v = np.zeros((Bt, L, Dc))
    v[:, 5] = 1.0
    w = _rand((Dc, K), 7)
    out, _ = CV.causal_conv1d_silu(v, w)
    assert np.abs(out[:, :5]).sum() == 0.0
    for t in range(5, 9):
        assert np.allclose(out[0, t], silu(w[:, K - 1 - (t - 5)]), rtol=1e-15, atol=0)
    assert np.abs(out[:, 9]).sum() == 0.0


def test_initial_state_is_the_preceding_inputs():
    """Conv with a carried state == conv of [state; sequence] with the first K-1 outputs dropped."""
    Bt, L, Dc, K = 2, 20, 6, 4
    v, w, b, st = _rand((Bt, L, Dc), 8), _rand((Dc, K), 9), _rand(Dc, 10), _rand((Bt, K - 1, Dc), 11)
    u, new = CV.causal_conv1d(v, w, b, st)
    for bi in range(Bt):
        for c in range(Dc):
            seq = np.concatenate([st[bi, :, c], v[bi, :, c]])
            ref = np.convolve(seq, w[c, ::-1])[K - 1:K - 1 + L] + b[c]
            assert np.allclose(u[bi, :, c], ref, rtol=1e-13, atol=1e-13)
    assert np.array_equal(new, v[:, L - (K - 1):])


@pytest.mark.parametrize("L1", [0, 1, 2, 3, 17])
def test_split_resume_and_short_sequences(L1):
    """Running [0, L1) then [L1, L) with the carried state equals one run; this covers
    pieces shorter than K - 1, whose new state still holds older history."""
    Bt, L, Dc, K = 2, 19, 5, 4
    v, w, b = _rand((Bt, L, Dc), 12), _rand((Dc, K), 13), _rand(Dc, 14)
    full, st_full = CV.causal_conv1d_silu(v, w, b)
    o1, s1 = CV.causal_conv1d_silu(v[:, :L1], w, b)
    o2, s2 = CV.causal_conv1d_silu(v[:, L1:], w, b, s1)
    assert np.allclose(np.concatenate([o1, o2], axis=1), full, rtol=1e-14, atol=1e-14)
    assert np.array_equal(s2, st_full)


def test_decode_steps_equal_forward():
    Bt, L, Dc, K = 2, 12, 7, 4
    v, w, b = _rand((Bt, L, Dc), 15), _rand((Dc, K), 16), _rand(Dc, 17)
    full, st_full = CV.causal_conv1d_silu(v, w, b)
    st = None
    for t in range(L):
        o, st = CV.conv1d_silu_step_ref(st if st is not None else np.zeros((Bt, K - 1, Dc)), v[:, t], w, b)
        assert np.allclose(o, full[:, t], rtol=1e-14, atol=1e-14)
    assert np.array_equal(st, st_full)


def test_split_xbc_channel_order():
    H, P, G, N = 3, 4, 2, 5
    Dc = H * P + 2 * G * N
    out = np.arange(2 * 3 * Dc, dtype=np.float64).reshape(2, 3, Dc)
    x, B, C = CV.split_xbc(out, H, P, G, N)
    assert x.shape == (2, 3, H, P) and B.shape == (2, 3, G, N) and C.shape == (2, 3, G, N)
    assert x[1, 2, 2, 3] == out[1, 2, 2 * P + 3]
    assert B[0, 1, 1, 4] == out[0, 1, H * P + N + 4]
    assert C[1, 0, 0, 0] == out[1, 0, H * P + G * N]
