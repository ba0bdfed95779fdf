"""Pins of the gated RMSNorm oracle (oracle/gated_norm.py) to things other than itself: torch's
rms_norm (a library routine of the same definition, float64 on the CPU), a hand example, closed
forms (a constant group, scale invariance, unit mean square) and the independence of groups.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle.gated_norm import gated_rmsnorm


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("H,P,nh,eps,gate", [(4, 8, 4, 1e-5, True), (4, 8, 2, 0.5, True), (6, 4, 1, 1e-3, False),
                                            (3, 16, 3, 0.25, False)])
def test_matches_torch_rms_norm(H, P, nh, eps, gate):
    Bt, L = 2, 5
    y, z, w = _rand((Bt, L, H, P), 1), _rand((Bt, L, H, P), 2), _rand((H * P,), 3)
    out = gated_rmsnorm(y, z if gate else None, w, eps=eps, norm_heads=nh)
    ty = torch.from_numpy(y)
    g = ty * F.silu(torch.from_numpy(z)) if gate else ty
    g5 = g.reshape(Bt, L, H // nh, nh, P)
    ref = F.rms_norm(g5, (nh, P), eps=eps) * torch.from_numpy(w).reshape(H // nh, nh, P)
    np.testing.assert_allclose(out, ref.reshape(Bt, L, H, P).numpy(), rtol=1e-12, atol=1e-12)


def test_hand_example():
    # y = (3, 4), one head of two channels, no gate, eps = 0: rms = sqrt((9 + 16) / 2) = 3.5355339...
    out = gated_rmsnorm(np.array([3.0, 4.0]).reshape(1, 1, 1, 2), None, np.array([1.0, 2.0]), eps=0.0)
    np.testing.assert_allclose(out.ravel(), [3.0 / np.sqrt(12.5), 8.0 / np.sqrt(12.5)], rtol=1e-15)


def test_constant_group_closed_form():
    c, eps = -1.7, 0.3
    y = np.full((1, 3, 2, 5), c)
    w = _rand((10,), 4)
    out = gated_rmsnorm(y, None, w, eps=eps)
    np.testing.assert_allclose(out, np.broadcast_to(c / np.sqrt(c * c + eps) * w.reshape(2, 5), out.shape),
                               rtol=1e-14)


def test_scale_invariance_and_unit_mean_square():
    y = _rand((2, 4, 6, 8), 5)
    ones = np.ones(48)
    a = gated_rmsnorm(y, None, ones, eps=0.0, norm_heads=3)
    np.testing.assert_allclose(gated_rmsnorm(7.5 * y, None, ones, eps=0.0, norm_heads=3), a, rtol=1e-13)
    np.testing.assert_allclose(gated_rmsnorm(-y, None, ones, eps=0.0, norm_heads=3), -a, rtol=1e-13)
    ms = (a.reshape(2, 4, 2, 3 * 8) ** 2).mean(axis=-1)
    np.testing.assert_allclose(ms, 1.0, rtol=1e-13)


def test_groups_are_independent_and_gate_comes_first():
    y, z, w = _rand((1, 2, 4, 4), 6), _rand((1, 2, 4, 4), 7), _rand((16,), 8)
    a = gated_rmsnorm(y, z, w, eps=1e-2, norm_heads=2)
    y2 = y.copy()
    y2[:, :, 2:] *= 10.0                                   # only the second group of heads changes
    b = gated_rmsnorm(y2, z, w, eps=1e-2, norm_heads=2)
    np.testing.assert_array_equal(a[:, :, :2], b[:, :, :2])
    assert not np.allclose(a[:, :, 2:], b[:, :, 2:])
    # the gate multiplies before the norm: gating after the norm gives something else
    post = gated_rmsnorm(y, None, w, eps=1e-2, norm_heads=2) * (z / (1 + np.exp(-z)))
    assert not np.allclose(a, post)
