"""Pins of the oracle's low-rank forget gate against facts outside the oracle.

GTR paper, Method §1: the key-side forget gate is generated from the input by
a light low-rank projection with a temperature (the rank and the temperature
are lost on the page).  The oracle reads it as x = feat W + b per head channel
and log g = logsigmoid(x) / tau.  Each test below fails for a plausible slip:
a transposed or mis-indexed projection (head-major vs channel-major column), a
dropped bias, log(sigmoid) with the wrong sign or overflow at large |x|, the
temperature multiplied instead of divided, or a gate that is not the one the
recurrence then uses.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch


def _gate_inputs(B, gh, gw, H, dk, r, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    feat = rng.standard_normal((B, gh, gw, r)) * scale
    w = rng.standard_normal((r, H * dk)) * scale / math.sqrt(r)
    b = rng.standard_normal(H * dk) * 0.5
    return feat, w, b


def test_logsigmoid_matches_scipy_log_expit(oracle_mod):
    x = np.concatenate([np.linspace(-700, 700, 2801), np.linspace(-3, 3, 601),
                        [0.0, 1e-300, -1e-300, 36.0, -36.0, 745.0, -745.0]])
    got = oracle_mod.logsigmoid(x)
    ref = scipy.special.log_expit(x)
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, ref, rtol=1e-14, atol=0)


def test_logsigmoid_asymptotes(oracle_mod):
    # log sigma(x) -> x for x -> -inf, and -> -exp(-x) for x -> +inf
    for x in (-40.0, -100.0, -600.0):
        assert oracle_mod.logsigmoid(np.array([x]))[0] == pytest.approx(x, rel=1e-15)
    for x in (40.0, 100.0, 600.0):
        assert oracle_mod.logsigmoid(np.array([x]))[0] == pytest.approx(-math.exp(-x), rel=1e-12)
    assert oracle_mod.logsigmoid(np.array([0.0]))[0] == -math.log(2.0)


def test_zero_features_leave_the_bias_gate(oracle_mod):
    feat = np.zeros((1, 2, 3, 4))
    w = np.random.default_rng(0).standard_normal((4, 2 * 8))
    b = np.zeros(16)
    lg = oracle_mod.lowrank_log_g(feat, w, b, 16.0, 2, 8)
    assert lg.shape == (1, 2, 3, 2, 8)
    assert np.all(lg == -math.log(2.0) / 16.0)
    b2 = np.linspace(-3, 3, 16)
    lg2 = oracle_mod.lowrank_log_g(feat, w, b2, 2.0, 2, 8)
    ref = np.array([math.log(1.0 / (1.0 + math.exp(-t))) / 2.0 for t in b2]).reshape(2, 8)
    np.testing.assert_allclose(lg2[0, 1, 2], ref, rtol=1e-13)


def test_projection_brute_force_loops(oracle_mod):
    """Python loops over (token, head, channel, rank): column h*dk + c of W."""
    B, gh, gw, H, dk, r, tau = 2, 2, 3, 3, 4, 5, 3.0
    feat, w, b = _gate_inputs(B, gh, gw, H, dk, r, seed=1)
    got = oracle_mod.lowrank_log_g(feat, w, b, tau, H, dk)
    for bb in range(B):
        for y in range(gh):
            for x in range(gw):
                for h in range(H):
                    for c in range(dk):
                        s = b[h * dk + c]
                        for j in range(r):
                            s += feat[bb, y, x, j] * w[j, h * dk + c]
                        ref = -math.log1p(math.exp(-s)) / tau
                        assert got[bb, y, x, h, c] == pytest.approx(ref, rel=1e-12, abs=1e-15)


def test_gate_power_is_sigmoid(oracle_mod):
    """g^tau = sigmoid(x), with sigmoid from torch."""
    B, gh, gw, H, dk, r, tau = 1, 3, 4, 2, 8, 16, 16.0
    feat, w, b = _gate_inputs(B, gh, gw, H, dk, r, seed=2, scale=3.0)
    lg = oracle_mod.lowrank_log_g(feat, w, b, tau, H, dk)
    x = torch.from_numpy(feat).reshape(-1, r) @ torch.from_numpy(w) + torch.from_numpy(b)
    sig = torch.sigmoid(x).numpy().reshape(lg.shape)
    np.testing.assert_allclose(np.exp(tau * lg), sig, rtol=1e-12)
    assert np.all(lg <= 0.0)


def test_fwd_lowrank_is_fwd_with_that_gate(oracle_mod):
    """The recurrence uses the projected gate of its own head and channel."""
    B, gh, gw, H, dk, dv, r, tau = 1, 4, 5, 2, 8, 8, 4, 4.0
    rng = np.random.default_rng(3)
    q, k = (rng.standard_normal((B, gh, gw, H, dk)) for _ in range(2))
    v, z = (rng.standard_normal((B, gh, gw, H, dv)) for _ in range(2))
    rw = 1.0 + 0.1 * rng.standard_normal(dv)
    feat, w, b = _gate_inputs(B, gh, gw, H, dk, r, seed=4, scale=2.0)
    xg = np.einsum("bywj,jn->bywn", feat, w) + b
    lg_ref = (scipy.special.log_expit(xg) / tau).reshape(B, gh, gw, H, dk)
    for direction in range(4):
        got = oracle_mod.fwd_lowrank(q, k, v, feat, w, b, tau, z, rw, direction)
        ref = oracle_mod.fwd(q, k, v, lg_ref, z, rw, direction)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
    # swapping the two heads' gate columns changes the result (the mapping matters)
    w_sw = np.concatenate([w[:, dk:], w[:, :dk]], axis=1)
    b_sw = np.concatenate([b[dk:], b[:dk]])
    other = oracle_mod.fwd_lowrank(q, k, v, feat, w_sw, b_sw, tau, z, rw, 0)
    assert np.max(np.abs(other - oracle_mod.fwd_lowrank(q, k, v, feat, w, b, tau, z, rw, 0))) > 1e-3


def test_lowrank_rejects_bad_shapes(oracle_mod):
    feat, w, b = _gate_inputs(1, 2, 2, 2, 4, 3, seed=5)
    with pytest.raises(ValueError):
        oracle_mod.lowrank_log_g(feat, w[:, :-1], b, 1.0, 2, 4)
    with pytest.raises(ValueError):
        oracle_mod.lowrank_log_g(feat, w, b, 0.0, 2, 4)
