"""Pins of the fp64 backward oracle (oracle/backward.py) against facts outside it.

(1) torch autograd of an independent fp64 forward written as the O(L^2) closed
form o_t = sum_{s<=t} ((q_t exp(A_t - A_s)) . k_s) v_s (A = inclusive cumulative
log-gate) with torch's own rms_norm and silu, its scan order built here from
reshapes and flips of the grid (not from the oracle's order); (2) central finite
differences of the C forward oracle along random directions; (3) the oracle's
forward states reproduce the C oracle's output.  All three run in every scan
direction.  A slip in any gradient term (a missing decay in the reverse
recurrence, the gate gradient taken at the wrong state, the RMSNorm backward
without its projection term, silu' wrong) fails (1) and (2); a wrong scan order
in any direction fails all three.
"""
import numpy as np
import pytest
import torch

from oracle import backward as ob


def _inputs(B, gh, gw, H, dk, dv, seed, temp=4.0):
    rng = np.random.default_rng(seed)
    q, k = rng.standard_normal((2, B, gh, gw, H, dk))
    v, z, dy = rng.standard_normal((3, B, gh, gw, H, dv))
    lg = -np.logaddexp(0.0, -rng.standard_normal((B, gh, gw, H, dk))) / temp
    w = 1.0 + 0.1 * rng.standard_normal(dv)
    return q, k, v, lg, z, w, dy


def _scan_order(gh, gw, direction):
    """Grid index of each scan step, from the grid itself: LR the row-major
    raster, RL its reverse, TB the row-major raster of the transposed grid
    (columns top to bottom, left to right), BT its reverse."""
    grid = np.arange(gh * gw).reshape(gh, gw)
    raster = grid.T.ravel() if direction >= 2 else grid.ravel()
    return raster[::-1].copy() if direction & 1 else raster


def test_scan_order_by_hand():
    # 2 x 3 grid: positions 0 1 2 / 3 4 5
    assert _scan_order(2, 3, 0).tolist() == [0, 1, 2, 3, 4, 5]
    assert _scan_order(2, 3, 1).tolist() == [5, 4, 3, 2, 1, 0]
    assert _scan_order(2, 3, 2).tolist() == [0, 3, 1, 4, 2, 5]
    assert _scan_order(2, 3, 3).tolist() == [5, 2, 4, 1, 3, 0]


def _torch_closed_form(q, k, v, lg, z, w, direction, eps=1e-5):
    """Independent forward: O(L^2) closed form per sequence, torch ops, fp64."""
    B, gh, gw, H, dk = q.shape
    dv = v.shape[-1]
    L = gh * gw
    order = torch.as_tensor(_scan_order(gh, gw, direction))
    inv = torch.empty_like(order)
    inv[order] = torch.arange(L)
    def seq(x, d):
        return x.reshape(B, L, H, d)[:, order].permute(0, 2, 1, 3)   # [B, H, L, d]
    Q, K, V, A, Z = seq(q, dk), seq(k, dk), seq(v, dv), seq(lg, dk).cumsum(2), seq(z, dv)
    decay = torch.exp(A[:, :, :, None, :] - A[:, :, None, :, :])     # [B,H,t,s,dk]
    mask = torch.tril(torch.ones(L, L, dtype=torch.bool))
    scores = (Q[:, :, :, None, :] * decay * K[:, :, None, :, :]).sum(-1)
    scores = torch.where(mask, scores, torch.zeros((), dtype=scores.dtype))
    O = scores @ V
    Y = torch.nn.functional.rms_norm(O, (dv,), weight=w, eps=eps) * torch.nn.functional.silu(Z)
    return Y.permute(0, 2, 1, 3)[:, inv].reshape(B, gh, gw, H, dv)


@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_matches_torch_autograd_of_closed_form(direction):
    B, gh, gw, H, dk, dv = 2, 3, 5, 2, 4, 3
    arrs = _inputs(B, gh, gw, H, dk, dv, seed=direction)
    q, k, v, lg, z, w, dy = (torch.tensor(a, dtype=torch.float64, requires_grad=i < 6)
                             for i, a in enumerate(arrs))
    y = _torch_closed_form(q, k, v, lg, z, w, direction)
    (y * dy).sum().backward()
    got = ob.bwd(*arrs, direction)
    for name, t in (("dq", q), ("dk", k), ("dv", v), ("dlog_g", lg), ("dz", z), ("drms_w", w)):
        np.testing.assert_allclose(got[name], t.grad.numpy(), rtol=1e-9, atol=1e-11,
                                   err_msg=name)


@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_central_differences_of_the_c_oracle(oracle_mod, direction):
    B, gh, gw, H, dk, dv = 1, 4, 3, 2, 3, 4
    arrs = list(_inputs(B, gh, gw, H, dk, dv, seed=7 + direction))
    dy = arrs[6]
    got = ob.bwd(*arrs, direction)
    rng = np.random.default_rng(8)
    h = 1e-6
    for i, name in enumerate(("dq", "dk", "dv", "dlog_g", "dz", "drms_w")):
        d = rng.standard_normal(arrs[i].shape)
        plus = list(arrs[:6]); minus = list(arrs[:6])
        plus[i] = arrs[i] + h * d
        minus[i] = arrs[i] - h * d
        lp = (oracle_mod.fwd(*plus, direction) * dy).sum()
        lm = (oracle_mod.fwd(*minus, direction) * dy).sum()
        fd = (lp - lm) / (2 * h)
        an = (got[name] * d).sum()
        assert an == pytest.approx(fd, rel=1e-6, abs=1e-8), name


def test_restricted_sequences_match_full_run():
    arrs = _inputs(2, 3, 4, 3, 4, 4, seed=9)
    full = ob.bwd(*arrs, 1)
    part = ob.bwd(*arrs, 1, bh=[1, 4])
    for name in ("dq", "dk", "dv", "dlog_g", "dz"):
        np.testing.assert_array_equal(part[name][0, :, :, 1], full[name][0, :, :, 1])
        np.testing.assert_array_equal(part[name][1, :, :, 1], full[name][1, :, :, 1])
        assert np.isnan(part[name][0, :, :, 0]).all()


@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_forward_states_reproduce_the_c_oracle(oracle_mod, direction):
    arrs = _inputs(2, 3, 5, 2, 4, 3, seed=20 + direction)
    got = ob.bwd(*arrs, direction)["y"]
    ref = oracle_mod.fwd(*arrs[:6], direction)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
