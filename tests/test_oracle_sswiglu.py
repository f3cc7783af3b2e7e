"""Pins of the oracle's Spatial SwiGLU middle against facts outside the oracle.

GTR write-up, Method §2: the value branch of the expanded SwiGLU projection is
reshaped to the 2-D token grid and mixed by a depthwise convolution before the
SiLU-gated product (kernel size lost on the page; the library takes it as an
argument).  Each test below fails for a plausible slip: a flipped kernel
(convolution instead of cross-correlation), swapped grid axes, wrong padding,
gate and value halves swapped, sigmoid instead of SiLU, or a dropped bias.
"""
import numpy as np
import pytest
import torch


def _case(B, gh, gw, F, k, seed):
    rng = np.random.default_rng(seed)
    u = rng.standard_normal((B, gh, gw, 2 * F))
    w = rng.standard_normal((F, k, k))
    b = rng.standard_normal(F)
    return u, w, b


@pytest.mark.parametrize("k", [1, 3, 5, 7])
def test_conv_matches_torch_conv2d(oracle_mod, k):
    """Depthwise conv == torch conv2d(groups=F, padding=k//2) in float64."""
    B, gh, gw, F = 2, 6, 9, 5
    u, w, b = _case(B, gh, gw, F, k, seed=k)
    val = u[..., F:]
    got = oracle_mod.depthwise_conv2d(val, w, b)
    x = torch.from_numpy(val).permute(0, 3, 1, 2)                  # [B, F, gh, gw]
    ref = torch.nn.functional.conv2d(x, torch.from_numpy(w)[:, None], torch.from_numpy(b),
                                     padding=k // 2, groups=F)
    np.testing.assert_allclose(got, ref.permute(0, 2, 3, 1).numpy(), rtol=1e-12, atol=1e-12)


def test_mix_matches_torch_silu_product(oracle_mod):
    B, gh, gw, F, k = 1, 5, 4, 6, 3
    u, w, b = _case(B, gh, gw, F, k, seed=11)
    got = oracle_mod.sswiglu_mix(u, w, b)
    x = torch.from_numpy(u[..., F:]).permute(0, 3, 1, 2)
    conv = torch.nn.functional.conv2d(x, torch.from_numpy(w)[:, None], torch.from_numpy(b),
                                      padding=1, groups=F).permute(0, 2, 3, 1)
    ref = torch.nn.functional.silu(torch.from_numpy(u[..., :F])) * conv
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_delta_kernel_reduces_to_swiglu(oracle_mod):
    B, gh, gw, F, k = 1, 4, 7, 3, 5
    u, _, b = _case(B, gh, gw, F, k, seed=2)
    w = np.zeros((F, k, k))
    w[:, k // 2, k // 2] = 1.0
    gate, val = u[..., :F], u[..., F:]
    ref = gate / (1.0 + np.exp(-gate)) * (val + b)
    np.testing.assert_allclose(oracle_mod.sswiglu_mix(u, w, b), ref, rtol=1e-14)


def test_brute_force_loops(oracle_mod):
    """Python loops with an asymmetric kernel and a non-square grid."""
    B, gh, gw, F, k = 1, 3, 4, 2, 3
    u, w, b = _case(B, gh, gw, F, k, seed=5)
    got = oracle_mod.depthwise_conv2d(u[..., F:], w, b)
    for y in range(gh):
        for x in range(gw):
            for f in range(F):
                s = b[f]
                for i in range(k):
                    for j in range(k):
                        yy, xx = y + i - 1, x + j - 1
                        if 0 <= yy < gh and 0 <= xx < gw:
                            s += w[f, i, j] * u[0, yy, xx, F + f]
                assert got[0, y, x, f] == pytest.approx(s, rel=1e-13, abs=1e-13)


def test_zero_padding_counts(oracle_mod):
    """Constant field, all-ones 3x3 kernel: 4 taps at corners, 6 on edges, 9 inside."""
    val = np.full((1, 5, 6, 2), 2.0)
    got = oracle_mod.depthwise_conv2d(val, np.ones((2, 3, 3)), np.zeros(2))
    assert got[0, 0, 0, 0] == 8.0 and got[0, 4, 5, 1] == 8.0
    assert got[0, 0, 2, 0] == 12.0 and got[0, 2, 0, 1] == 12.0
    assert got[0, 2, 3, 0] == 18.0


def test_cross_correlation_orientation(oracle_mod):
    """A single tap at kernel (0, 2) reads the neighbour one row up, one column right."""
    F, k = 1, 3
    val = np.arange(20.0).reshape(1, 4, 5, 1)
    w = np.zeros((F, k, k))
    w[0, 0, 2] = 1.0
    got = oracle_mod.depthwise_conv2d(val, w, np.zeros(1))
    assert got[0, 2, 2, 0] == val[0, 1, 3, 0]
    assert got[0, 0, 2, 0] == 0.0          # above the grid: zero padding
    assert got[0, 2, 4, 0] == 0.0          # right of the grid


def test_rejects_bad_shapes(oracle_mod):
    with pytest.raises(ValueError):
        oracle_mod.depthwise_conv2d(np.zeros((1, 2, 2, 3)), np.zeros((3, 2, 2)), np.zeros(3))
    with pytest.raises(ValueError):
        oracle_mod.depthwise_conv2d(np.zeros((1, 2, 2, 3)), np.zeros((4, 3, 3)), np.zeros(4))
