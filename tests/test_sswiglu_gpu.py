"""GPU parity of the Spatial SwiGLU middle (gtr_sswiglu_mix) against the fp64 oracle.

m = SiLU(gate) * (depthwise k x k convolution of value + bias), zero padding.
The kernel computes in fp32 and rounds m once to the I/O type, so the bar is
elementwise: every 16-bit output within one unit in the last place of the
oracle's value rounded to the I/O type (a rounding boundary crossed by the
fp32 result) plus the fp32 error bound of the sum, |SiLU(gate)| (|b| +
sum |w| |value|) (k^2 + 2) 2^-24, and rel-L2 <= 1e-3; float32 I/O within
rel-L2 1e-6.
"""
import numpy as np
import pytest
import torch

import gated_token_recurrence_amd as g
from gated_token_recurrence_amd import workloads as W

from _helpers import to_dev, to_f64

pytestmark = pytest.mark.gpu

SIG_BITS = {"f16": 11, "bf16": 8}
MIN_QUANTUM = {"f16": 2.0 ** -24, "bf16": 2.0 ** -133}  # subnormal spacing


def _note(msg):
    print(msg, flush=True)


def _run(x, dtype):
    u = to_dev(x["u"], dtype)
    out = g.sswiglu_mix(u, torch.from_numpy(x["w_conv"]).cuda(), torch.from_numpy(x["b_conv"]).cuda())
    torch.cuda.synchronize()
    return to_f64(out)


def _fp32_bound(oracle_mod, u64, w, b):
    """|SiLU(gate)| (|b| + sum |w| |value|) (k^2 + 2) 2^-24: the fp32 error of m."""
    F, k = w.shape[0], w.shape[1]
    gate = u64[..., :F]
    s_abs = oracle_mod.depthwise_conv2d(np.abs(u64[..., F:]), np.abs(w), np.abs(b))
    return np.abs(gate / (1.0 + np.exp(-gate))) * s_abs * (k * k + 2) * 2.0 ** -24


def _check(got, ref, dtype, oracle_mod, what, bound=0.0):
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    if dtype == "f32":
        rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
        assert rel <= 1e-6, f"{what}: rel-L2 {rel:.2e}"
        return rel
    r = oracle_mod.round_io(ref, dtype)
    d = np.abs(got - r)
    _, e = np.frexp(np.abs(r))
    ulp = np.maximum(np.ldexp(1.0, e - SIG_BITS[dtype]), MIN_QUANTUM[dtype])
    bad = d > ulp + bound
    assert not bad.any(), (f"{what}: {bad.sum()} outputs off by more than one unit in the last "
                           f"place (worst {d[bad].max():.3e})")
    rel = np.linalg.norm(got - r) / np.linalg.norm(r)
    assert rel <= 1e-3, f"{what}: rel-L2 {rel:.2e}"
    return rel


SHAPES = [
    # B, gh, gw, F, k, dtype
    (1, 7, 9, 8, 3, "f16"),
    (2, 5, 33, 24, 3, "bf16"),
    (1, 13, 16, 64, 3, "f16"),
    (1, 1, 1, 16, 3, "bf16"),
    (1, 1, 40, 16, 3, "f16"),
    (1, 40, 1, 16, 3, "bf16"),
    (1, 9, 21, 40, 1, "f16"),
    (1, 9, 21, 40, 5, "bf16"),
    (1, 11, 18, 32, 7, "f16"),
    (1, 6, 17, 4096, 3, "bf16"),   # two channel blocks per strip
    (1, 5, 19, 2056, 5, "f16"),    # ragged channel block
    (1, 8, 10, 16, 3, "f32"),
    (2, 9, 23, 24, 5, "f32"),
    (1, 5, 6, 8, 7, "f32"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_sswiglu_shapes(oracle_mod, shape):
    B, gh, gw, F, k, dtype = shape
    x = W.make_sswiglu(B, gh, gw, F, k, dtype, seed=B * 1000 + gh * 10 + k)
    _note(f"sswiglu {shape}")
    got = _run(x, dtype)
    u64 = W.io_to_f64(x["u"], dtype)
    ref = oracle_mod.sswiglu_mix(u64, x["w_conv"], x["b_conv"])
    _check(got, ref, dtype, oracle_mod, f"sswiglu {shape}",
           _fp32_bound(oracle_mod, u64, x["w_conv"], x["b_conv"]))


@pytest.mark.parametrize("name", ["sswiglu_640", "sswiglu_1024"])
def test_sswiglu_workloads(oracle_mod, name):
    """The benchmarked shapes; for the 8-image batch the oracle checks images 0 and 7."""
    w = W.SSWIGLU_WORKLOADS[name]
    x = W.make_sswiglu_inputs(w)
    _note(f"sswiglu workload {name}")
    got = _run(x, w.dtype)
    u64 = W.io_to_f64(x["u"], w.dtype)
    for b in sorted({0, w.B - 1}):
        ref = oracle_mod.sswiglu_mix(u64[b:b + 1], x["w_conv"], x["b_conv"])
        rel = _check(got[b:b + 1], ref, w.dtype, oracle_mod, f"{name} image {b}",
                     _fp32_bound(oracle_mod, u64[b:b + 1], x["w_conv"], x["b_conv"]))
        _note(f"  image {b}: rel-L2 {rel:.2e}")


def test_sswiglu_wide_strips_ragged(oracle_mod):
    """Enough row blocks for the 64-column strips, with a ragged last strip (100 =
    64 + 36 columns) and a ragged last row block (65 rows)."""
    B, gh, gw, F, k, dtype = 8, 65, 100, 256, 3, "bf16"
    x = W.make_sswiglu(B, gh, gw, F, k, dtype, seed=99)
    _note("sswiglu wide strips 8x65x100x256")
    got = _run(x, dtype)
    u64 = W.io_to_f64(x["u"], dtype)
    ref = oracle_mod.sswiglu_mix(u64, x["w_conv"], x["b_conv"])
    _check(got, ref, dtype, oracle_mod, "wide strips",
           _fp32_bound(oracle_mod, u64, x["w_conv"], x["b_conv"]))


def test_sswiglu_back_to_back_is_bitwise_stable(oracle_mod):
    x = W.make_sswiglu(1, 12, 20, 64, 3, "bf16", seed=3)
    a = _run(x, "bf16")
    assert np.array_equal(a, _run(x, "bf16"))
