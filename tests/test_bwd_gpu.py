"""GPU parity of the backward pass (gtr_gla_bwd) against the fp64 backward oracle.

The kernels compute in fp32 from the same (rounded) inputs the oracle gets, so:
float32 gradients (every gradient for float32 I/O; dlog_g and drms_w always)
within rel-L2 1e-4 of the oracle; 16-bit gradients (dq, dk, dv, dz) within
rel-L2 1e-3 of the oracle rounded to the I/O type.  An absolute allowance is
added: 1e-10 per element, and for dlog_g the fp32 bound of a cancelling sum,
64 2^-24 sqrt(L) || |q dq| + |k dk| ||: the kernels form the gate gradient as
a reverse cumulative sum of q dq - k dk, whose terms cancel (exactly, for a
scan's first token, where the gradient is zero), so its error scales with
those terms rather than with the result.
"""
import numpy as np
import pytest
import torch

import gated_token_recurrence_amd as g
from gated_token_recurrence_amd import workloads as W

from _helpers import inputs_f64, inputs_to_dev, to_dev, to_f64

pytestmark = pytest.mark.gpu

IO_GRADS = ("dq", "dk", "dv", "dz")


def _note(msg):
    print(msg, flush=True)


def _run_case(oracle_mod, x, dtype, direction, chunk=0, bh=None, seed=0):
    from oracle import backward as ob
    shape_v = x["v"].shape
    dy = W.cast_io(np.random.default_rng(seed).standard_normal(shape_v), dtype)
    t = inputs_to_dev(x, dtype)
    grads, n = g.gla_bwd(t["q"], t["k"], t["v"], t["log_g"], t["z"], t["rms_w"],
                         to_dev(dy, dtype), direction, chunk=chunk)
    torch.cuda.synchronize()
    # 9 launches on the fp32 path; 7 on the matrix-core path (16-bit I/O,
    # dk = dv = 64, chunk <= 64): forward summaries and scan, the epilogue backward
    # with the reverse summaries, its token-serial fallback for flagged chunks (which
    # also completes drms_w), the reverse scan, the gradients, their fallback
    mfma = dtype != "f32" and x["q"].shape[4] == 64 and x["v"].shape[4] == 64 and (chunk or 64) <= 64
    assert n == (7 if mfma else 9), n
    f = inputs_f64(x, dtype)
    ref = ob.bwd(f["q"], f["k"], f["v"], f["log_g"], f["z"], f["rms_w"],
                 W.io_to_f64(dy, dtype), direction, bh=bh)
    H = x["q"].shape[3]
    L = x["q"].shape[1] * x["q"].shape[2]
    gate_terms = np.abs(f["q"] * ref["dq"]) + np.abs(f["k"] * ref["dk"])
    worst = {}
    for name, got_t in grads.items():
        got = to_f64(got_t)
        r = ref[name]
        terms = gate_terms
        if bh is not None and name != "drms_w":
            sel = [(s // H, s % H) for s in bh]
            got = np.stack([got[b, :, :, h] for b, h in sel])
            r = np.stack([r[b, :, :, h] for b, h in sel])
            terms = np.stack([gate_terms[b, :, :, h] for b, h in sel])
        if name == "drms_w" and bh is not None:
            continue  # summed over the chosen sequences only
        assert np.isfinite(got).all(), f"{name}: non-finite"
        if dtype != "f32" and name in IO_GRADS:
            r = oracle_mod.round_io(r, dtype)
            tol = 1e-3
        else:
            tol = 1e-4
        allow = 1e-10 * np.sqrt(r.size)
        if name == "dlog_g":
            allow += 64 * 2.0 ** -24 * np.sqrt(L) * np.linalg.norm(terms)
        err = np.linalg.norm(got - r)
        rel = err / (np.linalg.norm(r) + allow / tol)
        worst[name] = rel
        assert err <= tol * np.linalg.norm(r) + allow, (
            f"{name}: error {err:.2e}, rel-L2 {err / max(np.linalg.norm(r), 1e-300):.2e} > {tol:.0e}")
    _note("  " + " ".join(f"{k} {v:.1e}" for k, v in worst.items()))


SHAPES = [
    # B, gh, gw, H, dk, dv, dtype, chunk
    (1, 7, 9, 2, 32, 32, "f32", 16),
    (2, 5, 13, 3, 64, 64, "f32", 32),
    (1, 9, 7, 2, 128, 64, "f32", 64),
    (1, 6, 11, 1, 32, 128, "f32", 128),
    (1, 17, 15, 2, 64, 64, "f16", 64),
    (2, 12, 12, 2, 64, 128, "bf16", 64),
    (1, 1, 1, 2, 64, 64, "f16", 64),
    (1, 1, 70, 1, 64, 64, "bf16", 32),
    (1, 70, 1, 1, 64, 64, "f16", 16),
    (2, 9, 13, 3, 64, 64, "bf16", 64),   # matrix path, two images
    (1, 64, 64, 2, 64, 64, "f16", 32),   # matrix path, 128 chunks per sequence of one-chunk segments
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_shapes(oracle_mod, shape):
    B, gh, gw, H, dk, dv, dtype, chunk = shape
    x = W.make_custom(B, gh, gw, H, dk, dv, dtype, seed=B * 100 + gh + dk)
    _note(f"bwd {shape}")
    _run_case(oracle_mod, x, dtype, direction=1, chunk=chunk, seed=3)


@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_bwd_directions(oracle_mod, direction):
    x = W.make_custom(1, 9, 11, 2, 64, 64, "f32", seed=40 + direction)
    _note(f"bwd direction {direction}")
    _run_case(oracle_mod, x, "f32", direction, chunk=16, seed=direction)


@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_bwd_matrix_path_directions(oracle_mod, direction):
    """The matrix-core path in every scan order (fp16, 24 x 20 grid: 8 chunks per
    sequence with a 32-token tail)."""
    x = W.make_custom(1, 24, 20, 2, 64, 64, "f16", seed=50 + direction)
    _note(f"bwd matrix path direction {direction}")
    _run_case(oracle_mod, x, "f16", direction, chunk=64, seed=20 + direction)


@pytest.mark.parametrize("log_g", [0.0, -1e-4, -3.0])
def test_bwd_extreme_gates(oracle_mod, log_g):
    x = W.make_custom(1, 8, 12, 2, 64, 64, "f32", seed=7, log_g_const=log_g)
    _note(f"bwd constant log_g {log_g}")
    _run_case(oracle_mod, x, "f32", 2, chunk=32, seed=1)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("log_g", [0.0, -1e-4, -0.5, -3.0])
def test_bwd_matrix_path_gates(oracle_mod, dtype, log_g):
    """16-bit I/O on the matrix-core gradients; -3.0 per token spans far more than
    64 log2 units per chunk, so every chunk falls back to the token-serial kernels."""
    x = W.make_custom(1, 11, 13, 2, 64, 64, dtype, seed=17, log_g_const=log_g)
    _note(f"bwd matrix path {dtype} constant log_g {log_g}")
    _run_case(oracle_mod, x, dtype, 1, chunk=64, seed=5)


def test_bwd_matrix_path_mixed_spans(oracle_mod):
    """Some chunks in range, others flagged (one channel decays fast in the second
    half of the scan only)."""
    x = W.make_custom(1, 16, 16, 2, 64, 64, "f16", seed=23)
    lg = x["log_g"].reshape(1, 256, 2, 64)
    lg[:, 128:, 1, 5] = -3.0
    x["log_g"] = np.ascontiguousarray(lg.reshape(x["log_g"].shape))
    _note("bwd matrix path mixed spans")
    _run_case(oracle_mod, x, "f16", 0, chunk=64, seed=6)


def test_bwd_mixer_640_sampled(oracle_mod):
    """The 1.6K-token workload (H = 6, fp16), three sequences checked."""
    w = W.WORKLOADS["mixer_640"]
    x = W.make_inputs(w)
    _note("bwd mixer_640")
    _run_case(oracle_mod, x, w.dtype, 0, chunk=w.chunk, bh=[0, 3, 5], seed=11)


def test_bwd_mixer_2048_sampled(oracle_mod):
    """The 16.4K-token workload the benchmark times (H = 12, fp16): 12-chunk ranges of the
    matrix-core kernels cross sequence boundaries (256 chunks per sequence); the first, a
    middle and the last sequence checked."""
    w = W.WORKLOADS["mixer_2048"]
    x = W.make_inputs(w)
    _note("bwd mixer_2048 (sequences 0, 5, 11)")
    _run_case(oracle_mod, x, w.dtype, 0, chunk=w.chunk, bh=[0, 5, 11], seed=12)


def test_bwd_ranges_cross_sequences(oracle_mod):
    """201 chunks per sequence (67 x 192 grid, H = 3): two-chunk ranges, every other one
    straddling a sequence boundary; bf16, direction 3."""
    x = W.make_custom(1, 67, 192, 3, 64, 64, "bf16", seed=31)
    _note("bwd 201-chunk sequences")
    _run_case(oracle_mod, x, "bf16", 3, chunk=64, bh=[0, 1, 2], seed=13)


@pytest.mark.parametrize("shape", [(1, 48, 48, 3, "f16", 2), (1, 96, 96, 4, "bf16", 1)],
                         ids=["one-chunk-segments", "two-chunk-ranges"])
def test_forward_states_roundtrip(shape):
    """gla_fwd_states equals gla_fwd, and the backward given its states equals the
    backward that recomputes them, bit for bit (the same kernels on the same segments),
    with two launches fewer."""
    from gated_token_recurrence_amd import _lib
    B, gh, gw, H, dtype, direction = shape
    x = W.make_custom(B, gh, gw, H, 64, 64, dtype, seed=B + gh + H)
    t = inputs_to_dev(x, dtype)
    args = (t["q"], t["k"], t["v"], t["log_g"], t["z"], t["rms_w"])
    _note(f"forward states {shape}")
    ref = g.gla_fwd(*args, direction, chunk=64, path=_lib.PATH_MFMA)
    out, states = g.gla_fwd_states(*args, direction, chunk=64)
    torch.cuda.synchronize()
    assert states.numel() * 4 == g.gla_states_bytes(B, H, gh, gw, 64, 64, 64, t["q"].dtype)
    assert torch.equal(out, ref)
    dy = to_dev(W.cast_io(np.random.default_rng(4).standard_normal(x["v"].shape), dtype), dtype)
    a, na = g.gla_bwd(*args, dy, direction, chunk=64)
    b, nb = g.gla_bwd(*args, dy, direction, chunk=64, states=states)
    torch.cuda.synchronize()
    assert (na, nb) == (7, 5)
    for name in a:
        assert torch.equal(a[name], b[name]), name


def test_bwd_is_deterministic():
    x = W.make_custom(1, 10, 10, 2, 64, 64, "bf16", seed=5)
    t = inputs_to_dev(x, "bf16")
    dy = to_dev(W.cast_io(np.random.default_rng(2).standard_normal(x["v"].shape), "bf16"), "bf16")
    a, _ = g.gla_bwd(t["q"], t["k"], t["v"], t["log_g"], t["z"], t["rms_w"], dy, 3)
    b, _ = g.gla_bwd(t["q"], t["k"], t["v"], t["log_g"], t["z"], t["rms_w"], dy, 3)
    torch.cuda.synchronize()
    for name in a:
        assert torch.equal(a[name], b[name]), name
