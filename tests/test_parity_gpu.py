"""GPU parity: libgtrscan (through its C ABI) against the fp64 oracle.

Bar: float32 I/O within rel-L2 1e-5 of the oracle; 16-bit I/O within rel-L2
1e-3 and max-abs 2e-2 of the oracle rounded to the I/O type.
"""
import numpy as np
import pytest
import torch

import gated_token_recurrence_amd as g
from gated_token_recurrence_amd import workloads as W

from _helpers import assert_parity, errors, inputs_f64, inputs_to_dev, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _note(msg):
    print(msg, flush=True)


def _run(x, dtype, direction, chunk=0, path=g.PATH_AUTO):
    t = inputs_to_dev(x, dtype)
    out = g.gla_fwd(t["q"], t["k"], t["v"], t["log_g"], t["z"], t["rms_w"], direction,
                    chunk=chunk, path=path)
    torch.cuda.synchronize()
    return to_f64(out)


def _oracle(oracle_mod, x, dtype, direction, bh=None):
    f = inputs_f64(x, dtype)
    return oracle_mod.fwd(f["q"], f["k"], f["v"], f["log_g"], f["z"], f["rms_w"], direction, bh=bh)


@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_tiny_fp32_all_directions(oracle_mod, direction):
    w = W.WORKLOADS["tiny"]
    x = W.make_inputs(w)
    _note(f"tiny fp32 direction={direction} chunk={w.chunk}")
    got = _run(x, w.dtype, direction, chunk=w.chunk)
    ref = _oracle(oracle_mod, x, w.dtype, direction)
    assert_parity(got, ref, w.dtype, oracle_mod, f"tiny dir {direction}")


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
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("path", [g.PATH_SERIAL])
def test_ragged_shapes(oracle_mod, shape, path):
    B, gh, gw, H, dk, dv, dtype, chunk = shape
    x = W.make_custom(B, gh, gw, H, dk, dv, dtype, seed=1 + SHAPES.index(shape))
    for direction in range(4):
        _note(f"shape {shape} path {path} direction {direction}")
        got = _run(x, dtype, direction, chunk=chunk, path=path)
        ref = _oracle(oracle_mod, x, dtype, direction)
        assert_parity(got, ref, dtype, oracle_mod, f"{shape} dir {direction}")


@pytest.mark.parametrize("chunk", [16, 32, 64, 128])
def test_chunk_sizes_agree(oracle_mod, chunk):
    x = W.make_custom(1, 20, 20, 2, 64, 64, "f32", seed=7)
    _note(f"chunk invariance chunk={chunk}")
    got = _run(x, "f32", 2, chunk=chunk, path=g.PATH_SERIAL)
    ref = _oracle(oracle_mod, x, "f32", 2)
    assert_parity(got, ref, "f32", oracle_mod, f"chunk {chunk}")


@pytest.mark.parametrize("log_g", [0.0, -1e-4, -20.0])
def test_extreme_gates(oracle_mod, log_g):
    x = W.make_custom(1, 16, 16, 2, 64, 64, "f32", seed=3, log_g_const=log_g)
    for direction in (0, 3):
        _note(f"constant log_g={log_g} direction={direction}")
        got = _run(x, "f32", direction, chunk=64, path=g.PATH_SERIAL)
        ref = _oracle(oracle_mod, x, "f32", direction)
        assert_parity(got, ref, "f32", oracle_mod, f"log_g {log_g}")


@pytest.mark.parametrize("name", ["mixer_640", "mixer_640_wide"])
def test_mixer_640_workloads(oracle_mod, name):
    w = W.WORKLOADS[name]
    x = W.make_inputs(w)
    ref_cache = {}
    for direction in range(4):
        _note(f"{name} direction {direction}")
        got = _run(x, w.dtype, direction, chunk=w.chunk)
        ref_cache[direction] = _oracle(oracle_mod, x, w.dtype, direction)
        rel, mx = assert_parity(got, ref_cache[direction], w.dtype, oracle_mod,
                                f"{name} dir {direction}")
        urel, _ = errors(got, ref_cache[direction], "f32", oracle_mod)
        _note(f"  rel-L2 {rel:.2e} (unrounded {urel:.2e}) max-abs {mx:.2e}")


def test_run_to_run_bitwise(oracle_mod):
    w = W.WORKLOADS["mixer_640"]
    x = W.make_inputs(w)
    _note("determinism mixer_640")
    a = _run(x, w.dtype, 1)
    for _ in range(3):
        assert np.array_equal(a, _run(x, w.dtype, 1))


def test_small_stack(oracle_mod):
    nb, B, gh, gw, H, dk, dv, dtype = 5, 2, 9, 10, 2, 64, 128, "bf16"
    blocks = [W.make_custom(B, gh, gw, H, dk, dv, dtype, seed=100 + i) for i in range(nb)]
    stk = {key: np.stack([b[key] for b in blocks]) for key in ("q", "k", "v", "z", "log_g", "rms_w")}
    t = inputs_to_dev(stk, dtype)
    _note("stack 5 blocks bf16")
    out = g.gla_stack_fwd(t["q"], t["k"], t["v"], t["log_g"], t["z"], t["rms_w"], 1, chunk=32)
    torch.cuda.synchronize()
    got = to_f64(out)
    refs = oracle_mod.stack_fwd([inputs_f64(b, dtype) for b in blocks], 1, dtype)
    for i in range(nb):
        assert_parity(got[i], refs[i], dtype, oracle_mod, f"stack block {i}")
