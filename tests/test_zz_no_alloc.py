"""gtr_gla_fwd_noalloc (the entry point that allocates nothing) against gtr_gla_fwd.

Both are called through the C ABI on the same device inputs.  The no-allocation
call keeps its states in the library's fixed device scratch and takes the
matrix-core path wherever gtr_gla_fwd's AUTO takes the matrix-core or the
single-launch path (the token-serial path otherwise), so its outputs must equal
gtr_gla_fwd_path's on that path bit for bit (same kernels, same plan), and
gtr_gla_fwd's within the oracle bar.  Calls in a row, each smaller than the one
before, show that the shared scratch carries nothing from one call into the
next; the smaller ones also meet the oracle bar.
"""
import ctypes

import numpy as np
import pytest
import torch

from gated_token_recurrence_amd import _lib, workloads as W

from _helpers import assert_parity, inputs_f64, inputs_to_dev, to_f64

pytestmark = pytest.mark.gpu

DT = {"f32": _lib.GTR_F32, "f16": _lib.GTR_F16, "bf16": _lib.GTR_BF16}


def _call(fn, t, shape, direction, chunk, dtype, *path):
    B, gh, gw, H, dk, dv = shape
    out = torch.empty_like(t["v"])
    st = fn(t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), t["log_g"].data_ptr(),
            t["z"].data_ptr(), t["rms_w"].data_ptr(), out.data_ptr(), B, H, gh, gw, dk, dv,
            direction, chunk, DT[dtype], *path, torch.cuda.current_stream().cuda_stream)
    _lib.check(st)
    return out


CASES = [
    # (B, gh, gw, H, dk, dv), dtype, chunk, direction: the 16.4K-token workload
    # (matrix-core path, 8.7 MB of states), then smaller calls on both paths; the
    # 576-token batch-one call is one gtr_gla_fwd sends to the single-launch path
    ((1, 128, 128, 12, 64, 64), "f16", 64, 0),
    ((1, 40, 40, 6, 64, 64), "f16", 64, 2),
    ((2, 12, 12, 2, 64, 128), "bf16", 64, 3),
    ((1, 24, 24, 4, 64, 64), "bf16", 64, 1),
    ((1, 8, 8, 2, 32, 32), "f32", 16, 1),
]


def test_noalloc_equals_gtr_gla_fwd_two_calls(oracle_mod):
    lib = _lib.load()
    for i, (shape, dtype, chunk, direction) in enumerate(CASES):
        print(f"no-alloc case {i}: shape {shape} {dtype} chunk {chunk} direction {direction}",
              flush=True)
        x = W.make_custom(*shape, dtype, seed=900 + i)
        t = inputs_to_dev(x, dtype)
        B, gh, gw, H, dk, dv = shape
        auto = lib.gtr_gla_auto_path(B, H, gh, gw, dk, dv, chunk, DT[dtype])
        assert auto >= 0, _lib.last_error()
        if i == 3:
            assert auto == _lib.PATH_FAST, "the batch-one case should take the single-launch path"
        path = _lib.PATH_SERIAL if auto == _lib.PATH_SERIAL else _lib.PATH_MFMA
        ref = _call(lib.gtr_gla_fwd_path, t, shape, direction, chunk, dtype, path)
        fwd = _call(lib.gtr_gla_fwd, t, shape, direction, chunk, dtype)
        got = _call(lib.gtr_gla_fwd_noalloc, t, shape, direction, chunk, dtype)
        again = _call(lib.gtr_gla_fwd_noalloc, t, shape, direction, chunk, dtype)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"case {i}: differs from gtr_gla_fwd_path({path})"
        assert torch.equal(again, ref), f"case {i}: second call differs"
        if auto == path:
            assert torch.equal(got, fwd), f"case {i}: differs from gtr_gla_fwd"
        if i > 0:  # the smaller calls also against the oracle, as is gtr_gla_fwd's output
            f = inputs_f64(x, dtype)
            r = oracle_mod.fwd(f["q"], f["k"], f["v"], f["log_g"], f["z"], f["rms_w"], direction)
            assert_parity(to_f64(got), r, dtype, oracle_mod, f"no-alloc case {i}")
            assert_parity(to_f64(fwd), r, dtype, oracle_mod, f"gtr_gla_fwd case {i}")
