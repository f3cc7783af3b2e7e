"""GPU parity of the low-rank gate entry point (gtr_gla_lowrank_fwd) against the
fp64 oracle: log g = logsigmoid(feat . gate_w + gate_b) / tau, then the mixer.

Bar as for gtr_gla_fwd: 16-bit I/O within rel-L2 1e-3 and max-abs 2e-2 of the
oracle rounded to the I/O type; float32 I/O within rel-L2 1e-5.  The launch
count tells which way the call went: the gate formed inside the summary and
output kernels launches what a plain call on the matrix-core path launches;
log_g written out first adds the projection launch to the plain call's.
"""
import ctypes

import numpy as np
import pytest
import torch

import gated_token_recurrence_amd as g
from gated_token_recurrence_amd import _lib, workloads as W

from _helpers import assert_parity, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)


def _dev(x, dtype):
    t = {key: to_dev(x[key], dtype) for key in ("q", "k", "v", "z", "feat", "gate_w")}
    t["gate_b"] = torch.from_numpy(x["gate_b"]).cuda()
    t["rms_w"] = torch.from_numpy(x["rms_w"]).cuda()
    return t


def _run(x, dtype, direction, chunk=0, path=g.PATH_AUTO):
    t = _dev(x, dtype)
    out, n = g.gla_lowrank_fwd(t["q"], t["k"], t["v"], t["feat"], t["gate_w"], t["gate_b"],
                               x["tau"], t["z"], t["rms_w"], direction, chunk=chunk, path=path)
    torch.cuda.synchronize()
    return to_f64(out), n


def _oracle(oracle_mod, x, dtype, direction, bh=None):
    f = {key: W.io_to_f64(x[key], dtype) for key in ("q", "k", "v", "z", "feat", "gate_w")}
    return oracle_mod.fwd_lowrank(f["q"], f["k"], f["v"], f["feat"], f["gate_w"],
                                  x["gate_b"].astype(np.float64), x["tau"], f["z"],
                                  x["rms_w"].astype(np.float64), direction, bh=bh)


def _plain_launches(x, shape, direction, chunk, path):
    """Launches of a plain mixer call of the same shape on the path the low-rank call
    resolves to (under AUTO the matrix-core path where the shape has one, never the
    single launch)."""
    B, gh, gw, H, dk, dv, dtype = shape
    lib = _lib.load()
    if path == g.PATH_AUTO:
        auto = lib.gtr_gla_auto_path(B, H, gh, gw, dk, dv, chunk, W.DTYPE_CODE[dtype])
        path = g.PATH_SERIAL if auto == g.PATH_SERIAL else g.PATH_MFMA
    t = _dev(x, dtype)
    log_g = torch.full((B, gh, gw, H, dk), -0.1, dtype=torch.float32, device="cuda")
    out = torch.empty_like(t["v"])
    n = ctypes.c_int(0)
    _lib.check(lib.gtr_gla_fwd_events(
        t["q"].data_ptr(), t["k"].data_ptr(), t["v"].data_ptr(), log_g.data_ptr(),
        t["z"].data_ptr(), t["rms_w"].data_ptr(), out.data_ptr(), B, H, gh, gw, dk, dv,
        direction, chunk, W.DTYPE_CODE[dtype], path, None, 0, ctypes.byref(n),
        torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return n.value


def _case(oracle_mod, shape, direction=0, chunk=0, path=g.PATH_AUTO, rank=16, gate=None,
          seed=7, **kw):
    """gate: "fused" (formed in the kernels) or "written" (log_g written out first)."""
    B, gh, gw, H, dk, dv, dtype = shape
    x = W.make_lowrank(B, gh, gw, H, dk, dv, dtype, seed=seed, rank=rank, **kw)
    _note(f"lowrank {shape} dir={direction} chunk={chunk} path={path} rank={rank}")
    got, n = _run(x, dtype, direction, chunk=chunk, path=path)
    ref = _oracle(oracle_mod, x, dtype, direction)
    rel, mx = assert_parity(got, ref, dtype, oracle_mod, f"lowrank {shape}")
    if gate is not None:
        plain = _plain_launches(x, shape, direction, chunk,
                                g.PATH_MFMA if gate == "fused" else path)
        want = plain if gate == "fused" else plain + 1
        assert n == want, f"{n} launches, expected {want} (gate {gate})"
    return rel, mx


FUSED_SHAPES = [
    # B, gh, gw, H, dk, dv, dtype  (rank 16, chunk 64: gate formed in the kernels)
    (1, 17, 15, 2, 64, 64, "f16"),
    (1, 17, 15, 2, 64, 64, "bf16"),
    (3, 13, 9, 2, 64, 64, "bf16"),
    (2, 21, 13, 3, 64, 64, "f16"),
    (1, 1, 1, 2, 64, 64, "f16"),
    (1, 1, 70, 1, 64, 64, "bf16"),
    (1, 70, 1, 3, 64, 64, "f16"),
]


@pytest.mark.parametrize("shape", FUSED_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_fused_gate_shapes(oracle_mod, shape):
    _case(oracle_mod, shape, gate="fused")


@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_fused_gate_directions(oracle_mod, direction):
    _case(oracle_mod, (2, 19, 23, 2, 64, 64, "f16"), direction=direction, gate="fused")


@pytest.mark.parametrize("sc", [1, 3, 7])
def test_fused_gate_ranges_across_heads(oracle_mod, sc):
    """Short segments: workgroup ranges that cross several heads reload the head's
    projection at each crossing (summary and output kernels)."""
    lib = _lib.load()
    lib.gtr_set_segment_chunks(sc)
    try:
        _case(oracle_mod, (2, 16, 12, 3, 64, 64, "bf16"), direction=1, gate="fused")
        _case(oracle_mod, (1, 10, 10, 5, 64, 64, "f16"), direction=2, gate="fused")
    finally:
        lib.gtr_set_segment_chunks(0)


def test_fused_gate_saturated_and_fast_decaying_channels(oracle_mod):
    """Channels with g ~ 1 (bias +12) and channels whose decay over a chunk spans more
    than 64 log2 units (bias -14: the chunks run token by token)."""
    H, dk = 2, 64
    shift = np.zeros(H * dk)
    shift[::7] = 12.0
    shift[3::11] = -14.0
    _case(oracle_mod, (1, 20, 16, H, 64, 64, "f16"), direction=0, gate="fused", bias_shift=shift)
    _case(oracle_mod, (1, 20, 16, H, 64, 64, "bf16"), direction=3, gate="fused", bias_shift=shift)


@pytest.mark.parametrize("case", [
    # shape, chunk, path, rank
    ((1, 17, 15, 2, 64, 64, "f16"), 0, g.PATH_AUTO, 8),      # another rank
    ((1, 17, 15, 2, 64, 64, "bf16"), 0, g.PATH_AUTO, 1),
    ((1, 11, 13, 2, 64, 64, "f16"), 0, g.PATH_AUTO, 48),
    ((2, 12, 12, 2, 64, 128, "bf16"), 0, g.PATH_AUTO, 16),   # dv = 128
    ((1, 9, 10, 3, 64, 64, "f16"), 32, g.PATH_AUTO, 16),     # chunk 32
    ((1, 9, 7, 2, 32, 32, "f32"), 16, g.PATH_AUTO, 16),      # float32 I/O
    ((1, 6, 11, 2, 128, 64, "f32"), 64, g.PATH_AUTO, 5),
    ((1, 17, 15, 2, 64, 64, "f16"), 0, g.PATH_SERIAL, 16),
    ((1, 17, 15, 2, 64, 64, "bf16"), 0, g.PATH_FAST, 16),
], ids=lambda c: f"{'x'.join(map(str, c[0]))}-c{c[1]}-p{c[2]}-r{c[3]}")
def test_written_out_gate_paths(oracle_mod, case):
    shape, chunk, path, rank = case
    _case(oracle_mod, shape, chunk=chunk, path=path, rank=rank, gate="written")


def test_fused_gate_back_to_back_is_bitwise_stable(oracle_mod):
    x = W.make_lowrank(1, 24, 24, 3, 64, 64, "f16", seed=11)
    a, _ = _run(x, "f16", 1)
    for _ in range(2):
        b, _ = _run(x, "f16", 1)
        assert np.array_equal(a, b)


@pytest.mark.timeout(300)
def test_lowrank_mixer_2048_full_size(oracle_mod):
    """The 16.4K-token shapes (B 1, 128 x 128, H 12, fp16) with rank-16 gate inputs,
    all directions, in the configuration the benchmark times."""
    w = W.WORKLOADS["mixer_2048"]
    x = W.make_lowrank_inputs(w)
    for direction in range(4):
        _note(f"lowrank mixer_2048 direction {direction}")
        got, n = _run(x, w.dtype, direction, chunk=w.chunk)
        assert n == 3
        ref = _oracle(oracle_mod, x, w.dtype, direction)
        rel, mx = assert_parity(got, ref, w.dtype, oracle_mod, f"lowrank mixer_2048 dir {direction}")
        _note(f"  rel-L2 {rel:.2e} max-abs {mx:.2e}")
