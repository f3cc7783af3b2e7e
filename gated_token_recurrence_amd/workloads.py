"""Seeded synthetic workloads for the Key-only GLA token mixer.

This module only draws random numbers and casts them to the I/O element type.
It holds none of the mixer's arithmetic, so the fp64 oracle (under ``oracle/``)
and the HIP path can both be fed from it without sharing any method code.

Shapes follow the GTR write-up ("端侧实时感知新标杆！通用线性骨干网络GTR开源"):
Method §1 gives the stride-16 patch grid and the 12-block stack, Method §4
the two kernel-benchmark lengths (about 1.6K and 16.4K tokens).  The pages fix
no head count, head width, batch or value distribution; the values below are
the workload definitions this library is measured on.

Layout of every tensor is token-major grid order ``[B, grid_h, grid_w, H, d]``.
I/O tensors are returned as numpy arrays of the I/O type; bf16 (which numpy
lacks) is carried as ``uint16`` bit patterns.  ``log_g`` and ``rms_w`` are
always float32.

Recipe (per workload, per block of a stack):
  rng = numpy.random.Generator(PCG64(seed)), seed = 1000 * workload_id + block
  draw order: q, k, v, z, x_gate, rms_w, then the saturated-channel mask
  q, k, v, z = scale * N(0, 1), drawn in float64 and rounded to the I/O type
  log_g = float32(logsigmoid(x_gate) / 16), x_gate ~ N(0, 1)
  rms_w = 1 (tiny workload) or 1 + 0.1 * N(0, 1)
  saturated (wide mixer only): round(0.1 * H * dk) of the (h, c) key channels,
  chosen without replacement, get log_g = -1e-4 * U[0, 1) for every token.

Low-rank gate inputs (the gate formed inside the library from rank-r
features; GTR paper, Method §1):
  seed = 1000 * workload_id + 500 + block; draw order: q, k, v, z, feat,
  gate_w, gate_b, rms_w
  feat ~ N(0, 1) [B, grid_h, grid_w, r] and gate_w ~ N(0, 1) / sqrt(r)
  [r, H * dk], both rounded to the I/O type; gate_b ~ N(0, 0.5^2) float32
  [H * dk], plus an optional per-channel shift; tau = 16, r = 16.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

DTYPES = ("f32", "f16", "bf16")
DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
DTYPE_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
DIRECTIONS = ("LR", "RL", "TB", "BT")


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int            # workload id, used in the seed
    name: str
    B: int
    grid_h: int
    grid_w: int
    H: int
    dk: int
    dv: int
    dtype: str
    scale: float        # std of q, k, v, z
    unit_rms_w: bool
    chunk: int
    n_blocks: int = 1
    saturated_frac: float = 0.0

    @property
    def L(self) -> int:
        return self.grid_h * self.grid_w

    @property
    def tokens(self) -> int:
        return self.B * self.L

    def compulsory_bytes(self, residual: bool = False) -> int:
        """Bytes one call must move: q, k, v, z read, out written, fp32 log_g read."""
        s = DTYPE_BYTES[self.dtype]
        per = (2 * self.dk + 3 * self.dv) * s + 4 * self.dk
        if residual:
            per += self.dv * s
        return self.B * self.L * self.H * per + 4 * self.dv

    def compulsory_bytes_lowrank(self, rank: int = 16) -> int:
        """Bytes of one call with the gate formed from rank-r features: q, k, v, z
        read and out written per token-head, the features per token, the
        projection and bias once."""
        s = DTYPE_BYTES[self.dtype]
        per_th = (2 * self.dk + 3 * self.dv) * s
        return (self.B * self.L * (self.H * per_th + rank * s)
                + rank * self.H * self.dk * s + 4 * self.H * self.dk + 4 * self.dv)

    def algorithmic_flops(self, chunk: int | None = None) -> int:
        """Chunkwise work: K^T V summary, Q.S_prev, causal scores and P.V."""
        c = chunk or self.chunk
        per = 4 * self.dk * self.dv + (c + 1) * (self.dk + self.dv)
        return self.B * self.L * self.H * per


WORKLOADS = {
    "tiny": Workload(0, "tiny", 1, 8, 8, 2, 32, 32, "f32", 1.0, True, 16),
    "mixer_640": Workload(1, "mixer_640", 1, 40, 40, 6, 64, 64, "f16", 1 / 8, False, 64),
    "mixer_640_wide": Workload(2, "mixer_640_wide", 1, 40, 40, 16, 64, 64, "bf16", 1 / 8,
                               False, 64, saturated_frac=0.1),
    "mixer_2048": Workload(3, "mixer_2048", 1, 128, 128, 12, 64, 64, "f16", 1 / 8, False, 64),
    "stack_1024": Workload(4, "stack_1024", 8, 64, 64, 12, 64, 128, "bf16", 1 / 8, False, 64,
                           n_blocks=12),
}


# ---------------------------------------------------------------- casting --
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def cast_io(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Cast a float64 draw to the I/O representation (bf16 as uint16 bits)."""
    if dtype == "f32":
        return x64.astype(np.float32)
    if dtype == "f16":
        return x64.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x64.astype(np.float32))
    raise ValueError(dtype)


def io_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of an I/O array to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a).astype(np.float64)


def logsigmoid_over(x: np.ndarray, temp: float) -> np.ndarray:
    """float32(log(sigmoid(x)) / temp), evaluated stably in float64."""
    ls = -(np.maximum(-x, 0.0) + np.log1p(np.exp(-np.abs(x))))
    return (ls / temp).astype(np.float32)


# ------------------------------------------------------------- generation --
def make_inputs(w: Workload, block: int = 0, seed: int | None = None,
                B: int | None = None) -> dict:
    """Draw one block's inputs.  ``B`` may override the batch (used for reduced tests)."""
    Bn = w.B if B is None else B
    rng = np.random.Generator(np.random.PCG64(1000 * w.wid + block if seed is None else seed))
    qk_shape = (Bn, w.grid_h, w.grid_w, w.H, w.dk)
    v_shape = (Bn, w.grid_h, w.grid_w, w.H, w.dv)
    out = {}
    for name, shape in (("q", qk_shape), ("k", qk_shape), ("v", v_shape), ("z", v_shape)):
        out[name] = cast_io(rng.standard_normal(shape) * w.scale, w.dtype)
    x_gate = rng.standard_normal(qk_shape)
    log_g = logsigmoid_over(x_gate, 16.0)
    if w.unit_rms_w:
        rms_w = np.ones(w.dv, dtype=np.float32)
    else:
        rms_w = (1.0 + 0.1 * rng.standard_normal(w.dv)).astype(np.float32)
    if w.saturated_frac > 0:
        n_ch = w.H * w.dk
        n_sat = int(round(w.saturated_frac * n_ch))
        chans = rng.choice(n_ch, size=n_sat, replace=False)
        u = rng.random((Bn, w.grid_h, w.grid_w, n_sat))
        flat = log_g.reshape(Bn, w.grid_h, w.grid_w, n_ch)
        flat[..., chans] = (-1e-4 * u).astype(np.float32)
        log_g = flat.reshape(qk_shape)
    out["log_g"] = np.ascontiguousarray(log_g, dtype=np.float32)
    out["rms_w"] = rms_w
    return out


def make_custom(B: int, grid_h: int, grid_w: int, H: int, dk: int, dv: int, dtype: str,
                seed: int, scale: float = 0.125, gate_temp: float = 16.0,
                log_g_const: float | None = None) -> dict:
    """Inputs for parity and edge-case tests at arbitrary shapes."""
    w = Workload(-1, "custom", B, grid_h, grid_w, H, dk, dv, dtype, scale, False, 64)
    rng = np.random.Generator(np.random.PCG64(seed))
    qk_shape = (B, grid_h, grid_w, H, dk)
    v_shape = (B, grid_h, grid_w, H, dv)
    out = {}
    for name, shape in (("q", qk_shape), ("k", qk_shape), ("v", v_shape), ("z", v_shape)):
        out[name] = cast_io(rng.standard_normal(shape) * scale, dtype)
    x_gate = rng.standard_normal(qk_shape)
    if log_g_const is None:
        out["log_g"] = np.ascontiguousarray(logsigmoid_over(x_gate, gate_temp))
    else:
        out["log_g"] = np.full(qk_shape, log_g_const, dtype=np.float32)
    out["rms_w"] = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    out["_workload"] = w
    return out


def make_lowrank(B: int, grid_h: int, grid_w: int, H: int, dk: int, dv: int, dtype: str,
                 seed: int, rank: int = 16, tau: float = 16.0, scale: float = 0.125,
                 feat_scale: float = 1.0, bias_shift=None) -> dict:
    """Inputs of a call whose gate comes from rank-r features.

    ``bias_shift``: optional float array [H * dk] added to gate_b (saturated
    channels take a large positive shift, fast-decaying ones a negative one).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    qk_shape = (B, grid_h, grid_w, H, dk)
    v_shape = (B, grid_h, grid_w, H, dv)
    out = {}
    for name, shape in (("q", qk_shape), ("k", qk_shape), ("v", v_shape), ("z", v_shape)):
        out[name] = cast_io(rng.standard_normal(shape) * scale, dtype)
    out["feat"] = cast_io(rng.standard_normal((B, grid_h, grid_w, rank)) * feat_scale, dtype)
    out["gate_w"] = cast_io(rng.standard_normal((rank, H * dk)) / math.sqrt(rank), dtype)
    b = rng.standard_normal(H * dk) * 0.5
    if bias_shift is not None:
        b = b + np.asarray(bias_shift, dtype=np.float64)
    out["gate_b"] = b.astype(np.float32)
    out["tau"] = float(tau)
    out["rms_w"] = (1.0 + 0.1 * rng.standard_normal(dv)).astype(np.float32)
    return out


def make_lowrank_inputs(w: Workload, block: int = 0, rank: int = 16, tau: float = 16.0,
                        B: int | None = None) -> dict:
    """A workload's shapes with low-rank gate inputs (seed 1000 * id + 500 + block)."""
    Bn = w.B if B is None else B
    return make_lowrank(Bn, w.grid_h, w.grid_w, w.H, w.dk, w.dv, w.dtype,
                        seed=1000 * w.wid + 500 + block, rank=rank, tau=tau, scale=w.scale)


@dataclasses.dataclass(frozen=True)
class SSwiGLUWorkload:
    """Shapes of the Spatial SwiGLU middle: u = [B, grid_h, grid_w, 2F] in, m = [.., F] out."""
    wid: int
    name: str
    B: int
    grid_h: int
    grid_w: int
    F: int
    k: int
    dtype: str

    @property
    def tokens(self) -> int:
        return self.B * self.grid_h * self.grid_w

    def compulsory_bytes(self) -> int:
        """u read once, m written once, kernel taps and bias once."""
        s = DTYPE_BYTES[self.dtype]
        return self.tokens * 3 * self.F * s + self.F * (self.k * self.k + 1) * 4


SSWIGLU_WORKLOADS = {
    # 12-block backbone shapes at 1024 x 1024 (stride 16), width 768, SwiGLU hidden 2048
    "sswiglu_1024": SSwiGLUWorkload(10, "sswiglu_1024", 8, 64, 64, 2048, 3, "bf16"),
    # 640 x 640 input, batch one
    "sswiglu_640": SSwiGLUWorkload(11, "sswiglu_640", 1, 40, 40, 2048, 3, "f16"),
}


def make_sswiglu(B: int, grid_h: int, grid_w: int, F: int, k: int, dtype: str, seed: int) -> dict:
    """Inputs of the Spatial SwiGLU middle.  Draw order: u, w_conv, b_conv.
    u ~ N(0, 1) rounded to the I/O type; w_conv ~ N(0, 1) / k float32 [F, k, k];
    b_conv ~ N(0, 0.1^2) float32 [F]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = {"u": cast_io(rng.standard_normal((B, grid_h, grid_w, 2 * F)), dtype)}
    out["w_conv"] = (rng.standard_normal((F, k, k)) / k).astype(np.float32)
    out["b_conv"] = (0.1 * rng.standard_normal(F)).astype(np.float32)
    return out


def make_sswiglu_inputs(w: SSwiGLUWorkload) -> dict:
    return make_sswiglu(w.B, w.grid_h, w.grid_w, w.F, w.k, w.dtype, seed=1000 * w.wid)


def rotation_sets(bytes_per_set: int, min_total: int = 512 << 20) -> int:
    """Number of buffer sets needed so repeated calls do not re-read the 256 MB cache."""
    return max(1, math.ceil(min_total / max(1, bytes_per_set)))
