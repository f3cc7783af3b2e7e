"""fp64 CPU oracle for the Key-only GLA token mixer -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this package.  The library's product path never imports it, and it imports
nothing from the library: inputs come in as plain numpy arrays.

``fwd`` is the single mixer call (the step recurrence of the GTR write-up
"端侧实时感知新标杆！通用线性骨干网络GTR开源", Method §1, evaluated token by
token in double precision by ``gtr_oracle.c``).  ``stack_fwd`` chains blocks:
block i scans in direction (first + i) mod 4 (Method §1: LR, RL, TB, BT cycle
with depth) and takes ``v_i + out_{i-1}``, rounded to the I/O type, as its
value input (the residual feed of the stacked workload).

``lowrank_log_g`` forms the forget gate from rank-r gate features (Method §1:
a light low-rank projection of the input with a temperature; rank and
temperature are lost on the page, the library takes them as arguments):
x = feat W + b per head channel, log g = logsigmoid(x) / tau.  ``fwd_lowrank``
is ``fwd`` with that gate.

``sswiglu_mix`` is the fused middle of the Spatial SwiGLU feed-forward block
(Method §2: in the channel expansion the value branch is reshaped to the 2-D
grid and mixed by a depthwise convolution; the page's kernel size was lost):
from the expanded projection u = [gate | value], m = SiLU(gate) * (DWConv(value)
+ bias), zero padding, cross-correlation as in common deep-learning
frameworks.

``backward.bwd`` (module ``oracle.backward``) is the fp64 backward pass of one
mixer call, written from the chain rule.

``round_io`` is this package's own IEEE round-to-nearest-even to the I/O type.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gtr_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgtr_oracle.so")
_lib = None

RMS_EPS = 1e-5  # RMSNorm epsilon: the page gives none; this is the library convention


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, no FP contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-fno-fast-math", "-std=c11", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.gtr_oracle_fwd.restype = ctypes.c_int
        lib.gtr_oracle_fwd.argtypes = [dp] * 7 + [ctypes.c_int] * 7 + [
            ctypes.c_double, ctypes.c_int, ctypes.POINTER(ctypes.c_int64), ctypes.c_int64]
        lib.gtr_oracle_threads.restype = ctypes.c_int
        lib.gtr_oracle_set_threads.restype = None
        lib.gtr_oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def threads() -> int:
    return _load().gtr_oracle_threads()


def set_threads(n: int) -> None:
    """Threads of later oracle calls (the OpenMP runtime's setting)."""
    _load().gtr_oracle_set_threads(int(n))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def fwd(q, k, v, log_g, z, rms_w, direction: int, eps: float = RMS_EPS,
        epilogue: bool = True, bh=None) -> np.ndarray:
    """One mixer call in fp64.  Arrays are float64 (or exactly widened), grid order.

    ``bh``: optional iterable of b*H + h sequence indices to compute; the other
    outputs are NaN.
    """
    q, k, v, log_g = _f64(q), _f64(k), _f64(v), _f64(log_g)
    B, gh, gw, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or log_g.shape != q.shape or v.shape[:4] != q.shape[:4]:
        raise ValueError("shape mismatch")
    zz = _f64(z) if epilogue else np.zeros(1)
    ww = _f64(rms_w) if epilogue else np.zeros(1)
    out = np.full(v.shape, np.nan) if bh is not None else np.zeros(v.shape)
    if bh is not None:
        bh_arr = np.ascontiguousarray(np.asarray(list(bh), dtype=np.int64))
        bh_ptr, n_bh = bh_arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), len(bh_arr)
    else:
        bh_arr, bh_ptr, n_bh = None, None, 0
    rc = _load().gtr_oracle_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(zz), _ptr(ww),
                                _ptr(out), B, H, gh, gw, dk, dv, int(direction), float(eps),
                                1 if epilogue else 0, bh_ptr, n_bh)
    if rc != 0:
        raise RuntimeError("oracle rejected its arguments")
    return out


# ------------------------------------------------------------ low-rank gate --
def logsigmoid(x) -> np.ndarray:
    """log(1 / (1 + exp(-x))) in float64, without overflow for either sign:
    log sigma(x) = min(x, 0) - log(1 + exp(-|x|))."""
    x = _f64(x)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def lowrank_log_g(feat, gate_w, gate_b, tau: float, H: int, dk: int) -> np.ndarray:
    """Forget gate from rank-r features (Method §1, the gate projection).

    feat: [B, gh, gw, r] (one feature vector per token, shared by the heads);
    gate_w: [r, H*dk]; gate_b: [H*dk]; tau > 0.  Head h, key channel c takes
    column h*dk + c:  log_g[..., h, c] = logsigmoid(feat . gate_w[:, h*dk + c]
    + gate_b[h*dk + c]) / tau.  Returns float64 [B, gh, gw, H, dk].
    """
    feat, gate_w, gate_b = _f64(feat), _f64(gate_w), _f64(gate_b)
    r = feat.shape[-1]
    if gate_w.shape != (r, H * dk) or gate_b.shape != (H * dk,) or not tau > 0:
        raise ValueError("gate shapes or temperature")
    x = feat @ gate_w + gate_b                      # [B, gh, gw, H*dk]
    return (logsigmoid(x) / float(tau)).reshape(feat.shape[:-1] + (H, dk))


def fwd_lowrank(q, k, v, feat, gate_w, gate_b, tau, z, rms_w, direction: int,
                eps: float = RMS_EPS, bh=None) -> np.ndarray:
    """``fwd`` with the gate formed by ``lowrank_log_g`` (never rounded)."""
    H, dk = q.shape[3], q.shape[4]
    return fwd(q, k, v, lowrank_log_g(feat, gate_w, gate_b, tau, H, dk), z, rms_w,
               direction, eps=eps, bh=bh)


# -------------------------------------------------------------- S-SwiGLU mix --
def depthwise_conv2d(val, w, b) -> np.ndarray:
    """Depthwise k x k cross-correlation on the grid, zero padding, 'same' size.

    val: [B, gh, gw, F] (channels last); w: [F, k, k] (k odd); b: [F].
    out[., y, x, f] = b[f] + sum_{i, j} w[f, i, j] * val[., y + i - k//2, x + j - k//2, f]
    """
    val, w, b = _f64(val), _f64(w), _f64(b)
    F, k, k2 = w.shape
    if k != k2 or k % 2 != 1 or val.shape[-1] != F or b.shape != (F,):
        raise ValueError("conv shapes")
    r = k // 2
    B, gh, gw, _ = val.shape
    vp = np.pad(val, ((0, 0), (r, r), (r, r), (0, 0)))
    out = np.broadcast_to(b, val.shape).copy()
    for i in range(k):
        for j in range(k):
            out += w[:, i, j] * vp[:, i:i + gh, j:j + gw, :]
    return out


def sswiglu_mix(u, w, b) -> np.ndarray:
    """Spatial SwiGLU middle (Method §2): u = [B, gh, gw, 2F] = [gate | value];
    returns m = SiLU(gate) * depthwise_conv2d(value, w, b) in float64."""
    u = _f64(u)
    F = u.shape[-1] // 2
    if u.shape[-1] != 2 * F:
        raise ValueError("u must hold gate and value halves")
    gate, val = u[..., :F], u[..., F:]
    silu = gate / (1.0 + np.exp(-gate))
    return silu * depthwise_conv2d(val, w, b)


# ------------------------------------------------------------------ rounding --
_FORMATS = {
    # (significand bits incl. the implicit one, smallest quantum exponent, largest finite)
    "f32": (24, -149, (2.0 - 2.0 ** -23) * 2.0 ** 127),
    "f16": (11, -24, 65504.0),
    "bf16": (8, -133, (2.0 - 2.0 ** -7) * 2.0 ** 127),
}


def round_io(x, dtype: str) -> np.ndarray:
    """Round float64 values to the I/O type (nearest, ties to even); return float64.

    Written from the IEEE 754 definition: the quantum of a value with binary
    exponent e (x = m * 2**e, 0.5 <= |m| < 1) is 2**(e - p), clamped below at
    the format's subnormal quantum; beyond the largest finite value the result
    overflows to infinity.
    """
    p, qmin, big = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    qexp = np.maximum(e.astype(np.int64) - p, qmin)
    scale = np.ldexp(1.0, qexp)
    r = np.rint(x / scale) * scale          # np.rint rounds half to even
    r = np.where(np.abs(r) > big, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def stack_fwd(blocks, first_direction: int, dtype: str, eps: float = RMS_EPS, bh=None):
    """Chain of mixer calls.  ``blocks`` is a list of dicts with float64 q, k, v,
    log_g, z, rms_w.  Returns the list of fp64 outputs (before rounding); the
    value fed forward is the rounded output, as the library stores it."""
    outs = []
    prev = None
    for i, blk in enumerate(blocks):
        v = _f64(blk["v"])
        if prev is not None:
            v = round_io(v + round_io(prev, dtype), dtype)
        o = fwd(blk["q"], blk["k"], v, blk["log_g"], blk["z"], blk["rms_w"],
                (first_direction + i) % 4, eps=eps, bh=bh)
        outs.append(o)
        prev = o
    return outs
