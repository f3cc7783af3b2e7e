"""Key-only gated-linear-attention token mixer of GTR on MI355X (gfx950).

Python binding of libgtrscan (``include/gtrscan.h``).  torch supplies device
memory and the current stream; the mixer itself runs in the library's HIP
kernels.  ``gla_fwd`` is one block's mixer call, ``gla_stack_fwd`` a stack of
blocks with the direction cycle and the residual feed, ``gla_lowrank_fwd`` a
mixer call whose forget gate the library forms from rank-r gate features.
"""
from __future__ import annotations

import torch

from . import _lib
from ._lib import (GtrError, PATH_AUTO, PATH_FAST, PATH_MFMA, PATH_SERIAL)  # noqa: F401

__all__ = ["gla_fwd", "gla_fwd_states", "gla_states_bytes", "gla_stack_fwd", "gla_lowrank_fwd",
           "gla_bwd", "sswiglu_mix", "GtrError", "DIRECTIONS", "dtype_code", "version"]

DIRECTIONS = {"LR": 0, "RL": 1, "TB": 2, "BT": 3}
_DT = {torch.float32: _lib.GTR_F32, torch.float16: _lib.GTR_F16, torch.bfloat16: _lib.GTR_BF16}


def dtype_code(dt: torch.dtype) -> int:
    if dt not in _DT:
        raise TypeError(f"unsupported I/O dtype {dt}")
    return _DT[dt]


def version() -> int:
    return _lib.load().gtr_version()


def _dir(direction) -> int:
    return DIRECTIONS[direction] if isinstance(direction, str) else int(direction)


def _check_tensors(named, device):
    for name, t in named:
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def gla_fwd(q, k, v, log_g, z, rms_w, direction=0, chunk: int = 0, path: int = PATH_AUTO,
            out=None):
    """One mixer call.  q, k, log_g: [B, gh, gw, H, dk]; v, z: [B, gh, gw, H, dv];
    rms_w: [dv] float32; log_g float32; q, k, v, z one I/O dtype.  Returns out."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    B, gh, gw, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or log_g.shape != q.shape:
        raise ValueError("k and log_g must have q's shape")
    if v.shape != (B, gh, gw, H, dv) or z.shape != v.shape or rms_w.shape != (dv,):
        raise ValueError("v, z must be [B, gh, gw, H, dv] and rms_w [dv]")
    if not (q.dtype == k.dtype == v.dtype == z.dtype):
        raise TypeError("q, k, v, z must share one dtype")
    if log_g.dtype != torch.float32 or rms_w.dtype != torch.float32:
        raise TypeError("log_g and rms_w must be float32")
    if out is None:
        out = torch.empty_like(v)
    _check_tensors((("q", q), ("k", k), ("v", v), ("log_g", log_g), ("z", z),
                    ("rms_w", rms_w), ("out", out)), dev)
    if out.shape != v.shape or out.dtype != v.dtype:
        raise ValueError("out must match v")
    lib = _lib.load()
    with torch.cuda.device(dev):
        st = lib.gtr_gla_fwd_path(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_g.data_ptr(),
                                  z.data_ptr(), rms_w.data_ptr(), out.data_ptr(), B, H, gh, gw,
                                  dk, dv, _dir(direction), int(chunk), dtype_code(q.dtype),
                                  int(path), _stream_ptr(dev))
    _lib.check(st)
    return out


def gla_states_bytes(B, H, gh, gw, dk, dv, chunk, dtype) -> int:
    """Bytes of the forward segment states of this shape (0: the shape has none)."""
    return int(_lib.load().gtr_gla_states_bytes(B, H, gh, gw, dk, dv, int(chunk), dtype_code(dtype)))


def gla_fwd_states(q, k, v, log_g, z, rms_w, direction=0, chunk: int = 0):
    """``gla_fwd`` on the matrix-core path that also returns the forward segment states
    (a float32 tensor) for ``gla_bwd(..., states=...)``.  Returns (out, states)."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    B, gh, gw, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or log_g.shape != q.shape or v.shape != (B, gh, gw, H, dv) or \
            z.shape != v.shape or rms_w.shape != (dv,):
        raise ValueError("shape mismatch")
    if not (q.dtype == k.dtype == v.dtype == z.dtype):
        raise TypeError("q, k, v, z must share one dtype")
    if log_g.dtype != torch.float32 or rms_w.dtype != torch.float32:
        raise TypeError("log_g and rms_w must be float32")
    out = torch.empty_like(v)
    _check_tensors((("q", q), ("k", k), ("v", v), ("log_g", log_g), ("z", z),
                    ("rms_w", rms_w), ("out", out)), dev)
    nbytes = gla_states_bytes(B, H, gh, gw, dk, dv, chunk, q.dtype)
    if nbytes == 0:
        raise ValueError("this shape has no forward states (16-bit I/O, dk = dv = 64, chunk 64)")
    states = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
    lib = _lib.load()
    with torch.cuda.device(dev):
        st = lib.gtr_gla_fwd_states(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_g.data_ptr(),
                                    z.data_ptr(), rms_w.data_ptr(), out.data_ptr(), B, H, gh, gw,
                                    dk, dv, _dir(direction), int(chunk), dtype_code(q.dtype),
                                    states.data_ptr(), nbytes, _stream_ptr(dev))
    _lib.check(st)
    return out, states


def gla_stack_fwd(q, k, v, log_g, z, rms_w, first_direction=0, chunk: int = 0, out=None):
    """Stack of blocks: every tensor has a leading [n_blocks] dimension; rms_w is
    [n_blocks, dv].  Returns out [n_blocks, B, gh, gw, H, dv] (every block's output)."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    nb, B, gh, gw, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or log_g.shape != q.shape:
        raise ValueError("k and log_g must have q's shape")
    if v.shape != (nb, B, gh, gw, H, dv) or z.shape != v.shape or rms_w.shape != (nb, dv):
        raise ValueError("v, z must be [n, B, gh, gw, H, dv] and rms_w [n, dv]")
    if not (q.dtype == k.dtype == v.dtype == z.dtype):
        raise TypeError("q, k, v, z must share one dtype")
    if log_g.dtype != torch.float32 or rms_w.dtype != torch.float32:
        raise TypeError("log_g and rms_w must be float32")
    if out is None:
        out = torch.empty_like(v)
    _check_tensors((("q", q), ("k", k), ("v", v), ("log_g", log_g), ("z", z),
                    ("rms_w", rms_w), ("out", out)), dev)
    lib = _lib.load()
    with torch.cuda.device(dev):
        st = lib.gtr_gla_stack_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), log_g.data_ptr(),
                                   z.data_ptr(), rms_w.data_ptr(), out.data_ptr(), nb, B, H, gh,
                                   gw, dk, dv, _dir(first_direction), int(chunk),
                                   dtype_code(q.dtype), _stream_ptr(dev))
    _lib.check(st)
    return out


def gla_lowrank_fwd(q, k, v, feat, gate_w, gate_b, tau: float, z, rms_w, direction=0,
                    chunk: int = 0, path: int = PATH_AUTO, out=None, events=None):
    """One mixer call with the gate log g = logsigmoid(feat . gate_w + gate_b) / tau.

    feat: [B, gh, gw, r] and gate_w: [r, H*dk] of the I/O dtype; gate_b: [H*dk]
    float32; the rest as ``gla_fwd``.  ``events``: optional list of HIP event
    handles (ints) recorded around the launches.  Returns (out, n_launches).
    """
    import ctypes
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    B, gh, gw, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or v.shape != (B, gh, gw, H, dv) or z.shape != v.shape:
        raise ValueError("k must have q's shape; v, z must be [B, gh, gw, H, dv]")
    r = feat.shape[-1]
    if feat.shape != (B, gh, gw, r) or gate_w.shape != (r, H * dk) or gate_b.shape != (H * dk,):
        raise ValueError("feat [B, gh, gw, r], gate_w [r, H*dk], gate_b [H*dk] expected")
    if rms_w.shape != (dv,):
        raise ValueError("rms_w must be [dv]")
    if not (q.dtype == k.dtype == v.dtype == z.dtype == feat.dtype == gate_w.dtype):
        raise TypeError("q, k, v, z, feat, gate_w must share one dtype")
    if gate_b.dtype != torch.float32 or rms_w.dtype != torch.float32:
        raise TypeError("gate_b and rms_w must be float32")
    if out is None:
        out = torch.empty_like(v)
    _check_tensors((("q", q), ("k", k), ("v", v), ("feat", feat), ("gate_w", gate_w),
                    ("gate_b", gate_b), ("z", z), ("rms_w", rms_w), ("out", out)), dev)
    if out.shape != v.shape or out.dtype != v.dtype:
        raise ValueError("out must match v")
    n_ev = 0 if events is None else len(events)
    ev_arr = (ctypes.c_void_p * max(1, n_ev))(*(events or []))
    n_launch = ctypes.c_int(0)
    lib = _lib.load()
    with torch.cuda.device(dev):
        st = lib.gtr_gla_lowrank_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), feat.data_ptr(),
                                     gate_w.data_ptr(), gate_b.data_ptr(), float(tau), r,
                                     z.data_ptr(), rms_w.data_ptr(), out.data_ptr(), B, H, gh, gw,
                                     dk, dv, _dir(direction), int(chunk), dtype_code(q.dtype),
                                     int(path), ev_arr, n_ev, ctypes.byref(n_launch),
                                     _stream_ptr(dev))
    _lib.check(st)
    return out, n_launch.value


def sswiglu_mix(u, w_conv, b_conv, out=None):
    """Spatial SwiGLU middle: u [B, gh, gw, 2F] = [gate | value] (I/O dtype),
    w_conv [F, k, k] and b_conv [F] float32.  Returns m [B, gh, gw, F] =
    SiLU(gate) * (depthwise k x k convolution of value + b_conv)."""
    dev = u.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    B, gh, gw, F2 = u.shape
    F = F2 // 2
    if F2 != 2 * F or w_conv.dim() != 3 or w_conv.shape[0] != F or \
            w_conv.shape[1] != w_conv.shape[2] or b_conv.shape != (F,):
        raise ValueError("u [B, gh, gw, 2F], w_conv [F, k, k], b_conv [F] expected")
    if w_conv.dtype != torch.float32 or b_conv.dtype != torch.float32:
        raise TypeError("w_conv and b_conv must be float32")
    if out is None:
        out = torch.empty((B, gh, gw, F), dtype=u.dtype, device=dev)
    _check_tensors((("u", u), ("w_conv", w_conv), ("b_conv", b_conv), ("out", out)), dev)
    if out.shape != (B, gh, gw, F) or out.dtype != u.dtype:
        raise ValueError("out must be [B, gh, gw, F] of u's dtype")
    lib = _lib.load()
    with torch.cuda.device(dev):
        st = lib.gtr_sswiglu_mix(u.data_ptr(), w_conv.data_ptr(), b_conv.data_ptr(),
                                 out.data_ptr(), B, gh, gw, F, int(w_conv.shape[1]),
                                 dtype_code(u.dtype), _stream_ptr(dev))
    _lib.check(st)
    return out


def gla_bwd(q, k, v, log_g, z, rms_w, dout, direction=0, chunk: int = 0, events=None,
            states=None):
    """Backward pass of ``gla_fwd`` (same inputs, no residual) given dout = dL/dout.
    ``states``: the forward segment states from ``gla_fwd_states`` with the same inputs
    and arguments (skips their recomputation), or None.

    Returns (grads, n_launches) with grads a dict of dq, dk, dv (I/O dtype), dlog_g
    (float32), dz (I/O dtype) and drms_w ([dv] float32)."""
    import ctypes
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    B, gh, gw, H, dk = q.shape
    dv = v.shape[-1]
    if k.shape != q.shape or log_g.shape != q.shape or v.shape != (B, gh, gw, H, dv) or \
            z.shape != v.shape or dout.shape != v.shape or rms_w.shape != (dv,):
        raise ValueError("shape mismatch")
    if not (q.dtype == k.dtype == v.dtype == z.dtype == dout.dtype):
        raise TypeError("q, k, v, z, dout must share one dtype")
    if log_g.dtype != torch.float32 or rms_w.dtype != torch.float32:
        raise TypeError("log_g and rms_w must be float32")
    _check_tensors((("q", q), ("k", k), ("v", v), ("log_g", log_g), ("z", z),
                    ("rms_w", rms_w), ("dout", dout)), dev)
    if states is not None:
        if states.dtype != torch.float32:
            raise TypeError("states must be float32")
        _check_tensors((("states", states),), dev)
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
         "dlog_g": torch.empty_like(log_g), "dz": torch.empty_like(z),
         "drms_w": torch.empty_like(rms_w)}
    n_ev = 0 if events is None else len(events)
    ev_arr = (ctypes.c_void_p * max(1, n_ev))(*(events or []))
    n_launch = ctypes.c_int(0)
    lib = _lib.load()
    with torch.cuda.device(dev):
        st = lib.gtr_gla_bwd_states(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), log_g.data_ptr(), z.data_ptr(),
            rms_w.data_ptr(), dout.data_ptr(), g["dq"].data_ptr(), g["dk"].data_ptr(),
            g["dv"].data_ptr(), g["dlog_g"].data_ptr(), g["dz"].data_ptr(), g["drms_w"].data_ptr(),
            B, H, gh, gw, dk, dv, _dir(direction), int(chunk), dtype_code(q.dtype),
            None if states is None else states.data_ptr(),
            0 if states is None else states.numel() * 4, ev_arr, n_ev, ctypes.byref(n_launch),
            _stream_ptr(dev))
    _lib.check(st)
    return g, n_launch.value
