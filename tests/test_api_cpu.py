"""Host-side checks of the C ABI (no GPU needed): exports, versions, argument errors."""
import ctypes
import os
import re

import pytest
import torch

from gated_token_recurrence_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = []
    for hdr in os.listdir(os.path.join(ROOT, "include")):
        if hdr.endswith(".h"):
            text = open(os.path.join(ROOT, "include", hdr)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"\b(gtr_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_functions()
    assert {"gtr_gla_fwd", "gtr_gla_stack_fwd", "gtr_last_error"} <= set(declared)
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in include/ but not exported"
    assert set(_lib.EXPORTS) == set(declared)


def test_version():
    assert _lib.load().gtr_version() == 100


P = [(i + 1) << 36 for i in range(7)]  # distinct far-apart fake pointers, never dereferenced


def _call(**kw):
    a = dict(B=1, H=2, gh=8, gw=8, dk=32, dv=32, direction=0, chunk=16, dtype=0)
    a.update(kw)
    lib = _lib.load()
    return lib.gtr_gla_fwd(*P, a["B"], a["H"], a["gh"], a["gw"], a["dk"], a["dv"],
                           a["direction"], a["chunk"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), _lib.GTR_ERR_ARG), (dict(H=-1), _lib.GTR_ERR_ARG),
    (dict(gh=0), _lib.GTR_ERR_ARG), (dict(direction=4), _lib.GTR_ERR_ARG),
    (dict(direction=-1), _lib.GTR_ERR_ARG), (dict(chunk=48), _lib.GTR_ERR_ARG),
    (dict(dtype=3), _lib.GTR_ERR_ARG), (dict(dk=48), _lib.GTR_ERR_UNSUPPORTED),
    (dict(dv=256), _lib.GTR_ERR_UNSUPPORTED),
])
def test_bad_arguments_are_rejected(kw, status):
    assert _call(**kw) == status
    assert _lib.last_error() != ""


def test_null_pointer_is_rejected():
    lib = _lib.load()
    st = lib.gtr_gla_fwd(None, *P[1:], 1, 1, 8, 8, 32, 32, 0, 0, 0, None)
    assert st == _lib.GTR_ERR_ARG and "null" in _lib.last_error()


def test_out_aliasing_input_is_rejected():
    lib = _lib.load()
    st = lib.gtr_gla_fwd(*P[:6], P[0], 1, 1, 8, 8, 32, 32, 0, 0, 0, None)
    assert st == _lib.GTR_ERR_ARG and "overlaps" in _lib.last_error()


def test_stack_rejects_bad_block_count():
    lib = _lib.load()
    st = lib.gtr_gla_stack_fwd(*P, 0, 1, 1, 8, 8, 32, 32, 0, 0, 0, None)
    assert st == _lib.GTR_ERR_ARG


def test_misaligned_element_is_rejected():
    lib = _lib.load()
    q = P[0] + 1  # an odd address for 16-bit elements
    st = lib.gtr_gla_fwd(q, *P[1:], 1, 1, 8, 8, 64, 64, 0, 0, _lib.GTR_F16, None)
    assert st == _lib.GTR_ERR_ARG and "aligned" in _lib.last_error()
    lg = P[3] + 2  # log_g is float32
    st = lib.gtr_gla_fwd(*P[:3], lg, *P[4:], 1, 1, 8, 8, 64, 64, 0, 0, _lib.GTR_F16, None)
    assert st == _lib.GTR_ERR_ARG and "aligned" in _lib.last_error()


@pytest.mark.parametrize("which", range(7))
def test_matrix_paths_need_16_byte_rows(which):
    # a row pointer off by 8 bytes (a contiguous view with a storage offset) is
    # refused by the explicit matrix-core and single-launch paths before any
    # device work; AUTO sends such a call to the token-serial path instead
    lib = _lib.load()
    ptrs = list(P)
    ptrs[which] += 8
    if which == 5:  # rms_w is read element by element: 8 bytes off is fine everywhere
        return
    for path in (_lib.PATH_MFMA, _lib.PATH_FAST):
        st = lib.gtr_gla_fwd_path(*ptrs, 1, 2, 8, 8, 64, 64, 0, 64, _lib.GTR_F16, path, None)
        assert st == _lib.GTR_ERR_UNSUPPORTED and "16-byte" in _lib.last_error(), (which, path)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device error path")
def test_misaligned_rows_still_reach_the_device_on_auto():
    lib = _lib.load()
    ptrs = list(P)
    ptrs[0] += 8
    st = lib.gtr_gla_fwd(*ptrs, 1, 2, 8, 8, 64, 64, 0, 64, _lib.GTR_F16, None)
    assert st == _lib.GTR_ERR_HIP  # accepted; fails only for want of a device


def test_stack_checks_paths_before_the_device():
    lib = _lib.load()
    ptrs = list(P)
    ptrs[1] += 8
    # AUTO inside a stack routes a misaligned stack to the token-serial path: the
    # call gets as far as the device check
    st = lib.gtr_gla_stack_fwd(*ptrs, 2, 1, 1, 8, 8, 64, 64, 0, 0, _lib.GTR_F16, None)
    assert st in (_lib.GTR_ERR_HIP, _lib.GTR_OK) or torch.cuda.device_count() > 0


def test_noalloc_refuses_calls_beyond_the_scratch():
    # 12 sequences of 16384 tokens on the token-serial path (float32 I/O): about
    # 50 MB of chunk states, more than the 32 MiB fixed scratch; refused before
    # any device work (the fake pointers are never touched)
    lib = _lib.load()
    st = lib.gtr_gla_fwd_noalloc(*P, 1, 12, 128, 128, 64, 64, 0, 64, _lib.GTR_F32, None)
    assert st == _lib.GTR_ERR_UNSUPPORTED and "scratch" in _lib.last_error()


@pytest.mark.parametrize("args,path", [
    # (B, H, grid_h, grid_w, dk, dv, chunk, dtype): batch one, at most 16 chunks per
    # sequence -> single launch; more chunks or batches -> three launches
    ((1, 12, 28, 28, 64, 64, 64, _lib.GTR_BF16), _lib.PATH_FAST),
    ((1, 12, 32, 32, 64, 64, 64, _lib.GTR_BF16), _lib.PATH_FAST),
    ((1, 12, 32, 34, 64, 64, 64, _lib.GTR_BF16), _lib.PATH_MFMA),
    ((1, 12, 8, 8, 64, 128, 32, _lib.GTR_F16), _lib.PATH_FAST),
    ((1, 12, 12, 32, 64, 64, 32, _lib.GTR_F16), _lib.PATH_FAST),
    ((1, 12, 13, 32, 64, 64, 32, _lib.GTR_F16), _lib.PATH_MFMA),
    ((1, 12, 24, 24, 64, 64, 32, _lib.GTR_BF16), _lib.PATH_MFMA),
    ((1, 12, 40, 40, 64, 64, 64, _lib.GTR_BF16), _lib.PATH_MFMA),
    ((2, 12, 16, 16, 64, 64, 64, _lib.GTR_BF16), _lib.PATH_MFMA),
    ((1, 12, 16, 16, 64, 64, 64, _lib.GTR_F32), _lib.PATH_SERIAL),
    ((1, 12, 16, 16, 32, 32, 64, _lib.GTR_BF16), _lib.PATH_SERIAL),
], ids=["fast-13-chunks", "fast-16-chunks", "mfma-17-chunks", "fast-64-dv128", "fast-12-chunks-of-32", "mfma-13-chunks-of-32", "mfma-18-chunks", "mfma-25-chunks", "mfma-batch",
        "serial-f32", "serial-dk32"])
def test_auto_path_choice(args, path):
    assert _lib.load().gtr_gla_auto_path(*args) == path, _lib.last_error()


def test_unknown_path_is_rejected():
    lib = _lib.load()
    st = lib.gtr_gla_fwd_path(*P, 1, 1, 8, 8, 32, 32, 0, 0, 0, 9, None)
    assert st == _lib.GTR_ERR_ARG


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device error path")
def test_valid_call_without_device_reports_hip_error():
    assert _call() == _lib.GTR_ERR_HIP
    assert "device" in _lib.last_error()


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "gated_token_recurrence_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b|gtr_oracle|libgtr_oracle",
                                     text, flags=re.M), f


PL = [(i + 1) << 36 for i in range(11)]  # q k v feat gate_w gate_b _ _ z rms_w out


def _lowrank(**kw):
    a = dict(tau=16.0, rank=16, B=1, H=2, gh=8, gw=8, dk=64, dv=64, direction=0, chunk=0,
             dtype=1, path=0, ptrs=None)
    a.update(kw)
    p = a["ptrs"] or PL
    lib = _lib.load()
    n = ctypes.c_int(-1)
    st = lib.gtr_gla_lowrank_fwd(p[0], p[1], p[2], p[3], p[4], p[5], a["tau"], a["rank"], p[8],
                                 p[9], p[10], a["B"], a["H"], a["gh"], a["gw"], a["dk"], a["dv"],
                                 a["direction"], a["chunk"], a["dtype"], a["path"], None, 0,
                                 ctypes.byref(n), None)
    return st, n.value


@pytest.mark.parametrize("kw", [
    dict(rank=0), dict(rank=257), dict(tau=0.0), dict(tau=-1.0), dict(tau=float("inf")),
    dict(tau=float("nan")), dict(B=0), dict(direction=5), dict(path=7), dict(chunk=24),
])
def test_lowrank_bad_arguments_are_rejected(kw):
    st, n = _lowrank(**kw)
    assert st == _lib.GTR_ERR_ARG, _lib.last_error()
    assert _lib.last_error() != "" and n == 0


def test_lowrank_null_and_misaligned_gate_pointers():
    for i in (3, 4, 5):
        p = list(PL)
        p[i] = None
        st, _ = _lowrank(ptrs=p)
        assert st == _lib.GTR_ERR_ARG and "null" in _lib.last_error()
        p = list(PL)
        p[i] = PL[i] + 8
        st, _ = _lowrank(ptrs=p)
        assert st == _lib.GTR_ERR_ARG and "aligned" in _lib.last_error()


def test_lowrank_out_aliasing_is_rejected():
    p = list(PL)
    p[10] = PL[3]  # out on top of feat
    st, _ = _lowrank(ptrs=p)
    assert st == _lib.GTR_ERR_ARG and "overlaps" in _lib.last_error()


def test_lowrank_events_need_an_array():
    lib = _lib.load()
    st = lib.gtr_gla_lowrank_fwd(*PL[:6], 16.0, 16, *PL[8:], 1, 2, 8, 8, 64, 64, 0, 0, 1, 0,
                                 None, 2, None, None)
    assert st == _lib.GTR_ERR_ARG


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="checks the no-device error path")
def test_lowrank_valid_call_without_device_reports_hip_error():
    st, n = _lowrank()
    assert st == _lib.GTR_ERR_HIP and n == 0


def _sswiglu(**kw):
    a = dict(B=1, gh=4, gw=4, F=16, k=3, dtype=1, ptrs=None)
    a.update(kw)
    p = a["ptrs"] or PL[:4]
    return _lib.load().gtr_sswiglu_mix(p[0], p[1], p[2], p[3], a["B"], a["gh"], a["gw"], a["F"],
                                       a["k"], a["dtype"], None)


@pytest.mark.parametrize("kw", [dict(B=0), dict(gh=-1), dict(F=0), dict(F=12), dict(k=2),
                                dict(k=9), dict(dtype=5)])
def test_sswiglu_bad_arguments_are_rejected(kw):
    assert _sswiglu(**kw) == _lib.GTR_ERR_ARG
    assert _lib.last_error() != ""


def test_sswiglu_null_misaligned_and_aliasing():
    p = list(PL[:4])
    p[1] = None
    assert _sswiglu(ptrs=p) == _lib.GTR_ERR_ARG and "null" in _lib.last_error()
    p = list(PL[:4])
    p[3] = PL[3] + 8
    assert _sswiglu(ptrs=p) == _lib.GTR_ERR_ARG and "aligned" in _lib.last_error()
    p = list(PL[:4])
    p[3] = PL[0] + 64
    assert _sswiglu(ptrs=p) == _lib.GTR_ERR_ARG and "overlaps" in _lib.last_error()


def test_states_sizes():
    """Forward segment states exist for 16-bit I/O at dk = dv = 64, chunk 64: one
    dk x dv float32 state per segment.  16.4K tokens, 12 heads: 3072 chunks in ranges of 6
    (512 starts), plus the 12 sequence starts, less the 4 starts both share = 520 segments."""
    lib = _lib.load()
    assert lib.gtr_gla_states_bytes(1, 12, 128, 128, 64, 64, 64, _lib.GTR_F16) == 520 * 64 * 64 * 4
    assert lib.gtr_gla_states_bytes(1, 12, 128, 128, 64, 64, 0, _lib.GTR_BF16) == 520 * 64 * 64 * 4
    for args in ((1, 12, 128, 128, 64, 64, 64, _lib.GTR_F32), (1, 12, 128, 128, 64, 128, 64, _lib.GTR_F16),
                 (1, 12, 128, 128, 64, 64, 32, _lib.GTR_F16), (0, 12, 128, 128, 64, 64, 64, _lib.GTR_F16)):
        assert lib.gtr_gla_states_bytes(*args) == 0, args


def test_states_argument_errors():
    lib = _lib.load()
    need = lib.gtr_gla_states_bytes(1, 2, 8, 8, 64, 64, 64, _lib.GTR_F16)
    assert need > 0
    S = 9 << 36
    # forward: null or short buffer, unsupported shape, buffer on top of an input
    st = lib.gtr_gla_fwd_states(*P, 1, 2, 8, 8, 64, 64, 0, 0, 1, None, need, None)
    assert st == _lib.GTR_ERR_ARG and "null states" in _lib.last_error()
    st = lib.gtr_gla_fwd_states(*P, 1, 2, 8, 8, 64, 64, 0, 0, 1, S, need - 4, None)
    assert st == _lib.GTR_ERR_ARG and "states buffer" in _lib.last_error()
    st = lib.gtr_gla_fwd_states(*P, 1, 2, 8, 8, 64, 64, 0, 32, 1, S, need, None)
    assert st == _lib.GTR_ERR_UNSUPPORTED
    st = lib.gtr_gla_fwd_states(*P, 1, 2, 8, 8, 64, 64, 0, 0, 1, P[2], need, None)
    assert st == _lib.GTR_ERR_ARG and "overlap" in _lib.last_error()
    # backward: short buffer, unsupported shape, a gradient on top of the states
    P13 = [(i + 1) << 36 for i in range(13)]
    st = lib.gtr_gla_bwd_states(*P13, 1, 2, 8, 8, 64, 64, 0, 0, 1, S, need - 4, None, 0, None, None)
    assert st == _lib.GTR_ERR_ARG and "states buffer" in _lib.last_error()
    st = lib.gtr_gla_bwd_states(*P13, 1, 2, 8, 8, 64, 64, 0, 0, 0, S, need, None, 0, None, None)
    assert st == _lib.GTR_ERR_UNSUPPORTED
    st = lib.gtr_gla_bwd_states(*P13, 1, 2, 8, 8, 64, 64, 0, 0, 1, P13[8], need, None, 0, None, None)
    assert st == _lib.GTR_ERR_ARG and "overlaps the states" in _lib.last_error()


def test_bwd_argument_errors():
    lib = _lib.load()
    P13 = [(i + 1) << 36 for i in range(13)]
    n = ctypes.c_int(-1)
    # null gradient
    args = list(P13)
    args[9] = None
    st = lib.gtr_gla_bwd(*args, 1, 2, 8, 8, 64, 64, 0, 0, 1, None, 0, ctypes.byref(n), None)
    assert st == _lib.GTR_ERR_ARG and "null" in _lib.last_error() and n.value == 0
    # a gradient on top of an input
    args = list(P13)
    args[7] = P13[0]
    st = lib.gtr_gla_bwd(*args, 1, 2, 8, 8, 64, 64, 0, 0, 1, None, 0, None, None)
    assert st == _lib.GTR_ERR_ARG and "overlaps" in _lib.last_error()
    # bad sizes and enums go through the forward's checks
    st = lib.gtr_gla_bwd(*P13, 1, 2, 8, 8, 48, 64, 0, 0, 1, None, 0, None, None)
    assert st == _lib.GTR_ERR_UNSUPPORTED
    st = lib.gtr_gla_bwd(*P13, 1, 2, 8, 8, 64, 64, 7, 0, 1, None, 0, None, None)
    assert st == _lib.GTR_ERR_ARG
