"""fp64 CPU oracle for the Kimi Delta Attention (KDA) forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import, call, link or execute anything in
this package.  The product path (the HIP library and its binding) never does,
and the oracle shares no code with it.

Contents
  kda_oracle.c   token-by-token fp64 recurrence (C, OpenMP over independent
                 (sequence, head, column-block) units) -- the definition.
  reference.py   NumPy fp64 twin of the recurrence, and the chunkwise WY / UT
                 form written step by step from the derivation, used to pin
                 the recurrence.
  layer.py       fp64 definitions of the layer's elementwise steps around the
                 recurrence (q/k L2 norm, log sigmoid and sigmoid of logits,
                 RMS norm x weight x sigmoid output gate), pinned by
                 ``tests/test_oracle_layer.py``.
  backward.py    gradients of the forward: autograd of the recurrence (pinned
                 to finite differences) and the hand-derived backward of the
                 chunkwise form (pinned to autograd), ``tests/test_oracle_backward.py``.
  build.py       gcc build of the C oracle.

Every function is pinned by ``tests/test_oracle_pins.py`` against closed
forms, special cases and the worked values printed on the pages (fixtures in
``tests/golden/``).  For generic decaying inputs the pages print no numeric
KDA output, so there the recurrence is pinned by agreement with the
independently written chunkwise form.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import backward, layer, reference  # noqa: F401  (re-export)
from .reference import chunkwise, recurrent, decode_step as decode_step_np  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def load_c_oracle(build_if_missing: bool = True):
    """Load (building with gcc if needed) the C oracle library."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(os.path.join(_HERE, "kda_oracle.c"))):
        if not build_if_missing:
            raise FileNotFoundError(_LIB_PATH)
        from .build import build
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.kda_oracle_prefill.restype = ctypes.c_int
    lib.kda_oracle_prefill.argtypes = [
        ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, dp, dp, dp, dp, dp, ctypes.c_double, dp, dp, dp,
        ctypes.c_int32, ctypes.c_int32]
    lib.kda_oracle_decode_step.restype = ctypes.c_int
    lib.kda_oracle_decode_step.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        dp, dp, dp, dp, dp, ctypes.c_double, dp, dp, ctypes.c_int32]
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    lib.kda_oracle_max_threads.argtypes = []
    _lib = lib
    return lib


def _c64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def prefill(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None,
            col_block=32, n_threads=0):
    """C fp64 recurrence over packed tokens; returns (o, final_state).

    q, k, g: [T, H, d_k]; v: [T, H, d_v]; beta: [T, H]; initial_state
    [N, H, d_k, d_v] or None; cu_seqlens [N+1] or None (one sequence).
    """
    lib = load_c_oracle()
    q, k, v, g, beta = map(_c64, (q, k, v, g, beta))
    T, H, dk = k.shape
    dv = v.shape[-1]
    cu = np.array([0, T] if cu_seqlens is None else list(cu_seqlens), dtype=np.int64)
    n = len(cu) - 1
    s0 = None if initial_state is None else _c64(initial_state)
    o = np.zeros((T, H, dv))
    sf = np.zeros((n, H, dk, dv))
    rc = lib.kda_oracle_prefill(n, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
                                _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), float(scale),
                                _ptr(s0), _ptr(o), _ptr(sf), int(col_block), int(n_threads))
    if rc != 0:
        raise ValueError("kda_oracle_prefill rejected its arguments")
    return o, sf


def decode_step(q, k, v, g, beta, scale, state, n_threads=0):
    """C fp64 decode step; returns (o, new_state). Shapes [N, H, ...]."""
    lib = load_c_oracle()
    q, k, v, g, beta = map(_c64, (q, k, v, g, beta))
    N, H, dk = k.shape
    dv = v.shape[-1]
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    o = np.zeros((N, H, dv))
    rc = lib.kda_oracle_decode_step(N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                    _ptr(beta), float(scale), _ptr(st), _ptr(o), int(n_threads))
    if rc != 0:
        raise ValueError("kda_oracle_decode_step rejected its arguments")
    return o, st


def max_threads() -> int:
    return int(load_c_oracle().kda_oracle_max_threads())
