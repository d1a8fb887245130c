"""Seeded synthetic inputs for the KDA forward pass (shared by tests and bench).

This module only draws random inputs.  It holds none of the operator's
arithmetic: it neither evaluates the recurrence nor any part of the chunkwise
form.  Both the GPU path and the fp64 oracle consume exactly the tensors it
returns (the oracle up-casts the stored bf16 / fp32 values exactly).

Distributions (the five standard workloads)
  q, k    N(0, 1) per element, then L2-normalised per token and head (the
          layer normalises keys and queries before the operator; the operator
          itself does not), then rounded to the storage dtype.
  v       N(0, 1), rounded to the storage dtype.
  beta    sigmoid(N(0, 1)), fp32.
  g       per-token, per-channel log-decay log a = log sigmoid(z) with
          z ~ U(z_lo, z_hi), computed stably as -log1p(exp(-z)) in fp64 and
          stored fp32.  z ~ U(2, 9) gives a in (0.881, 0.99988);
          z ~ U(4, 12) gives a in (0.982, 0.999994).
  S0      N(0, sigma^2) fp32 where a workload has a nonzero initial state
          (sigma is a standard deviation).
  lengths integers uniform on [lo, hi], both ends included.

Generation uses ``numpy.random.default_rng`` streams keyed by the workload's
seed (1000+i for workload i), the tensor (lengths 0, q 1, k 2, v 3,
beta-logits 4, z 5, S0 6) and the block of BLOCK_TOKENS tokens: block b of
tensor j comes from ``default_rng([seed, j, b])``; decode step s of workload 3
uses ``default_rng([1003, 1000 + s, j, 0])``.  Blocks are independent, so they
are drawn in parallel threads, and the result is deterministic for a given
seed.  Normal draws are float32; host memory stays bounded by the block size.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

BLOCK_TOKENS = 4096  # token block for drawing large tensors (fixes the stream)


@dataclass(frozen=True)
class Workload:
    """Shape and distribution of one standard workload."""
    idx: int
    name: str
    kind: str                 # "prefill" or "decode"
    H: int
    dk: int
    dv: int
    dtype: str                # storage dtype of q, k, v, o: "f32" or "bf16"
    z_range: tuple
    B: int = 1                # prefill: rows of equal length (no cu_seqlens)
    T: int = 0                # prefill: tokens per row
    chunk: int = 64
    s0_std: Optional[float] = None
    n_seqs: int = 0           # varlen: number of packed sequences
    len_range: tuple = (0, 0)
    n_sessions: int = 0       # decode
    steps: int = 0            # decode
    state_std: float = 0.0    # decode
    description: str = field(default="", compare=False)

    @property
    def seed(self) -> int:
        return 1000 + self.idx

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)


WORKLOADS = {
    1: Workload(1, "tiny", "prefill", H=1, dk=16, dv=16, dtype="f32", z_range=(2.0, 9.0),
                B=1, T=64, chunk=16,
                description="B=1 H=1 T=64 d=16 chunk=16 fp32, zero initial state"),
    2: Workload(2, "prefill", "prefill", H=8, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0),
                B=2, T=2048, chunk=64, s0_std=0.01,
                description="B=2 H=8 T=2048 d=128 chunk=64 bf16, S0 ~ N(0, 0.01^2)"),
    3: Workload(3, "decode", "decode", H=32, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0),
                n_sessions=128, steps=256, state_std=0.05,
                description="128 sessions x 32 heads, d=128, one token per step, 256 steps, "
                            "fp32 state ~ N(0, 0.05^2) (268 MB) updated in place"),
    4: Workload(4, "varlen", "prefill", H=32, dk=128, dv=128, dtype="bf16", z_range=(2.0, 9.0),
                chunk=64, n_seqs=8, len_range=(1024, 16384),
                description="8 packed sequences, lengths U{1024..16384}, H=32 d=128 chunk=64 bf16, "
                            "zero initial states"),
    5: Workload(5, "long", "prefill", H=32, dk=128, dv=128, dtype="bf16", z_range=(4.0, 12.0),
                B=1, T=131072, chunk=64, s0_std=0.01,
                description="B=1 H=32 T=131072 d=128 chunk=64 bf16, z ~ U(4,12), "
                            "S0 ~ N(0, 0.01^2)"),
}


def torch_dtype(name: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


_POOL = None


def _pool():
    global _POOL
    if _POOL is None:
        import concurrent.futures as cf
        import os
        _POOL = cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4))
    return _POOL


def _blocks(n_tok):
    return [(b, t0, min(n_tok, t0 + BLOCK_TOKENS))
            for b, t0 in enumerate(range(0, n_tok, BLOCK_TOKENS))]


TENSOR_ID = dict(lengths=0, q=1, k=2, v=3, beta=4, z=5, s0=6)


def _normal_rows(key, n_tok, H, d, normalize, out_dtype):
    """[n_tok, H, d] N(0,1) (float32 draws), optionally L2-normalised per row
    (float64 norms), rounded to ``out_dtype``.  ``key`` = [seed, tensor id]."""
    out = torch.empty((n_tok, H, d), dtype=out_dtype)

    def fill(blk):
        b, t0, t1 = blk
        x = torch.from_numpy(np.random.default_rng(key + [b]).standard_normal(
            (t1 - t0, H, d), dtype=np.float32))
        if normalize:
            x64 = x.double()
            x = (x64 / torch.linalg.vector_norm(x64, dim=-1, keepdim=True)).float()
        out[t0:t1] = x.to(out_dtype)

    list(_pool().map(fill, _blocks(n_tok)))
    return out


def _log_decay(key, n_tok, H, dk, z_range):
    """[n_tok, H, dk] fp32 log sigmoid(z) = -log1p(exp(-z)) in fp64, z ~ U(z_lo, z_hi)."""
    out = torch.empty((n_tok, H, dk), dtype=torch.float32)
    lo, hi = z_range

    def fill(blk):
        b, t0, t1 = blk
        z = torch.from_numpy(np.random.default_rng(key + [b]).uniform(lo, hi, size=(t1 - t0, H, dk)))
        out[t0:t1] = torch.log1p(torch.exp(-z)).neg_().float()

    list(_pool().map(fill, _blocks(n_tok)))
    return out


def _beta(key, n_tok, H):
    """[n_tok, H] fp32 sigmoid(N(0, 1))."""
    out = torch.empty((n_tok, H), dtype=torch.float32)
    for b, t0, t1 in _blocks(n_tok):
        x = torch.from_numpy(np.random.default_rng(key + [b]).standard_normal((t1 - t0, H)))
        out[t0:t1] = torch.sigmoid(x).float()
    return out


def _s0(key, n, H, dk, dv, std):
    x = np.random.default_rng(key + [0]).standard_normal((n, H, dk, dv), dtype=np.float32)
    return torch.from_numpy(x * np.float32(std))


def _draw(seed_key, total, H, dk, dv, dtype, z_range):
    """q, k, v, beta, g for ``total`` packed tokens; seed_key = [seed] or [seed, step]."""
    td = torch_dtype(dtype)
    T = TENSOR_ID
    q = _normal_rows(seed_key + [T["q"]], total, H, dk, True, td)
    k = _normal_rows(seed_key + [T["k"]], total, H, dk, True, td)
    v = _normal_rows(seed_key + [T["v"]], total, H, dv, False, td)
    beta = _beta(seed_key + [T["beta"]], total, H)
    g = _log_decay(seed_key + [T["z"]], total, H, dk, z_range)
    return q, k, v, beta, g


def make_prefill(*, H, dk, dv, dtype, z_range, seed, B=1, T=0, lengths=None,
                 s0_std=None):
    """Seeded prefill inputs.

    Either B rows of T tokens (``lengths`` None; tensors [B, T, H, d], no
    cu_seqlens) or packed sequences of the given ``lengths`` (tensors
    [1, sum(lengths), H, d] plus ``cu_seqlens`` int32 [N+1]).
    Returns a dict of CPU tensors plus metadata.
    """
    if lengths is not None:
        lengths = [int(x) for x in lengths]
        total = sum(lengths)
        rows, row_len = 1, total
        cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32))
        n_seqs = len(lengths)
    else:
        total, rows, row_len = B * T, B, T
        cu = None
        n_seqs = B
    q, k, v, beta, g = _draw([seed], total, H, dk, dv, dtype, z_range)
    s0 = None if s0_std is None else _s0([seed, TENSOR_ID["s0"]], n_seqs, H, dk, dv, s0_std)
    shape4 = lambda x: x.reshape(rows, row_len, *x.shape[1:])  # noqa: E731
    return dict(q=shape4(q), k=shape4(k), v=shape4(v), g=shape4(g), beta=shape4(beta),
                initial_state=s0, cu_seqlens=cu, scale=1.0 / math.sqrt(dk),
                n_seqs=n_seqs, dtype=dtype)


def varlen_lengths(w: Workload):
    """Seeded sequence lengths of a varlen workload."""
    rng = np.random.default_rng([w.seed, TENSOR_ID["lengths"]])
    lo, hi = w.len_range
    return [int(x) for x in rng.integers(lo, hi + 1, size=w.n_seqs)]


def make_workload(idx: int):
    """Inputs of standard prefill workload ``idx`` (1, 2, 4 or 5)."""
    w = WORKLOADS[idx]
    if w.kind != "prefill":
        raise ValueError("workload %d is a decode workload; use make_decode_state/step" % idx)
    if w.n_seqs:
        return make_prefill(H=w.H, dk=w.dk, dv=w.dv, dtype=w.dtype, z_range=w.z_range,
                            seed=w.seed, lengths=varlen_lengths(w), s0_std=w.s0_std)
    return make_prefill(H=w.H, dk=w.dk, dv=w.dv, dtype=w.dtype, z_range=w.z_range,
                        seed=w.seed, B=w.B, T=w.T, s0_std=w.s0_std)


def make_decode_state(w: Workload = WORKLOADS[3], n_sessions=None, H=None):
    """Initial decode state [N, H, d_k, d_v] fp32 ~ N(0, state_std^2)."""
    N = n_sessions or w.n_sessions
    Hh = H or w.H
    st = torch.empty((N, Hh, w.dk, w.dv), dtype=torch.float32)

    def fill(n):
        x = np.random.default_rng([w.seed, TENSOR_ID["s0"], n]).standard_normal(
            (Hh, w.dk, w.dv), dtype=np.float32)
        st[n] = torch.from_numpy(x * np.float32(w.state_std))

    list(_pool().map(fill, range(N)))
    return st


def make_decode_step(step: int, w: Workload = WORKLOADS[3], n_sessions=None, H=None):
    """Fresh seeded tokens of decode step ``step``: q, k, v [N, H, d], g, beta."""
    N = n_sessions or w.n_sessions
    Hh = H or w.H
    q, k, v, beta, g = _draw([w.seed, 1000 + step], N, Hh, w.dk, w.dv, w.dtype, w.z_range)
    return dict(q=q, k=k, v=v, g=g, beta=beta, scale=w.scale)


def to64(t):
    """Exact up-cast of a stored tensor to a float64 numpy array."""
    if t is None:
        return None
    return t.detach().to("cpu", torch.float64).numpy()
