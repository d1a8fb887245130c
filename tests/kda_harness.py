"""Shared helpers for the GPU tests: run the HIP path through the binding and
the fp64 oracle on the same stored inputs, and compare.

Error metric: relative Frobenius error over the whole compared tensor,
||x - x_ref||_F / ||x_ref||_F, with x_ref the fp64 oracle and x up-cast.
"""
from __future__ import annotations

import numpy as np
import torch

import kda_workloads as W
import oracle

TOL = {"f32": 1e-4, "bf16": 5e-3}


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def to_dev(inp):
    d = {}
    for k_, v_ in inp.items():
        d[k_] = v_.to("cuda") if isinstance(v_, torch.Tensor) else v_
    return d


def packed(inp, name):
    """[T_total, H, d] fp64 view of a stored [B, T, H, d] tensor."""
    t = W.to64(inp[name])
    return t.reshape(-1, *t.shape[2:])


def cu_list(inp):
    if inp["cu_seqlens"] is not None:
        return [int(x) for x in inp["cu_seqlens"].tolist()]
    B, T = inp["q"].shape[:2]
    return [b * T for b in range(B + 1)]


def gpu_prefill(inp, chunk, **kw):
    import gated_delta_rule_80_amd as K
    d = to_dev(inp)
    o, fs = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                        initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
                        chunk_size=chunk, **kw)
    torch.cuda.synchronize()
    o64 = o.double().cpu().numpy()
    return o64.reshape(-1, *o64.shape[2:]), (None if fs is None else fs.double().cpu().numpy())


def oracle_prefill(inp, heads=None, cols=None):
    """fp64 oracle on the stored inputs, optionally on a subset of heads and
    value columns (columns of the value space evolve independently, so a column
    subset of v and S0 gives exactly those columns of o and of the state)."""
    q, k, v, g = (packed(inp, n) for n in ("q", "k", "v", "g"))
    b = W.to64(inp["beta"]).reshape(-1, inp["beta"].shape[-1])
    s0 = W.to64(inp["initial_state"])
    if heads is not None:
        q, k, v, g, b = q[:, heads], k[:, heads], v[:, heads], g[:, heads], b[:, heads]
        s0 = None if s0 is None else s0[:, heads]
    if cols is not None:
        v = v[..., cols]
        s0 = None if s0 is None else s0[..., cols]
    return oracle.prefill(q, k, v, g, b, inp["scale"], s0, cu_list(inp))


def check_prefill(inp, chunk, heads=None, cols=None, tol=None, **kw):
    """Run both sides and assert the tolerance; returns (err_o, err_s)."""
    tol = TOL[inp["dtype"]] if tol is None else tol
    o, fs = gpu_prefill(inp, chunk, **kw)
    o_ref, s_ref = oracle_prefill(inp, heads, cols)
    if heads is not None:
        o, fs = o[:, heads], fs[:, heads]
    if cols is not None:
        o, fs = o[..., cols], fs[..., cols]
    eo, es = rel_err(o, o_ref), rel_err(fs, s_ref)
    print("prefill err o %.3e  S %.3e  (tol %.0e)" % (eo, es, tol), flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(fs))
    assert eo <= tol and es <= tol, (eo, es)
    return eo, es
