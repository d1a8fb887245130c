"""Shared helpers for the GPU tests: run the HIP path through the binding and
the fp64 oracle on the same stored inputs, and compare.

Error metric: relative Frobenius error ||x - x_ref||_F / ||x_ref||_F, with
x_ref the fp64 oracle and x up-cast, over three scopes, each asserted against
the tolerance:
  - the whole compared tensor (o, and the final states);
  - every (sequence, head) pair separately (o rows of that pair; its state);
  - every 64-token chunk of every (sequence, head) pair (o only), chunks
    counted from each sequence's first token.
A whole-tensor norm alone would let a single corrupted token row or chunk
through; the per-pair and per-chunk maxima localise it.
"""
from __future__ import annotations

import numpy as np
import torch

import kda_workloads as W
import oracle

TOL = {"f32": 1e-4, "bf16": 5e-3}
LOCAL_CHUNK = 64   # tokens per chunk of the per-chunk maxima (the prefill's chunk)


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def _rel(num2, den2):
    """Elementwise sqrt(num2 / den2); where the reference is exactly zero the
    absolute error is reported instead."""
    den2 = np.where(den2 > 0, den2, 1.0)
    return np.sqrt(num2 / den2)


def local_errors(o, o_ref, cu, chunk=LOCAL_CHUNK):
    """Per-(sequence, head) and per-chunk relative errors of packed outputs.

    o, o_ref: [T_total, H, cols]; cu: sequence boundaries [N+1] (packed rows).
    Returns (pair_err [N, H], chunk_err [n_chunks, H]); empty sequences
    contribute no rows.
    """
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    d2 = ((o - o_ref) ** 2).sum(axis=-1)          # [T, H]
    r2 = (o_ref ** 2).sum(axis=-1)
    T = d2.shape[0]
    seq_of = np.empty(T, dtype=np.int64)
    chunk_of = np.empty(T, dtype=np.int64)
    n_chunks = 0
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        seq_of[a:b] = n
        local = np.arange(b - a) // chunk
        chunk_of[a:b] = n_chunks + local
        n_chunks += int(-(-(b - a) // chunk))
    N = len(cu) - 1
    H = d2.shape[1]
    pair_num = np.zeros((N, H))
    pair_den = np.zeros((N, H))
    np.add.at(pair_num, seq_of, d2)
    np.add.at(pair_den, seq_of, r2)
    ch_num = np.zeros((n_chunks, H))
    ch_den = np.zeros((n_chunks, H))
    np.add.at(ch_num, chunk_of, d2)
    np.add.at(ch_den, chunk_of, r2)
    nonempty = np.array([int(cu[n + 1]) > int(cu[n]) for n in range(N)])
    return _rel(pair_num, pair_den)[nonempty], _rel(ch_num, ch_den)


def state_pair_errors(fs, s_ref):
    """Relative error of every (sequence, head) state: [N, H]."""
    fs = np.asarray(fs, dtype=np.float64)
    s_ref = np.asarray(s_ref, dtype=np.float64)
    num = ((fs - s_ref) ** 2).sum(axis=(-2, -1))
    den = (s_ref ** 2).sum(axis=(-2, -1))
    return _rel(num, den)


def assert_close(o, o_ref, fs, s_ref, cu, tol, label="prefill"):
    """Whole-tensor, per-(sequence, head) and per-chunk errors, all <= tol."""
    assert np.all(np.isfinite(o)), "non-finite output"
    eo = rel_err(o, o_ref)
    pair_o, chunk_o = local_errors(o, o_ref, cu)
    res = {"o": eo, "o_pair_max": float(pair_o.max()) if pair_o.size else 0.0,
           "o_chunk_max": float(chunk_o.max()) if chunk_o.size else 0.0}
    if fs is not None:
        assert np.all(np.isfinite(fs)), "non-finite final state"
        res["S"] = rel_err(fs, s_ref)
        res["S_pair_max"] = float(state_pair_errors(fs, s_ref).max())
    print("%s err: %s (tol %.0e)" % (label, "  ".join("%s %.3e" % kv for kv in res.items()), tol),
          flush=True)
    for key, val in res.items():
        assert val <= tol, (key, val, res)
    return res


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


def _select(t, heads, cols):
    """Head and value-column subset of a [..., H, d] device tensor, taken on the
    device before the copy to the host."""
    if heads is not None:
        t = t[..., heads, :]
    if cols is not None:
        t = t[..., cols]
    return t


def gpu_prefill(inp, chunk, heads=None, cols=None, **kw):
    """HIP prefill through the binding; returns o [T_total, H', cols'] and the
    final states [N, H', d_k, cols'] (or None) as fp64 numpy arrays."""
    import gated_delta_rule_80_amd as K
    d = to_dev(inp)
    o, fs = K.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                        initial_state=d["initial_state"], cu_seqlens=d["cu_seqlens"],
                        chunk_size=chunk, **kw)
    torch.cuda.synchronize()
    o = _select(o, heads, cols)
    o64 = o.double().cpu().numpy()
    o64 = o64.reshape(-1, *o64.shape[2:])
    if fs is None:
        return o64, None
    if heads is not None:
        fs = fs[:, heads]
    if cols is not None:
        fs = fs[..., cols]
    return o64, fs.double().cpu().numpy()


def oracle_prefill(inp, heads=None, cols=None):
    """fp64 oracle on the stored inputs, optionally on a subset of heads and
    value columns (columns of the value space evolve independently, so a column
    subset of v and S0 gives exactly those columns of o and of the state)."""
    sel = lambda t: t if heads is None else t[:, heads]  # noqa: E731
    q, k, g = (sel(packed(inp, n)) for n in ("q", "k", "g"))
    v = sel(packed(inp, "v"))
    b = W.to64(inp["beta"]).reshape(-1, inp["beta"].shape[-1])
    b = b if heads is None else b[:, heads]
    s0 = W.to64(inp["initial_state"])
    if s0 is not None and heads is not None:
        s0 = s0[:, heads]
    if cols is not None:
        v = v[..., cols]
        s0 = None if s0 is None else s0[..., cols]
    return oracle.prefill(q, k, v, g, b, inp["scale"], s0, cu_list(inp))


def check_prefill(inp, chunk, heads=None, cols=None, tol=None, **kw):
    """Run both sides and assert the tolerance on every scope; returns
    (err_o, err_s) over the whole compared tensors."""
    tol = TOL[inp["dtype"]] if tol is None else tol
    o, fs = gpu_prefill(inp, chunk, heads=heads, cols=cols, **kw)
    o_ref, s_ref = oracle_prefill(inp, heads, cols)
    res = assert_close(o, o_ref, fs, s_ref, cu_list(inp), tol)
    return res["o"], res.get("S", 0.0)
