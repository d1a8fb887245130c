"""NumPy fp64 oracle for the KDA forward pass (test infrastructure only).

Two independent formulations of the same operator, both in float64:

* :func:`recurrent` -- the token-by-token recurrence, a twin of the C oracle
  written separately in NumPy.
* :func:`chunkwise` -- the chunkwise WY / UT form, taken step by step from
  "Understanding Kimi Delta Attention" (A. Flores), sections "The triangular
  system" and "Putting the chunks together", in that page's notation and sign
  convention: A_ij = -beta_i k_i^T Gamma_{j->i} k_j (j < i), (I - A) T = I,
  R = T B L, U = T B V, Z = U - R S0, O = Qbar S0 + H Z,
  S_out = Gamma_C S0 + Kbar_out^T Z.

The chunkwise form reaches the recurrent result exactly up to rounding order;
agreement between the two is one of the oracle's pins.  Neither function is
used by the GPU path, and neither imports anything from it.  Only tests, the
smoke check and the benchmark's CPU-baseline leg may call this module.

Layouts (packed tokens, heads second):
  q, k, g: [T_total, H, d_k]   v: [T_total, H, d_v]   beta: [T_total, H]
  initial_state / final state: [N, H, d_k, d_v]       o: [T_total, H, d_v]
``g`` is the per-token log-decay log a_t (<= 0), not a cumulative sum.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

__all__ = ["recurrent", "chunkwise", "decode_step", "packed_bounds", "solve_unit_lower"]


def packed_bounds(total_tokens: int, cu_seqlens=None):
    """Sequence boundaries [(start, end), ...] for packed tokens."""
    if cu_seqlens is None:
        return [(0, total_tokens)]
    cu = [int(x) for x in cu_seqlens]
    if cu[0] != 0 or any(b < a for a, b in zip(cu[:-1], cu[1:])) or cu[-1] != total_tokens:
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T_total")
    return list(zip(cu[:-1], cu[1:]))


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def recurrent(q, k, v, g, beta, scale, initial_state=None, cu_seqlens=None):
    """Token-by-token KDA recurrence in fp64.

    Per token, for every head at once ("Understanding Kimi Delta Attention",
    box "KDA: retain, predict, correct"; query scale from "Demystifying Kimi
    Delta Attention", first display):
      S_bar = Diag(exp(g_t)) S      (retain, rows = key channels)
      v_hat = S_bar^T k_t           (predict from what survived the decay)
      S     = S_bar + beta_t k_t (v_t - v_hat)^T   (correct)
      o_t   = S^T (scale q_t)       (read the updated state)
    Returns (o, final_state).
    """
    q, k, v, g, beta = map(_as64, (q, k, v, g, beta))
    T, H, dk = k.shape
    dv = v.shape[-1]
    bounds = packed_bounds(T, cu_seqlens)
    o = np.zeros((T, H, dv))
    finals = np.zeros((len(bounds), H, dk, dv))
    for n, (t0, t1) in enumerate(bounds):
        S = np.zeros((H, dk, dv)) if initial_state is None else _as64(initial_state)[n].copy()
        for t in range(t0, t1):
            S = np.exp(g[t])[:, :, None] * S
            v_hat = np.einsum("hrc,hr->hc", S, k[t])
            S = S + beta[t][:, None, None] * k[t][:, :, None] * (v[t] - v_hat)[:, None, :]
            o[t] = np.einsum("hrc,hr->hc", S, scale * q[t])
        finals[n] = S
    return o, finals


def decode_step(q, k, v, g, beta, scale, state):
    """One recurrent step for [N, H] independent pairs; returns (o, new_state).

    Identical body to :func:`recurrent` with a length-1 sequence per pair.
    """
    q, k, v, g, beta, state = map(_as64, (q, k, v, g, beta, state))
    S = np.exp(g)[..., :, None] * state
    v_hat = np.einsum("nhrc,nhr->nhc", S, k)
    S = S + beta[..., None, None] * k[..., :, None] * (v - v_hat)[..., None, :]
    o = np.einsum("nhrc,nhr->nhc", S, scale * q)
    return o, S


def solve_unit_lower(A):
    """T with (I - A) T = I for strictly lower triangular A (a library
    triangular solve; "The triangular system": I - A is lower triangular with
    unit diagonal, so the system has a unique solution)."""
    C = A.shape[0]
    return solve_triangular(np.eye(C) - A, np.eye(C), lower=True, unit_diagonal=True)


def _chunk(qc, kc, vc, gc, bc, scale, S0):
    """One chunk of one head, following the UT-style transform step by step.

    qc, kc, gc: [C, d_k]; vc: [C, d_v]; bc: [C]; S0: [d_k, d_v].
    """
    C = kc.shape[0]
    # cumulative log-decay g_i = sum_{r<=i} log alpha_r (inclusive), and
    # Gamma_{j->i} = Diag(exp(g_i - g_j)) from differences of cumulative logs
    # ("Putting the chunks together", box "First: represent decay stably").
    G = np.cumsum(gc, axis=0)
    # A_ij = -beta_i k_i^T Gamma_{j->i} k_j for j < i, zero otherwise
    # ("The triangular system", box "Two definitions that organize everything").
    A = np.zeros((C, C))
    for i in range(C):
        for j in range(i):
            A[i, j] = -bc[i] * np.sum(kc[i] * np.exp(G[i] - G[j]) * kc[j])
    # (I - A) T = I, unit lower triangular.
    T = solve_unit_lower(A)
    # L_i = (Gamma_i k_i)^T, B = Diag(beta); R = T B L, U = T B V, Z = U - R S0
    # (box "The compact UT-style transform").
    Lm = np.exp(G) * kc
    Bm = np.diag(bc)
    R = T @ Bm @ Lm
    U = T @ Bm @ vc
    Z = U - R @ S0
    # H_ij = q_i^T Gamma_{j->i} k_j for j <= i; rows of Qbar are (Gamma_i q_i)^T
    # (box "Outputs as matrix multiplications").  The query carries the
    # d_k^{-1/2} read scale ("Demystifying Kimi Delta Attention").
    qs = scale * qc
    Hm = np.zeros((C, C))
    for i in range(C):
        for j in range(i + 1):
            Hm[i, j] = np.sum(qs[i] * np.exp(G[i] - G[j]) * kc[j])
    Qbar = np.exp(G) * qs
    O = Qbar @ S0 + Hm @ Z
    # S_out = Gamma_C S0 + Kbar_out^T Z, row j of Kbar_out = (Gamma_{j->C} k_j)^T
    # (box "One state crosses the chunk boundary").
    Kbar = np.exp(G[-1][None, :] - G) * kc
    S_out = np.exp(G[-1])[:, None] * S0 + Kbar.T @ Z
    return O, S_out


def chunkwise(q, k, v, g, beta, scale, chunk_size, initial_state=None, cu_seqlens=None):
    """Chunkwise WY / UT-transform evaluation in fp64; returns (o, final_state).

    Each sequence is cut into chunks of ``chunk_size`` tokens starting at its
    first token; the last chunk of a sequence may be shorter.  Chunks never
    straddle sequences.  One state crosses each chunk boundary.
    """
    q, k, v, g, beta = map(_as64, (q, k, v, g, beta))
    T, H, dk = k.shape
    dv = v.shape[-1]
    bounds = packed_bounds(T, cu_seqlens)
    o = np.zeros((T, H, dv))
    finals = np.zeros((len(bounds), H, dk, dv))
    for n, (t0, t1) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else _as64(initial_state)[n, h].copy()
            for c0 in range(t0, t1, chunk_size):
                c1 = min(c0 + chunk_size, t1)
                O, S = _chunk(q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], g[c0:c1, h],
                              beta[c0:c1, h], scale, S)
                o[c0:c1, h] = O
            finals[n, h] = S
    return o, finals
