"""fp64 oracle for the gradients of the KDA forward pass (test infrastructure
only: only tests, the smoke check and the benchmark's CPU-baseline leg may call
this module; the GPU path never imports it).

The pages motivate the chunkwise form by training ("Kimi Delta Attention: How
It Works, Step by Step", the questions on why chunking matters for training)
but derive no gradients.  Two formulations are given here:

* :func:`recurrent_grads` -- the definition: reverse-mode automatic
  differentiation (PyTorch autograd, float64, CPU) of the token recurrence
  written out with plain tensor operations.  Pinned against central finite
  differences of :func:`oracle.reference.recurrent`, an independently written
  forward.
* :func:`chunkwise_grads` -- the backward of the chunkwise WY / UT form of
  "Understanding Kimi Delta Attention" (A. Flores), sections "The triangular
  system" and "Putting the chunks together", derived by hand step by step in
  that page's notation and sign convention.  Pinned against
  :func:`recurrent_grads`.

The loss whose gradients are returned is L = sum(o * do) + sum(S_T * dS_T):
``do`` is the upstream gradient of the output and ``dfinal`` that of each
sequence's final state (zero if None).  Gradients are returned for q, k, v, g
(the per-token log-decay), beta and the initial state.

Layouts as in :mod:`oracle.reference`: q, k, g [T_total, H, d_k], v and do
[T_total, H, d_v], beta [T_total, H], states [N, H, d_k, d_v].
"""
from __future__ import annotations

import numpy as np

from .reference import packed_bounds, solve_unit_lower

__all__ = ["recurrent_grads", "chunkwise_grads"]


def _as64(x):
    return np.asarray(x, dtype=np.float64)


def recurrent_grads(q, k, v, g, beta, scale, do, initial_state=None, dfinal=None,
                    cu_seqlens=None):
    """Gradients of L = <o, do> + <S_T, dfinal> by autograd of the recurrence.

    Per token and head (the retain / predict / correct / read steps of the
    forward recurrence):
      S_bar = Diag(e^{g_t}) S;  v_hat = S_bar^T k_t;
      S = S_bar + beta_t k_t (v_t - v_hat)^T;  o_t = S^T (scale q_t).
    Returns a dict with dq, dk, dv, dg, dbeta and, when an initial state is
    given, dinitial_state (float64 numpy arrays).
    """
    import torch

    T, H, dk = _as64(k).shape
    dv = _as64(v).shape[-1]
    t = {n: torch.tensor(_as64(x), dtype=torch.float64, requires_grad=True)
         for n, x in (("q", q), ("k", k), ("v", v), ("g", g), ("beta", beta))}
    bounds = packed_bounds(T, cu_seqlens)
    s0 = None
    if initial_state is not None:
        s0 = torch.tensor(_as64(initial_state), dtype=torch.float64, requires_grad=True)
    do_t = torch.tensor(_as64(do), dtype=torch.float64)
    loss = torch.zeros((), dtype=torch.float64)
    for n, (a, b) in enumerate(bounds):
        S = s0[n] if s0 is not None else torch.zeros((H, dk, dv), dtype=torch.float64)
        for i in range(a, b):
            Sbar = torch.exp(t["g"][i])[:, :, None] * S
            vhat = (Sbar * t["k"][i][:, :, None]).sum(dim=1)
            u = t["beta"][i][:, None] * (t["v"][i] - vhat)
            S = Sbar + t["k"][i][:, :, None] * u[:, None, :]
            o = (S * (scale * t["q"][i])[:, :, None]).sum(dim=1)
            loss = loss + (o * do_t[i]).sum()
        if dfinal is not None:
            loss = loss + (S * torch.tensor(_as64(dfinal)[n], dtype=torch.float64)).sum()
    loss.backward()
    out = {"d" + n: (x.grad.numpy() if x.grad is not None else np.zeros(x.shape))
           for n, x in t.items()}
    if s0 is not None:
        out["dinitial_state"] = s0.grad.numpy()
    return out


def _pair_decay(G):
    """E[i, j, c] = e^{G_ic - G_jc} for j <= i, 0 above the diagonal (the
    exponent is never positive where it is used)."""
    C = G.shape[0]
    diff = G[:, None, :] - G[None, :, :]
    keep = np.tril(np.ones((C, C), dtype=bool))[:, :, None]
    return np.where(keep, np.exp(np.minimum(diff, 0.0)), 0.0)


def _chunk_forward(qc, kc, vc, gc, bc, scale, S0):
    """One chunk of the WY / UT form, keeping what the backward needs."""
    C = kc.shape[0]
    strict = np.tril(np.ones((C, C)), -1)
    incl = np.tril(np.ones((C, C)))
    G = np.cumsum(gc, axis=0)
    E = _pair_decay(G)
    # A_ij = -beta_i k_i^T Gamma_{j->i} k_j (j < i); (I - A) T = I
    Kt = np.einsum("ic,jc,ijc->ij", kc, kc, E) * strict
    A = -bc[:, None] * Kt
    T = solve_unit_lower(A)
    # R = T B L, U = T B V with L_i = (Gamma_i k_i)^T; Z = U - R S0
    Lm = np.exp(G) * kc
    BL = bc[:, None] * Lm
    BV = bc[:, None] * vc
    R = T @ BL
    U = T @ BV
    Z = U - R @ S0
    # H_ij = (s q_i)^T Gamma_{j->i} k_j (j <= i); Qbar_i = Gamma_i s q_i
    qs = scale * qc
    Hm = np.einsum("ic,jc,ijc->ij", qs, kc, E) * incl
    Qbar = np.exp(G) * qs
    O = Qbar @ S0 + Hm @ Z
    # S_out = Gamma_C S0 + Kbar^T Z, Kbar_j = Gamma_{j->C} k_j
    eGC = np.exp(G[-1])
    Kbar = np.exp(G[-1][None, :] - G) * kc
    S_out = eGC[:, None] * S0 + Kbar.T @ Z
    saved = dict(qc=qc, kc=kc, vc=vc, bc=bc, qs=qs, G=G, E=E, Kt=Kt, T=T, Lm=Lm, BL=BL, BV=BV,
                 R=R, Z=Z, Hm=Hm, Qbar=Qbar, eGC=eGC, Kbar=Kbar, S0=S0, strict=strict, incl=incl)
    return O, S_out, saved


def _chunk_backward(sv, scale, dO, dS_out):
    """Reverse of :func:`_chunk_forward` given dL/dO and dL/dS_out.

    Each block undoes one forward step, last step first; the gradients of
    the decay collect in dG (per row of the cumulative log-decay) and become
    dg by a reverse cumulative sum, since G_i = sum_{r <= i} g_r.
    """
    kc, vc, bc, qs, G, E = sv["kc"], sv["vc"], sv["bc"], sv["qs"], sv["G"], sv["E"]
    T, Lm, BL, BV, R, Z = sv["T"], sv["Lm"], sv["BL"], sv["BV"], sv["R"], sv["Z"]
    Hm, Qbar, eGC, Kbar, S0 = sv["Hm"], sv["Qbar"], sv["eGC"], sv["Kbar"], sv["S0"]
    dG = np.zeros_like(G)
    # S_out = Gamma_C S0 + Kbar^T Z
    dS0 = eGC[:, None] * dS_out
    dGC = eGC * (dS_out * S0).sum(axis=1)
    dKbar = Z @ dS_out.T
    dZ = Kbar @ dS_out
    # O = Qbar S0 + H Z
    dQbar = dO @ S0.T
    dS0 += Qbar.T @ dO
    dH = (dO @ Z.T) * sv["incl"]
    dZ += Hm.T @ dO
    # Z = U - R S0
    dU = dZ
    dR = -dZ @ S0.T
    dS0 -= R.T @ dZ
    # U = T (B V), R = T (B L)
    dT = dU @ BV.T + dR @ BL.T
    dBV = T.T @ dU
    dBL = T.T @ dR
    dv = bc[:, None] * dBV
    dL = bc[:, None] * dBL
    dbeta = (dBV * vc).sum(axis=1) + (dBL * Lm).sum(axis=1)
    # T = (I - A)^{-1}: dT = T dA T, so dL/dA = T^T (dL/dT) T^T on A's support
    dA = (T.T @ dT @ T.T) * sv["strict"]
    # A_ij = -beta_i Kt_ij, Kt_ij = sum_c k_ic k_jc e^{G_ic - G_jc}
    dbeta -= (dA * sv["Kt"]).sum(axis=1)
    dKt = -bc[:, None] * dA
    dk = np.einsum("ij,jc,ijc->ic", dKt, kc, E) + np.einsum("ij,ic,ijc->jc", dKt, kc, E)
    term = dKt[:, :, None] * kc[:, None, :] * kc[None, :, :] * E
    dG += term.sum(axis=1) - term.sum(axis=0)
    # H_ij = sum_c qs_ic k_jc e^{G_ic - G_jc}
    dqs = np.einsum("ij,jc,ijc->ic", dH, kc, E)
    dk += np.einsum("ij,ic,ijc->jc", dH, qs, E)
    term = dH[:, :, None] * qs[:, None, :] * kc[None, :, :] * E
    dG += term.sum(axis=1) - term.sum(axis=0)
    # Qbar = e^{G} qs, L = e^{G} k, Kbar = e^{G_C - G} k
    dqs += dQbar * np.exp(G)
    dG += dQbar * Qbar
    dk += dL * np.exp(G)
    dG += dL * Lm
    dk += dKbar * np.exp(G[-1][None, :] - G)
    dG -= dKbar * Kbar
    dGC += (dKbar * Kbar).sum(axis=0)
    # G_C is the last row of G; G = cumsum(g)
    dG[-1] += dGC
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return dict(dq=scale * dqs, dk=dk, dv=dv, dg=dg, dbeta=dbeta), dS0


def chunkwise_grads(q, k, v, g, beta, scale, chunk_size, do, initial_state=None, dfinal=None,
                    cu_seqlens=None):
    """Gradients of L = <o, do> + <S_T, dfinal> through the chunkwise form.

    Forward over each sequence's chunks keeping the chunk-start states, then
    backward over the chunks in reverse order, carrying dL/dS across chunk
    boundaries just as the forward carries S.  Same return value as
    :func:`recurrent_grads`.
    """
    q, k, v, g, beta, do = map(_as64, (q, k, v, g, beta, do))
    T, H, dk = k.shape
    dv = v.shape[-1]
    bounds = packed_bounds(T, cu_seqlens)
    out = {n: np.zeros(x.shape) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g),
                                             ("dbeta", beta))}
    dinit = np.zeros((len(bounds), H, dk, dv))
    for n, (t0, t1) in enumerate(bounds):
        for h in range(H):
            S = np.zeros((dk, dv)) if initial_state is None else _as64(initial_state)[n, h].copy()
            saved = []
            for c0 in range(t0, t1, chunk_size):
                c1 = min(c0 + chunk_size, t1)
                _, S, sv = _chunk_forward(q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], g[c0:c1, h],
                                          beta[c0:c1, h], scale, S)
                saved.append((c0, c1, sv))
            dS = np.zeros((dk, dv)) if dfinal is None else _as64(dfinal)[n, h].copy()
            for c0, c1, sv in reversed(saved):
                gr, dS = _chunk_backward(sv, scale, do[c0:c1, h], dS)
                for name, val in gr.items():
                    out[name][c0:c1, h] = val
            dinit[n, h] = dS
    if initial_state is not None:
        out["dinitial_state"] = dinit
    return out
