"""Planted mistakes in copies of the oracle must fail at least one pin (CPU).

Each mutant is a plausible error in writing the recurrence or the chunkwise
form (a dropped term, a wrong sign, order or index, a transposed operand).
The pins are only worth something if every such mutant trips one of them.
"""
import numpy as np
import pytest

from oracle import reference
import oracle_pins as P


def make_recurrent(mut):
    """NumPy recurrence with one planted mistake ``mut``."""
    def run(q, k, v, g, beta, scale, s0, cu):
        q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
        T, H, dk = k.shape
        dv = v.shape[-1]
        bounds = reference.packed_bounds(T, cu)
        o = np.zeros((T, H, dv))
        fin = np.zeros((len(bounds), H, dk, dv))
        for n, (t0, t1) in enumerate(bounds):
            S = np.zeros((H, dk, dv)) if s0 is None else np.array(s0[n], dtype=np.float64)
            for t in range(t0, t1):
                a = np.exp(g[t])
                if mut == "g_not_exp":
                    a = 1.0 + g[t]
                S_prev = S
                if mut != "decay_after":
                    S = (a[:, None, :] * S) if mut == "decay_columns" else a[:, :, None] * S
                base = S_prev if mut == "predict_undecayed" else S
                v_hat = np.einsum("hrc,hr->hc", base, k[t])
                if mut == "predict_with_query":
                    v_hat = np.einsum("hrc,hr->hc", base, q[t])
                b = beta[t]
                if mut == "beta_dropped":
                    b = np.ones_like(b)
                err = v[t] - v_hat
                if mut == "sign":
                    err = v_hat - v[t]
                if mut == "additive":
                    err = v[t]
                S_new = S + b[:, None, None] * k[t][:, :, None] * err[:, None, :]
                if mut == "decay_after":
                    S_new = a[:, :, None] * S_new
                read = S_prev if mut == "read_old_state" else S_new
                sc = 1.0 if mut == "no_scale" else scale
                if mut == "transposed_read":
                    o[t] = np.einsum("hrc,hc->hr", read, sc * q[t])
                else:
                    o[t] = np.einsum("hrc,hr->hc", read, sc * q[t])
                S = S_new
            fin[n] = S
        return o, fin
    return run


RECURRENT_MUTANTS = ["g_not_exp", "decay_after", "decay_columns", "predict_undecayed",
                     "predict_with_query", "beta_dropped", "sign", "additive",
                     "read_old_state", "no_scale", "transposed_read"]


def all_pins_pass(run):
    failures = []
    for pin in P.RUN_PINS:
        try:
            ok, detail = pin(run)
        except Exception as e:  # a shape error is a failed pin too
            ok, detail = False, repr(e)
        if not ok:
            failures.append((pin.__name__, detail))
    try:
        ok, _ = P.pin_chunkwise_equivalence(run, reference.chunkwise)
    except Exception:
        ok = False
    if not ok:
        failures.append(("pin_chunkwise_equivalence", ""))
    return failures


def test_unmutated_copy_passes():
    assert all_pins_pass(make_recurrent(None)) == []


@pytest.mark.parametrize("mut", RECURRENT_MUTANTS)
def test_recurrent_mutant_is_caught(mut):
    assert all_pins_pass(make_recurrent(mut)), "mutant %s passed every pin" % mut


def make_chunk(mut):
    """Chunkwise form with one planted mistake, run at C = 16."""
    def _chunk(qc, kc, vc, gc, bc, scale, S0):
        C = kc.shape[0]
        G = np.cumsum(gc, axis=0)
        if mut == "exclusive_cumsum":
            G = G - gc
        A = np.zeros((C, C))
        for i in range(C):
            for j in range(i):
                A[i, j] = -bc[i] * np.sum(kc[i] * np.exp(G[i] - G[j]) * kc[j])
        if mut == "A_sign":
            A = -A
        if mut == "A_beta_column":
            A = A / bc[:, None] * bc[None, :]
        T = reference.solve_unit_lower(A)
        if mut == "T_transposed":
            T = T.T
        Lm = np.exp(G) * kc
        Bm = np.diag(bc)
        R = T @ Bm @ Lm
        U = T @ Bm @ vc
        Z = U - R @ S0
        qs = scale * qc
        Hm = np.zeros((C, C))
        for i in range(C):
            for j in range(i + (0 if mut == "H_strict" else 1)):
                Hm[i, j] = np.sum(qs[i] * np.exp(G[i] - G[j]) * kc[j])
        Qbar = np.exp(G) * qs
        O = Qbar @ S0 + Hm @ Z
        Kbar = (np.exp(G) if mut == "Kbar_wrong_decay" else np.exp(G[-1][None, :] - G)) * kc
        dS0 = S0 if mut == "S0_undecayed" else np.exp(G[-1])[:, None] * S0
        return O, dS0 + Kbar.T @ Z

    def run(q, k, v, g, beta, scale, s0, cu):
        q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
        T, H, dk = k.shape
        dv = v.shape[-1]
        bounds = reference.packed_bounds(T, cu)
        o = np.zeros((T, H, dv))
        fin = np.zeros((len(bounds), H, dk, dv))
        for n, (t0, t1) in enumerate(bounds):
            for h in range(H):
                S = np.zeros((dk, dv)) if s0 is None else np.array(s0[n, h], dtype=np.float64)
                for c0 in range(t0, t1, 16):
                    c1 = min(c0 + 16, t1)
                    O, S = _chunk(q[c0:c1, h], k[c0:c1, h], v[c0:c1, h], g[c0:c1, h],
                                  beta[c0:c1, h], scale, S)
                    o[c0:c1, h] = O
                fin[n, h] = S
        return o, fin
    return run


CHUNK_MUTANTS = ["exclusive_cumsum", "A_sign", "A_beta_column", "T_transposed", "H_strict",
                 "Kbar_wrong_decay", "S0_undecayed"]


def test_unmutated_chunk_copy_matches_recurrence():
    def chunkwise_copy(q, k, v, g, beta, scale, C, s0, cu):
        return make_chunk(None)(q, k, v, g, beta, scale, s0, cu)
    ok, detail = P.pin_chunkwise_equivalence(reference.recurrent, chunkwise_copy)
    assert ok, detail


@pytest.mark.parametrize("mut", CHUNK_MUTANTS)
def test_chunk_mutant_is_caught(mut):
    def chunkwise_mut(q, k, v, g, beta, scale, C, s0, cu):
        return make_chunk(mut)(q, k, v, g, beta, scale, s0, cu)
    ok, _ = P.pin_chunkwise_equivalence(reference.recurrent, chunkwise_mut)
    assert not ok, "chunk mutant %s agreed with the recurrence" % mut
