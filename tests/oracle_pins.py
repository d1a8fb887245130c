"""Pins for the fp64 KDA oracle: what the pages and the mathematics fix.

Each pin takes a candidate implementation ``run(q, k, v, g, beta, scale,
initial_state, cu_seqlens) -> (o, final_state)`` (packed layout, float64) and
returns ``(ok, detail)``.  The same pins run on the real oracle (all must
hold) and on deliberately broken copies of it (at least one must fail), see
``test_oracle_pins.py`` and ``test_oracle_mutants.py``.

None of these pins re-types the oracle's own update: each checks a closed
form, a special case that reduces to another textbook rule, a printed worked
value (fixtures in ``tests/golden``), an independent algorithm, or an
invariant.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def random_inputs(rng, T, H, dk, dv, z_range=(2.0, 9.0), unit_keys=True, beta=None,
                  g_zero=False):
    """Small fp64 inputs [T, H, d] with the workloads' distributions."""
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_keys:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H)))) if beta is None else np.full((T, H), beta)
    if g_zero:
        g = np.zeros((T, H, dk))
    else:
        z = rng.uniform(*z_range, size=(T, H, dk))
        g = -np.log1p(np.exp(-z))
    return q, k, v, g, b


# ----------------------------------------------------------------------------
# P1: the chunkwise WY / UT form reproduces the recurrence
# ("Understanding Kimi Delta Attention": "The triangular system",
#  "Putting the chunks together"; the page's equivalence tests).
# ----------------------------------------------------------------------------
def pin_chunkwise_equivalence(run, chunkwise, tol=1e-12):
    rng = np.random.default_rng(11)
    lengths = [37, 0, 64, 1, 100]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    H, dk, dv = 2, 8, 6
    worst = 0.0
    for z_range in [(2.0, 9.0), (0.5, 3.0)]:
        q, k, v, g, b = random_inputs(rng, T, H, dk, dv, z_range)
        s0 = 0.3 * rng.standard_normal((len(lengths), H, dk, dv))
        o_r, s_r = run(q, k, v, g, b, 0.37, s0, cu)
        for C in (2, 16, 64):
            o_c, s_c = chunkwise(q, k, v, g, b, 0.37, C, s0, cu)
            worst = max(worst, rel_err(o_r, o_c), rel_err(s_r, s_c))
    return worst <= tol, "max rel err %.3e" % worst


# ----------------------------------------------------------------------------
# P2: a = 1 is DeltaNet, S <- (I - beta k k^T) S + beta k v^T
# ("Understanding Kimi Delta Attention", box "The delta rule"; expanded
#  transition in box "KDA as a structured state transition" with D = I).
# ----------------------------------------------------------------------------
def pin_deltanet(run, tol=1e-12):
    rng = np.random.default_rng(12)
    T, H, dk, dv = 20, 2, 5, 4
    q, k, v, g, b = random_inputs(rng, T, H, dk, dv, g_zero=True)
    s0 = rng.standard_normal((1, H, dk, dv))
    o, sf = run(q, k, v, g, b, 0.5, s0, [0, T])
    o_ref = np.zeros_like(o)
    for h in range(H):
        S = s0[0, h].copy()
        for t in range(T):
            kk = k[t, h][:, None]
            S = (np.eye(dk) - b[t, h] * kk @ kk.T) @ S + b[t, h] * kk @ v[t, h][None, :]
            o_ref[t, h] = S.T @ (0.5 * q[t, h])
        err = rel_err(sf[0, h], S)
        if err > tol:
            return False, "state err %.3e" % err
    err = rel_err(o, o_ref)
    return err <= tol, "o err %.3e" % err


def pin_wy_no_decay(run, tol=1e-12):
    """a = 1 over one chunk: S_out = (I - K^T T B K) S0 + K^T T B V with
    (I - A) T = I, A_ij = -beta_i k_i^T k_j for j < i
    ("Understanding Kimi Delta Attention", box "Where did WY go?")."""
    rng = np.random.default_rng(13)
    C, dk, dv = 12, 6, 5
    q, k, v, g, b = random_inputs(rng, C, 1, dk, dv, g_zero=True)
    s0 = rng.standard_normal((1, 1, dk, dv))
    _, sf = run(q, k, v, g, b, 1.0, s0, [0, C])
    K, V, beta = k[:, 0], v[:, 0], b[:, 0]
    A = -np.tril(beta[:, None] * (K @ K.T), -1)
    Tm = np.linalg.inv(np.eye(C) - A)
    Bm = np.diag(beta)
    S_wy = (np.eye(dk) - K.T @ Tm @ Bm @ K) @ s0[0, 0] + K.T @ Tm @ Bm @ V
    err = rel_err(sf[0, 0], S_wy)
    return err <= tol, "err %.3e" % err


# ----------------------------------------------------------------------------
# P3: beta = 0 is pure per-row decay; half-lives
# ("Kimi Delta Attention: a half-life per channel", "Promote the scalar to a
#  diagonal": Diag(a) scales row c by a[c]).
# ----------------------------------------------------------------------------
def pin_beta_zero(run, tol=1e-12):
    rng = np.random.default_rng(14)
    T, H, dk, dv = 30, 2, 7, 3
    q, k, v, g, _ = random_inputs(rng, T, H, dk, dv, z_range=(0.0, 4.0))
    b = np.zeros((T, H))
    s0 = rng.standard_normal((1, H, dk, dv))
    o, sf = run(q, k, v, g, b, 0.8, s0, [0, T])
    G = np.cumsum(g, axis=0)  # [T, H, dk]
    o_ref = np.einsum("thr,hrc,thr->thc", np.exp(G), s0[0], 0.8 * q)
    s_ref = np.exp(G[-1])[:, :, None] * s0[0]
    err = max(rel_err(o, o_ref), rel_err(sf[0], s_ref))
    return err <= tol, "err %.3e" % err


def _half_life_tokens(run, alpha):
    """Tokens until a single stored association has decayed below one half."""
    n = int(math.ceil(math.log(2.0) / -math.log(alpha))) + 2
    dk = dv = 1
    g = np.full((n, 1, dk), math.log(alpha))
    z = np.zeros((n, 1, dk))
    s0 = np.ones((1, 1, dk, dv))
    q = np.ones((n, 1, dk))
    o, _ = run(q, z, np.zeros((n, 1, dv)), g, np.zeros((n, 1)), 1.0, s0, [0, n])
    below = np.nonzero(o[:, 0, 0] < 0.5)[0]
    return int(below[0]) + 1 if len(below) else None


def pin_half_lives(run):
    gl = golden("half_lives.json")
    slow = _half_life_tokens(run, gl["alpha_slow"])
    fast = _half_life_tokens(run, gl["alpha_fast"])
    ok = (slow is not None and abs(slow - gl["half_life_slow_about"]) <=
          gl["half_life_slow_rel_tol"] * gl["half_life_slow_about"]
          and fast is not None and fast <= gl["half_life_fast_below"])
    return ok, "slow %s fast %s" % (slow, fast)


def pin_inverse_decay_range(run):
    """1/gamma after 64 / 128 steps of a = 0.9 (orders 10^3 and 10^6)."""
    gl = golden("decay_range.json")
    mags = []
    for n in gl["positions"]:
        g = np.full((n, 1, 1), math.log(gl["alpha"]))
        z = np.zeros((n, 1, 1))
        _, sf = run(np.ones((n, 1, 1)), z, z, g, np.zeros((n, 1)), 1.0,
                    np.ones((1, 1, 1, 1)), [0, n])
        mags.append(int(round(math.log10(1.0 / sf[0, 0, 0, 0]))))
    return mags == gl["inverse_gamma_order_of_magnitude"], "orders %s" % mags


# ----------------------------------------------------------------------------
# P4: overwrite vs additive, partial write
# ("Understanding Kimi Delta Attention", Figure 01; boxes "Does the write
#  work?" and "Try it with numbers").
# ----------------------------------------------------------------------------
def _read_after_write(run, S_read, v_target, beta, dk=4, dv=1, g=None):
    """State with read S^T k = S_read at unit key e_1; one token writes v_target.
    The query equals the key and scale = 1, so o_t = S_t^T k."""
    k = np.zeros((1, 1, dk))
    k[0, 0, 0] = 1.0
    s0 = np.zeros((1, 1, dk, dv))
    s0[0, 0, 0, 0] = S_read
    s0[0, 0, 1:, 0] = 5.0  # other key channels hold unrelated content
    gg = np.zeros((1, 1, dk)) if g is None else g
    o, _ = run(k, k, np.full((1, 1, dv), v_target), gg, np.full((1, 1), beta), 1.0, s0, [0, 1])
    return float(o[0, 0, 0])


def pin_additive_vs_delta(run, tol=1e-12):
    gl = golden("additive_vs_delta.json")
    delta = _read_after_write(run, gl["read_before"], gl["written_value"], 1.0)
    additive = gl["read_before"] + gl["written_value"]  # S + k v^T read at the unit key
    ok = abs(delta - gl["delta_read_after_beta_1"]) <= tol and additive == gl["additive_read_after"] \
        and abs(delta - additive) > 1.0
    return ok, "delta read %r, additive read %r" % (delta, additive)


def pin_partial_write(run, tol=1e-12):
    gl = golden("partial_write.json")
    got = _read_after_write(run, gl["prediction"], gl["target"], gl["beta"])
    return abs(got - gl["read_after"]) <= tol, "read after %r" % got


def pin_read_after_write_general(run, tol=1e-12):
    """Unit key, any decay: S_t^T k = (1 - beta) (Diag(a) S)^T k + beta v.
    The prediction is taken from the DECAYED state ("Understanding Kimi
    Delta Attention": decay before prediction)."""
    rng = np.random.default_rng(15)
    dk, dv = 6, 5
    worst = 0.0
    for _ in range(5):
        k = rng.standard_normal(dk)
        k /= np.linalg.norm(k)
        S = rng.standard_normal((dk, dv))
        v = rng.standard_normal(dv)
        beta = rng.uniform(0, 1)
        a = rng.uniform(0.3, 1.0, dk)
        o, _ = run(k[None, None], k[None, None], v[None, None], np.log(a)[None, None],
                   np.full((1, 1), beta), 1.0, S[None, None], [0, 1])
        v_hat = (a[:, None] * S).T @ k
        worst = max(worst, rel_err(o[0, 0], (1 - beta) * v_hat + beta * v))
    return worst <= tol, "err %.3e" % worst


# ----------------------------------------------------------------------------
# P5: exact overwrite with orthonormal keys (linear attention)
# ("Understanding Kimi Delta Attention", "Learning to overwrite": beta = 1
#  returns v; "A fixed-size associative memory": S^T q = sum_i v_i (k_i^T q)).
# ----------------------------------------------------------------------------
def pin_orthonormal_overwrite(run, tol=1e-12):
    rng = np.random.default_rng(16)
    dk, dv, T = 8, 5, 8
    Qf, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qf.T[:T]                           # orthonormal rows
    V = rng.standard_normal((T, dv))
    qs = rng.standard_normal((T, dk))
    o, sf = run(qs[:, None], K[:, None], V[:, None], np.zeros((T, 1, dk)), np.ones((T, 1)),
                0.25, None, [0, T])
    err_s = rel_err(sf[0, 0], K.T @ V)
    o_lin = np.stack([0.25 * sum((qs[t] @ K[j]) * V[j] for j in range(t + 1)) for t in range(T)])
    reads = np.stack([sf[0, 0].T @ K[j] for j in range(T)])
    err = max(err_s, rel_err(o[:, 0], o_lin), rel_err(reads, V))
    return err <= tol, "err %.3e" % err


# ----------------------------------------------------------------------------
# P6: the delta step is one gradient step on J(S) = 1/2 ||S^T k - v||^2
# ("Understanding Kimi Delta Attention", box "An online reconstruction
#  objective").  The gradient is taken by central differences (exact up to
#  rounding for a quadratic).
# ----------------------------------------------------------------------------
def pin_gradient_step(run, tol=1e-8):
    rng = np.random.default_rng(17)
    dk, dv = 5, 4
    S = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk)
    v = rng.standard_normal(dv)
    beta = 0.7
    J = lambda M: 0.5 * np.sum((M.T @ k - v) ** 2)  # noqa: E731
    grad = np.zeros_like(S)
    eps = 1e-3
    for r in range(dk):
        for c in range(dv):
            E = np.zeros_like(S)
            E[r, c] = eps
            grad[r, c] = (J(S + E) - J(S - E)) / (2 * eps)
    _, sf = run(np.zeros((1, 1, dk)), k[None, None], v[None, None], np.zeros((1, 1, dk)),
                np.full((1, 1), beta), 1.0, S[None, None], [0, 1])
    err = rel_err(sf[0, 0], S - beta * grad)
    return err <= tol, "err %.3e" % err


# ----------------------------------------------------------------------------
# P7: two transitions, F2 F1 = I - b1 k1 k1^T - b2 k2 k2^T + b2 b1 k2 (k2^T k1) k1^T
# ("Understanding Kimi Delta Attention", box "Two transitions already reveal
#  the pattern").  With v = 0 the state after two tokens is F2 F1 S0.
# ----------------------------------------------------------------------------
def pin_two_step_product(run, tol=1e-12):
    rng = np.random.default_rng(18)
    dk, dv = 6, 3
    k1, k2 = rng.standard_normal(dk), rng.standard_normal(dk)
    b1, b2 = 0.6, 0.3
    S0 = rng.standard_normal((dk, dv))
    F = (np.eye(dk) - b1 * np.outer(k1, k1) - b2 * np.outer(k2, k2)
         + b2 * b1 * (k2 @ k1) * np.outer(k2, k1))
    K = np.stack([k1, k2])[:, None]
    _, sf = run(np.zeros((2, 1, dk)), K, np.zeros((2, 1, dv)), np.zeros((2, 1, dk)),
                np.array([[b1], [b2]]), 1.0, S0[None, None], [0, 2])
    err = rel_err(sf[0, 0], F @ S0)
    return err <= tol, "err %.3e" % err


# ----------------------------------------------------------------------------
# P9: a scalar gate (every channel equal) is Gated DeltaNet,
# S_t = alpha_t (I - beta k k^T) S_{t-1} + beta k v^T
# ("Understanding Kimi Delta Attention", "Learning what to forget"; the
#  scalar-gated rule of "Kimi Delta Attention: a half-life per channel").
# ----------------------------------------------------------------------------
def pin_scalar_gate(run, tol=1e-12):
    rng = np.random.default_rng(19)
    T, dk, dv = 25, 6, 4
    q, k, v, _, b = random_inputs(rng, T, 1, dk, dv)
    alpha = rng.uniform(0.5, 1.0, T)
    g = np.repeat(np.log(alpha)[:, None, None], dk, axis=2)
    s0 = rng.standard_normal((1, 1, dk, dv))
    o, sf = run(q, k, v, g, b, 0.4, s0, [0, T])
    S = s0[0, 0].copy()
    o_ref = np.zeros((T, dv))
    for t in range(T):
        kk = k[t, 0][:, None]
        S = alpha[t] * (np.eye(dk) - b[t, 0] * kk @ kk.T) @ S + b[t, 0] * kk @ v[t, 0][None, :]
        o_ref[t] = S.T @ (0.4 * q[t, 0])
    err = max(rel_err(sf[0, 0], S), rel_err(o[:, 0], o_ref))
    return err <= tol, "err %.3e" % err


# ----------------------------------------------------------------------------
# P10: structural invariants ("Understanding Kimi Delta Attention", box "One
# state crosses the chunk boundary": the fixed-size state is all that carries
# over; columns of the value space evolve independently).
# ----------------------------------------------------------------------------
def pin_structure(run, tol=1e-12):
    rng = np.random.default_rng(20)
    lengths = [9, 0, 14, 5]
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)])
    H, dk, dv = 3, 5, 4
    q, k, v, g, b = random_inputs(rng, T, H, dk, dv)
    s0 = rng.standard_normal((len(lengths), H, dk, dv))
    o, sf = run(q, k, v, g, b, 0.5, s0, cu)
    errs = []
    # varlen packing == separate calls; zero-length sequence returns S0
    for n in range(len(lengths)):
        a, e = cu[n], cu[n + 1]
        o1, s1 = run(q[a:e], k[a:e], v[a:e], g[a:e], b[a:e], 0.5, s0[n:n + 1], [0, e - a])
        errs += [rel_err(o[a:e], o1) if e > a else 0.0, rel_err(sf[n], s1[0])]
    errs.append(rel_err(sf[1], s0[1]))
    # split invariance: final state of a prefix continues the sequence
    a, e = cu[2], cu[3]
    m = a + 6
    o_p, s_p = run(q[a:m], k[a:m], v[a:m], g[a:m], b[a:m], 0.5, s0[2:3], [0, m - a])
    o_s, s_s = run(q[m:e], k[m:e], v[m:e], g[m:e], b[m:e], 0.5, s_p, [0, e - m])
    errs += [rel_err(np.concatenate([o_p, o_s]), o[a:e]), rel_err(s_s[0], sf[2])]
    # value-column permutation equivariance and head independence
    perm = rng.permutation(dv)
    o_pm, s_pm = run(q, k, v[..., perm], g, b, 0.5, s0[..., perm], cu)
    errs += [rel_err(o_pm, o[..., perm]), rel_err(s_pm, sf[..., perm])]
    o_h, s_h = run(q[:, 1:2], k[:, 1:2], v[:, 1:2], g[:, 1:2], b[:, 1:2], 0.5, s0[:, 1:2], cu)
    errs += [rel_err(o_h, o[:, 1:2]), rel_err(s_h, sf[:, 1:2])]
    worst = max(errs)
    return worst <= tol, "max err %.3e" % worst


def pin_decode_matches_prefill(run, decode_step, tol=1e-12):
    """T decode steps on (session, head) pairs equal a T-token prefill."""
    rng = np.random.default_rng(21)
    T, N, H, dk, dv = 7, 3, 2, 5, 4
    q, k, v, g, b = random_inputs(rng, T * N, H, dk, dv)
    s0 = rng.standard_normal((N, H, dk, dv))
    cu = [T * n for n in range(N + 1)]
    o, sf = run(q, k, v, g, b, 0.5, s0, cu)
    st = s0.copy()
    errs = []
    for t in range(T):
        idx = [n * T + t for n in range(N)]
        od, st = decode_step(q[idx], k[idx], v[idx], g[idx], b[idx], 0.5, st)
        errs.append(rel_err(od, o[idx]))
    errs.append(rel_err(st, sf))
    worst = max(errs)
    return worst <= tol, "max err %.3e" % worst


RUN_PINS = [
    pin_deltanet, pin_wy_no_decay, pin_beta_zero, pin_half_lives, pin_inverse_decay_range,
    pin_additive_vs_delta, pin_partial_write, pin_read_after_write_general,
    pin_orthonormal_overwrite, pin_gradient_step, pin_two_step_product, pin_scalar_gate,
    pin_structure,
]


def neumann_inverse(A):
    """(I - A)^{-1} = sum_{p < C} A^p for strictly lower triangular A
    ("Understanding Kimi Delta Attention", box "A finite sum of causal paths")."""
    C = A.shape[0]
    out = np.eye(C)
    P = np.eye(C)
    for _ in range(1, C):
        P = P @ A
        out = out + P
    return out

