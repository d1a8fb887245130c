"""Pins for the gradient oracle (oracle/backward.py).  CPU only.

* The autograd gradients of the recurrence are pinned to central finite
  differences of oracle.reference.recurrent, a forward written separately.
* The hand-derived chunkwise backward is pinned to the autograd gradients on
  random inputs (several chunk sizes, packed and empty sequences, strong
  decays), so a dropped term, a wrong sign or a transposed operand anywhere in
  the derivation shows up.
* Special cases with known answers.
"""
import numpy as np
import pytest

from oracle import backward as B
from oracle import reference as R

NAMES = ("q", "k", "v", "g", "beta")


def inputs(T, H, dk, dv, seed, g_range=(-1.0, 0.0), n_seqs=1):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(T, H, dk)) / np.sqrt(dk)
    k = rng.normal(size=(T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.normal(size=(T, H, dv))
    g = rng.uniform(*g_range, size=(T, H, dk))
    beta = rng.uniform(0.1, 0.9, size=(T, H))
    s0 = 0.3 * rng.normal(size=(n_seqs, H, dk, dv))
    do = rng.normal(size=(T, H, dv))
    dfin = rng.normal(size=(n_seqs, H, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta), s0, do, dfin


def loss(x, s0, do, dfin, scale, cu=None):
    o, fin = R.recurrent(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, s0, cu)
    return float((o * do).sum() + (fin * dfin).sum())


def rel(a, b):
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


@pytest.mark.parametrize("cu", [None, [0, 2, 2, 6]])
def test_autograd_matches_finite_differences(cu):
    n_seqs = 1 if cu is None else len(cu) - 1
    x, s0, do, dfin = inputs(6, 1, 3, 2, seed=3, n_seqs=n_seqs)
    scale = 0.7
    gr = B.recurrent_grads(x["q"], x["k"], x["v"], x["g"], x["beta"], scale, do, s0, dfin, cu)
    h = 1e-6
    for name in NAMES + ("s0",):
        base = s0 if name == "s0" else x[name]
        fd = np.zeros(base.shape)
        for idx in np.ndindex(base.shape):
            vals = []
            for sgn in (1.0, -1.0):
                pert = base.copy()
                pert[idx] += sgn * h
                if name == "s0":
                    vals.append(loss(x, pert, do, dfin, scale, cu))
                else:
                    vals.append(loss(dict(x, **{name: pert}), s0, do, dfin, scale, cu))
            fd[idx] = (vals[0] - vals[1]) / (2 * h)
        key = "dinitial_state" if name == "s0" else "d" + name
        assert rel(gr[key], fd) < 1e-7, (name, rel(gr[key], fd))


@pytest.mark.parametrize("chunk", [1, 4, 7, 16, 64])
def test_chunkwise_backward_matches_autograd(chunk):
    x, s0, do, dfin = inputs(37, 2, 6, 5, seed=11)
    a = B.recurrent_grads(*(x[n] for n in NAMES), 0.5, do, s0, dfin)
    c = B.chunkwise_grads(*(x[n] for n in NAMES), 0.5, chunk, do, s0, dfin)
    for key in a:
        assert rel(c[key], a[key]) < 1e-10, (key, rel(c[key], a[key]))


def test_chunkwise_backward_packed_sequences():
    cu = [0, 5, 5, 22, 37]
    x, s0, do, dfin = inputs(37, 2, 4, 3, seed=12, n_seqs=4)
    a = B.recurrent_grads(*(x[n] for n in NAMES), 0.5, do, s0, dfin, cu)
    c = B.chunkwise_grads(*(x[n] for n in NAMES), 0.5, 8, do, s0, dfin, cu)
    for key in a:
        assert rel(c[key], a[key]) < 1e-10, key
    # the empty sequence passes the final-state gradient straight through
    assert np.allclose(c["dinitial_state"][1], dfin[1], rtol=0, atol=0)


def test_chunkwise_backward_strong_decays():
    x, s0, do, dfin = inputs(40, 1, 5, 4, seed=13, g_range=(-5.0, 0.0))
    a = B.recurrent_grads(*(x[n] for n in NAMES), 0.5, do, s0, dfin)
    c = B.chunkwise_grads(*(x[n] for n in NAMES), 0.5, 16, do, s0, dfin)
    for key in a:
        assert rel(c[key], a[key]) < 1e-9, key


def test_zero_beta_gives_no_value_gradient():
    """beta = 0: v never enters the state, so dv = 0 exactly; the write
    strength still has a gradient."""
    x, s0, do, dfin = inputs(20, 1, 4, 3, seed=14)
    x["beta"][:] = 0.0
    c = B.chunkwise_grads(*(x[n] for n in NAMES), 0.5, 8, do, s0, dfin)
    assert np.all(c["dv"] == 0.0)
    assert np.linalg.norm(c["dbeta"]) > 0


def test_gradients_flow_only_through_read_when_queries_vanish():
    """q = 0 and no final-state gradient: the loss does not depend on k, v, g,
    beta or the initial state, while dq = scale S_t do_t is nonzero."""
    x, s0, do, _ = inputs(20, 2, 4, 3, seed=15)
    x["q"][:] = 0.0
    c = B.chunkwise_grads(*(x[n] for n in NAMES), 0.5, 8, do, s0, None)
    for key in ("dk", "dv", "dg", "dbeta", "dinitial_state"):
        assert np.all(c[key] == 0.0), key
    assert np.linalg.norm(c["dq"]) > 0


def test_pins_catch_planted_mistakes():
    """A backward with one step dropped or mis-signed must fail the comparison
    with autograd: here the decay term of Kbar and the sign of dA."""
    x, s0, do, dfin = inputs(30, 1, 4, 3, seed=16)
    a = B.recurrent_grads(*(x[n] for n in NAMES), 0.5, do, s0, dfin)
    orig = B._chunk_backward

    def no_reverse_cumsum(sv, scale, dO, dS):
        gr, dS0 = orig(sv, scale, dO, dS)
        gr["dg"] = np.diff(np.concatenate([gr["dg"], np.zeros((1, gr["dg"].shape[1]))]),
                           axis=0) * -1.0   # dG instead of its reverse cumulative sum
        return gr, dS0

    def wrong_sign_state(sv, scale, dO, dS):
        gr, dS0 = orig(sv, scale, dO, dS)
        return gr, -dS0

    for mutant in (no_reverse_cumsum, wrong_sign_state):
        B._chunk_backward = mutant
        try:
            c = B.chunkwise_grads(*(x[n] for n in NAMES), 0.5, 8, do, s0, dfin)
        finally:
            B._chunk_backward = orig
        assert max(rel(c[key], a[key]) for key in a) > 1e-3, mutant.__name__
