"""Pins for the layer-step oracle (oracle/layer.py): closed forms, identities
and special cases that a plausible mistake (a sign, an axis, a mean for a sum,
a missing epsilon) would break.  CPU only."""
import math

import numpy as np
import pytest

from oracle import layer as L

RNG = np.random.default_rng(2024)


# ---------------------------------------------------------------- log sigmoid, sigmoid
def test_log_sigmoid_matches_its_definition_where_that_is_representable():
    x = np.linspace(-30.0, 30.0, 601)
    naive = np.array([math.log(1.0 / (1.0 + math.exp(-t))) for t in x])
    # the naive form loses relative precision where log sigmoid(x) ~ -e^-x is tiny
    assert np.allclose(L.log_sigmoid(x), naive, rtol=1e-12, atol=1e-15)


def test_log_sigmoid_extremes():
    # -log(1 + e^800) = -800 - log(1 + e^-800) = -800 to double precision; the
    # naive formula overflows there.
    assert L.log_sigmoid(-800.0) == -800.0
    assert L.log_sigmoid(800.0) == 0.0
    assert L.log_sigmoid(0.0) == pytest.approx(-math.log(2.0), rel=1e-15)


def test_sigmoid_identities():
    x = RNG.normal(size=1000) * 10
    assert np.allclose(L.sigmoid(x) + L.sigmoid(-x), 1.0, rtol=0, atol=1e-15)
    assert L.sigmoid(0.0) == 0.5
    assert np.all((L.sigmoid(x) > 0) & (L.sigmoid(x) < 1) | (np.abs(x) > 36))


def test_log_sigmoid_equals_the_workload_decay():
    """The synthetic inputs draw log a as -log1p(e^-z) (an independent
    formula); for every z the two must agree."""
    z = RNG.uniform(-20, 20, size=2000)
    assert np.allclose(L.log_sigmoid(z), -np.log1p(np.exp(-z)), rtol=1e-13, atol=0)


def test_sigmoid_retention_gives_the_half_life_of_the_pages():
    """a = sigmoid(z) = 0.9 has a half-life of log(1/2) / log(0.9) = 6.58 steps
    ("Kimi Delta Attention: a half-life per channel")."""
    z = math.log(0.9 / 0.1)
    assert math.log(0.5) / L.log_sigmoid(z) == pytest.approx(6.5788, abs=1e-4)


# ---------------------------------------------------------------- L2 normalisation
def test_l2norm_gives_unit_rows_and_keeps_direction():
    x = RNG.normal(size=(7, 3, 128)) * RNG.uniform(0.1, 10, size=(7, 3, 1))
    y = L.l2norm(x, 0.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, atol=1e-14)
    ratio = x / y
    assert np.allclose(ratio, ratio[..., :1], rtol=1e-13)


def test_l2norm_epsilon():
    x = RNG.normal(size=(5, 16))
    eps = 0.25
    n = np.linalg.norm(x, axis=-1)
    assert np.allclose(np.linalg.norm(L.l2norm(x, eps), axis=-1), n / np.sqrt(n * n + eps),
                       rtol=1e-14)
    assert np.all(L.l2norm(np.zeros((2, 8)), 1e-6) == 0.0)


# ---------------------------------------------------------------- output stage
def test_output_stage_special_cases():
    w = RNG.uniform(0.5, 2.0, size=8)
    ones = np.ones((3, 8))
    # a constant row of ones has RMS 1: the output is weight x sigmoid(gate)
    g = RNG.normal(size=(3, 8))
    assert np.allclose(L.output_rmsnorm_gate(ones, g, w, 0.0), w * L.sigmoid(g), rtol=1e-15)
    # gate 0 halves; a saturated gate passes the normalised row
    o = RNG.normal(size=(4, 8))
    a = L.output_rmsnorm_gate(o, np.zeros_like(o), np.ones(8), 0.0)
    b = L.output_rmsnorm_gate(o, np.full_like(o, 60.0), np.ones(8), 0.0)
    assert np.allclose(a, 0.5 * b, rtol=1e-15)
    assert np.allclose(np.sqrt((b * b).mean(axis=-1)), 1.0, rtol=1e-14)
    # invariant to the scale of o (eps = 0), and eps only shrinks
    assert np.allclose(L.output_rmsnorm_gate(3.7 * o, g[:1].repeat(4, 0), w, 0.0),
                       L.output_rmsnorm_gate(o, g[:1].repeat(4, 0), w, 0.0), rtol=1e-14)
    big = L.output_rmsnorm_gate(o, np.zeros_like(o), np.ones(8), 1.0)
    assert np.all(np.abs(big) <= np.abs(a) + 1e-15)


# ---------------------------------------------------------------- the form mapping
def test_inputs_in_plain_form():
    T, H, d = 10, 3, 16
    q, k = RNG.normal(size=(T, H, d)), RNG.normal(size=(T, H, d))
    gs, b = RNG.normal(size=(T, H)), RNG.normal(size=(T, H))
    q1, k1, g1, b1 = L.inputs_in_plain_form(q, k, gs, b, d_k=d, gate="scalar",
                                            gate_is_logit=True, beta_is_logit=True,
                                            l2norm_qk=True, eps=1e-6)
    assert np.allclose(np.linalg.norm(q1, axis=-1), 1.0, atol=1e-6)
    assert np.allclose(np.linalg.norm(k1, axis=-1), 1.0, atol=1e-6)
    assert g1.shape == (T, H, d) and np.all(g1 == L.log_sigmoid(gs)[..., None])
    assert np.all(b1 == L.sigmoid(b))
    _, _, g0, b0 = L.inputs_in_plain_form(q, k, None, b, d_k=d, gate="none")
    assert np.all(g0 == 0.0) and np.all(b0 == b)
    q2, k2, g2, _ = L.inputs_in_plain_form(q, k, RNG.normal(size=(T, H, d)), b, d_k=d)
    assert np.all(q2 == q) and np.all(k2 == k) and g2.shape == (T, H, d)


# ---------------------------------------------------------------- planted mistakes
def test_pins_catch_planted_mistakes():
    x = np.linspace(-5, 5, 101)
    assert not np.allclose(np.log(1 - L.sigmoid(x)), L.log_sigmoid(x))   # log(1 - sigmoid)
    y = RNG.normal(size=(4, 32))
    rms_instead_of_norm = y / np.sqrt((y * y).mean(axis=-1, keepdims=True))
    assert not np.allclose(np.linalg.norm(rms_instead_of_norm, axis=-1), 1.0, atol=1e-6)
    wrong_axis = y / np.sqrt((y * y).mean(axis=0, keepdims=True))
    assert not np.allclose(wrong_axis, L.output_rmsnorm_gate(y, np.full_like(y, 60.0),
                                                             np.ones(32), 0.0), rtol=1e-6)
