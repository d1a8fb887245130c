"""fp64 oracle for the elementwise steps of a KDA layer around the recurrence
(test infrastructure only: only tests, the smoke check and the benchmark's
CPU-baseline leg may call this module; the GPU path never imports it).

The pages place these steps around the core without fixing every detail:

* queries and keys are normalised before the recurrence ("Kimi Delta
  Attention: How It Works, Step by Step", question 16; "Demystifying Kimi
  Delta Attention" notes the keys are normalised).  Reading taken: L2
  normalisation over the d_k channels of each (token, head), x / sqrt(sum x^2
  + eps);
* the per-channel retention is a sigmoid of a projection ("Kimi Delta
  Attention: a half-life per channel", section "Promote the scalar to a
  diagonal": a_t = sigmoid(x_t W_a)), so log a = log sigmoid(x);
* the write strength lies in [0, 1]; reading taken: beta = sigmoid(x);
* after the recurrence the layer applies output gating and RMS normalisation
  ("Understanding Kimi Delta Attention", section "From mathematics to the
  GPU").  Reading taken: out = o / sqrt(mean o^2 + eps) * weight *
  sigmoid(gate) over the d_v channels of each (token, head).

Each function is the plain definition, evaluated in float64; log sigmoid uses
the overflow-free form min(x, 0) - log1p(exp(-|x|)), which equals
log(1 / (1 + exp(-x))) exactly in real arithmetic.
"""
from __future__ import annotations

import numpy as np

__all__ = ["l2norm", "log_sigmoid", "sigmoid", "output_rmsnorm_gate", "inputs_in_plain_form"]


def l2norm(x, eps):
    """x / sqrt(sum over the last axis of x^2 + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).sum(axis=-1, keepdims=True) + eps)


def log_sigmoid(x):
    """log(sigmoid(x)) = -log(1 + e^-x), without overflow for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    """1 / (1 + e^-x)."""
    x = np.asarray(x, dtype=np.float64)
    return np.exp(log_sigmoid(x))


def output_rmsnorm_gate(o, gate, weight, eps):
    """o / sqrt(mean over the last axis of o^2 + eps) * weight * sigmoid(gate)."""
    o = np.asarray(o, dtype=np.float64)
    rms = np.sqrt((o * o).mean(axis=-1, keepdims=True) + eps)
    return o / rms * np.asarray(weight, dtype=np.float64) * sigmoid(gate)


def inputs_in_plain_form(q, k, g, beta, *, d_k, gate="per_channel", gate_is_logit=False,
                         beta_is_logit=False, l2norm_qk=False, eps=1e-6):
    """Maps inputs given in one of the layer's forms to the plain operator's
    inputs (normalised q, k; per-channel log-decay; write strength), in fp64.

    gate: "per_channel" (g [..., d_k]), "scalar" (g [...], one value shared by
    the d_k channels) or "none" (g ignored: log a = 0)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if l2norm_qk:
        q, k = l2norm(q, eps), l2norm(k, eps)
    if gate == "none":
        g_full = np.zeros(k.shape)
    else:
        g = np.asarray(g, dtype=np.float64)
        if gate_is_logit:
            g = log_sigmoid(g)
        g_full = np.repeat(g[..., None], d_k, axis=-1) if gate == "scalar" else g
    beta = np.asarray(beta, dtype=np.float64)
    if beta_is_logit:
        beta = sigmoid(beta)
    return q, k, g_full, beta
