"""Brute-force fp64 reference for tiny inputs -- TEST INFRASTRUCTURE ONLY.

A second, independent route to the same definition as `kda_oracle.c`: it
forms every token's dk x dk transition matrix explicitly,
A_t = (I - beta_t k_t k_t^T) Diag(alpha_t) with alpha_t = exp(g_t), and
multiplies matrices, where the C oracle applies the forget / erase / write
steps of page "Exercices", Niveau 2 Q7 to the state in place.  The KCP pair
of a segment (page "Exercices", Niveau 3 Q21) is the product of its A_t and
the state it builds from zero.  Only for dk, dv of a few dozen and short
sequences.
"""
from __future__ import annotations

import numpy as np


def _np(x):
    import torch
    if isinstance(x, torch.Tensor):
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def transition(k_t, g_t, beta_t):
    """A_t = (I - beta k k^T) Diag(exp(g))."""
    k_t = np.asarray(k_t, dtype=np.float64)
    dk = k_t.size
    return (np.eye(dk) - beta_t * np.outer(k_t, k_t)) @ np.diag(np.exp(g_t))


def sequence(q, k, v, g, beta, z=None, S0=None, scale=1.0):
    """One head: q, k [T, dk]; v, z [T, dv]; g [T, dk]; beta [T].  Returns (y [T, dv], S_T)."""
    q, k, v, g, beta = _np(q), _np(k), _np(v), _np(g), _np(beta)
    z = None if z is None else _np(z)
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else _np(S0).copy()
    y = np.zeros((T, dv))
    for t in range(T):
        S = transition(k[t], g[t], beta[t]) @ S + beta[t] * np.outer(k[t], v[t])
        o = scale * (S.T @ q[t])
        if z is not None:
            o = o / (1.0 + np.exp(-z[t]))
        y[t] = o
    return y, S


def _sigmoid_tanh(x):
    """sigmoid(x) = (1 + tanh(x / 2)) / 2, a route independent of exp."""
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def fused_sequence(q_raw, k_raw, v, a, b, z=None, S0=None, scale=1.0, eps=1e-6, g_min=-5.0):
    """One head from raw inputs: unit q and k by x / hypot(||x||, sqrt(eps)),
    g = g_min sigmoid(a), beta = sigmoid(b) (sigmoid through tanh), then
    `sequence`.  q_raw, k_raw, a [T, dk]; v, z [T, dv]; b [T]."""
    q_raw, k_raw, a, b = _np(q_raw), _np(k_raw), _np(a), _np(b)
    se = np.sqrt(eps)
    qh = np.stack([x / np.hypot(np.linalg.norm(x), se) for x in q_raw])
    kh = np.stack([x / np.hypot(np.linalg.norm(x), se) for x in k_raw])
    return sequence(qh, kh, v, g_min * _sigmoid_tanh(a), _sigmoid_tanh(b), z, S0, scale)


def pair(k, v, g, beta):
    """KCP pair (M, Sloc) of one head's segment: M = A_T ... A_1, Sloc from zero."""
    k, v, g, beta = _np(k), _np(v), _np(g), _np(beta)
    T, dk = k.shape
    M = np.eye(dk)
    Sloc = np.zeros((dk, v.shape[1]))
    for t in range(T):
        A = transition(k[t], g[t], beta[t])
        M = A @ M
        Sloc = A @ Sloc + beta[t] * np.outer(k[t], v[t])
    return M, Sloc
