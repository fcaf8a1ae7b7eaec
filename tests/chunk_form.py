"""Chunkwise WY/UT form of the gated delta rule in fp64 numpy.

A second, independent statement of the method, used only to pin the oracle
(which is the plain token recurrence).  It follows the step list of the page
"Add parallel chunked prefill for channelwise gated delta rule" (executorch
PR #21061, Summary): per-channel log-decay prefixes, causal query/key terms,
the beta-folded triangular transform, WY pseudo-keys and pseudo-values, and
the inter-chunk state carry, with a short final chunk handled by the same
code.  The formulas are the plain reading of those step names; for a chunk of
L <= C tokens entered with state S:

    Gamma_r = sum_{s<=r} g_s                      (per key channel)
    Qt = Q*e^Gamma, Kt = K*e^Gamma, Kh = K*e^-Gamma, Ke = K*e^(Gamma_L - Gamma)
    A  = strict_lower(diag(beta) Kt Kh^T)
    Tm = (I + A)^-1
    W  = Tm diag(beta) Kt,   Ut = Tm diag(beta) V
    U  = Ut - W S
    O  = scale * (Qt S + lower(Qt Kh^T) U)
    S' = diag(e^Gamma_L) S + Ke^T U

The input handling (L2 normalisation, gates, head repeat) is restated here
with numpy rather than shared with the oracle.
"""
from __future__ import annotations

import math

import numpy as np

GATE_CHANNEL, GATE_SCALAR, GATE_SCALAR_FUSED = 0, 1, 2


def _l2n(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)


def log_decay(gate_kind, gate_in, dk, A_log=None, dt_bias=None):
    """g [B,T,H_v,dk] from any gate kind (sequence layout)."""
    g = np.asarray(gate_in, np.float64)
    if gate_kind == GATE_CHANNEL:
        return g
    if gate_kind == GATE_SCALAR_FUSED:
        z = g + np.asarray(dt_bias, np.float64)[None, None, :]
        sp = np.where(z > 0, z + np.log1p(np.exp(-np.abs(z))), np.log1p(np.exp(np.minimum(z, 0))))
        g = -np.exp(np.asarray(A_log, np.float64))[None, None, :] * sp
    return np.repeat(g[..., None], dk, axis=-1)


def chunked(q, k, v, gate_kind, gate_in, beta_logit, state0=None, A_log=None, dt_bias=None,
            scale=1.0, l2norm=True, chunk=64):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, Hqk, dk = q.shape
    Hv, dv = v.shape[2], v.shape[3]
    rep = Hv // Hqk
    if l2norm:
        q, k = _l2n(q), _l2n(k)
    g = log_decay(gate_kind, gate_in, dk, A_log, dt_bias)
    beta = 1.0 / (1.0 + np.exp(-np.asarray(beta_logit, np.float64)))
    S_all = np.zeros((B, Hv, dk, dv)) if state0 is None else np.array(state0, np.float64)
    o = np.zeros((B, T, Hv, dv))
    for b in range(B):
        for h in range(Hv):
            S = S_all[b, h]
            hq = h // rep
            for t0 in range(0, T, chunk):
                t1 = min(T, t0 + chunk)
                L = t1 - t0
                Q = q[b, t0:t1, hq]
                K = k[b, t0:t1, hq]
                V = v[b, t0:t1, h]
                bt = beta[b, t0:t1, h]
                G = np.cumsum(g[b, t0:t1, h], axis=0)
                Qt, Kt, Kh = Q * np.exp(G), K * np.exp(G), K * np.exp(-G)
                Ke = K * np.exp(G[-1][None, :] - G)
                A = np.tril(bt[:, None] * (Kt @ Kh.T), -1)
                Tm = np.linalg.inv(np.eye(L) + A)
                W = Tm @ (bt[:, None] * Kt)
                Ut = Tm @ (bt[:, None] * V)
                U = Ut - W @ S
                o[b, t0:t1, h] = scale * (Qt @ S + np.tril(Qt @ Kh.T) @ U)
                S = np.exp(G[-1])[:, None] * S + Ke.T @ U
            S_all[b, h] = S
    return o, S_all


def stable_softplus(z: float) -> float:
    return z + math.log1p(math.exp(-z)) if z > 0 else math.log1p(math.exp(z))
