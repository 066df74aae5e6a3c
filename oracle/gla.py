"""Gated linear attention, per token and per chunk, in fp64 (test infrastructure).

Source: "ZeCO: Zero Communication Overhead Sequence Parallelism for Linear
Attention" (paper summary), section "Gated Linear Attention (GLA) Formulation":
each token decays the state by a per-key-dimension factor alpha_t in (0,1)^{d_k}
and adds the outer product of its key and value; the output reads the state with
the query. In the ``d_v x d_k`` orientation used here, with log-gates
g_t = log alpha_t:

    S_t[v, k] = exp(g_t[k]) * S_{t-1}[v, k] + v_t[v] * k_t[k],
    o_t       = S_t q_t                       (inclusive read-out).

The shard starts from an incoming state S_0, which is how a device's local
sequence enters in that page's section "Global State Update Formula" (eq. 6).

``gla_recurrent`` is the definition and the parity reference. ``gla_chunk`` is
the page's chunk form (state recurrence over chunks, inter- plus intra-chunk
output), kept to pin the reading of the intra-chunk key scaling: the section
prints K o Gamma, the forward algorithm's description divides the keys by
Lambda; only the latter equals the recurrence, which a test checks.

Pins (tests/test_oracle_gla.py): with zero log-gates the output is the textbook
causal linear attention tril(Q K^T) V + Q S_0^T; eq. 6 (final state from S_0 is
the decayed S_0 plus the state from zero); the decay acts on key columns; one
token from zero gives v (k . q); chunk form == recurrence for C in {1, 16, 64}.
"""
from __future__ import annotations

import numpy as np


def gla_recurrent(q, k, v, log_g, S0=None):
    """q, k, log_g: [N][T][d_k]; v: [N][T][d_v]; S0: [N][d_v][d_k] or None.
    Returns (o [N][T][d_v], S_T [N][d_v][d_k]) in fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    lg = np.asarray(log_g, np.float64)
    N, T, dk = k.shape
    dv = v.shape[2]
    S = np.zeros((N, dv, dk)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    o = np.empty((N, T, dv))
    for t in range(T):
        S = np.exp(lg[:, t])[:, None, :] * S + v[:, t][:, :, None] * k[:, t][:, None, :]
        o[:, t] = np.einsum("nvk,nk->nv", S, q[:, t])
    return o, S


def gla_chunk(q, k, v, log_g, S0=None, chunk=64):
    """The chunk form, with in-chunk cumulative log-decay b (inclusive):
    Lambda = exp(b), Gamma = exp(b_C - b), gamma = exp(b_C);
    O = (Q o Lambda) S^T + [((Q o Lambda)(K / Lambda)^T) o M] V,
    S <- gamma (on key columns) o S + ((K o Gamma)^T V)^T.
    T must be a multiple of ``chunk``."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    lg = np.asarray(log_g, np.float64)
    N, T, dk = k.shape
    dv = v.shape[2]
    if T % chunk:
        raise ValueError("T must be a multiple of chunk")
    M = np.tril(np.ones((chunk, chunk)))
    o = np.empty((N, T, dv))
    S = np.zeros((N, dv, dk)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    for c0 in range(0, T, chunk):
        sl = slice(c0, c0 + chunk)
        b = np.cumsum(lg[:, sl], axis=1)                  # [N][C][d_k]
        Qt = q[:, sl] * np.exp(b)                          # Q o Lambda
        Kt = k[:, sl] * np.exp(-b)                         # K / Lambda
        Kg = k[:, sl] * np.exp(b[:, -1:, :] - b)           # K o Gamma
        A = np.einsum("nrk,njk->nrj", Qt, Kt) * M
        o[:, sl] = np.einsum("nrk,nvk->nrv", Qt, S) + np.einsum("nrj,njv->nrv", A, v[:, sl])
        S = np.exp(b[:, -1])[:, None, :] * S + np.einsum("njv,njk->nvk", v[:, sl], Kg)
    return o, S
