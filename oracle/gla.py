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
``gla_recurrent_bwd`` (reverse mode through the recurrence) is pinned by torch
autograd of a separately written forward, by central differences, by the textbook
gradients of causal linear attention at zero log-gates, and by ZeCO's chunk-level
state-gradient recurrence and the gate-gradient identity.
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


def gla_recurrent_bwd(q, k, v, log_g, S0, dO, dST=None, ckpt=64):
    """Gradients of the per-token recurrence ``gla_recurrent`` by reverse-mode
    differentiation token by token, in fp64: for the scalar
    L = sum(dO o o) + sum(dST o S_T), returns (dq, dk, dv, dlog_g, dS0).

    Going backward with dS the gradient of L with respect to S_t:
        dS   += do_t q_t^T                    (o_t = S_t q_t)
        dq_t  = S_t^T do_t
        dv_t  = dS k_t,   dk_t = dS^T v_t     (S_t = ... + v_t k_t^T)
        dg_t  = sum_v dS o exp(g_t) o S_{t-1} (per key column)
        dS    = exp(g_t) o dS                 (-> gradient with respect to S_{t-1})
    and dS0 is the final dS. The states S_{t-1}, S_t are recomputed forward from
    checkpoints every ``ckpt`` tokens (no division by decays). ZeCO's backward
    (section "The Backward Algorithm and Gradient Flow") states the chunk-level
    form of the dS recurrence, dS = gamma o dS + Q~^T dO; a test checks it.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    lg = np.asarray(log_g, np.float64)
    dO = np.asarray(dO, np.float64)
    N, T, dk = k.shape
    dv = v.shape[2]
    S = np.zeros((N, dv, dk)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    marks = {}
    for t in range(T):
        if t % ckpt == 0:
            marks[t] = S.copy()
        S = np.exp(lg[:, t])[:, None, :] * S + v[:, t][:, :, None] * k[:, t][:, None, :]
    dS = np.zeros((N, dv, dk)) if dST is None else np.array(dST, dtype=np.float64, copy=True)
    dq, dk_, dv_, dg = (np.empty_like(q), np.empty_like(k), np.empty_like(v), np.empty_like(lg))
    for c0 in (range(((T - 1) // ckpt) * ckpt, -1, -ckpt) if T else ()):
        c1 = min(T, c0 + ckpt)
        states = [marks[c0]]                              # S_{c0-1}, S_{c0}, ..., S_{c1-1}
        for t in range(c0, c1):
            states.append(np.exp(lg[:, t])[:, None, :] * states[-1]
                          + v[:, t][:, :, None] * k[:, t][:, None, :])
        for t in range(c1 - 1, c0 - 1, -1):
            St, Sp = states[t - c0 + 1], states[t - c0]
            dS = dS + dO[:, t][:, :, None] * q[:, t][:, None, :]
            dq[:, t] = np.einsum("nvk,nv->nk", St, dO[:, t])
            dv_[:, t] = np.einsum("nvk,nk->nv", dS, k[:, t])
            dk_[:, t] = np.einsum("nvk,nv->nk", dS, v[:, t])
            e = np.exp(lg[:, t])
            dg[:, t] = np.einsum("nvk,nvk->nk", dS, Sp) * e
            dS = e[:, None, :] * dS
    return dq, dk_, dv_, dg, dS
