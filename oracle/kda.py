"""Kimi Delta Attention recurrence, token by token, in fp64 (test infrastructure).

Source: "LeapQuant: an 8-bit recurrent state that stops rounding every token",
section "The state, from the update rule up". KDA replaces Gated DeltaNet's scalar
decay with a vector alpha_t, one factor per key channel. The page writes both
models as one update (eq. 1), in its d_k x d_v orientation (keys index rows):

    S_t = Diag(alpha_t) S_{t-1} + beta_t k_t (v_t - S_{t-1}^T (alpha_t o k_t))^T,
    o_t = S_t^T q_t,

and states that KDA's own form (I - beta k k^T) Diag(alpha) S + beta k v^T expands
to it. With the correction u_t = beta_t (v_t - S_{t-1}^T (alpha_t o k_t)) every token
is a decay followed by one rank-one write (eq. 3): S_t = Diag(alpha_t) S_{t-1} +
k_t u_t^T.

This module keeps the states in the library's [d_v][d_k] layout (the transpose of
the page's): S_t = S_{t-1} Diag(alpha_t) + u_t k_t^T, o_t = S_t q_t.

``kda_recurrent`` follows eq. 1 / eq. 3 in that layout. ``kda_recurrent_explicit``
multiplies by KDA's own matrices in the page's orientation and transposes at the
end; it is meant for small cases, and a test checks that the two agree.

Pins (tests/test_oracle_kda.py): exact rational brute force on 4x4 states through
KDA's own matrix form; a vector decay with equal entries is Gated DeltaNet (the
GDN oracle); beta = 0 is pure per-channel decay, S_T = S_0 Diag(prod alpha);
alpha = 1 is the plain delta rule; beta = 1 with a unit key stores v exactly along
k (S_t k_t = v_t).
"""
from __future__ import annotations

import numpy as np


def kda_recurrent(q, k, v, alpha, beta, S0=None):
    """Run the KDA recurrence over T tokens for N independent heads.

    q, k: [N][T][d_k]; v: [N][T][d_v]; alpha: [N][T][d_k] (per key channel);
    beta: [N][T]; S0: [N][d_v][d_k] or None (zero).
    Returns (o [N][T][d_v], S_T [N][d_v][d_k]) in fp64.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    N, T, dk = k.shape
    dv = v.shape[2]
    S = np.zeros((N, dv, dk)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    o = np.empty((N, T, dv))
    for t in range(T):
        a = alpha[:, t]                           # [N, d_k]
        b = beta[:, t][:, None]                   # [N, 1]
        kt, qt, vt = k[:, t], q[:, t], v[:, t]
        u = b * (vt - np.einsum("nvk,nk->nv", S, a * kt))   # correction u_t
        S = S * a[:, None, :] + u[:, :, None] * kt[:, None, :]
        o[:, t] = np.einsum("nvk,nk->nv", S, qt)
    return o, S


def kda_recurrent_explicit(q, k, v, alpha, beta, S0=None):
    """Same recurrence through KDA's own form in the page's d_k x d_v orientation,
    P_t = (I - beta_t k_t k_t^T) Diag(alpha_t), S_t = P_t S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t, one head at a time; the final state is returned transposed to
    [d_v][d_k]. Works on any element type numpy can multiply (fp64 or Fraction
    objects). For small cases only (O(T d^3))."""
    N, T, dk = len(k), len(k[0]), len(k[0][0])
    dv = len(v[0][0])
    exact = not isinstance(k, np.ndarray) or k.dtype == object
    dt = object if exact else np.float64
    o = np.empty((N, T, dv), dtype=dt)
    S_out = np.empty((N, dv, dk), dtype=dt)
    for n in range(N):
        if S0 is None:
            Sk = np.zeros((dk, dv), dtype=dt) if not exact else np.array([[0] * dv for _ in range(dk)], dtype=object)
        else:
            Sk = np.array(S0[n], dtype=dt).T.copy()
        for t in range(T):
            kt = np.array(k[n][t], dtype=dt).reshape(dk, 1)
            vt = np.array(v[n][t], dtype=dt).reshape(dv, 1)
            qt = np.array(q[n][t], dtype=dt).reshape(dk, 1)
            at = np.array(alpha[n][t], dtype=dt)
            bt = beta[n][t]
            eye = np.array([[1 if i == j else 0 for j in range(dk)] for i in range(dk)], dtype=dt)
            diag = np.array([[at[i] if i == j else 0 for j in range(dk)] for i in range(dk)], dtype=dt)
            P = (eye - bt * (kt @ kt.T)) @ diag
            Sk = P @ Sk + bt * (kt @ vt.T)
            o[n, t] = (Sk.T @ qt).reshape(dv)
        S_out[n] = Sk.T
    return o, S_out


def kda_chunk_wy(q, k, v, alpha, beta, S0=None, chunk=64):
    """Chunkwise form of the KDA recurrence (UT-transform reading; the pages print
    no chunk form). Unrolling eq. 3 with per-channel decays inside a chunk, with
    local positions r, j, b_r = sum_{i<=r} log alpha_i (a vector over key channels)
    and Gamma_r = exp(b_r), rows of K, V, Q, U being tokens:

        (I + L) U = diag(beta) V - diag(beta) (K o Gamma) S_0^T,
            L[r, j] = beta_r sum_c k_r[c] k_j[c] exp(b_r[c] - b_j[c]) for j < r,
        O   = (Q o Gamma) S_0^T + A U,
            A[r, j] = sum_c q_r[c] k_j[c] exp(b_r[c] - b_j[c]) for j <= r,
        S_C = S_0 Diag(Gamma_C) + U^T (K o exp(b_C - b)).

    This is the Gated DeltaNet chunk form with the decay moved inside the key and
    query products, as gated linear attention carries it. Not used for GPU parity
    (the recurrence is the definition); a test checks it equals ``kda_recurrent``.
    T must be a multiple of ``chunk``.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    N, T, dk = k.shape
    dv = v.shape[2]
    if T % chunk:
        raise ValueError("T must be a multiple of chunk")
    o = np.empty((N, T, dv))
    S_out = np.empty((N, dv, dk))
    I = np.eye(chunk)
    for n in range(N):
        S = np.zeros((dv, dk)) if S0 is None else np.array(S0[n], dtype=np.float64)
        for c0 in range(0, T, chunk):
            sl = slice(c0, c0 + chunk)
            K, V, Q = k[n, sl], v[n, sl], q[n, sl]
            bt = beta[n, sl]
            b = np.cumsum(np.log(alpha[n, sl]), axis=0)           # [C][d_k]
            diff = b[:, None, :] - b[None, :, :]                   # b_r - b_j
            low = np.tril(np.ones((chunk, chunk), bool))
            E = np.where(low[:, :, None], np.exp(np.minimum(diff, 0.0)), 0.0)   # j <= r only
            G = np.einsum("rc,jc,rjc->rj", K, K, E)
            L = np.tril(bt[:, None] * G, -1)
            A = np.einsum("rc,jc,rjc->rj", Q, K, E)
            Gam = np.exp(b)
            rhs = bt[:, None] * V - bt[:, None] * ((K * Gam) @ S.T)
            U = np.linalg.solve(I + L, rhs)
            o[n, sl] = (Q * Gam) @ S.T + A @ U
            S = S * Gam[-1][None, :] + U.T @ (K * np.exp(b[-1] - b))
        S_out[n] = S
    return o, S_out
