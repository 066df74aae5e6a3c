"""Gated DeltaNet recurrence, token by token, in fp64 (test infrastructure).

Source: "LeapQuant: an 8-bit recurrent state that stops rounding every token",
section "The state, from the update rule up": the delta rule erases what the
memory returns for k_t before writing (the fast-weight form), Gated DeltaNet
adds a scalar decay alpha_t in (0,1) per head per token, and in the
``d_v x d_k`` orientation the update reads

    S_t = alpha_t * S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t                                    (read-out after the write).

``gdn_recurrent`` uses the expanded rank-one form of the same update (eq. 3 of
that section, transposed): u_t = beta_t (v_t - alpha_t S_{t-1} k_t),
S_t = alpha_t S_{t-1} + u_t k_t^T. ``gdn_recurrent_explicit`` multiplies by the
explicit matrix (I - beta k k^T) and is meant for small cases; a test checks the
two agree.

Pins (tests/test_oracle_gdn.py): exact rational brute force on 4x4 states;
beta = 1 with a unit key stores v exactly along k; alpha = 1, beta = 0 leaves
the state unchanged; beta = 0 is pure decay; orthonormal keys with
alpha = beta = 1 recall every stored value; the page's own d_k x d_v forms of
the delta rule and of eq. 1.
"""
from __future__ import annotations

import numpy as np


def gdn_recurrent(q, k, v, alpha, beta, S0=None):
    """Run the Gated DeltaNet recurrence over T tokens for N independent heads.

    q, k: [N][T][d_k]; v: [N][T][d_v]; alpha, beta: [N][T]; S0: [N][d_v][d_k]
    or None (zero). Returns (o [N][T][d_v], S_T [N][d_v][d_k]) in fp64.
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
        a = alpha[:, t][:, None]              # [N,1]
        b = beta[:, t][:, None]
        kt, qt, vt = k[:, t], q[:, t], v[:, t]
        Sk = np.einsum("nvk,nk->nv", S, kt)   # S_{t-1} k_t
        u = b * (vt - a * Sk)                 # correction u_t
        S = a[:, :, None] * S + u[:, :, None] * kt[:, None, :]
        o[:, t] = np.einsum("nvk,nk->nv", S, qt)
    return o, S


def gdn_recurrent_explicit(q, k, v, alpha, beta, S0=None):
    """Same recurrence with the explicit (I - beta k k^T) matrix, one head at a
    time. For small cases only (O(T d^3))."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, T, dk = k.shape
    dv = v.shape[2]
    o = np.empty((N, T, dv))
    S_out = np.empty((N, dv, dk))
    for n in range(N):
        S = np.zeros((dv, dk)) if S0 is None else np.array(S0[n], dtype=np.float64)
        for t in range(T):
            kt = k[n, t][:, None]
            P = np.eye(dk) - beta[n, t] * (kt @ kt.T)
            S = alpha[n, t] * (S @ P) + beta[n, t] * (v[n, t][:, None] @ kt.T)
            o[n, t] = S @ q[n, t]
        S_out[n] = S
    return o, S_out


def gdn_chunk_wy(q, k, v, alpha, beta, S0=None, chunk=64):
    """Chunkwise form of the same recurrence (the WY / UT-transform reading).

    The pages give no chunk form for the delta rule; this one is derived from
    eq. 3 by unrolling inside a chunk. With local positions r, j = 1..C,
    g_r = prod_{i<=r} alpha_i, and rows of K, V, Q, U being tokens:

        (I + L) U = diag(beta) V - diag(beta g) K S_0^T,
            L[r, j] = beta_r (g_r / g_j) (k_r . k_j) for j < r, else 0,
        O   = diag(g) Q S_0^T + (M o (g_r / g_j) o Q K^T) U,  M lower incl. diag,
        S_C = g_C S_0 + U^T diag(g_C / g) K.

    Not used for GPU parity (the recurrence is the definition); a test checks
    it equals ``gdn_recurrent`` for C in {1, 16, 64}, which pins this reading.
    Ratios g_r / g_j are formed as exp of differences of cumulative log-decays.
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
    M = np.tril(np.ones((chunk, chunk)))
    I = np.eye(chunk)
    for n in range(N):
        S = np.zeros((dv, dk)) if S0 is None else np.array(S0[n], dtype=np.float64)
        for c0 in range(0, T, chunk):
            sl = slice(c0, c0 + chunk)
            K, V, Q = k[n, sl], v[n, sl], q[n, sl]
            b = beta[n, sl]
            lg = np.cumsum(np.log(alpha[n, sl]))          # log g_r
            g = np.exp(lg)
            ratio = np.exp(np.minimum(lg[:, None] - lg[None, :], 0.0))  # g_r / g_j for j <= r
            L = np.tril(b[:, None] * ratio * (K @ K.T), -1)
            rhs = b[:, None] * V - (b * g)[:, None] * (K @ S.T)
            U = np.linalg.solve(I + L, rhs)
            A = M * ratio * (Q @ K.T)
            o[n, sl] = g[:, None] * (Q @ S.T) + A @ U
            gC = g[-1]
            S = gC * S + U.T @ (np.exp(lg[-1] - lg)[:, None] * K)
        S_out[n] = S
    return o, S_out
