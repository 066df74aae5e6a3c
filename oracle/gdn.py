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

``gdn_recurrent_bwd`` (reverse mode through the rank-one form) is pinned by torch
autograd of a separately written forward (the explicit matrix form), by central
differences, and by the closed form at alpha = 1, beta = 0 (a constant state).
``gdn_chunk_wy_bwd`` is the chunk-form backward that the GPU follows (pages
silent; derived from the chunk form below), pinned by equality with the
reverse-mode gradients.
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


def gdn_recurrent_bwd(q, k, v, alpha, beta, S0, dO, dST=None, ckpt=64):
    """Gradients of ``gdn_recurrent`` by reverse-mode differentiation token by token,
    in fp64: for the scalar L = sum(dO o o) + sum(dST o S_T), returns
    (dq, dk, dv, dalpha, dbeta, dS0).

    Forward step (rank-one form): y = S_{t-1} k_t, u_t = beta_t (v_t - alpha_t y),
    S_t = alpha_t S_{t-1} + u_t k_t^T, o_t = S_t q_t. Going backward with dS the
    gradient with respect to S_t:
        dS    += do_t q_t^T;           dq_t = S_t^T do_t
        du     = dS k_t;               dk_t = dS^T u_t
        dv_t   = beta_t du;            dbeta_t = du . (v_t - alpha_t y)
        dy     = -alpha_t beta_t du;   dk_t += S_{t-1}^T dy
        dalpha_t = sum(dS o S_{t-1}) - beta_t du . y
        dS     = alpha_t dS + dy k_t^T   (-> gradient with respect to S_{t-1})
    The states are recomputed forward from checkpoints every ``ckpt`` tokens.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    dO = np.asarray(dO, np.float64)
    N, T, dk = k.shape
    dv = v.shape[2]

    def step(S, t):
        y = np.einsum("nvk,nk->nv", S, k[:, t])
        u = beta[:, t][:, None] * (v[:, t] - alpha[:, t][:, None] * y)
        return alpha[:, t][:, None, None] * S + u[:, :, None] * k[:, t][:, None, :], y, u

    S = np.zeros((N, dv, dk)) if S0 is None else np.array(S0, dtype=np.float64, copy=True)
    marks = {}
    for t in range(T):
        if t % ckpt == 0:
            marks[t] = S.copy()
        S = step(S, t)[0]
    dS = np.zeros((N, dv, dk)) if dST is None else np.array(dST, dtype=np.float64, copy=True)
    dq, dk_, dv_ = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    da, db = np.empty_like(alpha), np.empty_like(beta)
    for c0 in (range(((T - 1) // ckpt) * ckpt, -1, -ckpt) if T else ()):
        c1 = min(T, c0 + ckpt)
        states, ys, us = [marks[c0]], [], []
        for t in range(c0, c1):
            Sn, y, u = step(states[-1], t)
            states.append(Sn)
            ys.append(y)
            us.append(u)
        for t in range(c1 - 1, c0 - 1, -1):
            i = t - c0
            St, Sp, y, u = states[i + 1], states[i], ys[i], us[i]
            a, b = alpha[:, t][:, None], beta[:, t][:, None]
            dS = dS + dO[:, t][:, :, None] * q[:, t][:, None, :]
            dq[:, t] = np.einsum("nvk,nv->nk", St, dO[:, t])
            du = np.einsum("nvk,nk->nv", dS, k[:, t])
            dk_[:, t] = np.einsum("nvk,nv->nk", dS, u)
            dv_[:, t] = b * du
            db[:, t] = np.einsum("nv,nv->n", du, v[:, t] - a * y)
            dy = -a * b * du
            dk_[:, t] += np.einsum("nvk,nv->nk", Sp, dy)
            da[:, t] = np.einsum("nvk,nvk->n", dS, Sp) - beta[:, t] * np.einsum("nv,nv->n", du, y)
            dS = a[:, :, None] * dS + dy[:, :, None] * k[:, t][:, None, :]
    return dq, dk_, dv_, da, db, dS


def gdn_chunk_wy_bwd(q, k, v, alpha, beta, S0, dO, dST=None, chunk=64):
    """Chunk-form backward of ``gdn_chunk_wy`` (the pages give none; derived here).

    Per chunk, with the forward's T, W, U~, U = U~ - W S_0^T, A = M o (g_r/g_j) o QK^T
    and K^ = diag(g_C/g) K, and dS the gradient with respect to the state after the
    chunk:
        dU  = A^T dO + K^ dS^T
        dA  = (dO U^T) o M,   dA' = dA o (g_r/g_j)
        dQ  = dA' K + diag(g) dO S_0
        dK  = dA'^T Q + diag(g_C/g) U dS + diag(beta g) T^T dW + dL' K + dL'^T K
        dW  = -dU S_0,  dV = diag(beta) T^T dU
        dL  = -(T^T dW W^T + T^T dU U~^T) o strict_lower,  dL' = dL o (g_r/g_j) o beta_r
        dbeta = g o rowdot(T^T dW, K) + rowdot(T^T dU, V) + rowsum(dL o (g_r/g_j) o KK^T)
        dS_0 = g_C dS + dO^T diag(g) Q - dU^T W        (the state-gradient scan)
    The decay enters the recurrence only through q_t e^{B_t} and v_t e^{-B_t} (B the
    cumulative log-decay over the sequence; dividing S_t by e^{B_t} removes the decay),
    so dL/dB_t = q_t . dq_t - v_t . dv_t and d log alpha_t = sum_{s >= t} dL/dB_s.
    The part of that sum beyond the chunk is a shift of B on every later token, i.e.
    a scaling of the state the next chunk starts from, so it equals sum(dS o S) with S
    the state after the chunk and dS its gradient (dST o S_T after the last chunk):
        d log alpha_t = sum_{s >= t in the chunk} (q_s . dq_s - v_s . dv_s) + sum(dS_a o S_a),
    and dalpha = d log alpha / alpha. Returns (dq, dk, dv, dalpha, dbeta, dS0). T must
    be a multiple of ``chunk``.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    dO = np.asarray(dO, np.float64)
    N, T, dk = k.shape
    dv = v.shape[2]
    if T % chunk:
        raise ValueError("T must be a multiple of chunk")
    M = np.tril(np.ones((chunk, chunk)))
    Ms = np.tril(np.ones((chunk, chunk)), -1)
    I = np.eye(chunk)
    dq, dk_, dv_ = np.empty_like(q), np.empty_like(k), np.empty_like(v)
    dlog, dbeta = np.empty_like(alpha), np.empty_like(beta)
    dS0 = np.empty((N, dv, dk))
    for n in range(N):
        S = np.zeros((dv, dk)) if S0 is None else np.array(S0[n], dtype=np.float64)
        starts = []
        for c0 in range(0, T, chunk):      # forward: the state before every chunk
            starts.append(S)
            sl = slice(c0, c0 + chunk)
            K, V, bt = k[n, sl], v[n, sl], beta[n, sl]
            lg = np.cumsum(np.log(alpha[n, sl]))
            g = np.exp(lg)
            Gam = np.exp(np.minimum(lg[:, None] - lg[None, :], 0.0))
            Tm = np.linalg.inv(I + Ms * bt[:, None] * Gam * (K @ K.T))
            U = Tm @ (bt[:, None] * V) - Tm @ ((bt * g)[:, None] * K) @ S.T
            S = g[-1] * S + U.T @ (np.exp(lg[-1] - lg)[:, None] * K)
        starts.append(S)                    # the final state, after the last chunk
        dS = np.zeros((dv, dk)) if dST is None else np.array(dST[n], dtype=np.float64)
        for ci in range(T // chunk - 1, -1, -1):
            boundary = float((dS * starts[ci + 1]).sum())
            sl = slice(ci * chunk, ci * chunk + chunk)
            Q, K, V, bt, dOc, Sb = q[n, sl], k[n, sl], v[n, sl], beta[n, sl], dO[n, sl], starts[ci]
            lg = np.cumsum(np.log(alpha[n, sl]))
            g = np.exp(lg)
            Gam = np.exp(np.minimum(lg[:, None] - lg[None, :], 0.0))
            KK = K @ K.T
            Tm = np.linalg.inv(I + Ms * bt[:, None] * Gam * KK)
            W = Tm @ ((bt * g)[:, None] * K)
            Ut = Tm @ (bt[:, None] * V)
            U = Ut - W @ Sb.T
            A = M * Gam * (Q @ K.T)
            Kh = np.exp(lg[-1] - lg)[:, None] * K
            dU = A.T @ dOc + Kh @ dS.T
            dAg = M * (dOc @ U.T) * Gam
            dQ = dAg @ K + g[:, None] * (dOc @ Sb)
            dW = -dU @ Sb
            dXW, dXU = Tm.T @ dW, Tm.T @ dU
            dL = -Ms * (dXW @ W.T + dXU @ Ut.T)
            dLb = dL * Gam * bt[:, None]
            dK = dAg.T @ Q + np.exp(lg[-1] - lg)[:, None] * (U @ dS) + (bt * g)[:, None] * dXW + dLb @ K + dLb.T @ K
            dV = bt[:, None] * dXU
            dbeta[n, sl] = g * np.einsum("rc,rc->r", dXW, K) + np.einsum("rv,rv->r", dXU, V) + (dL * Gam * KK).sum(1)
            dq[n, sl], dk_[n, sl], dv_[n, sl] = dQ, dK, dV
            dB = np.einsum("tk,tk->t", Q, dQ) - np.einsum("tv,tv->t", V, dV)
            dlog[n, sl] = np.cumsum(dB[::-1])[::-1] + boundary
            dS = g[-1] * dS + dOc.T @ (g[:, None] * Q) - dU.T @ W
        dS0[n] = dS
    return dq, dk_, dv_, dlog / alpha, dbeta, dS0
