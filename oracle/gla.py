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
``zeco_local``, ``zeco_all_scan_step``, ``zeco_output`` and ``zeco_forward``
take ZeCO's three forward phases in the page's order (local chunk states and
cumulative decays from zero, the All-Scan update, outputs from the received
state); they are pinned by the recurrence over the whole sequence for several
device and block counts, by the closed form of the cumulative decays and by the
local states at the chunk boundaries. ``zeco_bwd_local_state`` and ``zeco_backward``
take the backward's phases (local state gradient from zero, the backward All-Scan,
gradients from the received state gradient); pinned by reverse mode through the
recurrence over the whole sequence.
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


def zeco_local(k, v, log_g, chunk=64):
    """Phase 1 of ZeCO's forward on one device (page section "Local State
    Computation"): from a zero state, the chunk states and the cumulative decays

        S_[n]      = gamma_[n] (on key columns) o S_[n-1] + ((K o Gamma)^T V)^T,
        gamma~_[n] = gamma~_[n-1] o gamma_[n],      gamma_[n] = exp(b_C of chunk n),

    for n = 1..nc, with S_[0] = 0 and gamma~_[0] = 1. Returns
    (S [N][nc+1][d_v][d_k], gam [N][nc+1][d_k])."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    lg = np.asarray(log_g, np.float64)
    N, T, dk = k.shape
    dv = v.shape[2]
    if T % chunk:
        raise ValueError("T must be a multiple of chunk")
    nc = T // chunk
    S = np.zeros((N, nc + 1, dv, dk))
    gam = np.ones((N, nc + 1, dk))
    for n in range(nc):
        sl = slice(n * chunk, (n + 1) * chunk)
        b = np.cumsum(lg[:, sl], axis=1)
        Kg = k[:, sl] * np.exp(b[:, -1:, :] - b)            # K o Gamma
        gamma = np.exp(b[:, -1])                            # chunk decay per key
        S[:, n + 1] = gamma[:, None, :] * S[:, n] + np.einsum("njv,njk->nvk", v[:, sl], Kg)
        gam[:, n + 1] = gam[:, n] * gamma
    return S, gam


def zeco_all_scan_step(S_local, gam_total, S_recv=None, blocks=1):
    """One device's step of All-Scan (page section "All-Scan Collective
    Communication"): the key channels are cut into ``blocks`` contiguous blocks,
    and each block of the state to send is the received block decayed by the
    device's total cumulative decay plus the local final state's block,
    S_send = gamma~_[N] (on key columns) o S_recv + S_[N]. The start device has
    nothing to receive (``S_recv`` None) and sends its local state.
    S_local, S_recv: [N][d_v][d_k]; gam_total: [N][d_k]."""
    S_local = np.asarray(S_local, np.float64)
    if S_recv is None:
        return S_local.copy()
    S_recv = np.asarray(S_recv, np.float64)
    gam_total = np.asarray(gam_total, np.float64)
    dk = S_local.shape[2]
    out = np.empty_like(S_local)
    edges = np.linspace(0, dk, blocks + 1).astype(int)
    for k0, k1 in zip(edges[:-1], edges[1:]):
        out[:, :, k0:k1] = gam_total[:, None, k0:k1] * S_recv[:, :, k0:k1] + S_local[:, :, k0:k1]
    return out


def zeco_output(q, k, v, log_g, S_states, gam, S_in=None, chunk=64):
    """Phase 3 of ZeCO's forward (page section "The Complete Forward Algorithm"):
    per chunk n, from the local state before it and the received state,

        O_[n] = Q~_[n] (S_[n-1] + gamma~_[n-1] o S_in)^T + P_[n] V_[n],
        Q~ = Q o Lambda,  P = (Q~ (K / Lambda)^T) o M,

    with Lambda = exp(b), b the inclusive in-chunk cumulative log-gate and M lower
    triangular including the diagonal (the inclusive read-out o_t = S_t q_t).
    S_states, gam: as returned by ``zeco_local``; S_in None is a zero state."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    lg = np.asarray(log_g, np.float64)
    N, T, dk = k.shape
    dv = v.shape[2]
    M = np.tril(np.ones((chunk, chunk)))
    o = np.empty((N, T, dv))
    for n in range(T // chunk):
        sl = slice(n * chunk, (n + 1) * chunk)
        b = np.cumsum(lg[:, sl], axis=1)
        Qt = q[:, sl] * np.exp(b)
        Kt = k[:, sl] * np.exp(-b)
        S = S_states[:, n]
        if S_in is not None:
            S = S + gam[:, n][:, None, :] * np.asarray(S_in, np.float64)
        P = np.einsum("nrk,njk->nrj", Qt, Kt) * M
        o[:, sl] = np.einsum("nrk,nvk->nrv", Qt, S) + np.einsum("nrj,njv->nrv", P, v[:, sl])
    return o


def zeco_forward(q, k, v, log_g, devices, S0=None, chunk=64, blocks=1):
    """ZeCO's forward over ``devices`` devices, run one after the other here: the
    sequence is cut into that many contiguous shards of whole chunks; each runs
    phase 1 from a zero state; All-Scan passes the states along the devices in
    order, starting from S0 (None = zero); each device then computes its outputs
    from the state it received. Returns (o [N][T][d_v], S_T [N][d_v][d_k])."""
    T = np.asarray(k).shape[1]
    if T % (devices * chunk):
        raise ValueError("T must be a multiple of devices * chunk")
    L = T // devices
    outs = []
    S_recv = None if S0 is None else np.asarray(S0, np.float64)
    for p in range(devices):
        sl = slice(p * L, (p + 1) * L)
        Ss, gam = zeco_local(k[:, sl], v[:, sl], log_g[:, sl], chunk)
        S_send = zeco_all_scan_step(Ss[:, -1], gam[:, -1], S_recv, blocks)
        outs.append(zeco_output(q[:, sl], k[:, sl], v[:, sl], log_g[:, sl], Ss, gam, S_recv, chunk))
        S_recv = S_send
    return np.concatenate(outs, axis=1), S_recv


def zeco_bwd_local_state(q, log_g, dO, chunk=64):
    """Phase 1 of ZeCO's backward on one device (page section "The Backward
    Algorithm and Gradient Flow"): from dS = 0 at the shard's end, per chunk in
    reverse, dS <- gamma (on key columns) o dS + (dO^T (Q o Lambda)), Lambda = exp(b)
    inclusive; the result is the gradient with respect to the state the shard
    starts from, counting only the shard's own outputs. Returns [N][d_v][d_k]."""
    q = np.asarray(q, np.float64)
    lg = np.asarray(log_g, np.float64)
    dO = np.asarray(dO, np.float64)
    N, T, dk = q.shape
    dv = dO.shape[2]
    dS = np.zeros((N, dv, dk))
    for n in range(T // chunk - 1, -1, -1):
        sl = slice(n * chunk, (n + 1) * chunk)
        b = np.cumsum(lg[:, sl], axis=1)
        dS = np.exp(b[:, -1])[:, None, :] * dS + np.einsum("ntv,ntk->nvk", dO[:, sl], q[:, sl] * np.exp(b))
    return dS


def zeco_backward(q, k, v, log_g, dO, devices, S0=None, dST=None, chunk=64, blocks=1):
    """ZeCO's backward over ``devices`` devices, run one after the other here: the
    forward's All-Scan gives each device the state it starts from; phase 1 gives
    each device its local dS_[0]; the backward All-Scan passes the state gradient
    from the last device to the first, each sending gamma~_[N] o dS_recv + dS_[0];
    each device then forms its gradients from its incoming state and the received
    state gradient (``gla_recurrent_bwd`` of its shard). Returns (dq, dk, dv, dlog_g,
    dS0) for the whole sequence."""
    T = np.asarray(k).shape[1]
    if T % (devices * chunk):
        raise ValueError("T must be a multiple of devices * chunk")
    L = T // devices
    sls = [slice(p * L, (p + 1) * L) for p in range(devices)]
    S_in, gam_tot = [], []
    S = None if S0 is None else np.asarray(S0, np.float64)
    for sl in sls:
        Ss, gam = zeco_local(k[:, sl], v[:, sl], log_g[:, sl], chunk)
        S_in.append(S)
        gam_tot.append(gam[:, -1])
        S = zeco_all_scan_step(Ss[:, -1], gam[:, -1], S, blocks)
    local = [zeco_bwd_local_state(q[:, sl], log_g[:, sl], dO[:, sl], chunk) for sl in sls]
    dS_recv = [None] * devices
    d = None if dST is None else np.asarray(dST, np.float64)
    for p in range(devices - 1, -1, -1):
        dS_recv[p] = d
        d = zeco_all_scan_step(local[p], gam_tot[p], d, blocks)
    grads = [gla_recurrent_bwd(q[:, sl], k[:, sl], v[:, sl], log_g[:, sl], S_in[p], dO[:, sl], dS_recv[p])
             for p, sl in enumerate(sls)]
    out = [np.concatenate([g[i] for g in grads], axis=1) for i in range(4)]
    return (*out, d)


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
