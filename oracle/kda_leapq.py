"""LeapQuant's windowed 8-bit state for Kimi Delta Attention, done literally
(test infrastructure).

Source: "LeapQuant: an 8-bit recurrent state that stops rounding every token".
KDA (section "The state, from the update rule up") decays the state with one
factor per key channel: in the library's [d_v][d_k] layout
S_t = S_{t-1} Diag(alpha_t) + u_t k_t^T with u_t = beta_t (v_t - S_{t-1} (alpha_t o k_t))
and o_t = S_t q_t. The window leap of section "Fix one" (eq. 4 and eq. 10) is
written with diagonal decays, the products Gamma_{a:b} = Diag(alpha_a ... alpha_b):

    S_m   = S_hat_0 Gamma_{1:m} + sum_j u_j k_j^T Gamma_{j+1:m}            (eq. 4)
    S_m y = S_hat_0 (Gamma_{1:m} y) + sum_j u_j (k_j . (Gamma_{j+1:m} y))   (eq. 10)

and the page notes that the decays are diagonal and accumulate incrementally, and
that the smoothing factors fold into the vector Gamma x before it meets the
integer matrix (section "Fix three"). The compensator tokens enter the window
ahead of the real tokens with decay 1, so they decay with the stored residual by
Gamma_{1:m}. The page's KDA buffer also keeps each buffered token's per-channel
decay (its Gbuf tensor); here every buffered quantity is fp32, as in the GDN path.

The flush (rebuild, compensator fit, subtraction, smoothing, one rounding) is the
one of ``oracle.leapq``: it acts on a dense state and does not depend on the
decay. Decays are multiplied, never divided.

Inputs are token-major like ``oracle.leapq``: q, k [T][N][d_k], v [T][N][d_v],
alpha [T][N][d_k], beta [T][N].

Pins (tests/test_oracle_kda_leapq.py): equal decays on every channel reproduce
the Gated DeltaNet windowed oracle; the eq. 10 read-out equals the eq. 4 dense
state applied to the vector; a stored state that the INT8 grid holds exactly
reproduces the exact KDA recurrence (``oracle.kda.kda_recurrent``) through a
whole window; window 1 with rank 0 and no smoothing equals ``per_step_int8``,
the per-token rounding of eq. 2 written separately.
"""
from __future__ import annotations

import numpy as np

from . import leapq


def _suffix(buf, j, dk, n):
    """Gamma_{j+1:m} for the m records of buf: the product of their decays after
    record j (j = -1 gives Gamma_{1:m}), [N][d_k]."""
    g = np.ones((n, dk))
    for (_, _, a) in buf[j + 1:]:
        g = g * a
    return g


def readout(st, buf, y):
    """Eq. 10 with diagonal decays: S_m y for every head, where buf holds the m
    records (k_j, u_j, alpha_j) of the open window. The stored part goes through
    the integer matrix with the smoothing and Gamma_{1:m} folded into the vector."""
    y = np.asarray(y, np.float64)
    n, dk = y.shape
    x = _suffix(buf, -1, dk, n) * y                                   # Gamma_{1:m} y
    Z = st["Z"].astype(np.float64)
    out = st["s"] * np.einsum("nvk,nk->nv", Z, st["c"] * x) / float(st.get("Q", 127))
    out = out + np.einsum("nrv,nr->nv", st["ut"], np.einsum("nrk,nk->nr", st["kt"], x))
    for j, (kj, uj, _) in enumerate(buf):
        out = out + uj * np.sum(kj * (_suffix(buf, j, dk, n) * y), axis=-1)[:, None]
    return out


def rebuild(st, buf):
    """Eq. 4 with diagonal decays: the dense state after the buffered records,
    one record at a time, S <- S Diag(alpha_j) + u_j k_j^T."""
    S = leapq.dequant(st)
    for (kj, uj, a) in buf:
        S = S * a[:, None, :] + uj[:, :, None] * kj[:, None, :]
    return S


def window_run(st, q, k, v, alpha, beta, buf_dtype=np.float32):
    """One window's read-outs from a given stored state (teacher forcing):
    per token u = beta (v - S_m (alpha o k)), the record (k, u, alpha) appended,
    o = S_{m+1} q. Returns (o [W][N][d_v], buf records)."""
    buf = []
    o = np.empty(np.asarray(v).shape)
    for t in range(np.asarray(q).shape[0]):
        a = np.asarray(alpha[t], np.float64)
        b = np.asarray(beta[t], np.float64)
        kt = np.asarray(k[t], np.float64)
        Sk = readout(st, buf, a * kt)
        u = b[:, None] * (np.asarray(v[t], np.float64) - Sk)
        u = u.astype(buf_dtype).astype(np.float64)
        buf.append((kt, u, a))
        o[t] = readout(st, buf, np.asarray(q[t], np.float64))
    return o, buf


def decode_run(q, k, v, alpha, beta, S0, Q0, window=16, rank=4, iters=1,
               smooth_mode=0, buf_dtype=np.float32):
    """The windowed scheme over T tokens: the initial state is encoded by one
    flush, then every ``window`` real tokens the state is rebuilt (eq. 4) and
    flushed once. Returns dict(o [T][N][d_v], st, buf)."""
    q = np.asarray(q, np.float64)
    st = leapq.flush(S0, Q0, rank, iters, smooth_mode)
    buf = []
    o = np.empty(np.asarray(v).shape)
    for t in range(q.shape[0]):
        a = np.asarray(alpha[t], np.float64)
        b = np.asarray(beta[t], np.float64)
        kt = np.asarray(k[t], np.float64)
        Sk = readout(st, buf, a * kt)
        u = b[:, None] * (np.asarray(v[t], np.float64) - Sk)
        u = u.astype(buf_dtype).astype(np.float64)
        buf.append((kt, u, a))
        o[t] = readout(st, buf, q[t])
        if len(buf) == window:
            st = leapq.flush(rebuild(st, buf), Q0, rank, iters, smooth_mode)
            buf = []
    return dict(o=o, st=st, buf=buf)


def per_step_int8(q, k, v, alpha, beta, S0):
    """Eq. 2 for KDA: the state requantised after every token (symmetric INT8,
    one scale per value channel, no smoothing, no compensators), u from the
    stored state: S_t = S_hat_{t-1} Diag(alpha_t) + u_t k_t^T. Written apart from
    the windowed path; returns (o, Z, s)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)

    def quant(S):
        s = leapq.fp32(np.max(np.abs(S), axis=-1))
        with np.errstate(divide="ignore", invalid="ignore"):
            x = np.where(s[:, :, None] > 0, S * (127.0 / s[:, :, None]), 0.0)
        return leapq.round_codes(x.astype(np.float32)), s

    Z, s = quant(np.asarray(S0, np.float64))
    o = np.empty(v.shape)
    for t in range(q.shape[0]):
        Sh = s[:, :, None] * Z.astype(np.float64) / 127.0
        a = np.asarray(alpha[t], np.float64)
        b = np.asarray(beta[t], np.float64)[:, None]
        u = b * (v[t] - np.einsum("nvk,nk->nv", Sh, a * k[t]))
        S = Sh * a[:, None, :] + u[:, :, None] * k[t][:, None, :]
        o[t] = np.einsum("nvk,nk->nv", S, q[t])
        Z, s = quant(S)
    return o, Z, s
