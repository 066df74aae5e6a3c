"""LeapQuant windowed 8-bit Gated DeltaNet state, done literally (test infrastructure).

Source: "LeapQuant: an 8-bit recurrent state that stops rounding every token"
(ai.satyajit.si). Every state is ``[d_v][d_k]`` (rows = value channels); the
page's ``d_k x d_v`` formulas are used transposed. Arithmetic is fp64 except
where the page (or the workload) fixes a storage precision, which is applied
at the point of storage:

* codes: symmetric INT8 in [-127, 127], one fp32 scale per value channel, the
  step being the channel's largest magnitude over 127 (section "Fix two", the
  quantiser paragraph, and the dequantised payload (Z/127) B of section "Fix
  three"); ``bits`` = 6 or 4 narrows the grid to [-Q, Q], Q = 2^(bits-1) - 1, in
  the same int8 container (the widths of section "Fix two"'s compensator-count
  paragraph, where the paper pairs them with 6 compensator tokens);
* row smoothing: one fp32 factor per key channel, the square root of that
  channel's mean magnitude over the value channels (section "Fix three", eq. 7),
  clamped below at 1e-12; mode 1 uses the root of the mean square instead and
  mode 2 disables smoothing;
* compensator tokens: r rank-one pieces kept in fp16 (section "Fix two", eq. 5),
  entering the window ahead of the real tokens with decay 1, so they decay with
  the residual;
* window buffer: per real token (k_t, u_t, alpha_t) in fp32.

A window (section "Fix one", eq. 4 and eq. 10): a decode step reads the stored
state and the buffer, computes its correction u_t = beta_t (v_t - alpha_t S k_t)
and output o_t = S_t q_t through the read-out identity of eq. 10, appends its
record and writes no state. After W real tokens the state is rebuilt densely,
new compensator tokens are fitted and subtracted, the residual is smoothed and
rounded once (the window flush).

The compensator fit follows the procedure the page reports for the released
flush kernel: ``iters`` rounds (default 1) of subspace iteration from a fixed
random start block Q0 (passed in), each orthonormalised by CholeskyQR2; the
Gram matrix of each CholeskyQR pass is shifted by 1e-6 * trace + 1e-30 so that a
rank-deficient or zero state stays finite. The exact top-r singular pairs
(Eckart-Young) are available with ``svd=True`` for reference, not for parity.

Quantiser decisions are taken in fp32, the precision of the GPU path (the page
fixes no other): the pre-rounding value is float32(R / c * 127 / s) and the code
is clamp(rint(x), -127, 127) with round-half-to-even. A value channel whose
residual is all zero stores scale 0 and codes 0.

Pins (tests/test_oracle_leapq.py): window 1, rank 0, no smoothing equals the
per-token rounding of eq. 2 (``per_step_int8``, a separate code path); the eq. 10
read-out equals the dense eq. 4 state applied to the vector; ``window_run`` from a
stored state the grid holds exactly, with an fp64 buffer, equals the exact Gated
DeltaNet recurrence (read-outs, corrections and rebuild), and from the encoded
initial state equals ``decode_run``'s windows; a rank <= r state
leaves a zero residual; Eckart-Young for the SVD mode; per-entry reconstruction
error within half a step; codes invariant under power-of-two scaling; stored
bytes 19,456 per 128 x 128 head; the page's BF16/FP16 decay-freezing counts
for the fp16/bf16 rounding used.
"""
from __future__ import annotations

import numpy as np

SHIFT_REL = 1e-6
SHIFT_ABS = 1e-30
SMOOTH_FLOOR = 1e-12


# ----------------------------------------------------------------- helpers

def fp16(x):
    """Round to IEEE binary16, nearest-even (numpy's cast), back to fp64."""
    return np.asarray(x, np.float64).astype(np.float16).astype(np.float64)


def fp32(x):
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def qmax(bits):
    """Largest code of the symmetric b-bit grid, 2^(b-1) - 1 (127 at 8 bits)."""
    if not 2 <= bits <= 8:
        raise ValueError("bits must be in 2..8")
    return (1 << (bits - 1)) - 1


def round_codes(x32, bits=8):
    """Code decision on fp32 pre-rounding values: clamp(rint(x), -Q, Q)."""
    x32 = np.asarray(x32, np.float32)
    Q = qmax(bits)
    return np.clip(np.rint(x32), -Q, Q).astype(np.int8)


def cholqr2(Z):
    """Orthonormalise the columns of Z ([..][d][r]) by two CholeskyQR passes,
    each with the Gram shift described in the module docstring."""
    Z = np.asarray(Z, np.float64)
    r = Z.shape[-1]
    eye = np.eye(r)
    for _ in range(2):
        G = np.swapaxes(Z, -1, -2) @ Z
        tr = np.trace(G, axis1=-2, axis2=-1)[..., None, None]
        G = G + (SHIFT_REL * tr + SHIFT_ABS) * eye
        L = np.linalg.cholesky(G)
        # Z <- Z L^{-T}: solve L Y = Z^T for Y, then Z = Y^T
        Z = np.swapaxes(np.linalg.solve(L, np.swapaxes(Z, -1, -2)), -1, -2)
    return Z


def smoothing(R, mode):
    """Per key channel factor c_k from the residual R ([N][d_v][d_k])."""
    if mode == 0:
        c = np.sqrt(np.mean(np.abs(R), axis=-2))
    elif mode == 1:
        c = np.sqrt(np.mean(R * R, axis=-2))
    elif mode == 2:
        return np.ones(R.shape[:-2] + (R.shape[-1],))
    else:
        raise ValueError("smooth_mode must be 0, 1 or 2")
    return np.maximum(c, SMOOTH_FLOOR)


# ----------------------------------------------------------------- flush

def fit_compensators(S, Q0, rank=4, iters=1, svd=False):
    """Key directions of the r compensator tokens, [N][d_k][r] with orthonormal
    columns: ``iters`` rounds of Q <- orth(S^T (S Q)) from Q0, or the top-r right
    singular vectors with ``svd``. The value parts are S Q."""
    S = np.asarray(S, np.float64)
    N, dv, dk = S.shape
    if svd:
        _, _, Vt = np.linalg.svd(S)
        return np.swapaxes(Vt[:, :rank, :], -1, -2)
    Q = np.broadcast_to(np.asarray(Q0, np.float64)[:, :rank], (N, dk, rank))
    for _ in range(iters):
        Y = S @ Q                                              # [N][dv][r]
        Q = cholqr2(np.swapaxes(S, -1, -2) @ Y)                # [N][dk][r]
    return Q


def flush(S, Q0=None, rank=4, iters=1, smooth_mode=0, svd=False, bits=8):
    """Encode dense states S ([N][d_v][d_k]) into the stored form (codes on the
    symmetric ``bits``-bit grid).

    Returns dict(Z int8 [N][dv][dk], s fp32 [N][dv], c fp32 [N][dk],
    kt fp16 [N][r][dk], ut fp16 [N][r][dv], pre fp32 [N][dv][dk]) with the
    float fields as fp64 arrays holding exactly representable values.
    """
    S = np.asarray(S, np.float64)
    N, dv, dk = S.shape
    if rank > 0:
        Q = fit_compensators(S, Q0, rank, iters, svd)
        kt = fp16(np.swapaxes(Q, -1, -2))                      # [N][r][dk]
        ut = fp16(np.swapaxes(S @ Q, -1, -2))                  # [N][r][dv]
        R = S - np.swapaxes(ut, -1, -2) @ kt                   # subtract the stored pieces
    else:
        kt = np.zeros((N, 0, dk))
        ut = np.zeros((N, 0, dv))
        R = S
    out = encode_residual(R, smooth_mode, bits)
    out.update(kt=kt, ut=ut)
    return out


def encode_residual(R, smooth_mode=0, bits=8):
    """Smooth and round a residual R ([N][d_v][d_k]) once: returns dict(Z, s, c,
    pre) -- codes, value-channel scales, key-channel smoothing factors (fp32) and
    the fp32 pre-rounding values -- and Q. With Q = 2^(bits-1) - 1 (127 at 8 bits)
    and s_v = max_k |R/c| (fp32): pre = (R/c) (Q/s_v), codes = clamp(rint(pre), -Q, Q);
    the channel dequantises as s_v Z / Q."""
    R = np.asarray(R, np.float64)
    Q = qmax(bits)
    c = fp32(smoothing(R, smooth_mode))                        # [N][dk]
    Rc = R / c[:, None, :]
    s = fp32(np.max(np.abs(Rc), axis=-1))                      # [N][dv]
    with np.errstate(divide="ignore", invalid="ignore"):
        pre = np.where(s[:, :, None] > 0, Rc * (float(Q) / s[:, :, None]), 0.0)
    pre = pre.astype(np.float32)
    Z = round_codes(pre, bits)
    return dict(Z=Z, s=s, c=c, pre=pre, Q=Q)


def dequant(st):
    """Dense stored state: C-smoothed dequantised residual plus the fp16
    compensator pieces, S_hat[v,k] = s_v Z[v,k] / Q c_k + sum_r ut_r[v] kt_r[k]
    (Q = 127 at 8 bits)."""
    Z = st["Z"].astype(np.float64)
    S = st["s"][:, :, None] * (Z / float(st.get("Q", 127))) * st["c"][:, None, :]
    return S + np.swapaxes(st["ut"], -1, -2) @ st["kt"]


def stored_bytes(dv, dk, rank):
    """Bytes of one head at rest: INT8 codes, fp32 value-channel scales and
    key-channel smoothing factors, fp16 compensator pairs."""
    return dv * dk * 1 + (dv + dk) * 4 + rank * (dk + dv) * 2


# ----------------------------------------------------------------- window

def readout(st, buf, x):
    """Eq. 10: S_m x for every head, where m = len(buf) records (k, u, a) of
    the current window: Gamma_{1:m} S_hat_0 x + sum_j Gamma_{j+1:m} u_j (k_j . x).
    x: [N][d_k]. The stored part is evaluated through the integer matrix with the
    smoothing folded into the vector, as the page describes."""
    x = np.asarray(x, np.float64)
    Z = st["Z"].astype(np.float64)
    y = st["s"] * np.einsum("nvk,nk->nv", Z, st["c"] * x) / float(st.get("Q", 127))
    y = y + np.einsum("nrv,nr->nv", st["ut"], np.einsum("nrk,nk->nr", st["kt"], x))
    m = len(buf)
    g = np.ones(x.shape[0])
    for (_, _, a) in buf:
        g = g * a
    out = g[:, None] * y
    for j, (kj, uj, _) in enumerate(buf):
        gj = np.ones(x.shape[0])
        for (_, _, a) in buf[j + 1:m]:
            gj = gj * a
        out = out + gj[:, None] * uj * np.sum(kj * x, axis=-1)[:, None]
    return out


def rebuild(st, buf):
    """Eq. 4: the dense state after the buffered records,
    S_m = Gamma_{1:m} S_hat_0 + sum_j Gamma_{j+1:m} u_j k_j^T."""
    S = dequant(st)
    for (kj, uj, a) in buf:
        S = a[:, None, None] * S + uj[:, :, None] * kj[:, None, :]
    return S


def decode_run(q, k, v, alpha, beta, S0, Q0, window=16, rank=4, iters=1,
               smooth_mode=0, buf_dtype=np.float32, collect=False, bits=8):
    """The windowed scheme over T tokens for N heads (inputs [T][N][d], gates
    [T][N], S0 [N][d_v][d_k]). The initial state is encoded by one flush before
    the first token; after every ``window`` real tokens the state is rebuilt and
    flushed. Returns dict(o [T][N][d_v], stored state after the last flush or the
    current window's state, buf (records of the open window)); with
    ``collect`` also the stored state at every window start."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    alpha = np.asarray(alpha, np.float64)
    beta = np.asarray(beta, np.float64)
    T = q.shape[0]
    st = flush(S0, Q0, rank, iters, smooth_mode, bits=bits)
    starts = [st] if collect else None
    buf = []
    o = np.empty(v.shape)
    for t in range(T):
        a, b = alpha[t], beta[t]
        Sk = readout(st, buf, k[t])
        u = b[:, None] * (v[t] - a[:, None] * Sk)
        u = u.astype(buf_dtype).astype(np.float64)
        buf.append((k[t], u, a))
        o[t] = readout(st, buf, q[t])
        if len(buf) == window:
            st = flush(rebuild(st, buf), Q0, rank, iters, smooth_mode, bits=bits)
            buf = []
            if collect:
                starts.append(st)
    out = dict(o=o, st=st, buf=buf)
    if collect:
        out["starts"] = starts
    return out


def window_run(st, q, k, v, alpha, beta, buf_dtype=np.float32):
    """One window's read-outs from a given stored state (teacher forcing):
    returns (o [W][N][d_v], buf records)."""
    buf = []
    W = q.shape[0]
    o = np.empty(np.asarray(v).shape)
    for t in range(W):
        a = np.asarray(alpha[t], np.float64)
        b = np.asarray(beta[t], np.float64)
        kt = np.asarray(k[t], np.float64)
        Sk = readout(st, buf, kt)
        u = (b[:, None] * (np.asarray(v[t], np.float64) - a[:, None] * Sk))
        u = u.astype(buf_dtype).astype(np.float64)
        buf.append((kt, u, a))
        o[t] = readout(st, buf, np.asarray(q[t], np.float64))
    return o, buf


# ----------------------------------------------------------------- eq. 2

def per_step_int8(q, k, v, alpha, beta, S0, bits=8):
    """Eq. 2 (section "Rounding every token"): the state is requantised after
    every token, S_t = alpha_t S_hat_{t-1} + k_t u_t^T (transposed here) with
    u_t computed from the stored state, S_hat_t = quant(S_t). Symmetric b-bit codes
    (Q = 2^(b-1) - 1) with one scale per value channel, the step being the channel's
    largest magnitude over Q; no smoothing, no compensator tokens. Written
    independently of the windowed path; returns (o, Z, m) with m the channels'
    largest magnitudes (the dequantised state is m Z / Q)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    Q = float(qmax(bits))

    def quant(S):
        m = fp32(np.max(np.abs(S), axis=-1))
        with np.errstate(divide="ignore", invalid="ignore"):
            x = np.where(m[:, :, None] > 0, S * (Q / m[:, :, None]), 0.0)
        Z = np.clip(np.rint(x.astype(np.float32)), -Q, Q).astype(np.int8)
        return Z, m

    Z, m = quant(np.asarray(S0, np.float64))
    o = np.empty(v.shape)
    for t in range(q.shape[0]):
        Sh = m[:, :, None] * Z.astype(np.float64) / Q
        a = np.asarray(alpha[t], np.float64)[:, None]
        b = np.asarray(beta[t], np.float64)[:, None]
        u = b * (v[t] - a * np.einsum("nvk,nk->nv", Sh, k[t]))
        S = a[:, :, None] * Sh + u[:, :, None] * k[t][:, None, :]
        o[t] = np.einsum("nvk,nk->nv", S, q[t])
        Z, m = quant(S)
    return o, Z, m


def bf16(x):
    """Round to bfloat16, nearest-even, back to fp64 (8 significant bits)."""
    x32 = np.ascontiguousarray(np.asarray(x, np.float64), dtype=np.float32)
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def per_step_bf16(q, k, v, alpha, beta, S0):
    """The state kept in BF16 and re-rounded after every token (section "Rounding
    every token", the BF16 case): u_t from the stored state, S_t = alpha_t S_{t-1} +
    u_t k_t^T computed exactly, then rounded to bf16 (nearest even) per entry.
    Returns (o, S_T)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    S = bf16(S0)
    o = np.empty(v.shape)
    for t in range(q.shape[0]):
        a = np.asarray(alpha[t], np.float64)[:, None]
        b = np.asarray(beta[t], np.float64)[:, None]
        u = b * (v[t] - a * np.einsum("nvk,nk->nv", S, k[t]))
        Sn = a[:, :, None] * S + u[:, :, None] * k[t][:, None, :]
        o[t] = np.einsum("nvk,nk->nv", Sn, q[t])
        S = bf16(Sn)
    return o, S
